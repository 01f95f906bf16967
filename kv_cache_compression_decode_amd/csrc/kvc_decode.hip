// Fused decode: range decode -> dequantize / anchor+delta reconstruction ->
// store into the [layer][K/V][token][channel] binary16 KV cache.
//
// CacheGen page, 核心方法: each chunk's bitstream is decoded on the GPU back
// to tensors; tokens of a 10-token group depend only on their anchor (no
// delta chain); symbols were arithmetic-coded against per channel-layer
// models, anchors and deltas separately.
//
// Work decomposition (gfx950, wave64):
//  * a workgroup owns one (layer*2+kv row, block of 64 channels) and a group
//    of chunks (normally every chunk of the call), and stages the 64
//    channels' anchor models and their delta models of every level the group
//    uses into LDS once;
//  * its W waves take the group's chunks two at a time (the host sorts a
//    group's chunks by level, so the two chunks of a pair mostly share one
//    alphabet size); every lane decodes the streams of its channel in both
//    chunks in lockstep, so each lane runs two independent dependency chains
//    and one LDS copy of the models serves every chunk of the group;
//  * all lanes of a wave are at the same token, so the anchor/delta switch
//    and the search depth are wave-uniform, and the 64 results of a token are
//    64 consecutive channels: one coalesced 128-byte store per stream,
//    addressed from a wave-uniform base;
//  * symbols are found by binary search of the cumulative tables: 8 steps
//    for anchors, b steps for a b-bit delta alphabet, the two streams'
//    probes interleaved;
//  * stream bytes are staged per lane in a 16-byte LDS ring fed in 8-byte
//    blocks: at every group boundary a lane whose ring has room stores the
//    block it loaded earlier and issues the load of the next one, so
//    global-memory latency is off the per-symbol path; a rare slow path
//    refills a ring that runs low.  Loads go through a buffer resource
//    bounded by the container size, so the block after a stream's last byte
//    may be loaded unconditionally (past the container end it reads as zero);
//  * LDS rows use odd dword strides so that lanes reading the same entry
//    index of their own tables hit different banks;
//  * blocks are numbered so that the groups of one (row, channel block) run
//    on the same XCD.
#include "kvc_internal.h"

namespace kvc {

namespace {

constexpr uint32_t kMaxWaves = kDecodeMaxWaves;  // waves per workgroup (host picks W <= this)
constexpr uint32_t kSlots = 2;                   // streams per lane
constexpr uint32_t kAStride = 129;  // dwords per staged anchor model (cum[0..256] + pad)
constexpr uint32_t kDStride = 33;   // dwords per staged delta model (cum[0..63] + pad)
constexpr uint32_t kRing = 5;       // dwords per lane ring: 16 bytes + mirror of bytes 0..3
constexpr uint32_t kXcds = 8;

// Explicit address spaces for the LDS tables / rings and the output, so that
// every access compiles to a ds_* or global_* instruction (a generic "flat"
// access counts against both wait counters).
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) const uint16_t lds_cu16;
typedef __attribute__((address_space(3))) const uint8_t lds_cu8;
typedef __attribute__((address_space(1))) uint8_t gbyte;

// t = floor(code / r) for r in [2^9, 2^17).  The float estimate is biased
// down by 2^-5, more than its worst error for quotients below 2^16, so it is
// t or t - 1 and one compare fixes it; it never exceeds the true quotient,
// so q * r <= code cannot wrap.  A quotient >= 2^15 (a corrupt stream) is
// always returned as >= 2^15.
__device__ inline uint32_t quotient(uint32_t code, uint32_t r) {
  const float fr = (float)r;
  const float fc = (float)code;
  const uint32_t q = (uint32_t)(int32_t)__builtin_fmaf(fc, __builtin_amdgcn_rcpf(fr), -0.03125f);
  const uint32_t p = __umul24(q, r);  // q < 2^24, r < 2^17: exact in 32 bits
  return q + (code - p >= r ? 1u : 0u);
}

struct Stream {
  uint32_t voff;        // byte offset of the stream in its container
  lds_u32 *ring;        // this lane's ring in LDS (16 bytes + 4 mirrored)
  uint32_t code, range;
  uint32_t rpos;        // bytes consumed
  uint32_t wpos;        // bytes written to the ring (a multiple of 8)
  uint32_t b0, b1;      // the 8 bytes at wpos, loaded ahead (memory order)
  uint32_t n;
  uint32_t nbytes;
  uint32_t tor;         // OR of every quotient: >= 2^15 flags a corrupt stream
  int32_t M;
  float lo, sa, dl, ahat;

  __device__ inline void load_block(__amdgpu_buffer_rsrc_t src) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(src, voff + wpos, 0, 0);
    b0 = v[0];
    b1 = v[1];
  }
  __device__ inline void write_block() {  // b0, b1 into the free ring half
    const uint32_t h = (wpos >> 2) & 2;     // dword 0 or 2
    ring[h] = b0;
    ring[h + 1] = b1;
    if (h == 0) ring[4] = b0;
    wpos += 8;
  }
  // At a group boundary: store the block loaded earlier if its half of the
  // ring is free, then load the block that follows the ring's contents.
  __device__ inline void maintain(__amdgpu_buffer_rsrc_t src) {
    if (wpos - rpos <= 8) {
      write_block();
      load_block(src);
    }
  }
  // Make sure the next symbol's (at most 2) bytes are in the ring (rare).
  __device__ inline void ensure(__amdgpu_buffer_rsrc_t src) {
    if (__builtin_expect(wpos - rpos < 2, 0)) {
      write_block();
      load_block(src);
    }
  }
};

// One token of Q streams of a lane, in lockstep: range decode, dequantize.
// kSteps binary-search steps cover symbol indices [0, 2^kSteps); entries past
// a model's alphabet are >= 0x8000 and never taken for a valid target.  Writes the value to
// store (binary16 bits, or the symbol) to v[q].
template <uint32_t Q, bool kSymbols, bool kAnchor, uint32_t kSteps>
__device__ inline void step(Stream *st, lds_cu16 *ta, lds_cu16 *const *td,
                            const __amdgpu_buffer_rsrc_t *src, uint32_t *v) {
#pragma unroll
  for (uint32_t q = 0; q < Q; ++q) st[q].ensure(src[q]);
  uint32_t r[Q], t[Q], s[Q], cs[Q], cn[Q];
#pragma unroll
  for (uint32_t q = 0; q < Q; ++q) {
    r[q] = st[q].range >> kPrec;
    t[q] = quotient(st[q].code, r[q]);
    st[q].tor |= t[q];
  }
  // binary search of the cumulative table, the streams' probes interleaved
  lds_cu16 *p[Q];
#pragma unroll
  for (uint32_t q = 0; q < Q; ++q) p[q] = kAnchor ? ta : td[q];
  lds_cu16 *base[Q];
#pragma unroll
  for (uint32_t q = 0; q < Q; ++q) base[q] = p[q];
#pragma unroll
  for (uint32_t sz = 1u << (kSteps - 1); sz; sz >>= 1) {
    uint32_t probe[Q];
#pragma unroll
    for (uint32_t q = 0; q < Q; ++q) probe[q] = p[q][sz];
#pragma unroll
    for (uint32_t q = 0; q < Q; ++q)
      if (probe[q] <= t[q]) p[q] += sz;
  }
#pragma unroll
  for (uint32_t q = 0; q < Q; ++q) {
    s[q] = (uint32_t)(p[q] - base[q]);
    cs[q] = p[q][0];
    cn[q] = p[q][1];
  }
  uint32_t in[Q];
#pragma unroll
  for (uint32_t q = 0; q < Q; ++q) {
    lds_cu8 *rb = (lds_cu8 *)st[q].ring + (st[q].rpos & 15);
    in[q] = ((uint32_t)rb[0] << 8) | rb[1];  // the next two stream bytes
  }
#pragma unroll
  for (uint32_t q = 0; q < Q; ++q) {
    Stream &x = st[q];
    // 24-bit multiplies: r < 2^17 and cumulative counts <= 2^16.  Every
    // interval of the staged tables is nonempty (the profiler gives every
    // symbol a nonzero frequency; pads increase), so range >= r >= 2^9 here
    // and >= 2^24 after the shift: the count of leading zeros is defined.
    x.code -= __umul24(r[q], cs[q]);
    const uint32_t range = __umul24(r[q], cn[q] - cs[q]);
    // whole bytes to shift in: 0, 1 or 2
    const uint32_t lz = (uint32_t)__builtin_clz(range);
    const uint32_t sh = lz & 24u;
    x.range = range << sh;
    x.code = (x.code << sh) | (in[q] >> ((16 - sh) & 31));
    x.rpos += lz >> 3;
    if constexpr (kSymbols) {
      v[q] = s[q];
    } else {
      float y;
      if constexpr (kAnchor) {
        x.ahat = __builtin_fmaf((float)s[q], x.sa, x.lo);
        y = x.ahat;
      } else {
        y = __builtin_fmaf((float)((int32_t)s[q] - x.M), x.dl, x.ahat);
      }
      v[q] = f2h(y);
    }
  }
}

template <bool kSymbols>
__device__ inline void put(gbyte *base, uint32_t lane, uint32_t v) {
  if constexpr (kSymbols)
    base[lane] = (uint8_t)v;
  else
    ((__attribute__((address_space(1))) uint16_t *)base)[lane] = (uint16_t)v;
}

// Wave-uniform 64-bit pointer (kept in scalar registers).
__device__ inline gbyte *uniform_ptr(gbyte *p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (gbyte *)(((uint64_t)hi << 32) | lo);
}

// The delta tokens of one group (tokens j+1 .. jend-1) of both streams.
template <bool kSymbols, uint32_t kSteps>
__device__ inline void delta_run(Stream *st, lds_cu16 *ta, lds_cu16 *const *td,
                                 const __amdgpu_buffer_rsrc_t *src, gbyte **ob, uint64_t ld,
                                 uint32_t lane, uint32_t count) {
  for (uint32_t i = 0; i < count; ++i) {
    uint32_t v[2];
    step<2, kSymbols, false, kSteps>(st, ta, td, src, v);
    put<kSymbols>(ob[0], lane, v[0]);
    put<kSymbols>(ob[1], lane, v[1]);
    ob[0] += ld;
    ob[1] += ld;
  }
}

template <bool kSymbols>
__device__ inline void delta_dispatch(uint32_t steps, Stream *st, lds_cu16 *ta,
                                      lds_cu16 *const *td, const __amdgpu_buffer_rsrc_t *src,
                                      gbyte **ob, uint64_t ld, uint32_t lane, uint32_t count) {
  switch (steps) {
    case 2: delta_run<kSymbols, 2>(st, ta, td, src, ob, ld, lane, count); break;
    case 3: delta_run<kSymbols, 3>(st, ta, td, src, ob, ld, lane, count); break;
    case 4: delta_run<kSymbols, 4>(st, ta, td, src, ob, ld, lane, count); break;
    case 5: delta_run<kSymbols, 5>(st, ta, td, src, ob, ld, lane, count); break;
    default: delta_run<kSymbols, 6>(st, ta, td, src, ob, ld, lane, count); break;
  }
}

template <bool kSymbols>
__device__ inline void single_step(uint32_t steps, bool anchor, Stream *st, lds_cu16 *ta,
                                   lds_cu16 *const *td, const __amdgpu_buffer_rsrc_t *src,
                                   uint32_t *v) {
  if (anchor) {
    step<1, kSymbols, true, 8>(st, ta, td, src, v);
    return;
  }
  switch (steps) {
    case 2: step<1, kSymbols, false, 2>(st, ta, td, src, v); break;
    case 3: step<1, kSymbols, false, 3>(st, ta, td, src, v); break;
    case 4: step<1, kSymbols, false, 4>(st, ta, td, src, v); break;
    case 5: step<1, kSymbols, false, 5>(st, ta, td, src, v); break;
    default: step<1, kSymbols, false, 6>(st, ta, td, src, v); break;
  }
}

}  // namespace

template <bool kSymbols>
__global__ __launch_bounds__(kMaxWaves *kWave) void k_decode(
    Desc d, const ChunkInfo *__restrict__ ci, const DecodeGroup *__restrict__ groups,
    uint32_t n_groups, uint32_t n_units, const uint8_t *__restrict__ valid,
    const uint32_t *__restrict__ offsets, const uint8_t *__restrict__ tables,
    void *__restrict__ out, uint32_t T_total, int32_t *status) {
  // ---- which (unit, chunk group) this block owns (XCD-aware numbering)
  const uint32_t id = blockIdx.x;
  const uint32_t local = id / kXcds;
  const uint32_t unit = (local / n_groups) * kXcds + id % kXcds;
  const uint32_t grp = local % n_groups;
  if (unit >= n_units) return;
  const uint32_t ncb = (d.C + kWave - 1) / kWave;
  const uint32_t row = unit / ncb, cb = unit % ncb;
  const uint32_t c0 = cb * kWave;
  const uint32_t nv = d.C - c0 < kWave ? d.C - c0 : kWave;
  const uint32_t m0 = row * d.C + c0;
  const uint32_t S = n_streams(d);
  const DecodeGroup gp = groups[grp];
  const uint32_t level_mask = gp.level;  // bit l: the group has chunks of level l
  const uint32_t nlev_used = __builtin_popcount(level_mask);
  const uint32_t n_waves = blockDim.x / kWave;

  extern __shared__ uint32_t lds_raw[];
  lds_u32 *lds = (lds_u32 *)lds_raw;
  lds_u32 *sA = lds;                                // [64][kAStride] anchor cum
  lds_u32 *sD = sA + kWave * kAStride;              // [levels used][64][kDStride] delta cum
  lds_u32 *sR = sD + nlev_used * kWave * kDStride;  // [waves][kSlots][64][kRing] rings

  // ---- stage the 64 channels' anchor models and the used levels' delta models
  const uint32_t tid = threadIdx.x;
  {
    const uint32_t *gA = reinterpret_cast<const uint32_t *>(tables + kTablesHdr) +
                         (uint64_t)m0 * (kAnchorStride / 2);
    for (uint32_t i = tid; i < nv * kAStride; i += blockDim.x) {
      const uint32_t mm = i / kAStride, w = i % kAStride;
      sA[i] = gA[(uint64_t)mm * (kAnchorStride / 2) + w];
    }
    uint32_t slot = 0;
    for (uint32_t lv = 0; lv < d.nlev; ++lv) {
      if (!((level_mask >> lv) & 1u)) continue;
      const uint32_t *gD = reinterpret_cast<const uint32_t *>(
                               tables + kTablesHdr + (uint64_t)S * kAnchorStride * 2) +
                           ((uint64_t)lv * S + m0) * (kDeltaStride / 2);
      lds_u32 *dst = sD + slot * kWave * kDStride;
      for (uint32_t i = tid; i < nv * kDStride; i += blockDim.x) {
        const uint32_t mm = i / kDStride, w = i % kDStride;
        const uint32_t v =
            w < kDeltaStride / 2 ? gD[(uint64_t)mm * (kDeltaStride / 2) + w] : 0xFFFFFFFFu;
        // entries past cum[A] (0xFFFF in the blob) become 0x8000 + index:
        // above any valid target and strictly increasing, so even a corrupt
        // stream's search never yields an empty interval
        uint32_t lo16 = v & 0xFFFFu, hi16 = v >> 16;
        lo16 = lo16 == 0xFFFFu ? 0x8000u + 2 * w : lo16;
        hi16 = hi16 == 0xFFFFu ? 0x8001u + 2 * w : hi16;
        dst[i] = lo16 | (hi16 << 16);
      }
      ++slot;
    }
  }
  __syncthreads();
  const uint32_t lane = tid % kWave;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  if (lane >= nv) return;

  lds_cu16 *ta = (lds_cu16 *)(sA + lane * kAStride);
  const uint32_t third = third_of(row >> 1, d.L);
  const uint32_t esz = kSymbols ? 1u : 2u;
  const uint64_t ld = (uint64_t)d.C * esz;
  const uint32_t m = m0 + lane;
  const uint32_t npairs = (gp.count + 1) / 2;

  for (uint32_t pair = wave; pair < npairs; pair += n_waves) {
    lds_cu16 *td[kSlots];
    Stream st[kSlots];
    gbyte *ob[kSlots];  // wave-uniform output row of the current token
    __amdgpu_buffer_rsrc_t src[kSlots];
    uint32_t steps = 2;
    bool active[kSlots];
#pragma unroll
    for (uint32_t q = 0; q < kSlots; ++q) {
      Stream &s = st[q];
      const uint32_t idx = 2 * pair + q;
      const uint32_t k = gp.start + (idx < gp.count ? idx : 0u);
      active[q] = idx < gp.count && valid[k];
      s.n = 0;
      s.tor = 0;
      s.ring = sR + ((wave * kSlots + q) * kWave + lane) * kRing;
      ob[q] = (gbyte *)out;
      td[q] = (lds_cu16 *)(sD + lane * kDStride);
      src[q] = __builtin_amdgcn_make_buffer_rsrc((void *)ci[k].cont, (short)0, 0, kBufferWord3);
      if (!active[q]) continue;
      const ChunkInfo c = ci[k];
      const uint32_t lslot = __builtin_popcount(level_mask & ((1u << c.level) - 1u));
      td[q] = (lds_cu16 *)(sD + (lslot * kWave + lane) * kDStride);
      const uint32_t b = d.bits[c.level][third];
      steps = b > steps ? b : steps;
      s.M = (1 << (b - 1)) - 1;
      const uint32_t *rec = reinterpret_cast<const uint32_t *>(c.records + (uint64_t)m * kRecBytes);
      s.lo = __builtin_bit_cast(float, rec[0]);
      s.sa = __builtin_bit_cast(float, rec[1]);
      s.dl = __builtin_bit_cast(float, rec[2]);
      s.nbytes = rec[3];
      s.voff = (uint32_t)(kHdrBytes + (uint64_t)kRecBytes * S) + offsets[(uint64_t)k * S + m];
      s.n = c.n_tokens;
      // containers are below 2^32 bytes (checked on the host)
      src[q] = __builtin_amdgcn_make_buffer_rsrc((void *)c.cont, (short)0,
                                                 (int)(uint32_t)c.cont_bytes, kBufferWord3);
      ob[q] = uniform_ptr((gbyte *)out + (((uint64_t)row * T_total + c.first_token) * d.C + c0) * esz);
      s.ahat = 0.0f;
      // prime the ring with 16 bytes and start loading the next 8
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(src[q], s.voff, 0, 0);
      s.ring[0] = v[0];
      s.ring[1] = v[1];
      s.ring[2] = v[2];
      s.ring[3] = v[3];
      s.ring[4] = v[0];
      s.wpos = 16;
      s.load_block(src[q]);
      s.code = bswap32(v[0]);
      s.rpos = 4;
      s.range = 0xFFFFFFFFu;
    }
    steps = __builtin_amdgcn_readfirstlane(steps);

    // Both streams live: one lockstep step per token, so the two dependency
    // chains interleave; only the rare ring refills branch.
    const uint32_t nmin = st[0].n < st[1].n ? st[0].n : st[1].n;
    const uint32_t nmax = st[0].n > st[1].n ? st[0].n : st[1].n;
    uint32_t j = 0;
    while (j < nmin) {
      st[0].maintain(src[0]);
      st[1].maintain(src[1]);
      {
        uint32_t v[2];
        step<2, kSymbols, true, 8>(st, ta, td, src, v);
        put<kSymbols>(ob[0], lane, v[0]);
        put<kSymbols>(ob[1], lane, v[1]);
        ob[0] += ld;
        ob[1] += ld;
      }
      const uint32_t jend = j + d.G < nmin ? j + d.G : nmin;
      delta_dispatch<kSymbols>(steps, st, ta, td, src, ob, ld, lane, jend - j - 1);
      j = jend;
    }
    // Tail: one stream left (odd chunk count, or a shorter last chunk).
    uint32_t g = nmin % d.G;
    for (; j < nmax; ++j) {
      const bool anchor = g == 0;
      g = g + 1 == d.G ? 0 : g + 1;
#pragma unroll
      for (uint32_t q = 0; q < kSlots; ++q) {
        if (j < st[q].n) {
          if (anchor) st[q].maintain(src[q]);
          uint32_t v;
          single_step<kSymbols>(steps, anchor, &st[q], ta, &td[q], &src[q], &v);
          put<kSymbols>(ob[q], lane, v);
          ob[q] += ld;
        }
      }
    }
#pragma unroll
    for (uint32_t q = 0; q < kSlots; ++q)
      if (active[q] && ((st[q].tor >> kPrec) != 0 || st[q].rpos != st[q].nbytes))
        set_status(status, KVC_ERR_CORRUPT_STREAM);
  }
}

size_t decode_lds_bytes(uint32_t levels, uint32_t waves) {
  return sizeof(uint32_t) * ((size_t)kWave * kAStride + (size_t)levels * kWave * kDStride +
                             (size_t)waves * kSlots * kWave * kRing);
}

hipError_t launch_decode(const Desc &d, const ChunkInfo *dev_chunks, const DecodeGroup *groups,
                         uint32_t n_groups, uint32_t levels, uint32_t waves, const uint8_t *valid,
                         const uint32_t *offsets, const uint8_t *tables, void *out,
                         uint32_t T_total, bool symbols, int32_t *status, hipStream_t stream) {
  const uint32_t ncb = (d.C + kWave - 1) / kWave;
  const uint32_t n_units = 2u * d.L * ncb;
  const uint64_t blocks = (uint64_t)((n_units + kXcds - 1) / kXcds) * kXcds * n_groups;
  const size_t lds = decode_lds_bytes(levels, waves);
  if (symbols)
    hipLaunchKernelGGL(k_decode<true>, dim3((uint32_t)blocks), dim3(waves * kWave), lds, stream,
                       d, dev_chunks, groups, n_groups, n_units, valid, offsets, tables, out,
                       T_total, status);
  else
    hipLaunchKernelGGL(k_decode<false>, dim3((uint32_t)blocks), dim3(waves * kWave), lds, stream,
                       d, dev_chunks, groups, n_groups, n_units, valid, offsets, tables, out,
                       T_total, status);
  return hipGetLastError();
}

}  // namespace kvc
