// Fused decode: range decode -> dequantize / anchor+delta reconstruction ->
// store into the [layer][K/V][token][channel] binary16 KV cache.
//
// CacheGen page, 核心方法: each chunk's bitstream is decoded on the GPU back
// to tensors; tokens of a 10-token group depend only on their anchor (no
// delta chain); symbols were arithmetic-coded against per channel-layer
// models, anchors and deltas separately.
//
// Work decomposition (gfx950, wave64):
//  * the call's chunks are split into groups of up to 8; a workgroup owns
//    one (layer*2+kv row, block of 64 channels) and one group, and stages the
//    64 channels' anchor models and their delta models of every level the
//    group uses.  It has 4 waves, and every lane of wave w decodes the
//    streams of its channel in two chunks of the group (slots 2w, 2w+1) in
//    lockstep, so one LDS copy of the 64 channels' models serves 8 streams
//    and each lane runs two independent dependency chains;
//  * all lanes of a wave are at the same token, so the anchor/delta switch
//    is wave-uniform and the 64 results of a token are 64 consecutive
//    channels: one coalesced 128-byte store per stream, addressed from a
//    wave-uniform (scalar) base;
//  * symbols are found by binary search of the cumulative tables (8 steps
//    for anchors, 6 for deltas), the two streams' probes interleaved;
//  * stream bytes are staged per lane in a 32-byte LDS ring: at every group
//    boundary a lane writes the 16 bytes it loaded at the previous boundary
//    and issues the next load, so global-memory latency is off the
//    per-symbol path; a rare slow path refills a ring that runs low;
//  * LDS rows use odd dword strides so that lanes reading the same entry
//    index of their own tables hit different banks;
//  * blocks are numbered so that the groups of one (row, channel block) run
//    on the same XCD back to back and share its L2.
#include "kvc_internal.h"

namespace kvc {

namespace {

constexpr uint32_t kWaves = 4;          // waves per workgroup
constexpr uint32_t kSlots = 2;          // streams per lane
constexpr uint32_t kAStride = 129;      // dwords per staged anchor model (cum[0..256] + pad)
constexpr uint32_t kDStride = 33;       // dwords per staged delta model (cum[0..63] + pad)
constexpr uint32_t kRing = 9;           // dwords per lane ring: 32 bytes + mirror of bytes 0..3
constexpr uint32_t kXcds = 8;

// Global-memory view of the stream words: loads through it are plain
// global_load instructions, which count only against the vector-memory
// counter, so waiting for an LDS result never waits for a prefetch.
typedef __attribute__((address_space(1))) const uint32_t gword;
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
  const gword *src;     // the stream's words in the container
  lds_u32 *ring;        // this lane's ring in LDS (32 bytes + 4 mirrored)
  uint32_t code, range;
  uint32_t rpos;        // bytes consumed
  uint32_t wpos;        // bytes written to the ring (a multiple of 16)
  uint32_t wlast;       // index of the stream's last readable word
  uint32_t nbytes;
  uint32_t p0, p1, p2, p3;  // the 16 bytes at wpos, loaded ahead (memory order)
  uint32_t n;
  int32_t M;
  float lo, sa, dl, ahat;
  bool active;
  bool bad;

  // Load the 16 bytes at wpos.  The word index is clamped to the stream's
  // last word instead of being guarded, so the load is unconditional and
  // nothing waits for it before the bytes are stored into the ring; bytes
  // past the end of a stream are never consumed by a valid stream.
  __device__ inline void load_block() {
    const uint32_t w = wpos >> 2;
    p0 = src[min(w, wlast)];
    p1 = src[min(w + 1, wlast)];
    p2 = src[min(w + 2, wlast)];
    p3 = src[min(w + 3, wlast)];
  }
  __device__ inline void write_block() {  // p0..p3 into the free ring slot
    const uint32_t slot = (wpos >> 2) & 7;  // 0 or 4
    ring[slot] = p0;
    ring[slot + 1] = p1;
    ring[slot + 2] = p2;
    ring[slot + 3] = p3;
    if (slot == 0) ring[8] = p0;
    wpos += 16;
  }
  // At a group boundary: store the block loaded at the previous boundary if
  // its slot is free, then load the block that follows the ring's contents.
  __device__ inline void maintain() {
    if (wpos - rpos <= 16) write_block();
    load_block();
  }
  // Make sure the next symbol's (at most 2) bytes are in the ring (rare).
  __device__ inline void ensure() {
    if (__builtin_expect(wpos - rpos < 2, 0)) {
      write_block();
      load_block();
    }
  }
};

// One token of Q streams of a lane, in lockstep: range decode, dequantize.
// Writes the value to store (binary16 bits, or the symbol) to v[q].
template <uint32_t Q, bool kSymbols, bool kAnchor>
__device__ inline void step(Stream *st, lds_cu16 *ta, lds_cu16 *const *td, uint32_t *v) {
  uint32_t r[Q], t[Q], s[Q], cs[Q], cn[Q];
#pragma unroll
  for (uint32_t q = 0; q < Q; ++q) {
    r[q] = st[q].range >> kPrec;
    t[q] = quotient(st[q].code, r[q]);
    if (t[q] >= kTot) {
      st[q].bad = true;
      t[q] = kTot - 1;
    }
  }
  // binary search of the cumulative table, the streams' probes interleaved
  constexpr uint32_t kTop = kAnchor ? 128u : 32u;
  lds_cu16 *p[Q];
#pragma unroll
  for (uint32_t q = 0; q < Q; ++q) p[q] = kAnchor ? ta : td[q];
  lds_cu16 *base[Q];
#pragma unroll
  for (uint32_t q = 0; q < Q; ++q) base[q] = p[q];
#pragma unroll
  for (uint32_t step = kTop; step; step >>= 1) {
    uint32_t probe[Q];
#pragma unroll
    for (uint32_t q = 0; q < Q; ++q) probe[q] = p[q][step];
#pragma unroll
    for (uint32_t q = 0; q < Q; ++q)
      if (probe[q] <= t[q]) p[q] += step;
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
    lds_cu8 *rb = (lds_cu8 *)st[q].ring + (st[q].rpos & 31);
    in[q] = ((uint32_t)rb[0] << 8) | rb[1];  // the next two stream bytes
  }
#pragma unroll
  for (uint32_t q = 0; q < Q; ++q) {
    Stream &x = st[q];
    // 24-bit multiplies: r < 2^17 and cumulative counts <= 2^16
    x.code -= __umul24(r[q], cs[q]);
    const uint32_t range = __umul24(r[q], cn[q] - cs[q]);
    // whole bytes to shift in: 0, 1 or 2 (range >= 2^9 with valid tables)
    const uint32_t k = (uint32_t)__builtin_clz(range | 1u) >> 3;
    const uint32_t sh = k << 3;
    x.range = range << sh;
    x.code = (x.code << sh) | (in[q] >> ((16 - sh) & 31));
    x.rpos += k;
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

}  // namespace

template <bool kSymbols>
__global__ __launch_bounds__(kWaves *kWave) void k_decode(
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

  extern __shared__ uint32_t lds_raw[];
  lds_u32 *lds = (lds_u32 *)lds_raw;
  lds_u32 *sA = lds;                                // [64][kAStride] anchor cum
  lds_u32 *sD = sA + kWave * kAStride;              // [levels used][64][kDStride] delta cum
  lds_u32 *sR = sD + nlev_used * kWave * kDStride;  // [kWaves*kSlots][64][kRing] rings

  // ---- stage the 64 channels' anchor models and this level's delta models
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
        dst[i] = w < kDeltaStride / 2 ? gD[(uint64_t)mm * (kDeltaStride / 2) + w] : 0xFFFFFFFFu;
      }
      ++slot;
    }
  }
  __syncthreads();
  const uint32_t lane = tid % kWave;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  if (lane >= nv) return;
  (void)nlev_used;

  lds_cu16 *ta = (lds_cu16 *)(sA + lane * kAStride);
  const uint32_t third = third_of(row >> 1, d.L);
  const uint32_t esz = kSymbols ? 1u : 2u;
  lds_cu16 *td[kSlots];
  Stream st[kSlots];
  gbyte *ob[kSlots];  // wave-uniform output row of the current token
  uint32_t nmax = 0;
#pragma unroll
  for (uint32_t q = 0; q < kSlots; ++q) {
    Stream &s = st[q];
    const uint32_t slot = wave * kSlots + q;
    const uint32_t k = slot < gp.count ? gp.chunk[slot] : 0u;
    s.active = slot < gp.count && valid[k];
    s.bad = false;
    s.n = 0;
    s.ring = sR + ((wave * kSlots + q) * kWave + lane) * kRing;
    ob[q] = (gbyte *)out;
    td[q] = (lds_cu16 *)(sD + lane * kDStride);
    if (!s.active) continue;
    const ChunkInfo c = ci[k];
    const uint32_t lslot = __builtin_popcount(level_mask & ((1u << c.level) - 1u));
    td[q] = (lds_cu16 *)(sD + (lslot * kWave + lane) * kDStride);
    s.M = (1 << (d.bits[c.level][third] - 1)) - 1;
    const uint32_t m = m0 + lane;
    const uint32_t *rec = reinterpret_cast<const uint32_t *>(c.records + (uint64_t)m * kRecBytes);
    s.lo = __builtin_bit_cast(float, rec[0]);
    s.sa = __builtin_bit_cast(float, rec[1]);
    s.dl = __builtin_bit_cast(float, rec[2]);
    s.nbytes = rec[3];
    s.src = (const gword *)(c.cont + kHdrBytes + (uint64_t)kRecBytes * S +
                            offsets[(uint64_t)k * S + m]);
    s.wlast = (uint32_t)(pad4(s.nbytes) >> 2) - 1;  // nbytes >= 4 in a valid chunk
    s.n = c.n_tokens;
    ob[q] = (gbyte *)out + (((uint64_t)row * T_total + c.first_token) * d.C + c0) * esz;
    s.ahat = 0.0f;
    // prime the ring with 32 bytes and start loading the next 16
    s.wpos = 0;
    s.load_block();
    s.write_block();
    s.load_block();
    s.write_block();
    s.load_block();
    s.code = bswap32(s.ring[0]);
    s.rpos = 4;
    s.range = 0xFFFFFFFFu;
    nmax = s.n > nmax ? s.n : nmax;
  }

  const uint64_t ld = (uint64_t)d.C * esz;
  // Both streams live: one lockstep step per token, so the two dependency
  // chains interleave; only the rare ring refills branch.
  const uint32_t nmin = st[0].n < st[1].n ? st[0].n : st[1].n;
  uint32_t j = 0;
  while (j < nmin) {
    st[0].maintain();
    st[1].maintain();
    st[0].ensure();
    st[1].ensure();
    {
      uint32_t v[2];
      step<2, kSymbols, true>(st, ta, td, v);
      put<kSymbols>(ob[0], lane, v[0]);
      put<kSymbols>(ob[1], lane, v[1]);
      ob[0] += ld;
      ob[1] += ld;
    }
    const uint32_t jend = j + d.G < nmin ? j + d.G : nmin;
    for (++j; j < jend; ++j) {
      st[0].ensure();
      st[1].ensure();
      uint32_t v[2];
      step<2, kSymbols, false>(st, ta, td, v);
      put<kSymbols>(ob[0], lane, v[0]);
      put<kSymbols>(ob[1], lane, v[1]);
      ob[0] += ld;
      ob[1] += ld;
    }
  }
  // Tail: one stream left (odd chunk count, or a shorter last chunk).
  uint32_t g = nmin % d.G;
  for (; j < nmax; ++j) {
    const bool anchor = g == 0;
    g = g + 1 == d.G ? 0 : g + 1;
#pragma unroll
    for (uint32_t q = 0; q < kSlots; ++q) {
      if (j < st[q].n) {
        if (anchor) st[q].maintain();
        st[q].ensure();
        uint32_t v;
        if (anchor)
          step<1, kSymbols, true>(&st[q], ta, &td[q], &v);
        else
          step<1, kSymbols, false>(&st[q], ta, &td[q], &v);
        put<kSymbols>(ob[q], lane, v);
        ob[q] += ld;
      }
    }
  }
#pragma unroll
  for (uint32_t q = 0; q < kSlots; ++q)
    if (st[q].active && (st[q].bad || st[q].rpos != st[q].nbytes))
      set_status(status, KVC_ERR_CORRUPT_STREAM);
}

size_t decode_lds_bytes(uint32_t max_levels) {
  return sizeof(uint32_t) * ((size_t)kWave * kAStride + (size_t)max_levels * kWave * kDStride +
                             (size_t)kWaves * kSlots * kWave * kRing);
}

hipError_t launch_decode(const Desc &d, const ChunkInfo *dev_chunks, const DecodeGroup *groups,
                         uint32_t n_groups, uint32_t max_levels_hint, const uint8_t *valid,
                         const uint32_t *offsets, const uint8_t *tables, void *out,
                         uint32_t T_total, bool symbols, int32_t *status, hipStream_t stream) {
  const uint32_t ncb = (d.C + kWave - 1) / kWave;
  const uint32_t n_units = 2u * d.L * ncb;
  const uint64_t blocks = (uint64_t)((n_units + kXcds - 1) / kXcds) * kXcds * n_groups;
  // LDS for the group that uses the most levels (the host's count)
  const size_t lds = decode_lds_bytes(max_levels_hint);
  if (symbols)
    hipLaunchKernelGGL(k_decode<true>, dim3((uint32_t)blocks), dim3(kWaves * kWave), lds, stream,
                       d, dev_chunks, groups, n_groups, n_units, valid, offsets, tables, out,
                       T_total, status);
  else
    hipLaunchKernelGGL(k_decode<false>, dim3((uint32_t)blocks), dim3(kWaves * kWave), lds, stream,
                       d, dev_chunks, groups, n_groups, n_units, valid, offsets, tables, out,
                       T_total, status);
  return hipGetLastError();
}

}  // namespace kvc
