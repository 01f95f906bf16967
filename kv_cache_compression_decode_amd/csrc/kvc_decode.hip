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
//    of up to 8 chunks of the call; it has 4 waves, and every lane of wave w
//    decodes the streams of its channel in two chunks (slots 2w and 2w+1) in
//    lockstep, so one LDS copy of the 64 channels' models serves 8 streams
//    and each lane has two independent dependency chains;
//  * all lanes of a wave are at the same token, so the anchor/delta model
//    switch is wave-uniform and the 64 lanes' binary16 results for a token
//    are 64 consecutive channels: one coalesced 128-byte store per stream;
//  * stream bytes are staged per lane in a 32-byte LDS ring: at every group
//    boundary (every 10 tokens) a lane writes the 16 bytes it loaded at the
//    previous boundary and issues the next load, so global-memory latency is
//    off the per-symbol path; a rare slow path refills a ring that runs low
//    inside a group;
//  * model tables use odd dword strides so that lanes reading the same entry
//    index of their own tables hit different LDS banks;
//  * blocks are numbered so that the chunk groups of one (row, channel
//    block) run on the same XCD back to back and share its L2.
#include "kvc_internal.h"

namespace kvc {

namespace {

constexpr uint32_t kWaves = 4;          // waves per workgroup
constexpr uint32_t kSlots = 2;          // streams per lane
constexpr uint32_t kGroupChunks = kWaves * kSlots;
constexpr uint32_t kAStride = 129;      // dwords per staged anchor model (cum[0..256] + pad)
constexpr uint32_t kDStride = 33;       // dwords per staged delta model (cum[0..63] + pad)
constexpr uint32_t kRing = 9;           // dwords per lane ring: 8 + mirror of dword 0
constexpr uint32_t kXcds = 8;

// t = floor(code / r) for r in [2^9, 2^17), exact for t <= 2^15 and
// clamped to at most 2^15 + 1 otherwise (the caller rejects t >= 2^15).
__device__ inline uint32_t quotient(uint32_t code, uint32_t r) {
  const float fr = (float)r;
  const float fc = (float)code;
  uint32_t q = (uint32_t)(fc * __builtin_amdgcn_rcpf(fr));
  q = q > kTot ? kTot : q;
  const uint32_t p = q * r;  // < 2^32
  if (p > code) {
    q -= 1;
  } else if (code - p >= r) {
    q += 1;
  }
  return q;
}

// Global-memory view of the stream words: loads through it are plain
// global_load instructions, which count only against the vector-memory
// counter, so waiting for an LDS result never waits for a prefetch.
typedef __attribute__((address_space(1))) const uint32_t gword;

struct Stream {
  const gword *src;     // the stream's words in the container
  uint32_t *ring;       // this lane's ring in LDS
  const uint16_t *td;   // delta model of this stream's level (LDS)
  uint64_t o;           // output element index of the current token
  uint32_t code, range;
  uint32_t rpos;        // bytes consumed
  uint32_t wpos;        // bytes written to the ring (a multiple of 16)
  uint32_t wlast;       // index of the stream's last readable word
  uint32_t nbytes;
  uint32_t p0, p1, p2, p3;  // the 16 bytes at wpos, loaded ahead (memory order)
  bool active;          // this slot has a valid chunk
  bool bad;
  uint32_t n;
  int32_t M;
  float lo, sa, dl, ahat;

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
  // p0..p3 into the free ring slot, as big-endian words (the first byte of
  // the stream is the most significant byte of the decoder's code).
  __device__ inline void write_block() {
    const uint32_t slot = (wpos >> 2) & 7;  // 0 or 4
    const uint32_t b0 = bswap32(p0);
    ring[slot] = b0;
    ring[slot + 1] = bswap32(p1);
    ring[slot + 2] = bswap32(p2);
    ring[slot + 3] = bswap32(p3);
    if (slot == 0) ring[8] = b0;
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
  __device__ inline uint32_t peek4() const {  // 4 bytes at rpos, big-endian
    const uint32_t i = (rpos >> 2) & 7;
    const uint64_t w = ((uint64_t)ring[i] << 32) | ring[i + 1];
    return (uint32_t)((w << ((rpos & 3) * 8)) >> 32);
  }
};

template <uint32_t kSteps>
__device__ inline uint32_t search(const uint16_t *tab, uint32_t t) {
  uint32_t s = 0;
#pragma unroll
  for (uint32_t step = 1u << (kSteps - 1); step; step >>= 1)
    if (tab[s + step] <= t) s += step;
  return s;
}

// One symbol of one stream: range decode, dequantize, store.
template <bool kSymbols, bool anchor>
__device__ inline void step(Stream &st, const uint16_t *ta, void *out) {
  const uint32_t r = st.range >> kPrec;
  uint32_t t = quotient(st.code, r);
  if (t >= kTot) {
    st.bad = true;
    t = kTot - 1;
  }
  const uint16_t *tab = anchor ? ta : st.td;
  const uint32_t s = anchor ? search<8>(ta, t) : search<6>(st.td, t);
  const uint32_t cs = tab[s];
  uint32_t f = (uint32_t)tab[s + 1] - cs;
  if (f == 0 || f > kTot) {  // only with damaged tables
    st.bad = true;
    f = 1;
  }
  st.code -= r * cs;
  uint32_t range = r * f;
  if (range < 512u) {  // impossible with valid tables; keeps the shift bounded
    st.bad = true;
    range = 1u << 24;
  }
  const uint32_t sh = (uint32_t)__builtin_clz(range) & 24u;  // 0, 8 or 16 bits to shift in
  st.range = range << sh;
  const uint32_t in = st.peek4();
  st.code = (uint32_t)(((((uint64_t)st.code) << 32) | in) << sh >> 32);
  st.rpos += sh >> 3;
  if constexpr (kSymbols) {
    static_cast<uint8_t *>(out)[st.o] = (uint8_t)s;
  } else {
    float v;
    if constexpr (anchor) {
      st.ahat = __builtin_fmaf((float)s, st.sa, st.lo);
      v = st.ahat;
    } else {
      v = __builtin_fmaf((float)((int32_t)s - st.M), st.dl, st.ahat);
    }
    static_cast<uint16_t *>(out)[st.o] = f2h(v);
  }
}

}  // namespace

template <bool kSymbols>
__global__ __launch_bounds__(kWaves *kWave) void k_decode(
    Desc d, const ChunkInfo *__restrict__ ci, uint32_t n_chunks, uint32_t n_groups,
    uint32_t n_units, uint32_t level_mask, const uint8_t *__restrict__ valid,
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
  const uint32_t k_begin = (uint32_t)(((uint64_t)grp * n_chunks) / n_groups);
  const uint32_t k_end = (uint32_t)(((uint64_t)(grp + 1) * n_chunks) / n_groups);

  extern __shared__ uint32_t lds[];
  uint32_t *sA = lds;                               // [64][kAStride]
  uint32_t *sD = sA + kWave * kAStride;             // [levels used][64][kDStride]
  const uint32_t nslots = __builtin_popcount(level_mask);
  uint32_t *sR = sD + nslots * kWave * kDStride;    // [kWaves*kSlots][64][kRing]

  // ---- stage the 64 channels' models (anchor + every level used)
  const uint32_t tid = threadIdx.x;
  {
    const uint32_t *gA = reinterpret_cast<const uint32_t *>(tables + kTablesHdr) +
                         (uint64_t)m0 * (kAnchorStride / 2);
    for (uint32_t i = tid; i < nv * kAStride; i += blockDim.x) {
      const uint32_t mm = i / kAStride, w = i % kAStride;
      sA[i] = gA[(uint64_t)mm * (kAnchorStride / 2) + w];
    }
    const uint32_t *gD = reinterpret_cast<const uint32_t *>(
        tables + kTablesHdr + (uint64_t)S * kAnchorStride * 2);
    uint32_t slot = 0;
    for (uint32_t lv = 0; lv < d.nlev; ++lv) {
      if (!((level_mask >> lv) & 1u)) continue;
      const uint32_t *src = gD + ((uint64_t)lv * S + m0) * (kDeltaStride / 2);
      uint32_t *dst = sD + slot * kWave * kDStride;
      for (uint32_t i = tid; i < nv * kDStride; i += blockDim.x) {
        const uint32_t mm = i / kDStride, w = i % kDStride;
        dst[i] = w < kDeltaStride / 2 ? src[(uint64_t)mm * (kDeltaStride / 2) + w] : 0xFFFFFFFFu;
      }
      ++slot;
    }
  }
  __syncthreads();
  const uint32_t wave = tid / kWave, lane = tid % kWave;
  if (lane >= nv) return;

  const uint16_t *ta = reinterpret_cast<const uint16_t *>(sA + lane * kAStride);
  const uint32_t third = third_of(row >> 1, d.L);
  Stream st[kSlots];
  uint32_t nmax = 0;
#pragma unroll
  for (uint32_t q = 0; q < kSlots; ++q) {
    Stream &s = st[q];
    const uint32_t k = k_begin + wave * kSlots + q;
    s.active = k < k_end && valid[k];
    s.bad = false;
    s.n = 0;
    s.ring = sR + ((wave * kSlots + q) * kWave + lane) * kRing;
    if (!s.active) continue;
    const ChunkInfo c = ci[k];
    const uint32_t lslot = __builtin_popcount(level_mask & ((1u << c.level) - 1u));
    s.td = reinterpret_cast<const uint16_t *>(sD + (lslot * kWave + lane) * kDStride);
    const uint32_t b = d.bits[c.level][third];
    s.M = (1 << (b - 1)) - 1;
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
    s.o = ((uint64_t)row * T_total + c.first_token) * d.C + c0 + lane;
    s.ahat = 0.0f;
    // prime the ring with 32 bytes and start loading the next 16
    s.wpos = 0;
    s.load_block();
    s.write_block();
    s.load_block();
    s.write_block();
    s.load_block();
    s.code = s.ring[0];
    s.rpos = 4;
    s.range = 0xFFFFFFFFu;
    nmax = s.n > nmax ? s.n : nmax;
  }

  const uint64_t ld = d.C;
  for (uint32_t j0 = 0; j0 < nmax; j0 += d.G) {
    // group boundary: ring upkeep, then the anchor token
#pragma unroll
    for (uint32_t q = 0; q < kSlots; ++q) {
      Stream &s = st[q];
      if (j0 < s.n) {
        s.maintain();
        s.ensure();
        step<kSymbols, true>(s, ta, out);
        s.o += ld;
      }
    }
    const uint32_t jend = j0 + d.G < nmax ? j0 + d.G : nmax;
    for (uint32_t j = j0 + 1; j < jend; ++j) {
#pragma unroll
      for (uint32_t q = 0; q < kSlots; ++q) {
        Stream &s = st[q];
        if (j < s.n) {
          s.ensure();
          step<kSymbols, false>(s, ta, out);
          s.o += ld;
        }
      }
    }
  }
#pragma unroll
  for (uint32_t q = 0; q < kSlots; ++q)
    if (st[q].active && (st[q].bad || st[q].rpos != st[q].nbytes))
      set_status(status, KVC_ERR_CORRUPT_STREAM);
}

size_t decode_lds_bytes(uint32_t level_mask) {
  return sizeof(uint32_t) * ((size_t)kWave * kAStride +
                             (size_t)__builtin_popcount(level_mask) * kWave * kDStride +
                             (size_t)kGroupChunks * kWave * kRing);
}

hipError_t launch_decode(const Desc &d, const ChunkInfo *dev_chunks, uint32_t n_chunks,
                         uint32_t level_mask, const uint8_t *valid, const uint32_t *offsets,
                         const uint8_t *tables, void *out, uint32_t T_total, bool symbols,
                         int32_t *status, hipStream_t stream) {
  const uint32_t ncb = (d.C + kWave - 1) / kWave;
  const uint32_t n_units = 2u * d.L * ncb;
  const uint32_t n_groups = (n_chunks + kGroupChunks - 1) / kGroupChunks;
  const uint64_t blocks = (uint64_t)((n_units + kXcds - 1) / kXcds) * kXcds * n_groups;
  const size_t lds = decode_lds_bytes(level_mask);
  if (symbols)
    hipLaunchKernelGGL(k_decode<true>, dim3((uint32_t)blocks), dim3(kWaves * kWave), lds, stream,
                       d, dev_chunks, n_chunks, n_groups, n_units, level_mask, valid, offsets,
                       tables, out, T_total, status);
  else
    hipLaunchKernelGGL(k_decode<false>, dim3((uint32_t)blocks), dim3(kWaves * kWave), lds, stream,
                       d, dev_chunks, n_chunks, n_groups, n_units, level_mask, valid, offsets,
                       tables, out, T_total, status);
  return hipGetLastError();
}

}  // namespace kvc
