// Fused decode: range decode -> dequantize / anchor+delta reconstruction ->
// store into the [layer][K/V][token][channel] binary16 KV cache.
//
// CacheGen page, 核心方法: each chunk's bitstream is decoded on the GPU back
// to tensors; tokens of a 10-token group depend only on their anchor (no
// delta chain); symbols were arithmetic-coded against per channel-layer
// models, anchors and deltas separately.
//
// Work decomposition (gfx950, wave64): one wavefront per
// (chunk, layer*2+kv row, block of 64 channels); lane i decodes the stream of
// channel c0+i.  All lanes of a wave are at the same token j at the same
// time, so the anchor/delta model switch is wave-uniform, and the 64 lanes'
// binary16 results for token j are 64 consecutive channels: one fully
// coalesced 128-byte store per token.  The lanes' 64 probability models are
// staged in LDS once per wave.
#include "kvc_internal.h"

namespace kvc {

namespace {

// Per-lane reader of a big-endian byte string stored in 4-byte words.
struct ByteReader {
  const uint32_t *wp;
  uint32_t nwords;  // readable words: pad4(nbytes) / 4
  uint32_t widx;    // next word to load
  uint32_t cur;     // current word, next byte in the top 8 bits
  uint32_t avail;   // bytes left in cur
  uint32_t pos;     // bytes consumed so far

  __device__ inline uint32_t next() {
    if (avail == 0) {
      cur = widx < nwords ? bswap32(wp[widx]) : 0u;
      ++widx;
      avail = 4;
    }
    const uint32_t b = cur >> 24;
    cur <<= 8;
    --avail;
    ++pos;
    return b;
  }
};

// t = floor(code / r) for r in [2^9, 2^17), exact for t <= 2^15 and
// clamped to at most 2^15 + 1 otherwise (the caller rejects t >= 2^15).
__device__ inline uint32_t quotient(uint32_t code, uint32_t r) {
  const float fr = (float)r;
  const float fc = (float)code;
  uint32_t q = (uint32_t)(fc * __builtin_amdgcn_rcpf(fr));
  q = q > kTot ? kTot : q;
  uint32_t p = q * r;  // < 2^32
  if (p > code) {
    q -= 1;
  } else if (code - p >= r) {
    q += 1;
  }
  return q;
}

}  // namespace

template <bool kSymbols>
__global__ __launch_bounds__(64) void k_decode(Desc d, const ChunkInfo *__restrict__ ci,
                                               const uint8_t *__restrict__ valid,
                                               const uint32_t *__restrict__ offsets,
                                               const uint8_t *__restrict__ tables,
                                               void *__restrict__ out, uint32_t T_total,
                                               int32_t *status) {
  const uint32_t cb = blockIdx.x, row = blockIdx.y, k = blockIdx.z;
  if (!valid[k]) return;
  __shared__ uint16_t sA[kWave * kAnchorStride];
  __shared__ uint16_t sD[kWave * kDeltaStride];
  const uint32_t lane = threadIdx.x;
  const uint32_t S = n_streams(d);
  const uint32_t c0 = cb * kWave;
  const uint32_t nv = d.C - c0 < kWave ? d.C - c0 : kWave;
  const uint32_t m0 = row * d.C + c0;
  const ChunkInfo c = ci[k];
  const uint32_t level = c.level;
  const uint32_t b = d.bits[level][third_of(row >> 1, d.L)];
  const int32_t M = (1 << (b - 1)) - 1;

  // Stage the wave's 64 anchor models and 64 delta models (this level) in LDS.
  {
    const uint4 *srcA =
        reinterpret_cast<const uint4 *>(tables + kTablesHdr + (uint64_t)m0 * kAnchorStride * 2);
    uint4 *dstA = reinterpret_cast<uint4 *>(sA);
    const uint32_t nA = nv * (kAnchorStride * 2 / 16);
    for (uint32_t i = lane; i < nA; i += kWave) dstA[i] = srcA[i];
    const uint64_t delta_off = kTablesHdr + (uint64_t)S * kAnchorStride * 2;
    const uint4 *srcD = reinterpret_cast<const uint4 *>(
        tables + delta_off + ((uint64_t)level * S + m0) * kDeltaStride * 2);
    uint4 *dstD = reinterpret_cast<uint4 *>(sD);
    const uint32_t nD = nv * (kDeltaStride * 2 / 16);
    for (uint32_t i = lane; i < nD; i += kWave) dstD[i] = srcD[i];
  }
  __syncthreads();
  if (lane >= nv) return;

  const uint32_t m = m0 + lane;
  const uint8_t *rec = c.records + (uint64_t)m * kRecBytes;
  const float lo = __builtin_bit_cast(float, *reinterpret_cast<const uint32_t *>(rec));
  const float sa = __builtin_bit_cast(float, *reinterpret_cast<const uint32_t *>(rec + 4));
  const float dl = __builtin_bit_cast(float, *reinterpret_cast<const uint32_t *>(rec + 8));
  const uint32_t nbytes = *reinterpret_cast<const uint32_t *>(rec + 12);
  const uint8_t *payload = c.cont + kHdrBytes + (uint64_t)kRecBytes * S + offsets[(uint64_t)k * S + m];

  const uint16_t *ta = sA + lane * kAnchorStride;
  const uint16_t *td = sD + lane * kDeltaStride;

  bool bad = nbytes < 4;
  ByteReader br;
  br.wp = reinterpret_cast<const uint32_t *>(payload);
  br.nwords = (uint32_t)(pad4(nbytes) >> 2);
  br.widx = 1;
  br.cur = 0;
  br.avail = 0;
  br.pos = 4;
  uint32_t code = bad ? 0u : bswap32(br.wp[0]);
  uint32_t range = 0xFFFFFFFFu;

  const uint64_t ld = d.C;
  uint64_t o = ((uint64_t)row * T_total + c.first_token) * ld + c0 + lane;
  const uint32_t n = c.n_tokens;
  float ahat = 0.0f;
  uint32_t g = 0;  // position inside the current group
  for (uint32_t j = 0; j < n; ++j, o += ld) {
    const bool anchor = g == 0;
    g = g + 1 == d.G ? 0 : g + 1;
    const uint32_t r = range >> kPrec;
    uint32_t t = quotient(code, r);
    if (t >= kTot) {
      bad = true;
      t = kTot - 1;
    }
    uint32_t s = 0;
    const uint16_t *tab = anchor ? ta : td;
    if (anchor) {
#pragma unroll
      for (uint32_t step = 128; step; step >>= 1)
        if (tab[s + step] <= t) s += step;
    } else {
#pragma unroll
      for (uint32_t step = 32; step; step >>= 1)
        if (tab[s + step] <= t) s += step;
    }
    const uint32_t cs = tab[s];
    uint32_t f = (uint32_t)tab[s + 1] - cs;
    if (f == 0 || f > kTot) {  // only with damaged tables
      bad = true;
      f = 1;
    }
    code -= r * cs;
    range = r * f;
    if (range < 512u) {  // impossible with valid tables; keeps the loop finite
      bad = true;
      range = 1u << 24;
    }
    while (range < (1u << 24)) {
      code = (code << 8) | br.next();
      range <<= 8;
    }
    if constexpr (kSymbols) {
      static_cast<uint8_t *>(out)[o] = (uint8_t)s;
    } else {
      float v;
      if (anchor) {
        ahat = __builtin_fmaf((float)s, sa, lo);
        v = ahat;
      } else {
        v = __builtin_fmaf((float)((int32_t)s - M), dl, ahat);
      }
      static_cast<uint16_t *>(out)[o] = f2h(v);
    }
  }
  if (bad || br.pos != nbytes) set_status(status, KVC_ERR_CORRUPT_STREAM);
}

hipError_t launch_decode(const Desc &d, const ChunkInfo *dev_chunks, uint32_t n_chunks,
                         const uint8_t *valid, const uint32_t *offsets, const uint8_t *tables,
                         void *out, uint32_t T_total, bool symbols, int32_t *status,
                         hipStream_t stream) {
  const dim3 grid((d.C + kWave - 1) / kWave, 2u * d.L, n_chunks);
  if (symbols)
    hipLaunchKernelGGL(k_decode<true>, grid, dim3(kWave), 0, stream, d, dev_chunks, valid,
                       offsets, tables, out, T_total, status);
  else
    hipLaunchKernelGGL(k_decode<false>, grid, dim3(kWave), 0, stream, d, dev_chunks, valid,
                       offsets, tables, out, T_total, status);
  return hipGetLastError();
}

}  // namespace kvc
