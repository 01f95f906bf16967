// Incremental refinement: profile and encode of the refinement layer.
//
// CacheGen page, 局限与 Future Work: send a low-quality version of the KV
// first and refinement bits after it.  The refinement layer of a chunk
// leaves its base layer (the container at the chosen level) untouched and
// codes, per stream, the residual e = x - xh against the base layer's
// binary32 reconstruction xh (anchors fma(qa, sa, lo), other tokens
// fma(q, dl, ahat)): one E-bit symmetric mid-tread scale for the stream's
// anchor tokens, Da = max |e| / Me, one for its other tokens, Dd, symbols
// q + Me with q = rint(e / D) clamped to [-Me, Me], range-coded in token
// order against two models per (level, layer, K/V, channel).  The refined
// value is binary16(fma(q, D, xh)).
//
// Refinement tables blob (device; written by kvc_profile_refine):
//   128-byte header: u32 magic "KVRT", version, L, C, G, chunk, E, n_levels,
//   cdf precision; delta bits [4][3] at 36; u64 refinement id at 48, u64
//   base profile id at 56, u64 models at 64, u64 section offsets at 72 and
//   80, u64 total bytes at 88;
//   then cumulative frequencies [n_levels][2LC][64] u16 for anchor tokens,
//   then the same for the other tokens (cum[0..A], pads 0xFFFF).
// Refinement container ("KVCR"): the base container's layout with records
// {f32 Da, f32 Dd, u32 0, u32 nbytes} and the payload in the same reading
// order; header byte 7 holds E, bytes 56..63 the base profile id.
//
// Kernels:
//   k_refine_count     : one wave per (row, 64 channels); per profiling chunk
//                        and level, the base quantizer, the residual maxima,
//                        then the refinement symbols counted in LDS;
//   k_refine_normalize : counts -> cumulative tables and model hashes;
//   k_refine_final     : header and refinement id;
//   k_refine_stats     : per (chunk, unit), one wave: each stream's base side
//                        information, its two scales and the exact coded
//                        length of its refinement symbols;
//   k_refine_emit      : per (chunk, unit), one wave: each stream's bytes
//                        (the newest 8 held in a register, where a carry is
//                        one add; older ones in the wave's lane-interleaved
//                        scratch), then the reading rule replayed to put
//                        every block in its place;
//   k_refine_header    : the 64-byte headers.
// Both coding kernels copy each lane's two models into LDS once per item.
// Encode is offline: one wave per item and a replay pass after the coder
// keep the kernels short, at about 3x the base encode's time.
#include "kvc_internal.h"

namespace kvc {

hipError_t launch_rowhash(const Desc &d, const uint64_t *model_hash, uint64_t *row_hash,
                          hipStream_t stream);
hipError_t launch_index(const Desc &d, const ChunkInfo *dev_chunks, uint32_t n_chunks,
                        uint64_t *row_sums, uint32_t *flags, uint32_t *offsets, uint8_t *valid,
                        uint64_t *payload, const uint8_t *tables, int check_header_flag,
                        int32_t *status, hipStream_t stream);
hipError_t launch_encode_layout(const Desc &d, uint32_t n_chunks, const uint64_t *payload,
                                uint64_t *chunk_off_ws, uint64_t *chunk_off_out, uint64_t out_cap,
                                uint32_t *fits, uint32_t *redo, int32_t *status,
                                hipStream_t stream);

namespace {

__device__ inline uint32_t ffbh32(uint32_t v) {
  uint32_t r;
  __asm__("v_ffbh_u32 %0, %1" : "=v"(r) : "v"(v));
  return r;
}

// The anchor-token (kind 0) and other-token (kind 1) cumulative table of
// stream m at level lv.
__device__ inline const uint16_t *refine_cum(const uint8_t *rtables, const Desc &d, uint32_t lv,
                                             uint32_t kind, uint32_t m) {
  const uint64_t S = n_streams(d);
  return reinterpret_cast<const uint16_t *>(rtables + kTablesHdr) +
         (((uint64_t)kind * d.nlev + lv) * S + m) * kDeltaStride;
}

// A lane's two refinement tables (cum[0..A], A = 2^E - 1) copied to its
// column of a wave's LDS copy [2][64 entries][64 lanes], read back by the
// same lane only (so no barrier): the coder's per-token lookups then wait on
// LDS, not on memory.
struct RefineCumLds {
  uint16_t e[2][kDeltaStride][kWave];
};
__device__ inline void stage_refine_cum(RefineCumLds &t, const uint16_t *ca, const uint16_t *cd,
                                        uint32_t A, uint32_t lane) {
  for (uint32_t i = 0; i <= A; ++i) {
    t.e[0][i][lane] = ca[i];
    t.e[1][i][lane] = cd[i];
  }
}

// One stream's base side information at Mb = 2^(b-1) - 1 and the maxima of
// |x - xh| over its anchor tokens and its other tokens.  Returns false if a
// value is not finite.
__device__ inline bool refine_scan(Column &x, uint32_t n, uint32_t G, int32_t Mb, float &lo,
                                   float &sa, float &dl, float &amax, float &dmax) {
  float maxabs;
  const bool finite = stream_stats(x, n, G, lo, sa, maxabs);
  dl = maxabs / (float)Mb;
  const float inv_sa = recip_or_zero(sa), inv_dl = recip_or_zero(dl);
  float ahat = 0.0f, am = 0.0f, dm = 0.0f;
  const float l0 = lo, s0 = sa, d0 = dl;
  for_each_group_token<2, kTokenBatch>(x, n, G, [&](float v, auto anchor) {
    if constexpr (decltype(anchor)::value) {
      ahat = __builtin_fmaf((float)quant_anchor(v, l0, s0, inv_sa), s0, l0);
      const float a = __builtin_fabsf(v - ahat);
      if (a > am) am = a;
    } else {
      const float xh = __builtin_fmaf((float)quant_delta(v - ahat, d0, inv_dl, Mb), d0, ahat);
      const float a = __builtin_fabsf(v - xh);
      if (a > dm) dm = a;
    }
  });
  amax = am;
  dmax = dm;
  return finite;
}

// The refinement symbols of one stream (q + Me), in token order, calling
// f(symbol, anchor_token).
template <class F>
__device__ inline void refine_symbols(Column &x, uint32_t n, uint32_t G, int32_t Mb, int32_t Me,
                                      float lo, float sa, float dl, float Da, float Dd, F &&f) {
  const float inv_sa = recip_or_zero(sa), inv_dl = recip_or_zero(dl);
  const float inv_a = recip_or_zero(Da), inv_d = recip_or_zero(Dd);
  float ahat = 0.0f;
  for_each_group_token<2, kTokenBatch>(x, n, G, [&](float v, auto anchor) {
    if constexpr (decltype(anchor)::value) {
      ahat = __builtin_fmaf((float)quant_anchor(v, lo, sa, inv_sa), sa, lo);
      f((uint32_t)(quant_delta(v - ahat, Da, inv_a, Me) + Me), true);
    } else {
      const float xh = __builtin_fmaf((float)quant_delta(v - ahat, dl, inv_dl, Mb), dl, ahat);
      f((uint32_t)(quant_delta(v - xh, Dd, inv_d, Me) + Me), false);
    }
  });
}

}  // namespace

// ------------------------------------------------------------- profiling
__global__ __launch_bounds__(64) void k_refine_count(Desc d, uint32_t ebits,
                                                     const uint16_t *__restrict__ kv, uint32_t T,
                                                     uint32_t *__restrict__ counts,
                                                     int32_t *status) {
  const uint32_t cb = blockIdx.x, row = blockIdx.y;
  const uint32_t lane = threadIdx.x;
  const uint32_t c0 = cb * kWave;
  if (c0 + lane >= d.C) return;
  const uint32_t m = row * d.C + c0 + lane;
  const uint32_t stride = 2u * d.nlev * kDeltaStride;  // [level][kind][64]
  extern __shared__ uint16_t hist[];                   // [stride][kWave]
  for (uint32_t i = 0; i < stride; ++i) hist[i * kWave + lane] = 0;
  uint32_t *cnt = counts + (uint64_t)m * stride;
  for (uint32_t i = 0; i < stride; ++i) cnt[i] = 0;
  const int32_t Me = (1 << (ebits - 1)) - 1;
  const uint64_t ld = d.C;
  const uint32_t third = third_of(row >> 1, d.L);
  const uint32_t nchunks = (T + d.chunk - 1) / d.chunk;
  for (uint32_t k = 0; k < nchunks; ++k) {
    const uint32_t t0 = k * d.chunk;
    const uint32_t n = T - t0 < d.chunk ? T - t0 : d.chunk;
    Column x{reinterpret_cast<const uint8_t *>(kv + ((uint64_t)row * T + t0) * ld + c0), 2 * ld,
             2 * lane};
    for (uint32_t lv = 0; lv < d.nlev; ++lv) {
      const int32_t Mb = (1 << (d.bits[lv][third] - 1)) - 1;
      float lo, sa, dl, amax, dmax;
      if (!refine_scan(x, n, d.G, Mb, lo, sa, dl, amax, dmax)) set_status(status, KVC_ERR_NONFINITE);
      const float Da = amax / (float)Me, Dd = dmax / (float)Me;
      const uint32_t base = lv * 2u * kDeltaStride;
      refine_symbols(x, n, d.G, Mb, Me, lo, sa, dl, Da, Dd, [&](uint32_t s, bool anchor) {
        hist[(base + (anchor ? 0u : kDeltaStride) + s) * kWave + lane] += 1;
      });
    }
    // flush: at most chunk_tokens (<= 65535) counts per bin per chunk
    for (uint32_t i = 0; i < stride; ++i) {
      const uint32_t v = hist[i * kWave + lane];
      if (v) {
        cnt[i] += v;
        hist[i * kWave + lane] = 0;
      }
    }
  }
}

__global__ __launch_bounds__(64) void k_refine_normalize(Desc d, uint32_t ebits,
                                                         const uint32_t *__restrict__ counts,
                                                         uint8_t *__restrict__ rtables,
                                                         uint64_t *__restrict__ model_hash) {
  const uint32_t S = n_streams(d);
  const uint32_t m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= S) return;
  const uint32_t A = (1u << ebits) - 1u;
  const uint32_t *cnt = counts + (uint64_t)m * (2u * d.nlev * kDeltaStride);
  uint16_t *sec = reinterpret_cast<uint16_t *>(rtables + kTablesHdr);
  uint64_t h = kFnvOffset;
  for (uint32_t lv = 0; lv < d.nlev; ++lv)
    for (uint32_t kind = 0; kind < 2; ++kind)
      h = normalize_one(cnt + (lv * 2u + kind) * kDeltaStride, A,
                        sec + (((uint64_t)kind * d.nlev + lv) * S + m) * kDeltaStride,
                        kDeltaStride, h);
  model_hash[m] = h;
}

__global__ void k_refine_final(Desc d, uint32_t ebits, const uint64_t *__restrict__ row_hash,
                               const uint8_t *__restrict__ base_tables,
                               uint8_t *__restrict__ rtables) {
  if (threadIdx.x != 0) return;
  const uint64_t base_id = *reinterpret_cast<const uint64_t *>(base_tables + 48);
  uint64_t h = kFnvOffset;
  h = fnv_u32(h, d.L);
  h = fnv_u32(h, d.C);
  h = fnv_u32(h, d.G);
  h = fnv_u32(h, d.chunk);
  h = fnv_u32(h, 8u);
  h = fnv_u32(h, d.nlev);
  h = fnv_u32(h, kPrec);
  for (uint32_t lv = 0; lv < d.nlev; ++lv)
    for (uint32_t t = 0; t < 3; ++t) h = fnv_byte(h, d.bits[lv][t]);
  h = fnv_u32(h, ebits);
  h = fnv_u64(h, base_id);
  for (uint32_t r = 0; r < 2u * d.L; ++r) h = fnv_u64(h, row_hash[r]);
  const uint64_t S = n_streams(d);
  uint32_t *w = reinterpret_cast<uint32_t *>(rtables);
  w[0] = kRefineTablesMagic;
  w[1] = kRefineVersion;
  w[2] = d.L;
  w[3] = d.C;
  w[4] = d.G;
  w[5] = d.chunk;
  w[6] = ebits;
  w[7] = d.nlev;
  w[8] = kPrec;
  uint8_t *bits = rtables + 36;
  for (uint32_t lv = 0; lv < 4; ++lv)
    for (uint32_t t = 0; t < 3; ++t) bits[lv * 3 + t] = lv < d.nlev ? d.bits[lv][t] : 0;
  uint64_t *q = reinterpret_cast<uint64_t *>(rtables + 48);
  const uint64_t sec = (uint64_t)d.nlev * S * kDeltaStride * 2;
  q[0] = h;                      // 48: refinement id
  q[1] = base_id;                // 56: base profile id
  q[2] = S;                      // 64: models per kind and level
  q[3] = kTablesHdr;             // 72: anchor-token section
  q[4] = kTablesHdr + sec;       // 80: other-token section
  q[5] = kTablesHdr + 2 * sec;   // 88: total bytes
  for (uint32_t off = 96; off < kTablesHdr; off += 8)
    *reinterpret_cast<uint64_t *>(rtables + off) = 0;
}

// ---------------------------------------------------------------- encode
// Which (chunk, unit) item a wave takes, and the unit's first stream.
struct RefineItem {
  uint32_t k, row, c0, nv;
};
__device__ inline RefineItem refine_item(const Desc &d, uint32_t item) {
  const uint32_t ncb = (d.C + kWave - 1) / kWave;
  const uint32_t n_units = 2u * d.L * ncb;
  RefineItem it;
  it.k = item / n_units;
  const uint32_t unit = item % n_units;
  it.row = unit / ncb;
  it.c0 = (unit % ncb) * kWave;
  it.nv = d.C - it.c0 < kWave ? d.C - it.c0 : kWave;
  return it;
}

// Per stream: base side information (workspace side [K][2LC] {lo, sa, dl,
// 0}) and the refinement record {Da, Dd, 0, nbytes} (workspace records),
// nbytes = 4 + the renormalisation shifts of its refinement symbols.
__global__ __launch_bounds__(kWave) void k_refine_stats(
    Desc d, uint32_t ebits, const ChunkInfo *__restrict__ ci, uint32_t n_items,
    const uint8_t *__restrict__ rtables, const uint16_t *__restrict__ kv, uint32_t T,
    float *__restrict__ side, uint8_t *__restrict__ records, int32_t *status) {
  const uint32_t lane = threadIdx.x;
  const uint32_t S = n_streams(d);
  const int32_t Me = (1 << (ebits - 1)) - 1;
  if (!refine_tables_match(d, ebits, rtables)) {
    if (blockIdx.x == 0 && lane == 0) set_status(status, KVC_ERR_PROFILE_MISMATCH);
    return;
  }
  __shared__ RefineCumLds cum_lds;
  for (uint32_t item = blockIdx.x; item < n_items; item += gridDim.x) {
    const RefineItem it = refine_item(d, item);
    if (lane >= it.nv) continue;
    const ChunkInfo c = ci[it.k];
    const uint32_t m = it.row * d.C + it.c0 + lane;
    const int32_t Mb = (1 << (d.bits[c.level][third_of(it.row >> 1, d.L)] - 1)) - 1;
    Column x{reinterpret_cast<const uint8_t *>(kv + ((uint64_t)it.row * T + c.first_token) * d.C +
                                               it.c0),
             2ull * d.C, 2 * lane};
    float lo, sa, dl, amax, dmax;
    if (!refine_scan(x, c.n_tokens, d.G, Mb, lo, sa, dl, amax, dmax))
      set_status(status, KVC_ERR_NONFINITE);
    const float Da = amax / (float)Me, Dd = dmax / (float)Me;
    stage_refine_cum(cum_lds, refine_cum(rtables, d, c.level, 0, m),
                     refine_cum(rtables, d, c.level, 1, m), 2u * (uint32_t)Me + 1u, lane);
    uint32_t range = 0xFFFFFFFFu, shifts = 0;
    refine_symbols(x, c.n_tokens, d.G, Mb, Me, lo, sa, dl, Da, Dd, [&](uint32_t s, bool anchor) {
      const uint32_t kind = anchor ? 0u : 1u;
      range = __umul24(range >> kPrec,
                       (uint32_t)cum_lds.e[kind][s + 1][lane] - cum_lds.e[kind][s][lane]);
      const uint32_t sh = ffbh32(range) & 24u;
      range <<= sh;
      shifts += sh >> 3;
    });
    float *sd = side + ((uint64_t)it.k * S + m) * 4;
    sd[0] = lo;
    sd[1] = sa;
    sd[2] = dl;
    sd[3] = 0.0f;
    uint32_t *rec = reinterpret_cast<uint32_t *>(records + ((uint64_t)it.k * S + m) * kRecBytes);
    rec[0] = __builtin_bit_cast(uint32_t, Da);
    rec[1] = __builtin_bit_cast(uint32_t, Dd);
    rec[2] = 0;
    rec[3] = 4u + shifts;
  }
}

// Per (chunk, unit): every stream's bytes into the lane's linear scratch,
// then the reading rule replayed to place the blocks; also the records.
__global__ __launch_bounds__(kWave) void k_refine_emit(
    Desc d, uint32_t ebits, const ChunkInfo *__restrict__ ci, uint32_t n_items,
    const uint8_t *__restrict__ rtables, const uint16_t *__restrict__ kv, uint32_t T,
    const float *__restrict__ side, const uint8_t *__restrict__ records,
    const uint32_t *__restrict__ offsets, const uint64_t *__restrict__ chunk_off,
    const uint32_t *__restrict__ fits, uint8_t *__restrict__ scratch, uint32_t lane_stride,
    uint8_t *__restrict__ out, int32_t *status) {
  if (*fits == 0 || !refine_tables_match(d, ebits, rtables)) return;
  const uint32_t lane = threadIdx.x;
  const uint32_t S = n_streams(d);
  const int32_t Me = (1 << (ebits - 1)) - 1;
  const uint32_t cap = (uint32_t)pad8(4u + 2u * d.chunk);
  // the wave's scratch, lanes interleaved dword by dword: byte p of lane l at
  // (p / 4) * 256 + 4 l + p % 4, so the 64 lanes' stores at nearby stream
  // positions share a few cache lines; the bytes first, then the shifts
  uint8_t *wbuf = scratch + (uint64_t)blockIdx.x * kWave * lane_stride;
  uint8_t *wshifts = wbuf + (uint64_t)kWave * cap;
  __shared__ RefineCumLds cum_lds;
  auto at = [&](uint8_t *base, uint32_t p) -> uint8_t & {
    return base[(uint64_t)(p >> 2) * (4 * kWave) + 4 * lane + (p & 3u)];
  };
  for (uint32_t item = blockIdx.x; item < n_items; item += gridDim.x) {
    const RefineItem it = refine_item(d, item);
    if (lane >= it.nv) continue;
    const ChunkInfo c = ci[it.k];
    const uint32_t n = c.n_tokens;
    const uint32_t m = it.row * d.C + it.c0 + lane;
    const int32_t Mb = (1 << (d.bits[c.level][third_of(it.row >> 1, d.L)] - 1)) - 1;
    const float *sd = side + ((uint64_t)it.k * S + m) * 4;
    const uint32_t *rin =
        reinterpret_cast<const uint32_t *>(records + ((uint64_t)it.k * S + m) * kRecBytes);
    const float Da = __builtin_bit_cast(float, rin[0]);
    const float Dd = __builtin_bit_cast(float, rin[1]);
    const uint32_t nbytes = rin[3];
    uint8_t *cont = out + chunk_off[it.k];
    uint32_t *rout = reinterpret_cast<uint32_t *>(cont + kHdrBytes + (uint64_t)m * kRecBytes);
    rout[0] = rin[0];
    rout[1] = rin[1];
    rout[2] = 0;
    rout[3] = nbytes;
    stage_refine_cum(cum_lds, refine_cum(rtables, d, c.level, 0, m),
                     refine_cum(rtables, d, c.level, 1, m), 2u * (uint32_t)Me + 1u, lane);
    Column x{reinterpret_cast<const uint8_t *>(kv + ((uint64_t)it.row * T + c.first_token) * d.C +
                                               it.c0),
             2ull * d.C, 2 * lane};
    // the stream's bytes: the newest (up to 8) held in `win`, newest lowest,
    // where a carry is one add; older bytes leave to the scratch four at a
    // time (positions pos - nwin.. are held, so pos - nwin stays a multiple
    // of 4); a carry through all held bytes goes on into the scratch
    uint64_t low = 0, win = 0;
    uint32_t range = 0xFFFFFFFFu, pos = 0, nwin = 0, j = 0, shw = 0;
    bool bad = false;
    auto put_dword = [&](uint8_t *base, uint32_t p, uint32_t v) {
      *reinterpret_cast<uint32_t *>(&at(base, p)) = v;
    };
    auto push = [&](uint32_t byte) {
      if (nwin == 8) {
        // the oldest four held bytes, oldest first in memory
        if (pos - 8u + 4u <= cap) put_dword(wbuf, pos - 8u, __builtin_bswap32((uint32_t)(win >> 32)));
        else bad = true;
        win &= 0xFFFFFFFFull;
        nwin = 4;
      }
      win = (win << 8) | byte;
      ++nwin;
      ++pos;
    };
    refine_symbols(x, n, d.G, Mb, Me, sd[0], sd[1], sd[2], Da, Dd, [&](uint32_t s, bool anchor) {
      const uint32_t kind = anchor ? 0u : 1u;
      const uint32_t cs = cum_lds.e[kind][s][lane];
      const uint32_t f = (uint32_t)cum_lds.e[kind][s + 1][lane] - cs;
      const uint32_t r = range >> kPrec;
      // (HIP's __umul24 returns int: widen the product through uint32_t)
      low += (uint64_t)(uint32_t)__umul24(r, cs);
      range = __umul24(r, f);
      if (low >> 32) {
        low &= 0xFFFFFFFFull;
        const uint64_t w1 = win + 1u;
        const bool out = nwin == 8 ? w1 == 0 : (w1 >> (8u * nwin)) != 0;
        win = nwin == 8 ? w1 : w1 & ((1ull << (8u * nwin)) - 1u);
        if (out) {  // every held byte was 0xFF: on into the scratch (rare)
          uint32_t p = pos - nwin;
          for (;;) {
            if (p == 0) {  // a carry past the first byte: impossible for valid models
              bad = true;
              break;
            }
            --p;
            const uint8_t nb = (uint8_t)(at(wbuf, p) + 1u);
            at(wbuf, p) = nb;
            if (nb != 0) break;
          }
        }
      }
      const uint32_t sh = ffbh32(range) & 24u;
      for (uint32_t t = 0; t < sh; t += 8) {
        push((uint32_t)(low >> 24) & 0xFFu);
        low = (low << 8) & 0xFFFFFFFFull;
      }
      range <<= sh;
      // the shift counts (bytes per token), four tokens to a dword
      shw |= (sh >> 3) << (8u * (j & 3u));
      if ((j & 3u) == 3u) {
        put_dword(wshifts, j & ~3u, shw);
        shw = 0;
      }
      ++j;
    });
    if (j & 3u) put_dword(wshifts, j & ~3u, shw);
    for (uint32_t t = 0; t < 4; ++t) {
      push((uint32_t)(low >> 24) & 0xFFu);
      low = (low << 8) & 0xFFFFFFFFull;
    }
    // the held bytes, then zeros to the block end
    for (uint32_t i = 0; i < nwin; ++i) {
      const uint32_t p = pos - nwin + i;
      if (p < cap) at(wbuf, p) = (uint8_t)(win >> (8u * (nwin - 1u - i)));
      else bad = true;
    }
    bad = bad || pos != nbytes;
    for (uint32_t p = pos; p < cap && (p & 7u) != 0; ++p) at(wbuf, p) = 0;

    // the reading rule: a lane's i-th request takes the unit's next payload
    // block, requests of one step in lane order
    const uint32_t nblk = bad ? 0u : (uint32_t)(pad8(nbytes) / kBlock);
    uint8_t *pay = cont + kHdrBytes + (uint64_t)kRecBytes * S +
                   offsets[(uint64_t)it.k * S + it.row * d.C + it.c0];
    auto copy_block = [&](uint32_t blk, uint32_t slot) {
      uint32_t *dst = reinterpret_cast<uint32_t *>(pay + (uint64_t)slot * kBlock);
      dst[0] = *reinterpret_cast<const uint32_t *>(&at(wbuf, blk * kBlock));
      dst[1] = *reinterpret_cast<const uint32_t *>(&at(wbuf, blk * kBlock + 4));
    };
    uint32_t cnt = 0, R = 4, W = 16, q = 0;
    for (uint32_t blk = 0; blk < 3; ++blk) {
      const bool req = blk < nblk;
      const uint64_t mask = __builtin_amdgcn_ballot_w64(req);
      if (req) {
        copy_block(blk, cnt + lanes_below(mask));
        ++q;
      }
      cnt += (uint32_t)__builtin_popcountll(mask);
    }
    uint32_t g = 0;
    for (uint32_t jj = 0; jj < n; ++jj) {
      const uint32_t ahead = W - R;
      const bool need = g == 0 ? ahead <= 8u : ahead < 2u;
      const bool req = need && q < nblk;
      const uint64_t mask = __builtin_amdgcn_ballot_w64(req);
      if (req) {
        copy_block(q, cnt + lanes_below(mask));
        ++q;
      }
      if (need) W += kBlock;
      cnt += (uint32_t)__builtin_popcountll(mask);
      R += at(wshifts, jj);
      g = g + 1 == d.G ? 0 : g + 1;
    }
    if (bad || R != nbytes || q != nblk) set_status(status, KVC_ERR_CORRUPT_STREAM);
  }
}

__global__ void k_refine_header(Desc d, uint32_t ebits, const ChunkInfo *__restrict__ ci,
                                uint32_t n_chunks, const uint8_t *__restrict__ rtables,
                                const uint64_t *__restrict__ payload,
                                const uint64_t *__restrict__ chunk_off,
                                const uint32_t *__restrict__ fits, uint8_t *__restrict__ out) {
  if (*fits == 0) return;
  for (uint32_t k = threadIdx.x; k < n_chunks; k += blockDim.x) {
    const ChunkInfo c = ci[k];
    uint32_t *h = reinterpret_cast<uint32_t *>(out + chunk_off[k]);
    const uint32_t level = c.level;
    const uint64_t rid = *reinterpret_cast<const uint64_t *>(rtables + 48);
    const uint64_t bid = *reinterpret_cast<const uint64_t *>(rtables + 56);
    h[0] = kRefineContainerMagic;
    h[1] = kRefineVersion | (level << 16) | (ebits << 24);
    h[2] = d.G | (kPrec << 16) | ((uint32_t)d.bits[level][0] << 24);
    h[3] = (uint32_t)d.bits[level][1] | ((uint32_t)d.bits[level][2] << 8);
    h[4] = d.L;
    h[5] = d.C;
    h[6] = c.n_tokens;
    h[7] = c.first_token;
    h[8] = (uint32_t)rid;
    h[9] = (uint32_t)(rid >> 32);
    h[10] = (uint32_t)payload[k];
    h[11] = (uint32_t)(payload[k] >> 32);
    h[12] = d.chunk;
    h[13] = n_streams(d);
    h[14] = (uint32_t)bid;
    h[15] = (uint32_t)(bid >> 32);
  }
}

// ---------------------------------------------------------------- launch
size_t refine_count_lds_bytes(const Desc &d) {
  return (size_t)2 * d.nlev * kDeltaStride * kWave * sizeof(uint16_t);
}

hipError_t launch_profile_refine(const Desc &d, uint32_t ebits, const uint16_t *kv, uint32_t T,
                                 const uint8_t *base_tables, uint8_t *rtables, uint32_t *counts,
                                 uint64_t *model_hash, uint64_t *row_hash, int32_t *status,
                                 hipStream_t stream) {
  const uint32_t S = n_streams(d);
  hipLaunchKernelGGL(k_refine_count, dim3((d.C + kWave - 1) / kWave, 2u * d.L), dim3(kWave),
                     refine_count_lds_bytes(d), stream, d, ebits, kv, T, counts, status);
  hipLaunchKernelGGL(k_refine_normalize, dim3((S + 63) / 64), dim3(64), 0, stream, d, ebits,
                     counts, rtables, model_hash);
  hipError_t e = launch_rowhash(d, model_hash, row_hash, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_refine_final, dim3(1), dim3(64), 0, stream, d, ebits, row_hash,
                     base_tables, rtables);
  return hipGetLastError();
}

// Scratch of one k_refine_emit lane: a stream's bytes (at most 4 + 2 per
// token, in whole blocks), then one byte per token.
uint32_t refine_emit_lane_bytes(uint32_t chunk) {
  return (uint32_t)(pad8(4u + 2u * (uint64_t)chunk) + pad8(chunk));
}

hipError_t launch_encode_refine(const Desc &d, uint32_t ebits, const uint8_t *rtables,
                                const uint16_t *kv, uint32_t T, const ChunkInfo *dev_chunks,
                                uint32_t n_chunks, uint32_t stat_blocks, uint32_t emit_blocks,
                                float *side, uint8_t *records, uint64_t *row_sums,
                                uint32_t *flags, uint32_t *offsets, uint8_t *valid,
                                uint64_t *payload, uint64_t *chunk_off_ws, uint32_t *fits,
                                uint32_t *spare, uint8_t *scratch, uint8_t *out, uint64_t out_cap,
                                uint64_t *chunk_off_out, int32_t *status, hipStream_t stream) {
  const uint32_t ncb = (d.C + kWave - 1) / kWave;
  const uint32_t n_items = n_chunks * 2u * d.L * ncb;
  hipLaunchKernelGGL(k_refine_stats, dim3(stat_blocks), dim3(kWave), 0, stream, d, ebits,
                     dev_chunks, n_items, rtables, kv, T, side, records, status);
  hipError_t e = launch_index(d, dev_chunks, n_chunks, row_sums, flags, offsets, valid, payload,
                              rtables, 0, status, stream);
  if (e != hipSuccess) return e;
  e = launch_encode_layout(d, n_chunks, payload, chunk_off_ws, chunk_off_out, out_cap, fits, spare,
                           status, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_refine_emit, dim3(emit_blocks), dim3(kWave), 0, stream, d, ebits,
                     dev_chunks, n_items, rtables, kv, T, side, records, offsets, chunk_off_ws,
                     fits, scratch, refine_emit_lane_bytes(d.chunk), out, status);
  hipLaunchKernelGGL(k_refine_header, dim3(1), dim3(256), 0, stream, d, ebits, dev_chunks,
                     n_chunks, rtables, payload, chunk_off_ws, fits, out);
  return hipGetLastError();
}

}  // namespace kvc
