// Offline profiling: per channel-layer symbol distributions, anchors and
// deltas separately, normalised to 2^15 (CacheGen page, 核心方法 step 3 and
// 关键观察 observation 3: distributions profiled offline per channel-layer
// combination and reused across contexts of the same model).
//
//   k_profile_count     : one wavefront per (row, 64-channel block); lane =
//                         channel; every profiling chunk is quantized
//                         (anchors once, deltas once per level) and counted
//                         into a per-lane u16 histogram in LDS, flushed to the
//                         u32 counts in the workspace after every chunk;
//   k_profile_normalize : per model, counts -> frequencies -> cumulative
//                         table (pads 0xFFFF), and the model's FNV-1a;
//   k_profile_rowhash   : per (layer, K/V) row, FNV-1a over its model hashes;
//   k_profile_final     : blob header and the profile id.
#include "kvc_internal.h"

namespace kvc {

__host__ __device__ inline uint32_t count_stride(uint32_t nlev) {
  return kAnchorAlpha + nlev * kDeltaStride;
}

__global__ __launch_bounds__(64) void k_profile_count(Desc d, const uint16_t *__restrict__ kv,
                                                      uint32_t T, uint32_t *__restrict__ counts,
                                                      int32_t *status) {
  const uint32_t cb = blockIdx.x, row = blockIdx.y;
  const uint32_t lane = threadIdx.x;
  const uint32_t c0 = cb * kWave;
  if (c0 + lane >= d.C) return;
  const uint32_t m = row * d.C + c0 + lane;
  const uint32_t stride = count_stride(d.nlev);
  // lane-private histogram, lane-interleaved so that lanes hit distinct banks
  extern __shared__ uint16_t hist[];  // [stride][kWave]
  for (uint32_t i = 0; i < stride; ++i) hist[i * kWave + lane] = 0;
  uint32_t *cnt = counts + (uint64_t)m * stride;
  for (uint32_t i = 0; i < stride; ++i) cnt[i] = 0;

  const uint64_t ld = d.C;
  const uint32_t third = third_of(row >> 1, d.L);
  const uint32_t nchunks = (T + d.chunk - 1) / d.chunk;
  for (uint32_t k = 0; k < nchunks; ++k) {
    const uint32_t t0 = k * d.chunk;
    const uint32_t n = T - t0 < d.chunk ? T - t0 : d.chunk;
    Column x{reinterpret_cast<const uint8_t *>(kv + ((uint64_t)row * T + t0) * ld + c0), 2 * ld,
             2 * lane};
    float lo, sa, maxabs;
    if (!stream_stats(x, n, d.G, lo, sa, maxabs)) set_status(status, KVC_ERR_NONFINITE);
    const float inv_sa = recip_or_zero(sa);
    // anchors
    for (uint32_t j = 0; j < n; j += d.G) {
      const uint32_t qa = quant_anchor(x.at(j), lo, sa, inv_sa);
      hist[qa * kWave + lane] += 1;
    }
    // deltas, once per level
    for (uint32_t lv = 0; lv < d.nlev; ++lv) {
      const uint32_t b = d.bits[lv][third];
      const int32_t M = (1 << (b - 1)) - 1;
      const float dl = maxabs / (float)M;
      const float inv_dl = recip_or_zero(dl);
      const uint32_t base = kAnchorAlpha + lv * kDeltaStride;
      float ahat = 0.0f;
      uint32_t g = 0;
      for (uint32_t j = 0; j < n; ++j) {
        const float v = x.at(j);
        if (g == 0) {
          ahat = __builtin_fmaf((float)quant_anchor(v, lo, sa, inv_sa), sa, lo);
        } else {
          const uint32_t s = (uint32_t)(quant_delta(v - ahat, dl, inv_dl, M) + M);
          hist[(base + s) * kWave + lane] += 1;
        }
        g = g + 1 == d.G ? 0 : g + 1;
      }
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

__global__ __launch_bounds__(64) void k_profile_normalize(Desc d, const uint32_t *__restrict__ counts,
                                                          uint8_t *__restrict__ tables,
                                                          uint64_t *__restrict__ model_hash) {
  const uint32_t S = n_streams(d);
  const uint32_t m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= S) return;
  const uint32_t stride = count_stride(d.nlev);
  const uint32_t *cnt = counts + (uint64_t)m * stride;
  const uint32_t third = third_of(m / (2u * d.C), d.L);
  uint16_t *cumA = reinterpret_cast<uint16_t *>(tables + kTablesHdr) + (uint64_t)m * kAnchorStride;
  uint64_t h = normalize_one(cnt, kAnchorAlpha, cumA, kAnchorStride, kFnvOffset);
  uint16_t *deltas =
      reinterpret_cast<uint16_t *>(tables + kTablesHdr + (uint64_t)S * kAnchorStride * 2);
  for (uint32_t lv = 0; lv < d.nlev; ++lv) {
    const uint32_t A = (1u << d.bits[lv][third]) - 1u;
    h = normalize_one(cnt + kAnchorAlpha + lv * kDeltaStride, A,
                      deltas + ((uint64_t)lv * S + m) * kDeltaStride, kDeltaStride, h);
  }
  model_hash[m] = h;
}

__global__ void k_profile_rowhash(Desc d, const uint64_t *__restrict__ model_hash,
                                  uint64_t *__restrict__ row_hash) {
  const uint32_t row = blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= 2u * d.L) return;
  uint64_t h = kFnvOffset;
  for (uint32_t c = 0; c < d.C; ++c) h = fnv_u64(h, model_hash[(uint64_t)row * d.C + c]);
  row_hash[row] = h;
}

__global__ void k_profile_final(Desc d, const uint64_t *__restrict__ row_hash,
                                uint8_t *__restrict__ tables) {
  if (threadIdx.x != 0) return;
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
  for (uint32_t r = 0; r < 2u * d.L; ++r) h = fnv_u64(h, row_hash[r]);
  const uint64_t S = n_streams(d);
  uint32_t *w = reinterpret_cast<uint32_t *>(tables);
  w[0] = kTablesMagic;
  w[1] = kTablesVersion;
  w[2] = d.L;
  w[3] = d.C;
  w[4] = d.G;
  w[5] = d.chunk;
  w[6] = 8u;
  w[7] = d.nlev;
  w[8] = kPrec;
  uint8_t *bits = tables + 36;
  for (uint32_t lv = 0; lv < 4; ++lv)
    for (uint32_t t = 0; t < 3; ++t) bits[lv * 3 + t] = lv < d.nlev ? d.bits[lv][t] : 0;
  uint64_t *q = reinterpret_cast<uint64_t *>(tables + 48);
  q[0] = h;                                             // 48: profile id
  q[1] = S;                                             // 56: models
  q[2] = kTablesHdr;                                    // 64: anchor section
  q[3] = kTablesHdr + S * kAnchorStride * 2;            // 72: delta section
  q[4] = q[3] + (uint64_t)d.nlev * S * kDeltaStride * 2;  // 80: total bytes
  for (uint32_t off = 88; off < kTablesHdr; off += 8)
    *reinterpret_cast<uint64_t *>(tables + off) = 0;
}

// Per (layer, K/V) row, FNV-1a over the row's model hashes (shared with the
// refinement profile).
hipError_t launch_rowhash(const Desc &d, const uint64_t *model_hash, uint64_t *row_hash,
                          hipStream_t stream) {
  hipLaunchKernelGGL(k_profile_rowhash, dim3((2u * d.L + 63) / 64), dim3(64), 0, stream, d,
                     model_hash, row_hash);
  return hipGetLastError();
}

hipError_t launch_profile(const Desc &d, const uint16_t *kv, uint32_t T, uint8_t *tables,
                          uint32_t *counts, uint64_t *model_hash, uint64_t *row_hash,
                          int32_t *status, hipStream_t stream) {
  const uint32_t S = n_streams(d);
  const size_t lds = (size_t)count_stride(d.nlev) * kWave * sizeof(uint16_t);
  hipLaunchKernelGGL(k_profile_count, dim3((d.C + kWave - 1) / kWave, 2u * d.L), dim3(kWave), lds,
                     stream, d, kv, T, counts, status);
  hipLaunchKernelGGL(k_profile_normalize, dim3((S + 63) / 64), dim3(64), 0, stream, d, counts,
                     tables, model_hash);
  hipLaunchKernelGGL(k_profile_rowhash, dim3((2u * d.L + 63) / 64), dim3(64), 0, stream, d,
                     model_hash, row_hash);
  hipLaunchKernelGGL(k_profile_final, dim3(1), dim3(64), 0, stream, d, row_hash, tables);
  return hipGetLastError();
}

}  // namespace kvc
