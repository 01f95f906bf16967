// Internal definitions shared by the libkvc kernels and host code.
//
// Layouts (little-endian, all written and read only by this library and by
// whoever follows the same published format):
//   container  : 64-byte header, 2LC records of 16 bytes {f32 lo, f32 sa,
//                f32 dl, u32 nbytes}, then the payload: per unit (one
//                (layer, K/V) row and up to 64 consecutive channels), in
//                unit order, the unit's streams' 8-byte blocks in the order
//                the decoder's reading rule asks for them (kvc_decode.hip).
//   tables blob: 128-byte header, anchor cumulative frequencies
//                [2LC][ANCHOR_STRIDE] u16, delta cumulative frequencies
//                [n_levels][2LC][DELTA_STRIDE] u16.
#pragma once

#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>

#include "kvc.h"

namespace kvc {

constexpr uint32_t kPrec = 15;
constexpr uint32_t kTot = 1u << kPrec;
constexpr uint32_t kAnchorAlpha = 256;
constexpr uint32_t kAnchorStride = 264;  // u16 entries per anchor model: cum[0..256] + pad
constexpr uint32_t kDeltaStride = 64;    // u16 entries per delta model: cum[0..A] + pad
constexpr uint32_t kHdrBytes = 64;
constexpr uint32_t kRecBytes = 16;
constexpr uint32_t kTablesHdr = 128;
constexpr uint32_t kWave = 64;
constexpr uint32_t kMaxChunksPerBatch = 64;

constexpr uint32_t kContainerMagic = 0x3143564Bu;  // "KVC1"
constexpr uint32_t kTablesMagic = 0x5443564Bu;     // "KVCT"
constexpr uint32_t kFormatVersion = 2;  // containers: block-interleaved unit payloads
constexpr uint32_t kTablesVersion = 1;
// Refinement layer: its tables blob ("KVRT") and containers ("KVCR").
constexpr uint32_t kRefineTablesMagic = 0x5452564Bu;     // "KVRT"
constexpr uint32_t kRefineContainerMagic = 0x5243564Bu;  // "KVCR"
constexpr uint32_t kRefineVersion = 1;

// Per-chunk description kept in the workspace.
struct ChunkInfo {
  const uint8_t *cont;     // container (decode) or nullptr (encode)
  const uint8_t *records;  // the chunk's 2LC stream records
  uint64_t cont_bytes;     // container size (decode)
  uint32_t first_token;    // destination token (decode) / source token (encode)
  uint32_t n_tokens;
  uint32_t level;
  uint32_t out_tokens;     // decode: token capacity T of the chunk's output cache
  void *out;               // decode: the chunk's output cache [L][2][T][C]
};
static_assert(sizeof(ChunkInfo) == 48, "ChunkInfo layout");

struct ChunkBatch {
  ChunkInfo c[kMaxChunksPerBatch];
};

// A group of chunks decoded by one workgroup per (row, channel block): the
// chunk table entries [start, start + count), which the host orders by level.
struct DecodeGroup {
  uint32_t level;  // bit l set: the group holds chunks of level l
  uint32_t start;
  uint32_t count;
  uint32_t pad;
};
static_assert(sizeof(DecodeGroup) == 16, "DecodeGroup layout");

// Decode workgroups have at most this many waves; a wave decodes one of the
// group's chunks at a time.
constexpr uint32_t kDecodeMaxWaves = 16;
// Encode workgroups have at most this many waves (one chunk each at a time).
constexpr uint32_t kEncodeMaxWaves = 16;
// LDS per decode or emit workgroup that still lets two of them share a CU.
constexpr uint32_t kLdsBudget = 80u * 1024u;

// Fourth dword of a raw buffer resource on gfx9-family GPUs (32-bit data
// format, no swizzle): loads are bounds-checked against num_records bytes.
constexpr int32_t kBufferWord3 = 0x00020000;

struct GroupBatch {
  DecodeGroup g[kMaxChunksPerBatch];
};

// Descriptor values used inside kernels.
struct Desc {
  uint32_t L, C, G, chunk, nlev;
  uint8_t bits[4][3];
};

__host__ __device__ inline uint32_t third_of(uint32_t l, uint32_t L) { return (3u * l) / L; }
__host__ __device__ inline uint32_t n_streams(const Desc &d) { return 2u * d.L * d.C; }
// Payload blocks: a stream's bytes are cut into 8-byte blocks (the last one
// zero-padded); a unit (one row, up to 64 consecutive channels) stores its
// streams' blocks in the order its reader asks for them.
constexpr uint32_t kBlock = 8;
__host__ __device__ inline uint64_t pad8(uint64_t v) { return (v + 7u) & ~uint64_t(7); }

// 64-bit FNV-1a (Fowler / Noll / Vo), published offset basis and prime.
constexpr uint64_t kFnvOffset = 0xcbf29ce484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001b3ull;
__host__ __device__ inline uint64_t fnv_byte(uint64_t h, uint32_t b) {
  return (h ^ (b & 0xFFu)) * kFnvPrime;
}
__host__ __device__ inline uint64_t fnv_u16(uint64_t h, uint32_t v) {
  h = fnv_byte(h, v);
  return fnv_byte(h, v >> 8);
}
__host__ __device__ inline uint64_t fnv_u32(uint64_t h, uint32_t v) {
  h = fnv_u16(h, v);
  return fnv_u16(h, v >> 16);
}
__host__ __device__ inline uint64_t fnv_u64(uint64_t h, uint64_t v) {
  h = fnv_u32(h, (uint32_t)v);
  return fnv_u32(h, (uint32_t)(v >> 32));
}

// Rank of this lane among the set lanes of `mask` below it.
__device__ inline uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Record the first device-side error of a call.
__device__ inline void set_status(int32_t *st, int32_t code) {
  atomicCAS(st, 0, code);
}

// binary16 bits -> binary32 (exact) and binary32 -> binary16 bits (round to
// nearest even in the default rounding mode; subnormals kept).
__device__ inline float h2f(uint16_t b) {
  _Float16 h = __builtin_bit_cast(_Float16, b);
  return (float)h;
}
__device__ inline uint16_t f2h(float f) {
  // The value must be rounded to binary32 first.  Without this register
  // barrier the backend folds an fma that feeds the conversion into one
  // mixed-precision fma (v_fma_mixlo_f16) that rounds only once, straight to
  // binary16, which differs from fp16(fp32(a*b+c)) in rare double-rounding
  // cases.
  __asm__("" : "+v"(f));
  _Float16 h = (_Float16)f;
  return __builtin_bit_cast(uint16_t, h);
}

// Byte-swap a 32-bit word: the payload is a big-endian byte string.
__device__ inline uint32_t bswap32(uint32_t v) { return __builtin_bswap32(v); }

__device__ inline bool is_finite(float v) { return __builtin_isfinite(v); }

// --------------------------------------------------------------- quantizer
// One stream = column c of x (stride `ld` elements), tokens 0..n-1.
// Anchors: j % G == 0, 8-bit affine over [min, max] of the anchors
// (first occurrence kept on ties: strict comparisons).
//
// rintf(num / den) with the correctly rounded quotient, from the product
// y = num * inv, inv = 1 / den rounded: y is within |q| 1.5 2^-23 of the
// rounded quotient q, at most 2^-14 for the |q| <= 257 of both quantizers,
// so the two round to the same integer unless y lies within that distance
// of a half-integer; only then (rarely, and per lane) is the division done.
// The quantizers' denominators are normal (sa >= 2^-24 / 255 and dl > 2^-70
// for binary16 inputs), so inv is finite.
// The test is wave-uniform (a branch on the ballot, not a divergent one),
// and the rare division is done by the whole wave.
__device__ inline float rint_quot(float num, float den, float inv) {
  const float y = num * inv;
  float r = __builtin_rintf(y);
  // y - r is exact and at most 1/2 in magnitude: within 2^-13 of a
  // half-integer means |y - r| >= 1/2 - 2^-13 (a binary32 constant)
  const bool near_half = __builtin_fabsf(y - r) >= 0.5f - 0x1p-13f;
  if (__builtin_amdgcn_ballot_w64(near_half) != 0) {
    const float e = __builtin_rintf(num / den);
    r = near_half ? e : r;
  }
  return r;
}

// 1 / s, or 0 for a zero scale.  A zero scale quantizes everything to 0:
// sa = 0 only when every anchor equals lo, dl = 0 only when every delta is
// 0, so the numerator times 0 is 0 (for finite inputs), far from a
// half-integer.
__device__ inline float recip_or_zero(float s) { return s == 0.0f ? 0.0f : 1.0f / s; }

// inv_sa = recip_or_zero(sa)
__device__ inline uint32_t quant_anchor(float x, float lo, float sa, float inv_sa) {
  int q = (int)rint_quot(x - lo, sa, inv_sa);
  q = q < 0 ? 0 : q;
  q = q > 255 ? 255 : q;
  return (uint32_t)q;
}

// inv_dl = recip_or_zero(dl)
__device__ inline int32_t quant_delta(float d, float dl, float inv_dl, int32_t M) {
  int q = (int)rint_quot(d, dl, inv_dl);
  q = q < -M ? -M : q;
  q = q > M ? M : q;
  return q;
}

// A lane's column of binary16 KV values: token j of the lane's channel is
// at base + j * ld2 + loff, with base the same for the whole wave.  The
// empty asm makes the lane offset opaque at every load, so that the
// address stays "scalar base + 32-bit lane offset" (a global load with a
// scalar base and no per-lane 64-bit address arithmetic).
struct Column {
  const uint8_t *base;  // wave-uniform
  uint64_t ld2;         // bytes from one token to the next
  uint32_t loff;        // this lane's byte offset
  // the lane's value in the token row that starts at the wave-uniform `row`
  typedef __attribute__((address_space(1))) const uint8_t grow;
  __device__ inline float in_row(grow *row) {
    __asm__("" : "+v"(loff));
    return h2f(*reinterpret_cast<__attribute__((address_space(1))) const uint16_t *>(row + loff));
  }
  __device__ inline float at(uint32_t j) { return in_row((grow *)(base + (uint64_t)j * ld2)); }
};

// Visits the tokens first, first + step, ... (< n) of a lane's column in
// order, calling f(value).  The values are loaded kBatch at a time, so a
// wave waits for memory once per batch rather than once per token.  The row
// address is a wave-uniform pointer advanced by one stride per token (one
// 64-bit scalar add) rather than recomputed from the token index (a 64-bit
// scalar multiply and add per load).
template <uint32_t kBatch, class F>
__device__ inline void for_each_token(Column &x, uint32_t first, uint32_t step, uint32_t n,
                                      F &&f) {
  uint32_t j = first;
  const uint64_t stride = (uint64_t)step * x.ld2;
  Column::grow *row = (Column::grow *)(x.base + (uint64_t)first * x.ld2);
  for (; j + (kBatch - 1) * step < n; j += kBatch * step) {
    float v[kBatch];
#pragma unroll
    for (uint32_t u = 0; u < kBatch; ++u) {
      v[u] = x.in_row(row);
      row += stride;
      // one running pointer: no per-token offsets precomputed in registers
      __asm__("" : "+s"(row));
    }
#pragma unroll
    for (uint32_t u = 0; u < kBatch; ++u) f(v[u]);
  }
  for (; j < n; j += step) {
    f(x.in_row(row));
    row += stride;
  }
}
constexpr uint32_t kTokenBatch = 16;

// Visits every token of a lane's column in order, calling f(value, tag) with
// tag std::true_type for a group's anchor and std::false_type for the other
// tokens.  With groups of the pages' size (10 tokens) whole groups are loaded
// kGroups at a time and visited unrolled, so the anchor/delta choice and the
// group position cost nothing per token; other group sizes and a partial
// last group go through for_each_token with a running group position.
constexpr uint32_t kGroup10 = 10;

template <uint32_t kGroups, uint32_t kBatch, class F>
__device__ inline void for_each_group_token(Column &x, uint32_t n, uint32_t G, F &&f) {
  uint32_t j = 0;
  if (G == kGroup10) {
    Column::grow *row = (Column::grow *)x.base;
    for (; j + kGroups * kGroup10 <= n; j += kGroups * kGroup10) {
      float v[kGroups * kGroup10];
#pragma unroll
      for (uint32_t u = 0; u < kGroups * kGroup10; ++u) {
        v[u] = x.in_row(row);
        row += x.ld2;
        __asm__("" : "+s"(row));
      }
#pragma unroll
      for (uint32_t gi = 0; gi < kGroups; ++gi) {
        f(v[gi * kGroup10], std::true_type{});
#pragma unroll
        for (uint32_t u = 1; u < kGroup10; ++u) f(v[gi * kGroup10 + u], std::false_type{});
      }
    }
  }
  // j is a multiple of G here
  uint32_t g = 0;
  for_each_token<kBatch>(x, j, 1, n, [&](float v) {
    if (g == 0) {
      f(v, std::true_type{});
    } else {
      f(v, std::false_type{});
    }
    g = g + 1 == G ? 0 : g + 1;
  });
}

// Stream statistics: lo, sa (anchor scale) and maxabs of the closed-loop
// deltas.  Returns false if a value is not finite.
__device__ inline bool stream_stats(Column &x, uint32_t n, uint32_t G, float &lo_out,
                                    float &sa_out, float &maxabs_out) {
  float lo = x.at(0);
  float hi = lo;
  for_each_token<kTokenBatch>(x, G, G, n, [&](float v) {
    if (v < lo) lo = v;
    if (v > hi) hi = v;
  });
  const float sa = (hi - lo) / 255.0f;
  const float inv_sa = recip_or_zero(sa);
  bool finite = true;
  float maxabs = 0.0f;
  float ahat = 0.0f;
  for_each_group_token<2, kTokenBatch>(x, n, G, [&](float v, auto anchor) {
    finite = finite && is_finite(v);
    if constexpr (decltype(anchor)::value) {
      ahat = __builtin_fmaf((float)quant_anchor(v, lo, sa, inv_sa), sa, lo);
    } else {
      const float a = __builtin_fabsf(v - ahat);
      if (a > maxabs) maxabs = a;
    }
  });
  lo_out = lo;
  sa_out = sa;
  maxabs_out = maxabs;
  return finite;
}

// counts -> frequencies (floor of 1, remainder to the most frequent symbol,
// lowest index on ties); writes cum[0..A] and pads 0xFFFF; returns the FNV
// state after hashing the frequencies.
__device__ inline uint64_t normalize_one(const uint32_t *cnt, uint32_t A, uint16_t *cum,
                                         uint32_t stride_entries, uint64_t h) {
  uint64_t N = 0;
  uint32_t arg = 0;
  for (uint32_t s = 0; s < A; ++s) {
    N += cnt[s];
    if (cnt[s] > cnt[arg]) arg = s;
  }
  uint32_t sum = 0;
  if (N != 0) {
    for (uint32_t s = 0; s < A; ++s) sum += 1u + (uint32_t)(((uint64_t)cnt[s] * (kTot - A)) / N);
  }
  uint32_t acc = 0;
  for (uint32_t s = 0; s < A; ++s) {
    uint32_t f;
    if (N == 0) {
      f = kTot / A + (s < kTot % A ? 1u : 0u);
    } else {
      f = 1u + (uint32_t)(((uint64_t)cnt[s] * (kTot - A)) / N);
      if (s == arg) f += kTot - sum;
    }
    cum[s] = (uint16_t)acc;
    acc += f;
    h = fnv_u16(h, f);
  }
  cum[A] = (uint16_t)acc;  // == 2^15
  for (uint32_t s = A + 1; s < stride_entries; ++s) cum[s] = 0xFFFFu;
  return h;
}

// The refinement tables blob was made for this descriptor and E.
__device__ inline bool refine_tables_match(const Desc &d, uint32_t ebits, const uint8_t *rt) {
  const uint32_t *w = reinterpret_cast<const uint32_t *>(rt);
  return w[0] == kRefineTablesMagic && w[1] == kRefineVersion && w[2] == d.L && w[3] == d.C &&
         w[4] == d.G && w[5] == d.chunk && w[6] == ebits && w[7] == d.nlev && w[8] == kPrec;
}

// Workspace layout helpers.
__host__ __device__ inline uint64_t align256(uint64_t v) { return (v + 255u) & ~uint64_t(255); }

}  // namespace kvc
