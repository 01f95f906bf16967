/*
 * kvc_oracle.c -- plain, slow, obviously-correct CPU oracle for the
 * CacheGen-style KV-cache codec.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product (the HIP library and its
 * Python binding) includes, links or calls this file; only the tests, the
 * package entry's smoke check and the benchmark's CPU-baseline leg do.  It
 * shares no code, header, table or constant generator with the HIP path.
 *
 * Source of the method: the CacheGen wiki page ("CacheGen: KV Cache
 * Compression and Streaming for Fast LLM Serving", SIGCOMM 2024 summary),
 * section "核心方法" (core method):
 *   - KV is split along tokens into chunks of about 1.5K tokens, each encoded
 *     independently;
 *   - change-based encoding: groups of 10 consecutive tokens, the first token
 *     of a group is the anchor, kept at higher precision (8-bit), the other
 *     tokens store their delta to the anchor (no delta chain);
 *   - layer-wise quantization: layers split into front / middle / back
 *     thirds, coarser delta quantization for deeper thirds;
 *   - arithmetic coding of the quantized symbols with a probability model
 *     profiled offline per channel-layer combination, anchors and deltas
 *     modelled separately.
 * Where the page leaves a step open, the reading implemented here is the
 * one stated beside the code (and listed with the project's design notes):
 *   R1 quantizer: one scale set per stream (chunk, layer, K/V, channel);
 *      affine 8-bit anchors over [min, max] of the stream's anchors;
 *      symmetric mid-tread deltas with 2^(b-1)-1 steps each side.
 *   R2 deltas are taken against the *reconstructed* anchor (closed loop).
 *   R3 layer third of layer l is floor(3 l / L).
 *   R4 arithmetic coder: a static multi-symbol range coder (after G. N. N.
 *      Martin, "Range encoding", 1979) with 32-bit range, 15-bit model
 *      precision, byte renormalisation below 2^24, carry propagation into the
 *      emitted bytes and a 4-byte flush.
 *   R5 model normalisation: floor of 1 count per symbol, the remainder to the
 *      most frequent symbol (lowest index on ties).
 *   R6 container: 64-byte header, 16-byte record per stream, then the
 *      payload of the units (a unit: one (layer, K/V) row and a block of up
 *      to 64 consecutive channels) in (layer, K/V, channel block) order.
 *   R17 a unit's payload holds its streams' bytes cut into 8-byte blocks (the
 *      last one zero-padded), in the order in which the reference reader
 *      (unit_reader below) asks for them.
 *   R19 incremental refinement (the page's future work: low-quality KV
 *      first, refinement bits after): a second layer per chunk that
 *      quantizes the residual against the base layer's binary32
 *      reconstruction (section "refinement" at the end of this file).
 * Arithmetic: IEEE-754 binary32 with round-to-nearest-even, correctly
 * rounded division, true fused multiply-add, no flush-to-zero, no
 * contraction (build with -ffp-contract=off).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- errors */
#define ORC_OK 0
#define ORC_ERR_ARG -1
#define ORC_ERR_SHAPE -2
#define ORC_ERR_PROFILE -3
#define ORC_ERR_CORRUPT -4
#define ORC_ERR_NONFINITE -5
#define ORC_ERR_CAPACITY -6

/* ------------------------------------------------------------- constants */
#define PREC 15u
#define TOT (1u << PREC)
#define HDR_BYTES 64u
#define REC_BYTES 16u
#define MAX_DELTA_ALPHA 64u /* storage stride for a delta model */
#define ANCHOR_ALPHA 256u

/* The codec parameters, passed from Python as 19 u32 words:
 *   [0] L  [1] C  [2] group_tokens  [3] chunk_tokens  [4] anchor_bits
 *   [5] n_levels  [6] cdf_prec_bits  [7..18] delta_bits[level][third]   */
typedef struct {
  uint32_t L, C, G, chunk, abits, nlev, prec;
  uint32_t bits[4][3];
} params;

static int read_params(const uint32_t *w, params *p) {
  p->L = w[0];
  p->C = w[1];
  p->G = w[2];
  p->chunk = w[3];
  p->abits = w[4];
  p->nlev = w[5];
  p->prec = w[6];
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 3; ++j) p->bits[i][j] = w[7 + 3 * i + j];
  if (p->L == 0 || p->C == 0 || p->G == 0 || p->chunk == 0) return ORC_ERR_ARG;
  if (p->abits != 8 || p->prec != PREC) return ORC_ERR_ARG;
  if (p->nlev < 1 || p->nlev > 4) return ORC_ERR_ARG;
  for (uint32_t i = 0; i < p->nlev; ++i)
    for (int j = 0; j < 3; ++j)
      if (p->bits[i][j] < 2 || p->bits[i][j] > 6) return ORC_ERR_ARG;
  return ORC_OK;
}

static uint32_t third_of(uint32_t l, uint32_t L) { return (3u * l) / L; } /* R3 */
static uint32_t n_streams(const params *p) { return 2u * p->L * p->C; }
static uint32_t delta_alpha(uint32_t b) { return (1u << b) - 1u; }     /* 2M+1 */
static int32_t delta_m(uint32_t b) { return (int32_t)(1u << (b - 1)) - 1; } /* M */

/* ------------------------------------------------ binary16 <-> binary32 */
/* Exact widening of a binary16 bit pattern. */
float orc_h2f(uint16_t h) {
  const uint32_t sign = (uint32_t)(h >> 15) & 1u;
  const uint32_t exp = (uint32_t)(h >> 10) & 0x1Fu;
  const uint32_t man = (uint32_t)h & 0x3FFu;
  float v;
  if (exp == 0)
    v = ldexpf((float)man, -24); /* zero or subnormal: man * 2^-24 */
  else if (exp == 31)
    v = man ? NAN : INFINITY;
  else
    v = ldexpf((float)(man | 0x400u), (int)exp - 25);
  return sign ? -v : v;
}

/* binary32 -> binary16, round to nearest, ties to even; subnormals kept,
 * overflow to infinity.  Written on the bit patterns. */
uint16_t orc_f2h(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  const uint32_t exp = (u >> 23) & 0xFFu;
  uint32_t man = u & 0x7FFFFFu;
  if (exp == 0xFF) return (uint16_t)(sign | 0x7C00u | (man ? 0x200u : 0u));
  const int e = (int)exp - 127; /* unbiased exponent */
  if (e > 15) return (uint16_t)(sign | 0x7C00u);
  if (e >= -14) {
    /* normal binary16 candidate: keep 10 of 23 fraction bits */
    uint32_t hexp = (uint32_t)(e + 15);
    uint32_t hman = man >> 13;
    const uint32_t rest = man & 0x1FFFu;
    if (rest > 0x1000u || (rest == 0x1000u && (hman & 1u))) {
      hman += 1;
      if (hman == 0x400u) {
        hman = 0;
        hexp += 1;
        if (hexp == 31) return (uint16_t)(sign | 0x7C00u);
      }
    }
    return (uint16_t)(sign | (hexp << 10) | hman);
  }
  /* subnormal (or zero) binary16: the result is q * 2^-24 */
  if (exp == 0) return sign; /* a binary32 zero or subnormal is below 2^-126 */
  man |= 0x800000u;          /* 24-bit significand: value = man * 2^(e-23) */
  /* value / 2^-24 = man * 2^(e+1) = man >> rs with rs = -(e+1) >= 14 */
  const int rs = -(e + 1);
  if (rs >= 25) return sign; /* value <= 2^-26 * (2 - 2^-23): rounds to zero */
  const uint32_t q = man >> rs;
  const uint32_t rem = man & ((1u << rs) - 1u);
  const uint32_t half = 1u << (rs - 1);
  uint32_t r = q;
  if (rem > half || (rem == half && (q & 1u))) r += 1;
  return (uint16_t)(sign | r); /* r may reach 0x400: the smallest normal */
}

/* --------------------------------------------------------------- FNV-1a */
/* 64-bit FNV-1a (Fowler, Noll, Vo): offset basis and prime as published. */
#define FNV_OFFSET 0xcbf29ce484222325ull
#define FNV_PRIME 0x100000001b3ull
uint64_t orc_fnv1a64(const uint8_t *data, uint64_t n, uint64_t h) {
  for (uint64_t i = 0; i < n; ++i) {
    h ^= data[i];
    h *= FNV_PRIME;
  }
  return h;
}
static uint64_t fnv_u16(uint64_t h, uint16_t v) {
  const uint8_t b[2] = {(uint8_t)v, (uint8_t)(v >> 8)};
  return orc_fnv1a64(b, 2, h);
}
static uint64_t fnv_u32(uint64_t h, uint32_t v) {
  const uint8_t b[4] = {(uint8_t)v, (uint8_t)(v >> 8), (uint8_t)(v >> 16), (uint8_t)(v >> 24)};
  return orc_fnv1a64(b, 4, h);
}
static uint64_t fnv_u64(uint64_t h, uint64_t v) {
  h = fnv_u32(h, (uint32_t)v);
  return fnv_u32(h, (uint32_t)(v >> 32));
}

/* ------------------------------------------------------ quantizer (R1, R2) */
/*
 * Quantize one stream x[0..n-1] (binary32 values widened from binary16).
 * Anchors are tokens j with j % G == 0 (change-based encoding: groups of G
 * tokens, the first is the anchor).  Outputs the stream's side information
 * (lo, sa, dl) and its symbol sequence in token order: anchor symbols in
 * [0, 255], delta symbols in [0, 2M] (q + M).
 */
int orc_quantize(const float *x, uint32_t n, uint32_t G, uint32_t dbits, float *lo_out,
                 float *sa_out, float *dl_out, int32_t *sym) {
  for (uint32_t j = 0; j < n; ++j)
    if (!isfinite(x[j])) return ORC_ERR_NONFINITE;
  /* anchors: 8-bit affine quantizer over [min, max] of this stream's anchors */
  float lo = x[0], hi = x[0];
  for (uint32_t j = G; j < n; j += G) {
    if (x[j] < lo) lo = x[j];
    if (x[j] > hi) hi = x[j];
  }
  const float sa = (hi - lo) / 255.0f;
  /* closed loop: reconstruct every anchor first */
  float maxabs = 0.0f;
  for (uint32_t j = 0; j < n; ++j) {
    const uint32_t g0 = j - (j % G);
    if (j == g0) {
      int qa = 0;
      if (sa != 0.0f) {
        const float v = rintf((x[j] - lo) / sa);
        qa = (int)v;
        if (qa < 0) qa = 0;
        if (qa > 255) qa = 255;
      }
      sym[j] = qa;
    } else {
      const float ahat = fmaf((float)sym[g0], sa, lo);
      const float d = x[j] - ahat;
      const float a = fabsf(d);
      if (a > maxabs) maxabs = a;
    }
  }
  const int32_t M = delta_m(dbits);
  const float dl = maxabs / (float)M;
  for (uint32_t j = 0; j < n; ++j) {
    const uint32_t g0 = j - (j % G);
    if (j == g0) continue;
    const float ahat = fmaf((float)sym[g0], sa, lo);
    const float d = x[j] - ahat;
    int q = 0;
    if (dl != 0.0f) {
      const float v = rintf(d / dl);
      q = (int)v;
      if (q < -M) q = -M;
      if (q > M) q = M;
    }
    sym[j] = q + M;
  }
  *lo_out = lo;
  *sa_out = sa;
  *dl_out = dl;
  return ORC_OK;
}

/* Reconstruction: one binary32 fma per element, then binary16 RNE.
 * Anchor token: fp16(ahat), ahat = fma(qa, sa, lo).
 * Delta token:  fp16(fma(q, dl, ahat)) with the binary32 ahat. */
void orc_dequantize(const int32_t *sym, uint32_t n, uint32_t G, uint32_t dbits, float lo,
                    float sa, float dl, uint16_t *out) {
  const int32_t M = delta_m(dbits);
  float ahat = 0.0f;
  for (uint32_t j = 0; j < n; ++j) {
    if (j % G == 0) {
      ahat = fmaf((float)sym[j], sa, lo);
      out[j] = orc_f2h(ahat);
    } else {
      const float v = fmaf((float)(sym[j] - M), dl, ahat);
      out[j] = orc_f2h(v);
    }
  }
}

/* ------------------------------------------------- normalisation (R5) */
/* Counts -> frequencies summing to 2^15, every frequency at least 1. */
void orc_normalize(const uint64_t *counts, uint32_t A, uint32_t *f) {
  uint64_t N = 0;
  for (uint32_t s = 0; s < A; ++s) N += counts[s];
  if (N == 0) {
    for (uint32_t s = 0; s < A; ++s) f[s] = TOT / A + (s < TOT % A ? 1u : 0u);
    return;
  }
  uint64_t sum = 0;
  uint32_t arg = 0;
  for (uint32_t s = 0; s < A; ++s) {
    f[s] = 1u + (uint32_t)((counts[s] * (uint64_t)(TOT - A)) / N);
    sum += f[s];
    if (counts[s] > counts[arg]) arg = s;
  }
  f[arg] += (uint32_t)(TOT - sum);
}

/* ------------------------------------------------------ range coder (R4) */
typedef struct {
  const uint32_t *fA; /* anchor frequencies, 256 entries */
  const uint32_t *fD; /* delta frequencies, AD entries */
  uint32_t AD;
  uint32_t G;
} model_pair;

/* cumulative frequency below symbol s, by summation */
static uint32_t cum_below(const uint32_t *f, uint32_t s) {
  uint32_t c = 0;
  for (uint32_t k = 0; k < s; ++k) c += f[k];
  return c;
}

/*
 * Encode n symbols.  Symbol j uses the anchor model iff j % G == 0, else the
 * delta model.  Returns the number of bytes written, or a negative error.
 */
int64_t orc_rc_encode(const int32_t *sym, uint32_t n, uint32_t G, const uint32_t *fA,
                      uint32_t AA, const uint32_t *fD, uint32_t AD, uint8_t *out, uint64_t cap) {
  uint64_t low = 0;
  uint32_t range = 0xFFFFFFFFu;
  uint64_t pos = 0;
  for (uint32_t j = 0; j < n; ++j) {
    const int anchor = (j % G) == 0;
    const uint32_t *f = anchor ? fA : fD;
    const uint32_t A = anchor ? AA : AD;
    if (sym[j] < 0 || (uint32_t)sym[j] >= A) return ORC_ERR_ARG;
    const uint32_t s = (uint32_t)sym[j];
    const uint32_t r = range >> PREC;
    low += (uint64_t)r * cum_below(f, s);
    range = r * f[s];
    if (low >= (1ull << 32)) {
      /* carry into the bytes already emitted */
      low -= (1ull << 32);
      uint64_t k = pos;
      for (;;) {
        if (k == 0) return ORC_ERR_CORRUPT; /* carry past the first byte: impossible */
        --k;
        out[k] = (uint8_t)(out[k] + 1u);
        if (out[k] != 0) break;
      }
    }
    while (range < (1u << 24)) {
      if (pos >= cap) return ORC_ERR_CAPACITY;
      out[pos++] = (uint8_t)(low >> 24);
      low = (low << 8) & 0xFFFFFFFFull;
      range <<= 8;
    }
  }
  for (int i = 0; i < 4; ++i) {
    if (pos >= cap) return ORC_ERR_CAPACITY;
    out[pos++] = (uint8_t)(low >> 24);
    low = (low << 8) & 0xFFFFFFFFull;
  }
  return (int64_t)pos;
}

/* Decode n symbols from exactly nbytes bytes; any inconsistency is
 * reported as a corrupt stream. */
/* The decoder as a state machine, one symbol per step (the reference reader
 * of R17 interleaves the steps of several streams). */
typedef struct {
  uint32_t code, range;
  uint64_t pos; /* bytes consumed */
} rc_dec;

static int rc_dec_init(rc_dec *d, const uint8_t *in, uint64_t nbytes) {
  if (nbytes < 4) return ORC_ERR_CORRUPT;
  d->code = ((uint32_t)in[0] << 24) | ((uint32_t)in[1] << 16) | ((uint32_t)in[2] << 8) |
            (uint32_t)in[3];
  d->range = 0xFFFFFFFFu;
  d->pos = 4;
  return ORC_OK;
}

static int rc_dec_step(rc_dec *d, const uint8_t *in, uint64_t nbytes, const uint32_t *f,
                       uint32_t A, int32_t *sym) {
  const uint32_t r = d->range >> PREC;
  const uint32_t t = d->code / r;
  if (t >= TOT) return ORC_ERR_CORRUPT;
  /* linear search for the symbol whose interval holds t */
  uint32_t s = 0, c = 0;
  while (s < A && c + f[s] <= t) {
    c += f[s];
    ++s;
  }
  if (s >= A) return ORC_ERR_CORRUPT;
  d->code -= r * c;
  d->range = r * f[s];
  *sym = (int32_t)s;
  while (d->range < (1u << 24)) {
    if (d->pos >= nbytes) return ORC_ERR_CORRUPT;
    d->code = (d->code << 8) | in[d->pos++];
    d->range <<= 8;
  }
  return ORC_OK;
}

int orc_rc_decode(const uint8_t *in, uint64_t nbytes, uint32_t n, uint32_t G,
                  const uint32_t *fA, uint32_t AA, const uint32_t *fD, uint32_t AD,
                  int32_t *sym) {
  rc_dec d;
  int st = rc_dec_init(&d, in, nbytes);
  if (st) return st;
  for (uint32_t j = 0; j < n; ++j) {
    const int anchor = (j % G) == 0;
    st = rc_dec_step(&d, in, nbytes, anchor ? fA : fD, anchor ? AA : AD, &sym[j]);
    if (st) return st;
  }
  if (d.pos != nbytes) return ORC_ERR_CORRUPT;
  return ORC_OK;
}

/* Bytes shifted in by each symbol of a stream (k[j] in 0..2), for checks of
 * the reference reader; same arguments as orc_rc_decode. */
int orc_rc_shifts(const uint8_t *in, uint64_t nbytes, uint32_t n, uint32_t G, const uint32_t *fA,
                  uint32_t AA, const uint32_t *fD, uint32_t AD, uint8_t *k) {
  rc_dec d;
  int st = rc_dec_init(&d, in, nbytes);
  if (st) return st;
  for (uint32_t j = 0; j < n; ++j) {
    const int anchor = (j % G) == 0;
    const uint64_t before = d.pos;
    int32_t s;
    st = rc_dec_step(&d, in, nbytes, anchor ? fA : fD, anchor ? AA : AD, &s);
    if (st) return st;
    k[j] = (uint8_t)(d.pos - before);
  }
  return d.pos == nbytes ? ORC_OK : ORC_ERR_CORRUPT;
}

/* ---------------------------------------------------------- tables / ids */
/* Frequency tables as the oracle keeps them:
 *   fA[m][256]                    anchor model of stream m
 *   fD[level][m][64]              delta model (first 2^b - 1 entries used)
 * with m = (l*2 + kv)*C + c.                                              */

static uint64_t desc_hash(const params *p) {
  uint64_t h = FNV_OFFSET;
  h = fnv_u32(h, p->L);
  h = fnv_u32(h, p->C);
  h = fnv_u32(h, p->G);
  h = fnv_u32(h, p->chunk);
  h = fnv_u32(h, p->abits);
  h = fnv_u32(h, p->nlev);
  h = fnv_u32(h, p->prec);
  for (uint32_t i = 0; i < p->nlev; ++i)
    for (int j = 0; j < 3; ++j) {
      const uint8_t b = (uint8_t)p->bits[i][j];
      h = orc_fnv1a64(&b, 1, h);
    }
  return h;
}

/* profile id: FNV-1a over (descriptor, then for each (layer, K/V) row the
 * FNV-1a of that row's per-model FNV-1a values); a model's value covers its
 * anchor frequencies then its delta frequencies level by level (u16, LE). */
uint64_t orc_profile_id(const uint32_t *pw, const uint16_t *fA, const uint16_t *fD) {
  params p;
  if (read_params(pw, &p)) return 0;
  const uint32_t S = n_streams(&p);
  uint64_t h = desc_hash(&p);
  for (uint32_t row = 0; row < 2 * p.L; ++row) {
    const uint32_t l = row / 2;
    uint64_t hr = FNV_OFFSET;
    for (uint32_t c = 0; c < p.C; ++c) {
      const uint32_t m = row * p.C + c;
      uint64_t hm = FNV_OFFSET;
      for (uint32_t s = 0; s < ANCHOR_ALPHA; ++s) hm = fnv_u16(hm, fA[(size_t)m * ANCHOR_ALPHA + s]);
      for (uint32_t lv = 0; lv < p.nlev; ++lv) {
        const uint32_t A = delta_alpha(p.bits[lv][third_of(l, p.L)]);
        const uint16_t *f = fD + ((size_t)lv * S + m) * MAX_DELTA_ALPHA;
        for (uint32_t s = 0; s < A; ++s) hm = fnv_u16(hm, f[s]);
      }
      hr = fnv_u64(hr, hm);
    }
    h = fnv_u64(h, hr);
  }
  return h;
}

static void widen_stream(const uint16_t *kv, const params *p, uint32_t T, uint32_t m,
                         uint32_t t0, uint32_t n, float *x) {
  const uint32_t row = m / p->C, c = m % p->C;
  const uint16_t *base = kv + (size_t)row * T * p->C;
  for (uint32_t j = 0; j < n; ++j) x[j] = orc_h2f(base[(size_t)(t0 + j) * p->C + c]);
}

/*
 * Offline profiling: for every profiling chunk and every stream,
 * quantize (anchors once, deltas once per level), count symbols per model,
 * normalise.  kv: binary16 [L][2][T][C], chunked by chunk_tokens.
 */
int orc_profile(const uint32_t *pw, const uint16_t *kv, uint32_t T, uint16_t *fA, uint16_t *fD,
                uint64_t *profile_id) {
  params p;
  int st = read_params(pw, &p);
  if (st) return st;
  if (T == 0) return ORC_ERR_SHAPE;
  const uint32_t S = n_streams(&p);
  const uint32_t nchunks = (T + p.chunk - 1) / p.chunk;
  int err = ORC_OK;
#pragma omp parallel for schedule(dynamic, 16)
  for (long mm = 0; mm < (long)S; ++mm) {
    const uint32_t m = (uint32_t)mm;
    const uint32_t l = m / (2 * p.C);
    float *x = (float *)malloc(sizeof(float) * p.chunk);
    int32_t *sym = (int32_t *)malloc(sizeof(int32_t) * p.chunk);
    uint64_t ca[ANCHOR_ALPHA];
    uint64_t cd[4][MAX_DELTA_ALPHA];
    memset(ca, 0, sizeof ca);
    memset(cd, 0, sizeof cd);
    for (uint32_t k = 0; k < nchunks; ++k) {
      const uint32_t t0 = k * p.chunk;
      const uint32_t n = (T - t0 < p.chunk) ? T - t0 : p.chunk;
      widen_stream(kv, &p, T, m, t0, n, x);
      for (uint32_t lv = 0; lv < p.nlev; ++lv) {
        const uint32_t b = p.bits[lv][third_of(l, p.L)];
        float lo, sa, dl;
        if (orc_quantize(x, n, p.G, b, &lo, &sa, &dl, sym)) {
#pragma omp atomic write
          err = ORC_ERR_NONFINITE;
          break;
        }
        for (uint32_t j = 0; j < n; ++j) {
          if (j % p.G == 0) {
            if (lv == 0) ca[sym[j]]++; /* anchors do not depend on the level */
          } else {
            cd[lv][sym[j]]++;
          }
        }
      }
    }
    uint32_t f[ANCHOR_ALPHA];
    orc_normalize(ca, ANCHOR_ALPHA, f);
    for (uint32_t s = 0; s < ANCHOR_ALPHA; ++s) fA[(size_t)m * ANCHOR_ALPHA + s] = (uint16_t)f[s];
    for (uint32_t lv = 0; lv < p.nlev; ++lv) {
      const uint32_t A = delta_alpha(p.bits[lv][third_of(l, p.L)]);
      orc_normalize(cd[lv], A, f);
      uint16_t *dst = fD + ((size_t)lv * S + m) * MAX_DELTA_ALPHA;
      for (uint32_t s = 0; s < MAX_DELTA_ALPHA; ++s) dst[s] = (uint16_t)(s < A ? f[s] : 0u);
    }
    free(x);
    free(sym);
  }
  if (err) return err;
  *profile_id = orc_profile_id(pw, fA, fD);
  return ORC_OK;
}

/* ------------------------------------------------------- container (R6) */
static void put_u16(uint8_t *b, uint16_t v) { b[0] = (uint8_t)v; b[1] = (uint8_t)(v >> 8); }
static void put_u32(uint8_t *b, uint32_t v) {
  for (int i = 0; i < 4; ++i) b[i] = (uint8_t)(v >> (8 * i));
}
static void put_u64(uint8_t *b, uint64_t v) {
  for (int i = 0; i < 8; ++i) b[i] = (uint8_t)(v >> (8 * i));
}
static uint16_t get_u16(const uint8_t *b) { return (uint16_t)(b[0] | (b[1] << 8)); }
static uint32_t get_u32(const uint8_t *b) {
  uint32_t v = 0;
  for (int i = 3; i >= 0; --i) v = (v << 8) | b[i];
  return v;
}
static uint64_t get_u64(const uint8_t *b) {
  uint64_t v = 0;
  for (int i = 7; i >= 0; --i) v = (v << 8) | b[i];
  return v;
}
static void put_f32(uint8_t *b, float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  put_u32(b, u);
}
static float get_f32(const uint8_t *b) {
  const uint32_t u = get_u32(b);
  float f;
  memcpy(&f, &u, 4);
  return f;
}
static uint64_t pad8(uint64_t v) { return (v + 7u) & ~(uint64_t)7u; }

/* the container's upper size bound for n tokens: each symbol emits at most
 * two bytes, plus the 4-byte flush, rounded up to whole 8-byte blocks */
uint64_t orc_container_bound(const uint32_t *pw, uint32_t n) {
  params p;
  if (read_params(pw, &p)) return 0;
  return HDR_BYTES + (uint64_t)REC_BYTES * n_streams(&p) +
         (uint64_t)n_streams(&p) * pad8(4u + 2u * (uint64_t)n);
}

static void widen_freqs(const uint16_t *src, uint32_t A, uint32_t *dst) {
  for (uint32_t s = 0; s < A; ++s) dst[s] = src[s];
}

/* ------------------------------------------------------------ units (R6) */
#define UNIT_LANES 64u
#define BLOCK 8u

static uint32_t n_units(const params *p) {
  return 2u * p->L * ((p->C + UNIT_LANES - 1) / UNIT_LANES);
}
/* first stream and stream count of unit u */
static void unit_span(const params *p, uint32_t u, uint32_t *m0, uint32_t *nv) {
  const uint32_t ncb = (p->C + UNIT_LANES - 1) / UNIT_LANES;
  const uint32_t row = u / ncb, cb = u % ncb;
  *m0 = row * p->C + cb * UNIT_LANES;
  *nv = (p->C - cb * UNIT_LANES < UNIT_LANES) ? p->C - cb * UNIT_LANES : UNIT_LANES;
}

/*
 * R17: the reference reader of one unit, which fixes the order of the unit's
 * 8-byte blocks in the payload.  Every lane l (stream m0 + l) decodes its
 * stream; R is the number of bytes its decoder has consumed, W the number of
 * bytes it holds ready (the "delivered" blocks), q the next block it has not
 * asked for.  A request hands out the next payload slot, lanes in increasing
 * order within a step:
 *   - start: every lane asks for its blocks 0, 1 and 2 (block index outer,
 *     lane inner); W = 16, R = 4;
 *   - before token j, every lane for which
 *       j % G == 0 ? W - R <= 8 : W - R < 2
 *     takes its next block (W += 8) and asks for block q (q += 1), if its
 *     stream has a block q;
 *   - then every lane decodes symbol j (R grows by the bytes it shifts in).
 * A lane never reads a byte it does not hold (W - R >= 2 before a token, a
 * symbol shifts in at most 2 bytes), and never holds more than 16 bytes
 * ahead (W - R <= 16).
 * Encode mode (`streams` given): copies each requested block from the
 * stream's contiguous bytes (zero-padded to whole blocks) into `slots_out`.
 * Decode mode (`slots_in` given): gathers each requested block from the
 * payload into the lane's buffer and decodes from it.  Both decode every
 * symbol (into sym [nv][n] when given) and return ORC_ERR_CORRUPT if a
 * stream does not decode to exactly its nbytes.  `order` (optional) receives
 * lane << 16 | block for every slot.
 */
/* The models one lane's stream is coded with: symbol j uses (fa, AA) when
 * j % G == 0 and (fd, AD) otherwise. */
typedef struct {
  uint32_t fa[ANCHOR_ALPHA], fd[MAX_DELTA_ALPHA];
  uint32_t AA, AD;
} lane_models;

static int unit_reader_models(const params *p, const lane_models *mods, uint32_t nv, uint32_t n,
                              const uint32_t *nb, const uint8_t *const *streams,
                              const uint8_t *slots_in, uint64_t n_slots, uint8_t *slots_out,
                              int32_t *sym, uint32_t *order) {
  uint32_t nblk[UNIT_LANES], q[UNIT_LANES], W[UNIT_LANES];
  uint8_t *own[UNIT_LANES];
  const uint8_t *buf[UNIT_LANES];
  rc_dec dec[UNIT_LANES];
  int err = ORC_OK;
  for (uint32_t l = 0; l < nv; ++l) {
    nblk[l] = (uint32_t)(pad8(nb[l]) / BLOCK);
    q[l] = 0;
    W[l] = 16;
    own[l] = NULL;
    if (streams) {
      buf[l] = streams[l];
    } else {
      own[l] = (uint8_t *)calloc((size_t)nblk[l] + 1, BLOCK);
      buf[l] = own[l];
    }
  }
  uint64_t next = 0;
#define REQUEST(l)                                                                     \
  do {                                                                                 \
    if (q[l] < nblk[l]) {                                                              \
      const uint64_t slot = next++;                                                    \
      if (slot >= n_slots) {                                                           \
        err = ORC_ERR_CORRUPT;                                                         \
      } else if (streams) {                                                            \
        memcpy(slots_out + slot * BLOCK, buf[l] + (size_t)q[l] * BLOCK, BLOCK);        \
      } else {                                                                         \
        memcpy(own[l] + (size_t)q[l] * BLOCK, slots_in + slot * BLOCK, BLOCK);         \
      }                                                                                \
      if (order && slot < n_slots) order[slot] = (l << 16) | q[l];                     \
      ++q[l];                                                                          \
    }                                                                                  \
  } while (0)
  for (uint32_t blk = 0; blk < 3; ++blk)
    for (uint32_t l = 0; l < nv; ++l) REQUEST(l);
  for (uint32_t l = 0; l < nv && !err; ++l) err = rc_dec_init(&dec[l], buf[l], nb[l]);
  for (uint32_t j = 0; j < n && !err; ++j) {
    const int anchor = (j % p->G) == 0;
    for (uint32_t l = 0; l < nv; ++l) {
      const uint64_t ahead = W[l] - dec[l].pos; /* R <= W always */
      if (anchor ? ahead <= 8 : ahead < 2) {
        W[l] += BLOCK;
        REQUEST(l);
      }
    }
    for (uint32_t l = 0; l < nv && !err; ++l) {
      int32_t s;
      err = anchor ? rc_dec_step(&dec[l], buf[l], nb[l], mods[l].fa, mods[l].AA, &s)
                   : rc_dec_step(&dec[l], buf[l], nb[l], mods[l].fd, mods[l].AD, &s);
      if (sym) sym[(size_t)l * n + j] = s;
    }
  }
#undef REQUEST
  for (uint32_t l = 0; l < nv && !err; ++l)
    if (dec[l].pos != nb[l]) err = ORC_ERR_CORRUPT;
  if (!err && next != n_slots) err = ORC_ERR_CORRUPT; /* every block asked for once */
  for (uint32_t l = 0; l < nv; ++l) free(own[l]);
  return err;
}

/* The base layer's models of the unit's lanes at `level`. */
static int unit_reader(const params *p, const uint16_t *fA, const uint16_t *fD, uint32_t level,
                       uint32_t m0, uint32_t nv, uint32_t n, const uint32_t *nb,
                       const uint8_t *const *streams, const uint8_t *slots_in, uint64_t n_slots,
                       uint8_t *slots_out, int32_t *sym, uint32_t *order) {
  const uint32_t S = n_streams(p);
  lane_models *mods = (lane_models *)malloc(sizeof(lane_models) * UNIT_LANES);
  if (!mods) return ORC_ERR_CAPACITY;
  for (uint32_t l = 0; l < nv; ++l) {
    const uint32_t m = m0 + l;
    const uint32_t b = p->bits[level][third_of(m / (2 * p->C), p->L)];
    mods[l].AA = ANCHOR_ALPHA;
    mods[l].AD = delta_alpha(b);
    widen_freqs(fA + (size_t)m * ANCHOR_ALPHA, ANCHOR_ALPHA, mods[l].fa);
    widen_freqs(fD + ((size_t)level * S + m) * MAX_DELTA_ALPHA, mods[l].AD, mods[l].fd);
  }
  const int err = unit_reader_models(p, mods, nv, n, nb, streams, slots_in, n_slots, slots_out,
                                     sym, order);
  free(mods);
  return err;
}

/*
 * Encode chunk `chunk` (tokens [chunk*chunk_tokens, +n)) of kv [L][2][T][C]
 * at compression level `level` into one container.  Returns its size in
 * bytes, or a negative error.
 */
int64_t orc_encode_chunk(const uint32_t *pw, const uint16_t *fA, const uint16_t *fD,
                         uint64_t profile_id, const uint16_t *kv, uint32_t T, uint32_t chunk,
                         uint32_t level, uint8_t *out, uint64_t cap) {
  params p;
  int st = read_params(pw, &p);
  if (st) return st;
  if (level >= p.nlev) return ORC_ERR_ARG;
  const uint64_t t0 = (uint64_t)chunk * p.chunk;
  if (t0 >= T) return ORC_ERR_SHAPE;
  const uint32_t n = (uint32_t)((T - t0 < p.chunk) ? T - t0 : p.chunk);
  const uint32_t S = n_streams(&p);
  const uint64_t slot = pad8(4u + 2u * (uint64_t)n);
  uint8_t *scratch = (uint8_t *)calloc((size_t)S, (size_t)slot);
  float *side = (float *)malloc(sizeof(float) * 3u * S);
  uint32_t *nb = (uint32_t *)malloc(sizeof(uint32_t) * S);
  if (!scratch || !side || !nb) {
    free(scratch);
    free(side);
    free(nb);
    return ORC_ERR_CAPACITY;
  }
  int err = ORC_OK;
  /* every stream's bytes, contiguous */
#pragma omp parallel for schedule(dynamic, 16)
  for (long mm = 0; mm < (long)S; ++mm) {
    const uint32_t m = (uint32_t)mm;
    const uint32_t l = m / (2 * p.C);
    const uint32_t b = p.bits[level][third_of(l, p.L)];
    float *x = (float *)malloc(sizeof(float) * n);
    int32_t *sym = (int32_t *)malloc(sizeof(int32_t) * n);
    uint32_t fa[ANCHOR_ALPHA], fd[MAX_DELTA_ALPHA];
    widen_stream(kv, &p, T, m, (uint32_t)t0, n, x);
    int e = orc_quantize(x, n, p.G, b, &side[3 * m], &side[3 * m + 1], &side[3 * m + 2], sym);
    if (!e) {
      widen_freqs(fA + (size_t)m * ANCHOR_ALPHA, ANCHOR_ALPHA, fa);
      widen_freqs(fD + ((size_t)level * S + m) * MAX_DELTA_ALPHA, delta_alpha(b), fd);
      const int64_t w = orc_rc_encode(sym, n, p.G, fa, ANCHOR_ALPHA, fd, delta_alpha(b),
                                      scratch + (size_t)m * slot, slot);
      if (w < 0)
        e = (int)w;
      else
        nb[m] = (uint32_t)w;
    }
    if (e) {
#pragma omp critical
      err = e;
    }
    free(x);
    free(sym);
  }
  if (err) {
    free(scratch);
    free(side);
    free(nb);
    return err;
  }
  uint64_t payload = 0;
  for (uint32_t m = 0; m < S; ++m) payload += pad8(nb[m]);
  const uint64_t total = HDR_BYTES + (uint64_t)REC_BYTES * S + payload;
  if (total > cap) {
    free(scratch);
    free(side);
    free(nb);
    return ORC_ERR_CAPACITY;
  }
  memset(out, 0, (size_t)total);
  /* header */
  memcpy(out, "KVC1", 4);
  put_u16(out + 4, 2);
  out[6] = (uint8_t)level;
  out[7] = (uint8_t)p.abits;
  put_u16(out + 8, (uint16_t)p.G);
  out[10] = (uint8_t)p.prec;
  for (int j = 0; j < 3; ++j) out[11 + j] = (uint8_t)p.bits[level][j];
  put_u32(out + 16, p.L);
  put_u32(out + 20, p.C);
  put_u32(out + 24, n);
  put_u32(out + 28, (uint32_t)t0);
  put_u64(out + 32, profile_id);
  put_u64(out + 40, payload);
  put_u32(out + 48, p.chunk);
  put_u32(out + 52, S);
  /* records */
  for (uint32_t m = 0; m < S; ++m) {
    uint8_t *rec = out + HDR_BYTES + (size_t)REC_BYTES * m;
    put_f32(rec, side[3 * m]);
    put_f32(rec + 4, side[3 * m + 1]);
    put_f32(rec + 8, side[3 * m + 2]);
    put_u32(rec + 12, nb[m]);
  }
  /* payload: each unit's blocks in the reference reader's order (R17) */
  uint64_t *uoff = (uint64_t *)malloc(sizeof(uint64_t) * (n_units(&p) + 1));
  uoff[0] = 0;
  for (uint32_t u = 0; u < n_units(&p); ++u) {
    uint32_t m0, nv;
    unit_span(&p, u, &m0, &nv);
    uint64_t sz = 0;
    for (uint32_t l = 0; l < nv; ++l) sz += pad8(nb[m0 + l]);
    uoff[u + 1] = uoff[u] + sz;
  }
  uint8_t *pay = out + HDR_BYTES + (size_t)REC_BYTES * S;
#pragma omp parallel for schedule(dynamic, 4)
  for (long uu = 0; uu < (long)n_units(&p); ++uu) {
    const uint32_t u = (uint32_t)uu;
    uint32_t m0, nv;
    unit_span(&p, u, &m0, &nv);
    const uint8_t *streams[UNIT_LANES];
    for (uint32_t l = 0; l < nv; ++l) streams[l] = scratch + (size_t)(m0 + l) * slot;
    const int e = unit_reader(&p, fA, fD, level, m0, nv, n, nb + m0, streams, NULL,
                              (uoff[u + 1] - uoff[u]) / BLOCK, pay + uoff[u], NULL, NULL);
    if (e) {
#pragma omp critical
      err = e;
    }
  }
  free(uoff);
  free(scratch);
  free(side);
  free(nb);
  return err ? err : (int64_t)total;
}

/* ------------------------------------------------------ decode */
typedef struct {
  uint32_t n, level;
  uint64_t payload;
} chunk_hdr;

static int check_header(const params *p, uint64_t profile_id, const uint8_t *c, uint64_t nbytes,
                        chunk_hdr *h) {
  const uint32_t S = n_streams(p);
  if (nbytes < HDR_BYTES + (uint64_t)REC_BYTES * S) return ORC_ERR_CORRUPT;
  if (memcmp(c, "KVC1", 4) != 0 || get_u16(c + 4) != 2) return ORC_ERR_CORRUPT;
  h->level = c[6];
  h->n = get_u32(c + 24);
  h->payload = get_u64(c + 40);
  if (h->level >= p->nlev || c[7] != p->abits || get_u16(c + 8) != p->G || c[10] != p->prec)
    return ORC_ERR_CORRUPT;
  for (int j = 0; j < 3; ++j)
    if (c[11 + j] != p->bits[h->level][j]) return ORC_ERR_CORRUPT;
  if (get_u32(c + 16) != p->L || get_u32(c + 20) != p->C || get_u32(c + 48) != p->chunk ||
      get_u32(c + 52) != S)
    return ORC_ERR_CORRUPT;
  if (h->n == 0 || h->n > p->chunk) return ORC_ERR_CORRUPT;
  if (get_u64(c + 32) != profile_id) return ORC_ERR_PROFILE;
  if (HDR_BYTES + (uint64_t)REC_BYTES * S + h->payload != nbytes) return ORC_ERR_CORRUPT;
  uint64_t sum = 0;
  for (uint32_t m = 0; m < S; ++m) sum += pad8(get_u32(c + HDR_BYTES + (size_t)REC_BYTES * m + 12));
  if (sum != h->payload) return ORC_ERR_CORRUPT;
  return ORC_OK;
}

/* Per-stream block offsets of a container (relative to the payload start):
 * the exclusive prefix sum of the streams' lengths rounded up to whole
 * 8-byte blocks.  A unit's payload starts at its first stream's offset. */
int orc_stream_offsets(const uint32_t *pw, const uint8_t *c, uint64_t nbytes, uint32_t *offs) {
  params p;
  int st = read_params(pw, &p);
  if (st) return st;
  const uint32_t S = n_streams(&p);
  if (nbytes < HDR_BYTES + (uint64_t)REC_BYTES * S) return ORC_ERR_CORRUPT;
  uint64_t acc = 0;
  for (uint32_t m = 0; m < S; ++m) {
    offs[m] = (uint32_t)acc;
    acc += pad8(get_u32(c + HDR_BYTES + (size_t)REC_BYTES * m + 12));
  }
  return ORC_OK;
}

/* Run the reference reader over unit u of a checked container: symbols
 * [nv][n], and optionally each lane's contiguous stream bytes (`bytes`,
 * nv pointers of pad8(nbytes) bytes) and the slot order. */
static int read_unit(const params *p, const uint16_t *fA, const uint16_t *fD, const uint8_t *c,
                     const chunk_hdr *h, const uint32_t *offs, uint32_t u, int32_t *sym,
                     uint32_t *order) {
  const uint32_t S = n_streams(p);
  uint32_t m0, nv, nb[UNIT_LANES];
  unit_span(p, u, &m0, &nv);
  uint64_t sz = 0;
  for (uint32_t l = 0; l < nv; ++l) {
    nb[l] = get_u32(c + HDR_BYTES + (size_t)REC_BYTES * (m0 + l) + 12);
    sz += pad8(nb[l]);
  }
  const uint8_t *pay = c + HDR_BYTES + (size_t)REC_BYTES * S + offs[m0];
  return unit_reader(p, fA, fD, h->level, m0, nv, h->n, nb, NULL, pay, sz / BLOCK, NULL, sym,
                     order);
}

static void dequantize_lane(const params *p, const uint8_t *c, const chunk_hdr *h, uint32_t m,
                            const int32_t *sym, uint16_t *vals) {
  const uint32_t l = m / (2 * p->C);
  const uint32_t b = p->bits[h->level][third_of(l, p->L)];
  const uint8_t *rec = c + HDR_BYTES + (size_t)REC_BYTES * m;
  orc_dequantize(sym, h->n, p->G, b, get_f32(rec), get_f32(rec + 4), get_f32(rec + 8), vals);
}

/*
 * Decode one container into out [L][2][T_total][C] at tokens
 * [first_token, first_token + n).  `level` and `n_tokens` must match the
 * header (they are what the caller asked to fetch).
 */
int orc_decode_chunk(const uint32_t *pw, const uint16_t *fA, const uint16_t *fD,
                     uint64_t profile_id, const uint8_t *c, uint64_t nbytes, uint32_t first_token,
                     uint32_t n_tokens, uint32_t level, uint16_t *out, uint32_t T_total) {
  params p;
  int st = read_params(pw, &p);
  if (st) return st;
  chunk_hdr h;
  st = check_header(&p, profile_id, c, nbytes, &h);
  if (st) return st;
  if (h.n != n_tokens || h.level != level) return ORC_ERR_ARG;
  if ((uint64_t)first_token + n_tokens > T_total) return ORC_ERR_SHAPE;
  const uint32_t S = n_streams(&p);
  uint32_t *offs = (uint32_t *)malloc(sizeof(uint32_t) * S);
  orc_stream_offsets(pw, c, nbytes, offs);
  int err = ORC_OK;
#pragma omp parallel for schedule(dynamic, 4)
  for (long uu = 0; uu < (long)n_units(&p); ++uu) {
    const uint32_t u = (uint32_t)uu;
    uint32_t m0, nv;
    unit_span(&p, u, &m0, &nv);
    int32_t *sym = (int32_t *)malloc(sizeof(int32_t) * (size_t)nv * h.n);
    uint16_t *vals = (uint16_t *)malloc(sizeof(uint16_t) * h.n);
    const int e = read_unit(&p, fA, fD, c, &h, offs, u, sym, NULL);
    if (e) {
#pragma omp critical
      err = e;
    } else {
      for (uint32_t l = 0; l < nv; ++l) {
        const uint32_t m = m0 + l;
        dequantize_lane(&p, c, &h, m, sym + (size_t)l * h.n, vals);
        const uint32_t row = m / p.C, ch = m % p.C;
        uint16_t *dst = out + (size_t)row * T_total * p.C;
        for (uint32_t j = 0; j < h.n; ++j) dst[(size_t)(first_token + j) * p.C + ch] = vals[j];
      }
    }
    free(sym);
    free(vals);
  }
  free(offs);
  return err;
}

/* Decode selected streams of one container: values [count][n] (binary16)
 * and symbols [count][n]; for checks at sizes too large to decode whole
 * (each stream's whole unit is read). */
int orc_decode_streams(const uint32_t *pw, const uint16_t *fA, const uint16_t *fD,
                       uint64_t profile_id, const uint8_t *c, uint64_t nbytes,
                       const uint32_t *ids, uint32_t count, uint16_t *vals, int32_t *syms) {
  params p;
  int st = read_params(pw, &p);
  if (st) return st;
  chunk_hdr h;
  st = check_header(&p, profile_id, c, nbytes, &h);
  if (st) return st;
  const uint32_t S = n_streams(&p);
  const uint32_t ncb = (p.C + UNIT_LANES - 1) / UNIT_LANES;
  uint32_t *offs = (uint32_t *)malloc(sizeof(uint32_t) * S);
  int32_t *usym = (int32_t *)malloc(sizeof(int32_t) * (size_t)UNIT_LANES * h.n);
  orc_stream_offsets(pw, c, nbytes, offs);
  int err = ORC_OK;
  uint32_t last = 0xFFFFFFFFu; /* the unit whose symbols usym holds */
  for (uint32_t i = 0; i < count && !err; ++i) {
    if (ids[i] >= S) {
      err = ORC_ERR_ARG;
      break;
    }
    const uint32_t m = ids[i];
    const uint32_t u = (m / p.C) * ncb + (m % p.C) / UNIT_LANES;
    uint32_t m0, nv;
    unit_span(&p, u, &m0, &nv);
    if (u != last) {
      err = read_unit(&p, fA, fD, c, &h, offs, u, usym, NULL);
      if (err) break;
      last = u;
    }
    memcpy(syms + (size_t)i * h.n, usym + (size_t)(m - m0) * h.n, sizeof(int32_t) * h.n);
    dequantize_lane(&p, c, &h, m, syms + (size_t)i * h.n, vals + (size_t)i * h.n);
  }
  free(usym);
  free(offs);
  return err;
}

/* For checks of the payload layout: the slot order of unit u (lane << 16 |
 * block per slot; n_slots = the unit's payload bytes / 8) and the unit's
 * number of lanes. */
int orc_unit_order(const uint32_t *pw, const uint16_t *fA, const uint16_t *fD,
                   uint64_t profile_id, const uint8_t *c, uint64_t nbytes, uint32_t u,
                   uint32_t *order, uint64_t order_cap, uint32_t *nv_out) {
  params p;
  int st = read_params(pw, &p);
  if (st) return st;
  chunk_hdr h;
  st = check_header(&p, profile_id, c, nbytes, &h);
  if (st) return st;
  if (u >= n_units(&p)) return ORC_ERR_ARG;
  const uint32_t S = n_streams(&p);
  uint32_t m0, nv;
  unit_span(&p, u, &m0, &nv);
  uint64_t sz = 0;
  for (uint32_t l = 0; l < nv; ++l) sz += pad8(get_u32(c + HDR_BYTES + (size_t)REC_BYTES * (m0 + l) + 12));
  if (sz / BLOCK > order_cap) return ORC_ERR_CAPACITY;
  uint32_t *offs = (uint32_t *)malloc(sizeof(uint32_t) * S);
  orc_stream_offsets(pw, c, nbytes, offs);
  int32_t *sym = (int32_t *)malloc(sizeof(int32_t) * (size_t)nv * h.n);
  st = read_unit(&p, fA, fD, c, &h, offs, u, sym, order);
  free(sym);
  free(offs);
  *nv_out = nv;
  return st;
}

/* The reference reader on an explicit trace, for worked examples: nv lanes
 * with nblk[l] blocks each and per-token shift counts k[l][j] (bytes shifted
 * in by symbol j); writes the slot order (lane << 16 | block) and returns
 * the number of slots, or a negative error.  Mirrors unit_reader's request
 * rule without decoding. */
int64_t orc_block_order_trace(uint32_t nv, uint32_t n, uint32_t G, const uint32_t *nblk,
                              const uint8_t *k, uint32_t *order, uint64_t cap) {
  if (nv > UNIT_LANES) return ORC_ERR_ARG;
  uint32_t q[UNIT_LANES], W[UNIT_LANES], R[UNIT_LANES];
  uint64_t next = 0;
  for (uint32_t l = 0; l < nv; ++l) {
    q[l] = 0;
    W[l] = 16;
    R[l] = 4;
  }
  for (uint32_t blk = 0; blk < 3; ++blk)
    for (uint32_t l = 0; l < nv; ++l)
      if (q[l] < nblk[l]) {
        if (next >= cap) return ORC_ERR_CAPACITY;
        order[next++] = (l << 16) | q[l]++;
      }
  for (uint32_t j = 0; j < n; ++j) {
    const int anchor = (j % G) == 0;
    for (uint32_t l = 0; l < nv; ++l) {
      const uint32_t ahead = W[l] - R[l];
      if (anchor ? ahead <= 8 : ahead < 2) {
        W[l] += BLOCK;
        if (q[l] < nblk[l]) {
          if (next >= cap) return ORC_ERR_CAPACITY;
          order[next++] = (l << 16) | q[l]++;
        }
      }
    }
    for (uint32_t l = 0; l < nv; ++l) R[l] += k[(size_t)l * n + j];
  }
  return (int64_t)next;
}

/* Thread count for the parallel loops (streams are independent, so the
 * results do not depend on it). */
void orc_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
int orc_get_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Array forms of the binary16 conversions, for exhaustive checks. */
void orc_f2h_array(const float *x, uint16_t *out, uint64_t n) {
  for (uint64_t i = 0; i < n; ++i) out[i] = orc_f2h(x[i]);
}
/* Convert the binary32 bit patterns start .. start+n-1 (exhaustive checks). */
void orc_f2h_patterns(uint32_t start, uint64_t n, uint16_t *out) {
#pragma omp parallel for schedule(static)
  for (long long i = 0; i < (long long)n; ++i) {
    const uint32_t u = start + (uint32_t)i;
    float f;
    memcpy(&f, &u, 4);
    out[i] = orc_f2h(f);
  }
}
void orc_h2f_array(const uint16_t *h, float *out, uint64_t n) {
  for (uint64_t i = 0; i < n; ++i) out[i] = orc_h2f(h[i]);
}

/* =========================================================== refinement
 * R19: incremental, SVC-like refinement (CacheGen page, 局限与 Future Work:
 * send a low-quality version of the KV first, then refinement bits).  The
 * page describes no scheme; the reading taken here is a two-layer successive
 * refinement that leaves the base layer untouched:
 *   - the base layer of a chunk is its container at the chosen level, coded
 *     exactly as above;
 *   - the refinement layer quantizes, per stream, the residual
 *       e[j] = x[j] - xh[j]
 *     against the base reconstruction in binary32, before its binary16
 *     rounding (anchors xh = fma(qa, sa, lo); deltas xh = fma(q, dl, ahat)),
 *     with a symmetric mid-tread quantizer of E bits (Me = 2^(E-1) - 1):
 *     one scale over the stream's anchor tokens, Da = max |e| / Me, and one
 *     over its other tokens, Dd = max |e| / Me (the base layer keeps anchors
 *     and deltas apart the same way); q = D == 0 ? 0 : clamp(rint(e / D),
 *     -Me, Me); symbol q + Me in the alphabet 2^E - 1;
 *   - the refinement symbols are range-coded in token order with two models
 *     per (level, layer, K/V, channel): one for anchor tokens and one for
 *     the others, profiled and normalised like the base models;
 *   - refined output: binary16(fma(q, D, xh)), one binary32 rounding then
 *     one binary16 rounding.
 * Its container ("KVCR") has the base container's layout: a 64-byte header,
 * 2LC records {f32 Da, f32 Dd, u32 0, u32 nbytes}, then the payload in the
 * reference reader's block order (R17). */

#define REFINE_MAX_BITS 6u

/* Base reconstruction of one stream in binary32 (before binary16). */
static void base_recon(const int32_t *sym, uint32_t n, uint32_t G, uint32_t dbits, float lo,
                       float sa, float dl, float *xh) {
  const int32_t M = delta_m(dbits);
  float ahat = 0.0f;
  for (uint32_t j = 0; j < n; ++j) {
    if (j % G == 0) {
      ahat = fmaf((float)sym[j], sa, lo);
      xh[j] = ahat;
    } else {
      xh[j] = fmaf((float)(sym[j] - M), dl, ahat);
    }
  }
}

/* The refinement quantizer of one stream: from x and its base
 * reconstruction xh, the two scales and the symbols (q + Me). */
static void refine_quantize_xh(const float *x, const float *xh, uint32_t n, uint32_t G,
                               uint32_t ebits, float *Da_out, float *Dd_out, int32_t *esym) {
  const int32_t Me = delta_m(ebits);
  float amax = 0.0f, dmax = 0.0f;
  for (uint32_t j = 0; j < n; ++j) {
    const float a = fabsf(x[j] - xh[j]);
    if (j % G == 0) {
      if (a > amax) amax = a;
    } else {
      if (a > dmax) dmax = a;
    }
  }
  const float Da = amax / (float)Me, Dd = dmax / (float)Me;
  for (uint32_t j = 0; j < n; ++j) {
    const float D = (j % G == 0) ? Da : Dd;
    int q = 0;
    if (D != 0.0f) {
      q = (int)rintf((x[j] - xh[j]) / D);
      if (q < -Me) q = -Me;
      if (q > Me) q = Me;
    }
    esym[j] = q + Me;
  }
  *Da_out = Da;
  *Dd_out = Dd;
}

/* One stream: base quantization at dbits, then the refinement quantizer at
 * ebits.  Outputs the base side info and symbols and the refinement scales
 * and symbols. */
int orc_refine_quantize(const float *x, uint32_t n, uint32_t G, uint32_t dbits, uint32_t ebits,
                        float *lo, float *sa, float *dl, int32_t *sym, float *Da, float *Dd,
                        int32_t *esym) {
  if (ebits < 2 || ebits > REFINE_MAX_BITS) return ORC_ERR_ARG;
  int st = orc_quantize(x, n, G, dbits, lo, sa, dl, sym);
  if (st) return st;
  float *xh = (float *)malloc(sizeof(float) * (n ? n : 1));
  if (!xh) return ORC_ERR_CAPACITY;
  base_recon(sym, n, G, dbits, *lo, *sa, *dl, xh);
  refine_quantize_xh(x, xh, n, G, ebits, Da, Dd, esym);
  free(xh);
  return ORC_OK;
}

/* Refined reconstruction of one stream: binary16(fma(q, D, xh)). */
void orc_refine_dequantize(const int32_t *sym, const int32_t *esym, uint32_t n, uint32_t G,
                           uint32_t dbits, uint32_t ebits, float lo, float sa, float dl, float Da,
                           float Dd, uint16_t *out) {
  const int32_t Me = delta_m(ebits);
  float *xh = (float *)malloc(sizeof(float) * (n ? n : 1));
  base_recon(sym, n, G, dbits, lo, sa, dl, xh);
  for (uint32_t j = 0; j < n; ++j) {
    const float D = (j % G == 0) ? Da : Dd;
    out[j] = orc_f2h(fmaf((float)(esym[j] - Me), D, xh[j]));
  }
  free(xh);
}

/* Refinement profile id: FNV-1a over the descriptor, E (u32) and the base
 * profile id (u64), then for each (layer, K/V) row the FNV-1a of that row's
 * per-model FNV-1a values; a model's value covers, level by level, its
 * anchor-token frequencies then its other-token frequencies (u16, LE). */
uint64_t orc_refine_profile_id(const uint32_t *pw, uint32_t ebits, uint64_t base_id,
                               const uint16_t *fEA, const uint16_t *fED) {
  params p;
  if (read_params(pw, &p)) return 0;
  const uint32_t S = n_streams(&p);
  const uint32_t A = delta_alpha(ebits);
  uint64_t h = desc_hash(&p);
  h = fnv_u32(h, ebits);
  h = fnv_u64(h, base_id);
  for (uint32_t row = 0; row < 2 * p.L; ++row) {
    uint64_t hr = FNV_OFFSET;
    for (uint32_t c = 0; c < p.C; ++c) {
      const uint32_t m = row * p.C + c;
      uint64_t hm = FNV_OFFSET;
      for (uint32_t lv = 0; lv < p.nlev; ++lv) {
        const uint16_t *fa = fEA + ((size_t)lv * S + m) * MAX_DELTA_ALPHA;
        const uint16_t *fd = fED + ((size_t)lv * S + m) * MAX_DELTA_ALPHA;
        for (uint32_t s = 0; s < A; ++s) hm = fnv_u16(hm, fa[s]);
        for (uint32_t s = 0; s < A; ++s) hm = fnv_u16(hm, fd[s]);
      }
      hr = fnv_u64(hr, hm);
    }
    h = fnv_u64(h, hr);
  }
  return h;
}

/* Refinement profiling: over every profiling chunk, every stream and every
 * level, count the refinement symbols of anchor tokens (fEA) and of the
 * other tokens (fED) per (level, stream), normalise to 2^15.  Tables
 * fEA/fED: [n_levels][2LC][64] u16 (first 2^E - 1 entries used). */
int orc_profile_refine(const uint32_t *pw, const uint16_t *kv, uint32_t T, uint32_t ebits,
                       uint64_t base_id, uint16_t *fEA, uint16_t *fED, uint64_t *refine_id) {
  params p;
  int st = read_params(pw, &p);
  if (st) return st;
  if (ebits < 2 || ebits > REFINE_MAX_BITS) return ORC_ERR_ARG;
  if (T == 0) return ORC_ERR_SHAPE;
  const uint32_t S = n_streams(&p);
  const uint32_t A = delta_alpha(ebits);
  const uint32_t nchunks = (T + p.chunk - 1) / p.chunk;
  int err = ORC_OK;
#pragma omp parallel for schedule(dynamic, 16)
  for (long mm = 0; mm < (long)S; ++mm) {
    const uint32_t m = (uint32_t)mm;
    const uint32_t l = m / (2 * p.C);
    float *x = (float *)malloc(sizeof(float) * p.chunk);
    int32_t *sym = (int32_t *)malloc(sizeof(int32_t) * p.chunk);
    int32_t *esym = (int32_t *)malloc(sizeof(int32_t) * p.chunk);
    uint64_t ca[4][MAX_DELTA_ALPHA], cd[4][MAX_DELTA_ALPHA];
    memset(ca, 0, sizeof ca);
    memset(cd, 0, sizeof cd);
    for (uint32_t k = 0; k < nchunks; ++k) {
      const uint32_t t0 = k * p.chunk;
      const uint32_t n = (T - t0 < p.chunk) ? T - t0 : p.chunk;
      widen_stream(kv, &p, T, m, t0, n, x);
      for (uint32_t lv = 0; lv < p.nlev; ++lv) {
        float lo, sa, dl, Da, Dd;
        if (orc_refine_quantize(x, n, p.G, p.bits[lv][third_of(l, p.L)], ebits, &lo, &sa, &dl,
                                sym, &Da, &Dd, esym)) {
#pragma omp atomic write
          err = ORC_ERR_NONFINITE;
          break;
        }
        for (uint32_t j = 0; j < n; ++j) {
          if (j % p.G == 0)
            ca[lv][esym[j]]++;
          else
            cd[lv][esym[j]]++;
        }
      }
    }
    uint32_t f[MAX_DELTA_ALPHA];
    for (uint32_t lv = 0; lv < p.nlev; ++lv) {
      uint16_t *da = fEA + ((size_t)lv * S + m) * MAX_DELTA_ALPHA;
      uint16_t *dd = fED + ((size_t)lv * S + m) * MAX_DELTA_ALPHA;
      orc_normalize(ca[lv], A, f);
      for (uint32_t s = 0; s < MAX_DELTA_ALPHA; ++s) da[s] = (uint16_t)(s < A ? f[s] : 0u);
      orc_normalize(cd[lv], A, f);
      for (uint32_t s = 0; s < MAX_DELTA_ALPHA; ++s) dd[s] = (uint16_t)(s < A ? f[s] : 0u);
    }
    free(x);
    free(sym);
    free(esym);
  }
  if (err) return err;
  *refine_id = orc_refine_profile_id(pw, ebits, base_id, fEA, fED);
  return ORC_OK;
}

/* The refinement models of the unit's lanes at `level`. */
static void refine_models(const params *p, const uint16_t *fEA, const uint16_t *fED,
                          uint32_t level, uint32_t ebits, uint32_t m0, uint32_t nv,
                          lane_models *mods) {
  const uint32_t S = n_streams(p);
  for (uint32_t l = 0; l < nv; ++l) {
    const uint32_t m = m0 + l;
    mods[l].AA = mods[l].AD = delta_alpha(ebits);
    widen_freqs(fEA + ((size_t)level * S + m) * MAX_DELTA_ALPHA, mods[l].AA, mods[l].fa);
    widen_freqs(fED + ((size_t)level * S + m) * MAX_DELTA_ALPHA, mods[l].AD, mods[l].fd);
  }
}

/*
 * The refinement layer of chunk `chunk` of kv [L][2][T][C] over its base
 * layer at `level`, as one "KVCR" container.  Returns its size, or a
 * negative error.
 */
int64_t orc_encode_refine_chunk(const uint32_t *pw, const uint16_t *fEA, const uint16_t *fED,
                                uint64_t refine_id, uint64_t base_id, uint32_t ebits,
                                const uint16_t *kv, uint32_t T, uint32_t chunk, uint32_t level,
                                uint8_t *out, uint64_t cap) {
  params p;
  int st = read_params(pw, &p);
  if (st) return st;
  if (level >= p.nlev || ebits < 2 || ebits > REFINE_MAX_BITS) return ORC_ERR_ARG;
  const uint64_t t0 = (uint64_t)chunk * p.chunk;
  if (t0 >= T) return ORC_ERR_SHAPE;
  const uint32_t n = (uint32_t)((T - t0 < p.chunk) ? T - t0 : p.chunk);
  const uint32_t S = n_streams(&p);
  const uint32_t A = delta_alpha(ebits);
  const uint64_t slot = pad8(4u + 2u * (uint64_t)n);
  uint8_t *scratch = (uint8_t *)calloc((size_t)S, (size_t)slot);
  float *side = (float *)malloc(sizeof(float) * 2u * S);
  uint32_t *nb = (uint32_t *)malloc(sizeof(uint32_t) * S);
  if (!scratch || !side || !nb) {
    free(scratch);
    free(side);
    free(nb);
    return ORC_ERR_CAPACITY;
  }
  int err = ORC_OK;
#pragma omp parallel for schedule(dynamic, 16)
  for (long mm = 0; mm < (long)S; ++mm) {
    const uint32_t m = (uint32_t)mm;
    const uint32_t l = m / (2 * p.C);
    float *x = (float *)malloc(sizeof(float) * n);
    int32_t *sym = (int32_t *)malloc(sizeof(int32_t) * n);
    int32_t *esym = (int32_t *)malloc(sizeof(int32_t) * n);
    uint32_t fa[MAX_DELTA_ALPHA], fd[MAX_DELTA_ALPHA];
    float lo, sa, dl;
    widen_stream(kv, &p, T, m, (uint32_t)t0, n, x);
    int e = orc_refine_quantize(x, n, p.G, p.bits[level][third_of(l, p.L)], ebits, &lo, &sa, &dl,
                                sym, &side[2 * m], &side[2 * m + 1], esym);
    if (!e) {
      widen_freqs(fEA + ((size_t)level * S + m) * MAX_DELTA_ALPHA, A, fa);
      widen_freqs(fED + ((size_t)level * S + m) * MAX_DELTA_ALPHA, A, fd);
      const int64_t w =
          orc_rc_encode(esym, n, p.G, fa, A, fd, A, scratch + (size_t)m * slot, slot);
      if (w < 0)
        e = (int)w;
      else
        nb[m] = (uint32_t)w;
    }
    if (e) {
#pragma omp critical
      err = e;
    }
    free(x);
    free(sym);
    free(esym);
  }
  if (err) {
    free(scratch);
    free(side);
    free(nb);
    return err;
  }
  uint64_t payload = 0;
  for (uint32_t m = 0; m < S; ++m) payload += pad8(nb[m]);
  const uint64_t total = HDR_BYTES + (uint64_t)REC_BYTES * S + payload;
  if (total > cap) {
    free(scratch);
    free(side);
    free(nb);
    return ORC_ERR_CAPACITY;
  }
  memset(out, 0, (size_t)total);
  memcpy(out, "KVCR", 4);
  put_u16(out + 4, 1);
  out[6] = (uint8_t)level;
  out[7] = (uint8_t)ebits;
  put_u16(out + 8, (uint16_t)p.G);
  out[10] = (uint8_t)p.prec;
  for (int j = 0; j < 3; ++j) out[11 + j] = (uint8_t)p.bits[level][j];
  put_u32(out + 16, p.L);
  put_u32(out + 20, p.C);
  put_u32(out + 24, n);
  put_u32(out + 28, (uint32_t)t0);
  put_u64(out + 32, refine_id);
  put_u64(out + 40, payload);
  put_u32(out + 48, p.chunk);
  put_u32(out + 52, S);
  put_u64(out + 56, base_id);
  for (uint32_t m = 0; m < S; ++m) {
    uint8_t *rec = out + HDR_BYTES + (size_t)REC_BYTES * m;
    put_f32(rec, side[2 * m]);
    put_f32(rec + 4, side[2 * m + 1]);
    put_u32(rec + 8, 0);
    put_u32(rec + 12, nb[m]);
  }
  uint64_t *uoff = (uint64_t *)malloc(sizeof(uint64_t) * (n_units(&p) + 1));
  uoff[0] = 0;
  for (uint32_t u = 0; u < n_units(&p); ++u) {
    uint32_t m0, nv;
    unit_span(&p, u, &m0, &nv);
    uint64_t sz = 0;
    for (uint32_t l = 0; l < nv; ++l) sz += pad8(nb[m0 + l]);
    uoff[u + 1] = uoff[u] + sz;
  }
  uint8_t *pay = out + HDR_BYTES + (size_t)REC_BYTES * S;
#pragma omp parallel for schedule(dynamic, 4)
  for (long uu = 0; uu < (long)n_units(&p); ++uu) {
    const uint32_t u = (uint32_t)uu;
    uint32_t m0, nv;
    unit_span(&p, u, &m0, &nv);
    const uint8_t *streams[UNIT_LANES];
    for (uint32_t l = 0; l < nv; ++l) streams[l] = scratch + (size_t)(m0 + l) * slot;
    lane_models *mods = (lane_models *)malloc(sizeof(lane_models) * UNIT_LANES);
    refine_models(&p, fEA, fED, level, ebits, m0, nv, mods);
    const int e = unit_reader_models(&p, mods, nv, n, nb + m0, streams, NULL,
                                     (uoff[u + 1] - uoff[u]) / BLOCK, pay + uoff[u], NULL, NULL);
    free(mods);
    if (e) {
#pragma omp critical
      err = e;
    }
  }
  free(uoff);
  free(scratch);
  free(side);
  free(nb);
  return err ? err : (int64_t)total;
}

typedef struct {
  uint32_t n, level, ebits;
  uint64_t payload;
} refine_hdr;

static int check_refine_header(const params *p, uint64_t refine_id, uint64_t base_id,
                               const uint8_t *c, uint64_t nbytes, refine_hdr *h) {
  const uint32_t S = n_streams(p);
  if (nbytes < HDR_BYTES + (uint64_t)REC_BYTES * S) return ORC_ERR_CORRUPT;
  if (memcmp(c, "KVCR", 4) != 0 || get_u16(c + 4) != 1) return ORC_ERR_CORRUPT;
  h->level = c[6];
  h->ebits = c[7];
  h->n = get_u32(c + 24);
  h->payload = get_u64(c + 40);
  if (h->level >= p->nlev || h->ebits < 2 || h->ebits > REFINE_MAX_BITS ||
      get_u16(c + 8) != p->G || c[10] != p->prec)
    return ORC_ERR_CORRUPT;
  for (int j = 0; j < 3; ++j)
    if (c[11 + j] != p->bits[h->level][j]) return ORC_ERR_CORRUPT;
  if (get_u32(c + 16) != p->L || get_u32(c + 20) != p->C || get_u32(c + 48) != p->chunk ||
      get_u32(c + 52) != S)
    return ORC_ERR_CORRUPT;
  if (h->n == 0 || h->n > p->chunk) return ORC_ERR_CORRUPT;
  if (get_u64(c + 32) != refine_id || get_u64(c + 56) != base_id) return ORC_ERR_PROFILE;
  if (HDR_BYTES + (uint64_t)REC_BYTES * S + h->payload != nbytes) return ORC_ERR_CORRUPT;
  uint64_t sum = 0;
  for (uint32_t m = 0; m < S; ++m) sum += pad8(get_u32(c + HDR_BYTES + (size_t)REC_BYTES * m + 12));
  if (sum != h->payload) return ORC_ERR_CORRUPT;
  return ORC_OK;
}

/*
 * Decode a chunk's base container and its refinement container into out
 * [L][2][T_total][C] at tokens [first_token, first_token + n_tokens): the
 * refined values binary16(fma(q, D, xh)).  Both headers must agree with the
 * call (level, token count) and with each other; the refinement must belong
 * to these base tables.
 */
int orc_decode_refined_chunk(const uint32_t *pw, const uint16_t *fA, const uint16_t *fD,
                             uint64_t base_id, const uint8_t *c, uint64_t nbytes,
                             const uint16_t *fEA, const uint16_t *fED, uint64_t refine_id,
                             const uint8_t *rc, uint64_t rbytes, uint32_t first_token,
                             uint32_t n_tokens, uint32_t level, uint16_t *out, uint32_t T_total) {
  params p;
  int st = read_params(pw, &p);
  if (st) return st;
  chunk_hdr h;
  st = check_header(&p, base_id, c, nbytes, &h);
  if (st) return st;
  refine_hdr rh;
  st = check_refine_header(&p, refine_id, base_id, rc, rbytes, &rh);
  if (st) return st;
  if (h.n != n_tokens || h.level != level || rh.n != n_tokens || rh.level != level)
    return ORC_ERR_ARG;
  if (get_u32(c + 28) != get_u32(rc + 28)) return ORC_ERR_CORRUPT; /* same chunk */
  if ((uint64_t)first_token + n_tokens > T_total) return ORC_ERR_SHAPE;
  const uint32_t S = n_streams(&p);
  uint32_t *offs = (uint32_t *)malloc(sizeof(uint32_t) * S);
  uint32_t *roffs = (uint32_t *)malloc(sizeof(uint32_t) * S);
  orc_stream_offsets(pw, c, nbytes, offs);
  {
    uint64_t acc = 0;
    for (uint32_t m = 0; m < S; ++m) {
      roffs[m] = (uint32_t)acc;
      acc += pad8(get_u32(rc + HDR_BYTES + (size_t)REC_BYTES * m + 12));
    }
  }
  int err = ORC_OK;
#pragma omp parallel for schedule(dynamic, 4)
  for (long uu = 0; uu < (long)n_units(&p); ++uu) {
    const uint32_t u = (uint32_t)uu;
    uint32_t m0, nv;
    unit_span(&p, u, &m0, &nv);
    int32_t *sym = (int32_t *)malloc(sizeof(int32_t) * (size_t)nv * h.n);
    int32_t *esym = (int32_t *)malloc(sizeof(int32_t) * (size_t)nv * h.n);
    uint16_t *vals = (uint16_t *)malloc(sizeof(uint16_t) * h.n);
    lane_models *mods = (lane_models *)malloc(sizeof(lane_models) * UNIT_LANES);
    int e = read_unit(&p, fA, fD, c, &h, offs, u, sym, NULL);
    if (!e) {
      uint32_t nb[UNIT_LANES];
      uint64_t sz = 0;
      for (uint32_t l = 0; l < nv; ++l) {
        nb[l] = get_u32(rc + HDR_BYTES + (size_t)REC_BYTES * (m0 + l) + 12);
        sz += pad8(nb[l]);
      }
      refine_models(&p, fEA, fED, level, rh.ebits, m0, nv, mods);
      e = unit_reader_models(&p, mods, nv, h.n, nb, NULL,
                             rc + HDR_BYTES + (size_t)REC_BYTES * S + roffs[m0], sz / BLOCK, NULL,
                             esym, NULL);
    }
    if (e) {
#pragma omp critical
      err = e;
    } else {
      for (uint32_t l = 0; l < nv; ++l) {
        const uint32_t m = m0 + l;
        const uint8_t *rec = c + HDR_BYTES + (size_t)REC_BYTES * m;
        const uint8_t *rrec = rc + HDR_BYTES + (size_t)REC_BYTES * m;
        orc_refine_dequantize(sym + (size_t)l * h.n, esym + (size_t)l * h.n, h.n, p.G,
                              p.bits[level][third_of(m / (2 * p.C), p.L)], rh.ebits,
                              get_f32(rec), get_f32(rec + 4), get_f32(rec + 8), get_f32(rrec),
                              get_f32(rrec + 4), vals);
        const uint32_t row = m / p.C, ch = m % p.C;
        uint16_t *dst = out + (size_t)row * T_total * p.C;
        for (uint32_t j = 0; j < h.n; ++j) dst[(size_t)(first_token + j) * p.C + ch] = vals[j];
      }
    }
    free(sym);
    free(esym);
    free(vals);
    free(mods);
  }
  free(offs);
  free(roffs);
  return err;
}

/* The refinement symbols [count][n] of selected streams of a refinement
 * container (its header checked against the ids), for checks. */
int orc_decode_refine_symbols(const uint32_t *pw, const uint16_t *fEA, const uint16_t *fED,
                              uint64_t refine_id, uint64_t base_id, const uint8_t *rc,
                              uint64_t rbytes, const uint32_t *ids, uint32_t count,
                              int32_t *esyms) {
  params p;
  int st = read_params(pw, &p);
  if (st) return st;
  refine_hdr rh;
  st = check_refine_header(&p, refine_id, base_id, rc, rbytes, &rh);
  if (st) return st;
  const uint32_t S = n_streams(&p);
  const uint32_t ncb = (p.C + UNIT_LANES - 1) / UNIT_LANES;
  uint32_t *roffs = (uint32_t *)malloc(sizeof(uint32_t) * S);
  uint64_t acc = 0;
  for (uint32_t m = 0; m < S; ++m) {
    roffs[m] = (uint32_t)acc;
    acc += pad8(get_u32(rc + HDR_BYTES + (size_t)REC_BYTES * m + 12));
  }
  int32_t *usym = (int32_t *)malloc(sizeof(int32_t) * (size_t)UNIT_LANES * rh.n);
  lane_models *mods = (lane_models *)malloc(sizeof(lane_models) * UNIT_LANES);
  int err = ORC_OK;
  uint32_t last = 0xFFFFFFFFu;
  for (uint32_t i = 0; i < count && !err; ++i) {
    if (ids[i] >= S) {
      err = ORC_ERR_ARG;
      break;
    }
    const uint32_t m = ids[i];
    const uint32_t u = (m / p.C) * ncb + (m % p.C) / UNIT_LANES;
    uint32_t m0, nv;
    unit_span(&p, u, &m0, &nv);
    if (u != last) {
      uint32_t nb[UNIT_LANES];
      uint64_t sz = 0;
      for (uint32_t l = 0; l < nv; ++l) {
        nb[l] = get_u32(rc + HDR_BYTES + (size_t)REC_BYTES * (m0 + l) + 12);
        sz += pad8(nb[l]);
      }
      refine_models(&p, fEA, fED, rh.level, rh.ebits, m0, nv, mods);
      err = unit_reader_models(&p, mods, nv, rh.n, nb, NULL,
                               rc + HDR_BYTES + (size_t)REC_BYTES * S + roffs[m0], sz / BLOCK,
                               NULL, usym, NULL);
      if (err) break;
      last = u;
    }
    memcpy(esyms + (size_t)i * rh.n, usym + (size_t)(m - m0) * rh.n, sizeof(int32_t) * rh.n);
  }
  free(usym);
  free(mods);
  free(roffs);
  return err;
}
