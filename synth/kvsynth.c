/*
 * Seeded synthetic KV-cache generator.
 *
 * This module only produces input data.  It holds none of the codec's
 * arithmetic: it is shared by the CPU oracle's tests and by the GPU path's
 * tests and benchmark, and neither of those includes anything from here.
 *
 * Value model (one process per (layer, K/V, channel) across the whole
 * context):
 *     x[t] = mu + s * z[t],   z[t] = rho * z[t-1] + e[t],   e[t] ~ N(0, 1)
 *     z[0] ~ N(0, 1 / (1 - rho^2))            (stationary start)
 *     mu ~ N(0, 1),  s ~ LogNormal(0, 0.5),  rho fixed or U(rho_lo, rho_hi)
 * Outlier channels: exactly round(frac * C) channels per (layer, K/V),
 * chosen without replacement, get s multiplied by `outlier_scale`.
 * Everything is computed in binary64 and rounded once to binary16
 * (round to nearest, ties to even).
 *
 * Randomness: Philox4x32-10, the counter-based generator of Salmon, Moraes,
 * Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC 2011).
 * Every random draw is addressed by a counter, so the output does not
 * depend on the number of threads.
 *   counter word 0: index of the (layer, K/V, channel) process, or of the
 *                   (layer, K/V) row, or of the chunk
 *   counter word 1: draw kind (see KIND_*)
 *   counter word 2: draw index inside that kind (token pair for innovations)
 *   counter word 3: 0
 *   key: (seed low 32 bits, seed high 32 bits)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define KIND_PARAMS 0u   /* mu, log-s */
#define KIND_RHO 1u      /* per-channel rho */
#define KIND_OUTLIER 2u  /* outlier selection, per (layer, K/V) row */
#define KIND_INNOV 3u    /* AR(1) innovations, two tokens per counter */
#define KIND_LEVEL 4u    /* per-chunk level sequence */

static inline void philox_round(uint32_t c[4], const uint32_t k[2]) {
  const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
  const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
  const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
  const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
  const uint32_t n0 = hi1 ^ c[1] ^ k[0];
  const uint32_t n2 = hi0 ^ c[3] ^ k[1];
  c[0] = n0;
  c[1] = lo1;
  c[2] = n2;
  c[3] = lo0;
}

/* Philox4x32 with 10 rounds; the key is bumped by the Weyl constants
 * between rounds. */
void kvs_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2],
                       uint32_t out[4]) {
  uint32_t c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
  uint32_t k[2] = {key_in[0], key_in[1]};
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k[0] += 0x9E3779B9u;
      k[1] += 0xBB67AE85u;
    }
    philox_round(c, k);
  }
  memcpy(out, c, sizeof c);
}

/* Two uniforms in the open interval (0, 1), 53 bits each. */
static inline void uniforms2(uint64_t seed, uint32_t w0, uint32_t w1,
                             uint32_t w2, double *u0, double *u1) {
  const uint32_t ctr[4] = {w0, w1, w2, 0u};
  const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t r[4];
  kvs_philox4x32_10(ctr, key, r);
  const uint64_t a = ((uint64_t)r[0] << 21) ^ (uint64_t)(r[1] >> 11);
  const uint64_t b = ((uint64_t)r[2] << 21) ^ (uint64_t)(r[3] >> 11);
  const double inv = 1.0 / 9007199254740992.0; /* 2^-53 */
  *u0 = ((double)(a & ((1ull << 53) - 1)) + 0.5) * inv;
  *u1 = ((double)(b & ((1ull << 53) - 1)) + 0.5) * inv;
}

/* Box-Muller: two independent N(0,1) draws from two uniforms. */
static inline void normals2(uint64_t seed, uint32_t w0, uint32_t w1,
                            uint32_t w2, double *n0, double *n1) {
  double u0, u1;
  uniforms2(seed, w0, w1, w2, &u0, &u1);
  const double rad = sqrt(-2.0 * log(u0));
  const double ang = 6.283185307179586476925286766559 * u1;
  *n0 = rad * cos(ang);
  *n1 = rad * sin(ang);
}

/* binary64 -> binary16, round to nearest, ties to even (generator-local),
 * on the bit patterns. */
static uint16_t to_half(double v) {
  uint64_t u;
  memcpy(&u, &v, 8);
  const uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
  const uint64_t a = u & 0x7FFFFFFFFFFFFFFFull;
  if (a >= 0x7FF0000000000000ull) return (uint16_t)(sign | (a > 0x7FF0000000000000ull ? 0x7E00u : 0x7C00u));
  const int e = (int)(a >> 52) - 1023;
  if (e > 15) return (uint16_t)(sign | 0x7C00u);
  const uint64_t m53 = (a & ((1ull << 52) - 1)) | (e > -1023 ? (1ull << 52) : 0);
  if (e >= -14) {
    uint64_t hm = m53 >> 42; /* 11 significant bits incl. the hidden one */
    const uint64_t rest = m53 & ((1ull << 42) - 1), half = 1ull << 41;
    if (rest > half || (rest == half && (hm & 1))) hm += 1;
    int he = e + 15;
    if (hm == 0x800) {
      hm = 0x400;
      he += 1;
    }
    if (he >= 31) return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | (uint16_t)(he << 10) | (uint16_t)(hm & 0x3FF));
  }
  /* subnormal: value / 2^-24 = m53 * 2^(e - 52 + 24) = m53 >> rs */
  const int rs = 28 - e;
  if (rs >= 64) return sign;
  const uint64_t q = m53 >> rs;
  const uint64_t rem = m53 & ((1ull << rs) - 1), half = 1ull << (rs - 1);
  uint64_t r = q;
  if (rem > half || (rem == half && (q & 1))) r += 1;
  return (uint16_t)(sign | (uint16_t)r);
}

/*
 * Per-process parameters for all 2*L*C processes of a configuration.
 *   mu, s, rho: arrays of length 2*L*C, index m = (l*2 + kv)*C + c.
 * rho_mode 0: rho = rho_lo for all; 1: rho ~ U(rho_lo, rho_hi) per process.
 */
void kvs_params(uint64_t seed, uint32_t L, uint32_t C, int rho_mode,
                double rho_lo, double rho_hi, double outlier_frac,
                double outlier_scale, double *mu, double *s, double *rho,
                uint8_t *is_outlier) {
  const uint32_t S = 2u * L * C;
  for (uint32_t m = 0; m < S; ++m) {
    double n0, n1;
    normals2(seed, m, KIND_PARAMS, 0u, &n0, &n1);
    mu[m] = n0;
    s[m] = exp(0.5 * n1);
    if (rho_mode == 1) {
      double u0, u1;
      uniforms2(seed, m, KIND_RHO, 0u, &u0, &u1);
      rho[m] = rho_lo + (rho_hi - rho_lo) * u0;
    } else {
      rho[m] = rho_lo;
    }
    is_outlier[m] = 0;
  }
  const uint32_t k_out = (uint32_t)floor(outlier_frac * (double)C + 0.5);
  if (k_out == 0) return;
  uint32_t *perm = (uint32_t *)malloc(sizeof(uint32_t) * C);
  for (uint32_t row = 0; row < 2u * L; ++row) {
    for (uint32_t c = 0; c < C; ++c) perm[c] = c;
    /* partial Fisher-Yates: the first k_out entries are the chosen set */
    for (uint32_t i = 0; i < k_out; ++i) {
      double u0, u1;
      uniforms2(seed, row, KIND_OUTLIER, i, &u0, &u1);
      uint32_t j = i + (uint32_t)(u0 * (double)(C - i));
      if (j >= C) j = C - 1;
      const uint32_t t = perm[i];
      perm[i] = perm[j];
      perm[j] = t;
    }
    for (uint32_t i = 0; i < k_out; ++i) {
      const uint32_t m = row * C + perm[i];
      is_outlier[m] = 1;
      s[m] *= outlier_scale;
    }
  }
  free(perm);
}

/*
 * Generate tokens [0, T) of rows [row0, row1) (row = l*2 + kv) into
 * out[(row - row0)][T][C] binary16, using innovation seed `innov_seed` and
 * the given per-process parameters.  Rows are independent and are spread
 * over OpenMP threads.
 */
void kvs_generate(uint64_t innov_seed, uint32_t C, uint32_t T, uint32_t row0,
                  uint32_t row1, const double *mu, const double *s,
                  const double *rho, uint16_t *out) {
  const long nrows = (long)row1 - (long)row0;
#pragma omp parallel for schedule(dynamic, 1)
  for (long rr = 0; rr < nrows; ++rr) {
    const uint32_t row = row0 + (uint32_t)rr;
    double *z = (double *)malloc(sizeof(double) * C);
    double *e = (double *)malloc(sizeof(double) * 2 * C);
    uint16_t *dst = out + (size_t)rr * T * C;
    for (uint32_t t = 0; t < T; ++t) {
      if ((t & 1u) == 0) {
        for (uint32_t c = 0; c < C; ++c) {
          const uint32_t m = row * C + c;
          normals2(innov_seed, m, KIND_INNOV, t >> 1, &e[2 * c], &e[2 * c + 1]);
        }
      }
      for (uint32_t c = 0; c < C; ++c) {
        const uint32_t m = row * C + c;
        const double eps = e[2 * c + (t & 1u)];
        if (t == 0)
          z[c] = eps / sqrt(1.0 - rho[m] * rho[m]);
        else
          z[c] = rho[m] * z[c] + eps;
        dst[(size_t)t * C + c] = to_half(mu[m] + s[m] * z[c]);
      }
    }
    free(z);
    free(e);
  }
}

/* Raw innovations for tests of the generator itself: e[m][t]. */
void kvs_innovations(uint64_t innov_seed, uint32_t m0, uint32_t count,
                     uint32_t T, double *e) {
  for (uint32_t i = 0; i < count; ++i) {
    for (uint32_t t = 0; t < T; t += 2) {
      double a, b;
      normals2(innov_seed, m0 + i, KIND_INNOV, t >> 1, &a, &b);
      e[(size_t)i * T + t] = a;
      if (t + 1 < T) e[(size_t)i * T + t + 1] = b;
    }
  }
}

/* Seeded per-chunk level sequence: levels[k] = first Philox word mod n. */
void kvs_levels(uint64_t seed, uint32_t n_chunks, uint32_t n_levels,
                uint8_t *levels) {
  const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  for (uint32_t k = 0; k < n_chunks; ++k) {
    const uint32_t ctr[4] = {k, KIND_LEVEL, 0u, 0u};
    uint32_t r[4];
    kvs_philox4x32_10(ctr, key, r);
    levels[k] = (uint8_t)(r[0] % n_levels);
  }
}

uint16_t kvs_to_half(double v) { return to_half(v); }
