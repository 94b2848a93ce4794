/*
 * Seeded synthetic inputs for the MXFP4 MoE expert layer.
 *
 * This file is the input recipe only.  It draws the activations, the router
 * weights and the expert weights, and it packs the expert weights into the
 * storage format the layer consumes.  It does not route, decode, multiply or
 * combine anything: both the GPU library and the CPU oracle receive the bytes
 * it writes and compute the layer independently of each other.
 *
 * Random numbers: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) used as a counter-based
 * generator: draw n of stream `key` is the n-th SplitMix64 output started
 * from state `key`, so any element can be produced independently of the
 * others.  Normals: the Box-Muller transform (Box and Muller, 1958) on two
 * 24-bit uniforms, evaluated in single precision.
 *
 * Weight storage written here (per expert, rows of K elements, row-major):
 *   element c of a row sits in byte c/2 of that row, low nibble when c is
 *   even, high nibble when c is odd; one scale byte per 32 consecutive
 *   elements of a row.
 * The quantizer follows the OCP Microscaling rule for FP4 (E2M1) elements
 * with E8M0 block scales: shared exponent X = floor(log2(max|v|)) - 2,
 * clamped to [-127, 127]; element = v / 2^X rounded to the nearest E2M1
 * value, ties to the even mantissa, magnitudes above 6 saturate to 6; sign
 * bit set when v < 0; a block whose values are all zero gets X = -127.
 * (The pages cite the OCP MX format for the experts but give no rounding
 * rule; this is the plainest reading of that format.)
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* n-th output (n >= 0) of SplitMix64 started from state `key`. */
static inline uint64_t sm64_at(uint64_t key, uint64_t n) {
  return sm64_mix(key + (n + 1) * GOLDEN);
}

/* Key of an independent stream for (seed, tensor id, index). */
uint64_t synth_stream_key(uint64_t seed, uint32_t tensor, uint32_t index) {
  uint64_t k = sm64_at(seed, 0);
  k = sm64_at(k ^ ((uint64_t)tensor << 32 | index), 1);
  return k;
}

/* Raw 64-bit draw n of stream `key` (exposed for the permutation draw). */
uint64_t synth_u64(uint64_t key, uint64_t n) { return sm64_at(key, n); }

/* Standard normal number i of stream `key` (Box-Muller on draws 2*(i/2) and
 * 2*(i/2)+1; even i takes the cosine branch, odd i the sine branch). */
static inline void normal_pair(uint64_t key, uint64_t p, float* z0, float* z1) {
  uint64_t r1 = sm64_at(key, 2 * p);
  uint64_t r2 = sm64_at(key, 2 * p + 1);
  float u1 = (float)((r1 >> 40) + 1) * 0x1p-24f; /* (0, 1] */
  float u2 = (float)(r2 >> 40) * 0x1p-24f;       /* [0, 1) */
  float rad = sqrtf(-2.0f * logf(u1));
  float th = 6.2831853071795864769f * u2;
  float sn, cs;
  sincosf(th, &sn, &cs);
  *z0 = rad * cs;
  *z1 = rad * sn;
}

/* out[i] = stdev * normal(start + i), i in [0, n). */
void synth_normal_f32(uint64_t key, uint64_t start, int64_t n, float stdev, float* out) {
  int64_t i = 0;
  while (i < n) {
    uint64_t idx = start + (uint64_t)i;
    float z0, z1;
    normal_pair(key, idx >> 1, &z0, &z1);
    if ((idx & 1) == 0) {
      out[i++] = stdev * z0;
      if (i < n) out[i++] = stdev * z1;
    } else {
      out[i++] = stdev * z1;
    }
  }
}

/* fp32 -> bf16 bits, round to nearest even (inputs are finite). */
void synth_f32_to_bf16(const float* in, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) {
    uint32_t u;
    memcpy(&u, &in[i], 4);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    out[i] = (uint16_t)(u >> 16);
  }
}

/* Nearest E2M1 code magnitude (0..7) for a non-negative q, ties to even
 * mantissa, saturating at 6. */
static inline unsigned e2m1_round_mag(float q) {
  /* representable magnitudes by code: 0, .5, 1, 1.5, 2, 3, 4, 6 */
  if (q <= 0.25f) return 0;          /* tie 0.25 -> 0 (even) */
  if (q < 0.75f) return 1;           /* (0.25, 0.75) -> 0.5 */
  if (q <= 1.25f) return 2;          /* [0.75, 1.25] -> 1 (ties even) */
  if (q < 1.75f) return 3;           /* (1.25, 1.75) -> 1.5 */
  if (q <= 2.5f) return 4;           /* [1.75, 2.5] -> 2 */
  if (q < 3.5f) return 5;            /* (2.5, 3.5) -> 3 */
  if (q <= 5.0f) return 6;           /* [3.5, 5] -> 4 */
  return 7;                          /* (5, inf) -> 6 */
}

/* Quantize `rows` rows of K fp32 values (K % 32 == 0). */
void synth_quantize_mxfp4(const float* w, int64_t rows, int64_t K, uint8_t* packed,
                          uint8_t* scales) {
  const int64_t nb = K / 32;
  for (int64_t r = 0; r < rows; ++r) {
    const float* wr = w + r * K;
    uint8_t* pr = packed + r * (K / 2);
    uint8_t* sr = scales + r * nb;
    for (int64_t b = 0; b < nb; ++b) {
      const float* v = wr + b * 32;
      float amax = 0.0f;
      for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
      int X;
      if (amax == 0.0f) {
        X = -127;
      } else {
        int e;
        frexpf(amax, &e); /* amax = m * 2^e, m in [0.5, 1) */
        X = (e - 1) - 2;
        if (X < -127) X = -127;
        if (X > 127) X = 127;
      }
      sr[b] = (uint8_t)(X + 127);
      for (int i = 0; i < 32; i += 2) {
        unsigned code[2];
        for (int h = 0; h < 2; ++h) {
          float x = v[i + h];
          float q = ldexpf(fabsf(x), -X);
          code[h] = e2m1_round_mag(q) | (x < 0.0f ? 8u : 0u);
        }
        pr[(b * 32 + i) / 2] = (uint8_t)(code[0] | (code[1] << 4));
      }
    }
  }
}

/* Expert weights for experts [e0, e1) of a layer with hidden size d and
 * expert ffn size F.  Expert e's matrices (gate [F][d], up [F][d], down [d][F])
 * are drawn from streams (seed, 2 + m, e), m = 0, 1, 2, element (r, c) being
 * normal number r*K + c of its stream, times `stdev`.  Output per expert
 * (relative to expert e - e0):
 *   packed: gate F*d/2 | up F*d/2 | down d*F/2 bytes
 *   scales: gate F*d/32 | up F*d/32 | down d*F/32 bytes                    */
int synth_experts(uint64_t seed, int e0, int e1, int d, int F, float stdev, uint8_t* packed,
                  uint8_t* scales, int nthreads) {
  if (d % 32 || F % 32 || e1 < e0) return 1;
  const int64_t pb = (int64_t)3 * d * F / 2;
  const int64_t sb = (int64_t)3 * d * F / 32;
  const int64_t nrows = (int64_t)(e1 - e0) * (2 * (int64_t)F + d);
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  int err = 0;
#pragma omp parallel
  {
    float* buf = (float*)malloc(sizeof(float) * (size_t)(d > F ? d : F));
    if (!buf) {
#pragma omp atomic write
      err = 2;
    }
#pragma omp for schedule(dynamic, 64)
    for (int64_t g = 0; g < nrows; ++g) {
      if (!buf) continue;
      int64_t per = 2 * (int64_t)F + d;
      int e = (int)(g / per);
      int64_t rr = g % per;
      int m;
      int64_t r, K, poff, soff;
      if (rr < F) {
        m = 0; r = rr; K = d; poff = 0; soff = 0;
      } else if (rr < 2 * F) {
        m = 1; r = rr - F; K = d; poff = (int64_t)F * d / 2; soff = (int64_t)F * d / 32;
      } else {
        m = 2; r = rr - 2 * F; K = F; poff = (int64_t)F * d; soff = (int64_t)F * d / 16;
      }
      uint64_t key = synth_stream_key(seed, 2u + (uint32_t)m, (uint32_t)(e0 + e));
      synth_normal_f32(key, (uint64_t)(r * K), K, stdev, buf);
      synth_quantize_mxfp4(buf, 1, K, packed + e * pb + poff + r * (K / 2),
                           scales + e * sb + soff + r * (K / 32));
    }
    free(buf);
  }
  return err;
}
