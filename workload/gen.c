/*
 * Seeded synthetic inputs for the routed-expert MoE step: expert weights,
 * hidden states and router noise.  This file holds no part of the MoE step
 * itself (no routing, caching, expert arithmetic or merging): it only draws
 * numbers and writes them in the documented expert-bank byte layout.
 *
 * Random source: Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel
 * random numbers: as easy as 1, 2, 3", SC'11), a counter-based generator, so
 * any tensor (or any element of it) can be regenerated on its own.
 *   key     = (seed low 32 bits, seed high 32 bits)
 *   counter = (block index, stream id a, stream id b, stream id c)
 * Block j yields four 32-bit words; element i of a stream uses word i % 4 of
 * block i / 4.
 *
 * Uniforms: u = ((w >> 8) + 0.5) * 2^-24, strictly inside (0, 1) in double
 * (the float path used for normals may round the top values to 1.0, which
 * only yields a zero normal).
 * Normals: Box-Muller on word pairs (0,1) and (2,3) of a block, in float.
 *
 * Expert-bank byte layout (one bank == one device slot; H = hidden,
 * I = expert intermediate; every matrix row-major with its contraction axis
 * contiguous):
 *   f32  : W_gate[I][H] | W_up[I][H] | W_down[H][I]                  (float)
 *   bf16 : same order, bfloat16 (round-to-nearest-even from float)
 *   mxfp4: codes  W_gate[I][H/2] | W_up[I][H/2] | W_down[H][I/2]
 *          scales W_gate[I][H/32] | W_up[I][H/32] | W_down[H][I/32]
 *          codes are OCP MX e2m1, two per byte, low nibble = even element;
 *          scales are e8m0 (2^(s-127)), one per 32 consecutive elements of
 *          the contraction axis.
 * The MX quantiser below exists only to synthesise weights: shared exponent
 * floor(log2(amax)) - 2, values rounded to nearest (ties to even code) on the
 * e2m1 grid and saturated at 6.
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <omp.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static inline void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    uint64_t p0 = (uint64_t)PHILOX_M0 * c[0];
    uint64_t p1 = (uint64_t)PHILOX_M1 * c[2];
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c[1] ^ k0;
    uint32_t n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
    k0 += PHILOX_W0; k1 += PHILOX_W1;
  }
}

/* Raw block, exported for known-answer tests. */
void wl_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
  philox4x32_10(c, key[0], key[1]);
  memcpy(out, c, sizeof c);
}

static inline void block(uint64_t seed, uint32_t j, uint32_t a, uint32_t b, uint32_t cc,
                         uint32_t w[4]) {
  w[0] = j; w[1] = a; w[2] = b; w[3] = cc;
  philox4x32_10(w, (uint32_t)seed, (uint32_t)(seed >> 32));
}

static inline float u01(uint32_t w) { return ((float)(w >> 8) + 0.5f) * (1.0f / 16777216.0f); }

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u; memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* Normals of stream (a,b,c), elements [i0, i0+n), scaled by sigma.
 * Works in chunks of 4*NB elements so that the Philox rounds and the
 * Box-Muller transcendental calls vectorise. */
#define NB 128
static void normals_range(uint64_t seed, uint32_t a, uint32_t b, uint32_t c,
                          int64_t i0, int64_t n, float sigma, float* out) {
  uint32_t w0[NB], w1[NB], w2[NB], w3[NB];
  float z[4 * NB], ua[2 * NB], ub[2 * NB], ra[2 * NB], sn[2 * NB], cs[2 * NB];
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  const float two_pi = 6.28318530717958647692f;
  int64_t i = i0, end = i0 + n;
  while (i < end) {
    uint32_t j0 = (uint32_t)(i >> 2);
    for (int t = 0; t < NB; ++t) {
      uint32_t c0 = j0 + (uint32_t)t, c1 = a, c2 = b, c3 = c, kk0 = k0, kk1 = k1;
      for (int r = 0; r < 10; ++r) {
        uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
        uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ kk0;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ kk1;
        c1 = (uint32_t)p1; c3 = (uint32_t)p0; c0 = n0; c2 = n2;
        kk0 += PHILOX_W0; kk1 += PHILOX_W1;
      }
      w0[t] = c0; w1[t] = c1; w2[t] = c2; w3[t] = c3;
    }
    for (int t = 0; t < NB; ++t) {
      ua[t] = u01(w0[t]); ua[NB + t] = u01(w2[t]);
      ub[t] = two_pi * u01(w1[t]); ub[NB + t] = two_pi * u01(w3[t]);
    }
    for (int t = 0; t < 2 * NB; ++t) ra[t] = sqrtf(-2.0f * logf(ua[t]));
    for (int t = 0; t < 2 * NB; ++t) sn[t] = sinf(ub[t]);
    for (int t = 0; t < 2 * NB; ++t) cs[t] = cosf(ub[t]);
    for (int t = 0; t < NB; ++t) {
      z[4 * t + 0] = ra[t] * cs[t];
      z[4 * t + 1] = ra[t] * sn[t];
      z[4 * t + 2] = ra[NB + t] * cs[NB + t];
      z[4 * t + 3] = ra[NB + t] * sn[NB + t];
    }
    int64_t first = i - ((int64_t)j0 << 2);
    int64_t take = 4 * NB - first;
    if (take > end - i) take = end - i;
    for (int64_t t = 0; t < take; ++t) out[t] = sigma * z[first + t];
    out += take; i += take;
  }
}

/* Uniforms in double: ((w >> 8) + 0.5) * 2^-24 is exact there and lies
 * strictly inside (0, 1) (in float the top values round up to 1.0). */
void wl_uniform_f64(uint64_t seed, uint32_t a, uint32_t b, uint32_t c, int64_t n, double* out) {
  uint32_t w[4];
  for (int64_t i = 0; i < n; ++i) {
    if ((i & 3) == 0) block(seed, (uint32_t)(i >> 2), a, b, c, w);
    out[i] = ((double)(w[i & 3] >> 8) + 0.5) * (1.0 / 16777216.0);
  }
}

void wl_normal_f32(uint64_t seed, uint32_t a, uint32_t b, uint32_t c, int64_t n, float sigma,
                   float* out) {
  normals_range(seed, a, b, c, 0, n, sigma, out);
}

void wl_normal_bf16(uint64_t seed, uint32_t a, uint32_t b, uint32_t c, int64_t n, float sigma,
                    uint16_t* out) {
  float buf[2048];
  for (int64_t i = 0; i < n; i += 2048) {
    int64_t m = n - i < 2048 ? n - i : 2048;
    normals_range(seed, a, b, c, i, m, sigma, buf);
    for (int64_t t = 0; t < m; ++t) out[i + t] = f32_to_bf16_rne(buf[t]);
  }
}

/* e2m1 code of |v| (already divided by the block scale); ties go to the even
 * code, values above 6 saturate. */
static inline uint8_t e2m1_code(float a) {
  return (uint8_t)((a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) +
                   (a > 2.5f) + (a >= 3.5f) + (a > 5.0f));
}

/* Quantise rows x cols normals (cols % 32 == 0) of stream (a,b,c). */
static void mx_rows(uint64_t seed, uint32_t a, uint32_t b, uint32_t c, int64_t r0, int64_t nrows,
                    int64_t cols, float sigma, uint8_t* codes, uint8_t* scales) {
  float row[cols], inv[cols / 32];
  uint8_t cd[cols];
  for (int64_t r = r0; r < r0 + nrows; ++r) {
    normals_range(seed, a, b, c, r * cols, cols, sigma, row);
    for (int64_t g = 0; g < cols / 32; ++g) {
      const float* v = row + g * 32;
      float amax = 0.f;
      for (int t = 0; t < 32; ++t) amax = fmaxf(amax, fabsf(v[t]));
      int e = 0;
      uint8_t sbyte = 127;
      inv[g] = 1.f;
      if (amax > 0.f) {
        frexpf(amax, &e);            /* amax = m * 2^e, m in [0.5, 1) */
        int x = (e - 1) - 2;         /* floor(log2 amax) - emax(e2m1) */
        if (x < -127) x = -127;
        if (x > 127) x = 127;
        sbyte = (uint8_t)(x + 127);
        inv[g] = ldexpf(1.f, -x);
      }
      scales[r * (cols / 32) + g] = sbyte;
    }
    for (int64_t g = 0; g < cols / 32; ++g) {
      const float iv = inv[g];
      for (int t = 0; t < 32; ++t) {
        float q = row[g * 32 + t] * iv;
        uint8_t m = e2m1_code(fabsf(q));
        cd[g * 32 + t] = (uint8_t)(m | ((q < 0.f && m) ? 8 : 0));
      }
    }
    uint8_t* dst = codes + r * (cols / 2);
    for (int64_t j = 0; j < cols / 2; ++j) dst[j] = (uint8_t)(cd[2 * j] | (cd[2 * j + 1] << 4));
  }
}

/* Stream ids for weights: a = tag 1, b = flat expert id u, c = matrix (0 gate, 1 up, 2 down). */
#define TAG_WEIGHT 1u

int64_t wl_expert_bytes(int dtype, int64_t H, int64_t I) {
  if (dtype == 0) return 12 * H * I;
  if (dtype == 1) return 6 * H * I;
  if (dtype == 2) return 3 * H * I / 2 + 3 * H * I / 32;
  return -1;
}

/* Fill one expert bank of flat id u. */
static void fill_bank(uint64_t seed, int dtype, int64_t H, int64_t I, uint32_t u, float sigma,
                      uint8_t* dst) {
  if (dtype == 0) {
    float* p = (float*)dst;
    normals_range(seed, TAG_WEIGHT, u, 0, 0, I * H, sigma, p);
    normals_range(seed, TAG_WEIGHT, u, 1, 0, I * H, sigma, p + I * H);
    normals_range(seed, TAG_WEIGHT, u, 2, 0, H * I, sigma, p + 2 * I * H);
  } else if (dtype == 1) {
    uint16_t* p = (uint16_t*)dst;
    wl_normal_bf16(seed, TAG_WEIGHT, u, 0, I * H, sigma, p);
    wl_normal_bf16(seed, TAG_WEIGHT, u, 1, I * H, sigma, p + I * H);
    wl_normal_bf16(seed, TAG_WEIGHT, u, 2, H * I, sigma, p + 2 * I * H);
  } else {
    uint8_t* cg = dst;
    uint8_t* cu = cg + I * H / 2;
    uint8_t* cd = cu + I * H / 2;
    uint8_t* sg = cd + H * I / 2;
    uint8_t* su = sg + I * H / 32;
    uint8_t* sd = su + I * H / 32;
    mx_rows(seed, TAG_WEIGHT, u, 0, 0, I, H, sigma, cg, sg);
    mx_rows(seed, TAG_WEIGHT, u, 1, 0, I, H, sigma, cu, su);
    mx_rows(seed, TAG_WEIGHT, u, 2, 0, H, I, sigma, cd, sd);
  }
}

/* Fill banks u_begin..u_end-1 at dst + (u - u_begin) * stride, in parallel.
 * Returns 0, or -1 on bad arguments. */
int wl_fill_banks(uint64_t seed, int dtype, int64_t H, int64_t I, int64_t u_begin, int64_t u_end,
                  float sigma, void* dst, int64_t stride, int threads) {
  int64_t sb = wl_expert_bytes(dtype, H, I);
  if (sb < 0 || stride < sb || u_end < u_begin || (dtype == 2 && (H % 32 || I % 32))) return -1;
  if (threads <= 0) threads = omp_get_max_threads();
  uint8_t* base = (uint8_t*)dst;
#pragma omp parallel for schedule(dynamic, 1) num_threads(threads)
  for (int64_t u = u_begin; u < u_end; ++u) {
    uint8_t* p = base + (u - u_begin) * stride;
    fill_bank(seed, dtype, H, I, (uint32_t)u, sigma, p);
    if (stride > sb) memset(p + sb, 0, (size_t)(stride - sb));
  }
  return 0;
}

/* Many independent normal streams in parallel: stream s has ids (a, b0 + s, c). */
void wl_normal_bf16_streams(uint64_t seed, uint32_t a, uint32_t b0, uint32_t c, int64_t nstreams,
                            int64_t n, float sigma, uint16_t* out, int threads) {
  if (threads <= 0) threads = omp_get_max_threads();
#pragma omp parallel for schedule(static) num_threads(threads)
  for (int64_t s = 0; s < nstreams; ++s)
    wl_normal_bf16(seed, a, b0 + (uint32_t)s, c, n, sigma, out + s * n);
}

void wl_normal_f32_streams(uint64_t seed, uint32_t a, uint32_t b0, uint32_t c, int64_t nstreams,
                           int64_t n, float sigma, float* out, int threads) {
  if (threads <= 0) threads = omp_get_max_threads();
#pragma omp parallel for schedule(static) num_threads(threads)
  for (int64_t s = 0; s < nstreams; ++s)
    normals_range(seed, a, b0 + (uint32_t)s, c, 0, n, sigma, out + s * n);
}

void wl_uniform_f64_streams(uint64_t seed, uint32_t a, uint32_t b0, uint32_t c, int64_t nstreams,
                            int64_t n, double* out, int threads) {
  if (threads <= 0) threads = omp_get_max_threads();
#pragma omp parallel for schedule(static) num_threads(threads)
  for (int64_t s = 0; s < nstreams; ++s)
    wl_uniform_f64(seed, a, b0 + (uint32_t)s, c, n, out + s * n);
}
