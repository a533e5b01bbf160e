/*
 * moegen.c -- seeded synthetic inputs for the quantized MoE layer.
 *
 * This module produces input bytes only: activations, router weights and
 * biases, and expert weights already quantized to the two block formats the
 * layer consumes (NVFP4 and a Q6_K-style 6-bit format).  It holds none of the
 * layer's own arithmetic (no routing, no dequantized matmul, no combine); the
 * oracle and the GPU library both read the bytes written here.
 *
 * Random numbers: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) used as a counter-based
 * generator -- draw i of stream `key` is mix(key + (i+1)*golden) -- so every
 * element is addressable and the result does not depend on thread count.
 * Gaussians: Box-Muller in double precision, elements 2i and 2i+1 from draws
 * 2i and 2i+1.
 *
 * Byte layouts written here (the library's canonical input layouts):
 *   NVFP4 matrix W[N][K] (K % 16 == 0):
 *     codes  u8 [N][K/2]  element k of row n is nibble (k & 1) of byte k/2
 *                          (even element in the low nibble); E2M1 code, bit 3
 *                          is the sign, bits 2..1 exponent, bit 0 mantissa.
 *     scales u8 [N][K/16] E4M3 (fn) scale of elements 16b..16b+15.
 *     ts     f32          one per matrix.
 *   Q6_K-style matrix W[N][K] (K % 256 == 0): row n is K/256 superblocks of
 *     210 bytes each: ql[128] (low 4 bits of element i at byte i/2, nibble
 *     i&1), qh[64] (high 2 bits of element i at byte i/4, bits 2*(i&3)),
 *     sc int8[16] (one per 16-element sub-block), d fp16 little-endian[2].
 *     Element value = d * sc[i/16] * (q - 32), q = low | high << 4.
 */
#include <math.h>
#include <stdint.h>
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

static inline uint64_t draw(uint64_t key, uint64_t i) {
  return sm64_mix(key + (i + 1) * GOLDEN);
}

/* Stream key for (seed, tag, layer, step): each field is folded in through
 * the mixer so neighbouring values give unrelated streams. */
uint64_t moegen_key(uint64_t seed, uint64_t tag, uint64_t layer, uint64_t step) {
  uint64_t z = sm64_mix(seed + GOLDEN);
  z = sm64_mix(z ^ (tag * GOLDEN));
  z = sm64_mix(z ^ ((layer << 32) | (step & 0xffffffffULL)));
  return z;
}

uint64_t moegen_draw(uint64_t key, uint64_t i) { return draw(key, i); }

/* Standard normal number i of stream key (Box-Muller, double). */
static inline double normal_at(uint64_t key, uint64_t i) {
  uint64_t p = i >> 1;
  double u1 = ((double)(draw(key, 2 * p) >> 11) + 1.0) * 0x1.0p-53; /* (0,1] */
  double u2 = (double)(draw(key, 2 * p + 1) >> 11) * 0x1.0p-53;     /* [0,1) */
  double r = sqrt(-2.0 * log(u1));
  double a = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(a) : r * cos(a);
}

void moegen_normal_f64(uint64_t key, int64_t n, double std, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = std * normal_at(key, (uint64_t)i);
}

void moegen_normal_f32(uint64_t key, int64_t n, double std, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(std * normal_at(key, (uint64_t)i));
}

/* fp32 -> bf16 bits, round to nearest even (inputs are finite). */
static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

void moegen_normal_bf16(uint64_t key, int64_t n, double std, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = f32_to_bf16_rne((float)(std * normal_at(key, (uint64_t)i)));
}

/* ---- quantizer helpers (input production only) ---- */

/* E4M3 (fn variant) positive grid: byte b in 0..126 -> value. */
static double e4m3_grid[127];
static int e4m3_ready = 0;
static void e4m3_init(void) {
  if (e4m3_ready) return;
  for (int b = 0; b < 127; ++b) {
    int e = b >> 3, m = b & 7;
    e4m3_grid[b] = e ? ldexp(1.0 + m / 8.0, e - 7) : ldexp(m / 8.0, -6);
  }
  e4m3_ready = 1;
}

/* Nearest E4M3 byte to v >= 0, ties to the even byte, saturating at 448. */
static uint8_t e4m3_encode(double v) {
  if (!(v > 0)) return 0;
  if (v >= 448.0) return 126;
  int lo = 0, hi = 126; /* grid is increasing: find last grid <= v */
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (e4m3_grid[mid] <= v) lo = mid; else hi = mid - 1;
  }
  if (lo == 126) return 126;
  double a = e4m3_grid[lo], b = e4m3_grid[lo + 1];
  if (v - a < b - v) return (uint8_t)lo;
  if (v - a > b - v) return (uint8_t)(lo + 1);
  return (uint8_t)((lo & 1) ? lo + 1 : lo);
}

/* Nearest E2M1 magnitude code (0..7) to v >= 0, ties to the even code,
 * clamped to 6.0 (code 7).  Grid 0, .5, 1, 1.5, 2, 3, 4, 6. */
static uint8_t e2m1_mag_encode(double v) {
  if (v <= 0.25) return 0;
  if (v < 0.75) return 1;
  if (v <= 1.25) return 2;
  if (v < 1.75) return 3;
  if (v <= 2.5) return 4;
  if (v < 3.5) return 5;
  if (v <= 5.0) return 6;
  return 7;
}

/* Quantize fp32 W[N][K] (row-major) to NVFP4:
 *   ts = amax|W| / (6*448); block scale = E4M3_rne_sat(amax_b / (6*ts));
 *   code = nearest E2M1 to |w| / (scale_b * ts), ties even, clamp 6. */
void moegen_quant_nvfp4(const float* W, int64_t N, int64_t K, uint8_t* codes,
                        uint8_t* scales, float* ts_out) {
  e4m3_init();
  double amax = 0.0;
  for (int64_t i = 0; i < N * K; ++i) {
    double a = fabs((double)W[i]);
    if (a > amax) amax = a;
  }
  float ts = (float)(amax / (6.0 * 448.0));
  *ts_out = ts;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    const float* row = W + n * K;
    for (int64_t b = 0; b < K / 16; ++b) {
      double ab = 0.0;
      for (int i = 0; i < 16; ++i) {
        double a = fabs((double)row[16 * b + i]);
        if (a > ab) ab = a;
      }
      uint8_t sb = (ts > 0) ? e4m3_encode(ab / (6.0 * (double)ts)) : 0;
      scales[n * (K / 16) + b] = sb;
      double sv = e4m3_grid[sb] * (double)ts;
      for (int i = 0; i < 16; i += 2) {
        uint8_t c[2];
        for (int h = 0; h < 2; ++h) {
          double w = (double)row[16 * b + i + h];
          uint8_t m = (sv > 0) ? e2m1_mag_encode(fabs(w) / sv) : 0;
          c[h] = (uint8_t)(m | ((w < 0 && m) ? 8 : 0));
        }
        codes[n * (K / 2) + (16 * b + i) / 2] = (uint8_t)(c[0] | (c[1] << 4));
      }
    }
  }
}

/* double -> IEEE binary16 bits, round to nearest even (finite, no overflow
 * handling beyond saturation to max finite). */
static uint16_t f64_to_f16_rne(double v) {
  uint16_t sign = (v < 0) ? 0x8000 : 0;
  double a = fabs(v);
  if (a == 0) return sign;
  if (a >= 65504.0) return (uint16_t)(sign | 0x7bff);
  int e;
  frexp(a, &e); /* a = f * 2^e, f in [0.5,1) -> unbiased exp e-1 */
  int ue = e - 1;
  if (ue < -14) ue = -14; /* subnormal range shares exponent -14 */
  double q = ldexp(a, 10 - ue); /* significand in units of the last place */
  double r = nearbyint(q);      /* default rounding mode: nearest even */
  uint32_t mant = (uint32_t)r;
  uint32_t biased = (uint32_t)(ue + 15);
  if (mant >= 2048) { mant >>= 1; biased += 1; }
  if (mant < 1024) return (uint16_t)(sign | mant); /* subnormal */
  if (biased >= 31) return (uint16_t)(sign | 0x7bff);
  return (uint16_t)(sign | (biased << 10) | (mant - 1024));
}

static double f16_bits_to_f64(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v = e ? ldexp(1.0 + m / 1024.0, e - 15) : ldexp(m / 1024.0, -14);
  return s ? -v : v;
}

/* Quantize fp32 W[N][K] to the Q6_K-style superblock format described in the
 * header comment: s_j = amax_j/31; d = fp16(max_j s_j / 127);
 * sc_j = clamp(rne(s_j/d), -128, 127); q = clamp(rne(w/(d*sc_j)), -32, 31)+32. */
void moegen_quant_q6k(const float* W, int64_t N, int64_t K, uint8_t* out) {
  const int64_t nsb = K / 256;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t s = 0; s < nsb; ++s) {
      const float* w = W + n * K + s * 256;
      uint8_t* blk = out + (n * nsb + s) * 210;
      memset(blk, 0, 210);
      double sj[16], smax = 0.0;
      for (int j = 0; j < 16; ++j) {
        double a = 0.0;
        for (int i = 0; i < 16; ++i) {
          double v = fabs((double)w[16 * j + i]);
          if (v > a) a = v;
        }
        sj[j] = a / 31.0;
        if (sj[j] > smax) smax = sj[j];
      }
      uint16_t dbits = f64_to_f16_rne(smax / 127.0);
      double d = f16_bits_to_f64(dbits);
      int8_t sc[16];
      for (int j = 0; j < 16; ++j) {
        double r = (d > 0) ? nearbyint(sj[j] / d) : 0.0;
        if (r > 127) r = 127;
        if (r < -128) r = -128;
        sc[j] = (int8_t)r;
      }
      for (int i = 0; i < 256; ++i) {
        double den = d * (double)sc[i / 16];
        int q = 32;
        if (den != 0) {
          double r = nearbyint((double)w[i] / den);
          if (r > 31) r = 31;
          if (r < -32) r = -32;
          q = (int)r + 32;
        }
        blk[i >> 1] |= (uint8_t)((q & 15) << (4 * (i & 1)));
        blk[128 + (i >> 2)] |= (uint8_t)(((q >> 4) & 3) << (2 * (i & 3)));
      }
      memcpy(blk + 192, sc, 16);
      blk[208] = (uint8_t)(dbits & 0xff);
      blk[209] = (uint8_t)(dbits >> 8);
    }
  }
}

/* Quantize fp32 W[N][K] to Q8_0-style blocks of 32: d = fp16(amax/127),
 * q = clamp(rne(w/d), -127, 127); a block is d (fp16 little-endian, 2 bytes)
 * then the 32 int8 codes. */
void moegen_quant_q8_0(const float* W, int64_t N, int64_t K, uint8_t* out) {
  const int64_t nb = K / 32;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t b = 0; b < nb; ++b) {
      const float* w = W + n * K + b * 32;
      uint8_t* blk = out + (n * nb + b) * 34;
      double a = 0.0;
      for (int i = 0; i < 32; ++i) {
        double v = fabs((double)w[i]);
        if (v > a) a = v;
      }
      uint16_t dbits = f64_to_f16_rne(a / 127.0);
      double d = f16_bits_to_f64(dbits);
      blk[0] = (uint8_t)(dbits & 0xff);
      blk[1] = (uint8_t)(dbits >> 8);
      for (int i = 0; i < 32; ++i) {
        double r = (d > 0) ? nearbyint((double)w[i] / d) : 0.0;
        if (r > 127) r = 127;
        if (r < -127) r = -127;
        blk[2 + i] = (uint8_t)(int8_t)r;
      }
    }
  }
}

/* Gaussian N(0, std) fp32 matrix quantized to NVFP4 in one call. */
void moegen_nvfp4_normal(uint64_t key, int64_t N, int64_t K, double std,
                         float* scratch, uint8_t* codes, uint8_t* scales, float* ts) {
  moegen_normal_f32(key, N * K, std, scratch);
  moegen_quant_nvfp4(scratch, N, K, codes, scales, ts);
}

void moegen_q6k_normal(uint64_t key, int64_t N, int64_t K, double std,
                       float* scratch, uint8_t* out) {
  moegen_normal_f32(key, N * K, std, scratch);
  moegen_quant_q6k(scratch, N, K, out);
}

/* IQ3-style codebook blocks with our own grid: the 256 smallest vectors of
 * four positive odd integers <= 15 by squared norm, then lexicographically
 * (this generator's own copy, used to encode).  Superblock of 256 weights of a
 * row, 102 bytes: d fp16 | 8 x 4-bit s_j (32 weights each) | 64 grid indices
 * (4 weights each) | 32 sign bytes; w = d * (2 s_j + 1) * grid * sign. */
static uint8_t g3_grid[256][4];
static int16_t g3_index[8 * 8 * 8 * 8]; /* ((m-1)/2 digits, base 8) -> entry or -1 */

static void g3_init(void) {
  static int ready = 0;
  if (ready) return;
  for (int i = 0; i < 4096; ++i) g3_index[i] = -1;
  int n = 0;
  for (int norm = 4; n < 256; norm += 8)
    for (int v = 0; v < 4096 && n < 256; ++v) {  /* v's base-8 digits in lexicographic order */
      const int m0 = 2 * (v >> 9) + 1, m1 = 2 * ((v >> 6) & 7) + 1;
      const int m2 = 2 * ((v >> 3) & 7) + 1, m3 = 2 * (v & 7) + 1;
      if (m0 * m0 + m1 * m1 + m2 * m2 + m3 * m3 != norm) continue;
      g3_grid[n][0] = (uint8_t)m0; g3_grid[n][1] = (uint8_t)m1;
      g3_grid[n][2] = (uint8_t)m2; g3_grid[n][3] = (uint8_t)m3;
      g3_index[v] = (int16_t)n++;
    }
  ready = 1;
}

/* Quantize fp32 W[N][K] (K % 256 == 0): per 32-weight sub-block the unit
 * u_j = amax_j / 9 (9: the grid's largest magnitude), d = fp16(max_j u_j / 31),
 * s_j = nearest (u_j / d - 1) / 2
 * in [0, 15]; each group of 4 takes the nearest odd magnitudes when that
 * vector is in the grid, else the grid entry nearest in L2. */
void moegen_quant_iq3g(const float* W, int64_t N, int64_t K, uint8_t* out) {
  g3_init();
  const int64_t nb = K / 256;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t b = 0; b < nb; ++b) {
      const float* w = W + n * K + b * 256;
      uint8_t* blk = out + (n * nb + b) * 102;
      memset(blk, 0, 102);
      double u[8], umax = 0.0;
      for (int j = 0; j < 8; ++j) {
        double a = 0.0;
        for (int i = 0; i < 32; ++i) a = fmax(a, fabs((double)w[32 * j + i]));
        u[j] = a / 9.0;
        umax = fmax(umax, u[j]);
      }
      const uint16_t dbits = f64_to_f16_rne(umax / 31.0);
      const double d = f16_bits_to_f64(dbits);
      blk[0] = (uint8_t)(dbits & 0xff);
      blk[1] = (uint8_t)(dbits >> 8);
      if (!(d > 0.0)) continue;
      for (int j = 0; j < 8; ++j) {
        double sj = nearbyint((u[j] / d - 1.0) / 2.0);
        if (sj < 0) sj = 0;
        if (sj > 15) sj = 15;
        blk[2 + j / 2] |= (uint8_t)((int)sj << (4 * (j % 2)));
        const double unit = d * (2.0 * sj + 1.0);
        for (int g = 8 * j; g < 8 * j + 8; ++g) {
          double t[4];
          int code = 0;
          for (int i = 0; i < 4; ++i) {
            const float x = w[4 * g + i];
            if (x < 0) blk[70 + (4 * g + i) / 8] |= (uint8_t)(1u << ((4 * g + i) % 8));
            t[i] = fabs((double)x) / unit;
            double m = 2.0 * nearbyint((t[i] - 1.0) / 2.0) + 1.0;
            if (m < 1) m = 1;
            if (m > 15) m = 15;
            code = code * 8 + ((int)m - 1) / 2;
          }
          int e = g3_index[code];
          if (e < 0) {
            double best = 1e300;
            for (int c = 0; c < 256; ++c) {
              double err = 0.0;
              for (int i = 0; i < 4; ++i) {
                const double dd = t[i] - g3_grid[c][i];
                err += dd * dd;
              }
              if (err < best) { best = err; e = c; }
            }
          }
          blk[6 + g] = (uint8_t)e;
        }
      }
    }
  }
}

void moegen_iq3g_normal(uint64_t key, int64_t N, int64_t K, double std,
                        float* scratch, uint8_t* out) {
  moegen_normal_f32(key, N * K, std, scratch);
  moegen_quant_iq3g(scratch, N, K, out);
}

/* IQ1-style ternary-grid superblocks (the oracle's reading): grid = the 1024
 * vectors of eight values in {-1, 0, +1} with the fewest nonzero values, by
 * nonzero count, then lexicographically (-1 < 0 < +1; this generator's own
 * copy, used to encode).  Superblock of 256 weights of a row, 46 bytes:
 * d fp16 | 8 x 4-bit s_j (32 weights each) | 32 low index bytes (8 weights
 * each) | 8 bytes of 2-bit high index parts; w = d * (2 s_j + 1) * grid. */
static int16_t g1_index[6561]; /* base-3 code (digit = value + 1, value 0 first) -> entry or -1 */

static void g1_init(void) {
  static int ready = 0;
  if (ready) return;
  for (int i = 0; i < 6561; ++i) g1_index[i] = -1;
  int n = 0;
  for (int nz = 0; nz <= 8 && n < 1024; ++nz)
    for (int u = 0; u < 6561 && n < 1024; ++u) {
      int c = 0;
      for (int r = u, i = 0; i < 8; ++i, r /= 3) c += (r % 3) != 1;
      if (c == nz) g1_index[u] = (int16_t)n++;
    }
  ready = 1;
}

/* Quantize fp32 W[N][K] (K % 256 == 0): per 32-weight sub-block the unit
 * u_j = amax_j, d = fp16(max_j u_j / 31), s_j = nearest (u_j / d - 1) / 2 in
 * [0, 15]; each weight rounds to the nearest of -1, 0, +1 units (|w| >= unit/2
 * is nonzero) and while a group's vector is not in the grid its nonzero
 * value of least magnitude becomes 0. */
void moegen_quant_iq1g(const float* W, int64_t N, int64_t K, uint8_t* out) {
  g1_init();
  const int64_t nb = K / 256;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t b = 0; b < nb; ++b) {
      const float* w = W + n * K + b * 256;
      uint8_t* blk = out + (n * nb + b) * 46;
      memset(blk, 0, 46);
      double u[8], umax = 0.0;
      for (int j = 0; j < 8; ++j) {
        double a = 0.0;
        for (int i = 0; i < 32; ++i) a = fmax(a, fabs((double)w[32 * j + i]));
        u[j] = a;
        umax = fmax(umax, u[j]);
      }
      const uint16_t dbits = f64_to_f16_rne(umax / 31.0);
      const double d = f16_bits_to_f64(dbits);
      blk[0] = (uint8_t)(dbits & 0xff);
      blk[1] = (uint8_t)(dbits >> 8);
      int sj[8] = {0};
      if (d > 0.0)
        for (int j = 0; j < 8; ++j) {
          double v = nearbyint((u[j] / d - 1.0) / 2.0);
          sj[j] = v < 0 ? 0 : (v > 15 ? 15 : (int)v);
          blk[2 + j / 2] |= (uint8_t)(sj[j] << (4 * (j % 2)));
        }
      for (int g = 0; g < 32; ++g) {
        const double unit = d * (2.0 * sj[g / 4] + 1.0);
        double t[8];
        int v[8];
        for (int i = 0; i < 8; ++i) {
          t[i] = d > 0.0 ? (double)w[8 * g + i] / unit : 0.0;
          v[i] = fabs(t[i]) >= 0.5 ? (t[i] < 0 ? -1 : 1) : 0;
        }
        int e;
        for (;;) {
          int code = 0;
          for (int i = 0; i < 8; ++i) code = code * 3 + (v[i] + 1);
          e = g1_index[code];
          if (e >= 0) break;
          int m = -1;
          for (int i = 0; i < 8; ++i)
            if (v[i] != 0 && (m < 0 || fabs(t[i]) < fabs(t[m]))) m = i;
          v[m] = 0;
        }
        blk[6 + g] = (uint8_t)(e & 255);
        blk[38 + g / 4] |= (uint8_t)((e >> 8) << (2 * (g % 4)));
      }
    }
  }
}

void moegen_iq1g_normal(uint64_t key, int64_t N, int64_t K, double std,
                        float* scratch, uint8_t* out) {
  moegen_normal_f32(key, N * K, std, scratch);
  moegen_quant_iq1g(scratch, N, K, out);
}

void moegen_q8_0_normal(uint64_t key, int64_t N, int64_t K, double std,
                        float* scratch, uint8_t* out) {
  moegen_normal_f32(key, N * K, std, scratch);
  moegen_quant_q8_0(scratch, N, K, out);
}

/* Seeded permutation of 0..n-1 (Fisher-Yates driven by the stream). */
void moegen_permutation(uint64_t key, int32_t n, int32_t* out) {
  for (int32_t i = 0; i < n; ++i) out[i] = i;
  for (int32_t i = n - 1; i > 0; --i) {
    uint64_t r = draw(key, (uint64_t)i);
    int32_t j = (int32_t)(r % (uint64_t)(i + 1));
    int32_t t = out[i]; out[i] = out[j]; out[j] = t;
  }
}

/* Static router bias b[e] = -alpha * s * ln(rank_e), rank_e = 1 + perm[e]:
 * shapes the expert load toward a Zipf(s) profile over a seeded ranking. */
void moegen_zipf_bias(uint64_t key, int32_t E, double s, double alpha, float* bias,
                      int32_t* rank_out) {
  int32_t perm[4096];
  if (E > 4096) return;
  moegen_permutation(key, E, perm);
  for (int32_t e = 0; e < E; ++e) {
    bias[e] = (float)(-alpha * s * log((double)(perm[e] + 1)));
    if (rank_out) rank_out[e] = perm[e] + 1;
  }
}

int moegen_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
