/*
 * fp_oracle.c -- plain CPU reference for the floating-point quantization
 * modes (mxfp4, nvfp4, mxfp8): codes are small floats, one unsigned byte of
 * scale per group, no bias.
 *
 * TEST INFRASTRUCTURE ONLY (see qmm_oracle.h): the checker for the HIP path,
 * never linked into it.
 *
 * Source: "mlx 1.0.0 backend/cpu/quantized.cpp" -- the E2M1 value table
 * (FP4_LUT), to_fp4_e2m1, to_fp8_e8m0, dequantize_scale, the per-group
 * steps of fp_quantize_dequantize (absolute maximum, divided by the largest
 * code value, the scale stored in one byte, each element divided by the
 * decoded scale and encoded), and fp_qmm_t / fp_qmm_t_simd (a scale per
 * group times the group's sum of x * code value, accumulated in fp32).
 *
 * Modes (bits, group size): (4, 32) mxfp4, E2M1 codes, e8m0 scale;
 * (4, 16) nvfp4, E2M1 codes, E4M3 scale; (8, 32) mxfp8, E4M3 codes, e8m0
 * scale. 4-bit codes pack two per byte, the first in the low nibble.
 *
 * Readings where the page is silent: E4M3 encoding rounds to nearest even
 * and saturates to +-448 (the page calls a helper it does not print); the
 * e8m0 exponent round(log2 x) is taken with the exact logarithm; the scale
 * is rounded to T before use, as the page's dequantize_scale<T> does.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "qmm_oracle.h"

/* E2M1 values of codes 0..15 (sign in bit 3). */
static const float kE2M1[16] = {0.0f,  0.5f,  1.0f,  1.5f,  2.0f,  3.0f,  4.0f,  6.0f,
                                -0.0f, -0.5f, -1.0f, -1.5f, -2.0f, -3.0f, -4.0f, -6.0f};

float orc_fp4_value(uint8_t code) { return kE2M1[code & 15]; }

/* Nearest E2M1 value, ties to the even code, magnitudes above 5 to 6. */
uint8_t orc_fp4_encode(float x) {
  if (isnan(x)) return 0x7;
  const uint8_t sign = signbit(x) ? 0x8 : 0x0;
  const float a = fabsf(x);
  uint8_t c;
  if (a > 5.0f) c = 7;
  else if (a >= 3.5f) c = 6;
  else if (a > 2.5f) c = 5;
  else if (a >= 1.75f) c = 4;
  else if (a > 1.25f) c = 3;
  else if (a >= 0.75f) c = 2;
  else if (a > 0.25f) c = 1;
  else c = 0;
  return c | sign;
}

/* E4M3 (no infinities; 0x7f / 0xff are NaN): value of a byte. */
float orc_fp8_e4m3_value(uint8_t b) {
  const int e = (b >> 3) & 15, m = b & 7;
  float v;
  if (e == 15 && m == 7) v = NAN;
  else if (e == 0) v = ldexpf((float)m, -9);          /* m/8 * 2^-6 */
  else v = ldexpf(1.0f + (float)m / 8.0f, e - 7);
  return (b & 0x80) ? -v : v;
}

/* Round to the nearest E4M3 value, ties to even; magnitudes of 448 and
 * more (whose rounding would leave the format) saturate to 448. */
uint8_t orc_fp8_e4m3_encode(float x) {
  if (isnan(x)) return 0x7f;
  const uint8_t sign = signbit(x) ? 0x80 : 0x00;
  const float a = fabsf(x);
  if (a >= 448.0f) return sign | 0x7e;
  int e;
  frexpf(a, &e);          /* a = f * 2^e, f in [0.5, 1) */
  e -= 1;                 /* a in [2^e, 2^(e+1)) */
  if (a == 0.0f || e < -6) {
    /* subnormal grid: multiples of 2^-9; rintf rounds half to even */
    const int q = (int)rintf(ldexpf(a, 9));
    return sign | (uint8_t)q;   /* q == 8 is the smallest normal, 0x08 */
  }
  int q = (int)rintf((ldexpf(a, -e) - 1.0f) * 8.0f);
  if (q == 8) { q = 0; e += 1; }
  return sign | (uint8_t)(((e + 7) << 3) | q);
}

/* e8m0 exponent byte: n = round(log2 x) clamped to [-127, 127], stored
 * n + 127. Exact: with x = f * 2^e (f in [1, 2)), n = e + (f >= sqrt 2),
 * decided as x^2 >= 2^(2e+1) in double (exact for a float x). Zero and
 * negative x give 0; infinities and NaN 0xff. */
uint8_t orc_e8m0_encode(float x) {
  if (!isfinite(x)) return 0xff;
  if (x <= 0.0f) return 0x00;
  int e;
  frexp((double)x, &e);
  e -= 1;
  const double xx = (double)x * (double)x;
  int n = e + (xx >= ldexp(1.0, 2 * e + 1) ? 1 : 0);
  if (n < -127) n = -127;
  if (n > 127) n = 127;
  return (uint8_t)(n + 127);
}

/* Decoded scale before rounding to T: 2^(s-127) for an e8m0 byte (byte 0
 * also gives 2^-127), the E4M3 value for group size 16. */
static float fp_scale_f32(uint8_t s, int gs) {
  if (gs == 16) return orc_fp8_e4m3_value(s);
  return ldexpf(1.0f, (int)s - 127);
}

/* The scale as the matmul and dequantizer use it: rounded to T. */
float orc_fp_scale(uint8_t s, int gs, int dtype) {
  const float v = fp_scale_f32(s, gs);
  if (dtype == ORC_F16) return orc_f16_to_f32(orc_f32_to_f16(v));
  if (dtype == ORC_BF16) return orc_bf16_to_f32(orc_f32_to_bf16(v));
  return v;
}

static int fp_mode_ok(int bits, int gs) {
  if (bits == 4) return gs == 32 || gs == 16 ? 0 : -2;
  if (bits == 8) return gs == 32 ? 0 : -2;
  return -1;
}

static float code_value(const uint8_t* row, int64_t k, int bits) {
  if (bits == 8) return orc_fp8_e4m3_value(row[k]);
  const uint8_t b = row[k >> 1];
  return orc_fp4_value((k & 1) ? (b >> 4) : (b & 15));
}

int orc_fp_quantize(const void* w, int dtype, int64_t rows, int64_t K, int group_size,
                    int bits, uint8_t* wq, uint8_t* scales) {
  const int st = fp_mode_ok(bits, group_size);
  if (st) return st;
  if (dtype != ORC_F16 && dtype != ORC_BF16 && dtype != ORC_F32) return -4;
  if (rows < 1 || K < 1 || K % group_size) return -3;
  const int64_t G = K / group_size, rb = K * bits / 8;
  const float qmax = bits == 4 ? 6.0f : 448.0f;
  float buf[32];
  for (int64_t r = 0; r < rows; r++) {
    uint8_t* out = wq + r * rb;
    memset(out, 0, (size_t)rb);
    for (int64_t g = 0; g < G; g++) {
      const int64_t k0 = g * group_size;
      if (dtype == ORC_F32) memcpy(buf, (const float*)w + r * K + k0, group_size * 4);
      else orc_to_f32((const uint16_t*)w + r * K + k0, dtype, group_size, buf);
      float amax = 0.0f;
      for (int j = 0; j < group_size; j++) amax = fmaxf(amax, fabsf(buf[j]));
      const float s32 = amax / qmax;
      const uint8_t sc = group_size == 16 ? orc_fp8_e4m3_encode(s32) : orc_e8m0_encode(s32);
      scales[r * G + g] = sc;
      const float sd = fp_scale_f32(sc, group_size);   /* the page divides by the float scale */
      for (int j = 0; j < group_size; j++) {
        const float v = sd == 0.0f ? 0.0f : buf[j] / sd;
        const int64_t k = k0 + j;
        if (bits == 8) {
          out[k] = orc_fp8_e4m3_encode(v);
        } else {
          const uint8_t c = orc_fp4_encode(v);
          out[k >> 1] |= (k & 1) ? (uint8_t)(c << 4) : c;
        }
      }
    }
  }
  return 0;
}

int orc_fp_dequantize(const uint8_t* wq, const uint8_t* scales, int dtype, int64_t rows,
                      int64_t K, int group_size, int bits, float* w32, void* w_out) {
  const int st = fp_mode_ok(bits, group_size);
  if (st) return st;
  if (dtype != ORC_F16 && dtype != ORC_BF16 && dtype != ORC_F32) return -4;
  if (rows < 1 || K < 1 || K % group_size) return -3;
  const int64_t G = K / group_size, rb = K * bits / 8;
  for (int64_t r = 0; r < rows; r++) {
    for (int64_t k = 0; k < K; k++) {
      const float s = orc_fp_scale(scales[r * G + k / group_size], group_size, dtype);
      const float v = s * code_value(wq + r * rb, k, bits);
      if (w32) w32[r * K + k] = v;
      if (w_out) {
        if (dtype == ORC_F32) ((float*)w_out)[r * K + k] = v;
        else orc_from_f32(&v, dtype, 1, (uint16_t*)w_out + r * K + k);
      }
    }
  }
  return 0;
}

/* y[m,n] = sum over groups g of s[n,g] * (sum over k in g of x[m,k] * v[n,k]),
 * fp32, groups and k ascending, no fused multiply-add. */
int orc_fp_qmm_t(const void* x, const uint8_t* wq, const uint8_t* scales, int dtype, int64_t M,
                 int64_t N, int64_t K, int group_size, int bits, float* y32, void* y_out,
                 int nthreads) {
  const int st = fp_mode_ok(bits, group_size);
  if (st) return st;
  if (dtype != ORC_F16 && dtype != ORC_BF16 && dtype != ORC_F32) return -4;
  if (M < 1 || N < 1 || K < 1 || K % group_size) return -3;
  const int64_t G = K / group_size, rb = K * bits / 8;
  if (nthreads < 1) nthreads = 1;
  float* xall = (float*)malloc((size_t)M * K * sizeof(float));
  if (!xall) return -3;
#pragma omp parallel for num_threads(nthreads) schedule(static)
  for (int64_t m = 0; m < M; m++) {
    float* xr = xall + m * K;
    if (dtype == ORC_F32) memcpy(xr, (const float*)x + m * K, (size_t)K * 4);
    else orc_to_f32((const uint16_t*)x + m * K, dtype, K, xr);
    for (int64_t n = 0; n < N; n++) {
      float acc = 0.0f;
      for (int64_t g = 0; g < G; g++) {
        const float s = orc_fp_scale(scales[n * G + g], group_size, dtype);
        float gsum = 0.0f;
        for (int64_t k = g * group_size; k < (g + 1) * group_size; k++) {
          const float p = xr[k] * code_value(wq + n * rb, k, bits);
          gsum = gsum + p;
        }
        const float t = s * gsum;
        acc = acc + t;
      }
      if (y32) y32[m * N + n] = acc;
      if (y_out) {
        if (dtype == ORC_F32) ((float*)y_out)[m * N + n] = acc;
        else orc_from_f32(&acc, dtype, 1, (uint16_t*)y_out + m * N + n);
      }
    }
  }
  free(xall);
  return 0;
}

/* Non-transposed product in an fp mode (the page's fp_qmm): the weight
 * W [K, N] is quantized along N (row k holds N codes, one scale byte per
 * group of N), y[m,n] = sum over k ascending of x[m,k] * w[k,n] with
 * w[k,n] = scale_T(s[k, n/gs]) * v(code[k,n]) (exact in fp32), products and
 * sums in fp32, no fused multiply-add. */
int orc_fp_qmm_n(const void* x, const uint8_t* wq, const uint8_t* scales, int dtype, int64_t M,
                 int64_t N, int64_t K, int group_size, int bits, float* y32, void* y_out,
                 int nthreads) {
  const int st = fp_mode_ok(bits, group_size);
  if (st) return st;
  if (dtype != ORC_F16 && dtype != ORC_BF16 && dtype != ORC_F32) return -4;
  if (M < 1 || N < 1 || K < 1 || N % group_size) return -3;
  float* w = (float*)malloc((size_t)K * N * sizeof(float));
  float* xall = (float*)malloc((size_t)M * K * sizeof(float));
  if (!w || !xall) {
    free(w);
    free(xall);
    return -3;
  }
  const int rc = orc_fp_dequantize(wq, scales, dtype, K, N, group_size, bits, w, NULL);
  if (rc) {
    free(w);
    free(xall);
    return rc;
  }
  if (nthreads < 1) nthreads = 1;
  for (int64_t m = 0; m < M; m++) {
    if (dtype == ORC_F32) memcpy(xall + m * K, (const float*)x + m * K, (size_t)K * 4);
    else orc_to_f32((const uint16_t*)x + m * K, dtype, K, xall + m * K);
  }
#pragma omp parallel for collapse(2) num_threads(nthreads) schedule(static)
  for (int64_t m = 0; m < M; m++) {
    for (int64_t n = 0; n < N; n++) {
      float acc = 0.0f;
      for (int64_t k = 0; k < K; k++) {
        const float p = xall[m * K + k] * w[k * N + n];
        acc = acc + p;
      }
      if (y32) y32[m * N + n] = acc;
      if (y_out) {
        if (dtype == ORC_F32) ((float*)y_out)[m * N + n] = acc;
        else orc_from_f32(&acc, dtype, 1, (uint16_t*)y_out + m * N + n);
      }
    }
  }
  free(w);
  free(xall);
  return 0;
}
