/*
 * qmm_oracle.c -- plain CPU reference for affine group-wise quantization.
 *
 * TEST INFRASTRUCTURE ONLY (see qmm_oracle.h). Build with
 *   gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC
 * so that every float operation below is one IEEE binary32 operation with
 * round-to-nearest-even and nothing is fused or reassociated.
 */
#include "qmm_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* fp16 / bf16 <-> fp32, round to nearest even.                         */
/* ------------------------------------------------------------------ */

static uint32_t f32_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

static float bits_f32(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}

uint16_t orc_f32_to_f16(float f) {
  uint32_t x = f32_bits(f);
  uint32_t sign = (x >> 16) & 0x8000u;
  uint32_t ax = x & 0x7fffffffu;
  if (ax >= 0x7f800000u) { /* inf or nan */
    if (ax == 0x7f800000u) return (uint16_t)(sign | 0x7c00u);
    return (uint16_t)(sign | 0x7e00u | ((ax >> 13) & 0x3ffu));
  }
  /* 65520 = halfway between 65504 (odd significand) and 2^16: ties to inf */
  if (ax >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u);
  uint32_t e = ax >> 23;
  if (e < 113) {
    /* |f| < 2^-14: the result is an f16 subnormal (or zero) in units of
       2^-24. value = M * 2^(e-150) with M the 24-bit significand, so the
       count of 2^-24 units is M * 2^(e-126). */
    if (e == 0) return (uint16_t)sign; /* f32 subnormals are < 2^-126 */
    uint32_t M = (ax & 0x7fffffu) | 0x800000u;
    uint32_t shift = 126 - e; /* >= 14 */
    if (shift > 24) return (uint16_t)sign;
    uint32_t m = M >> shift;
    uint32_t rem = M & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (m & 1u))) m++;
    return (uint16_t)(sign | m);
  }
  uint32_t h = ((e - 112) << 10) | ((ax & 0x7fffffu) >> 13);
  uint32_t rem = ax & 0x1fffu;
  if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h++;
  return (uint16_t)(sign | h);
}

float orc_f16_to_f32(uint16_t hv) {
  uint32_t h = hv;
  uint32_t sign = (h & 0x8000u) << 16;
  uint32_t e = (h >> 10) & 0x1fu;
  uint32_t m = h & 0x3ffu;
  if (e == 0x1f) return bits_f32(sign | 0x7f800000u | (m << 13));
  if (e == 0) {
    /* zero or subnormal: m * 2^-24, exact in binary32 */
    float v = (float)m * 5.9604644775390625e-08f;
    return sign ? -v : v;
  }
  return bits_f32(sign | ((e + 112) << 23) | (m << 13));
}

uint16_t orc_f32_to_bf16(float f) {
  uint32_t x = f32_bits(f);
  if ((x & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((x >> 16) | 0x40u);
  uint32_t lsb = (x >> 16) & 1u;
  x += 0x7fffu + lsb;
  return (uint16_t)(x >> 16);
}

float orc_bf16_to_f32(uint16_t h) { return bits_f32((uint32_t)h << 16); }

static float load_t(const void* p, int dtype, int64_t i) {
  if (dtype == ORC_F16) return orc_f16_to_f32(((const uint16_t*)p)[i]);
  if (dtype == ORC_BF16) return orc_bf16_to_f32(((const uint16_t*)p)[i]);
  return ((const float*)p)[i];
}

static void store_t(void* p, int dtype, int64_t i, float v) {
  if (dtype == ORC_F16)
    ((uint16_t*)p)[i] = orc_f32_to_f16(v);
  else if (dtype == ORC_BF16)
    ((uint16_t*)p)[i] = orc_f32_to_bf16(v);
  else
    ((float*)p)[i] = v;
}

void orc_to_f32(const void* src, int dtype, int64_t n, float* dst) {
  for (int64_t i = 0; i < n; i++) dst[i] = load_t(src, dtype, i);
}

void orc_from_f32(const float* src, int dtype, int64_t n, void* dst) {
  for (int64_t i = 0; i < n; i++) store_t(dst, dtype, i, src[i]);
}

/* ------------------------------------------------------------------ */
/* Argument checks: bits in {2,3,4,5,6,8}, group size in {32,64,128}    */
/* ([P4] the bits / group-size switches of the qmm dispatch).           */
/* ------------------------------------------------------------------ */

static int check_args(int dtype, int64_t K, int gs, int bits) {
  if (!(bits == 2 || bits == 3 || bits == 4 || bits == 5 || bits == 6 ||
        bits == 8))
    return -1;
  if (!(gs == 32 || gs == 64 || gs == 128)) return -2;
  if (K < 1 || K % gs != 0) return -3;
  if (!(dtype == ORC_F16 || dtype == ORC_BF16 || dtype == ORC_F32)) return -4;
  return 0;
}

int64_t orc_row_bytes(int64_t K, int bits) { return K * bits / 8; }

/* ------------------------------------------------------------------ */
/* Quantizer ([P3] item 1 a-c; the rounding and fp32 arithmetic of [P4]  */
/* quantize). Per group of gs weights:                                   */
/*  1. the anchor is the extreme of larger magnitude (the maximum when    */
/*     |min| == |max|), the step spans from it to the other extreme over  */
/*     2^bits - 1 levels, at least 1e-7 in magnitude, negative when the   */
/*     anchor is the maximum (codes then count down from it);             */
/*  2. zero point: the anchor is k = rint(anchor / step) steps from 0;    */
/*     for k != 0 the step becomes anchor / k and the offset (bias) is    */
/*     the anchor, so 0 lies on the grid; for k == 0 the offset is 0;     */
/*  3. each weight's code is rint((w - offset) / step), clamped to the    */
/*     levels, written into the row's little-endian bit stream at bit     */
/*     k*bits. [P4] packs power-of-two widths into 4-byte words, 3 and 5  */
/*     bits as 8 values in 3 / 5 bytes and 6 bits as 4 values in 3 bytes */
/*     (get_pack_factor, get_bytes_per_pack), each pack little-endian:    */
/*     the same bytes as this stream.                                     */
/* ------------------------------------------------------------------ */

typedef struct {
  float step, offset;
} qparams;

static void group_range(const void* w, int dtype, int64_t first, int n, float* lo, float* hi) {
  float a = INFINITY, b = -INFINITY;
  for (int j = 0; j < n; j++) {
    const float v = load_t(w, dtype, first + j);
    if (v < a) a = v;
    if (b < v) b = v;
  }
  *lo = a;
  *hi = b;
}

static qparams group_params(float lo, float hi, int bits) {
  const float levels = (float)((1 << bits) - 1);
  const int anchor_is_lo = fabsf(lo) > fabsf(hi);
  const float anchor = anchor_is_lo ? lo : hi;
  float step = (hi - lo) / levels;
  if (step < 1e-7f) step = 1e-7f;
  if (!anchor_is_lo) step = -step;
  qparams p = {step, 0.0f};
  const float k = rintf(anchor / step);
  if (k != 0.0f) {
    p.step = anchor / k;
    p.offset = anchor;
  }
  return p;
}

/* code of v, clamped to [0, 2^bits - 1] */
static uint32_t encode(float v, qparams p, int bits) {
  float q = rintf((v - p.offset) / p.step);
  const float top = (float)((1 << bits) - 1);
  if (q < 0.0f) q = 0.0f;
  if (q > top) q = top;
  return (uint32_t)q;
}

int orc_quantize(const void* w, int dtype, int64_t rows, int64_t K,
                 int group_size, int bits, uint8_t* wq, void* scales,
                 void* biases, float* s32, float* b32) {
  int rc = check_args(dtype, K, group_size, bits);
  if (rc) return rc;
  if (rows < 1) return -3;
  const int64_t groups_per_row = K / group_size;
  const int64_t row_bytes = K * bits / 8;
  for (int64_t r = 0; r < rows; r++) {
    uint8_t* stream = wq + r * row_bytes;
    memset(stream, 0, (size_t)row_bytes);
    for (int64_t g = 0; g < groups_per_row; g++) {
      const int64_t first = r * K + g * group_size, gi = r * groups_per_row + g;
      float lo, hi;
      group_range(w, dtype, first, group_size, &lo, &hi);
      const qparams p = group_params(lo, hi, bits);
      for (int j = 0; j < group_size; j++) {
        const uint32_t c = encode(load_t(w, dtype, first + j), p, bits);
        const int64_t bit = (g * group_size + j) * bits;   /* position in the row */
        for (int t = 0; t < bits; t++)
          if ((c >> t) & 1u) stream[(bit + t) >> 3] |= (uint8_t)(1u << ((bit + t) & 7));
      }
      store_t(scales, dtype, gi, p.step);
      store_t(biases, dtype, gi, p.offset);
      if (s32) s32[gi] = p.step;
      if (b32) b32[gi] = p.offset;
    }
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* Unpack and dequantize ([P4] extract_bits, _qmm_t / _qmm_t_simd).     */
/* ------------------------------------------------------------------ */

uint32_t orc_unpack_code(const uint8_t* row, int64_t k, int bits) {
  int64_t bit = k * bits;
  int64_t byte = bit >> 3;
  int off = (int)(bit & 7);
  uint32_t window = row[byte];
  if (off + bits > 8) window |= (uint32_t)row[byte + 1] << 8;
  return (window >> off) & ((1u << bits) - 1u);
}

int orc_unpack(const uint8_t* wq, int64_t rows, int64_t K, int bits,
               uint8_t* codes) {
  if (rows < 1 || K < 1) return -3;
  const int64_t rb = orc_row_bytes(K, bits);
  for (int64_t n = 0; n < rows; n++)
    for (int64_t k = 0; k < K; k++)
      codes[n * K + k] = (uint8_t)orc_unpack_code(wq + n * rb, k, bits);
  return 0;
}

/* One dequantized weight: the stored scale times the code, plus the stored
 * bias, each operation rounded to binary32 (scale * code is exact for f16 and
 * bf16 scales, whose significands have at most 11 bits, since codes have at
 * most 8). */
static float deq(float s, float b, uint32_t q) {
  float sq = s * (float)q;
  return sq + b;
}

int orc_dequantize(const uint8_t* wq, const void* scales, const void* biases,
                   int dtype, int64_t rows, int64_t K, int group_size,
                   int bits, float* w32, void* w_out) {
  int rc = check_args(dtype, K, group_size, bits);
  if (rc) return rc;
  if (rows < 1) return -3;
  const int64_t rb = orc_row_bytes(K, bits);
  const int64_t G = K / group_size;
  for (int64_t n = 0; n < rows; n++) {
    for (int64_t k = 0; k < K; k++) {
      int64_t g = n * G + k / group_size;
      float v = deq(load_t(scales, dtype, g), load_t(biases, dtype, g),
                    orc_unpack_code(wq + n * rb, k, bits));
      if (w32) w32[n * K + k] = v;
      if (w_out) store_t(w_out, dtype, n * K + k, v);
    }
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* y = x . dequant(W)^T with fp32 accumulation ([P4] _qmm_t_simd).      */
/* ------------------------------------------------------------------ */

/* Every weight of W dequantized to fp32 (as orc_dequantize, rows split over
 * threads; each element's arithmetic is the same). */
static float* dequant_all(const uint8_t* wq, const void* scales,
                          const void* biases, int dtype, int64_t N, int64_t K,
                          int gs, int bits, int nthreads) {
  float* w32 = (float*)malloc(sizeof(float) * (size_t)(N * K));
  if (!w32) return NULL;
  const int64_t rb = orc_row_bytes(K, bits);
  const int64_t G = K / gs;
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
  for (int64_t n = 0; n < N; n++)
    for (int64_t k = 0; k < K; k++) {
      const int64_t g = n * G + k / gs;
      w32[n * K + k] = deq(load_t(scales, dtype, g), load_t(biases, dtype, g),
                           orc_unpack_code(wq + n * rb, k, bits));
    }
  return w32;
}

int orc_qmm_t_rows(const void* x, const uint8_t* wq, const void* scales,
                   const void* biases, int dtype, int64_t M, int64_t N,
                   int64_t K, int group_size, int bits, int64_t m0, int64_t m1,
                   float* y32, void* y_out, int nthreads) {
  int rc = check_args(dtype, K, group_size, bits);
  if (rc) return rc;
  if (M < 1 || N < 1 || m0 < 0 || m1 > M || m1 <= m0) return -3;
  float* w32 = dequant_all(wq, scales, biases, dtype, N, K, group_size, bits, nthreads);
  if (!w32) return -5;
  const int64_t rows = m1 - m0;
  float* xr = (float*)malloc(sizeof(float) * (size_t)(rows * K));
  if (!xr) {
    free(w32);
    return -5;
  }
  for (int64_t r = 0; r < rows; r++)
    for (int64_t k = 0; k < K; k++) xr[r * K + k] = load_t(x, dtype, (m0 + r) * K + k);
  if (nthreads < 1) nthreads = 1;
  /* threads split the (row, column) pairs, so one row of x also spreads
     over every thread; each output's sum keeps its k-ascending order */
#pragma omp parallel for collapse(2) num_threads(nthreads) schedule(static)
  for (int64_t r = 0; r < rows; r++) {
    for (int64_t n = 0; n < N; n++) {
      float acc = 0.0f;
      for (int64_t k = 0; k < K; k++) {
        float prod = xr[r * K + k] * w32[n * K + k];
        acc = acc + prod;
      }
      if (y32) y32[r * N + n] = acc;
      if (y_out) store_t(y_out, dtype, r * N + n, acc);
    }
  }
  free(xr);
  free(w32);
  return 0;
}

int orc_qmm_t(const void* x, const uint8_t* wq, const void* scales,
              const void* biases, int dtype, int64_t M, int64_t N, int64_t K,
              int group_size, int bits, float* y32, void* y_out,
              int nthreads) {
  return orc_qmm_t_rows(x, wq, scales, biases, dtype, M, N, K, group_size,
                        bits, 0, M, y32, y_out, nthreads);
}

/* ------------------------------------------------------------------ */
/* Non-transposed product ([P4] _qmm): W [K, N] quantized along its rows  */
/* (groups of N), y[m,n] = sum over k ascending of x[m,k] * w[k,n].      */
/* ------------------------------------------------------------------ */

int orc_qmm_n(const void* x, const uint8_t* wq, const void* scales,
              const void* biases, int dtype, int64_t M, int64_t N, int64_t K,
              int group_size, int bits, float* y32, void* y_out,
              int nthreads) {
  int rc = check_args(dtype, N, group_size, bits);
  if (rc) return rc;
  if (M < 1 || K < 1) return -3;
  /* the K stored rows, each N long with its groups along N */
  float* w32 = dequant_all(wq, scales, biases, dtype, K, N, group_size, bits, nthreads);
  if (!w32) return -5;
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for collapse(2) num_threads(nthreads) schedule(static)
  for (int64_t m = 0; m < M; m++) {
    for (int64_t n = 0; n < N; n++) {
      float acc = 0.0f;
      for (int64_t k = 0; k < K; k++) {
        float prod = load_t(x, dtype, m * K + k) * w32[k * N + n];
        acc = acc + prod;
      }
      if (y32) y32[m * N + n] = acc;
      if (y_out) store_t(y_out, dtype, m * N + n, acc);
    }
  }
  free(w32);
  return 0;
}

/* ------------------------------------------------------------------ */
/* Quantized conv2d, NHWC, implicit im2col ([P1] img2col + forward).    */
/* Patch element k of output pixel (b, oy, ox) in conv group g is       */
/* (dy, dx, c) with k = (dy*kw + dx)*Cg + c, reading                    */
/* x[b, oy*sh - ph + dy, ox*sw - pw + dx, g*Cg + c], zero outside.      */
/* ------------------------------------------------------------------ */

int orc_qconv2d_nhwc(const void* x, int64_t B, int64_t H, int64_t W,
                     int64_t C, const uint8_t* wq, const void* scales,
                     const void* biases, int64_t O, int kh, int kw,
                     int stride_h, int stride_w, int pad_h, int pad_w,
                     int groups, int dtype, int group_size, int bits,
                     float* y32, void* y_out, int nthreads) {
  if (groups < 1 || C % groups || O % groups) return -3;
  if (kh < 1 || kw < 1 || stride_h < 1 || stride_w < 1 || pad_h < 0 ||
      pad_w < 0 || B < 1 || H < 1 || W < 1)
    return -3;
  const int64_t Cg = C / groups, Og = O / groups;
  const int64_t K_true = (int64_t)kh * kw * Cg;
  const int64_t K_pad = (K_true + group_size - 1) / group_size * group_size;
  int rc = check_args(dtype, K_pad, group_size, bits);
  if (rc) return rc;
  const int64_t OH = (H + 2 * pad_h - kh) / stride_h + 1;
  const int64_t OW = (W + 2 * pad_w - kw) / stride_w + 1;
  if (OH < 1 || OW < 1) return -3;
  float* w32 = dequant_all(wq, scales, biases, dtype, O, K_pad, group_size, bits, nthreads);
  if (!w32) return -5;
  const int64_t npix = B * OH * OW;
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel num_threads(nthreads)
  {
    float* patch = (float*)malloc(sizeof(float) * (size_t)K_true);
#pragma omp for schedule(static)
    for (int64_t m = 0; m < npix; m++) {
      const int64_t b = m / (OH * OW);
      const int64_t oy = (m / OW) % OH;
      const int64_t ox = m % OW;
      for (int64_t g = 0; g < groups; g++) {
        for (int dy = 0; dy < kh; dy++)
          for (int dx = 0; dx < kw; dx++)
            for (int64_t c = 0; c < Cg; c++) {
              int64_t iy = oy * stride_h - pad_h + dy;
              int64_t ix = ox * stride_w - pad_w + dx;
              int64_t k = ((int64_t)dy * kw + dx) * Cg + c;
              float v = 0.0f;
              if (iy >= 0 && iy < H && ix >= 0 && ix < W)
                v = load_t(x, dtype, ((b * H + iy) * W + ix) * C + g * Cg + c);
              patch[k] = v;
            }
        for (int64_t o = 0; o < Og; o++) {
          const int64_t n = g * Og + o;
          float acc = 0.0f;
          for (int64_t k = 0; k < K_true; k++) {
            float prod = patch[k] * w32[n * K_pad + k];
            acc = acc + prod;
          }
          if (y32) y32[m * O + n] = acc;
          if (y_out) store_t(y_out, dtype, m * O + n, acc);
        }
      }
    }
    free(patch);
  }
  free(w32);
  return 0;
}
