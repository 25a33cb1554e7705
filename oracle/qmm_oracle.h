/*
 * qmm_oracle.h -- plain CPU reference for affine group-wise quantization.
 *
 * TEST INFRASTRUCTURE ONLY. This library is the checker for the HIP path:
 * only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load it. It shares no code, header, table or helper with the HIP
 * library, and the HIP library never calls it.
 *
 * Everything is row-major and contiguous. "T" is the storage type of
 * activations, scales, biases and outputs: ORC_F16, ORC_BF16 or ORC_F32,
 * passed as raw 2- or 4-byte words. All arithmetic is IEEE binary32 with
 * round-to-nearest-even; conversions to f16/bf16 are round-to-nearest-even.
 *
 * Sources (web pages, cited by title and section):
 *  [P1] "[Feature] Quantized Convolution 2D - Possible PR?" (mlx issue 2714):
 *       quantize_weights (reshape + zero-pad K), img2col, forward prose.
 *  [P3] "Improvements in the quantizer and dequantization kernel" (mlx PR
 *       1061): item 1 a-c, the quantizer rule.
 *  [P4] "mlx 1.0.0 backend/cpu/quantized.cpp": quantize (the per-group
 *       steps and the packing), get_pack_factor / get_bytes_per_pack,
 *       extract_bits, _qmm_t and _qmm_t_simd (dequantize + accumulate).
 */
#ifndef QMM_ORACLE_H
#define QMM_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F16 = 0, ORC_BF16 = 1, ORC_F32 = 2 };

/* Return codes: 0 ok, -1 bad bits, -2 bad group size, -3 bad shape,
 * -4 bad dtype. */

/* Scalar converters (hand-written round-to-nearest-even). */
uint16_t orc_f32_to_f16(float f);
float orc_f16_to_f32(uint16_t h);
uint16_t orc_f32_to_bf16(float f);
float orc_bf16_to_f32(uint16_t h);

/* Bulk converters, n elements. */
void orc_to_f32(const void* src, int dtype, int64_t n, float* dst);
void orc_from_f32(const float* src, int dtype, int64_t n, void* dst);

/* Bytes per packed row: K * bits / 8. */
int64_t orc_row_bytes(int64_t K, int bits);

/* Affine group-wise quantization of w[rows, K] (dtype T) into
 *   wq      : rows * K*bits/8 bytes (the caller may view it as uint32),
 *   scales  : [rows, K/gs] in T,
 *   biases  : [rows, K/gs] in T.
 * If s32/b32 are non-NULL they receive the fp32 scale and bias before the
 * final rounding to T (used by the invariant checks). */
int orc_quantize(const void* w, int dtype, int64_t rows, int64_t K,
                 int group_size, int bits, uint8_t* wq, void* scales,
                 void* biases, float* s32, float* b32);

/* Code k of a packed row (bit offset k*bits of the row's byte stream). */
uint32_t orc_unpack_code(const uint8_t* row, int64_t k, int bits);

/* Unpack all codes: codes[rows, K]. */
int orc_unpack(const uint8_t* wq, int64_t rows, int64_t K, int bits,
               uint8_t* codes);

/* Dequantize: w32[rows,K] = fl32(s*q + b) in fp32 (may be NULL) and
 * w_out[rows,K] = T(w32) (may be NULL). */
int orc_dequantize(const uint8_t* wq, const void* scales, const void* biases,
                   int dtype, int64_t rows, int64_t K, int group_size,
                   int bits, float* w32, void* w_out);

/* y32[M,N] = sum_k x[m,k] * w32[n,k], fp32, k ascending, no fused
 * multiply-add; y_out = T(y32). Either output may be NULL.
 * nthreads <= 1 runs single-threaded. */
int orc_qmm_t(const void* x, const uint8_t* wq, const void* scales,
              const void* biases, int dtype, int64_t M, int64_t N, int64_t K,
              int group_size, int bits, float* y32, void* y_out,
              int nthreads);

/* Same as orc_qmm_t for a subset of output rows [m0, m1) only; y32/y_out
 * then hold (m1-m0) rows. Used to check sampled rows of large problems. */
int orc_qmm_t_rows(const void* x, const uint8_t* wq, const void* scales,
                   const void* biases, int dtype, int64_t M, int64_t N,
                   int64_t K, int group_size, int bits, int64_t m0, int64_t m1,
                   float* y32, void* y_out, int nthreads);

/* Non-transposed product ("mlx 1.0.0 backend/cpu/quantized.cpp", _qmm):
 * W is [K, N], quantized along N (wq [K, N*bits/8] bytes, scales/biases
 * [K, N/gs]): y32[M,N] = sum_k x[m,k] * w32[k,n], fp32, k ascending, no
 * fused multiply-add; y_out = T(y32). Either output may be NULL. */
int orc_qmm_n(const void* x, const uint8_t* wq, const void* scales,
              const void* biases, int dtype, int64_t M, int64_t N, int64_t K,
              int group_size, int bits, float* y32, void* y_out,
              int nthreads);

/* Quantized 2-D convolution, NHWC, via the implicit im2col of [P1]:
 *   x  [B,H,W,C] (T), wq/scales/biases quantize the weight
 *   [O, kh, kw, C/groups] reshaped to [O, K_true] and zero-padded to
 *   K_pad = ceil(K_true/gs)*gs; y [B,OH,OW,O].
 * Output channel o of conv group g = o / (O/groups) reads input channels
 * [g*C/groups, (g+1)*C/groups). */
int orc_qconv2d_nhwc(const void* x, int64_t B, int64_t H, int64_t W,
                     int64_t C, const uint8_t* wq, const void* scales,
                     const void* biases, int64_t O, int kh, int kw,
                     int stride_h, int stride_w, int pad_h, int pad_w,
                     int groups, int dtype, int group_size, int bits,
                     float* y32, void* y_out, int nthreads);

/* ---- Floating-point modes (fp_oracle.c; "mlx 1.0.0
 * backend/cpu/quantized.cpp": FP4_LUT, to_fp4_e2m1, to_fp8_e8m0,
 * dequantize_scale, fp_quantize_dequantize, fp_qmm_t). (bits, group size):
 * (4, 32) mxfp4 = E2M1 codes + e8m0 scale; (4, 16) nvfp4 = E2M1 + E4M3
 * scale; (8, 32) mxfp8 = E4M3 codes + e8m0 scale. wq: rows * K*bits/8 bytes
 * (4-bit codes two per byte, first in the low nibble); scales: one byte per
 * group, [rows, K/gs]. */
float orc_fp4_value(uint8_t code);
uint8_t orc_fp4_encode(float x);
float orc_fp8_e4m3_value(uint8_t b);
uint8_t orc_fp8_e4m3_encode(float x);
uint8_t orc_e8m0_encode(float x);
/* decoded scale of byte s rounded to T (dtype), as the products use it */
float orc_fp_scale(uint8_t s, int group_size, int dtype);
int orc_fp_quantize(const void* w, int dtype, int64_t rows, int64_t K, int group_size,
                    int bits, uint8_t* wq, uint8_t* scales);
/* w32 = fl32(scale_T * value) (exact), w_out = T(w32); either may be NULL */
int orc_fp_dequantize(const uint8_t* wq, const uint8_t* scales, int dtype, int64_t rows,
                      int64_t K, int group_size, int bits, float* w32, void* w_out);
/* y[m,n] = sum_g scale_T[n,g] * sum_{k in g} x[m,k] * value[n,k], fp32,
 * ascending, no fused multiply-add; either output may be NULL */
int orc_fp_qmm_t(const void* x, const uint8_t* wq, const uint8_t* scales, int dtype, int64_t M,
                 int64_t N, int64_t K, int group_size, int bits, float* y32, void* y_out,
                 int nthreads);
int orc_fp_qmm_n(const void* x, const uint8_t* wq, const uint8_t* scales, int dtype, int64_t M,
                 int64_t N, int64_t K, int group_size, int bits, float* y32, void* y_out,
                 int nthreads);

#ifdef __cplusplus
}
#endif

#endif
