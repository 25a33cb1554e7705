// Floating-point quantization modes ("mlx 1.0.0 backend/cpu/quantized.cpp":
// FP4_LUT, to_fp4_e2m1, to_fp8_e8m0, dequantize_scale,
// fp_quantize_dequantize, fp_qmm_t). (bits, group size): (4, 32) mxfp4 =
// E2M1 codes with an e8m0 scale byte per group; (4, 16) nvfp4 = E2M1 codes
// with an E4M3 scale byte; (8, 32) mxfp8 = E4M3 codes with an e8m0 scale.
// No bias. 4-bit codes pack two per byte, the first in the low nibble.
//
// Codes are decoded with gfx950's OCP conversions (v_cvt_scalef32_pk_f32_fp4
// and _fp8 at scale 1, exact), the group scale is applied in fp32 after
// rounding it to T as the page's dequantize_scale<T> does.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "kernels.hpp"

namespace qmm {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- encoders
// E2M1 code of x: the grid {0, .5, 1, 1.5, 2, 3, 4, 6}; each midpoint between
// neighbours is passed when x exceeds it, or reaches it and the upper
// neighbour's code is even (ties to even); beyond 6 the top code. Sign in
// bit 3.
__device__ __forceinline__ uint32_t e2m1_encode(float x) {
  const float a = fabsf(x);
  uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
               (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
               (uint32_t)(a > 5.0f);
  if (a != a) c = 7;
  return c | ((__builtin_bit_cast(uint32_t, x) >> 28) & 8u);
}

// E4M3 (OCP, no infinities) with round to nearest even on the bit pattern;
// magnitudes of 448 and more saturate to 448 (0x7e).
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(x);
  if (a != a) return 0x7fu;
  if (a >= 448.0f) return sign | 0x7eu;
  if (a < 0.015625f) {                          // below 2^-6: multiples of 2^-9
    return sign | (uint32_t)__builtin_rintf(a * 512.0f);
  }
  const uint32_t au = u & 0x7fffffffu;
  const uint32_t e = (au >> 23) - 120u;         // biased 7: 2^-6 -> 1
  const uint32_t keep = (au >> 20) & 7u, rest = au & 0xfffffu;
  const uint32_t up = rest > 0x80000u || (rest == 0x80000u && (keep & 1u));
  return sign | ((e << 3) + keep + up);         // a carry moves into the exponent
}

// e8m0 exponent byte of x > 0: n = round(log2 x) (no ties exist: log2 x is
// never k + 1/2 for a float), clamped to [-127, 127], stored n + 127. For a
// normal x = 1.f * 2^e, n = e + (1.f >= sqrt 2), tested on the mantissa
// bits; below 2^-126 the only question is whether n reaches -126.
__device__ __forceinline__ uint32_t e8m0_encode(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  if ((u & 0x7f800000u) == 0x7f800000u) return 0xffu;   // inf / NaN
  if ((int32_t)u <= 0) return 0u;                        // zero or negative
  int n;
  if (u < 0x00800000u) {
    n = u >= 0x005a827au ? -126 : -127;   // 2^-126.5 = 0x5a8279.99.. * 2^-149
  } else {
    n = (int)(u >> 23) - 127 + ((u & 0x7fffffu) >= 0x3504f4u ? 1 : 0);
  }
  n = n < -127 ? -127 : (n > 127 ? 127 : n);
  return (uint32_t)(n + 127);
}

// ---------------------------------------------------------------- decoders
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  return __builtin_amdgcn_cvt_scalef32_f32_fp8(b, 1.0f, 0);
}

// Scale byte as stored, before rounding to T: 2^(s-127) (byte 0 too gives
// 2^-127), or the E4M3 value for groups of 16.
template <int GS>
__device__ __forceinline__ float scale_f32(uint32_t s) {
  if constexpr (GS == 16) return e4m3_value(s);
  return s == 0 ? __builtin_bit_cast(float, 0x00400000u) : __builtin_bit_cast(float, s << 23);
}

// The scale rounded to T. bf16 (and f32) hold every e8m0 and E4M3 value
// exactly; f16 holds E4M3 values and the powers 2^-24 .. 2^15, rounds
// smaller ones to 0 (2^-25 is a tie, to even) and larger ones to infinity.
template <class T, int GS>
__device__ __forceinline__ float scale_t(uint32_t s) {
  if constexpr (GS == 32 && __is_same(T, F16)) {
    if (s < 103u) return 0.0f;
    if (s > 142u) return __builtin_inff();
  }
  return scale_f32<GS>(s);
}

// ---------------------------------------------------------------- quantize
// One thread per group of GS consecutive elements of a row (groups of a
// row-major [rows, K] are consecutive): absolute maximum, scale =
// max / (6 or 448) stored in one byte, each element divided by the decoded
// scale and encoded.
template <class T, int BITS, int GS>
__global__ __launch_bounds__(256) void fp_quantize_kernel(const typename T::word* __restrict__ w,
                                                          int64_t ngroups,
                                                          uint8_t* __restrict__ wq,
                                                          uint8_t* __restrict__ sc) {
  const int64_t gi = blockIdx.x * 256ll + threadIdx.x;
  if (gi >= ngroups) return;
  constexpr int kWordBytes = sizeof(typename T::word);
  constexpr int kUnits = GS * kWordBytes / 16;
  float v[GS];
  const uint4* src = reinterpret_cast<const uint4*>(w + gi * GS);
#pragma unroll
  for (int i = 0; i < kUnits; i++) {
    const uint4 q = src[i];
    const uint32_t word[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; j++) {
      if constexpr (kWordBytes == 4) {
        v[i * 4 + j] = __builtin_bit_cast(float, word[j]);
      } else {
        v[i * 8 + 2 * j] = to_f32(T{}, (uint16_t)(word[j] & 0xffffu));
        v[i * 8 + 2 * j + 1] = to_f32(T{}, (uint16_t)(word[j] >> 16));
      }
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < GS; j++) amax = fmaxf(amax, fabsf(v[j]));
  const float s32 = amax / (BITS == 4 ? 6.0f : 448.0f);
  const uint32_t sb = GS == 16 ? e4m3_encode(s32) : e8m0_encode(s32);
  sc[gi] = (uint8_t)sb;
  const float sd = scale_f32<GS>(sb);
  constexpr int kWords = GS * BITS / 32;
  uint32_t out[kWords];
#pragma unroll
  for (int i = 0; i < kWords; i++) out[i] = 0u;
#pragma unroll
  for (int j = 0; j < GS; j++) {
    const float t = sd == 0.0f ? 0.0f : v[j] / sd;
    if constexpr (BITS == 4) out[j / 8] |= e2m1_encode(t) << (4 * (j % 8));
    else out[j / 4] |= e4m3_encode(t) << (8 * (j % 4));
  }
  uint8_t* dst = wq + gi * (GS * BITS / 8);
  if constexpr (kWords == 2) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(out[0], out[1]);
  } else {
#pragma unroll
    for (int i = 0; i < kWords / 4; i++)
      reinterpret_cast<uint4*>(dst)[i] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2],
                                                    out[4 * i + 3]);
  }
}

// ---------------------------------------------------------------- dequantize
// Decoded value of code j of a group: E2M1 or E4M3 at scale 1 (exact).
template <int BITS>
__device__ __forceinline__ void decode_word(uint32_t word, float* v) {
  if constexpr (BITS == 4) {
    // byte b holds codes 2b (low nibble) and 2b + 1
    const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 0);
    const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 1);
    const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 2);
    const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 3);
    v[0] = p0.x; v[1] = p0.y; v[2] = p1.x; v[3] = p1.y;
    v[4] = p2.x; v[5] = p2.y; v[6] = p3.x; v[7] = p3.y;
  } else {
    const f32x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(word, 1.0f, false);
    const f32x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(word, 1.0f, true);
    v[0] = lo.x; v[1] = lo.y; v[2] = hi.x; v[3] = hi.y;
  }
}

// One 32-bit word of codes (8 E2M1 or 4 E4M3) -> T pairs (k, k + 1), by the
// scale-1 conversions (exact: every code value is a T value)
template <class T, int BITS>
__device__ __forceinline__ void decode_pairs(uint32_t word, uint32_t* p) {
  if constexpr (BITS == 4) {
    if constexpr (__is_same(T, F16)) {
      p[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 0));
      p[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 1));
      p[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 2));
      p[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 3));
    } else {
      p[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, 0));
      p[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, 1));
      p[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, 2));
      p[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, 3));
    }
  } else {
    if constexpr (__is_same(T, F16)) {
      p[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, false));
      p[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, true));
    } else {
      p[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, false));
      p[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, true));
    }
  }
}

// T(s * v) for s >= 0 and an exact product: the word of the product with the
// sign of v restored (the compiler fuses a product converted to f16 into
// v_fma_mixlo_f16 with a +0 addend, which turns a -0 product into +0).
template <class T>
__device__ __forceinline__ uint32_t scaled_word(float s, float v) {
  const uint32_t h = from_f32(T{}, s * v);
  return h | ((__builtin_bit_cast(uint32_t, v) >> 16) & 0x8000u);
}

// One thread per group: w_out = T(scale_T * value) (the product is exact).
template <class T, int BITS, int GS>
__global__ __launch_bounds__(256) void fp_dequantize_kernel(const uint8_t* __restrict__ wq,
                                                            const uint8_t* __restrict__ sc,
                                                            int64_t ngroups,
                                                            typename T::word* __restrict__ out) {
  const int64_t gi = blockIdx.x * 256ll + threadIdx.x;
  if (gi >= ngroups) return;
  constexpr int kWords = GS * BITS / 32, kPer = 32 / BITS;
  uint32_t words[kWords];
  const uint8_t* src = wq + gi * (GS * BITS / 8);
  if constexpr (kWords == 2) {
    const uint2 q = *reinterpret_cast<const uint2*>(src);
    words[0] = q.x; words[1] = q.y;
  } else {
#pragma unroll
    for (int i = 0; i < kWords / 4; i++) {
      const uint4 q = reinterpret_cast<const uint4*>(src)[i];
      words[4 * i] = q.x; words[4 * i + 1] = q.y; words[4 * i + 2] = q.z; words[4 * i + 3] = q.w;
    }
  }
  const float s = scale_t<T, GS>(sc[gi]);
  float v[GS];
#pragma unroll
  for (int i = 0; i < kWords; i++) decode_word<BITS>(words[i], v + i * kPer);
  typename T::word* dst = out + gi * GS;
  if constexpr (sizeof(typename T::word) == 4) {
#pragma unroll
    for (int i = 0; i < GS / 4; i++)
      reinterpret_cast<float4*>(dst)[i] =
          make_float4(s * v[4 * i], s * v[4 * i + 1], s * v[4 * i + 2], s * v[4 * i + 3]);
  } else {
#pragma unroll
    for (int i = 0; i < GS / 8; i++) {
      uint32_t p[4];
#pragma unroll
      for (int j = 0; j < 4; j++)
        p[j] = scaled_word<T>(s, v[8 * i + 2 * j]) |
               (scaled_word<T>(s, v[8 * i + 2 * j + 1]) << 16);
      reinterpret_cast<uint4*>(dst)[i] = make_uint4(p[0], p[1], p[2], p[3]);
    }
  }
}

// ---------------------------------------------------------------- GEMV
// y[m, n] = T(sum over groups g of scale_T[n, g] * sum_{k in g} x[m, k] *
// value[n, k]) with fp32 accumulation. Workgroup = WV wavefronts x R rows of
// W for one row m of x (blockIdx.y); x[m] is staged in LDS as T. Each lane
// takes 16-byte units of a row (32 E2M1 or 16 E4M3 codes), unit u at lane
// u % 64, for R rows at once so that their loads overlap; the codes are
// decoded into T pairs and multiplied with the activation pairs by
// v_dot2_f32_{f16,bf16} (exact products, fp32 sums).
// Wavefronts per workgroup (WV) and rows per wavefront: see fp_qmv_t.

// Gathered products (GA): output batch z = blockIdx.z multiplies x batch
// lidx[z] (of nxb, M rows each) by weight batch ridx[z] (of nwb), indices
// clamped into range; a null array means z.
struct FpBatch {
  const int32_t* lidx;
  const int32_t* ridx;
  int nxb, nwb, M, B;
};

template <class T, int BITS, int GS, int kFpRows, bool GA, int WV>
__global__ __launch_bounds__(64 * WV) void fp_qmv_kernel(const typename T::word* __restrict__ x,
                                                     const uint8_t* __restrict__ wq,
                                                     const uint8_t* __restrict__ sc,
                                                     typename T::word* __restrict__ y, int N,
                                                     int K, FpBatch bt) {
  extern __shared__ uint4 xs4[];   // x[m] as T words, natural order
  const int m = blockIdx.y;
  if constexpr (GA) {
    const int z = blockIdx.z;
    int zx = z, zw = z;
    if (bt.lidx) {
      const int v = bt.lidx[z];
      zx = v < 0 ? 0 : (v >= bt.nxb ? bt.nxb - 1 : v);
    }
    if (bt.ridx) {
      const int v = bt.ridx[z];
      zw = v < 0 ? 0 : (v >= bt.nwb ? bt.nwb - 1 : v);
    }
    x += (int64_t)zx * bt.M * K;
    wq += (int64_t)zw * N * ((int64_t)K * BITS / 8);
    sc += (int64_t)zw * N * (K / GS);
    y += (int64_t)z * bt.M * N;
  }
  {
    // rows of x are 16-byte aligned (x is, and K % 32 == 0)
    const uint4* xr = reinterpret_cast<const uint4*>(x + (int64_t)m * K);
    for (int u = threadIdx.x; u < K / 8; u += 64 * WV) xs4[u] = xr[u];
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = (blockIdx.x * WV + wave) * kFpRows;
  constexpr int kCodes = 128 / BITS;            // codes per 16-byte unit
  const int units = K / kCodes;
  const int64_t rb = (int64_t)K * BITS / 8, G = K / GS;
  float acc[kFpRows];
#pragma unroll
  for (int r = 0; r < kFpRows; r++) acc[r] = 0.0f;

  for (int u = lane; u < units; u += 64) {
    u32x4 q[kFpRows];
#pragma unroll
    for (int r = 0; r < kFpRows; r++) {
      const int n = n0 + r < N ? n0 + r : N - 1;
      q[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wq + n * rb) + u);
    }
    // the unit's activations as T pairs (k, k + 1)
    const uint4* xv = xs4 + u * (kCodes / 8);
    uint32_t xw[kCodes / 2];
#pragma unroll
    for (int i = 0; i < kCodes / 8; i++) {
      const uint4 t = xv[i];
      xw[4 * i] = t.x; xw[4 * i + 1] = t.y; xw[4 * i + 2] = t.z; xw[4 * i + 3] = t.w;
    }
#pragma unroll
    for (int r = 0; r < kFpRows; r++) {
      const int n = n0 + r < N ? n0 + r : N - 1;
      const uint32_t words[4] = {q[r].x, q[r].y, q[r].z, q[r].w};
      // codes decoded into T pairs (k, k + 1), exactly: every E2M1 and E4M3
      // value is a T value
      uint32_t vp[kCodes / 2];
#pragma unroll
      for (int i = 0; i < 4; i++) decode_pairs<T, BITS>(words[i], vp + i * (kCodes / 8));
      // groups within the unit: BITS 4 -> 32 codes = 1 (GS 32) or 2 (GS 16)
      // groups; BITS 8 -> 16 codes = half of a group of 32
      constexpr int kGroups = kCodes >= GS ? kCodes / GS : 1;
      constexpr int kLen = kCodes >= GS ? GS : kCodes;
      const int64_t g0 = (int64_t)u * kCodes / GS;
#pragma unroll
      for (int g = 0; g < kGroups; g++) {
        // sum of x * value over the group's codes in fp32 (products of two
        // T values are exact in fp32)
        float gsum = 0.0f;
#pragma unroll
        for (int j = 0; j < kLen / 2; j++)
          gsum = dot2(T{}, xw[g * kLen / 2 + j], vp[g * kLen / 2 + j], gsum);
        acc[r] = fmaf(scale_t<T, GS>(sc[n * G + g0 + g]), gsum, acc[r]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kFpRows; r++) {
    float s = acc[r];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0 && n0 + r < N) y[(int64_t)m * N + n0 + r] = from_f32(T{}, s);
  }
}

// ---------------------------------------------------------------- launchers
template <class T, int BITS, int GS>
hipError_t fp_quantize_t(const void* w, int64_t rows, int64_t K, uint32_t* wq, uint8_t* sc,
                         hipStream_t st) {
  const int64_t ng = rows * (K / GS);
  hipLaunchKernelGGL((fp_quantize_kernel<T, BITS, GS>), dim3((unsigned)((ng + 255) / 256)),
                     dim3(256), 0, st, static_cast<const typename T::word*>(w), ng,
                     reinterpret_cast<uint8_t*>(wq), sc);
  return hipGetLastError();
}

template <class T, int BITS, int GS>
hipError_t fp_dequantize_t(const uint32_t* wq, const uint8_t* sc, int64_t rows, int64_t K,
                           void* out, hipStream_t st) {
  const int64_t ng = rows * (K / GS);
  hipLaunchKernelGGL((fp_dequantize_kernel<T, BITS, GS>), dim3((unsigned)((ng + 255) / 256)),
                     dim3(256), 0, st, reinterpret_cast<const uint8_t*>(wq), sc, ng,
                     static_cast<typename T::word*>(out));
  return hipGetLastError();
}

template <class T, int BITS, int GS, int R, int WV>
hipError_t fp_qmv_r(const void* x, const uint32_t* wq, const uint8_t* sc, int64_t M, int64_t N,
                    int64_t K, void* y, hipStream_t st, const FpBatch* bt) {
  const int64_t rows_per_block = WV * R;
  const dim3 grid((unsigned)((N + rows_per_block - 1) / rows_per_block), (unsigned)M,
                  bt ? (unsigned)bt->B : 1u);
  auto go = [&](auto kern, const FpBatch& b) {
    hipLaunchKernelGGL(kern, grid, dim3(64 * WV), (size_t)K * 2, st,
                       static_cast<const typename T::word*>(x),
                       reinterpret_cast<const uint8_t*>(wq), sc,
                       static_cast<typename T::word*>(y), (int)N, (int)K, b);
  };
  if (bt) go(fp_qmv_kernel<T, BITS, GS, R, true, WV>, *bt);
  else go(fp_qmv_kernel<T, BITS, GS, R, false, WV>, FpBatch{nullptr, nullptr, 1, 1, (int)M, 1});
  return hipGetLastError();
}

// Rows per wavefront and wavefronts per workgroup, measured on 4096 x 4096
// (f16, cold weights, every combination of 1/2/4 rows and 4/8 wavefronts):
// E2M1 codes run best with 8 wavefronts and the most rows per wavefront that
// still give 512 workgroups (mxfp4 M = 1 / 2 / 4: 4.24 / 5.03 / 7.34 us with
// 1 / 2 / 4 rows; nvfp4 4.22 / 5.34 / 7.25), E4M3 codes with 4 wavefronts of
// 2 rows once that gives 1024 workgroups (mxfp8 M = 2 / 4: 6.52 / 10.45 us,
// against 6.98 / 11.9 with 8 wavefronts of 1 row), else 8 wavefronts of 1
// row (M = 1: 5.79 us).
template <class T, int BITS, int GS>
hipError_t fp_qmv_t(const void* x, const uint32_t* wq, const uint8_t* sc, int64_t M, int64_t N,
                    int64_t K, void* y, hipStream_t st, const FpBatch* bt) {
  const int64_t want = BITS == 8 ? 1024 : 512, nb = bt ? bt->B : 1;
  auto blocks = [&](int64_t w, int64_t r) { return (N + w * r - 1) / (w * r) * M * nb; };
  if constexpr (BITS == 8) {
    if (blocks(4, 2) >= want) return fp_qmv_r<T, BITS, GS, 2, 4>(x, wq, sc, M, N, K, y, st, bt);
    return fp_qmv_r<T, BITS, GS, 1, 8>(x, wq, sc, M, N, K, y, st, bt);
  } else {
    if (blocks(8, 4) >= want) return fp_qmv_r<T, BITS, GS, 4, 8>(x, wq, sc, M, N, K, y, st, bt);
    if (blocks(8, 2) >= want) return fp_qmv_r<T, BITS, GS, 2, 8>(x, wq, sc, M, N, K, y, st, bt);
    if (blocks(8, 1) >= want) return fp_qmv_r<T, BITS, GS, 1, 8>(x, wq, sc, M, N, K, y, st, bt);
    return fp_qmv_r<T, BITS, GS, 1, 4>(x, wq, sc, M, N, K, y, st, bt);   // the most workgroups
  }
}

// mode dispatch: (4, 32) mxfp4, (4, 16) nvfp4, (8, 32) mxfp8
#define FP_DISPATCH(T, FN, ...)                                   \
  (bits == 4 ? (gs == 32 ? FN<T, 4, 32>(__VA_ARGS__)              \
                         : FN<T, 4, 16>(__VA_ARGS__))             \
             : FN<T, 8, 32>(__VA_ARGS__))

}  // namespace

hipError_t launch_fp_quantize(int dt, int bits, int gs, const void* w, int64_t rows, int64_t K,
                              uint32_t* wq, uint8_t* scales, hipStream_t st) {
  if (dt == 0) return FP_DISPATCH(F16, fp_quantize_t, w, rows, K, wq, scales, st);
  if (dt == 1) return FP_DISPATCH(BF16, fp_quantize_t, w, rows, K, wq, scales, st);
  return FP_DISPATCH(F32, fp_quantize_t, w, rows, K, wq, scales, st);
}

hipError_t launch_fp_dequantize(int dt, int bits, int gs, const uint32_t* wq,
                                const uint8_t* scales, int64_t rows, int64_t K, void* out,
                                hipStream_t st) {
  if (dt == 0) return FP_DISPATCH(F16, fp_dequantize_t, wq, scales, rows, K, out, st);
  if (dt == 1) return FP_DISPATCH(BF16, fp_dequantize_t, wq, scales, rows, K, out, st);
  return FP_DISPATCH(F32, fp_dequantize_t, wq, scales, rows, K, out, st);
}

hipError_t launch_fp_qmv(int dt, int bits, int gs, const void* x, const uint32_t* wq,
                         const uint8_t* scales, int64_t M, int64_t N, int64_t K, void* y,
                         hipStream_t st) {
  const FpBatch* none = nullptr;
  if (dt == 0) return FP_DISPATCH(F16, fp_qmv_t, x, wq, scales, M, N, K, y, st, none);
  return FP_DISPATCH(BF16, fp_qmv_t, x, wq, scales, M, N, K, y, st, none);
}

hipError_t launch_fp_gather_qmv(int dt, int bits, int gs, const void* x, int64_t nxb,
                                const int32_t* lidx, const uint32_t* wq, const uint8_t* scales,
                                int64_t nwb, const int32_t* ridx, int64_t B, int64_t M, int64_t N,
                                int64_t K, void* y, hipStream_t st) {
  const FpBatch bt{lidx, ridx, (int)nxb, (int)nwb, (int)M, (int)B};
  const FpBatch* p = &bt;
  if (dt == 0) return FP_DISPATCH(F16, fp_qmv_t, x, wq, scales, M, N, K, y, st, p);
  return FP_DISPATCH(BF16, fp_qmv_t, x, wq, scales, M, N, K, y, st, p);
}

}  // namespace qmm
