// Quantize and dequantize kernels.
//
// Quantizer rule: "Improvements in the quantizer and dequantization kernel"
// (mlx PR 1061) item 1 a-c; per-group steps and packing as in "mlx 1.0.0
// backend/cpu/quantized.cpp", function quantize. Every step is IEEE fp32
// (correctly rounded division, ties-to-even rint), so the codes, scales and
// biases are bit-identical to any other IEEE implementation of the steps.
//
// Work split: one group of GS elements is handled by GS/8 consecutive lanes,
// each owning 8 consecutive elements. The 8 codes of a lane are 8*BITS bits,
// i.e. exactly BITS whole bytes of the packed row, so lanes never share a
// byte.
#include "common.hpp"
#include "kernels.hpp"

namespace qmm {

template <class T>
__device__ __forceinline__ void load8(const typename T::word* p, float v[8]);

template <>
__device__ __forceinline__ void load8<F16>(const uint16_t* p, float v[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    v[2 * i] = to_f32(F16{}, (uint16_t)(w[i] & 0xffffu));
    v[2 * i + 1] = to_f32(F16{}, (uint16_t)(w[i] >> 16));
  }
}
template <>
__device__ __forceinline__ void load8<BF16>(const uint16_t* p, float v[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    v[2 * i] = __builtin_bit_cast(float, w[i] << 16);
    v[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void load8<F32>(const float* p, float v[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Store the BITS bytes of a lane's 8 packed codes at byte offset off.
template <int BITS>
__device__ __forceinline__ void store_codes(uint8_t* base, int64_t off,
                                            uint64_t v) {
  uint8_t* p = base + off;
  if constexpr (BITS == 2) {
    *reinterpret_cast<uint16_t*>(p) = (uint16_t)v;
  } else if constexpr (BITS == 4) {
    *reinterpret_cast<uint32_t*>(p) = (uint32_t)v;
  } else if constexpr (BITS == 8) {
    *reinterpret_cast<uint64_t*>(p) = v;
  } else if constexpr (BITS == 6) {
#pragma unroll
    for (int i = 0; i < 3; i++)
      reinterpret_cast<uint16_t*>(p)[i] = (uint16_t)(v >> (16 * i));
  } else {
#pragma unroll
    for (int i = 0; i < BITS; i++) p[i] = (uint8_t)(v >> (8 * i));
  }
}

template <int BITS>
__device__ __forceinline__ uint64_t load_codes(const uint8_t* base,
                                               int64_t off) {
  const uint8_t* p = base + off;
  if constexpr (BITS == 2) {
    return *reinterpret_cast<const uint16_t*>(p);
  } else if constexpr (BITS == 4) {
    return *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (BITS == 8) {
    return *reinterpret_cast<const uint64_t*>(p);
  } else if constexpr (BITS == 6) {
    uint64_t v = 0;
#pragma unroll
    for (int i = 0; i < 3; i++)
      v |= (uint64_t)reinterpret_cast<const uint16_t*>(p)[i] << (16 * i);
    return v;
  } else {
    uint64_t v = 0;
#pragma unroll
    for (int i = 0; i < BITS; i++) v |= (uint64_t)p[i] << (8 * i);
    return v;
  }
}

template <class T, int BITS, int GS>
__global__ __launch_bounds__(256) void quantize_kernel(
    const typename T::word* __restrict__ w, int64_t n_groups,
    uint8_t* __restrict__ wq, typename T::word* __restrict__ scales,
    typename T::word* __restrict__ biases) {
  constexpr int L = GS / 8;  // lanes per group
  const int64_t lane_g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t g = lane_g / L;
  const int j = (int)(lane_g % L);
  const bool valid = g < n_groups;

  float v[8];
  if (valid) {
    load8<T>(w + g * GS + j * 8, v);
  } else {
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = 0.0f;
  }
  float w_min = v[0], w_max = v[0];
#pragma unroll
  for (int i = 1; i < 8; i++) {
    w_min = fminf(w_min, v[i]);
    w_max = fmaxf(w_max, v[i]);
  }
#pragma unroll
  for (int o = L / 2; o >= 1; o >>= 1) {
    w_min = fminf(w_min, __shfl_xor(w_min, o));
    w_max = fmaxf(w_max, __shfl_xor(w_max, o));
  }

  const float n_bins = (float)((1 << BITS) - 1);
  const float eps = 1e-7f;
  // (a) bias candidate: the extreme of larger magnitude (max on a tie);
  // (b) scale from that extreme towards the other one
  const bool bias_is_min = fabsf(w_min) > fabsf(w_max);
  float scale = (w_max - w_min) / n_bins;
  scale = scale < eps ? eps : scale;
  scale = bias_is_min ? scale : -scale;
  // (c) put zero on the grid: the edge must be a whole number of steps away
  const float edge = bias_is_min ? w_min : w_max;
  const float q0 = __builtin_rintf(edge / scale);
  float bias = 0.0f;
  if (q0 != 0.0f) {
    scale = edge / q0;
    bias = edge;
  }

  // Codes rint((w - bias) / scale) with the correctly rounded quotient, at
  // the cost of a multiplication: t = d * fl(1/scale) lies within 3 * 2^-24
  // * |t| of the rounded quotient fl(d / scale), so both round to the same
  // integer unless t is that close to the half-integer between its floor and
  // ceiling (ties included); there the quotient itself is computed (a branch
  // a wavefront takes only when one of its lanes is that close; the margin
  // used is 16 times the bound).
  const float rscale = 1.0f / scale;
  float d[8], t[8];
  unsigned fix = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    d[i] = v[i] - bias;
    t[i] = d[i] * rscale;
    if (fabsf(t[i] - (floorf(t[i]) + 0.5f)) <= 0x1p-20f * fabsf(t[i])) fix |= 1u << i;
  }
  // a branch on the whole wavefront, so that the divisions are not computed
  // speculatively for every element
  if (__builtin_amdgcn_ballot_w64(fix != 0) != 0) {
#pragma unroll
    for (int i = 0; i < 8; i++)
      if ((fix >> i) & 1u) t[i] = d[i] / scale;
  }
  uint64_t packed = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    float q = __builtin_rintf(t[i]);
    q = q < 0.0f ? 0.0f : q;
    q = q > n_bins ? n_bins : q;
    packed |= (uint64_t)(uint32_t)q << (i * BITS);
  }
  if (valid) {
    store_codes<BITS>(wq, g * (GS * BITS / 8) + (int64_t)j * BITS, packed);
    if (j == 0) {
      scales[g] = from_f32(T{}, scale);
      biases[g] = from_f32(T{}, bias);
    }
  }
}

template <class T, int BITS, int GS>
__global__ __launch_bounds__(256) void dequantize_kernel(
    const uint8_t* __restrict__ wq, const typename T::word* __restrict__ scales,
    const typename T::word* __restrict__ biases, int64_t n8,
    typename T::word* __restrict__ out) {
  // scale * code and + bias are two separately rounded operations: HIP
  // contracts mul + add into an FMA by default, which differs for f32 scales
#pragma clang fp contract(off)
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n8) return;
  const int64_t e = t * 8;  // first element; 8 elements never cross a group
  const int64_t g = e / GS;
  const float s = to_f32(T{}, scales[g]);
  const float b = to_f32(T{}, biases[g]);
  const uint64_t packed = load_codes<BITS>(wq, t * BITS);
  typename T::word r[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const float q = (float)(uint32_t)((packed >> (i * BITS)) & ((1u << BITS) - 1u));
    r[i] = from_f32(T{}, s * q + b);
  }
  if constexpr (sizeof(typename T::word) == 2) {
    uint4 u;
    u.x = (uint32_t)r[0] | ((uint32_t)r[1] << 16);
    u.y = (uint32_t)r[2] | ((uint32_t)r[3] << 16);
    u.z = (uint32_t)r[4] | ((uint32_t)r[5] << 16);
    u.w = (uint32_t)r[6] | ((uint32_t)r[7] << 16);
    *reinterpret_cast<uint4*>(out + e) = u;
  } else {
    float4* o = reinterpret_cast<float4*>(out + e);
    o[0] = make_float4(r[0], r[1], r[2], r[3]);
    o[1] = make_float4(r[4], r[5], r[6], r[7]);
  }
}

// ----------------------------------------------------------------- launch

template <class T, int BITS, int GS>
static hipError_t launch_quantize_t(const void* w, int64_t rows, int64_t K,
                                    uint32_t* wq, void* s, void* b,
                                    hipStream_t st) {
  const int64_t n_groups = rows * (K / GS);
  const int64_t lanes = n_groups * (GS / 8);
  const int64_t blocks = (lanes + 255) / 256;
  hipLaunchKernelGGL((quantize_kernel<T, BITS, GS>), dim3((unsigned)blocks),
                     dim3(256), 0, st,
                     static_cast<const typename T::word*>(w), n_groups,
                     reinterpret_cast<uint8_t*>(wq),
                     static_cast<typename T::word*>(s),
                     static_cast<typename T::word*>(b));
  return hipGetLastError();
}

template <class T, int BITS, int GS>
static hipError_t launch_dequantize_t(const uint32_t* wq, const void* s,
                                      const void* b, int64_t rows, int64_t K,
                                      void* out, hipStream_t st) {
  const int64_t n8 = rows * K / 8;
  const int64_t blocks = (n8 + 255) / 256;
  hipLaunchKernelGGL((dequantize_kernel<T, BITS, GS>), dim3((unsigned)blocks),
                     dim3(256), 0, st,
                     reinterpret_cast<const uint8_t*>(wq),
                     static_cast<const typename T::word*>(s),
                     static_cast<const typename T::word*>(b), n8,
                     static_cast<typename T::word*>(out));
  return hipGetLastError();
}

template <class T, int BITS>
static hipError_t quant_gs(int gs, const void* w, int64_t rows, int64_t K,
                           uint32_t* wq, void* s, void* b, hipStream_t st) {
  switch (gs) {
    case 32: return launch_quantize_t<T, BITS, 32>(w, rows, K, wq, s, b, st);
    case 64: return launch_quantize_t<T, BITS, 64>(w, rows, K, wq, s, b, st);
    default: return launch_quantize_t<T, BITS, 128>(w, rows, K, wq, s, b, st);
  }
}

template <class T, int BITS>
static hipError_t dequant_gs(int gs, const uint32_t* wq, const void* s,
                             const void* b, int64_t rows, int64_t K, void* out,
                             hipStream_t st) {
  switch (gs) {
    case 32: return launch_dequantize_t<T, BITS, 32>(wq, s, b, rows, K, out, st);
    case 64: return launch_dequantize_t<T, BITS, 64>(wq, s, b, rows, K, out, st);
    default: return launch_dequantize_t<T, BITS, 128>(wq, s, b, rows, K, out, st);
  }
}

template <class T>
static hipError_t quant_bits(int bits, int gs, const void* w, int64_t rows,
                             int64_t K, uint32_t* wq, void* s, void* b,
                             hipStream_t st) {
  switch (bits) {
    case 2: return quant_gs<T, 2>(gs, w, rows, K, wq, s, b, st);
    case 3: return quant_gs<T, 3>(gs, w, rows, K, wq, s, b, st);
    case 4: return quant_gs<T, 4>(gs, w, rows, K, wq, s, b, st);
    case 5: return quant_gs<T, 5>(gs, w, rows, K, wq, s, b, st);
    case 6: return quant_gs<T, 6>(gs, w, rows, K, wq, s, b, st);
    default: return quant_gs<T, 8>(gs, w, rows, K, wq, s, b, st);
  }
}

template <class T>
static hipError_t dequant_bits(int bits, int gs, const uint32_t* wq,
                               const void* s, const void* b, int64_t rows,
                               int64_t K, void* out, hipStream_t st) {
  switch (bits) {
    case 2: return dequant_gs<T, 2>(gs, wq, s, b, rows, K, out, st);
    case 3: return dequant_gs<T, 3>(gs, wq, s, b, rows, K, out, st);
    case 4: return dequant_gs<T, 4>(gs, wq, s, b, rows, K, out, st);
    case 5: return dequant_gs<T, 5>(gs, wq, s, b, rows, K, out, st);
    case 6: return dequant_gs<T, 6>(gs, wq, s, b, rows, K, out, st);
    default: return dequant_gs<T, 8>(gs, wq, s, b, rows, K, out, st);
  }
}

hipError_t launch_quantize(int dt, int bits, int gs, const void* w,
                           int64_t rows, int64_t K, uint32_t* wq, void* s,
                           void* b, hipStream_t st) {
  if (dt == 0) return quant_bits<F16>(bits, gs, w, rows, K, wq, s, b, st);
  if (dt == 1) return quant_bits<BF16>(bits, gs, w, rows, K, wq, s, b, st);
  return quant_bits<F32>(bits, gs, w, rows, K, wq, s, b, st);
}

hipError_t launch_dequantize(int dt, int bits, int gs, const uint32_t* wq,
                             const void* s, const void* b, int64_t rows,
                             int64_t K, void* out, hipStream_t st) {
  if (dt == 0) return dequant_bits<F16>(bits, gs, wq, s, b, rows, K, out, st);
  if (dt == 1) return dequant_bits<BF16>(bits, gs, wq, s, b, rows, K, out, st);
  return dequant_bits<F32>(bits, gs, wq, s, b, rows, K, out, st);
}

}  // namespace qmm
