// Device helpers shared by the MFMA kernels: operand types, MFMA wrappers
// and the dequantization of chunk pieces into MFMA B fragments.
#pragma once
#include <utility>

#include "common.hpp"

namespace qmm {

// the kernels are written with many small lambdas; all of them must be
// inlined (an outlined step would move the accumulators to scratch memory)
#define QMM_INLINE __attribute__((always_inline))

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Buffer resource over [base, base + bytes): raw (stride 0) 32-bit words;
// loads at offsets past `bytes` return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
// Offset that is out of range for every resource here (their sizes stay
// below 2^31): the load returns zeros.
constexpr uint32_t kOob = 0x80000000u;

// v_mfma_f32_32x32x16: A[i][k] from lane i%32 + 32*(k/8) (element k%8), B[k][j]
// from lane j + 32*(k/8), D[i][j] in lane j + 32*((i/4)%2), element
// 4*(i/8) + i%4. One wavefront sustains close to the matrix-core peak with
// four independent 32x32 accumulators (measured), unlike the 16x16x32 form.
__device__ __forceinline__ float16_t mfma32(F16, const uint4& a, const uint4& b,
                                            float16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(
      __builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ float16_t mfma32(BF16, const uint4& a, const uint4& b,
                                            float16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
      __builtin_bit_cast(bf8_t, a), __builtin_bit_cast(bf8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float4_t mfma16(F16, const uint4& a, const uint4& b,
                                           float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(
      __builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ float4_t mfma16(BF16, const uint4& a, const uint4& b,
                                           float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf8_t, a), __builtin_bit_cast(bf8_t, b), c, 0, 0, 0);
}

// ------------------------------------------------------------ dequant pieces
// A piece is a run of consecutive codes of a 32-code chunk whose magic pairs
// (see common.hpp) all lie inside the run: 8 codes for 4/6/8 bits, 16 for
// 2/3/5 bits. Pieces let the tile kernel spread the dequantization of the
// next K step between the MFMAs of the current one.
template <int BITS>
constexpr int piece_codes() {
  return (BITS == 2 || BITS == 3 || BITS == 5) ? 16 : 8;
}

template <int BITS, int C0, int PC>
constexpr bool piece_has_pair(int P) {
  for (int k = C0; k < C0 + PC; k++)
    if (pair_index<BITS>(k) == P) return true;
  return false;
}

// field offset o of magic pair P (both codes of a pair share it)
template <int BITS>
constexpr int pair_o(int P) {
  for (int k = 0; k < 32; k++)
    if (pair_index<BITS>(k) == P) return pair_off<F16, BITS>(k);
  return 0;
}
// byte selector of v_perm_b32(hi_src, lo_src, sel) that takes 16-bit half hl
// of lo_src into the low half and half hh of hi_src into the high half
constexpr uint32_t half_sel(int hl, int hh) {
  return (uint32_t)(2 * hl) | ((uint32_t)(2 * hl + 1) << 8) | ((uint32_t)(4 + 2 * hh) << 16) |
         ((uint32_t)(4 + 2 * hh + 1) << 24);
}

// codes [C0, C0+PC) of a chunk -> f16 pairs out[C0/2 .. (C0+PC)/2) with
// packed f16 arithmetic (cheap next to the MFMAs): magic pair (1024 + q*2^o)
// -> q exactly (times 2^-o, minus 1024*2^-o: both exact), then w = s*q + b
// rounded once (v_pk_fma_f16), then v_perm into natural code order. s2 and b2
// hold the scale and the bias in both halves.
template <int BITS, int C0, int PC>
__device__ __forceinline__ void dequant_piece_f16_pk(const uint32_t* w, uint32_t s2, uint32_t b2,
                                                     uint32_t m2, uint32_t magic,
                                                     uint32_t* out) {
  uint32_t pr[16];
  [&]<int... P>(std::integer_sequence<int, P...>) QMM_INLINE {
    ([&]() QMM_INLINE {
       if constexpr (piece_has_pair<BITS, C0, PC>(P)) {
         constexpr int o = pair_o<BITS>(P);
         constexpr uint16_t e = (uint16_t)((15 - o) << 10);              // 2^-o
         constexpr uint16_t f = (uint16_t)(0x8000 | ((25 - o) << 10));  // -1024 * 2^-o
         const half2_t mp = __builtin_bit_cast(half2_t, magic_pair<F16, BITS, P>(w, m2, magic));
         const half2_t q = __builtin_elementwise_fma(
             mp, __builtin_bit_cast(half2_t, (uint32_t)e * 0x10001u),
             __builtin_bit_cast(half2_t, (uint32_t)f * 0x10001u));
         pr[P] = __builtin_bit_cast(
             uint32_t, __builtin_elementwise_fma(q, __builtin_bit_cast(half2_t, s2),
                                                 __builtin_bit_cast(half2_t, b2)));
       } else {
         pr[P] = 0;
       }
     }(),
     ...);
  }(std::make_integer_sequence<int, 16>{});
  [&]<int... J>(std::integer_sequence<int, J...>) QMM_INLINE {
    ([&]() QMM_INLINE {
       constexpr int k = C0 + 2 * J;
       constexpr int pl = pair_index<BITS>(k), hl = pair_half<BITS>(k);
       constexpr int ph = pair_index<BITS>(k + 1), hh = pair_half<BITS>(k + 1);
       out[k / 2] = __builtin_amdgcn_perm(pr[ph], pr[pl], half_sel(hl, hh));
     }(),
     ...);
  }(std::make_integer_sequence<int, PC / 2>{});
}

// codes [C0, C0+8) of a chunk -> bf16 hi/lo pairs: w = fl32(s*q + b) (s*q is
// exact), hi = bf16(w), lo = bf16(w - hi), both rounded to nearest even by
// the packed hardware conversion (v_cvt_pk_bf16_f32, two values at a time)
template <int BITS, int C0>
__device__ __forceinline__ void dequant_piece_bf16(const uint32_t* w, float s, float b,
                                                   uint32_t* hi, uint32_t* lo) {
  [&]<int... J>(std::integer_sequence<int, J...>) QMM_INLINE {
    float f[8] = {fmaf(s, (float)code_at<BITS, C0 + J>(w), b)...};
#pragma unroll
    for (int k = 0; k < 8; k += 2) {
      const bf162_t h = {(__bf16)f[k], (__bf16)f[k + 1]};
      const uint32_t hu = __builtin_bit_cast(uint32_t, h);
      hi[(C0 + k) / 2] = hu;
      const float r0 = f[k] - __builtin_bit_cast(float, hu << 16);
      const float r1 = f[k + 1] - __builtin_bit_cast(float, hu & 0xffff0000u);
      const bf162_t l = {(__bf16)r0, (__bf16)r1};
      lo[(C0 + k) / 2] = __builtin_bit_cast(uint32_t, l);
    }
  }(std::make_integer_sequence<int, 8>{});
}

// ------------------------------------------------------------ fp-mode pieces
// Floating-point modes of the tile kernel: 1 mxfp4 (E2M1 codes, e8m0 scale
// per 32), 2 nvfp4 (E2M1, E4M3 scale per 16), 3 mxfp8 (E4M3 codes, e8m0 per
// 32). Codes are OCP E2M1 (two per byte, the first in the low nibble) or
// E4M3 (one per byte).

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// The group scale as the product uses it, rounded to T ("mlx 1.0.0
// backend/cpu/quantized.cpp", dequantize_scale<T>), as fp32 bits. e8m0 byte
// s is 2^(s-127) (byte 0 the fp32 subnormal 2^-127); f16 holds 2^-24 ..
// 2^15 of those, rounds smaller ones to 0 (2^-25 ties to even) and larger
// ones to infinity; bf16 holds them all. E4M3 values are exact in f16 and
// bf16.
template <class T, int FPM>
__device__ __forceinline__ uint32_t fp_scale_t_bits(uint32_t s) {
  if constexpr (FPM == 2) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_f32_fp8(s, 1.0f, 0));
  } else {
    if constexpr (__is_same(T, F16)) {
      if (s < 103u) return 0u;
      if (s > 142u) return 0x7f800000u;
    }
    return s == 0u ? 0x00400000u : (s << 23);
  }
}

// Eight codes (one word of E2M1 codes or two of E4M3) times the scale sc,
// as four T pairs in code order. With an e8m0 scale the scaled conversion
// applies the power of two exactly (the hardware takes only the scale's
// exponent, which is all an e8m0 value has); with an E4M3 scale the codes
// are converted at scale 1 and each multiplied by sc in fp32 (exact: at most
// 2 + 4 significant bits) before the rounding to T.
template <class T, int FPM>
__device__ __forceinline__ void fp_piece(const uint32_t* w, float sc, uint32_t* out) {
  constexpr bool kF16 = __is_same(T, F16);
  if constexpr (FPM == 3) {
    if constexpr (kF16) {
      out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[0], sc, false));
      out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[0], sc, true));
      out[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[1], sc, false));
      out[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[1], sc, true));
    } else {
      out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], sc, false));
      out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], sc, true));
      out[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], sc, false));
      out[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], sc, true));
    }
  } else if constexpr (FPM == 1) {
    if constexpr (kF16) {
      out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[0], sc, 0));
      out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[0], sc, 1));
      out[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[0], sc, 2));
      out[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[0], sc, 3));
    } else {
      out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[0], sc, 0));
      out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[0], sc, 1));
      out[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[0], sc, 2));
      out[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[0], sc, 3));
    }
  } else {
    f32x2_t v[4];
    v[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[0], 1.0f, 0);
    v[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[0], 1.0f, 1);
    v[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[0], 1.0f, 2);
    v[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[0], 1.0f, 3);
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const float a0 = v[q].x * sc, a1 = v[q].y * sc;
      if constexpr (kF16) {
        const half2_t hv = {(_Float16)a0, (_Float16)a1};
        out[q] = __builtin_bit_cast(uint32_t, hv);
      } else {
        const bf162_t bv = {(__bf16)a0, (__bf16)a1};
        out[q] = __builtin_bit_cast(uint32_t, bv);
      }
    }
  }
}

}  // namespace qmm
