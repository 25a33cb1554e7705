// Device helpers shared by the libqmm kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

// ----------------------------------------------------------------- types
// Element types are carried as raw storage words (uint16_t for f16/bf16,
// float for f32) so that every conversion is explicit.

struct F16 {
  using word = uint16_t;
  static constexpr uint32_t kMagic = 0x64006400u;  // half2(1024, 1024)
  static constexpr float kMagicF = 1024.0f;
};
struct BF16 {
  using word = uint16_t;
  static constexpr uint32_t kMagic = 0x43004300u;  // bf16x2(128, 128)
  static constexpr float kMagicF = 128.0f;
};
struct F32 {
  using word = float;
};

__device__ __forceinline__ float to_f32(F16, uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}
__device__ __forceinline__ float to_f32(BF16, uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}
__device__ __forceinline__ float to_f32(F32, float f) { return f; }

// fp32 -> f16 with the hardware conversion (round to nearest even under the
// default rounding mode).
__device__ __forceinline__ uint16_t from_f32(F16, float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
// fp32 -> bf16 with the hardware conversion (v_cvt_pk_bf16_f32: round to
// nearest even under the default rounding mode; NaN stays a NaN).
__device__ __forceinline__ uint16_t from_f32(BF16, float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ float from_f32(F32, float f) { return f; }

// ----------------------------------------------------------------- packing
// A row of K codes is a little-endian bit stream, code k at bit k*bits.
// Codes are handled in chunks of 32 consecutive codes (4*bits bytes), which
// always lie inside one quantization group (group sizes are multiples of 32).

template <int BITS>
struct Pack {
  static constexpr bool kPow2 = (BITS & (BITS - 1)) == 0;
  // codes per pack and bytes per pack: a 32-bit word for power-of-two
  // widths; 8 codes in 3 bytes (3-bit), 8 in 5 bytes (5-bit), 4 in 3 bytes
  // (6-bit)
  static constexpr int kVals = kPow2 ? 32 / BITS : (BITS == 6 ? 4 : 8);
  static constexpr int kBytes = kPow2 ? 4 : (BITS == 5 ? 5 : 3);
  static constexpr int kChunkBytes = 4 * BITS;  // 32 codes
  static constexpr int kChunkWords = BITS;
  static constexpr uint32_t kMask = (1u << BITS) - 1u;
};

// Two bytes of a chunk starting at compile-time byte offset o, in the low 16
// bits of the result (upper bits unspecified).
template <int O>
__device__ __forceinline__ uint32_t bytes2_at(const uint32_t* w) {
  constexpr int i = O / 4, s = O % 4;
  if constexpr (s <= 2) {
    return w[i] >> (8 * s);
  } else {
    return __builtin_amdgcn_alignbit(w[i + 1], w[i], 24);
  }
}

// Code j of a chunk held in 32-bit words (reference unpack, any width).
template <int BITS, int J>
__device__ __forceinline__ uint32_t code_at(const uint32_t* w) {
  constexpr int bit = J * BITS, i = bit / 32, off = bit % 32;
  if constexpr (off + BITS <= 32) {
    return (w[i] >> off) & Pack<BITS>::kMask;
  } else {
    return __builtin_amdgcn_alignbit(w[i + 1], w[i], off) & Pack<BITS>::kMask;
  }
}

// ------------------------------------------------------------ pair layout
// The streaming kernels turn codes into 16-bit float pairs with the
// "magic number" trick: a code field q*2^o (q < 2^BITS) OR-ed into the
// mantissa of MAGIC = 1024.0 (f16) or 128.0 (bf16) is exactly the float
// MAGIC + q*2^o, provided q*2^o fits the mantissa (10 bits for f16, 7 for
// bf16). Two codes go into one 32-bit register as (low half, high half).
// The streaming GEMV multiplies them with a pair of unscaled activations
// (v_dot2, fp32 sums kept apart per offset o) and scales each sum by 2^-o in
// fp32, which is exact; each product is then x*q plus an offset x*MAGIC*2^-o
// that depends on x only (removed through a per-chunk constant). The matrix
// kernels map MAGIC + q*2^o back to q with the same exact power-of-two factor.
// A field at in-half offset o <= max_off needs no shift; for f16 the offset
// is capped at 4.
// The order in which codes land in pairs depends on the width:
//  * power-of-two widths: inside each 32-bit word, field f of the low half
//    pairs with field f of the high half, i.e. code (word*V + f) with code
//    (word*V + f + V/2), V = codes per word;
//  * 3/5/6 bits: code j of pack 2r pairs with code j of pack 2r+1, both read
//    from two-byte windows at the same offset inside their packs.
// pair_index(k) / pair_half(k) / pair_off(k) give, for code k of a chunk
// (0..31), its pair (0..15), its half (0 low, 1 high) and its offset o.

template <class T> struct Mant;
template <> struct Mant<F16> { static constexpr int bits = 10, cap = 4; };
template <> struct Mant<BF16> { static constexpr int bits = 7, cap = 7; };

template <class T, int BITS>
__host__ __device__ constexpr int max_off() {
  const int m = Mant<T>::bits - BITS;
  return m < Mant<T>::cap ? m : Mant<T>::cap;
}

// power-of-two widths: right shift applied to the word for field f, and the
// field's remaining offset
template <class T, int BITS>
__host__ __device__ constexpr int pow2_shift(int f) {
  const int step = (max_off<T, BITS>() / BITS + 1) * BITS;
  return (BITS * f / step) * step;
}

template <int BITS>
__host__ __device__ constexpr int pair_index(int k) {
  if constexpr (Pack<BITS>::kPow2) {
    constexpr int V = Pack<BITS>::kVals, H = V / 2;
    return (k / V) * H + (k % V) % H;
  } else {
    constexpr int V = Pack<BITS>::kVals;
    return ((k / V) / 2) * V + k % V;
  }
}
template <int BITS>
__host__ __device__ constexpr int pair_half(int k) {
  if constexpr (Pack<BITS>::kPow2) {
    constexpr int V = Pack<BITS>::kVals, H = V / 2;
    return (k % V) / H;
  } else {
    constexpr int V = Pack<BITS>::kVals;
    return (k / V) % 2;
  }
}

// code of the low half of pair p (pair_index(pair_code(p)) == p)
template <int BITS>
__host__ __device__ constexpr int pair_code(int p) {
  if constexpr (Pack<BITS>::kPow2) {
    constexpr int V = Pack<BITS>::kVals, H = V / 2;
    return (p / H) * V + p % H;
  } else {
    constexpr int V = Pack<BITS>::kVals;
    return (p / V) * 2 * V + p % V;
  }
}

// window geometry of code j of a non-power-of-two pack
template <int BITS>
__host__ __device__ constexpr int win_start(int j) {
  constexpr int NB = Pack<BITS>::kBytes;
  return (j * BITS / 8) < (NB - 2) ? (j * BITS / 8) : (NB - 2);
}
template <int BITS>
__host__ __device__ constexpr int win_off(int j) {
  return j * BITS - 8 * win_start<BITS>(j);
}

// offset o of code k's field when it meets the magic number
template <class T, int BITS>
__host__ __device__ constexpr int pair_off(int k) {
  if constexpr (Pack<BITS>::kPow2) {
    constexpr int H = Pack<BITS>::kVals / 2;
    const int f = (k % Pack<BITS>::kVals) % H;
    return BITS * f - pow2_shift<T, BITS>(f);
  } else {
    const int off = win_off<BITS>(k % Pack<BITS>::kVals);
    return off <= max_off<T, BITS>() ? off : 0;
  }
}

// Offset classes: the distinct offsets o of a chunk's 16 pairs (at most 4;
// offset 0 is always present and is class 0). The streaming GEMV sums the
// products of each class apart and scales the sums by 2^-o in fp32.
template <class T, int BITS>
__host__ __device__ constexpr unsigned off_set() {
  unsigned m = 0;
  for (int p = 0; p < 16; p++) m |= 1u << pair_off<T, BITS>(pair_code<BITS>(p));
  return m;
}
template <class T, int BITS>
__host__ __device__ constexpr int n_off_classes() {
  int n = 0;
  for (int o = 0; o < 8; o++) n += (off_set<T, BITS>() >> o) & 1u;
  return n;
}
// class of pair p: rank of its offset among the offsets present
template <class T, int BITS>
__host__ __device__ constexpr int off_class(int p) {
  const int o = pair_off<T, BITS>(pair_code<BITS>(p));
  int c = 0;
  for (int i = 0; i < o; i++) c += (off_set<T, BITS>() >> i) & 1u;
  return c;
}
// offset of class c
template <class T, int BITS>
__host__ __device__ constexpr int class_off(int c) {
  for (int o = 0; o < 8; o++)
    if ((off_set<T, BITS>() >> o) & 1u) {
      if (c == 0) return o;
      c--;
    }
  return 0;
}
// position of pair p among the pairs of its class (pairs in index order)
template <class T, int BITS>
__host__ __device__ constexpr int rank_in_class(int p) {
  int r = 0;
  for (int q = 0; q < p; q++) r += off_class<T, BITS>(q) == off_class<T, BITS>(p);
  return r;
}

// Pair P (0..15) of a chunk as two magic floats (see above). m2 must hold
// kMask | kMask << 16 and magic the 32-bit magic pattern; both are passed in
// registers so that mask + or fuse into one v_and_or_b32.
template <class T, int BITS, int P>
__device__ __forceinline__ uint32_t magic_pair(const uint32_t* w, uint32_t m2,
                                               uint32_t magic) {
  if constexpr (Pack<BITS>::kPow2) {
    constexpr int H = Pack<BITS>::kVals / 2;
    constexpr int word = P / H, f = P % H;
    constexpr int sh = pow2_shift<T, BITS>(f);
    constexpr int o = BITS * f - sh;
    const uint32_t v = sh ? (w[word] >> sh) : w[word];
    return (v & (m2 << o)) | magic;
  } else {
    constexpr int V = Pack<BITS>::kVals, NB = Pack<BITS>::kBytes;
    constexpr int r = P / V, j = P % V;
    constexpr int ws = win_start<BITS>(j), off = win_off<BITS>(j);
    static_assert(off + BITS <= 16, "field must fit a two-byte window");
    const uint32_t lo = bytes2_at<(2 * r) * NB + ws>(w);
    const uint32_t hi = bytes2_at<(2 * r + 1) * NB + ws>(w);
    const uint32_t pr = (lo & 0xffffu) | (hi << 16);
    constexpr int o = pair_off<T, BITS>(j);
    constexpr int sh = off - o;
    const uint32_t v = sh ? (pr >> sh) : pr;
    return (v & (m2 << o)) | magic;
  }
}

// -------------------------------------------------------- dot products
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(F16, uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a),
                                __builtin_bit_cast(half2_t, b), c, false);
}
__device__ __forceinline__ float dot2(BF16, uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a),
                                         __builtin_bit_cast(bf162_t, b), c,
                                         false);
}

// ------------------------------------------------------------ misc
__host__ __device__ constexpr int ilog2(int v) {
  return v <= 1 ? 0 : 1 + ilog2(v / 2);
}

}  // namespace qmm
