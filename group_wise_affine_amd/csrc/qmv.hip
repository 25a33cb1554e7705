// Streaming quantized GEMV for small M (decode):
//   y[m, n] = sum_g ( s[n,g] * sum_{k in g} x[m,k] q[n,k]
//                   + b[n,g] * sum_{k in g} x[m,k] ),
// the group factorisation of y = x . (s*q + b)^T used by the Metal qmv in
// "Add the 3bit packed qmm_t" (affine_packed_qmv_fast_impl: result += s*accum
// + b*sum) with fp32 accumulation ("everything is float32" in qmv, mlx PR
// 1061 item 2).
//
// MI355X design (wave64):
//  * Each workgroup first stages up to MB rows of x into LDS, already
//    permuted into the pair order the weight unpacker produces (see
//    common.hpp), together with the fp32 sum of every 32-element chunk.
//  * A row of W is split over TPR lanes of one wavefront (64/TPR rows per
//    wavefront); a lane walks the row in 32-code chunks (4*bits bytes,
//    16 bytes at 4 bits) with stride TPR chunks, so a wavefront load covers
//    64/TPR contiguous row segments of TPR*4*bits bytes each.
//  * Codes become exact f16/bf16 values MAGIC + q with one shift and one
//    and-or per pair, and v_dot2_f32_{f16,bf16} multiplies them with the
//    activation pairs in fp32. The MAGIC offset is removed through the chunk
//    sum: s*sum(x*(MAGIC+q)) + (b - MAGIC*s)*sum(x) = sum(x*(s*q + b)).
//  * Every W byte is read once per MB rows of x; one pass serves all of them.
//  * Lanes of a row reduce with cross-lane shuffles; lane 0 writes y.
#include "common.hpp"
#include "kernels.hpp"

namespace qmm {

template <class T, int BITS>
struct QmvCfg {
  // bf16 cannot hold 128 + q exactly for 8-bit codes: that case runs in fp32
  static constexpr bool kF32 = (BITS == 8) && __is_same(T, BF16);
  static constexpr int kXWords = kF32 ? 32 : 16;  // LDS words per x chunk
};

template <int BITS>
__device__ __forceinline__ void load_chunk(const uint8_t* p, uint32_t w[BITS]) {
  if constexpr (BITS == 4) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
  } else if constexpr (BITS == 8) {
    const uint4 u = reinterpret_cast<const uint4*>(p)[0];
    const uint4 v = reinterpret_cast<const uint4*>(p)[1];
    w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
    w[4] = v.x; w[5] = v.y; w[6] = v.z; w[7] = v.w;
  } else if constexpr (BITS == 2) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    w[0] = u.x; w[1] = u.y;
  } else if constexpr (BITS == 6) {
#pragma unroll
    for (int i = 0; i < 3; i++) {
      const uint2 u = reinterpret_cast<const uint2*>(p)[i];
      w[2 * i] = u.x; w[2 * i + 1] = u.y;
    }
  } else {  // 3 and 5 bits: 4-byte aligned chunks
#pragma unroll
    for (int i = 0; i < BITS; i++) w[i] = reinterpret_cast<const uint32_t*>(p)[i];
  }
}

// sum over the chunk of x_pair . (MAGIC + q)_pair
template <class T, int BITS, int P = 0>
__device__ __forceinline__ float chunk_dot_pairs(const uint32_t* pairs,
                                                 const uint32_t* xp, float d) {
  if constexpr (P == 16) {
    return d;
  } else {
    d = dot2(T{}, pairs[P], xp[P], d);
    return chunk_dot_pairs<T, BITS, P + 1>(pairs, xp, d);
  }
}

template <class T, int BITS, int P = 0>
__device__ __forceinline__ void unpack_pairs(const uint32_t* w, uint32_t* pr) {
  if constexpr (P < 16) {
    pr[P] = magic_pair<BITS, P, T::kMagic>(w);
    unpack_pairs<T, BITS, P + 1>(w, pr);
  }
}

template <class T, int BITS, int MB>
__global__ __launch_bounds__(256) void qmv_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wq,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases,
    uint16_t* __restrict__ y, int M, int N, int K, int gs_log2,
    int tpr_log2) {
  using Cfg = QmvCfg<T, BITS>;
  constexpr int XW = Cfg::kXWords;
  extern __shared__ uint32_t smem[];
  const int nch = K >> 5;
  uint32_t* xs = smem;                                          // [MB][nch][XW]
  float* xsum = reinterpret_cast<float*>(smem + MB * nch * XW);  // [MB][nch]
  const int m0 = blockIdx.y * MB;

  // ---- stage x (permuted into pair order) and per-chunk sums
  for (int i = threadIdx.x; i < MB * nch; i += blockDim.x) {
    const int m = i / nch, c = i - m * nch;
    uint32_t px[XW];
    float sum = 0.0f;
    if (m0 + m < M) {
      const uint4* src =
          reinterpret_cast<const uint4*>(x + (int64_t)(m0 + m) * K + c * 32);
      uint32_t raw[16];
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const uint4 u = src[q];
        raw[4 * q] = u.x; raw[4 * q + 1] = u.y;
        raw[4 * q + 2] = u.z; raw[4 * q + 3] = u.w;
      }
      if constexpr (Cfg::kF32) {
#pragma unroll
        for (int k = 0; k < 32; k++) {
          const float f = to_f32(T{}, (uint16_t)(raw[k / 2] >> (16 * (k % 2))));
          px[k] = __builtin_bit_cast(uint32_t, f);
          sum += f;
        }
      } else {
#pragma unroll
        for (int p = 0; p < 16; p++) px[p] = 0;
#pragma unroll
        for (int k = 0; k < 32; k++) {
          const uint32_t h = (raw[k / 2] >> (16 * (k % 2))) & 0xffffu;
          px[pair_index<BITS>(k)] |= h << (16 * pair_half<BITS>(k));
          sum += to_f32(T{}, (uint16_t)h);
        }
      }
    } else {
#pragma unroll
      for (int p = 0; p < XW; p++) px[p] = 0;
    }
    uint4* dst = reinterpret_cast<uint4*>(xs + (int64_t)i * XW);
#pragma unroll
    for (int q = 0; q < XW / 4; q++)
      dst[q] = make_uint4(px[4 * q], px[4 * q + 1], px[4 * q + 2], px[4 * q + 3]);
    xsum[i] = sum;
  }
  __syncthreads();

  // ---- stream W
  const int tpr = 1 << tpr_log2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = lane >> tpr_log2, t = lane & (tpr - 1);
  const int row = (blockIdx.x * (blockDim.x >> 6) + wave) * (64 >> tpr_log2) + slot;
  const bool active = row < N;
  float acc[MB];
#pragma unroll
  for (int m = 0; m < MB; m++) acc[m] = 0.0f;

  if (active) {
    const int64_t row_bytes = (int64_t)K * BITS / 8;
    const uint8_t* wrow = wq + (int64_t)row * row_bytes;
    const uint16_t* srow = scales + (int64_t)row * (K >> gs_log2);
    const uint16_t* brow = biases + (int64_t)row * (K >> gs_log2);
    constexpr int U = 4;  // chunks in flight per lane
    for (int c0 = t; c0 < nch; c0 += U * tpr) {
      uint32_t wv[U][BITS];
      float sv[U], bv[U];
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int c = c0 + u * tpr;
        if (c < nch) {
          load_chunk<BITS>(wrow + (int64_t)c * (4 * BITS), wv[u]);
          const int g = (c << 5) >> gs_log2;
          sv[u] = to_f32(T{}, srow[g]);
          bv[u] = to_f32(T{}, brow[g]);
        }
      }
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int c = c0 + u * tpr;
        if (c < nch) {
          const float s = sv[u];
          if constexpr (Cfg::kF32) {
            float fq[32];
#pragma unroll
            for (int i = 0; i < 8; i++) {
              fq[4 * i + 0] = (float)((wv[u][i] >> 0) & 0xffu);
              fq[4 * i + 1] = (float)((wv[u][i] >> 8) & 0xffu);
              fq[4 * i + 2] = (float)((wv[u][i] >> 16) & 0xffu);
              fq[4 * i + 3] = (float)((wv[u][i] >> 24) & 0xffu);
            }
#pragma unroll
            for (int m = 0; m < MB; m++) {
              const float* xp = reinterpret_cast<const float*>(xs + (int64_t)(m * nch + c) * XW);
              float d = 0.0f;
#pragma unroll
              for (int k = 0; k < 32; k++) d = fmaf(xp[k], fq[k], d);
              acc[m] = fmaf(s, d, fmaf(bv[u], xsum[m * nch + c], acc[m]));
            }
          } else {
            const float boff = fmaf(-T::kMagicF, s, bv[u]);
            uint32_t pr[16];
            unpack_pairs<T, BITS>(wv[u], pr);
#pragma unroll
            for (int m = 0; m < MB; m++) {
              const uint32_t* xp = xs + (int64_t)(m * nch + c) * XW;
              const float d = chunk_dot_pairs<T, BITS>(pr, xp, 0.0f);
              acc[m] = fmaf(s, d, fmaf(boff, xsum[m * nch + c], acc[m]));
            }
          }
        }
      }
    }
  }

  // ---- reduce the TPR partial sums of each row
  for (int o = tpr >> 1; o >= 1; o >>= 1) {
#pragma unroll
    for (int m = 0; m < MB; m++) acc[m] += __shfl_xor(acc[m], o);
  }
  if (active && t == 0) {
#pragma unroll
    for (int m = 0; m < MB; m++)
      if (m0 + m < M) y[(int64_t)(m0 + m) * N + row] = from_f32(T{}, acc[m]);
  }
}

// ----------------------------------------------------------------- launch

static constexpr int kMaxLds = 64 * 1024;

template <class T, int BITS, int MB>
static hipError_t launch_mb(const void* x, const uint32_t* wq, const void* s,
                            const void* b, int M, int N, int K, int gs,
                            void* y, hipStream_t st) {
  using Cfg = QmvCfg<T, BITS>;
  const int nch = K / 32;
  // threads per row: enough workgroups to fill 256 CUs, at least one chunk
  // per lane
  int tpr = 16;
  while (tpr < 64 && (int64_t)N * tpr / 256 < 256 && nch >= 2 * tpr) tpr *= 2;
  while (tpr > 1 && tpr > nch) tpr /= 2;
  const int rows_per_block = 4 * (64 / tpr);
  const dim3 grid((N + rows_per_block - 1) / rows_per_block, (M + MB - 1) / MB);
  const size_t lds = (size_t)MB * nch * (Cfg::kXWords + 1) * 4;
  hipLaunchKernelGGL((qmv_kernel<T, BITS, MB>), grid, dim3(256), lds, st,
                     static_cast<const uint16_t*>(x),
                     reinterpret_cast<const uint8_t*>(wq),
                     static_cast<const uint16_t*>(s),
                     static_cast<const uint16_t*>(b),
                     static_cast<uint16_t*>(y), M, N, K, ilog2(gs), ilog2(tpr));
  return hipGetLastError();
}

template <class T, int BITS>
static hipError_t launch_t(const void* x, const uint32_t* wq, const void* s,
                           const void* b, int M, int N, int K, int gs, void* y,
                           hipStream_t st) {
  using Cfg = QmvCfg<T, BITS>;
  const int64_t per_row = (int64_t)(K / 32) * (Cfg::kXWords + 1) * 4;
  int mb_max = (int)(kMaxLds / per_row);
  int want = 1;  // smallest of 1, 2, 4, 8 covering M (8 at most)
  while (want < M && want < 8) want *= 2;
  while (want > 1 && want > mb_max) want /= 2;
  switch (want) {
    case 8: return launch_mb<T, BITS, 8>(x, wq, s, b, M, N, K, gs, y, st);
    case 4: return launch_mb<T, BITS, 4>(x, wq, s, b, M, N, K, gs, y, st);
    case 2: return launch_mb<T, BITS, 2>(x, wq, s, b, M, N, K, gs, y, st);
    default: return launch_mb<T, BITS, 1>(x, wq, s, b, M, N, K, gs, y, st);
  }
}

template <class T>
static hipError_t launch_bits(int bits, const void* x, const uint32_t* wq,
                              const void* s, const void* b, int M, int N,
                              int K, int gs, void* y, hipStream_t st) {
  switch (bits) {
    case 2: return launch_t<T, 2>(x, wq, s, b, M, N, K, gs, y, st);
    case 3: return launch_t<T, 3>(x, wq, s, b, M, N, K, gs, y, st);
    case 4: return launch_t<T, 4>(x, wq, s, b, M, N, K, gs, y, st);
    case 5: return launch_t<T, 5>(x, wq, s, b, M, N, K, gs, y, st);
    case 6: return launch_t<T, 6>(x, wq, s, b, M, N, K, gs, y, st);
    default: return launch_t<T, 8>(x, wq, s, b, M, N, K, gs, y, st);
  }
}

hipError_t launch_qmv(int dt, int bits, int gs, const void* x,
                      const uint32_t* wq, const void* s, const void* b,
                      int64_t M, int64_t N, int64_t K, void* y,
                      hipStream_t st) {
  if (dt == 0)
    return launch_bits<F16>(bits, x, wq, s, b, (int)M, (int)N, (int)K, gs, y, st);
  return launch_bits<BF16>(bits, x, wq, s, b, (int)M, (int)N, (int)K, gs, y, st);
}

}  // namespace qmm
