// Affine-packed layout ("Add the 3bit packed qmm_t": ops.cpp quantize with
// QuantizationType::AffinePacked, and the affine_packed_qmv kernels): rows of
// the affine-quantized weight are taken in blocks of RP = 4 (power-of-two
// bits) or 2 (3, 5, 6 bits). A block's scales and biases form one row holding,
// per group, the RP scales then the RP biases; for power-of-two bits the
// block's weight words are interleaved, word w of row r at w*RP + r. One
// 16-byte load then brings a word of each of 4 rows, another their scales
// and biases.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "kernels.hpp"

namespace qmm {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- pack
// One thread per (row block i, word w): the 4 rows' words w, as one 16-byte
// store at (i * kw + w) * 4 words.
__global__ __launch_bounds__(256) void apk_words_kernel(const uint32_t* __restrict__ wq,
                                                        int64_t n, int kw,
                                                        uint32_t* __restrict__ out) {
  const int64_t t = blockIdx.x * 256ll + threadIdx.x;
  if (t >= n) return;
  const int64_t i = t / kw, w = t - i * kw;
  const uint32_t* src = wq + 4 * i * kw + w;
  reinterpret_cast<uint4*>(out)[t] = make_uint4(src[0], src[kw], src[2 * kw], src[3 * kw]);
}

// One thread per (row block i, group g): RP scales then RP biases.
template <class W, int RP>
__global__ __launch_bounds__(256) void apk_scales_kernel(const W* __restrict__ s,
                                                         const W* __restrict__ b, int64_t n,
                                                         int G, W* __restrict__ out) {
  const int64_t t = blockIdx.x * 256ll + threadIdx.x;
  if (t >= n) return;
  const int64_t i = t / G, g = t - i * G;
  W* dst = out + t * 2 * RP;
#pragma unroll
  for (int r = 0; r < RP; r++) {
    dst[r] = s[(RP * i + r) * G + g];
    dst[RP + r] = b[(RP * i + r) * G + g];
  }
}

// ---------------------------------------------------------------- GEMV
// y[m, n] = sum over groups of s * sum x*q + b * sum x (fp32), power-of-two
// bits. Workgroup = kApkWaves wavefronts; kApkSplit of them share a row
// block of 4 rows, taking alternate runs of 64 words; one row m of x
// (blockIdx.y) is staged in LDS as fp32. A 16-byte load gives word w of all
// 4 rows of a block (32/BITS codes each), one 16-byte load the block's 4
// scales and 4 biases of the group; the wavefronts' sums meet in LDS.
// Measured (4096 x 4096, 4-bit g64, M = 1; waves per workgroup / per
// block): 4/1 9.85, 4/2 7.65, 4/4 6.97, 8/8 6.67, 8/4 6.20 us.
constexpr int kApkSplit = 4;   // wavefronts per row block
constexpr int kApkWaves = 8;   // wavefronts per workgroup (2 row blocks)

template <class T, int BITS>
__global__ __launch_bounds__(64 * kApkWaves) void apk_qmv_kernel(const uint16_t* __restrict__ x,
                                                      const uint32_t* __restrict__ wp,
                                                      const uint16_t* __restrict__ sbp,
                                                      uint16_t* __restrict__ y, int N, int K,
                                                      int gs_log2) {
  extern __shared__ float xs[];
  const int m = blockIdx.y;
  const uint16_t* xr = x + (int64_t)m * K;
  for (int k = threadIdx.x; k < K; k += 64 * kApkWaves) xs[k] = to_f32(T{}, xr[k]);
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = wave % kApkSplit;               // which runs of 64 words
  const int blk = blockIdx.x * (kApkWaves / kApkSplit) + wave / kApkSplit;
  const bool live = blk < N / 4;
  constexpr int kCpw = 32 / BITS;                 // codes per word
  constexpr uint32_t kMask = (1u << BITS) - 1u;
  const int kw = K / kCpw, G = K >> gs_log2;
  const u32x4* wrow = reinterpret_cast<const u32x4*>(wp + (int64_t)blk * kw * 4);
  const uint4* srow = reinterpret_cast<const uint4*>(sbp + (int64_t)blk * G * 8);
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int w = half * 64 + lane; live && w < kw; w += 64 * kApkSplit) {
    const u32x4 q = __builtin_nontemporal_load(wrow + w);
    const uint4 sb = srow[(w * kCpw) >> gs_log2];
    const uint32_t word[4] = {q.x, q.y, q.z, q.w};
    const uint32_t sbw[4] = {sb.x, sb.y, sb.z, sb.w};   // s0 s1 | s2 s3 | b0 b1 | b2 b3
    float xv[kCpw];
    const float4* xp = reinterpret_cast<const float4*>(xs + w * kCpw);
#pragma unroll
    for (int j = 0; j < kCpw / 4; j++) {
      const float4 t = xp[j];
      xv[4 * j] = t.x; xv[4 * j + 1] = t.y; xv[4 * j + 2] = t.z; xv[4 * j + 3] = t.w;
    }
    float sumx = 0.0f;
#pragma unroll
    for (int c = 0; c < kCpw; c++) sumx += xv[c];
#pragma unroll
    for (int r = 0; r < 4; r++) {
      float qs = 0.0f;
#pragma unroll
      for (int c = 0; c < kCpw; c++)
        qs = fmaf(xv[c], (float)((word[r] >> (c * BITS)) & kMask), qs);
      const float s = to_f32(T{}, (uint16_t)(sbw[r >> 1] >> (16 * (r & 1))));
      const float b = to_f32(T{}, (uint16_t)(sbw[2 + (r >> 1)] >> (16 * (r & 1))));
      acc[r] = fmaf(s, qs, fmaf(b, sumx, acc[r]));
    }
  }
  __shared__ float red[kApkWaves][4];
#pragma unroll
  for (int r = 0; r < 4; r++) {
    float v = acc[r];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0) red[wave][r] = v;
  }
  __syncthreads();
  if (half == 0 && live && lane < 4) {
    float v = 0.0f;
#pragma unroll
    for (int h = 0; h < kApkSplit; h++) v += red[wave + h][lane];
    y[(int64_t)m * N + 4 * blk + lane] = from_f32(T{}, v);
  }
}

template <class T>
hipError_t apk_qmv_t(int bits, int gs, const void* x, const uint32_t* wp, const void* sbp,
                     int64_t M, int64_t N, int64_t K, void* y, hipStream_t st) {
  constexpr int kBlocks = kApkWaves / kApkSplit;  // row blocks per workgroup
  const dim3 grid((unsigned)((N / 4 + kBlocks - 1) / kBlocks), (unsigned)M);
  const auto xp = static_cast<const uint16_t*>(x);
  const auto sp = static_cast<const uint16_t*>(sbp);
  const auto yp = static_cast<uint16_t*>(y);
  const size_t lds = (size_t)K * 4;
  switch (bits) {
    case 2: hipLaunchKernelGGL((apk_qmv_kernel<T, 2>), grid, dim3(64 * kApkWaves), lds, st, xp, wp, sp, yp,
                               (int)N, (int)K, ilog2(gs)); break;
    case 4: hipLaunchKernelGGL((apk_qmv_kernel<T, 4>), grid, dim3(64 * kApkWaves), lds, st, xp, wp, sp, yp,
                               (int)N, (int)K, ilog2(gs)); break;
    default: hipLaunchKernelGGL((apk_qmv_kernel<T, 8>), grid, dim3(64 * kApkWaves), lds, st, xp, wp, sp, yp,
                                (int)N, (int)K, ilog2(gs)); break;
  }
  return hipGetLastError();
}

template <class W>
hipError_t apk_scales_t(int rp, const void* s, const void* b, int64_t N, int64_t G, void* out,
                        hipStream_t st) {
  const int64_t n = N / rp * G;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (rp == 4)
    hipLaunchKernelGGL((apk_scales_kernel<W, 4>), grid, dim3(256), 0, st,
                       static_cast<const W*>(s), static_cast<const W*>(b), n, (int)G,
                       static_cast<W*>(out));
  else
    hipLaunchKernelGGL((apk_scales_kernel<W, 2>), grid, dim3(256), 0, st,
                       static_cast<const W*>(s), static_cast<const W*>(b), n, (int)G,
                       static_cast<W*>(out));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_affine_pack(int dt, int bits, int gs, const uint32_t* wq, const void* s,
                              const void* b, int64_t N, int64_t K, uint32_t* wq_packed,
                              void* sb_packed, hipStream_t st) {
  const bool pow2 = (bits & (bits - 1)) == 0;
  const int rp = pow2 ? 4 : 2;
  const int64_t G = K / gs;
  hipError_t e = dt == 2 ? apk_scales_t<float>(rp, s, b, N, G, sb_packed, st)
                         : apk_scales_t<uint16_t>(rp, s, b, N, G, sb_packed, st);
  if (e != hipSuccess || !pow2) return e;
  const int kw = (int)(K * bits / 32);
  const int64_t n = N / 4 * kw;
  hipLaunchKernelGGL(apk_words_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, wq, n,
                     kw, wq_packed);
  return hipGetLastError();
}

hipError_t launch_affine_packed_qmv(int dt, int bits, int gs, const void* x,
                                    const uint32_t* wq_packed, const void* sb_packed, int64_t M,
                                    int64_t N, int64_t K, void* y, hipStream_t st) {
  if (dt == 0) return apk_qmv_t<F16>(bits, gs, x, wq_packed, sb_packed, M, N, K, y, st);
  return apk_qmv_t<BF16>(bits, gs, x, wq_packed, sb_packed, M, N, K, y, st);
}

}  // namespace qmm
