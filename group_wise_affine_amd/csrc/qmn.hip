// Non-transposed quantized GEMV for small M (decode):
//   y[m, n] = sum_k x[m, k] * (s[k, n/gs] * q[k, n] + b[k, n/gs]),
// W stored [K, N] with its groups along N: the product the CPU backend's
// _qmm computes ("mlx 1.0.0 backend/cpu/quantized.cpp", the non-transposed
// branch of quantized_matmul), accumulated in fp32.
//
// MI355X design (wave64):
//  * The sum runs along the stored rows, so K is split over workgroups: a
//    workgroup owns 16 chunks of 32 columns and 128 rows of K. Lane l of
//    wavefront w (8 of them: two per SIMD issue arithmetic better than one)
//    takes chunk l % 16 and rows 4w + l/16 + 32i, i < 4, so one load
//    instruction covers four rows of 16 chunks. Every weight load of a lane
//    (one 32-code chunk per row, 4*bits bytes) is issued before any
//    arithmetic.
//  * A chunk lies in one group (gs >= 32), so per row a lane needs one scale
//    and one bias: acc[j] += (x*s) * q_j for its 32 columns and one bias sum
//    x*b shared by them.
//  * The 32 partial sums of a column (8 wavefronts x 4 row phases) are
//    added through LDS in a fixed order. With several K ranges, each
//    workgroup writes its fp32 partial row to the split-K workspace and a
//    second kernel adds the ranges in a fixed order (16 threads per output,
//    each with its loads in flight together).
#include <utility>

#include "common.hpp"
#include "kernels.hpp"

namespace qmm {
namespace {

constexpr int kQnWaves = 8;        // two wavefronts per SIMD
constexpr int kQnPhases = 4;       // row phases of a wavefront (lanes / 16)
constexpr int kQnRowsPerLane = 4;
constexpr int kQnChunks = 16;      // chunks of 32 columns per workgroup
constexpr int kQnRows = kQnWaves * kQnPhases * kQnRowsPerLane;   // 128 rows of K

// chunk of 32 codes (4*BITS bytes, 4-byte aligned) as BITS little-endian words
template <int BITS>
__device__ __forceinline__ void load_chunk_n(const uint8_t* p, uint32_t w[BITS]) {
  if constexpr (BITS % 4 == 0) {
#pragma unroll
    for (int h = 0; h < BITS / 4; h++) {
      const uint4 u = reinterpret_cast<const uint4*>(p)[h];
      w[4 * h] = u.x; w[4 * h + 1] = u.y; w[4 * h + 2] = u.z; w[4 * h + 3] = u.w;
    }
  } else if constexpr (BITS % 2 == 0) {
#pragma unroll
    for (int h = 0; h < BITS / 2; h++) {
      const uint2 u = reinterpret_cast<const uint2*>(p)[h];
      w[2 * h] = u.x; w[2 * h + 1] = u.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < BITS; i++) w[i] = reinterpret_cast<const uint32_t*>(p)[i];
  }
}

// acc[j] += xs * q_j over the chunk. For 2, 4 and 8 bits, each word is
// masked into 4 bytes per field offset (one shift and one and for 4 codes),
// which the byte-to-float conversions read directly; 3, 5 and 6 bits extract
// every code.
template <int BITS, int J>
__device__ __forceinline__ uint32_t chunk_code(const uint32_t* w);
template <int BITS>
__device__ __forceinline__ void fma_chunk(const uint32_t* w, float xs, float* acc) {
  if constexpr (BITS == 2 || BITS == 4 || BITS == 8) {
    constexpr int per = 8 / BITS;                        // codes per byte
    constexpr uint32_t bm = ((1u << BITS) - 1) * 0x01010101u;
#pragma unroll
    for (int i = 0; i < BITS; i++)                       // word i: codes 32i/BITS ...
#pragma unroll
      for (int t = 0; t < per; t++) {
        const uint32_t f = (w[i] >> (t * BITS)) & bm;
#pragma unroll
        for (int bb = 0; bb < 4; bb++) {
          const int j = (32 / BITS) * i + per * bb + t;
          acc[j] = fmaf(xs, (float)((f >> (8 * bb)) & 0xffu), acc[j]);
        }
      }
  } else {
    [&]<int... J>(std::integer_sequence<int, J...>) {
      ((acc[J] = fmaf(xs, (float)chunk_code<BITS, J>(w), acc[J])), ...);
    }(std::make_integer_sequence<int, 32>{});
  }
}

// code j of the chunk: bits [j*BITS, (j+1)*BITS) of its bit stream
template <int BITS, int J>
__device__ __forceinline__ uint32_t chunk_code(const uint32_t* w) {
  constexpr int b = J * BITS, wi = b / 32, sh = b % 32;
  constexpr uint32_t mask = (1u << BITS) - 1;
  if constexpr (sh + BITS <= 32)
    return (w[wi] >> sh) & mask;
  else
    return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & mask;
}

template <class T, int BITS>
__global__ __launch_bounds__(kQnWaves * 64) void qmn_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wq,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases,
    uint16_t* __restrict__ y, float* __restrict__ ws, int M, int N, int K, int gs_log2) {
  __shared__ float red[kQnWaves][64][33];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = N >> 5;
  const int c = blockIdx.x * kQnChunks + (lane & 15);
  const int cc = c < nch ? c : nch - 1;          // lanes past N re-read a chunk
  const int split = blockIdx.y, m = blockIdx.z;
  const int G = N >> gs_log2;
  const int g = (cc << 5) >> gs_log2;            // the chunk's group
  const int64_t row_bytes = (int64_t)N * BITS / 8;
  const int r0 = split * kQnRows + wave * kQnPhases + (lane >> 4);

  uint32_t w[kQnRowsPerLane][BITS];
  uint16_t sw[kQnRowsPerLane], bw[kQnRowsPerLane];
  float xv[kQnRowsPerLane];
#pragma unroll
  for (int i = 0; i < kQnRowsPerLane; i++) {
    const int k = r0 + kQnWaves * kQnPhases * i;
    const int kc = k < K ? k : K - 1;              // rows past K: x = 0
    load_chunk_n<BITS>(wq + (int64_t)kc * row_bytes + (int64_t)cc * (4 * BITS), w[i]);
    sw[i] = scales[(int64_t)kc * G + g];
    bw[i] = biases[(int64_t)kc * G + g];
    xv[i] = k < K ? to_f32(T{}, x[(int64_t)m * K + kc]) : 0.0f;
  }

  float acc[32];
#pragma unroll
  for (int j = 0; j < 32; j++) acc[j] = 0.0f;
  float bacc = 0.0f;
#pragma unroll
  for (int i = 0; i < kQnRowsPerLane; i++) {
    const float xs = xv[i] * to_f32(T{}, sw[i]);
    bacc = fmaf(xv[i], to_f32(T{}, bw[i]), bacc);
    fma_chunk<BITS>(w[i], xs, acc);
  }
#pragma unroll
  for (int j = 0; j < 32; j++) red[wave][lane][j] = acc[j] + bacc;
  __syncthreads();

  // thread t: column t of the block (chunk t / 32), its 32 partial sums in
  // wavefront then row-phase order
  const int cj = tid >> 5, jj = tid & 31;
  const int c_out = blockIdx.x * kQnChunks + cj;
  const bool col_ok = c_out < nch;
  const int64_t n = (int64_t)c_out * 32 + jj;
  float v = 0.0f;
#pragma unroll
  for (int wv = 0; wv < kQnWaves; wv++)
#pragma unroll
    for (int ph = 0; ph < kQnPhases; ph++) v += red[wv][16 * ph + cj][jj];
  if (gridDim.y == 1) {
    if (col_ok) y[(int64_t)m * N + n] = from_f32(T{}, v);
    return;
  }
  if (col_ok) ws[((int64_t)split * M + m) * N + n] = v;
}

// y[m, n] = sum over the S K ranges of the partial rows, in a fixed order: a
// block takes 16 outputs; thread p of an output adds ranges p, p+16, ...
// (its loads issued together, 8 at a time), then the 16 sums are added in
// order of p.
template <class T>
__global__ __launch_bounds__(256) void qmn_reduce_kernel(const float* __restrict__ ws,
                                                         uint16_t* __restrict__ y,
                                                         int64_t MN, int S) {
  __shared__ float part[16][17];
  const int o = threadIdx.x & 15, p = threadIdx.x >> 4;
  const int64_t e = (int64_t)blockIdx.x * 16 + o;
  float t = 0.0f;
  if (e < MN) {
    for (int s0 = p; s0 < S; s0 += 16 * 8) {
      float a[8];
#pragma unroll
      for (int u = 0; u < 8; u++) {
        const int sp = s0 + 16 * u;
        a[u] = sp < S ? ws[(int64_t)sp * MN + e] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < 8; u++) t += a[u];
    }
  }
  part[p][o] = t;
  __syncthreads();
  if (p == 0 && e < MN) {
    float v = part[0][o];
#pragma unroll
    for (int q = 1; q < 16; q++) v += part[q][o];
    y[e] = from_f32(T{}, v);
  }
}

template <class T, int BITS>
hipError_t launch_qmn_t(const void* x, const uint32_t* wq, const void* s, const void* b,
                        int M, int N, int K, int gs, void* y, float* ws, hipStream_t st) {
  const int nch = N / 32;
  const int S = (K + kQnRows - 1) / kQnRows;
  const dim3 grid((nch + kQnChunks - 1) / kQnChunks, S, M);
  hipLaunchKernelGGL((qmn_kernel<T, BITS>), grid, dim3(kQnWaves * 64), 0, st,
                     static_cast<const uint16_t*>(x), reinterpret_cast<const uint8_t*>(wq),
                     static_cast<const uint16_t*>(s), static_cast<const uint16_t*>(b),
                     static_cast<uint16_t*>(y), ws, M, N, K, ilog2(gs));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  const int64_t MN = (int64_t)M * N;
  hipLaunchKernelGGL((qmn_reduce_kernel<T>), dim3((unsigned)((MN + 15) / 16)), dim3(256), 0, st,
                     ws, static_cast<uint16_t*>(y), MN, S);
  return hipGetLastError();
}

template <class T>
hipError_t launch_qmn_bits(int bits, const void* x, const uint32_t* wq, const void* s,
                           const void* b, int M, int N, int K, int gs, void* y, float* ws,
                           hipStream_t st) {
  switch (bits) {
    case 2: return launch_qmn_t<T, 2>(x, wq, s, b, M, N, K, gs, y, ws, st);
    case 3: return launch_qmn_t<T, 3>(x, wq, s, b, M, N, K, gs, y, ws, st);
    case 4: return launch_qmn_t<T, 4>(x, wq, s, b, M, N, K, gs, y, ws, st);
    case 5: return launch_qmn_t<T, 5>(x, wq, s, b, M, N, K, gs, y, ws, st);
    case 6: return launch_qmn_t<T, 6>(x, wq, s, b, M, N, K, gs, y, ws, st);
    default: return launch_qmn_t<T, 8>(x, wq, s, b, M, N, K, gs, y, ws, st);
  }
}

}  // namespace

int64_t qmm_n_splits(int64_t K) { return (K + kQnRows - 1) / kQnRows; }

hipError_t launch_qmm_n(int dt, int bits, int gs, const void* x, const uint32_t* wq,
                        const void* s, const void* b, int64_t M, int64_t N, int64_t K, void* y,
                        hipStream_t st) {
  float* ws = splitk_workspace();
  if (!ws) return hipErrorInvalidSymbol;
  if (dt == 0)
    return launch_qmn_bits<F16>(bits, x, wq, s, b, (int)M, (int)N, (int)K, gs, y, ws, st);
  return launch_qmn_bits<BF16>(bits, x, wq, s, b, (int)M, (int)N, (int)K, gs, y, ws, st);
}

}  // namespace qmm
