// Measurement kernels for the decode GEMV's single-launch floor (built into
// libqmm_ceiling.so, used by the benchmark only; not part of libqmm):
//  * qmm_ceiling_read: one launch that streams a buffer from HBM with 16-byte
//    nontemporal loads (all of a lane's loads issued before any use) and
//    folds it into one word per workgroup -- the fastest a single launch of
//    that many bytes can read them;
//  * qmm_ceiling_empty: a launch of the given grid whose kernel does nothing
//    but end -- the fixed cost of dispatching that grid.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmm_ceiling.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kUnroll = 8;   // 16-byte loads in flight per lane per round

__global__ void read_kernel(const u32x4* __restrict__ src, int64_t n16,
                            uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; u++) {
      const int64_t j = i + u * stride;
      v[u] = j < n16 ? __builtin_nontemporal_load(src + j) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // one word per workgroup keeps the loads live
  acc = __reduce_or_sync(~0ull, acc);
  if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

__global__ void empty_kernel() {}

}  // namespace

extern "C" int qmm_ceiling_read(const void* src, int64_t bytes, void* sink, int blocks,
                                int threads, void* stream) {
  if (!src || !sink || bytes < 16 || bytes % 16 || blocks < 1 || threads < 64 ||
      threads > 1024 || threads % 64)
    return 1;
  hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(threads), 0, (hipStream_t)stream,
                     static_cast<const u32x4*>(src), bytes / 16, static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int qmm_ceiling_empty(int blocks, int threads, void* stream) {
  if (blocks < 1 || threads < 64 || threads > 1024 || threads % 64) return 1;
  hipLaunchKernelGGL(empty_kernel, dim3(blocks), dim3(threads), 0, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
