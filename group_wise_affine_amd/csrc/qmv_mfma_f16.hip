// MFMA GEMV, f16 instantiations, and the entry points of the MFMA GEMV.
#include "qmv_mfma_impl.hpp"

namespace qmm {

hipError_t launch_qmv_mfma_bf16(int bits, int gs, const void* x, const uint32_t* wq, const void* s,
                                const void* b, int64_t M, int64_t N, int64_t K, void* y,
                                hipStream_t st);

// LDS of the GEMV kernel: x rows plus padding and the 16 rows of scales and
// biases, or the reduction buffer if larger
size_t qmv_mfma_lds(int64_t M, int64_t K, int gs) {
  const size_t xb = (((size_t)M * (K + 8) + 7) & ~(size_t)7) * 2;
  const size_t sb = (size_t)2 * 16 * ((15 + 32 * (K / gs) + 15) / 16);
  const size_t rb = (size_t)kMvThreads * 4 * 4;
  return xb + sb > rb ? xb + sb : rb;
}

hipError_t launch_qmv_mfma(int dt, int bits, int gs, const void* x, const uint32_t* wq,
                           const void* s, const void* b, int64_t M, int64_t N, int64_t K,
                           void* y, hipStream_t st) {
  if (dt == 0) return launch_qmv_mfma_t<F16>(bits, gs, x, wq, s, b, M, N, K, y, st);
  return launch_qmv_mfma_bf16(bits, gs, x, wq, s, b, M, N, K, y, st);
}

}  // namespace qmm
