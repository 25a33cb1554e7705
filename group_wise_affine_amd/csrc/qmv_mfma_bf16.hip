// MFMA GEMV, bf16 instantiations.
#include "qmv_mfma_impl.hpp"

namespace qmm {

hipError_t launch_qmv_mfma_bf16(int bits, int gs, const void* x, const uint32_t* wq, const void* s,
                                const void* b, int64_t M, int64_t N, int64_t K, void* y,
                                hipStream_t st) {
  return launch_qmv_mfma_t<BF16>(bits, gs, x, wq, s, b, M, N, K, y, st);
}

}  // namespace qmm
