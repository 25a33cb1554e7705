// MFMA GEMV, bf16 instantiations.
#include "qmv_mfma_impl.hpp"

namespace qmm {

hipError_t launch_qmv_mfma_bf16(int bits, const MvLaunch& L, hipStream_t st) {
  return launch_qmv_mfma_t<BF16>(bits, L, st);
}

}  // namespace qmm
