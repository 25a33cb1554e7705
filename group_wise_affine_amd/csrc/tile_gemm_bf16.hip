// MFMA tile kernels: GEMM, bf16 instantiations.
#include "tile_impl.hpp"

namespace qmm {

hipError_t launch_tile_gemm_bf16(int bits, const GemmArgs& a, hipStream_t st) {
  return launch_bits<BF16, false, true>(bits, a, 1, st);
}

}  // namespace qmm
