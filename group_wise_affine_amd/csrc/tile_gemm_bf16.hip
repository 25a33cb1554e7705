// MFMA tile kernels: GEMM, bf16 instantiations.
#include "tile_impl.hpp"

namespace qmm {

hipError_t launch_tile_gemm_bf16(int bits, const GemmArgs& a, int batches, hipStream_t st) {
  return launch_bits<BF16, false, true>(bits, a, batches, st);
}

}  // namespace qmm
