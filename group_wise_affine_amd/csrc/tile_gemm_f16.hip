// MFMA tile kernels: GEMM, f16 instantiations.
#include "tile_impl.hpp"

namespace qmm {

hipError_t launch_tile_gemm_f16(int bits, const GemmArgs& a, int batches, hipStream_t st) {
  return launch_bits<F16, false, true>(bits, a, batches, st);
}

}  // namespace qmm
