// MFMA tile kernels: GEMM, f16 instantiations.
#include "tile_impl.hpp"

namespace qmm {

hipError_t launch_tile_gemm_f16(int bits, const GemmArgs& a, hipStream_t st) {
  return launch_bits<F16, false, true>(bits, a, 1, st);
}

}  // namespace qmm
