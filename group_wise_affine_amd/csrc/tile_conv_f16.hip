// MFMA tile kernels: convolution, f16 instantiations.
#include "tile_impl.hpp"

namespace qmm {

hipError_t launch_tile_conv_f16(int bits, const GemmArgs& a, int groups, bool dma,
                                hipStream_t st) {
  return dma ? launch_bits<F16, true, true>(bits, a, groups, st)
             : launch_bits<F16, true, false>(bits, a, groups, st);
}

}  // namespace qmm
