// MFMA tile kernels: convolution, bf16 instantiations.
#include "tile_impl.hpp"

namespace qmm {

hipError_t launch_tile_conv_bf16(int bits, const GemmArgs& a, int groups, bool dma,
                                hipStream_t st) {
  return dma ? launch_bits<BF16, true, true>(bits, a, groups, st)
             : launch_bits<BF16, true, false>(bits, a, groups, st);
}

}  // namespace qmm
