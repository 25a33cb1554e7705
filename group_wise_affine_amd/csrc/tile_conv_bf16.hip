// MFMA tile kernels: convolution, bf16 instantiations.
#include "tile_impl.hpp"

namespace qmm {

hipError_t launch_tile_conv_bf16(int bits, const GemmArgs& a, int groups, bool dma,
                                hipStream_t st) {
  // channel counts per group that are a multiple of 64 keep every K step in
  // one tap: those pieces are addressed without the k table
  if (dma && a.Cg % 64 == 0) return launch_bits<BF16, 2, true>(bits, a, groups, st);
  return dma ? launch_bits<BF16, 1, true>(bits, a, groups, st)
             : launch_bits<BF16, 1, false>(bits, a, groups, st);
}

}  // namespace qmm
