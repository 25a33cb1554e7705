// MFMA tile kernels in the floating-point modes (mxfp4, nvfp4, mxfp8), f16
// and bf16 instantiations.
#include "tile_impl.hpp"

namespace qmm {

hipError_t launch_tile_fp(int dt, int bits, int gs, const GemmArgs& a, hipStream_t st) {
  if (dt == 0) {
    if (bits == 8) return launch_shape<F16, 8, 0, true, 3>(a, 1, st);
    if (gs == 16) return launch_shape<F16, 4, 0, true, 2>(a, 1, st);
    return launch_shape<F16, 4, 0, true, 1>(a, 1, st);
  }
  if (bits == 8) return launch_shape<BF16, 8, 0, true, 3>(a, 1, st);
  if (gs == 16) return launch_shape<BF16, 4, 0, true, 2>(a, 1, st);
  return launch_shape<BF16, 4, 0, true, 1>(a, 1, st);
}

}  // namespace qmm
