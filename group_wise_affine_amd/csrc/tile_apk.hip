// MFMA tile kernels on the affine-packed layout, f16 and bf16 instantiations.
#include "tile_impl.hpp"

namespace qmm {

namespace {
template <class T>
hipError_t launch_apk_t(int bits, const GemmArgs& a, hipStream_t st) {
  switch (bits) {
    case 2: return launch_shape<T, 2, 0, true, 0, 4>(a, 1, st);
    case 3: return launch_shape<T, 3, 0, true, 0, 2>(a, 1, st);
    case 4: return launch_shape<T, 4, 0, true, 0, 4>(a, 1, st);
    case 5: return launch_shape<T, 5, 0, true, 0, 2>(a, 1, st);
    case 6: return launch_shape<T, 6, 0, true, 0, 2>(a, 1, st);
    default: return launch_shape<T, 8, 0, true, 0, 4>(a, 1, st);
  }
}
}  // namespace

hipError_t launch_tile_apk(int dt, int bits, const GemmArgs& a, hipStream_t st) {
  return dt == 0 ? launch_apk_t<F16>(bits, a, st) : launch_apk_t<BF16>(bits, a, st);
}

}  // namespace qmm
