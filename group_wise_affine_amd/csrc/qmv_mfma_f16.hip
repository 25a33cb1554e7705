// MFMA GEMV, f16 instantiations, and the entry points of the MFMA GEMV.
#include <mutex>

#include "qmv_mfma_impl.hpp"

namespace qmm {

// Split-K workspace of the MFMA GEMV: fp32 partial tiles (16 x 16, or two of
// them above 16 rows of x) of every row block and split of a launch, and one
// arrival counter per row block (zero at load; a wrapping increment brings
// it back to zero on the last arrival of each call). Calls that overlap on
// one device share them.
__device__ float g_mv_ws[kQmvMfmaWsFloats];
__device__ unsigned g_mv_cnt[kQmvMfmaCounters];

namespace {

constexpr int kMaxDevices = 64;

// addresses of the current device's workspace and counters
bool mv_workspace(float** ws, unsigned** cnt) {
  static std::mutex mu;
  static float* wsa[kMaxDevices] = {};
  static unsigned* cnta[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
  std::lock_guard<std::mutex> lock(mu);
  if (!wsa[dev]) {
    void *p = nullptr, *q = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_mv_ws)) != hipSuccess ||
        hipGetSymbolAddress(&q, HIP_SYMBOL(g_mv_cnt)) != hipSuccess)
      return false;
    wsa[dev] = static_cast<float*>(p);
    cnta[dev] = static_cast<unsigned*>(q);
  }
  *ws = wsa[dev];
  *cnt = cnta[dev];
  return true;
}

}  // namespace

hipError_t launch_qmv_mfma_bf16(int bits, const MvLaunch& L, hipStream_t st);

// LDS of the GEMV kernel: rows of x over a K range of klen plus padding and
// the 16 rows of scales and biases, or the reduction buffer if larger
size_t qmv_mfma_lds(int64_t M, int64_t klen, int64_t K, int gs, bool xsums) {
  const size_t mt = M > 16 ? 2 : 1;   // 16-row tiles of x
  const size_t xb = (((size_t)M * (klen + 8) + 7) & ~(size_t)7) * 2;
  const size_t sb = (size_t)2 * 16 * ((15 + 32 * (K / gs) + 15) / 16);
  const size_t gb = xsums ? (size_t)((klen + gs - 1) / gs) * 16 * mt * 4 : 0;   // group sums of x
  const size_t rb = (size_t)kMvThreads * 4 * 4 * mt;
  return xb + sb + gb > rb ? xb + sb + gb : rb;
}

hipError_t launch_qmv_mfma(int dt, int bits, int gs, const void* x, const uint32_t* wq,
                           const void* s, const void* b, int64_t M, int64_t N, int64_t K,
                           void* y, hipStream_t st) {
  MvLaunch L{x, s, b, wq, y, (int)M, (int)N, (int)K, gs, nullptr, nullptr};
  if (!mv_workspace(&L.ws, &L.cnt)) return hipErrorInvalidSymbol;
  if (dt == 0) return launch_qmv_mfma_t<F16>(bits, L, st);
  return launch_qmv_mfma_bf16(bits, L, st);
}

}  // namespace qmm
