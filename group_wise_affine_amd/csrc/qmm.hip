// Host side of the MFMA tile GEMM and the quantized conv2d: argument
// packing, the split-K workspace, and the routing between the GEMV kernels
// and the tile kernels (kernels in tile_impl.hpp, instantiated by
// tile_gemm_{f16,bf16}.hip and tile_conv_{f16,bf16}.hip).
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"
#include "tile_args.hpp"

namespace qmm {

// Split-K workspace, one per device (a static device array: no allocation
// at call time). Calls that overlap on one device share it.
__device__ float g_splitk_ws[kSplitWsFloats];

namespace {

constexpr int kMaxDevices = 64;

// address of the current device's workspace (looked up once per device)
float* splitk_ws() {
  static std::mutex mu;
  static float* addr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_splitk_ws)) != hipSuccess) return nullptr;
    addr[dev] = static_cast<float*>(p);
  }
  return addr[dev];
}

}  // namespace

float* splitk_workspace() { return splitk_ws(); }

hipError_t launch_qmm_mfma(int dt, int bits, int gs, const void* x,
                           const uint32_t* wq, const void* s, const void* b,
                           int64_t M, int64_t N, int64_t K, void* y,
                           hipStream_t st, int64_t batches) {
  return launch_gather_qmm_mfma(dt, bits, gs, x, batches, nullptr, wq, s, b, batches, nullptr,
                                batches, M, N, K, y, st);
}

hipError_t launch_gather_qmm_mfma(int dt, int bits, int gs, const void* x, int64_t nxb,
                                  const int32_t* lidx, const uint32_t* wq, const void* s,
                                  const void* b, int64_t nwb, const int32_t* ridx, int64_t B,
                                  int64_t M, int64_t N, int64_t K, void* y, hipStream_t st) {
  GemmArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.wq = reinterpret_cast<const uint8_t*>(wq);
  a.s = static_cast<const uint16_t*>(s);
  a.b = static_cast<const uint16_t*>(b);
  a.y = static_cast<uint16_t*>(y);
  a.M = (int)M; a.N = (int)N; a.K = (int)K;
  a.gs_log2 = ilog2(gs);
  a.ldy = N;
  a.magic = F16::kMagic;
  a.lidx = lidx; a.ridx = ridx;
  a.nxb = (int)nxb; a.nwb = (int)nwb;
  a.ws = splitk_ws();
  if (!a.ws) return hipErrorInvalidSymbol;
  return dt == 0 ? launch_tile_gemm_f16(bits, a, (int)B, st)
                 : launch_tile_gemm_bf16(bits, a, (int)B, st);
}

hipError_t launch_qconv_mfma(int dt, int bits, int gs, const void* x,
                             const ConvGeom& cg, const uint32_t* wq,
                             const void* s, const void* b, void* y,
                             hipStream_t st) {
  GemmArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.wq = reinterpret_cast<const uint8_t*>(wq);
  a.s = static_cast<const uint16_t*>(s);
  a.b = static_cast<const uint16_t*>(b);
  a.y = static_cast<uint16_t*>(y);
  a.M = (int)(cg.B * cg.OH * cg.OW);
  a.N = (int)cg.Og;
  a.K = (int)cg.K_pad;
  a.gs_log2 = ilog2(gs);
  a.ldy = cg.O;
  a.magic = F16::kMagic;
  a.H = (int)cg.H; a.W = (int)cg.W; a.C = (int)cg.C;
  a.OH = (int)cg.OH; a.OW = (int)cg.OW;
  a.kh = cg.kh; a.kw = cg.kw; a.sh = cg.sh; a.sw = cg.sw;
  a.ph = cg.ph; a.pw = cg.pw;
  a.Cg = (int)cg.Cg; a.Og = (int)cg.Og; a.K_true = (int)cg.K_true;
  // exact for dividends below 2^16 (steps and taps here are far fewer)
  auto div_mul = [](int d) { return d > 1 ? 0xffffffffu / (uint32_t)d + 1u : 0u; };
  a.cu = (int)(cg.Cg / 64);
  a.cu_mul = div_mul(a.cu);
  a.kw_mul = div_mul(cg.kw);
  // the DMA path needs 16-byte x pieces (8 channels of one tap) and a k
  // table (one entry per 8 channels, dy and dx below 256) that fits in LDS
  const int64_t nk = (cg.K_pad + 63) / 64;
  // (and x below 2^30 bytes, in range of one buffer resource)
  const bool dma = (cg.Cg % 8) == 0 && nk * 8 <= kKtabMax && cg.kh < 256 && cg.kw < 256 &&
                   cg.B * cg.H * cg.W * cg.C < ((int64_t)1 << 29);
  a.ws = splitk_ws();
  if (!a.ws) return hipErrorInvalidSymbol;
  return dt == 0 ? launch_tile_conv_f16(bits, a, cg.groups, dma, st)
                 : launch_tile_conv_bf16(bits, a, cg.groups, dma, st);
}

// The GEMV kernels' share of small M (see route()): up to 16 rows on the
// MFMA GEMV when x fits in LDS (K <= 4096 at 16 rows).
int crossover_m(int bits, int dt) {
  (void)bits;
  (void)dt;
  return kQmvMfmaMaxM + 1;
}

int64_t qmv_max_k(int bits, int dt) {
  const int64_t words = (bits == 8 && dt == 1) ? 34 : 18;
  return (64 * 1024 / (words * 4)) * 32;
}

Route route(int dt, int bits, int gs, int64_t M, int64_t N, int64_t K, bool allow_tile) {
  const bool dot2_ok = K <= qmv_max_k(bits, dt);
  const bool mfma_ok = qmv_mfma_fits(M, N, K, gs);
  if (dt == 0 && mfma_ok && (M >= 3 || (K > 8192 && N >= 4096) || !dot2_ok)) return kRouteQmvMfma;
  // bf16 dequantizes in fp32 and multiplies hi and lo halves: worth it from
  // 4 rows, and always for 8-bit codes, which the streaming GEMV handles in
  // fp32
  if (dt == 1 && mfma_ok && (M >= 4 || bits == 8 || !dot2_ok)) return kRouteQmvMfma;
  if (!allow_tile) return dot2_ok ? kRouteQmv : kRouteNone;
  // the MFMA GEMV does not take the shape: a few rows on the streaming GEMV
  // (one pass over W per 4 rows at K = 4096), the rest on the tile kernel
  if (M < (dt == 0 ? 4 : 8) && dot2_ok) return kRouteQmv;
  return kRouteTile;
}

}  // namespace qmm
