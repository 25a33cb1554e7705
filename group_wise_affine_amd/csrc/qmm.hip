// Host side of the MFMA tile GEMM and the quantized conv2d: argument
// packing, the split-K workspace, and the routing between the GEMV kernels
// and the tile kernels (kernels in tile_impl.hpp, instantiated by
// tile_gemm_{f16,bf16}.hip and tile_conv_{f16,bf16}.hip).
#include <atomic>
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"
#include "tile_args.hpp"

namespace qmm {

// Split-K workspace and the tile kernel's per-tile arrival counters, one of
// each per device (static device arrays: no allocation at call time). Calls
// that overlap on one device share them.
__device__ float g_splitk_ws[kSplitWsFloats];
__device__ unsigned g_tile_cnt[kTileCntMax];

namespace {

constexpr int kMaxDevices = 64;

struct SplitScratch {
  float* ws;
  unsigned* cnt;
};

// addresses of the current device's workspace and counters (looked up once
// per device)
SplitScratch split_scratch() {
  static std::mutex mu;
  static SplitScratch addr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return {};
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev].ws) {
    void *p = nullptr, *q = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_splitk_ws)) != hipSuccess ||
        hipGetSymbolAddress(&q, HIP_SYMBOL(g_tile_cnt)) != hipSuccess)
      return {};
    addr[dev] = {static_cast<float*>(p), static_cast<unsigned*>(q)};
  }
  return addr[dev];
}

// the tile kernel's scratch into a (false when the lookup failed)
bool set_scratch(GemmArgs& a) {
  const SplitScratch sc = split_scratch();
  a.ws = sc.ws;
  a.cnt = sc.cnt;
  return sc.ws && sc.cnt;
}

}  // namespace

float* splitk_workspace() { return split_scratch().ws; }
unsigned* tile_counters() { return split_scratch().cnt; }

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
  if (!set_scratch(a)) return hipErrorInvalidSymbol;
  return dt == 0 ? launch_tile_gemm_f16(bits, a, (int)B, st)
                 : launch_tile_gemm_bf16(bits, a, (int)B, st);
}

hipError_t launch_fp_qmm_mfma(int dt, int bits, int gs, const void* x, const uint32_t* wq,
                              const uint8_t* scales, int64_t M, int64_t N, int64_t K, void* y,
                              hipStream_t st) {
  GemmArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.wq = reinterpret_cast<const uint8_t*>(wq);
  a.s = reinterpret_cast<const uint16_t*>(scales);   // scale bytes
  a.b = nullptr;
  a.y = static_cast<uint16_t*>(y);
  a.M = (int)M; a.N = (int)N; a.K = (int)K;
  a.gs_log2 = ilog2(gs);
  a.ldy = N;
  a.nxb = 1; a.nwb = 1;
  if (!set_scratch(a)) return hipErrorInvalidSymbol;
  return launch_tile_fp(dt, bits, gs, a, st);
}

hipError_t launch_apk_mfma(int dt, int bits, int gs, const void* x, const uint32_t* wq_packed,
                           const void* sbp, int64_t M, int64_t N, int64_t K, void* y,
                           hipStream_t st) {
  GemmArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.wq = reinterpret_cast<const uint8_t*>(wq_packed);
  a.s = static_cast<const uint16_t*>(sbp);
  a.b = a.s;
  a.y = static_cast<uint16_t*>(y);
  a.M = (int)M; a.N = (int)N; a.K = (int)K;
  a.gs_log2 = ilog2(gs);
  a.ldy = N;
  a.magic = F16::kMagic;
  a.nxb = 1; a.nwb = 1;
  if (!set_scratch(a)) return hipErrorInvalidSymbol;
  return launch_tile_apk(dt, bits, a, st);
}

// The fp GEMV reads W once per row of x (from L2 after the first); the tile
// kernel once per 128 rows, at a nearly constant 8.4-12 us for M <= 8.
// Graph-timed with each kernel forced (f16, cold weights, 4096 x 4096,
// 2048 x 8192 and 8192 x 2048): the GEMV wins up to M = 4 (mxfp4), 6 (nvfp4)
// and 2 (mxfp8) on 4096 x 4096, to M = 6-8 / 8 / 4 on the long rows of
// 2048 x 8192, and to M = 3 / 4 / 2 on 8192 x 2048, whose 8192 rows per row
// of x cost the GEMV most. Returns the first M on the tile kernel.
int fp_crossover_m(int bits, int gs, int dt, int64_t N, int64_t K) {
  (void)dt;
  const bool wide = N >= 8192, deep = K >= 8192;
  if (bits == 8) return wide ? 3 : deep ? 5 : 3;   // mxfp8
  if (gs == 16) return wide ? 5 : deep ? 9 : 7;    // nvfp4
  return wide ? 4 : deep ? 8 : 5;                  // mxfp4
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
  if (!set_scratch(a)) return hipErrorInvalidSymbol;
  return dt == 0 ? launch_tile_conv_f16(bits, a, cg.groups, dma, st)
                 : launch_tile_conv_bf16(bits, a, cg.groups, dma, st);
}

// The GEMV kernels' share of small M (see route()): up to 16 rows on the
// MFMA GEMV when x fits in LDS (K <= 4096 at 16 rows).
namespace {
std::atomic<int> g_forced{kRouteNone};   // measurement override (force_route)
}  // namespace

void force_route(Route r) { g_forced.store((int)r, std::memory_order_relaxed); }
Route forced_route() { return (Route)g_forced.load(std::memory_order_relaxed); }

int64_t qmv_max_k(int bits, int dt) {
  const int64_t words = (bits == 8 && dt == 1) ? 34 : 18;
  return (64 * 1024 / (words * 4)) * 32;
}

Route route(int dt, int bits, int gs, int64_t M, int64_t N, int64_t K, bool allow_tile) {
  const bool dot2_ok = K <= qmv_max_k(bits, dt);
  const bool mfma_ok = qmv_mfma_fits(M, N, K, gs, dt, bits);
  switch (g_forced.load(std::memory_order_relaxed)) {
    case kRouteQmv: if (dot2_ok) return kRouteQmv; break;
    case kRouteQmvMfma: if (mfma_ok) return kRouteQmvMfma; break;
    case kRouteTile: if (allow_tile) return kRouteTile; break;
    default: break;
  }
  // Switch points from kernel-only times of the three kernels forced at
  // M = 1..32 (rocprofv3 kernel trace, g64, f16 and bf16 layers from
  // [512, 2048] to [8192, 2048]; cold weights):
  //  * the streaming GEMV reads W once per pass of up to 4 rows of x and
  //    costs ~5 us at M = 1 on a 9.4 MB layer, ~7 at 2 and ~10 at 3-4; the
  //    MFMA GEMV is nearly flat in M (6.2-7.0 us f16 on 4096 x 4096, 5.5-6.4
  //    on 8192 x 2048) but slower at M = 1;
  //  * bf16: the MFMA GEMV (8.3-9.7 us on 2048 x 8192 4-bit, 6.6-7.6 on
  //    8192 x 2048) wins from 3 rows on most layers, the streaming GEMV up
  //    to 2; with 8-bit codes the streaming GEMV works in fp32 and keeps
  //    only M = 1, and only where it runs its 2-chunk lane shape (4096 x
  //    4096: 7.7 against 10.3 us; 12.0 against 8.8 at M = 2); on layers of
  //    at most 2^20 weights it matches the MFMA GEMV at 8 rows and is
  //    5-9% faster from 12 to 32 rows (512 x 2048);
  //  * the tile kernel costs 8-18 us at M <= 32 whatever the layer size, so
  //    layers of at most 2^22 weights, whose streaming passes take ~1 us,
  //    stay on the streaming GEMV up to 32 rows.
  const bool gemv_fp32 = dt == 1 && bits == 8;
  const bool small = N * K <= ((int64_t)1 << 22);
  int64_t m0;   // first M on the MFMA GEMV
  if (!dot2_ok) m0 = 1;
  else if (gemv_fp32) m0 = qmv_two_chunk_shape(N, K, bits) ? 2 : 1;
  else if (dt == 0 && K > 8192 && N >= 4096) m0 = 1;   // long rows: few streaming passes fit
  else if (dt == 0) m0 = N * K >= ((int64_t)1 << 23) ? 2 : 3;
  else m0 = 3;
  // 17..32 rows (two row tiles, K ranges of at most 2048 codes): the MFMA
  // GEMV beats the tile kernel by 6-30% unless the shorter ranges split a
  // layer of >= 256 row blocks, doubling its workgroups (4096 x 4096: 11.7
  // against 10.9 us at M = 24)
  const bool rows_ok = M <= 16 || (N + 15) / 16 < 256 || K <= 2048;
  const bool tiny_bf16 = dt == 1 && !gemv_fp32 && dot2_ok && N * K <= ((int64_t)1 << 20) && M > 8;
  if (mfma_ok && M >= m0 && rows_ok && !tiny_bf16) return kRouteQmvMfma;
  if (!allow_tile) return dot2_ok ? kRouteQmv : kRouteNone;
  if (dot2_ok) {
    if (M < m0) return kRouteQmv;
    // the MFMA GEMV does not take the shape (more than 16 rows, or x too
    // long for LDS): a few rows, or a small layer, on the streaming GEMV
    if (M < (dt == 0 ? 4 : 8)) return kRouteQmv;
    if (!gemv_fp32 && M <= 32 && small) return kRouteQmv;
  }
  return kRouteTile;
}

}  // namespace qmm
