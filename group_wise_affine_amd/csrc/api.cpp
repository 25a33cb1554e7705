// libqmm C ABI: argument validation, routing and launch. Every check runs on
// the host before any launch; on error nothing is queued and the thread-local
// message is set. The checks mirror the argument errors of the mlx ops
// ("Add the 3bit packed qmm_t", ops.cpp extract_quantized_matmul_dims and
// quantized_matmul; "mlx 1.0.0 backend/cpu/quantized.cpp", the bits / group
// size / dtype switches).
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>

#include <limits>
#include <mutex>

#include "../../include/libqmm.h"
#include "kernels.hpp"
#include "tile_args.hpp"

namespace {

thread_local char g_err[512] = "";

qmm_status fail(qmm_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

bool valid_bits(int bits) {
  return bits == 2 || bits == 3 || bits == 4 || bits == 5 || bits == 6 || bits == 8;
}
bool valid_gs(int gs) { return gs == 32 || gs == 64 || gs == 128; }

qmm_status check_bits_gs(int bits, int gs) {
  if (!valid_bits(bits))
    return fail(QMM_E_BITS, "bits must be 2, 3, 4, 5, 6 or 8 (got %d)", bits);
  if (!valid_gs(gs))
    return fail(QMM_E_GROUP, "group_size must be 32, 64 or 128 (got %d)", gs);
  return QMM_OK;
}

qmm_status check_k(int64_t K, int gs) {
  if (K < 1 || K % gs != 0)
    return fail(QMM_E_SHAPE,
                "K (%lld) must be a positive multiple of group_size (%d); "
                "pad the weight rows with zeros",
                (long long)K, gs);
  return QMM_OK;
}

size_t elem_bytes(qmm_dtype dt) { return dt == QMM_F32 ? 4 : 2; }

// the stream (NULL: the current device's default stream) belongs to the
// current device, whose memory and static scratch the launch will use
qmm_status check_stream(const char* tag, void* stream) {
  if (!stream) return QMM_OK;
  int cur = -1;
  hipDevice_t sd = -1;
  if (hipGetDevice(&cur) != hipSuccess)
    return fail(QMM_E_LAUNCH, "%s: no current HIP device", tag);
  if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sd) != hipSuccess)
    return fail(QMM_E_ARG, "%s: stream is not a valid HIP stream", tag);
  if ((int)sd != cur)
    return fail(QMM_E_ARG, "%s: stream belongs to device %d, the current device is %d", tag,
                (int)sd, cur);
  return QMM_OK;
}

qmm_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(QMM_E_LAUNCH, "%s: launch failed: %s", what,
                hipGetErrorString(e));
  g_err[0] = 0;
  return QMM_OK;
}

constexpr int64_t kI32 = std::numeric_limits<int32_t>::max();

// Calls whose kernels may use the device's static scratch (the split-K
// workspace, the tile counters, the MFMA GEMV's partial tiles and counters)
// are ordered across streams: a call queued on another stream than the
// previous such call on the device first waits for that call's work (one
// event per device, recorded after each call's launches), so calls from
// different streams or host threads do not race on the scratch. During
// stream capture nothing is waited for or recorded: a capturing caller
// orders its own work.
constexpr int kMaxDev = 64;
std::recursive_mutex g_ord_mu;
hipEvent_t g_ord_ev[kMaxDev] = {};
hipStream_t g_ord_st[kMaxDev] = {};
bool g_ord_used[kMaxDev] = {};

class ScratchOrder {
 public:
  // uses_scratch false: the call's kernels touch no scratch (the streaming
  // GEMV), so it neither waits nor records
  explicit ScratchOrder(void* stream, bool uses_scratch = true)
      : st_(static_cast<hipStream_t>(stream)) {
    if (!uses_scratch) return;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st_, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return;
    g_ord_mu.lock();   // held until the launches are queued
    dev_ = dev;
    if (!g_ord_ev[dev] && hipEventCreateWithFlags(&g_ord_ev[dev], hipEventDisableTiming) != hipSuccess)
      g_ord_ev[dev] = nullptr;
    if (g_ord_ev[dev] && g_ord_used[dev] && g_ord_st[dev] != st_)
      (void)hipStreamWaitEvent(st_, g_ord_ev[dev], 0);
  }
  ~ScratchOrder() {
    if (dev_ < 0) return;
    if (g_ord_ev[dev_] && hipEventRecord(g_ord_ev[dev_], st_) == hipSuccess) {
      g_ord_st[dev_] = st_;
      g_ord_used[dev_] = true;
    }
    g_ord_mu.unlock();
  }
  ScratchOrder(const ScratchOrder&) = delete;
  ScratchOrder& operator=(const ScratchOrder&) = delete;

 private:
  hipStream_t st_;
  int dev_ = -1;
};

qmm_status check_matmul(const char* tag, const void* x, const uint32_t* wq,
                        const void* s, const void* b, qmm_dtype dt, int64_t M,
                        int64_t N, int64_t K, int gs, int bits, const void* y) {
  if (!x || !wq || !s || !b || !y)
    return fail(QMM_E_NULL, "%s: x, wq, scales, biases and y must be non-NULL",
                tag);
  qmm_status st = check_bits_gs(bits, gs);
  if (st) return st;
  if (dt != QMM_F16 && dt != QMM_BF16)
    return fail(QMM_E_DTYPE,
                "%s: only float16 and bfloat16 are supported (got dtype %d)",
                tag, (int)dt);
  if (M < 1 || N < 1)
    return fail(QMM_E_SHAPE, "%s: M (%lld) and N (%lld) must be >= 1", tag,
                (long long)M, (long long)N);
  st = check_k(K, gs);
  if (st) return st;
  if (M > kI32 || N > kI32 || K > kI32 || M * K > ((int64_t)1 << 40) ||
      N * K > ((int64_t)1 << 40) || M * N > ((int64_t)1 << 40))
    return fail(QMM_E_SHAPE, "%s: problem too large", tag);
  if (!aligned(x, 16) || !aligned(wq, 16) || !aligned(y, 16))
    return fail(QMM_E_ALIGN, "%s: x, wq and y must be 16-byte aligned", tag);
  if (!aligned(s, 2) || !aligned(b, 2))
    return fail(QMM_E_ALIGN, "%s: scales and biases must be 2-byte aligned",
                tag);
  return QMM_OK;
}

}  // namespace

extern "C" {

const char* qmm_last_error(void) { return g_err; }

int qmm_route(qmm_dtype dt, int bits, int group_size, int64_t M, int64_t N, int64_t K) {
  if ((dt != QMM_F16 && dt != QMM_BF16) || !valid_bits(bits) || !valid_gs(group_size) ||
      M < 1 || N < 1 || K < 1 || K % group_size != 0)
    return QMM_KERNEL_NONE;
  return (int)qmm::route((int)dt, bits, group_size, M, N, K, true);
}

int64_t qmm_crossover_m(qmm_dtype dt, int bits, int group_size, int64_t N, int64_t K) {
  // route() is a step function of M for fixed (dt, bits, group_size, N, K):
  // the GEMVs up to some M, the tile kernel from there on
  for (int64_t M = 1; M <= ((int64_t)1 << 20); M = M < 64 ? M + 1 : 2 * M) {
    const int r = qmm_route(dt, bits, group_size, M, N, K);
    if (r == QMM_KERNEL_NONE) return 0;
    if (r == QMM_KERNEL_TILE) {
      if (M <= 64) return M;
      int64_t lo = M / 2, hi = M;   // route(lo) is a GEMV, route(hi) the tile kernel
      while (hi - lo > 1) {
        const int64_t mid = (lo + hi) / 2;
        (qmm_route(dt, bits, group_size, mid, N, K) == QMM_KERNEL_TILE ? hi : lo) = mid;
      }
      return hi;
    }
  }
  return 0;
}

qmm_status qmm_force_kernel(int kernel) {
  if (kernel < QMM_KERNEL_NONE || kernel > QMM_KERNEL_TILE)
    return fail(QMM_E_ARG, "qmm_force_kernel: kernel %d is not one of QMM_KERNEL_*", kernel);
  qmm::force_route((qmm::Route)kernel);
  return QMM_OK;
}

qmm_status qmm_quantize(const void* w, qmm_dtype dt, int64_t rows, int64_t K,
                        int group_size, int bits, uint32_t* wq, void* scales,
                        void* biases, void* stream) {
  if (qmm_status ss = check_stream("qmm_quantize", stream)) return ss;
  if (!w || !wq || !scales || !biases)
    return fail(QMM_E_NULL, "qmm_quantize: w, wq, scales and biases must be non-NULL");
  qmm_status st = check_bits_gs(bits, group_size);
  if (st) return st;
  if (dt != QMM_F16 && dt != QMM_BF16 && dt != QMM_F32)
    return fail(QMM_E_DTYPE, "qmm_quantize: only floating point inputs are supported");
  if (rows < 1) return fail(QMM_E_SHAPE, "qmm_quantize: rows must be >= 1");
  st = check_k(K, group_size);
  if (st) return st;
  if (rows * K > ((int64_t)1 << 42))
    return fail(QMM_E_SHAPE, "qmm_quantize: problem too large");
  if (!aligned(w, 16) || !aligned(wq, 16))
    return fail(QMM_E_ALIGN, "qmm_quantize: w and wq must be 16-byte aligned");
  if (!aligned(scales, elem_bytes(dt)) || !aligned(biases, elem_bytes(dt)))
    return fail(QMM_E_ALIGN, "qmm_quantize: scales/biases misaligned");
  return launched(qmm::launch_quantize((int)dt, bits, group_size, w, rows, K, wq,
                                       scales, biases, (hipStream_t)stream),
                  "qmm_quantize");
}

qmm_status qmm_dequantize(const uint32_t* wq, const void* scales,
                          const void* biases, qmm_dtype dt, int64_t rows,
                          int64_t K, int group_size, int bits, void* w_out,
                          void* stream) {
  if (qmm_status ss = check_stream("qmm_dequantize", stream)) return ss;
  if (!wq || !scales || !biases || !w_out)
    return fail(QMM_E_NULL, "qmm_dequantize: wq, scales, biases and w_out must be non-NULL");
  qmm_status st = check_bits_gs(bits, group_size);
  if (st) return st;
  if (dt != QMM_F16 && dt != QMM_BF16 && dt != QMM_F32)
    return fail(QMM_E_DTYPE, "qmm_dequantize: only floating point outputs are supported");
  if (rows < 1) return fail(QMM_E_SHAPE, "qmm_dequantize: rows must be >= 1");
  st = check_k(K, group_size);
  if (st) return st;
  if (rows * K > ((int64_t)1 << 42))
    return fail(QMM_E_SHAPE, "qmm_dequantize: problem too large");
  if (!aligned(wq, 16) || !aligned(w_out, 16))
    return fail(QMM_E_ALIGN, "qmm_dequantize: wq and w_out must be 16-byte aligned");
  if (!aligned(scales, elem_bytes(dt)) || !aligned(biases, elem_bytes(dt)))
    return fail(QMM_E_ALIGN, "qmm_dequantize: scales/biases misaligned");
  return launched(qmm::launch_dequantize((int)dt, bits, group_size, wq, scales,
                                         biases, rows, K, w_out,
                                         (hipStream_t)stream),
                  "qmm_dequantize");
}

qmm_status qmv(const void* x, const uint32_t* wq, const void* scales,
               const void* biases, qmm_dtype dt, int64_t M, int64_t N,
               int64_t K, int group_size, int bits, void* y, void* stream) {
  if (qmm_status ss = check_stream("qmv", stream)) return ss;
  qmm_status st = check_matmul("qmv", x, wq, scales, biases, dt, M, N, K,
                               group_size, bits, y);
  if (st) return st;
  if (qmm::route((int)dt, bits, group_size, M, N, K, false) == qmm::kRouteNone)
    return fail(QMM_E_SHAPE, "qmv: K (%lld) exceeds the GEMV kernels' limits (%lld for this "
                "bits/dtype; M <= %d rows of x within %zu bytes of LDS for f16); use qmm_t",
                (long long)K, (long long)qmm::qmv_max_k(bits, (int)dt), qmm::kQmvMfmaMaxM,
                qmm::kQmvMfmaMaxLds);
  ScratchOrder ord(stream, qmm::route((int)dt, bits, group_size, M, N, K, false) !=
                              qmm::kRouteQmv);
  return launched(qmm::launch_qmv((int)dt, bits, group_size, x, wq, scales,
                                  biases, M, N, K, y, (hipStream_t)stream),
                  "qmv");
}

qmm_status qmm_t_batched(const void* x, const uint32_t* wq, const void* scales,
                         const void* biases, int64_t batches, int64_t w_batches, qmm_dtype dt,
                         int64_t M, int64_t N, int64_t K, int group_size, int bits, void* y,
                         void* stream) {
  if (qmm_status ss = check_stream("qmm_t_batched", stream)) return ss;
  qmm_status st = check_matmul("qmm_t_batched", x, wq, scales, biases, dt, M, N, K, group_size,
                               bits, y);
  if (st) return st;
  if (batches < 1 || batches > 65535)
    return fail(QMM_E_SHAPE, "qmm_t_batched: batches (%lld) must be in [1, 65535]",
                (long long)batches);
  if (w_batches != 1 && w_batches != batches)
    return fail(QMM_E_SHAPE,
                "qmm_t_batched: w_batches (%lld) must be 1 (one weight for every batch) or "
                "batches (%lld)",
                (long long)w_batches, (long long)batches);
  if (batches * M > kI32 || batches * M * K > ((int64_t)1 << 40) ||
      batches * M * N > ((int64_t)1 << 40) || w_batches * N * K > ((int64_t)1 << 40))
    return fail(QMM_E_SHAPE, "qmm_t_batched: problem too large");
  // one weight for every batch: the batches are the rows of one product
  if (w_batches == 1)
    return qmm_t(x, wq, scales, biases, dt, batches * M, N, K, group_size, bits, y, stream);
  const hipStream_t hs = (hipStream_t)stream;
  const int64_t es = 2;   // element bytes (f16 / bf16)
  const int64_t xs = M * K * es, ys = M * N * es, ws = N * (K * bits / 8),
                ss = N * (K / group_size) * es;
  const qmm::Route r = qmm::route((int)dt, bits, group_size, M, N, K, true);
  ScratchOrder ord(stream, r != qmm::kRouteQmv);
  // the streaming GEMV's rows: one gathered launch (batch b with weight b)
  if (r == qmm::kRouteQmv)
    return launched(qmm::launch_gather_qmv((int)dt, bits, group_size, x, batches, nullptr, wq,
                                           scales, biases, batches, nullptr, batches, M, N, K, y,
                                           hs),
                    "qmm_t_batched");
  if (r == qmm::kRouteTile && K >= qmm::kTileMaxK) {
    return fail(QMM_E_SHAPE, "qmm_t_batched: K (%lld) must be below %lld for the MFMA tile kernel",
                (long long)K, (long long)qmm::kTileMaxK);
  }
  // the MFMA GEMV's or the tile kernel's rows: the batches start at offsets
  // that keep x, wq and y 16-byte aligned
  if (xs % 16 != 0 || ys % 16 != 0 || ws % 16 != 0)
    return fail(QMM_E_ALIGN,
                "qmm_t_batched: per-batch offsets of x (%lld B), y (%lld B) and wq (%lld B) must be "
                "multiples of 16 bytes",
                (long long)xs, (long long)ys, (long long)ws);
  // tile kernel: one launch over all batches
  if (r == qmm::kRouteTile)
    return launched(qmm::launch_qmm_mfma((int)dt, bits, group_size, x, wq, scales, biases, M, N,
                                         K, y, hs, batches),
                    "qmm_t_batched");
  // MFMA GEMV: one launch per batch
  const char* xb = static_cast<const char*>(x);
  const char* wb = reinterpret_cast<const char*>(wq);
  const char* sb = static_cast<const char*>(scales);
  const char* bb = static_cast<const char*>(biases);
  char* yb = static_cast<char*>(y);
  for (int64_t i = 0; i < batches; i++) {
    const void* xi = xb + i * xs;
    const uint32_t* wi = reinterpret_cast<const uint32_t*>(wb + i * ws);
    const void* si = sb + i * ss;
    const void* bi = bb + i * ss;
    void* yi = yb + i * ys;
    const hipError_t e =
        qmm::launch_qmv((int)dt, bits, group_size, xi, wi, si, bi, M, N, K, yi, hs);
    if (e != hipSuccess) return launched(e, "qmm_t_batched");
  }
  return launched(hipSuccess, "qmm_t_batched");
}

qmm_status qmm_n(const void* x, const uint32_t* wq, const void* scales, const void* biases,
                 qmm_dtype dt, int64_t M, int64_t N, int64_t K, int group_size, int bits,
                 void* y, void* stream) {
  if (qmm_status ss = check_stream("qmm_n", stream)) return ss;
  if (!x || !wq || !scales || !biases || !y)
    return fail(QMM_E_NULL, "qmm_n: x, wq, scales, biases and y must be non-NULL");
  qmm_status st = check_bits_gs(bits, group_size);
  if (st) return st;
  if (dt != QMM_F16 && dt != QMM_BF16)
    return fail(QMM_E_DTYPE, "qmm_n: only float16 and bfloat16 are supported (got dtype %d)",
                (int)dt);
  if (M < 1 || K < 1)
    return fail(QMM_E_SHAPE, "qmm_n: M (%lld) and K (%lld) must be >= 1", (long long)M,
                (long long)K);
  if (N < 1 || N % group_size != 0)
    return fail(QMM_E_SHAPE,
                "qmm_n: N (%lld) must be a positive multiple of group_size (%d): the weight "
                "[K, N] is quantized along N",
                (long long)N, group_size);
  const int64_t S = qmm::qmm_n_splits(K);
  if (M > kI32 || S > 65535 || N > kI32 || M * K > ((int64_t)1 << 40) ||
      N * K > ((int64_t)1 << 40) || M * N > ((int64_t)1 << 40))
    return fail(QMM_E_SHAPE, "qmm_n: problem too large");
  // rows of x per launch: at most 65535, and with K split the partial sums of
  // a launch's rows must fit the split-K workspace
  int64_t chunk = 65535;
  if (S > 1) {
    const int64_t fit = qmm::kSplitWsFloats / (S * N);
    if (fit < 1)
      return fail(QMM_E_SHAPE,
                  "qmm_n: one row's %lld K ranges x N (%lld) partial sums exceed the split-K "
                  "workspace (%lld floats)",
                  (long long)S, (long long)N, (long long)qmm::kSplitWsFloats);
    chunk = fit < chunk ? fit : chunk;
  }
  if (!aligned(x, 16) || !aligned(wq, 16) || !aligned(y, 16))
    return fail(QMM_E_ALIGN, "qmm_n: x, wq and y must be 16-byte aligned");
  if (!aligned(scales, 2) || !aligned(biases, 2))
    return fail(QMM_E_ALIGN, "qmm_n: scales and biases must be 2-byte aligned");
  ScratchOrder ord(stream);
  // many rows of x: the MFMA tile kernel (one pass over W per 128 rows)
  if (qmm::qmm_n_tile_fits((int)dt, M, N, K, bits))
    return launched(qmm::launch_qmm_n_tile((int)dt, bits, group_size, x, wq, scales, biases, M, N,
                                           K, y, (hipStream_t)stream),
                    "qmm_n");
  if (M > chunk && ((chunk * K * 2) % 16 != 0 || (chunk * N * 2) % 16 != 0))
    return fail(QMM_E_ALIGN,
                "qmm_n: with more than %lld rows of x the rows are taken %lld at a time, whose "
                "x and y blocks must stay 16-byte aligned (K and N multiples of 8)",
                (long long)chunk, (long long)chunk);
  const char* xb = static_cast<const char*>(x);
  char* yb = static_cast<char*>(y);
  for (int64_t m0 = 0; m0 < M; m0 += chunk) {
    const int64_t mc = M - m0 < chunk ? M - m0 : chunk;
    const hipError_t e = qmm::launch_qmm_n((int)dt, bits, group_size, xb + m0 * K * 2, wq, scales,
                                           biases, mc, N, K, yb + m0 * N * 2,
                                           (hipStream_t)stream);
    if (e != hipSuccess) return launched(e, "qmm_n");
  }
  return launched(hipSuccess, "qmm_n");
}

}  // extern "C"

namespace {

// Checks shared by the gathered products (qmm_gather_qmv, qmm_gather_qmm).
qmm_status check_gather(const char* tag, const void* x, int64_t x_batches,
                        const int32_t* lhs_indices, const uint32_t* wq, const void* scales,
                        const void* biases, int64_t w_batches, const int32_t* rhs_indices,
                        int64_t batches, qmm_dtype dt, int64_t M, int64_t N, int64_t K,
                        int group_size, int bits, const void* y) {
  qmm_status st = check_matmul(tag, x, wq, scales, biases, dt, M, N, K, group_size, bits, y);
  if (st) return st;
  if (batches < 1 || batches > 65535)
    return fail(QMM_E_SHAPE, "%s: batches (%lld) must be in [1, 65535]", tag,
                (long long)batches);
  if (x_batches < 1 || w_batches < 1 || x_batches > kI32 || w_batches > kI32)
    return fail(QMM_E_SHAPE, "%s: x_batches (%lld) and w_batches (%lld) must be >= 1", tag,
                (long long)x_batches, (long long)w_batches);
  if (!lhs_indices && x_batches < batches)
    return fail(QMM_E_SHAPE, "%s: without lhs_indices, x needs one batch per output "
                "batch (%lld < %lld)", tag, (long long)x_batches, (long long)batches);
  if (!rhs_indices && w_batches < batches)
    return fail(QMM_E_SHAPE, "%s: without rhs_indices, W needs one batch per output "
                "batch (%lld < %lld)", tag, (long long)w_batches, (long long)batches);
  if (!aligned(lhs_indices, 4) || !aligned(rhs_indices, 4))
    return fail(QMM_E_ALIGN, "%s: index arrays must be 4-byte aligned", tag);
  if (x_batches * M * K > ((int64_t)1 << 40) || w_batches * N * K > ((int64_t)1 << 40) ||
      batches * M * N > ((int64_t)1 << 40) || batches * M > kI32)
    return fail(QMM_E_SHAPE, "%s: problem too large", tag);
  return QMM_OK;
}

}  // namespace

extern "C" {

qmm_status qmm_gather_qmm(const void* x, int64_t x_batches, const int32_t* lhs_indices,
                          const uint32_t* wq, const void* scales, const void* biases,
                          int64_t w_batches, const int32_t* rhs_indices, int64_t batches,
                          qmm_dtype dt, int64_t M, int64_t N, int64_t K, int group_size,
                          int bits, void* y, void* stream) {
  if (qmm_status ss = check_stream("qmm_gather_qmm", stream)) return ss;
  qmm_status st = check_gather("qmm_gather_qmm", x, x_batches, lhs_indices, wq, scales, biases,
                               w_batches, rhs_indices, batches, dt, M, N, K, group_size, bits,
                               y);
  if (st) return st;
  const hipStream_t hs = (hipStream_t)stream;
  // few rows per product: the gathered streaming GEMV
  if (qmm::route((int)dt, bits, group_size, M, N, K, true) == qmm::kRouteQmv)
    return launched(qmm::launch_gather_qmv((int)dt, bits, group_size, x, x_batches, lhs_indices,
                                           wq, scales, biases, w_batches, rhs_indices, batches,
                                           M, N, K, y, hs),
                    "qmm_gather_qmm");
  // the rest: the MFMA tile kernel, one launch, batch z in the grid
  if (K >= qmm::kTileMaxK)
    return fail(QMM_E_SHAPE, "qmm_gather_qmm: K (%lld) must be below %lld for the MFMA tile kernel",
                (long long)K, (long long)qmm::kTileMaxK);
  const int64_t xs = M * K * 2, ys = M * N * 2, ws = N * (K * bits / 8);
  if (xs % 16 != 0 || ys % 16 != 0 || ws % 16 != 0)
    return fail(QMM_E_ALIGN,
                "qmm_gather_qmm: per-batch sizes of x (%lld B), y (%lld B) and wq (%lld B) must be "
                "multiples of 16 bytes",
                (long long)xs, (long long)ys, (long long)ws);
  ScratchOrder ord(stream);
  return launched(qmm::launch_gather_qmm_mfma((int)dt, bits, group_size, x, x_batches,
                                              lhs_indices, wq, scales, biases, w_batches,
                                              rhs_indices, batches, M, N, K, y, hs),
                  "qmm_gather_qmm");
}

qmm_status qmm_gather_qmv(const void* x, int64_t x_batches, const int32_t* lhs_indices,
                          const uint32_t* wq, const void* scales, const void* biases,
                          int64_t w_batches, const int32_t* rhs_indices, int64_t batches,
                          qmm_dtype dt, int64_t M, int64_t N, int64_t K, int group_size,
                          int bits, void* y, void* stream) {
  if (qmm_status ss = check_stream("qmm_gather_qmv", stream)) return ss;
  qmm_status st = check_gather("qmm_gather_qmv", x, x_batches, lhs_indices, wq, scales, biases,
                               w_batches, rhs_indices, batches, dt, M, N, K, group_size, bits,
                               y);
  if (st) return st;
  if (K > qmm::qmv_max_k(bits, (int)dt))
    return fail(QMM_E_SHAPE, "qmm_gather_qmv: K (%lld) exceeds the streaming GEMV's limit (%lld "
                "for this bits/dtype)", (long long)K, (long long)qmm::qmv_max_k(bits, (int)dt));
  return launched(qmm::launch_gather_qmv((int)dt, bits, group_size, x, x_batches, lhs_indices,
                                         wq, scales, biases, w_batches, rhs_indices, batches, M,
                                         N, K, y, (hipStream_t)stream),
                  "qmm_gather_qmv");
}

}  // extern "C"

namespace {

qmm_status check_fp_mode(const char* tag, int bits, int gs) {
  if (bits != 4 && bits != 8)
    return fail(QMM_E_BITS, "%s: floating-point modes take bits 4 (mxfp4, nvfp4) or 8 (mxfp8), "
                "got %d", tag, bits);
  if (!(gs == 32 || (bits == 4 && gs == 16)))
    return fail(QMM_E_GROUP, "%s: group_size must be 32 (mxfp4, mxfp8) or 16 (nvfp4, bits 4), "
                "got %d with bits %d", tag, gs, bits);
  return QMM_OK;
}

}  // namespace

extern "C" {

qmm_status qmm_fp_quantize(const void* w, qmm_dtype dt, int64_t rows, int64_t K,
                           int group_size, int bits, uint32_t* wq, uint8_t* scales,
                           void* stream) {
  if (qmm_status ss = check_stream("qmm_fp_quantize", stream)) return ss;
  if (!w || !wq || !scales)
    return fail(QMM_E_NULL, "qmm_fp_quantize: w, wq and scales must be non-NULL");
  qmm_status st = check_fp_mode("qmm_fp_quantize", bits, group_size);
  if (st) return st;
  if (dt != QMM_F16 && dt != QMM_BF16 && dt != QMM_F32)
    return fail(QMM_E_DTYPE, "qmm_fp_quantize: only floating point inputs are supported");
  if (rows < 1) return fail(QMM_E_SHAPE, "qmm_fp_quantize: rows must be >= 1");
  st = check_k(K, group_size);
  if (st) return st;
  if (rows * K > ((int64_t)1 << 42))
    return fail(QMM_E_SHAPE, "qmm_fp_quantize: problem too large");
  if (!aligned(w, 16) || !aligned(wq, 16))
    return fail(QMM_E_ALIGN, "qmm_fp_quantize: w and wq must be 16-byte aligned");
  return launched(qmm::launch_fp_quantize((int)dt, bits, group_size, w, rows, K, wq, scales,
                                          (hipStream_t)stream),
                  "qmm_fp_quantize");
}

qmm_status qmm_fp_dequantize(const uint32_t* wq, const uint8_t* scales, qmm_dtype dt,
                             int64_t rows, int64_t K, int group_size, int bits, void* w_out,
                             void* stream) {
  if (qmm_status ss = check_stream("qmm_fp_dequantize", stream)) return ss;
  if (!wq || !scales || !w_out)
    return fail(QMM_E_NULL, "qmm_fp_dequantize: wq, scales and w_out must be non-NULL");
  qmm_status st = check_fp_mode("qmm_fp_dequantize", bits, group_size);
  if (st) return st;
  if (dt != QMM_F16 && dt != QMM_BF16 && dt != QMM_F32)
    return fail(QMM_E_DTYPE, "qmm_fp_dequantize: only floating point outputs are supported");
  if (rows < 1) return fail(QMM_E_SHAPE, "qmm_fp_dequantize: rows must be >= 1");
  st = check_k(K, group_size);
  if (st) return st;
  if (rows * K > ((int64_t)1 << 42))
    return fail(QMM_E_SHAPE, "qmm_fp_dequantize: problem too large");
  if (!aligned(wq, 16) || !aligned(w_out, 16))
    return fail(QMM_E_ALIGN, "qmm_fp_dequantize: wq and w_out must be 16-byte aligned");
  return launched(qmm::launch_fp_dequantize((int)dt, bits, group_size, wq, scales, rows, K,
                                            w_out, (hipStream_t)stream),
                  "qmm_fp_dequantize");
}

qmm_status qmm_fp_qmv(const void* x, const uint32_t* wq, const uint8_t* scales, qmm_dtype dt,
                      int64_t M, int64_t N, int64_t K, int group_size, int bits, void* y,
                      void* stream) {
  if (qmm_status ss = check_stream("qmm_fp_qmv", stream)) return ss;
  if (!x || !wq || !scales || !y)
    return fail(QMM_E_NULL, "qmm_fp_qmv: x, wq, scales and y must be non-NULL");
  qmm_status st = check_fp_mode("qmm_fp_qmv", bits, group_size);
  if (st) return st;
  if (dt != QMM_F16 && dt != QMM_BF16)
    return fail(QMM_E_DTYPE, "qmm_fp_qmv: only float16 and bfloat16 are supported (got dtype %d)",
                (int)dt);
  if (M < 1 || N < 1 || M > 65535 || N > kI32)
    return fail(QMM_E_SHAPE, "qmm_fp_qmv: M (%lld) must be in [1, 65535] and N (%lld) >= 1",
                (long long)M, (long long)N);
  if (K < 32 || K % 32 != 0 || K > qmm::kFpMaxK)
    return fail(QMM_E_SHAPE, "qmm_fp_qmv: K (%lld) must be a positive multiple of 32 up to %lld",
                (long long)K, (long long)qmm::kFpMaxK);
  if (N * K > ((int64_t)1 << 40) || M * N > ((int64_t)1 << 40))
    return fail(QMM_E_SHAPE, "qmm_fp_qmv: problem too large");
  if (!aligned(x, 16) || !aligned(wq, 16) || !aligned(y, 16))
    return fail(QMM_E_ALIGN, "qmm_fp_qmv: x, wq and y must be 16-byte aligned");
  return launched(qmm::launch_fp_qmv((int)dt, bits, group_size, x, wq, scales, M, N, K, y,
                                     (hipStream_t)stream),
                  "qmm_fp_qmv");
}

qmm_status qmm_fp_t(const void* x, const uint32_t* wq, const uint8_t* scales, qmm_dtype dt,
                    int64_t M, int64_t N, int64_t K, int group_size, int bits, void* y,
                    void* stream) {
  if (qmm_status ss = check_stream("qmm_fp_t", stream)) return ss;
  if (!x || !wq || !scales || !y)
    return fail(QMM_E_NULL, "qmm_fp_t: x, wq, scales and y must be non-NULL");
  qmm_status st = check_fp_mode("qmm_fp_t", bits, group_size);
  if (st) return st;
  if (dt != QMM_F16 && dt != QMM_BF16)
    return fail(QMM_E_DTYPE, "qmm_fp_t: only float16 and bfloat16 are supported (got dtype %d)",
                (int)dt);
  if (M < 1 || N < 1 || M > kI32 || N > kI32)
    return fail(QMM_E_SHAPE, "qmm_fp_t: M (%lld) and N (%lld) must be >= 1", (long long)M,
                (long long)N);
  if (K < 32 || K % 32 != 0)
    return fail(QMM_E_SHAPE, "qmm_fp_t: K (%lld) must be a positive multiple of 32", (long long)K);
  if (N * K > ((int64_t)1 << 40) || M * N > ((int64_t)1 << 40) || M * K > ((int64_t)1 << 40))
    return fail(QMM_E_SHAPE, "qmm_fp_t: problem too large");
  if (!aligned(x, 16) || !aligned(wq, 16) || !aligned(y, 16))
    return fail(QMM_E_ALIGN, "qmm_fp_t: x, wq and y must be 16-byte aligned");
  // (qmm_force_kernel: the GEMV or the tile kernel where it takes the shape)
  const qmm::Route f = qmm::forced_route();
  const bool gemv = (f == qmm::kRouteTile   ? false
                     : f == qmm::kRouteQmv ? true
                                           : M < qmm::fp_crossover_m(bits, group_size, (int)dt, N, K)) &&
                    M <= 65535 && K <= qmm::kFpMaxK;
  ScratchOrder ord(stream, !gemv);
  if (gemv)
    return launched(qmm::launch_fp_qmv((int)dt, bits, group_size, x, wq, scales, M, N, K, y,
                                       (hipStream_t)stream),
                    "qmm_fp_t");
  if (K >= qmm::kTileMaxK)
    return fail(QMM_E_SHAPE, "qmm_fp_t: K (%lld) must be below %lld for the MFMA tile kernel",
                (long long)K, (long long)qmm::kTileMaxK);
  return launched(qmm::launch_fp_qmm_mfma((int)dt, bits, group_size, x, wq, scales, M, N, K, y,
                                          (hipStream_t)stream),
                  "qmm_fp_t");
}

qmm_status qmm_fp_n(const void* x, const uint32_t* wq, const uint8_t* scales, qmm_dtype dt,
                    int64_t M, int64_t N, int64_t K, int group_size, int bits, void* y,
                    void* stream) {
  if (qmm_status ss = check_stream("qmm_fp_n", stream)) return ss;
  if (!x || !wq || !scales || !y)
    return fail(QMM_E_NULL, "qmm_fp_n: x, wq, scales and y must be non-NULL");
  qmm_status st = check_fp_mode("qmm_fp_n", bits, group_size);
  if (st) return st;
  if (dt != QMM_F16 && dt != QMM_BF16)
    return fail(QMM_E_DTYPE, "qmm_fp_n: only float16 and bfloat16 are supported (got dtype %d)",
                (int)dt);
  if (M < 1 || K < 1 || M > kI32 || K > kI32)
    return fail(QMM_E_SHAPE, "qmm_fp_n: M (%lld) and K (%lld) must be >= 1", (long long)M,
                (long long)K);
  if (N < 32 || N % 32 != 0 || N > kI32)
    return fail(QMM_E_SHAPE,
                "qmm_fp_n: N (%lld) must be a positive multiple of 32: the weight [K, N] is "
                "quantized along N",
                (long long)N);
  if (K % 8 != 0)
    return fail(QMM_E_SHAPE, "qmm_fp_n: K (%lld) must be a multiple of 8 (16-byte rows of x)",
                (long long)K);
  if (!qmm::qmm_n_tile_fits(0, 1 << 20, N, K, bits) || M * N > ((int64_t)1 << 40) ||
      M * K > ((int64_t)1 << 40))
    return fail(QMM_E_SHAPE, "qmm_fp_n: problem too large");
  if (!aligned(x, 16) || !aligned(wq, 16) || !aligned(y, 16))
    return fail(QMM_E_ALIGN, "qmm_fp_n: x, wq and y must be 16-byte aligned");
  ScratchOrder ord(stream);
  return launched(qmm::launch_fp_qmm_n_tile((int)dt, bits, group_size, x, wq, scales, M, N, K, y,
                                            (hipStream_t)stream),
                  "qmm_fp_n");
}

qmm_status qmm_fp_gather_qmv(const void* x, int64_t x_batches, const int32_t* lhs_indices,
                             const uint32_t* wq, const uint8_t* scales, int64_t w_batches,
                             const int32_t* rhs_indices, int64_t batches, qmm_dtype dt, int64_t M,
                             int64_t N, int64_t K, int group_size, int bits, void* y,
                             void* stream) {
  if (qmm_status ss = check_stream("qmm_fp_gather_qmv", stream)) return ss;
  if (!x || !wq || !scales || !y)
    return fail(QMM_E_NULL, "qmm_fp_gather_qmv: x, wq, scales and y must be non-NULL");
  qmm_status st = check_fp_mode("qmm_fp_gather_qmv", bits, group_size);
  if (st) return st;
  if (dt != QMM_F16 && dt != QMM_BF16)
    return fail(QMM_E_DTYPE, "qmm_fp_gather_qmv: only float16 and bfloat16 are supported");
  if (M < 1 || N < 1 || M > 65535 || N > kI32)
    return fail(QMM_E_SHAPE, "qmm_fp_gather_qmv: M (%lld) must be in [1, 65535] and N (%lld) >= 1",
                (long long)M, (long long)N);
  if (K < 32 || K % 32 != 0 || K > qmm::kFpMaxK)
    return fail(QMM_E_SHAPE, "qmm_fp_gather_qmv: K (%lld) must be a positive multiple of 32 up "
                "to %lld", (long long)K, (long long)qmm::kFpMaxK);
  if (batches < 1 || batches > 65535)
    return fail(QMM_E_SHAPE, "qmm_fp_gather_qmv: batches (%lld) must be in [1, 65535]",
                (long long)batches);
  if (x_batches < 1 || w_batches < 1 || x_batches > kI32 || w_batches > kI32)
    return fail(QMM_E_SHAPE, "qmm_fp_gather_qmv: x_batches (%lld) and w_batches (%lld) must be "
                ">= 1", (long long)x_batches, (long long)w_batches);
  if (!lhs_indices && x_batches < batches)
    return fail(QMM_E_SHAPE, "qmm_fp_gather_qmv: without lhs_indices, x needs one batch per "
                "output batch (%lld < %lld)", (long long)x_batches, (long long)batches);
  if (!rhs_indices && w_batches < batches)
    return fail(QMM_E_SHAPE, "qmm_fp_gather_qmv: without rhs_indices, W needs one batch per "
                "output batch (%lld < %lld)", (long long)w_batches, (long long)batches);
  if (x_batches * M * K > ((int64_t)1 << 40) || w_batches * N * K > ((int64_t)1 << 40) ||
      batches * M * N > ((int64_t)1 << 40))
    return fail(QMM_E_SHAPE, "qmm_fp_gather_qmv: problem too large");
  if (!aligned(lhs_indices, 4) || !aligned(rhs_indices, 4))
    return fail(QMM_E_ALIGN, "qmm_fp_gather_qmv: index arrays must be 4-byte aligned");
  if (!aligned(x, 16) || !aligned(wq, 16) || !aligned(y, 16))
    return fail(QMM_E_ALIGN, "qmm_fp_gather_qmv: x, wq and y must be 16-byte aligned");
  return launched(qmm::launch_fp_gather_qmv((int)dt, bits, group_size, x, x_batches, lhs_indices,
                                            wq, scales, w_batches, rhs_indices, batches, M, N, K,
                                            y, (hipStream_t)stream),
                  "qmm_fp_gather_qmv");
}

qmm_status qmm_affine_pack(const uint32_t* wq, const void* scales, const void* biases,
                           qmm_dtype dt, int64_t N, int64_t K, int group_size, int bits,
                           uint32_t* wq_packed, void* sb_packed, void* stream) {
  if (qmm_status ss = check_stream("qmm_affine_pack", stream)) return ss;
  const bool pow2 = (bits & (bits - 1)) == 0;
  if (!wq || !scales || !biases || !sb_packed || (pow2 && !wq_packed))
    return fail(QMM_E_NULL, "qmm_affine_pack: wq, scales, biases, sb_packed (and wq_packed for "
                "power-of-two bits) must be non-NULL");
  qmm_status st = check_bits_gs(bits, group_size);
  if (st) return st;
  if (dt != QMM_F16 && dt != QMM_BF16 && dt != QMM_F32)
    return fail(QMM_E_DTYPE, "qmm_affine_pack: scales must be float16, bfloat16 or float32");
  st = check_k(K, group_size);
  if (st) return st;
  const int rp = pow2 ? 4 : 2;
  if (N < 1 || N % rp != 0)
    return fail(QMM_E_SHAPE, "qmm_affine_pack: N (%lld) must be a positive multiple of %d for "
                "%d-bit codes", (long long)N, rp, bits);
  if (N * K > ((int64_t)1 << 40))
    return fail(QMM_E_SHAPE, "qmm_affine_pack: problem too large");
  if ((pow2 && (!aligned(wq, 16) || !aligned(wq_packed, 16))) ||
      !aligned(scales, elem_bytes(dt)) || !aligned(biases, elem_bytes(dt)) ||
      !aligned(sb_packed, elem_bytes(dt)))
    return fail(QMM_E_ALIGN, "qmm_affine_pack: wq and wq_packed must be 16-byte aligned, the "
                "scale arrays aligned to their element size");
  return launched(qmm::launch_affine_pack((int)dt, bits, group_size, wq, scales, biases, N, K,
                                          wq_packed, sb_packed, (hipStream_t)stream),
                  "qmm_affine_pack");
}

// Shared checks of the affine-packed products; gemv selects the GEMV limits.
static qmm_status check_affine_packed(const char* tag, const void* x, const uint32_t* wq_packed,
                                      const void* sb_packed, qmm_dtype dt, int64_t M, int64_t N,
                                      int64_t K, int group_size, int bits, const void* y) {
  if (!x || !wq_packed || !sb_packed || !y)
    return fail(QMM_E_NULL, "%s: x, wq_packed, sb_packed and y must be non-NULL", tag);
  qmm_status st = check_bits_gs(bits, group_size);
  if (st) return st;
  if (dt != QMM_F16 && dt != QMM_BF16)
    return fail(QMM_E_DTYPE, "%s: only float16 and bfloat16 are supported", tag);
  st = check_k(K, group_size);
  if (st) return st;
  const int rp = (bits & (bits - 1)) == 0 ? 4 : 2;
  if (M < 1 || N < rp || N % rp != 0 || M > kI32 || N > kI32)
    return fail(QMM_E_SHAPE, "%s: M (%lld) must be >= 1 and N (%lld) a positive multiple of %d "
                "(rows per block of the packed layout at %d bits)", tag, (long long)M,
                (long long)N, rp, bits);
  if (N * K > ((int64_t)1 << 40) || M * N > ((int64_t)1 << 40) || M * K > ((int64_t)1 << 40))
    return fail(QMM_E_SHAPE, "%s: problem too large", tag);
  if (!aligned(x, 16) || !aligned(wq_packed, 16) || !aligned(sb_packed, 16) || !aligned(y, 16))
    return fail(QMM_E_ALIGN, "%s: x, wq_packed, sb_packed and y must be 16-byte aligned", tag);
  return QMM_OK;
}

// GEMV on the packed layout: bits 2/4/8 the interleaved-row GEMV (K up to
// kFpMaxK), bits 3/5/6 the streaming GEMV with packed scale addressing (K up
// to its LDS-staged row).
static qmm_status packed_gemv(const char* tag, const void* x, const uint32_t* wq_packed,
                              const void* sb_packed, qmm_dtype dt, int64_t M, int64_t N,
                              int64_t K, int group_size, int bits, void* y, void* stream) {
  const bool pow2 = (bits & (bits - 1)) == 0;
  const int64_t kmax = pow2 ? qmm::kFpMaxK : qmm::qmv_max_k(bits, (int)dt);
  if (M > 65535 || K > kmax)
    return fail(QMM_E_SHAPE, "%s: the GEMV takes M (%lld) up to 65535 and K (%lld) up to %lld",
                tag, (long long)M, (long long)K, (long long)kmax);
  if (pow2)
    return launched(qmm::launch_affine_packed_qmv((int)dt, bits, group_size, x, wq_packed,
                                                  sb_packed, M, N, K, y, (hipStream_t)stream),
                    tag);
  return launched(qmm::launch_qmv_packed_sb((int)dt, bits, group_size, x, wq_packed, sb_packed,
                                            M, N, K, y, (hipStream_t)stream),
                  tag);
}

qmm_status qmv_affine_packed(const void* x, const uint32_t* wq_packed, const void* sb_packed,
                             qmm_dtype dt, int64_t M, int64_t N, int64_t K, int group_size,
                             int bits, void* y, void* stream) {
  if (qmm_status ss = check_stream("qmv_affine_packed", stream)) return ss;
  qmm_status st = check_affine_packed("qmv_affine_packed", x, wq_packed, sb_packed, dt, M, N, K,
                                      group_size, bits, y);
  if (st) return st;
  return packed_gemv("qmv_affine_packed", x, wq_packed, sb_packed, dt, M, N, K, group_size, bits,
                     y, stream);
}

// Rows of x from which the packed product takes the tile kernel: the
// interleaved-row GEMV reads W once per row of x, the streaming GEMV once
// per 4 rows.
static int64_t packed_crossover_m(int bits) { return (bits & (bits - 1)) == 0 ? 3 : 5; }

qmm_status qmm_t_affine_packed(const void* x, const uint32_t* wq_packed, const void* sb_packed,
                               qmm_dtype dt, int64_t M, int64_t N, int64_t K, int group_size,
                               int bits, void* y, void* stream) {
  if (qmm_status ss = check_stream("qmm_t_affine_packed", stream)) return ss;
  const char* tag = "qmm_t_affine_packed";
  qmm_status st = check_affine_packed(tag, x, wq_packed, sb_packed, dt, M, N, K, group_size, bits,
                                      y);
  if (st) return st;
  const bool pow2 = (bits & (bits - 1)) == 0;
  const int64_t kmax = pow2 ? qmm::kFpMaxK : qmm::qmv_max_k(bits, (int)dt);
  if (M < packed_crossover_m(bits) && K <= kmax)
    return packed_gemv(tag, x, wq_packed, sb_packed, dt, M, N, K, group_size, bits, y, stream);
  if (K >= qmm::kTileMaxK)
    return fail(QMM_E_SHAPE, "%s: K (%lld) must be below %lld for the MFMA tile kernel", tag,
                (long long)K, (long long)qmm::kTileMaxK);
  ScratchOrder ord(stream);
  return launched(qmm::launch_apk_mfma((int)dt, bits, group_size, x, wq_packed, sb_packed, M, N,
                                       K, y, (hipStream_t)stream),
                  tag);
}

qmm_status qmm_t(const void* x, const uint32_t* wq, const void* scales,
                 const void* biases, qmm_dtype dt, int64_t M, int64_t N,
                 int64_t K, int group_size, int bits, void* y, void* stream) {
  if (qmm_status ss = check_stream("qmm_t", stream)) return ss;
  qmm_status st = check_matmul("qmm_t", x, wq, scales, biases, dt, M, N, K,
                               group_size, bits, y);
  if (st) return st;
  const qmm::Route r = qmm::route((int)dt, bits, group_size, M, N, K, true);
  ScratchOrder ord(stream, r != qmm::kRouteQmv);
  if (r == qmm::kRouteQmv || r == qmm::kRouteQmvMfma)
    return launched(qmm::launch_qmv((int)dt, bits, group_size, x, wq, scales,
                                    biases, M, N, K, y, (hipStream_t)stream),
                    "qmm_t");
  if (K >= qmm::kTileMaxK)
    return fail(QMM_E_SHAPE, "qmm_t: K (%lld) must be below %lld for the MFMA tile kernel",
                (long long)K, (long long)qmm::kTileMaxK);
  return launched(qmm::launch_qmm_mfma((int)dt, bits, group_size, x, wq, scales,
                                       biases, M, N, K, y, (hipStream_t)stream),
                  "qmm_t");
}

qmm_status qconv2d_nhwc(const void* x, int64_t B, int64_t H, int64_t W,
                        int64_t C, const uint32_t* wq, const void* scales,
                        const void* biases, int64_t O, int kh, int kw,
                        int stride_h, int stride_w, int pad_h, int pad_w,
                        int groups, qmm_dtype dt, int group_size, int bits,
                        void* y, void* stream) {
  if (qmm_status ss = check_stream("qconv2d_nhwc", stream)) return ss;
  if (!x || !wq || !scales || !biases || !y)
    return fail(QMM_E_NULL, "qconv2d_nhwc: x, wq, scales, biases and y must be non-NULL");
  qmm_status st = check_bits_gs(bits, group_size);
  if (st) return st;
  if (dt != QMM_F16 && dt != QMM_BF16)
    return fail(QMM_E_DTYPE, "qconv2d_nhwc: only float16 and bfloat16 are supported");
  if (B < 1 || H < 1 || W < 1 || C < 1 || O < 1 || kh < 1 || kw < 1 ||
      stride_h < 1 || stride_w < 1 || pad_h < 0 || pad_w < 0 || groups < 1)
    return fail(QMM_E_SHAPE, "qconv2d_nhwc: sizes, kernel and strides must be >= 1, padding >= 0");
  if (C % groups || O % groups)
    return fail(QMM_E_SHAPE, "qconv2d_nhwc: C (%lld) and O (%lld) must be divisible by groups (%d)",
                (long long)C, (long long)O, groups);
  qmm::ConvGeom g{};
  g.B = B; g.H = H; g.W = W; g.C = C; g.O = O;
  g.kh = kh; g.kw = kw; g.sh = stride_h; g.sw = stride_w; g.ph = pad_h; g.pw = pad_w;
  g.groups = groups;
  g.OH = (H + 2 * (int64_t)pad_h - kh) / stride_h + 1;
  g.OW = (W + 2 * (int64_t)pad_w - kw) / stride_w + 1;
  if (H + 2 * (int64_t)pad_h < kh || W + 2 * (int64_t)pad_w < kw || g.OH < 1 || g.OW < 1)
    return fail(QMM_E_SHAPE, "qconv2d_nhwc: the kernel does not fit the padded input");
  g.Cg = C / groups;
  g.Og = O / groups;
  g.K_true = (int64_t)kh * kw * g.Cg;
  g.K_pad = (g.K_true + group_size - 1) / group_size * group_size;
  const int64_t npix = B * g.OH * g.OW;
  if (npix > kI32 || g.K_pad > kI32 || B * H * W * C > ((int64_t)1 << 40) ||
      npix * O > ((int64_t)1 << 40) || groups > 65535)
    return fail(QMM_E_SHAPE, "qconv2d_nhwc: problem too large");
  if (!aligned(x, 16) || !aligned(wq, 16) || !aligned(y, 16))
    return fail(QMM_E_ALIGN, "qconv2d_nhwc: x, wq and y must be 16-byte aligned");
  if (!aligned(scales, 2) || !aligned(biases, 2))
    return fail(QMM_E_ALIGN, "qconv2d_nhwc: scales and biases must be 2-byte aligned");
  ScratchOrder ord(stream);
  return launched(qmm::launch_qconv_mfma((int)dt, bits, group_size, x, g, wq,
                                         scales, biases, y, (hipStream_t)stream),
                  "qconv2d_nhwc");
}

}  // extern "C"
