// Host-side launchers of the libqmm kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

// dt: 0 = f16, 1 = bf16, 2 = f32 (same numbering as qmm_dtype).
hipError_t launch_quantize(int dt, int bits, int gs, const void* w,
                           int64_t rows, int64_t K, uint32_t* wq, void* s,
                           void* b, hipStream_t st);
hipError_t launch_dequantize(int dt, int bits, int gs, const uint32_t* wq,
                             const void* s, const void* b, int64_t rows,
                             int64_t K, void* out, hipStream_t st);

// Streaming GEMV, any M (re-reads W once per 8 rows of x at most).
hipError_t launch_qmv(int dt, int bits, int gs, const void* x,
                      const uint32_t* wq, const void* s, const void* b,
                      int64_t M, int64_t N, int64_t K, void* y,
                      hipStream_t st);

// MFMA tile GEMM: y[M,N] = x[M,K] . dequant(W)[N,K]^T. K must be below
// kTileMaxK (byte offsets inside a tile stay below 2^30, in range of the
// buffer resources the tile kernel reads through).
constexpr int64_t kTileMaxK = (int64_t)1 << 22;
hipError_t launch_qmm_mfma(int dt, int bits, int gs, const void* x,
                           const uint32_t* wq, const void* s, const void* b,
                           int64_t M, int64_t N, int64_t K, void* y,
                           hipStream_t st);

// Implicit-im2col conv on the MFMA tile GEMM.
struct ConvGeom {
  int64_t B, H, W, C, O, OH, OW;
  int kh, kw, sh, sw, ph, pw, groups;
  int64_t Cg, Og, K_true, K_pad;
};
hipError_t launch_qconv_mfma(int dt, int bits, int gs, const void* x,
                             const ConvGeom& g, const uint32_t* wq,
                             const void* s, const void* b, void* y,
                             hipStream_t st);

// Smallest M routed to the MFMA kernel by qmm_t.
int crossover_m(int bits, int dt);

}  // namespace qmm
