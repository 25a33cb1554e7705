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

// GEMV on the matrix cores, f16 / bf16, 1 <= M <= kQmvMfmaMaxM (one 16-row
// tile of x, two above 16 rows), K < kQmvMfmaMaxK (byte offsets of its
// buffer loads stay below 2^31), x[0:M] small enough for LDS
// (qmv_mfma_fits).
constexpr int kQmvMfmaMaxM = 32;
constexpr int64_t kQmvMfmaMaxK = (int64_t)1 << 25;
constexpr size_t kQmvMfmaMaxLds = 160 * 1024 - 256;   // LDS per CU, less static LDS
// split-K partial tiles of the MFMA GEMV (floats) and its arrival counters
// (one per row block of a split launch)
constexpr int64_t kQmvMfmaWsFloats = 256 * 8 * 256;
constexpr int kQmvMfmaCounters = 256;
// K split of the MFMA GEMV: layers with fewer than 256 blocks of 16 rows
// split K into ks ranges of sps steps (128 codes each) so that the launch
// fills the CUs, as long as each range keeps all 16 wavefronts busy; with
// more than 16 rows of x, ranges of at most 16 steps, so that 32 rows of x
// fit in LDS; klen = codes of the longest range.
struct QmvMfmaPlan {
  int ks, sps, klen;
};
inline QmvMfmaPlan qmv_mfma_plan(int64_t N, int64_t K, int64_t M) {
  const int64_t nsteps = (K / 32 + 3) / 4, rb = (N + 15) / 16;
  int64_t ks = 1;
  if (rb < 256) {
    ks = 256 / rb;
    if (ks > 8) ks = 8;
    if (ks > nsteps / 16) ks = nsteps / 16;   // every wavefront keeps a step
    if (ks < 1) ks = 1;
  }
  if (M > 16 && ks < (nsteps + 15) / 16) ks = (nsteps + 15) / 16;
  const int64_t sps = (nsteps + ks - 1) / ks;
  ks = (nsteps + sps - 1) / sps;          // no empty range
  const int64_t klen = sps * 128 < K ? sps * 128 : K;
  return {(int)ks, (int)sps, (int)klen};
}
// the MFMA GEMV multiplies the codes themselves (bf16, 4- and 8-bit codes)
// and keeps the group sums of x in LDS
inline bool qmv_mfma_exact(int dt, int bits) { return dt == 1 && (bits == 4 || bits == 8); }
size_t qmv_mfma_lds(int64_t M, int64_t klen, int64_t K, int gs, bool xsums);
inline bool qmv_mfma_fits(int64_t M, int64_t N, int64_t K, int gs, int dt, int bits) {
  if (M < 1 || M > kQmvMfmaMaxM || K >= kQmvMfmaMaxK) return false;
  const QmvMfmaPlan p = qmv_mfma_plan(N, K, M);
  // a split launch: at most 8 ranges, one counter per row block, the
  // partial tiles within the workspace
  const int64_t rb = (N + 15) / 16;
  if (p.ks > 8 || (p.ks > 1 && (rb > kQmvMfmaCounters ||
                                rb * p.ks * 256 * (M > 16 ? 2 : 1) > kQmvMfmaWsFloats)))
    return false;
  // the workgroup's 1024 threads copy x with at most 8 16-byte loads each,
  // the scales and biases with at most 2
  return qmv_mfma_lds(M, p.klen, K, gs, qmv_mfma_exact(dt, bits)) <= kQmvMfmaMaxLds &&
         M * (p.klen / 8) <= 8 * 1024 &&
         (15 + 32 * (K / gs) + 15) / 16 <= 2 * 1024;
}
// Non-transposed GEMV: y[M,N] = x[M,K] . dequant(W[K,N]) with W quantized
// along N (N % gs == 0). K is split into qmm_n_splits(K) ranges; with more
// than one, fp32 partial rows go to the split-K workspace
// ([split][M][N], within kSplitWsFloats) and a second kernel adds them.
int64_t qmm_n_splits(int64_t K);
hipError_t launch_qmm_n(int dt, int bits, int gs, const void* x, const uint32_t* wq,
                        const void* s, const void* b, int64_t M, int64_t N, int64_t K, void* y,
                        hipStream_t st);
// the current device's split-K workspace and the tile kernels' per-tile
// arrival counters (static device arrays), or null
float* splitk_workspace();
unsigned* tile_counters();
// Non-transposed product on the MFMA tile kernel (many rows of x, K split
// over workgroups when the output has few tiles), for K % 8 == 0 (16-byte x
// units) and W below 2 GiB, from 5 rows of x for f16 and 7 for bf16: the GEMV
// reads W once per row (4096 x 4096 4-bit: 9.7 / 15.5 / 19.3 us at M = 1 / 4
// / 6), the tile kernel once per 128 rows with K split (17.0 us at M = 8,
// 84 us at M = 1024; bf16 20.7 us at M = 8).
inline bool qmm_n_tile_fits(int dt, int64_t M, int64_t N, int64_t K, int bits) {
  return M >= (dt == 0 ? 5 : 7) && K % 8 == 0 && N * K * bits / 8 < ((int64_t)1 << 31) &&
         (M + 127) / 128 <= 65535 && K * 128 * 2 < ((int64_t)1 << 31);
}
hipError_t launch_qmm_n_tile(int dt, int bits, int gs, const void* x, const uint32_t* wq,
                             const void* s, const void* b, int64_t M, int64_t N, int64_t K,
                             void* y, hipStream_t st);
// the same kernel in the fp modes (scales: bytes [K, N/gs], no bias)
hipError_t launch_fp_qmm_n_tile(int dt, int bits, int gs, const void* x, const uint32_t* wq,
                                const uint8_t* scales, int64_t M, int64_t N, int64_t K, void* y,
                                hipStream_t st);

// Gathered streaming GEMV: for z < B, y[z] = x[lidx[z]] . dequant(W[ridx[z]])^T
// with x [nxb, M, K], W [nwb, N, K] (scales / biases [nwb, N, K/gs]) and
// y [B, M, N]; a null index array means z. Indices are clamped into range.
hipError_t launch_gather_qmv(int dt, int bits, int gs, const void* x, int64_t nxb,
                             const int32_t* lidx, const uint32_t* wq, const void* s,
                             const void* b, int64_t nwb, const int32_t* ridx, int64_t B,
                             int64_t M, int64_t N, int64_t K, void* y, hipStream_t st);
hipError_t launch_qmv_mfma(int dt, int bits, int gs, const void* x, const uint32_t* wq,
                           const void* s, const void* b, int64_t M, int64_t N,
                           int64_t K, void* y, hipStream_t st);

// MFMA tile GEMM: y[M,N] = x[M,K] . dequant(W)[N,K]^T. K must be below
// kTileMaxK (byte offsets inside a tile stay below 2^30, in range of the
// buffer resources the tile kernel reads through). With batches > 1 (at most
// 65535), one launch computes y[g] = x[g] . dequant(W[g])^T for every batch
// g of contiguous x [batches, M, K], W [batches, N, K] and y [batches, M, N]
// (every batch's x, wq and y 16-byte aligned; the split-K partial sums of
// all batches within the workspace).
constexpr int64_t kTileMaxK = (int64_t)1 << 22;
hipError_t launch_qmm_mfma(int dt, int bits, int gs, const void* x,
                           const uint32_t* wq, const void* s, const void* b,
                           int64_t M, int64_t N, int64_t K, void* y,
                           hipStream_t st, int64_t batches = 1);

// Gathered MFMA tile GEMM: for z < B, y[z] = x[lidx[z]] . dequant(W[ridx[z]])^T
// with x [nxb, M, K], W [nwb, N, K], y [B, M, N] (a null index array means
// z; indices are clamped into range). Same limits as launch_qmm_mfma with
// batches = B.
hipError_t launch_gather_qmm_mfma(int dt, int bits, int gs, const void* x, int64_t nxb,
                                  const int32_t* lidx, const uint32_t* wq, const void* s,
                                  const void* b, int64_t nwb, const int32_t* ridx, int64_t B,
                                  int64_t M, int64_t N, int64_t K, void* y, hipStream_t st);

// Floating-point modes, (bits, gs) in {(4, 32) mxfp4, (4, 16) nvfp4, (8, 32)
// mxfp8}: codes [rows, K*bits/8] bytes, one scale byte per group.
hipError_t launch_fp_quantize(int dt, int bits, int gs, const void* w, int64_t rows, int64_t K,
                              uint32_t* wq, uint8_t* scales, hipStream_t st);
hipError_t launch_fp_dequantize(int dt, int bits, int gs, const uint32_t* wq,
                                const uint8_t* scales, int64_t rows, int64_t K, void* out,
                                hipStream_t st);
// GEMV, f16 / bf16: K % 32 == 0, K <= kFpMaxK (x row staged in LDS as fp32),
// M <= 65535 (one pass over W per row of x).
constexpr int64_t kFpMaxK = 16384;
hipError_t launch_fp_qmv(int dt, int bits, int gs, const void* x, const uint32_t* wq,
                         const uint8_t* scales, int64_t M, int64_t N, int64_t K, void* y,
                         hipStream_t st);
// fp-mode product on the MFMA tile kernel, any M (same limits as
// launch_qmm_mfma: K below kTileMaxK, x, wq and y 16-byte aligned).
hipError_t launch_fp_qmm_mfma(int dt, int bits, int gs, const void* x, const uint32_t* wq,
                              const uint8_t* scales, int64_t M, int64_t N, int64_t K, void* y,
                              hipStream_t st);
// Rows of x from which qmm_fp_t takes the tile kernel instead of the fp GEMV.
int fp_crossover_m(int bits, int gs, int dt, int64_t N, int64_t K);
// Gathered fp GEMV: for z < B, y[z] = x[lidx[z]] . dequant(W[ridx[z]])^T with
// x [nxb, M, K], W [nwb, N, K] (codes and scale bytes), y [B, M, N]; a null
// index array means z, indices are clamped into range. B <= 65535.
hipError_t launch_fp_gather_qmv(int dt, int bits, int gs, const void* x, int64_t nxb,
                                const int32_t* lidx, const uint32_t* wq, const uint8_t* scales,
                                int64_t nwb, const int32_t* ridx, int64_t B, int64_t M, int64_t N,
                                int64_t K, void* y, hipStream_t st);

// Affine-packed layout: pack the affine-quantized wq / scales / biases of N
// rows (N % RP == 0, RP = 4 for power-of-two bits, else 2) and the GEMV on
// the packed layout (power-of-two bits, f16 / bf16, K <= kFpMaxK).
hipError_t launch_affine_pack(int dt, int bits, int gs, const uint32_t* wq, const void* s,
                              const void* b, int64_t N, int64_t K, uint32_t* wq_packed,
                              void* sb_packed, hipStream_t st);
hipError_t launch_affine_packed_qmv(int dt, int bits, int gs, const void* x,
                                    const uint32_t* wq_packed, const void* sb_packed, int64_t M,
                                    int64_t N, int64_t K, void* y, hipStream_t st);

// GEMV on the affine-packed layout of 3/5/6-bit weights (standard words,
// scales and biases interleaved in pairs of rows; N even): the streaming
// GEMV with packed scale addressing.
hipError_t launch_qmv_packed_sb(int dt, int bits, int gs, const void* x, const uint32_t* wq,
                                const void* sbp, int64_t M, int64_t N, int64_t K, void* y,
                                hipStream_t st);
// Product on the affine-packed layout on the MFMA tile kernel, any M (N a
// multiple of 4 for bits 2/4/8, of 2 otherwise; limits as launch_qmm_mfma).
hipError_t launch_apk_mfma(int dt, int bits, int gs, const void* x, const uint32_t* wq_packed,
                           const void* sbp, int64_t M, int64_t N, int64_t K, void* y,
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

// Kernel choice for y = x . dequant(W)^T, from measured kernel times (see
// route()): the streaming dot2 GEMV for a row or two of x (and for up to 32
// rows of small layers), the MFMA GEMV for up to 16 rows, the MFMA tile
// kernel for the rest. qmv never takes the tile kernel (kRouteNone when
// neither GEMV accepts the shape).
enum Route { kRouteNone = 0, kRouteQmv = 1, kRouteQmvMfma = 2, kRouteTile = 3 };
Route route(int dt, int bits, int gs, int64_t M, int64_t N, int64_t K, bool allow_tile);

// Largest K the streaming dot2 GEMV stages in LDS.
int64_t qmv_max_k(int bits, int dt);

// Whether the streaming GEMV runs one row of x of a single product in its
// 2-chunk, 8-wavefront lane shape (5-, 6- and 8-bit codes on layers that make
// one round of 256 to 320 workgroups with 4 chunks per lane, rows of at most
// 4096 codes): the launcher's own choice for M = 1.
bool qmv_two_chunk_shape(int64_t N, int64_t K, int bits);

// Measurement override: route() returns r wherever that kernel takes the
// shape (kRouteNone: the automatic choice everywhere).
void force_route(Route r);
Route forced_route();   // the current override (kRouteNone: automatic)

}  // namespace qmm
