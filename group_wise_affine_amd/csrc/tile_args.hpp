// Arguments of the MFMA tile kernels, shared by the host dispatch (qmm.hip)
// and the translation units that instantiate the kernels (tile_*.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

struct GemmArgs {
  uint32_t magic;    // magic-number pattern of the element type (f16 path)
  const uint16_t* x;
  const uint8_t* wq;
  const uint16_t* s;
  const uint16_t* b;
  uint16_t* y;
  int M, N, K;       // K: packed row length in codes (K_pad for conv)
  int gs_log2;
  int64_t ldy;       // row stride of y in elements
  // implicit im2col (conv only)
  int H, W, C, OH, OW, kh, kw, sh, sw, ph, pw, Cg, Og, K_true;
  // conv with Cg % 64 == 0: step t lies in tap t / cu (cu = Cg / 64) and tap
  // u in kernel row u / kw; quotients of such small numbers are
  // umulhi(n, mul) with mul = floor((2^32 - 1) / d) + 1 (0 for d == 1: the
  // quotient is n)
  int cu;
  uint32_t cu_mul, kw_mul;
  // split K (tile kernel only): blockIdx.y takes K steps [y*ksteps,
  // (y+1)*ksteps) and, with ksplit > 1, writes fp32 partial sums to the
  // split-K workspace ws ([split][M][ldy], for a batched GEMM
  // [split][batch][M][ldy]; kSplitWsFloats floats); the last workgroup of a
  // tile to arrive at its counter in cnt (kTileCntMax of them, each back at
  // zero after every call) adds the partial sums and writes y
  int ksplit, ksteps;
  float* ws;
  unsigned* cnt;
  // gathered GEMM (plain GEMM only): batch g multiplies x batch lidx[g] (of
  // nxb) by weight batch ridx[g] (of nwb), indices clamped into range; a
  // null array means g
  const int32_t* lidx;
  const int32_t* ridx;
  int nxb, nwb;
};

// Split-K workspace size: [split][M][ldy] fp32 partial sums, library-owned
// (a static device array of the host dispatch, passed to the kernels as ws).
constexpr int64_t kSplitWsFloats = (int64_t)16 << 20;   // 64 MiB
constexpr int kTileCntMax = 256;    // split tiles per launch (tiles x batches), at most
constexpr int kKtabMax = 4096;      // conv k-unit table entries (K_pad <= 32768)

// Tile kernel launchers, one translation unit each (they compile in
// parallel): plain GEMM and convolution, f16 and bf16. dma selects the
// buffer-load kernel for convolutions (else the gather kernel). The GEMM
// runs `batches` products of the same shape at once (blockIdx.z): batch g
// reads x + g*M*K, wq + g*N*K*bits/8 bytes, scales and biases + g*N*K/gs,
// and writes y + g*M*ldy.
hipError_t launch_tile_gemm_f16(int bits, const GemmArgs& a, int batches, hipStream_t st);
hipError_t launch_tile_gemm_bf16(int bits, const GemmArgs& a, int batches, hipStream_t st);
hipError_t launch_tile_conv_f16(int bits, const GemmArgs& a, int groups, bool dma,
                                hipStream_t st);
hipError_t launch_tile_conv_bf16(int bits, const GemmArgs& a, int groups, bool dma,
                                 hipStream_t st);
// Floating-point modes ((bits, gs) = (4, 32) mxfp4, (4, 16) nvfp4, (8, 32)
// mxfp8; dt 0 f16, 1 bf16): a.s points to the scale bytes [N, K/gs], a.b is
// unused.
hipError_t launch_tile_fp(int dt, int bits, int gs, const GemmArgs& a, hipStream_t st);
// Affine-packed layout (bits 2/4/8: rows interleaved in blocks of 4, words
// and scales; bits 3/5/6: scales in blocks of 2): a.wq the packed words,
// a.s = a.b the packed scale / bias array.
hipError_t launch_tile_apk(int dt, int bits, const GemmArgs& a, hipStream_t st);

}  // namespace qmm
