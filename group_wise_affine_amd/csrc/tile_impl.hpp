// MFMA tile GEMM for y = x . dequant(W)^T at large M (kernel templates,
// instantiated by tile_gemm_{f16,bf16}.hip and tile_conv_{f16,bf16}.hip), and the implicit-im2col
// quantized conv2d that feeds the same tile engine.
//
// Operation: "mlx 1.0.0 backend/cpu/quantized.cpp", _qmm_t (y[m,n] =
// sum_k x[m,k] * (s*q + b)); tile structure in the spirit of the Metal
// qmm_t of "Add the 3bit packed qmm_t" (per K step: an x tile, a W tile
// dequantized on chip, a multiply), rebuilt for gfx950.
//
// Two kernels:
//  * qmm_dma_kernel (plain GEMM, and convolutions whose per-group channel
//    count is a multiple of 8): x and packed W tiles are copied global ->
//    LDS by buffer loads that write LDS directly, three K steps ahead, into a
//    four-slot ring; each wavefront dequantizes its W operands of the next
//    step from LDS in small pieces placed between the MFMAs of the current
//    step (v_mfma_f32_32x32x16_{f16,bf16}, fp32 accumulators).
//  * qmm_mfma_kernel (the remaining convolutions): register-staged x
//    gathers, one K step of prefetch.
// W values are fl32(s*q + b) rounded to the element type. For bf16 a single
// rounding to 8 significand bits would cost ~1e-3 relative error, so W is
// split as hi = bf16(w), lo = bf16(w - hi) and both halves go through the
// MFMA (error ~2^-17 relative).
// The conv variants ("[Feature] Quantized Convolution 2D" issue, img2col +
// quantized_matmul) compute the im2col addresses inside the x loader: GEMM
// row m = output pixel (b, oy, ox), column k = (dy, dx, c) of conv group g =
// blockIdx.z, zero for taps outside the image and for the padded tail
// k >= K_true.
#pragma once
#include <utility>

#include "common.hpp"
#include "kernels.hpp"
#include "mfma_common.hpp"
#include "tile_args.hpp"

namespace qmm {
// internal linkage: every translation unit that includes this header has its
// own copy of the kernels it instantiates
namespace {


template <int BITS>
__device__ __forceinline__ void load_wchunk(const uint8_t* p, uint32_t w[BITS]) {
  if constexpr (BITS == 4) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
  } else if constexpr (BITS == 8) {
    const uint4 u = reinterpret_cast<const uint4*>(p)[0];
    const uint4 v = reinterpret_cast<const uint4*>(p)[1];
    w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
    w[4] = v.x; w[5] = v.y; w[6] = v.z; w[7] = v.w;
  } else if constexpr (BITS == 2) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    w[0] = u.x; w[1] = u.y;
  } else if constexpr (BITS == 6) {
#pragma unroll
    for (int i = 0; i < 3; i++) {
      const uint2 u = reinterpret_cast<const uint2*>(p)[i];
      w[2 * i] = u.x; w[2 * i + 1] = u.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < BITS; i++) w[i] = reinterpret_cast<const uint32_t*>(p)[i];
  }
}

// f16 dequantization of a 32-code chunk into 16 natural-order f16 pairs.
// Codes are first turned into magic f16 values 1024 + q*2^o (one v_and_or_b32
// per pair, see common.hpp); each is then mapped through one fp32 FMA with
// s*2^-o and b - 1024*s*2^-o and rounded once to f16 (v_fma_mix), giving
// f16(s*q + b) up to a 2^-14 |s| perturbation of the constant.
template <int BITS>
__device__ __forceinline__ void dequant_chunk_f16(const uint32_t* w, float s,
                                                  float b, uint32_t m2,
                                                  uint32_t magic, uint32_t* out) {
  uint32_t pr[16];
#pragma unroll
  for (int p = 0; p < 16; p++) pr[p] = 0;
  [&]<int... P>(std::integer_sequence<int, P...>) {
    ((pr[P] = magic_pair<F16, BITS, P>(w, m2, magic)), ...);
  }(std::make_integer_sequence<int, 16>{});
  float so[8], co[8];
#pragma unroll
  for (int o = 0; o < 8; o++) {
    so[o] = s * __builtin_bit_cast(float, (uint32_t)(127 - o) << 23);
    co[o] = fmaf(-1024.0f, so[o], b);
  }
#pragma unroll
  for (int k = 0; k < 32; k += 2) {
    float v[2];
#pragma unroll
    for (int e = 0; e < 2; e++) {
      const int kk = k + e;
      const int p = pair_index<BITS>(kk), h = pair_half<BITS>(kk);
      const int o = pair_off<F16, BITS>(kk);
      const float q = (float)__builtin_bit_cast(half2_t, pr[p])[h];
      v[e] = fmaf(q, so[o], co[o]);
    }
    // building the pair as a vector lets the two roundings land in the low
    // and high halves directly (v_fma_mixlo_f16 / v_fma_mixhi_f16)
    const half2_t hv = {(_Float16)v[0], (_Float16)v[1]};
    out[k / 2] = __builtin_bit_cast(uint32_t, hv);
  }
}

// bf16 dequantization of a chunk, split as hi = bf16(w), lo = bf16(w - hi)
// (four 8-code pieces)
template <int BITS>
__device__ __forceinline__ void dequant_chunk_bf16(const uint32_t* w, float s,
                                                   float b, uint32_t* hi,
                                                   uint32_t* lo) {
  dequant_piece_bf16<BITS, 0>(w, s, b, hi, lo);
  dequant_piece_bf16<BITS, 8>(w, s, b, hi, lo);
  dequant_piece_bf16<BITS, 16>(w, s, b, hi, lo);
  dequant_piece_bf16<BITS, 24>(w, s, b, hi, lo);
}

// Instruction interleave for one half step (one basic block): after the
// first LDS fragment reads, each MFMA is followed by one LDS read (next
// fragments), one global load while any remain and a few VALU instructions
// of the dequantization, so the VALU and memory work runs in the shadow of
// the matrix core; the rest of the VALU work and the LDS writes follow.
template <int NM, int NDR, int NVM, int NV>
__device__ __forceinline__ void interleave_half_step() {
  constexpr int first = NDR / (NM > 0 ? NM : 1) > 0 ? NDR - (NM - 1) : NDR;
  __builtin_amdgcn_sched_group_barrier(0x100, first > 0 ? first : 0, 0);
  [&]<int... I>(std::integer_sequence<int, I...>) {
    ((__builtin_amdgcn_sched_group_barrier(0x008, 1, 0),
      __builtin_amdgcn_sched_group_barrier(0x100, (I < NDR - first) ? 1 : 0, 0),
      __builtin_amdgcn_sched_group_barrier(0x020, (I < NVM) ? 1 : 0, 0),
      __builtin_amdgcn_sched_group_barrier(0x002, NV, 0)),
     ...);
  }(std::make_integer_sequence<int, NM>{});
}

constexpr int kBK = 64;       // K step
constexpr int kPad = 8;       // LDS row padding in 16-bit elements
constexpr int kLdsRow = kBK + kPad;

// Per-thread register state of one K step.
//  x part: A_VECS 16-byte vectors of the x tile (written to LDS).
//  W part: for each of the wavefront's FN 32-row blocks, the lane's raw
//  32-code chunk of its weight row plus that chunk's scale and bias words.
template <int BM, int BN, int BITS>
struct TileRegs {
  static constexpr int A_VECS = BM * kBK / 8 / 256;
  static constexpr int FN = BN / 64;
  uint4 a[A_VECS];
  bool al[A_VECS];
  uint32_t w[FN][BITS];
  uint16_t s[FN], b[FN];
  bool wl[FN];
};

// Workgroup tile BM x BN of y, 256 threads = 2x2 wavefronts, wavefront tile
// (BM/2) x (BN/2) of 32x32 MFMA tiles, K in steps of 64.
//
// K order inside a step: MFMA kk (0..3) takes, in lane group g = lane/32,
// the 8 elements k = 32g + 8kk .. +7 (the same permutation for x and W, so the
// product is unchanged). A lane's weight operand for a whole step is then one
// contiguous 32-code chunk of its W row, loaded straight from global memory
// and dequantized in registers by the wavefront that uses it: no LDS for W.
// x goes through two LDS stages (shared by the two wavefronts of a row).
// Registers hold the global loads of step k+2 and the dequantized weights of
// step k+1 while step k multiplies; one barrier per step.
template <class T, int BITS, int BM, int BN, bool CONV, bool CONV_VEC>
__global__ __launch_bounds__(256) void qmm_mfma_kernel(GemmArgs a) {
  constexpr bool kSplit = __is_same(T, BF16);
  constexpr int WTM = BM / 2, WTN = BN / 2;      // wavefront tile
  constexpr int FM = WTM / 32, FN = WTN / 32;    // 32x32 accumulator tiles
  using Regs = TileRegs<BM, BN, BITS>;
  constexpr int A_VECS = Regs::A_VECS;
  constexpr int A_STAGE = BM * kLdsRow;
  constexpr int NB = kSplit ? 2 : 1;             // weight operands per MFMA
  static_assert(A_VECS >= 1 && FN == Regs::FN, "tile shape");

  __shared__ __attribute__((aligned(16))) uint16_t As[2 * A_STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = CONV ? blockIdx.z : 0;
  // Tile order: workgroup i runs on XCD i % 8; give each XCD a contiguous
  // band of tiles (row-major over N fastest) so that its concurrent
  // workgroups share x rows and weight rows in its L2.
  int tile = blockIdx.x;
  {
    const int nt = gridDim.x;
    if ((nt & 7) == 0) tile = (tile & 7) * (nt >> 3) + (tile >> 3);
  }
  const int tiles_n = (a.N + BN - 1) / BN;
  const int m_blk = (tile / tiles_n) * BM, n_blk = (tile % tiles_n) * BN;

  const uint8_t* wq = a.wq;
  const uint16_t* sp = a.s;
  const uint16_t* bp = a.b;
  const int64_t w_row_bytes = (int64_t)a.K * BITS / 8;
  const int n_groups_row = a.K >> a.gs_log2;
  if constexpr (CONV) {
    wq += (int64_t)g * a.Og * w_row_bytes;
    sp += (int64_t)g * a.Og * n_groups_row;
    bp += (int64_t)g * a.Og * n_groups_row;
  }
  uint32_t magic_v, m2_s = Pack<BITS>::kMask | (Pack<BITS>::kMask << 16);
  asm volatile("v_mov_b32 %0, %1" : "=v"(magic_v) : "s"(a.magic));

  // ---- per-thread x rows (fixed across K steps)
  int a_row[A_VECS], a_kv[A_VECS];
  int pix_b[A_VECS], pix_y[A_VECS], pix_x[A_VECS];
  bool a_ok[A_VECS];
#pragma unroll
  for (int v = 0; v < A_VECS; v++) {
    const int idx = tid + 256 * v;
    a_row[v] = idx / (kBK / 8);
    a_kv[v] = idx % (kBK / 8);
    const int m = m_blk + a_row[v];
    a_ok[v] = m < a.M;
    if constexpr (CONV) {
      const int mm = a_ok[v] ? m : 0;
      pix_b[v] = mm / (a.OH * a.OW);
      const int r = mm - pix_b[v] * a.OH * a.OW;
      pix_y[v] = (r / a.OW) * a.sh - a.ph;
      pix_x[v] = (r % a.OW) * a.sw - a.pw;
    }
  }
  // weight rows of this lane (one per 32-row block of the wavefront tile)
  int w_n[FN];
  bool w_ok[FN];
#pragma unroll
  for (int j = 0; j < FN; j++) {
    const int n = n_blk + wn * WTN + 32 * j + (lane & 31);
    w_ok[j] = n < a.N;
    w_n[j] = w_ok[j] ? n : a.N - 1;
  }
  const int w_koff = 32 * (lane >> 5);  // this lane's 32 codes of a step

  const int nkt = (a.K + kBK - 1) / kBK;
  // Steps past the end (the phantom half of an odd step count) re-read the
  // last tile and are marked dead, so they contribute zeros.
  auto load_tile = [&](int kt_in, Regs& r) {
    const bool step_ok = kt_in < nkt;
    const int kt = step_ok ? kt_in : nkt - 1;
    const int k0 = kt * kBK;
#pragma unroll
    for (int v = 0; v < A_VECS; v++) {
      const int k = k0 + a_kv[v] * 8;
      if constexpr (!CONV) {
        const int kc = k < a.K ? k : a.K - 8;
        const int m = a_ok[v] ? m_blk + a_row[v] : a.M - 1;
        r.al[v] = step_ok && a_ok[v] && k < a.K;
        r.a[v] = *reinterpret_cast<const uint4*>(a.x + (int64_t)m * a.K + kc);
      } else if constexpr (CONV_VEC) {
        const int kk = k < a.K_true ? k : 0;
        const int tap = kk / a.Cg, c = kk - tap * a.Cg;
        const int dy = tap / a.kw, dx = tap - dy * a.kw;
        const int iy = pix_y[v] + dy, ix = pix_x[v] + dx;
        const bool in = step_ok && a_ok[v] && k < a.K_true && iy >= 0 && iy < a.H &&
                        ix >= 0 && ix < a.W;
        r.al[v] = in;
        const int iyc = in ? iy : 0, ixc = in ? ix : 0;
        r.a[v] = *reinterpret_cast<const uint4*>(
            a.x + (((int64_t)pix_b[v] * a.H + iyc) * a.W + ixc) * a.C + g * a.Cg + c);
      } else {
        uint16_t e[8];
#pragma unroll
        for (int i = 0; i < 8; i++) {
          e[i] = 0;
          const int kk = k + i;
          if (a_ok[v] && kk < a.K_true) {
            const int tap = kk / a.Cg, c = kk - tap * a.Cg;
            const int dy = tap / a.kw, dx = tap - dy * a.kw;
            const int iy = pix_y[v] + dy, ix = pix_x[v] + dx;
            if (iy >= 0 && iy < a.H && ix >= 0 && ix < a.W)
              e[i] = a.x[(((int64_t)pix_b[v] * a.H + iy) * a.W + ix) * a.C + g * a.Cg + c];
          }
        }
        r.al[v] = step_ok;
        r.a[v] = make_uint4(e[0] | (uint32_t)e[1] << 16, e[2] | (uint32_t)e[3] << 16,
                            e[4] | (uint32_t)e[5] << 16, e[6] | (uint32_t)e[7] << 16);
      }
    }
    const int kc = k0 + w_koff;
    const bool kc_ok = kc < a.K;
    const int kcc = kc_ok ? kc : a.K - 32;
    const int gi = kcc >> a.gs_log2;
#pragma unroll
    for (int j = 0; j < FN; j++) {
      r.wl[j] = step_ok && w_ok[j] && kc_ok;
      load_wchunk<BITS>(wq + (int64_t)w_n[j] * w_row_bytes + (int64_t)kcc * BITS / 8, r.w[j]);
      r.s[j] = sp[(int64_t)w_n[j] * n_groups_row + gi];
      r.b[j] = bp[(int64_t)w_n[j] * n_groups_row + gi];
    }
  };

  // x registers of one step -> LDS stage (masking, not branches)
  auto store_x = [&](const Regs& r, int stage) {
    uint16_t* as = As + stage * A_STAGE;
#pragma unroll
    for (int v = 0; v < A_VECS; v++) {
      const uint32_t keep = r.al[v] ? 0xffffffffu : 0u;
      *reinterpret_cast<uint4*>(&as[a_row[v] * kLdsRow + a_kv[v] * 8]) =
          make_uint4(r.a[v].x & keep, r.a[v].y & keep, r.a[v].z & keep, r.a[v].w & keep);
    }
  };

  // weight registers of one step -> MFMA B operands: bfr[j][h][kk] holds the
  // 8 values of k = 32*(lane/32) + 8*kk of row block j (h: bf16 hi / lo)
  auto dequant_w = [&](const Regs& r, uint4 (&bfr)[FN][NB][4]) {
#pragma unroll
    for (int j = 0; j < FN; j++) {
      const float sc = r.wl[j] ? to_f32(T{}, r.s[j]) : 0.0f;
      const float bi = r.wl[j] ? to_f32(T{}, r.b[j]) : 0.0f;
      uint32_t hi[16];
      if constexpr (kSplit) {
        uint32_t lo[16];
        dequant_chunk_bf16<BITS>(r.w[j], sc, bi, hi, lo);
#pragma unroll
        for (int kk = 0; kk < 4; kk++)
          bfr[j][1][kk] = make_uint4(lo[4 * kk], lo[4 * kk + 1], lo[4 * kk + 2], lo[4 * kk + 3]);
      } else {
        dequant_chunk_f16<BITS>(r.w[j], sc, bi, m2_s, magic_v, hi);
      }
#pragma unroll
      for (int kk = 0; kk < 4; kk++)
        bfr[j][0][kk] = make_uint4(hi[4 * kk], hi[4 * kk + 1], hi[4 * kk + 2], hi[4 * kk + 3]);
    }
  };

  float16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; i++)
#pragma unroll
    for (int j = 0; j < FN; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

  auto mma_step = [&](int stage, const uint4 (&bfr)[FN][NB][4]) {
    const uint16_t* as = As + stage * A_STAGE;
#pragma unroll
    for (int kk = 0; kk < 4; kk++) {
      const int kof = 32 * (lane >> 5) + 8 * kk;
      uint4 af[FM];
#pragma unroll
      for (int i = 0; i < FM; i++)
        af[i] = *reinterpret_cast<const uint4*>(
            &as[(wm * WTM + 32 * i + (lane & 31)) * kLdsRow + kof]);
#pragma unroll
      for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
#pragma unroll
          for (int h = 0; h < NB; h++) acc[i][j] = mfma32(T{}, af[i], bfr[j][h][kk], acc[i][j]);
    }
  };

  // ---- pipeline (unrolled by two so that register sets are static)
  Regs r0, r1;
  uint4 b0[FN][NB][4], b1[FN][NB][4];
  load_tile(0, r0);
  load_tile(1, r1);
  store_x(r0, 0);
  dequant_w(r0, b0);
  __syncthreads();
  constexpr int kMfma = 4 * FM * FN * NB;
  constexpr int kDsRead = 4 * FM;
  constexpr int kVmem = A_VECS + FN * 3;
  for (int kt = 0; kt < nkt; kt += 2) {
    // step kt: LDS stage 0 + b0; r1 holds step kt+1
    load_tile(kt + 2, r0);
    mma_step(0, b0);
    store_x(r1, 1);
    dequant_w(r1, b1);
    if constexpr (!CONV || CONV_VEC) interleave_half_step<kMfma, kDsRead, kVmem, 6>();
    __syncthreads();
    // step kt+1 (zeros past the end): LDS stage 1 + b1; r0 holds step kt+2
    load_tile(kt + 3, r1);
    mma_step(1, b1);
    store_x(r0, 0);
    dequant_w(r0, b0);
    if constexpr (!CONV || CONV_VEC) interleave_half_step<kMfma, kDsRead, kVmem, 6>();
    __syncthreads();
  }

  // ---- epilogue: accumulators -> T -> LDS tile -> 16-byte coalesced stores.
  // Lane holds column lane%32 and rows 8*(r/4) + 4*(lane/32) + r%4 of each
  // 32x32 tile.
  constexpr int CROW = BN + 8;
  static_assert(BM * CROW <= 2 * A_STAGE, "epilogue tile must fit the x stages");
  uint16_t* cs = As;
#pragma unroll
  for (int i = 0; i < FM; i++)
#pragma unroll
    for (int j = 0; j < FN; j++) {
      const int col = wn * WTN + 32 * j + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int row = wm * WTM + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        cs[row * CROW + col] = from_f32(T{}, acc[i][j][r]);
      }
    }
  __syncthreads();
  uint16_t* yb = a.y + (CONV ? (int64_t)g * a.Og : 0);
  constexpr int VPR = BN / 8;  // 16-byte vectors per tile row
  const bool vec_ok = (a.N % 8 == 0) && (a.ldy % 8 == 0);
#pragma unroll
  for (int it = 0; it < BM * VPR / 256; it++) {
    const int idx = tid + 256 * it;
    const int row = idx / VPR, cv = idx % VPR;
    const int m = m_blk + row, n = n_blk + cv * 8;
    if (m < a.M) {
      const uint16_t* src = &cs[row * CROW + cv * 8];
      if (vec_ok && n + 8 <= a.N) {
        *reinterpret_cast<uint4*>(yb + (int64_t)m * a.ldy + n) =
            *reinterpret_cast<const uint4*>(src);
      } else {
        for (int e = 0; e < 8; e++)
          if (n + e < a.N) yb[(int64_t)m * a.ldy + n + e] = src[e];
      }
    }
  }
}

// ------------------------------------------------------- LDS-DMA tile GEMM
//
// Main MFMA path (plain GEMM and convolutions whose per-group channel count
// is a multiple of 8). Per K step of 64 codes a workgroup needs a BM x 64 x
// tile and a BN x 64-code W tile; both are copied global -> LDS by the
// load-to-LDS form of the vector loads (no registers, no LDS store
// instructions), three steps ahead, into a ring of four LDS slots. The
// slots are separate LDS arrays: the compiler tracks pending LDS-DMA writes
// per array, so reading one slot does not wait for the copies into another.
// Every copy instruction moves 64 x 16 bytes (or 64 x 4) into consecutive
// LDS; which global piece each lane fetches implements the LDS layout:
//  * x slot: BM rows of 128 bytes (eight 16-byte units); unit c of row r sits
//    at position c ^ ((r >> 1) & 7), so the 32 rows read by one MFMA operand
//    load spread over all banks.
//  * W slot: BN rows of 8*BITS bytes (the row's 64 codes of the step); for
//    16-byte units the unit index is XOR-ed with a row-derived value for the
//    same reason.
// Scales and biases come in stages of 8 steps (512 codes): cooperative
// 2-byte loads (consecutive lanes on consecutive groups of a row), stored to
// LDS as (scale | bias << 16) words, double-buffered.
// While the MFMAs of step t run, each wavefront dequantizes its W operands of
// step t+1 from LDS into registers (same K permutation as above: lane group g
// takes codes 32g..32g+31 of the step). One wait + barrier per step.

typedef __attribute__((address_space(3))) void lds_void_t;



// U bytes per lane from rsrc at (voff + soff) into LDS at lds + 16*lane
// (lds must be the same in every lane of the wavefront).
template <int U>
__device__ __forceinline__ void dma_lds(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff,
                                        uint32_t soff) {
  static_assert(U == 4 || U == 16, "DMA unit");
  if constexpr (U == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, (int)voff, (int)soff, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 4, (int)voff, (int)soff, 0, 0);
}

// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt low bits 3:0, high bits 15:14;
// expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt vmcnt(N) lgkmcnt(0), then s_barrier. No memory fence: a fence
// would also wait for every LDS-DMA copy in flight (they count as pending LDS
// writes), which is exactly what the ring is meant to keep going. The empty
// asm statements keep the compiler from moving memory accesses across.
template <int N>
__device__ __forceinline__ void wait_vmcnt_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt lgkmcnt(0), then s_barrier (see wait_vmcnt_barrier)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((15 & 15) | (3 << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// empty asm that "uses" a value: keeps its computation in the current block
// (the compiler would otherwise sink the next step's dequantization past the
// copy-issue branches of that step, out of the MFMA shadow)
__device__ __forceinline__ void keep(const uint4& v) {
  asm volatile("" ::"v"(v.x), "v"(v.y), "v"(v.z), "v"(v.w));
}

constexpr int kStageSteps = 8;      // K steps per scale stage (512 codes)

template <int BM, int BN, int BITS, int KW, int SL, bool WU4 = false>
struct DmaGeo {
  // SL output slices, KW wavefronts per slice (each taking 1/KW of the codes
  // of every K step): SL*KW wavefronts
  static constexpr int NW = SL * KW, NT = 64 * NW;
  // slice grid (each W chunk is dequantized by exactly one wavefront):
  //  SL = 4: 1 x 4 slices of 128-wide tiles, 2 x 2 for 64 x 64 tiles;
  //  SL = 2: 1 x 2 slices (each 64 columns wide), so that every x fragment
  //  read from LDS feeds two MFMAs and the tile's x reads are halved
  static constexpr int WAVES_N = SL == 2 ? 2 : (BN >= 128 ? 4 : 2), WAVES_M = SL / WAVES_N;
  static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int A_ELEMS = BM * 64;          // x tile of one step
  static constexpr int A_BLOCKS = BM / 8;          // 8 rows per DMA instruction
  static constexpr int A_PER_WAVE = A_BLOCKS / NW;
  // W copy unit: 4 bytes when each lane must pick its own word (WU4: rows
  // interleaved in memory)
  static constexpr int WU = (!WU4 && (BITS == 8 || (BITS == 4 && BN == 128))) ? 16 : 4;
  static constexpr int W_ROW = 8 * BITS;           // bytes per W row and step
  static constexpr int W_BYTES = BN * W_ROW;
  static constexpr int UPR = W_ROW / WU;           // DMA units per W row
  static constexpr int W_BLOCKS = W_BYTES / WU / 64;
  static constexpr int W_HI = (W_BLOCKS + NW - 1) / NW;  // W instructions of wave 0
  static constexpr int W_LO = W_BLOCKS / NW;             // ... of the last wave
  static constexpr int SWZ = WU == 16 ? ilog2(16 / UPR) : 0;
  static_assert(A_BLOCKS % NW == 0 && W_BYTES % (64 * WU) == 0, "DMA blocks");
};

// f16 constants of a chunk for every field offset o: s*2^-o and b - 1024*s*2^-o
struct F16Consts {
  float so[8], co[8];
};
__device__ __forceinline__ void f16_consts(float s, float b, F16Consts& c) {
#pragma unroll
  for (int o = 0; o < 8; o++) {
    c.so[o] = s * __builtin_bit_cast(float, (uint32_t)(127 - o) << 23);
    c.co[o] = fmaf(-1024.0f, c.so[o], b);
  }
}

// codes [C0, C0+PC) of a chunk -> f16 pairs out[C0/2 .. (C0+PC)/2)
template <int BITS, int C0, int PC>
__device__ __forceinline__ void dequant_piece_f16(const uint32_t* w, const F16Consts& c,
                                                  uint32_t m2, uint32_t magic,
                                                  uint32_t* out) {
  uint32_t pr[16];
  [&]<int... P>(std::integer_sequence<int, P...>) QMM_INLINE {
    ([&]() QMM_INLINE {
       if constexpr (piece_has_pair<BITS, C0, PC>(P))
         pr[P] = magic_pair<F16, BITS, P>(w, m2, magic);
       else
         pr[P] = 0;
     }(),
     ...);
  }(std::make_integer_sequence<int, 16>{});
#pragma unroll
  for (int k = C0; k < C0 + PC; k += 2) {
    float v[2];
#pragma unroll
    for (int e = 0; e < 2; e++) {
      const int kk = k + e;
      const int p = pair_index<BITS>(kk), hf = pair_half<BITS>(kk);
      const int o = pair_off<F16, BITS>(kk);
      const float q = (float)__builtin_bit_cast(half2_t, pr[p])[hf];
      v[e] = fmaf(q, c.so[o], c.co[o]);
    }
    const half2_t hv = {(_Float16)v[0], (_Float16)v[1]};
    out[k / 2] = __builtin_bit_cast(uint32_t, hv);
  }
}

// slot (MFMA index) after which filler f of nf is emitted: the first kLead
// MFMAs cover the latency of the LDS reads, the fillers are spread evenly
// over the rest
constexpr int filler_slot(int f, int nf, int nm, int lead) {
  return lead + (f * (nm - lead)) / nf;
}

// CONV: 0 plain GEMM; 1 convolution, x pieces addressed through a k table in
// LDS; 2 convolution whose per-group channel count is a multiple of 64, so
// that the 64 codes of a K step lie in one tap and every piece of the step
// is addressed from the step's tap and channel (no table, no LDS read).
// KW = 2: two wavefronts per output slice (8 per workgroup, two per SIMD, so
// that one wavefront's MFMAs run while the other issues its dequantization
// and copies); wavefront w + 4 takes the upper 16 codes of each lane's
// 32-code chunk (MFMA slices 2 and 3 of the step), w the lower 16, and the
// pair's accumulators are added once, through LDS, after the last step.
//
// FPM != 0: a floating-point mode ("mlx 1.0.0 backend/cpu/quantized.cpp",
// fp_qmm_t): 1 mxfp4 (E2M1 codes, one e8m0 scale byte per 32), 2 nvfp4 (E2M1,
// one E4M3 scale byte per 16), 3 mxfp8 (E4M3 codes, e8m0 per 32); no bias.
// The scale rounded to T times a code is exact in T whenever it lies in T's
// range, so W reaches the MFMA as T values (no bf16 hi/lo split): for e8m0
// scales one scaled conversion per code pair (v_cvt_scalef32_pk_*, which
// applies a power-of-two scale exactly), for E4M3 scales the conversion at
// scale 1 and an fp32 product rounded to T.
//
// APK != 0: the affine-packed layout ("Add the 3bit packed qmm_t", ops.cpp
// quantize with AffinePacked): scales and biases in one array, rows in
// blocks of APK (4 for power-of-two bits, 2 otherwise), per block and group
// the APK scales then the APK biases; with APK = 4 the block's weight words
// are interleaved too (word w of row 4i + r at word 4w + r of packed row i),
// and the W copies use 4-byte units so that each lane fetches one row's word
// and the slot gets the plain row layout.
template <class T, int BITS, int BM, int BN, int CONV, int KW, int SL, int FPM, int APK = 0>
__global__ __launch_bounds__(64 * SL * KW) void qmm_dma_kernel(GemmArgs a) {
  using G = DmaGeo<BM, BN, BITS, KW, SL, APK == 4>;
  constexpr int NW = G::NW, NT = G::NT;
  constexpr bool kFp = FPM != 0;
  constexpr bool kSplit = !kFp && __is_same(T, BF16);
  constexpr int ES = kFp ? 1 : 2;                // bytes per scale element
  constexpr int kSgMax = FPM == 2 ? 32 : 16;     // groups per 512-code stage, at most
  constexpr int NB = kSplit ? 2 : 1;
  constexpr int FM = G::FM, FN = G::FN, WTM = G::WTM, WTN = G::WTN;
  constexpr int WU = G::WU, UPR = G::UPR;
  constexpr int KK = 4 / KW;                     // MFMA K slices per wavefront and step
  constexpr int CW = 32 / KW;                    // codes of a lane's chunk per wavefront
  constexpr int PC = (kSplit || kFp) ? 8 : piece_codes<BITS>();
  constexpr int NP = CW / PC;                    // pieces per wavefront and chunk
  constexpr int kM = KK * FM * FN * NB;          // MFMAs per step
  // x fragments: with several row blocks per wavefront and all four slices
  // (kJit) slice kk+2 is read while the MFMAs of slice kk run; otherwise the
  // next step's fragments are read during the current step (two buffers)
  constexpr bool kJit = KW == 1 && FM >= 2;
  constexpr int kNF = FN + FN * NP + (kJit ? 0 : KK * FM);  // fillers per step
  constexpr int kLead = kM >= 16 ? 4 : 1;
  static_assert(KW == 1 || KW == 2, "one or two wavefronts per slice");

  // one LDS array per ring slot (x tile, then W tile): the compiler tracks
  // pending LDS-DMA writes per array for a handful of arrays only
  constexpr int kSlotBytes = G::A_ELEMS * 2 + G::W_BYTES;
  __shared__ __attribute__((aligned(16))) uint8_t sl0[kSlotBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sl1[kSlotBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sl2[kSlotBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sl3[kSlotBytes];
  __shared__ uint32_t sct[2 * BN * (kSgMax + 1)];
  __shared__ uint32_t ktab[CONV == 1 ? kKtabMax : 1];
  // target of the filler W copies of wavefronts with one block fewer
  __shared__ __attribute__((aligned(16))) uint8_t wjunk[G::W_BLOCKS % NW ? 64 * WU : 16];

  auto slot = [&]<int S>() -> uint8_t* QMM_INLINE {
    if constexpr (S == 0) return sl0;
    else if constexpr (S == 1) return sl1;
    else if constexpr (S == 2) return sl2;
    else return sl3;
  };
  auto xslot = [&]<int S>() -> uint16_t* QMM_INLINE {
    return reinterpret_cast<uint16_t*>(slot.template operator()<S>());
  };
  auto wslot = [&]<int S>() -> uint8_t* QMM_INLINE {
    return slot.template operator()<S>() + G::A_ELEMS * 2;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63, h = lane >> 5, rr = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int w4 = wave & (SL - 1);                 // output slice
  const int kh = KW == 2 ? wave / SL : 0;         // part of each chunk
  const int wm = w4 / G::WAVES_N, wn = w4 % G::WAVES_N;
  // LDS ring slot k (for the end-of-kernel staging: each slice owns 4/SL)
  auto slot_at = [&](int k) -> uint8_t* QMM_INLINE {
    return k == 0 ? sl0 : k == 1 ? sl1 : k == 2 ? sl2 : sl3;
  };
  // blockIdx.z: the conv group, or the batch of a batched plain GEMM (x, W,
  // scales, biases and y of batch g follow those of batch g - 1; a gathered
  // GEMM takes x and W from the batches its index arrays name)
  const int g = blockIdx.z;
  int tile = blockIdx.x;
  {
    // workgroup i runs on XCD i % 8: give each XCD a contiguous band of tiles
    const int nt = gridDim.x;
    if ((nt & 7) == 0) tile = (tile & 7) * (nt >> 3) + (tile >> 3);
  }
  const int tiles_n = (a.N + BN - 1) / BN;
  const int m_blk = (tile / tiles_n) * BM, n_blk = (tile % tiles_n) * BN;

  const int K = a.K;                       // W row length in codes
  const int nk = (K + 63) >> 6;            // K steps
  const int sk = blockIdx.y;               // K split
  const int t0 = sk * a.ksteps;            // first step (a multiple of 8)
  const int t1 = t0 + a.ksteps < nk ? t0 + a.ksteps : nk;
  const int row_bytes = K / 8 * BITS;
  const int n_groups = K >> a.gs_log2;
  const uint8_t* wq = a.wq;
  const char* sp = reinterpret_cast<const char*>(a.s);   // ES bytes per element
  const char* bp = reinterpret_cast<const char*>(a.b);
  int gx = g;   // x batch of a batched GEMM
  if constexpr (CONV) {
    wq += (int64_t)g * a.Og * row_bytes;
    sp += (int64_t)g * a.Og * n_groups * ES;
    bp += (int64_t)g * a.Og * n_groups * ES;
  } else {
    int gw = g;
    if (a.lidx) {
      const int v = a.lidx[g];
      gx = v < 0 ? 0 : (v >= a.nxb ? a.nxb - 1 : v);
    }
    if (a.ridx) {
      const int v = a.ridx[g];
      gw = v < 0 ? 0 : (v >= a.nwb ? a.nwb - 1 : v);
    }
    wq += (int64_t)gw * a.N * row_bytes;
    sp += (int64_t)gw * a.N * n_groups * ES;
    bp += (int64_t)gw * a.N * n_groups * ES;
  }

  uint32_t magic_v;
  const uint32_t m2_s = Pack<BITS>::kMask | (Pack<BITS>::kMask << 16);
  asm volatile("v_mov_b32 %0, %1" : "=v"(magic_v) : "s"(a.magic));

  // ---- conv: k-unit table (dy, dx, channel) of every 8-channel unit
  if constexpr (CONV == 1) {
    for (int ku = tid; ku < nk * 8; ku += 256) {
      const int k = ku * 8;
      uint32_t e = 0xffffffffu;
      if (k < a.K_true) {
        const int tap = k / a.Cg, c0 = k - tap * a.Cg;
        const int dy = tap / a.kw, dx = tap - dy * a.kw;
        e = ((uint32_t)dy << 24) | ((uint32_t)dx << 16) | (uint32_t)c0;
      }
      ktab[ku] = e;
    }
    __syncthreads();
  }

  // ---- x pieces: instruction i of this wavefront fills rows 8*blk..+7 of a
  // slot, lane -> (row, position); the unit fetched is position ^ swizzle.
  // Plain GEMM: byte offset from the tile's first row (rows past M re-read
  // row M-1; their results are not stored). Conv: offsets from channel g*Cg
  // of the image, computed per step from the k table.
  const char* xbase = reinterpret_cast<const char*>(a.x) +
                      (CONV ? (int64_t)g * a.Cg * 2 : ((int64_t)gx * a.M + m_blk) * a.K * 2);
  const int64_t x_bytes =
      CONV ? (int64_t)(a.M / (a.OH * a.OW)) * a.H * a.W * a.C * 2 - (int64_t)g * a.Cg * 2
           : (int64_t)(a.M - m_blk) * a.K * 2;
  const __amdgpu_buffer_rsrc_t xr =
      make_rsrc(xbase, (uint32_t)(x_bytes < 0x7fffffff ? x_bytes : 0x7fffffff));
  uint32_t xoff[G::A_PER_WAVE];
  int xcol[G::A_PER_WAVE];
  int pix_b[CONV ? G::A_PER_WAVE : 1], pix_y[CONV ? G::A_PER_WAVE : 1],
      pix_x[CONV ? G::A_PER_WAVE : 1];
  // CONV == 2: element offset of the piece at tap (0, 0) of the row's output
  // pixel, modulo 2^32 (it may lie outside the image: only taps inside it
  // are read, and for those the sum below is the true offset)
  uint32_t pix_o[CONV == 2 ? G::A_PER_WAVE : 1];
#pragma unroll
  for (int i = 0; i < G::A_PER_WAVE; i++) {
    const int blk = NW * i + wave;
    const int r = 8 * blk + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    xcol[i] = 8 * c;
    const int m = m_blk + r;
    if constexpr (!CONV) {
      const int rc = m < a.M ? r : a.M - 1 - m_blk;
      xoff[i] = (uint32_t)(((int64_t)rc * a.K + 8 * c) * 2);
    } else {
      const int mm = m < a.M ? m : 0;
      const int b = mm / (a.OH * a.OW), rem = mm - b * a.OH * a.OW;
      const int oy = rem / a.OW, ox = rem - oy * a.OW;
      pix_b[i] = b * a.H;
      // rows past M get an impossible y so that every tap reads zeros
      pix_y[i] = m < a.M ? oy * a.sh - a.ph : -(1 << 28);
      pix_x[i] = ox * a.sw - a.pw;
      if constexpr (CONV == 2)
        pix_o[i] = (((uint32_t)pix_b[i] + (uint32_t)pix_y[i]) * (uint32_t)a.W +
                    (uint32_t)pix_x[i]) * (uint32_t)a.C + (uint32_t)xcol[i];
      xoff[i] = 0;
    }
  }

  // ---- W pieces: lane -> (row, unit) of a W slot; byte offset from the
  // tile's first row (rows past N re-read row N-1)
  const char* wbase = reinterpret_cast<const char*>(wq) + (int64_t)n_blk * row_bytes;
  const int64_t w_bytes = (int64_t)(a.N - n_blk) * row_bytes;
  const __amdgpu_buffer_rsrc_t wr =
      make_rsrc(wbase, (uint32_t)(w_bytes < 0x7fffffff ? w_bytes : 0x7fffffff));
  uint32_t woff[G::W_HI];
  int wuo[G::W_HI];
#pragma unroll
  for (int i = 0; i < G::W_HI; i++) {
    const int blk = NW * i + wave;
    const int ui = 64 * (blk < G::W_BLOCKS ? blk : 0) + lane;
    const int r = ui / UPR, p = ui % UPR;
    const int u = WU == 16 ? (p ^ ((r >> G::SWZ) & (UPR - 1))) : p;
    const int rc = n_blk + r < a.N ? r : a.N - 1 - n_blk;
    wuo[i] = WU * u;
    if constexpr (APK == 4)   // word u of row rc: word 4u + rc % 4 of packed row rc / 4
      woff[i] = (uint32_t)(rc >> 2) * (uint32_t)(4 * row_bytes) + (uint32_t)(4 * (4 * u + (rc & 3)));
    else
      woff[i] = (uint32_t)rc * (uint32_t)row_bytes + (uint32_t)(WU * u);
  }

  // ---- issue the copies of step tt into slot S. Pieces past the end of a
  // row (and whole steps past the end of K) get an out-of-range offset and
  // land as zeros; every wavefront issues the same number of copies every
  // step (those without a W block of their own copy zeros into wjunk), so one
  // vmcnt value fits all. No branches: a stage of steps stays one block.
  constexpr int kDma = G::A_PER_WAVE + G::W_HI;   // copies per step and wavefront
  // CHK = false: the caller guarantees that step tt lies inside K (whole
  // 64-code steps), so the copies skip the range checks (plain GEMM)
  auto issue_one = [&]<int S, int D, bool CHK>(int tt) QMM_INLINE {
    if constexpr (D < G::A_PER_WAVE) {
      constexpr int i = D;
      const int blk = NW * i + wave;
      uint16_t* xd = xslot.template operator()<S>() + blk * 512;
      if constexpr (CONV == 2) {
        // the step's 64 codes are channels [c0, c0 + 64) of tap (dy, dx)
        const int k0 = 64 * tt;
        const int tap = a.cu_mul ? (int)__umulhi((uint32_t)tt, a.cu_mul) : tt;
        const int c0 = k0 - 64 * tap * a.cu;
        const int dy = a.kw_mul ? (int)__umulhi((uint32_t)tap, a.kw_mul) : tap;
        const int dx = tap - dy * a.kw;
        const uint32_t dstep = (uint32_t)((dy * a.W + dx) * a.C + c0);   // uniform
        const int iy = pix_y[i] + dy, ix = pix_x[i] + dx;
        const bool in = k0 < a.K_true && (unsigned)iy < (unsigned)a.H &&
                        (unsigned)ix < (unsigned)a.W;
        dma_lds<16>(xr, xd, in ? (pix_o[i] + dstep) * 2u : kOob, 0);
      } else if constexpr (CONV) {
        const int ku = 8 * tt + (xcol[i] >> 3);
        const uint32_t e = ku < nk * 8 ? ktab[ku] : 0xffffffffu;
        const int dy = (int)(e >> 24), dx = (int)((e >> 16) & 0xff);
        const int iy = pix_y[i] + dy, ix = pix_x[i] + dx;
        const bool in = e != 0xffffffffu && (unsigned)iy < (unsigned)a.H &&
                        (unsigned)ix < (unsigned)a.W;
        const uint32_t off =
            (uint32_t)((((pix_b[i] + iy) * a.W + ix) * a.C + (int)(e & 0xffff)) * 2);
        dma_lds<16>(xr, xd, in ? off : kOob, 0);
      } else if constexpr (CHK) {
        const bool ok = 64 * tt + xcol[i] < K;
        dma_lds<16>(xr, xd, ok ? xoff[i] : kOob, 128u * tt);
      } else {
        dma_lds<16>(xr, xd, xoff[i], 128u * tt);
      }
    } else {
      constexpr int i = D - G::A_PER_WAVE;
      uint8_t* wd = wslot.template operator()<S>();
      const uint32_t wsoff = (uint32_t)(8 * BITS) * tt;   // byte of the step in a row
      const int blk = NW * i + wave;
      const bool real = G::W_BLOCKS % NW == 0 || blk < G::W_BLOCKS;
      bool ok = real;
      if constexpr (CHK) ok = ok && (int)wsoff + wuo[i] < row_bytes;
      // (interleaved rows: the step's words of a packed row start 4x further)
      dma_lds<WU>(wr, real ? (void*)(wd + blk * 64 * WU) : (void*)wjunk, ok ? woff[i] : kOob,
                  APK == 4 ? 4 * wsoff : wsoff);
    }
  };
  auto issue = [&]<int S>(int tt) QMM_INLINE {
    [&]<int... D>(std::integer_sequence<int, D...>) QMM_INLINE {
      (issue_one.template operator()<S, D, true>(tt), ...);
    }(std::make_integer_sequence<int, kDma>{});
  };
  // end of a step: wait until only the youngest step of copies is in flight,
  // then barrier
  // (in steps 1 and 2 of a stage the scale loads issued after step 1's copies
  // may stay in flight too; they must land by the end of step 3)
  auto step_sync = [&]<int U>() QMM_INLINE {
    constexpr int kSLoads = (kFp ? 1 : 2) * (BN * kSgMax / NT);
    wait_vmcnt<G::A_PER_WAVE + G::W_HI + ((U == 1 || U == 2) ? kSLoads : 0)>();
    lds_barrier();
  };

  // ---- scales and biases, in stages of 8 steps
  const int sg_log2 = 9 - a.gs_log2;          // groups per stage: 4, 8 or 16
  const int SG = 1 << sg_log2, SGP = SG + 1;
  // Each thread loads kSL scales and kSL biases per stage (element e =
  // thread + NT i modulo BN*SG: group e % SG of tile row e / SG; repeats
  // rewrite the same value) through buffer resources over the tile's rows, at
  // loop-invariant lane offsets plus a per-stage scalar offset. Groups past
  // the end of a row read the next row (or zeros): they only meet zero x.
  constexpr int kSL = BN * kSgMax / NT;
  // (packed: the tile's rows start at packed row n_blk / APK, whose 2 * APK
  // values per group make the same 2 * n_groups values per row)
  const char* sbase = sp + (int64_t)n_blk * n_groups * ES * (APK ? 2 : 1);
  const char* bbase = (kFp || APK) ? sbase : bp + (int64_t)n_blk * n_groups * ES;
  const int64_t s_bytes = (int64_t)(a.N - n_blk) * n_groups * ES * (APK ? 2 : 1);
  const uint32_t s_rb = (uint32_t)(s_bytes < 0x7fffffff ? s_bytes : 0x7fffffff);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(sbase, s_rb), br = make_rsrc(bbase, s_rb);
  uint32_t soffv[kSL], soffb[kSL];
  int sdst[kSL];
#pragma unroll
  for (int i = 0; i < kSL; i++) {
    const int e = (tid + NT * i) & (BN * SG - 1);
    const int grp = e & (SG - 1), row = e >> sg_log2;
    const int rc = n_blk + row < a.N ? row : a.N - 1 - n_blk;
    if constexpr (APK) {
      const int es = ((rc / APK) * n_groups + grp) * 2 * APK + rc % APK;
      soffv[i] = (uint32_t)(es * 2);
      soffb[i] = (uint32_t)((es + APK) * 2);
    } else {
      soffv[i] = (uint32_t)((rc * n_groups + grp) * ES);
      soffb[i] = soffv[i];
    }
    sdst[i] = row * SGP + grp;
  }
  uint32_t sreg[kSL], breg[kSL];
  constexpr int kSGrp = kSL >= 4 ? 4 : kSL;          // loads of a group (each array)
  auto scale_load_grp = [&]<int GR>(int j) QMM_INLINE {
    const uint32_t so = (uint32_t)(j * SG * ES * (APK ? 2 * APK : 1));
#pragma unroll
    for (int i = GR * kSGrp; i < (GR + 1) * kSGrp; i++) {
      if constexpr (kFp) {
        sreg[i] = __builtin_amdgcn_raw_buffer_load_b8(sr, soffv[i], so, 0);
      } else {
        sreg[i] = __builtin_amdgcn_raw_buffer_load_b16(sr, soffv[i], so, 0);
        breg[i] = __builtin_amdgcn_raw_buffer_load_b16(br, soffb[i], so, 0);
      }
    }
  };
  auto scale_load = [&](int j) QMM_INLINE {
    [&]<int... GR>(std::integer_sequence<int, GR...>) QMM_INLINE {
      (scale_load_grp.template operator()<GR>(j), ...);
    }(std::make_integer_sequence<int, kSL / kSGrp>{});
  };
  // affine: (scale | bias << 16) words; fp modes: the scale rounded to T,
  // as fp32 bits
  auto scale_store = [&](int j) QMM_INLINE {
    if constexpr (kFp) {
      uint32_t* base = sct + (j & 1) * BN * SGP;
#pragma unroll
      for (int i = 0; i < kSL; i++) base[sdst[i]] = fp_scale_t_bits<T, FPM>(sreg[i]);
    } else {
      uint16_t* base = reinterpret_cast<uint16_t*>(sct + (j & 1) * BN * SGP);
#pragma unroll
      for (int i = 0; i < kSL; i++) {
        base[2 * sdst[i]] = (uint16_t)sreg[i];
        base[2 * sdst[i] + 1] = (uint16_t)breg[i];
      }
    }
  };

  // ---- per-step register state (x fragments: see kJit)
  uint4 af[kJit ? 1 : 2][KK][FM];
  uint4 bq[2][FN][NB][KK];       // W operands (row block, hi/lo, K slice)
  uint32_t wc[FN][BITS];         // raw W chunk part of the next step
  uint32_t wfull[KW == 2 ? FN : 1][BITS];   // KW = 2: the whole chunk, as read
  uint32_t sbw[FN];              // (scale | bias << 16) of the next step
  uint32_t s2v[FN], b2v[FN];      // f16 scale / bias in both halves
  float sf[FN], bf[FN];           // bf16 path: scale / bias in fp32
  // fp modes: the scale of the wavefront's codes, and with groups of 16 and
  // one wavefront per slice the scale of the chunk's second group
  constexpr bool kTwoGroups = FPM == 2 && KW == 1;
  uint32_t sbw2[kTwoGroups ? FN : 1];
  float sfp[FN], sfp2[kTwoGroups ? FN : 1];

  // W chunks and scale words of step tt from slot S
  auto read_w = [&]<int S>(int tt) QMM_INLINE {
    const uint8_t* wsl = wslot.template operator()<S>();
    const uint32_t* scs = sct + ((tt >> 3) & 1) * BN * SGP;
    // group of the wavefront's first code (groups of 16 split a chunk)
    const int gl = (((tt & 7) << 6) + 32 * h + CW * kh) >> a.gs_log2;
#pragma unroll
    for (int j = 0; j < FN; j++) sbw[j] = scs[(wn * WTN + 32 * j + rr) * SGP + gl];
    if constexpr (kTwoGroups) {
#pragma unroll
      for (int j = 0; j < FN; j++) sbw2[j] = scs[(wn * WTN + 32 * j + rr) * SGP + gl + 1];
    }
#pragma unroll
    for (int j = 0; j < FN; j++) {
      const int r = wn * WTN + 32 * j + rr;
      // (vector-typed 16-byte loads: a load split into words and merged again
      // loses the information that it reads this slot only, and the compiler
      // then waits for every LDS copy in flight)
      uint32_t full[BITS];
      if constexpr (WU == 16 && BITS == 4) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(
            wsl + r * 32 + 16 * (h ^ ((r >> G::SWZ) & 1)));
#pragma unroll
        for (int q = 0; q < 4; q++) full[q] = v[q];
      } else if constexpr (WU == 16 && BITS == 8) {
#pragma unroll
        for (int e = 0; e < 2; e++) {
          const int u = (2 * h + e) ^ ((r >> G::SWZ) & 3);
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(wsl + r * 64 + 16 * u);
#pragma unroll
          for (int q = 0; q < 4; q++) full[4 * e + q] = v[q];
        }
      } else {
        const uint32_t* pw =
            reinterpret_cast<const uint32_t*>(wsl + r * (8 * BITS) + 4 * BITS * h);
#pragma unroll
        for (int q = 0; q < BITS; q++) full[q] = pw[q];
      }
#pragma unroll
      for (int q = 0; q < BITS; q++) {
        if constexpr (KW == 1) wc[j][q] = full[q];
        else wfull[j][q] = full[q];
      }
    }
  };
  // KW = 2: the wavefront's 16 codes of chunk J as codes 0..15 of a chunk
  // (the upper half starts at byte 2*BITS, a whole pack boundary for every
  // width, so the magic pairs of either half stay inside it). Done in the
  // step's first filler, so that the wait for the chunk's LDS read does not
  // hold up the step's first MFMA.
  auto take_part = [&]<int J>() QMM_INLINE {
    if constexpr (KW == 2) {
      constexpr int SB = 2 * BITS, NWD = (SB + 3) / 4;
      const uint32_t* full = wfull[J];
#pragma unroll
      for (int q = 0; q < BITS; q++) wc[J][q] = 0;
      [&]<int... Q>(std::integer_sequence<int, Q...>) QMM_INLINE {
        ([&]() QMM_INLINE {
           constexpr int b = SB + 4 * Q, iq = b / 4, sh = 8 * (b % 4);
           uint32_t up;
           if constexpr (sh == 0) up = full[iq];
           else up = __builtin_amdgcn_alignbit(iq + 1 < BITS ? full[iq + 1] : 0u, full[iq], sh);
           wc[J][Q] = kh ? up : full[Q];
         }(),
         ...);
      }(std::make_integer_sequence<int, NWD>{});
    }
  };
  // x fragment (the wavefront's K slice L, row block I) of slot S: slice
  // KK*kh + L of the step
  auto read_x = [&]<int S, int L, int I>(uint4 (&afr)[KK][FM]) QMM_INLINE {
    const uint16_t* xsl = xslot.template operator()<S>();
    const int ra = wm * WTM + 32 * I + rr;
    const int c = (4 * h + KK * kh + L) ^ ((ra >> 1) & 7);
    afr[L][I] = *reinterpret_cast<const uint4*>(xsl + ra * 64 + 8 * c);
  };
  auto prep = [&]<int J>() QMM_INLINE {
    take_part.template operator()<J>();
    if constexpr (kFp) {
      sfp[J] = __builtin_bit_cast(float, sbw[J]);
      if constexpr (kTwoGroups) sfp2[J] = __builtin_bit_cast(float, sbw2[J]);
    } else if constexpr (kSplit) {
      sf[J] = to_f32(T{}, (uint16_t)sbw[J]);
      bf[J] = to_f32(T{}, (uint16_t)(sbw[J] >> 16));
    } else {
      s2v[J] = __builtin_amdgcn_perm(sbw[J], sbw[J], 0x01000100u);
      b2v[J] = __builtin_amdgcn_perm(sbw[J], sbw[J], 0x03020302u);
    }
  };
  auto piece = [&]<int J, int P>(uint4 (&bqn)[FN][NB][KK]) QMM_INLINE {
    uint32_t hi[16], lo[16];
    if constexpr (kFp) {
      // codes [8P, 8P + 8) of the wavefront's part: slice P
      float sc = sfp[J];
      if constexpr (kTwoGroups) sc = P >= 2 ? sfp2[J] : sfp[J];
      uint32_t pr[4];
      fp_piece<T, FPM>(wc[J] + P * BITS / 4, sc, pr);
      bqn[J][0][P] = make_uint4(pr[0], pr[1], pr[2], pr[3]);
    } else if constexpr (kSplit) {
      dequant_piece_bf16<BITS, P * 8>(wc[J], sf[J], bf[J], hi, lo);
      bqn[J][1][P] = make_uint4(lo[4 * P], lo[4 * P + 1], lo[4 * P + 2], lo[4 * P + 3]);
      bqn[J][0][P] = make_uint4(hi[4 * P], hi[4 * P + 1], hi[4 * P + 2], hi[4 * P + 3]);
    } else {
      dequant_piece_f16_pk<BITS, P * PC, PC>(wc[J], s2v[J], b2v[J], m2_s, magic_v, hi);
#pragma unroll
      for (int kk = P * PC / 8; kk < (P + 1) * PC / 8; kk++)
        bqn[J][0][kk] = make_uint4(hi[4 * kk], hi[4 * kk + 1], hi[4 * kk + 2], hi[4 * kk + 3]);
    }
  };
  // filler F of a step: scale prep, a dequant piece, or (without kJit) an x
  // fragment read of the next step (slot SN)
  auto filler = [&]<int F, int SN>(uint4 (&afn)[KK][FM], uint4 (&bqn)[FN][NB][KK]) QMM_INLINE {
    if constexpr (F < FN) {
      prep.template operator()<F>();
    } else if constexpr (F < FN + FN * NP) {
      constexpr int idx = F - FN;
      piece.template operator()<idx % FN, idx / FN>(bqn);
    } else {
      constexpr int idx = F - FN - FN * NP;
      read_x.template operator()<SN, idx / FM, idx % FM>(afn);
    }
  };

  float16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; i++)
#pragma unroll
    for (int j = 0; j < FN; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

  // fillers of MFMA slot MM (next step's state goes to bq[1-C] and, without
  // kJit, af[1-C], from slot SN)
  auto slot_fill = [&]<int MM, int C, int SN>() QMM_INLINE {
    [&]<int... F>(std::integer_sequence<int, F...>) QMM_INLINE {
      ([&]() QMM_INLINE {
         if constexpr (filler_slot(F, kNF, kM, kLead) == MM) {
           filler.template operator()<F, SN>(af[kJit ? 0 : 1 - C], bq[1 - C]);
           __builtin_amdgcn_sched_barrier(0);
         }
       }(),
       ...);
    }(std::make_integer_sequence<int, kNF>{});
  };
  constexpr int kSlice = FM * FN * NB;       // MFMAs per K slice
  auto read_slice = [&]<int S, int KS>() QMM_INLINE {
    [&]<int... I>(std::integer_sequence<int, I...>) QMM_INLINE {
      (read_x.template operator()<S, KS, I>(af[0]), ...);
    }(std::make_integer_sequence<int, FM>{});
  };
  auto mfma_at = [&]<int MM, int C, int SC, int SN>() QMM_INLINE {
    constexpr int kk = MM / kSlice;
    constexpr int i = (MM / (FN * NB)) % FM;
    constexpr int j = (MM / NB) % FN;
    constexpr int e = MM % NB;
    acc[i][j] = mfma32(T{}, af[kJit ? 0 : C][kk][i], bq[C][j][e][kk], acc[i][j]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kJit && MM % kSlice == 0) {
      // x fragments two slices ahead (slices 0 and 1 of the next step during
      // slices 2 and 3): ax[kk+2] was last used in slice kk+2 of the previous
      // step
      if constexpr (kk < 2) read_slice.template operator()<SC, kk + 2>();
      else read_slice.template operator()<SN, kk - 2>();
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // copies of step tt+3 (slot SD) and, in step 1 of a stage, the scale loads
  // of the next stage, spread over the MFMA slots (a burst of copies would
  // stall on the address unit): copy d after MFMA 2d, the scale groups after
  // the last copy (the end-of-step vmcnt values count on that order)
  constexpr int kNGrp = kSL / kSGrp;
  auto extras = [&]<int MM, int SD, bool kScales, bool CHK>(int tt, int js) QMM_INLINE {
    [&]<int... D>(std::integer_sequence<int, D...>) QMM_INLINE {
      ([&]() QMM_INLINE {
         constexpr int slot = 2 * D < kM ? 2 * D : kM - 1;
         if constexpr (slot == MM) {
           issue_one.template operator()<SD, D, CHK>(tt + 3);
           __builtin_amdgcn_sched_barrier(0);
         }
       }(),
       ...);
    }(std::make_integer_sequence<int, kDma>{});
    if constexpr (kScales) {
      [&]<int... GR>(std::integer_sequence<int, GR...>) QMM_INLINE {
        ([&]() QMM_INLINE {
           constexpr int last = 2 * (kDma - 1) < kM ? 2 * (kDma - 1) : kM - 1;
           constexpr int slot = last + 1 + GR < kM ? last + 1 + GR : kM - 1;
           if constexpr (slot == MM) {
             scale_load_grp.template operator()<GR>(js + 1);
             __builtin_amdgcn_sched_barrier(0);
           }
         }(),
         ...);
      }(std::make_integer_sequence<int, kNGrp>{});
    }
  };

  // one step body: MFMAs from af/bq[C] (x slot SC); the next step's state
  // (slot SN) is built between them, in a fixed order, with the copies of
  // step tt+3 (slot SD)
  auto body = [&]<int C, int SC, int SN, int SD, bool kScales, bool CHK>(int tt,
                                                                         int js) QMM_INLINE {
    read_w.template operator()<SN>(tt + 1);
    __builtin_amdgcn_sched_barrier(0);
    [&]<int... M>(std::integer_sequence<int, M...>) QMM_INLINE {
      ((mfma_at.template operator()<M, C, SC, SN>(),
        extras.template operator()<M, SD, kScales, CHK>(tt, js),
        slot_fill.template operator()<M, C, SN>()),
       ...);
    }(std::make_integer_sequence<int, kM>{});
  };

  // ---- prologue: scales of stage 0, copies of steps 0..2, state of step 0
  const int js0 = t0 / kStageSteps;
  scale_load(js0);
  issue.template operator()<0>(t0);
  issue.template operator()<1>(t0 + 1);
  issue.template operator()<2>(t0 + 2);
  // the stage's scales and steps 0 and 1 (step 0's body builds step 1's
  // state from its slot); step 2 stays in flight, and the first step's end
  // waits for it
  wait_vmcnt<kDma>();
  scale_store(js0);
  wait_vmcnt_barrier<kDma>();
  read_w.template operator()<0>(t0);
  [&]<int... F>(std::integer_sequence<int, F...>) QMM_INLINE {
    (filler.template operator()<F, 0>(af[0], bq[0]), ...);
  }(std::make_integer_sequence<int, kNF>{});
  if constexpr (kJit) {
    read_slice.template operator()<0, 0>();
    read_slice.template operator()<0, 1>();
  }

  // every LDS read of the prologue has landed before the loop (so that the
  // compiler does not carry them into the loop body)
  __builtin_amdgcn_s_waitcnt((15 & 15) | (3 << 14) | (7 << 4));

  // ---- main loop: stages of 8 steps. Step tt multiplies from bq[tt % 2]
  // (built from slot tt % 4 during step tt-1) and builds bq[(tt+1) % 2] from
  // slot (tt+1) % 4; the copies of step tt+3 go to slot (tt+3) % 4, whose
  // last reads were made during step tt-2. Full stages run unguarded; only a
  // last partial stage checks each step against nk. Stages whose copies
  // (steps up to 8 js + 10) all lie inside K skip the copies' range checks.
  auto stage = [&]<bool kFull, bool CHK>(int js) QMM_INLINE {
    [&]<int... U>(std::integer_sequence<int, U...>) QMM_INLINE {
      (([&]() QMM_INLINE {
         const int tt = kStageSteps * js + U;
         if (kFull || tt < t1) {
           if constexpr (U == 4) scale_store(js + 1);
           body.template operator()<U % 2, U % 4, (U + 1) % 4, (U + 3) % 4, U == 1, CHK>(tt, js);
#pragma unroll
           for (int j = 0; j < FN; j++)
#pragma unroll
             for (int e = 0; e < NB; e++)
#pragma unroll
               for (int kk = 0; kk < KK; kk++) keep(bq[(U + 1) % 2][j][e][kk]);
           step_sync.template operator()<U>();
         }
       }()),
       ...);
    }(std::make_integer_sequence<int, kStageSteps>{});
  };
  const int n_full = (t1 - t0) / kStageSteps;
  int js = js0;
  if constexpr (!CONV) {
    const int kwhole = K >> 6;                 // whole 64-code steps
    const int js_safe = kwhole > 10 ? (kwhole - 10 + kStageSteps - 1) / kStageSteps : 0;
    const int js_u = js0 + n_full < js_safe ? js0 + n_full : js_safe;
    for (; js < js_u; js++) stage.template operator()<true, false>(js);
  }
  for (; js < js0 + n_full; js++) stage.template operator()<true, true>(js);
  if ((t1 - t0) % kStageSteps) stage.template operator()<false, true>(js0 + n_full);

  // ---- KW = 2: the upper-half wavefront adds its accumulators to its
  // pair's through the slice's ring slot (once every wavefront has passed
  // the first barrier, every copy has landed and every slot read is done);
  // lane-major, so each store and load instruction covers 256 contiguous
  // bytes
  if constexpr (KW == 2) {
    wait_vmcnt<0>();
    __syncthreads();
    // the slice's 32x32 tiles spread over its 4/SL slots
    constexpr int kTiles = FM * FN, kTps = kTiles / (4 / SL);
    static_assert(kTps * 16 * 64 * 4 <= kSlotBytes, "partial tiles must fit the slots");
    auto red = [&](int t) -> float* QMM_INLINE {
      return reinterpret_cast<float*>(slot_at(w4 * (4 / SL) + t / kTps)) + (t % kTps) * 16 * 64;
    };
    if (kh == 1) {
#pragma unroll
      for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
#pragma unroll
          for (int r = 0; r < 16; r++) red(i * FN + j)[r * 64 + lane] = acc[i][j][r];
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
      for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
#pragma unroll
          for (int r = 0; r < 16; r++) acc[i][j][r] += red(i * FN + j)[r * 64 + lane];
    }
  }

  // ---- split K: fp32 partial sums straight from the accumulators (lane:
  // column 32j + lane%32, rows 8(r/4) + 4(lane/32) + r%4 of each 32x32 tile;
  // each store instruction covers two 128-byte row pieces). The last
  // workgroup of the tile to arrive adds the ksplit partial sums in split
  // order (the same sum whichever workgroup arrives last) and writes y.
  // Partial sums and the counter use device-scope atomic accesses,
  // coherent across the per-XCD L2 caches; every store has completed before
  // the barrier that precedes the counter update, and the last workgroup
  // reads the partial sums only after its update has returned. The counter
  // is a wrapping increment with limit ksplit - 1, so the last arrival
  // leaves it at zero for the next call.
  if (a.ksplit > 1) {
    wait_vmcnt<0>();   // no copy may still be landing in LDS
    // conv: [split][M][ldy], the groups side by side in a row; batched GEMM:
    // [split][batch][M][ldy]
    const int64_t plane = CONV ? (int64_t)a.M * a.ldy : (int64_t)gridDim.z * a.M * a.ldy;
    float* ws0 = a.ws + (CONV ? (int64_t)g * a.Og : (int64_t)g * a.M * a.ldy);
    if (kh == 0) {
      float* ws = ws0 + sk * plane;
#pragma unroll
      for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++) {
          const int n = n_blk + wn * WTN + 32 * j + rr;
#pragma unroll
          for (int r = 0; r < 16; r++) {
            const int m = m_blk + wm * WTM + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
            // m * ldy + n < kSplitWsFloats = 2^24 floats per split: 24-bit product
            if (m < a.M && n < a.N)
              __hip_atomic_store(ws + __umul24((uint32_t)m, (uint32_t)a.ldy) + n, acc[i][j][r],
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
    }
    __builtin_amdgcn_s_waitcnt(0);   // the stores have completed
    __syncthreads();
    __shared__ unsigned last;
    if (tid == 0)
      last = __builtin_amdgcn_atomic_inc32(a.cnt + g * gridDim.x + blockIdx.x,
                                           (unsigned)(a.ksplit - 1), __ATOMIC_RELAXED,
                                           "agent") == (unsigned)(a.ksplit - 1);
    __syncthreads();
    if (!last) return;
    // the tile's partial sums as 16-byte units (row-major, BN / 4 per row),
    // all ksplit loads of a unit in flight together; agent-scope loads (sc1)
    constexpr int kUnits = BM * BN / 4 / NT;
    static_assert(BM * BN / 4 % NT == 0, "whole units per thread");
    const __amdgpu_buffer_rsrc_t pr = make_rsrc(ws0, 0x7fffffffu);
    uint16_t* yb = a.y + (CONV ? (int64_t)g * a.Og : (int64_t)g * a.M * a.ldy);
    auto finish = [&]<int KS>() QMM_INLINE {
#pragma unroll
      for (int i = 0; i < kUnits; i++) {
        const int u = tid + NT * i;
        const int m = m_blk + u / (BN / 4), n = n_blk + 4 * (u % (BN / 4));
        const bool in = m < a.M && n < a.N;
        // (the unit's byte offset in a plane: m * ldy + n < 2^24 floats)
        const uint32_t off = in ? 4u * (__umul24((uint32_t)m, (uint32_t)a.ldy) + n) : kOob;
        float4_t v[KS];
#pragma unroll
        for (int sp = 0; sp < KS; sp++)
          v[sp] = __builtin_bit_cast(
              float4_t, __builtin_amdgcn_raw_buffer_load_b128(
                            pr, off, (uint32_t)(sp * plane * 4), 16));
        float4_t t = v[0];
#pragma unroll
        for (int sp = 1; sp < KS; sp++) t += v[sp];
        if (in) {
          uint16_t* yp = yb + (int64_t)m * a.ldy + n;
          if (n + 4 <= a.N && (reinterpret_cast<uintptr_t>(yp) & 7) == 0) {
            uint2 o;
            o.x = (uint32_t)from_f32(T{}, t[0]) | ((uint32_t)from_f32(T{}, t[1]) << 16);
            o.y = (uint32_t)from_f32(T{}, t[2]) | ((uint32_t)from_f32(T{}, t[3]) << 16);
            *reinterpret_cast<uint2*>(yp) = o;
          } else {
            for (int e = 0; e < 4 && n + e < a.N; e++) yp[e] = from_f32(T{}, t[e]);
          }
        }
      }
    };
    switch (a.ksplit) {
      case 2: finish.template operator()<2>(); break;
      case 3: finish.template operator()<3>(); break;
      case 4: finish.template operator()<4>(); break;
      case 5: finish.template operator()<5>(); break;
      case 6: finish.template operator()<6>(); break;
      case 7: finish.template operator()<7>(); break;
      default: finish.template operator()<8>(); break;
    }
    return;
  }

  // ---- epilogue: each wavefront stages its WTM x WTN tile in "its" x slot
  // (all copies have landed and all slot reads are done), then writes rows
  // of 16-byte vectors.
  // (with KW = 2 the lower-half wavefronts write, the others only take part
  // in the barriers)
  wait_vmcnt<0>();
  __syncthreads();
  uint16_t* cs = reinterpret_cast<uint16_t*>(slot_at(w4 * (4 / SL)));
  constexpr int CROW = WTN + 8;
  static_assert(WTM * CROW * 2 <= kSlotBytes, "epilogue tile must fit a slot");
  if (kh == 0) {
#pragma unroll
  for (int i = 0; i < FM; i++)
#pragma unroll
    for (int j = 0; j < FN; j++) {
      const int col = 32 * j + rr;
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int row = 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
        cs[row * CROW + col] = from_f32(T{}, acc[i][j][r]);
      }
    }
  }
  __syncthreads();
  if (kh != 0) return;
  uint16_t* yb = a.y + (CONV ? (int64_t)g * a.Og : (int64_t)g * a.M * a.ldy);
  constexpr int VPR = WTN / 8;
  const bool vec_ok = (a.N % 8 == 0) && (a.ldy % 8 == 0);
#pragma unroll
  for (int it = 0; it < WTM * VPR / 64; it++) {
    const int idx = lane + 64 * it;
    const int row = idx / VPR, cv = idx % VPR;
    const int m = m_blk + wm * WTM + row, n = n_blk + wn * WTN + cv * 8;
    if (m < a.M) {
      const uint16_t* src = &cs[row * CROW + cv * 8];
      if (vec_ok && n + 8 <= a.N) {
        *reinterpret_cast<uint4*>(yb + (int64_t)m * a.ldy + n) =
            *reinterpret_cast<const uint4*>(src);
      } else {
        for (int e = 0; e < 8; e++)
          if (n + e < a.N) yb[(int64_t)m * a.ldy + n + e] = src[e];
      }
    }
  }
}

// gather kernel: convolutions whose per-group channel count is not a
// multiple of 8 (x pieces are not 16-byte units) or whose k table would not
// fit in LDS
template <class T, int BITS, int BM, int BN>
static hipError_t launch_gather(const GemmArgs& a, int groups, hipStream_t st) {
  const int tiles = ((a.N + BN - 1) / BN) * ((a.M + BM - 1) / BM);
  const dim3 grid(tiles, 1, groups);
  hipLaunchKernelGGL((qmm_mfma_kernel<T, BITS, BM, BN, true, false>), grid, dim3(256), 0,
                     st, a);
  return hipGetLastError();
}

// wavefronts per output slice of the DMA tile kernel: two (8 per workgroup,
// two per SIMD) where the x tile has a copy block for each of them
template <int BM>
constexpr int dma_kw() {
  return BM >= 64 ? 2 : 1;
}
// output slices of the DMA tile kernel: 4 (1 x 2 slices of 64 columns for
// 128 x 128 tiles halve the x reads from LDS, but one wavefront per SIMD
// cannot hide the rest: measured 19.4 against 16.1 us on 1024 x 4096 x 1024)
template <int BM, int BN>
constexpr int dma_sl() {
  return 4;
}

template <class T, int BITS, int BM, int BN, int CONV, int FPM = 0, int APK = 0>
static hipError_t launch_dma(GemmArgs a, int groups, hipStream_t st) {
  constexpr int KW = dma_kw<BM>(), SL = dma_sl<BM, BN>();
  const int tiles = ((a.N + BN - 1) / BN) * ((a.M + BM - 1) / BM);
  const dim3 grid(tiles, 1, groups);
  a.ksplit = 1;
  a.ksteps = ((a.K + 63) / 64 + kStageSteps - 1) / kStageSteps * kStageSteps;
  hipLaunchKernelGGL((qmm_dma_kernel<T, BITS, BM, BN, CONV, KW, SL, FPM, APK>), grid,
                     dim3(64 * SL * KW), 0, st, a);
  return hipGetLastError();
}

// Split-K plan for the 128 x 128 tile kernel: as many splits as keep the
// workgroups within one wave over the 256 CUs (a second, partial wave costs
// more than it saves), each split a whole number of 8-step stages, and the
// partial sums within the workspace. Returns 1 when K is not split.
// gemm (the plain f16 128 x 128 GEMM; bf16 runs two MFMAs per fragment and
// more dequantization per step, and its 64 x 64 tiles measured slower: M =
// 64, 2048 x 2048 25.3 us against 17.7 us split): each split also keeps >= 16 steps
// (shorter ones spend most of their time filling and draining the copy
// pipeline), and a split grid below 192 workgroups is used only when it
// offers at least the parallelism of unsplit 64 x 64 tiles, counting a
// 128-row tile as half a workgroup when M <= 64 (half its rows are
// padding). Measured: 512 x 2048 x 2048 22.1 us split 4 ways, 15.4 us on
// 64 x 64 tiles; 4096 x 320 x 2880 24.7 us split 2 ways (192 workgroups),
// 27.0 us on 64 x 64 tiles.
static int splitk_plan(const GemmArgs& a, int64_t tiles, int* ksteps, bool gemm = false,
                       int batches = 1) {
  const int nk = (a.K + 63) / 64;
  *ksteps = ((nk + kStageSteps - 1) / kStageSteps) * kStageSteps;
  if (tiles >= 192 || a.ldy % 4 != 0) return 1;
  int s = (int)(256 / tiles);
  if (s > 8) s = 8;
  if (s > nk / kStageSteps) s = nk / kStageSteps;
  if (gemm) {
    if (s > nk / 16) s = nk / 16;
    const int64_t t64 = (int64_t)((a.M + 63) / 64) * ((a.N + 63) / 64) * batches;
    if (s >= 2 && tiles * s < 192 && tiles * s * (a.M <= 64 ? 1 : 2) < 2 * t64) return 1;
  }
  while (s > 1 && (int64_t)s * batches * a.M * a.ldy > kSplitWsFloats) s--;
  if (s < 2) return 1;
  int per = (nk + s - 1) / s;
  per = ((per + kStageSteps - 1) / kStageSteps) * kStageSteps;
  *ksteps = per;
  return (nk + per - 1) / per;
}

// tile kernel over a BM x BN tiling with K split by plan (fp32 partial sums,
// added by the last workgroup of each tile)
template <class T, int BITS, int BM, int BN, int CONV, int FPM = 0, int APK = 0>
static hipError_t launch_dma_split(GemmArgs a, int groups, hipStream_t st) {
  const int tiles = ((a.N + BN - 1) / BN) * ((a.M + BM - 1) / BM);
  int ksteps = 0;
  a.ksplit = splitk_plan(a, (int64_t)tiles * groups, &ksteps,
                         !CONV && BM == 128 && (__is_same(T, F16) || FPM != 0), CONV ? 1 : groups);
  if (a.ksplit > 1 && (int64_t)tiles * groups > kTileCntMax) {   // one counter per tile
    a.ksplit = 1;
    ksteps = ((a.K + 63) / 64 + kStageSteps - 1) / kStageSteps * kStageSteps;
  }
  a.ksteps = ksteps;
  constexpr int KW = dma_kw<BM>(), SL = dma_sl<BM, BN>();
  hipLaunchKernelGGL((qmm_dma_kernel<T, BITS, BM, BN, CONV, KW, SL, FPM, APK>),
                     dim3(tiles, a.ksplit, groups), dim3(64 * SL * KW), 0, st, a);
  return hipGetLastError();
}

template <class T, int BITS, int CONV, bool DMA, int FPM = 0, int APK = 0>
static hipError_t launch_shape(GemmArgs a, int groups, hipStream_t st) {
  const int64_t tiles128 = (int64_t)((a.N + 127) / 128) * ((a.M + 127) / 128) * groups;
  // the plain f16 GEMM (and the fp modes, which run one MFMA per fragment in
  // either type) keep each split at least 16 steps long
  constexpr bool kGemmPlan = !CONV && (__is_same(T, F16) || FPM != 0);
  if constexpr (DMA) {
    // at most 32 rows: one 32-row block per tile (W is read once)
    if constexpr (!CONV) {
      if (a.M <= 32) return launch_dma_split<T, BITS, 32, 128, CONV, FPM, APK>(a, groups, st);
    }
    // 128-wide tiles that would leave more than half a tile of columns idle
    // (e.g. 160-channel conv groups): 64 x 64 tiles
    if (a.N % 128 != 0 && a.N % 128 < 64)
      return launch_dma<T, BITS, 64, 64, CONV, FPM, APK>(a, groups, st);
    if (tiles128 >= 192) return launch_dma<T, BITS, 128, 128, CONV, FPM, APK>(a, groups, st);
    int ks;
    if (splitk_plan(a, tiles128, &ks, kGemmPlan, CONV ? 1 : groups) > 1)
      return launch_dma_split<T, BITS, 128, 128, CONV, FPM, APK>(a, groups, st);
    return launch_dma<T, BITS, 64, 64, CONV, FPM, APK>(a, groups, st);
  } else {
    if (tiles128 >= 256) return launch_gather<T, BITS, 128, 128>(a, groups, st);
    return launch_gather<T, BITS, 64, 64>(a, groups, st);
  }
}

template <class T, int CONV, bool DMA>
static hipError_t launch_bits(int bits, const GemmArgs& a, int groups,
                              hipStream_t st) {
  switch (bits) {
    case 2: return launch_shape<T, 2, CONV, DMA>(a, groups, st);
    case 3: return launch_shape<T, 3, CONV, DMA>(a, groups, st);
    case 4: return launch_shape<T, 4, CONV, DMA>(a, groups, st);
    case 5: return launch_shape<T, 5, CONV, DMA>(a, groups, st);
    case 6: return launch_shape<T, 6, CONV, DMA>(a, groups, st);
    default: return launch_shape<T, 8, CONV, DMA>(a, groups, st);
  }
}

}  // namespace
}  // namespace qmm
