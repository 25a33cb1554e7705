// MFMA tile GEMM for y = x . dequant(W)^T at large M, and the implicit-im2col
// quantized conv2d that feeds the same tile engine.
//
// Operation: "mlx 1.0.0 backend/cpu/quantized.cpp", _qmm_t (y[m,n] =
// sum_k x[m,k] * (s*q + b)); tile structure in the spirit of the Metal
// qmm_t of "Add the 3bit packed qmm_t" (affine_packed_qmm_t_impl: per K
// step, load an x tile, dequantize a W tile into on-chip memory, multiply),
// rebuilt for gfx950:
//  * 256 threads = 4 wavefronts in a 2x2 grid; a workgroup owns a BM x BN
//    tile of y and walks K in steps of 64 (one f16/bf16 x tile and one
//    dequantized W tile in LDS, single-buffered, with the next step's global
//    loads in flight in registers while the MFMAs of the current one run).
//  * v_mfma_f32_16x16x32_{f16,bf16}: each wavefront holds
//    (BM/32) x (BN/32) accumulator tiles of 16x16 in fp32.
//  * W is dequantized once per workgroup and K step, w = fl32(s*q + b)
//    rounded to the element type. For bf16 a single rounding to 8
//    significand bits would cost ~1e-3 relative error, so W is split as
//    hi = bf16(w), lo = bf16(w - hi) and both halves go through the MFMA
//    (error ~2^-17 relative).
//  * The conv variant ("[Feature] Quantized Convolution 2D" issue, img2col
//    + quantized_matmul) computes the im2col patch addresses inside the x
//    tile loader: GEMM row m = output pixel (b, oy, ox), column k =
//    (dy, dx, c) of conv group g = blockIdx.z, zero for taps outside the
//    image and for the zero-padded tail k >= K_true.
#include <utility>

#include "common.hpp"
#include "kernels.hpp"

namespace qmm {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));

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
};

// v_mfma_f32_32x32x16: A[i][k] from lane i%32 + 32*(k/8) (element k%8), B[k][j]
// from lane j + 32*(k/8), D[i][j] in lane j + 32*((i/4)%2), element
// 4*(i/8) + i%4. One wavefront sustains close to the matrix-core peak with
// four independent 32x32 accumulators (measured), unlike the 16x16x32 form.
__device__ __forceinline__ float16_t mfma32(F16, const uint4& a, const uint4& b,
                                            float16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(
      __builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ float16_t mfma32(BF16, const uint4& a, const uint4& b,
                                            float16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
      __builtin_bit_cast(bf8_t, a), __builtin_bit_cast(bf8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float4_t mfma16(F16, const uint4& a, const uint4& b,
                                           float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(
      __builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ float4_t mfma16(BF16, const uint4& a, const uint4& b,
                                           float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf8_t, a), __builtin_bit_cast(bf8_t, b), c, 0, 0, 0);
}

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
    uint32_t v[2];
#pragma unroll
    for (int e = 0; e < 2; e++) {
      const int kk = k + e;
      const int p = pair_index<BITS>(kk), h = pair_half<BITS>(kk);
      const int o = pair_off<F16, BITS>(kk);
      const uint16_t hb = (uint16_t)(pr[p] >> (16 * h));
      const float q = (float)__builtin_bit_cast(_Float16, hb);
      v[e] = from_f32(F16{}, fmaf(q, so[o], co[o]));
    }
    out[k / 2] = v[0] | (v[1] << 16);
  }
}

// bf16 dequantization of a chunk, split as hi = bf16(w), lo = bf16(w - hi).
template <int BITS>
__device__ __forceinline__ void dequant_chunk_bf16(const uint32_t* w, float s,
                                                   float b, uint32_t* hi,
                                                   uint32_t* lo) {
  [&]<int... J>(std::integer_sequence<int, J...>) {
    float f[32] = {fmaf(s, (float)code_at<BITS, J>(w), b)...};
#pragma unroll
    for (int k = 0; k < 32; k += 2) {
      const uint16_t h0 = from_f32(BF16{}, f[k]), h1 = from_f32(BF16{}, f[k + 1]);
      hi[k / 2] = (uint32_t)h0 | ((uint32_t)h1 << 16);
      const uint16_t l0 = from_f32(BF16{}, f[k] - to_f32(BF16{}, h0));
      const uint16_t l1 = from_f32(BF16{}, f[k + 1] - to_f32(BF16{}, h1));
      lo[k / 2] = (uint32_t)l0 | ((uint32_t)l1 << 16);
    }
  }(std::make_integer_sequence<int, 32>{});
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

// ----------------------------------------------------------------- launch

template <class T, int BITS, int BM, int BN, bool CONV, bool CONV_VEC>
static hipError_t launch_tile(const GemmArgs& a, int groups, hipStream_t st) {
  const int tiles = ((a.N + BN - 1) / BN) * ((a.M + BM - 1) / BM);
  const dim3 grid(tiles, 1, groups);
  hipLaunchKernelGGL((qmm_mfma_kernel<T, BITS, BM, BN, CONV, CONV_VEC>), grid,
                     dim3(256), 0, st, a);
  return hipGetLastError();
}

template <class T, int BITS, bool CONV, bool CONV_VEC>
static hipError_t launch_shape(const GemmArgs& a, int groups, hipStream_t st) {
  const int64_t tiles128 = (int64_t)((a.N + 127) / 128) * ((a.M + 127) / 128) * groups;
  if (tiles128 >= 256)
    return launch_tile<T, BITS, 128, 128, CONV, CONV_VEC>(a, groups, st);
  return launch_tile<T, BITS, 64, 64, CONV, CONV_VEC>(a, groups, st);
}

template <class T, bool CONV, bool CONV_VEC>
static hipError_t launch_bits(int bits, const GemmArgs& a, int groups,
                              hipStream_t st) {
  switch (bits) {
    case 2: return launch_shape<T, 2, CONV, CONV_VEC>(a, groups, st);
    case 3: return launch_shape<T, 3, CONV, CONV_VEC>(a, groups, st);
    case 4: return launch_shape<T, 4, CONV, CONV_VEC>(a, groups, st);
    case 5: return launch_shape<T, 5, CONV, CONV_VEC>(a, groups, st);
    case 6: return launch_shape<T, 6, CONV, CONV_VEC>(a, groups, st);
    default: return launch_shape<T, 8, CONV, CONV_VEC>(a, groups, st);
  }
}

hipError_t launch_qmm_mfma(int dt, int bits, int gs, const void* x,
                           const uint32_t* wq, const void* s, const void* b,
                           int64_t M, int64_t N, int64_t K, void* y,
                           hipStream_t st) {
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
  if (dt == 0) return launch_bits<F16, false, false>(bits, a, 1, st);
  return launch_bits<BF16, false, false>(bits, a, 1, st);
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
  const bool vec = (cg.Cg % 8) == 0;
  if (dt == 0) {
    return vec ? launch_bits<F16, true, true>(bits, a, cg.groups, st)
               : launch_bits<F16, true, false>(bits, a, cg.groups, st);
  }
  return vec ? launch_bits<BF16, true, true>(bits, a, cg.groups, st)
             : launch_bits<BF16, true, false>(bits, a, cg.groups, st);
}

int crossover_m(int bits, int dt) {
  (void)bits;
  (void)dt;
  return 16;
}

}  // namespace qmm
