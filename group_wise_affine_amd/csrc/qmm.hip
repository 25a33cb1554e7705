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
#include "common.hpp"
#include "kernels.hpp"

namespace qmm {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

struct GemmArgs {
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

// Dequantize the 32 codes of a chunk: out[j] = fl32(s*q_j + b) (s*q exact).
template <int BITS, int J = 0>
__device__ __forceinline__ void dequant_chunk(const uint32_t* w, float s,
                                              float b, float* out) {
  if constexpr (J < 32) {
    out[J] = fmaf(s, (float)code_at<BITS, J>(w), b);
    dequant_chunk<BITS, J + 1>(w, s, b, out);
  }
}

__device__ __forceinline__ uint32_t pack2(F16, float a, float b) {
  return (uint32_t)from_f32(F16{}, a) | ((uint32_t)from_f32(F16{}, b) << 16);
}
__device__ __forceinline__ uint32_t pack2(BF16, float a, float b) {
  return (uint32_t)from_f32(BF16{}, a) | ((uint32_t)from_f32(BF16{}, b) << 16);
}

constexpr int kBK = 64;       // K step
constexpr int kPad = 8;       // LDS row padding in 16-bit elements
constexpr int kLdsRow = kBK + kPad;

template <class T, int BITS, int BM, int BN, bool CONV, bool CONV_VEC>
__global__ __launch_bounds__(256) void qmm_mfma_kernel(GemmArgs a) {
  constexpr bool kSplit = __is_same(T, BF16);
  constexpr int WTM = BM / 2, WTN = BN / 2;  // wavefront tile
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int A_VECS = BM * kBK / 8 / 256;  // 16-byte x vectors per thread
  constexpr int W_CHUNKS = BN * 2;            // 32-code chunks per K step
  constexpr int W_PER_T = (W_CHUNKS + 255) / 256;
  static_assert(A_VECS >= 1, "BM too small");

  __shared__ __attribute__((aligned(16))) uint16_t As[BM * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t Ws[BN * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t Wl[kSplit ? BN * kLdsRow : 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m_blk = blockIdx.y * BM, n_blk = blockIdx.x * BN;
  const int g = CONV ? blockIdx.z : 0;

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

  uint4 a_reg[A_VECS];
  uint32_t w_reg[W_PER_T][BITS];
  float s_reg[W_PER_T], b_reg[W_PER_T];

  auto load_tile = [&](int kt) {
    const int k0 = kt * kBK;
#pragma unroll
    for (int v = 0; v < A_VECS; v++) {
      const int k = k0 + a_kv[v] * 8;
      uint4 val = make_uint4(0, 0, 0, 0);
      if constexpr (!CONV) {
        if (a_ok[v] && k < a.K)
          val = *reinterpret_cast<const uint4*>(
              a.x + (int64_t)(m_blk + a_row[v]) * a.K + k);
      } else if constexpr (CONV_VEC) {
        if (a_ok[v] && k < a.K_true) {
          const int tap = k / a.Cg, c = k - tap * a.Cg;
          const int dy = tap / a.kw, dx = tap - dy * a.kw;
          const int iy = pix_y[v] + dy, ix = pix_x[v] + dx;
          if (iy >= 0 && iy < a.H && ix >= 0 && ix < a.W)
            val = *reinterpret_cast<const uint4*>(
                a.x + (((int64_t)pix_b[v] * a.H + iy) * a.W + ix) * a.C +
                g * a.Cg + c);
        }
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
              e[i] = a.x[(((int64_t)pix_b[v] * a.H + iy) * a.W + ix) * a.C +
                         g * a.Cg + c];
          }
        }
        val = make_uint4(e[0] | (uint32_t)e[1] << 16, e[2] | (uint32_t)e[3] << 16,
                         e[4] | (uint32_t)e[5] << 16, e[6] | (uint32_t)e[7] << 16);
      }
      a_reg[v] = val;
    }
#pragma unroll
    for (int u = 0; u < W_PER_T; u++) {
      const int ci = tid + 256 * u;
      const int n = n_blk + ci / 2;
      const int kc = k0 + (ci % 2) * 32;
#pragma unroll
      for (int i = 0; i < BITS; i++) w_reg[u][i] = 0;
      s_reg[u] = 0.0f;
      b_reg[u] = 0.0f;
      if (ci < W_CHUNKS && n < a.N && kc < a.K) {
        load_wchunk<BITS>(wq + (int64_t)n * w_row_bytes + (int64_t)kc * BITS / 8,
                          w_reg[u]);
        const int gi = kc >> a.gs_log2;
        s_reg[u] = to_f32(T{}, sp[(int64_t)n * n_groups_row + gi]);
        b_reg[u] = to_f32(T{}, bp[(int64_t)n * n_groups_row + gi]);
      }
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int v = 0; v < A_VECS; v++)
      *reinterpret_cast<uint4*>(&As[a_row[v] * kLdsRow + a_kv[v] * 8]) = a_reg[v];
#pragma unroll
    for (int u = 0; u < W_PER_T; u++) {
      const int ci = tid + 256 * u;
      if (ci < W_CHUNKS) {
        const int r = ci / 2, h = ci % 2;
        float f[32];
        dequant_chunk<BITS>(w_reg[u], s_reg[u], b_reg[u], f);
        uint32_t hi[16];
#pragma unroll
        for (int i = 0; i < 16; i++) hi[i] = pack2(T{}, f[2 * i], f[2 * i + 1]);
        uint4* dst = reinterpret_cast<uint4*>(&Ws[r * kLdsRow + h * 32]);
#pragma unroll
        for (int q = 0; q < 4; q++)
          dst[q] = make_uint4(hi[4 * q], hi[4 * q + 1], hi[4 * q + 2], hi[4 * q + 3]);
        if constexpr (kSplit) {
          uint32_t lo[16];
#pragma unroll
          for (int i = 0; i < 16; i++) {
            const float h0 = to_f32(BF16{}, (uint16_t)(hi[i] & 0xffffu));
            const float h1 = to_f32(BF16{}, (uint16_t)(hi[i] >> 16));
            lo[i] = pack2(BF16{}, f[2 * i] - h0, f[2 * i + 1] - h1);
          }
          uint4* dl = reinterpret_cast<uint4*>(&Wl[r * kLdsRow + h * 32]);
#pragma unroll
          for (int q = 0; q < 4; q++)
            dl[q] = make_uint4(lo[4 * q], lo[4 * q + 1], lo[4 * q + 2], lo[4 * q + 3]);
        }
      }
    }
  };

  float4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; i++)
#pragma unroll
    for (int j = 0; j < FN; j++) acc[i][j] = (float4_t){0.f, 0.f, 0.f, 0.f};

  const int nkt = (a.K + kBK - 1) / kBK;
  load_tile(0);
  for (int kt = 0; kt < nkt; kt++) {
    store_tile();
    __syncthreads();
    if (kt + 1 < nkt) load_tile(kt + 1);
#pragma unroll
    for (int kk = 0; kk < kBK / 32; kk++) {
      const int kof = kk * 32 + 8 * (lane >> 4);
      uint4 af[FM], bf[FN], bl[FN];
#pragma unroll
      for (int i = 0; i < FM; i++)
        af[i] = *reinterpret_cast<const uint4*>(
            &As[(wm * WTM + 16 * i + (lane & 15)) * kLdsRow + kof]);
#pragma unroll
      for (int j = 0; j < FN; j++) {
        bf[j] = *reinterpret_cast<const uint4*>(
            &Ws[(wn * WTN + 16 * j + (lane & 15)) * kLdsRow + kof]);
        if constexpr (kSplit)
          bl[j] = *reinterpret_cast<const uint4*>(
              &Wl[(wn * WTN + 16 * j + (lane & 15)) * kLdsRow + kof]);
      }
#pragma unroll
      for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++) {
          acc[i][j] = mfma16(T{}, af[i], bf[j], acc[i][j]);
          if constexpr (kSplit) acc[i][j] = mfma16(T{}, af[i], bl[j], acc[i][j]);
        }
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds rows 4*(lane/16)+r, column lane%16 of each tile
  uint16_t* yb = a.y + (CONV ? (int64_t)g * a.Og : 0);
#pragma unroll
  for (int i = 0; i < FM; i++)
#pragma unroll
    for (int j = 0; j < FN; j++) {
      const int n = n_blk + wn * WTN + 16 * j + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int m = m_blk + wm * WTM + 16 * i + 4 * (lane >> 4) + r;
        if (m < a.M && n < a.N) yb[(int64_t)m * a.ldy + n] = from_f32(T{}, acc[i][j][r]);
      }
    }
}

// ----------------------------------------------------------------- launch

template <class T, int BITS, int BM, int BN, bool CONV, bool CONV_VEC>
static hipError_t launch_tile(const GemmArgs& a, int groups, hipStream_t st) {
  const dim3 grid((a.N + BN - 1) / BN, (a.M + BM - 1) / BM, groups);
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
