// Non-transposed quantized product for many rows of x on the matrix cores:
//   y[m, n] = sum_k x[m, k] * (s[k, n/gs] * q[k, n] + b[k, n/gs]),
// W stored [K, N] with its groups along N ("mlx 1.0.0 backend/cpu/quantized.cpp",
// _qmm, the transpose = false branch of quantized_matmul), fp32 accumulation.
//
// MI355X design (wave64, gfx950):
//  * 128 x 128 output tiles, 4 wavefronts in a 2 x 2 layout (64 x 64 each:
//    2 x 2 v_mfma_f32_32x32x16 accumulators), K steps of 64.
//  * The MFMA wants 8 consecutive k of one output column per lane, while W
//    keeps the columns of a row together. So W is dequantized once per step
//    into an LDS tile stored column-major (ws[n][k]), from which the B
//    fragments are plain 16-byte reads, as the A fragments are from the x
//    tile (xs[m][k]). Thread (p, c, h) dequantizes rows 2p and 2p + 1 of the
//    step, columns 32c + 16h .. + 15 of the tile: 16 codes per row read from
//    the step's raw code tile in LDS, w = fl32(s q + b) as the dequantizer
//    computes it, written as (k, k + 1) pairs; bf16 stores w as two tiles,
//    hi = bf16(w) and lo = bf16(w - hi), multiplied separately (one bf16
//    rounding of w would cost ~1e-3 relative error).
//  * Step t + 1's x tile, raw code tile and scales are loaded into
//    registers while step t is dequantized and multiplied; two barriers per
//    step (raw codes and the W tile are single-buffered across them, x and
//    the W tile double-buffered).
//  * Loads go through buffer resources: rows of W and of the scales past K
//    read zero (so those k contribute nothing), rows of x past M read zero.
//  * FPM != 0: the floating-point modes (the page's fp_qmm): 1 mxfp4 (E2M1
//    codes, e8m0 scale per 32 columns), 2 nvfp4 (E2M1, E4M3 scale per 16), 3
//    mxfp8 (E4M3, e8m0 per 32), no bias; codes are decoded by gfx950's
//    conversions at scale 1 and multiplied by the scale rounded to T, which
//    is exact in T within T's range, so one W tile serves f16 and bf16.
//  * Few output tiles (the launch would leave CUs idle): K is split over up
//    to 8 workgroups per tile; each stores its fp32 partial tile to the
//    split-K workspace with device-scope stores and counts itself in on the
//    tile's wrapping counter, and the last to arrive adds the partial tiles
//    in split order (16-byte device-scope loads, all splits in flight) and
//    writes y.
#include "common.hpp"
#include "kernels.hpp"
#include "mfma_common.hpp"
#include "tile_args.hpp"

namespace qmm {
namespace {

constexpr int kQtM = 128, kQtN = 128, kQtK = 64;   // tile and K step
constexpr int kQtThreads = 256;
constexpr int kQtLd = kQtK + 8;                     // LDS row length (elements) of xs and ws

// the 8 E2M1 codes of a word (FPM 1, 2) or the 4 E4M3 codes (FPM 3) as fp32
template <int FPM>
__device__ __forceinline__ void fp_decode_word(uint32_t w, float* v) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  if constexpr (FPM == 3) {
    const f32x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
    const f32x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true);
    v[0] = lo[0]; v[1] = lo[1]; v[2] = hi[0]; v[3] = hi[1];
  } else {
    const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    v[0] = p0[0]; v[1] = p0[1]; v[2] = p1[0]; v[3] = p1[1];
    v[4] = p2[0]; v[5] = p2[1]; v[6] = p3[0]; v[7] = p3[1];
  }
}

template <class T, int BITS, int FPM = 0>
__global__ __launch_bounds__(kQtThreads) void qmn_tile_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wq,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases,
    uint16_t* __restrict__ y, int M, int N, int K, int gs_log2, int ksplit, int ksteps,
    float* __restrict__ ws, unsigned* __restrict__ cnt) {
  constexpr bool kFp = FPM != 0;
  constexpr bool kSplit = !kFp && __is_same(T, BF16);   // hi / lo W tiles
  constexpr int NB = kSplit ? 2 : 1;
  constexpr int kRowBytes = 16 * BITS;            // raw codes of one tile row (128 codes)
  constexpr int kRawUnits = kQtK * BITS;          // 16-byte units of the raw tile
  constexpr int kRawPer = (kRawUnits + kQtThreads - 1) / kQtThreads;
  constexpr int kXPer = kQtM * kQtK / 8 / kQtThreads;   // 16-byte x units per thread
  // dwords of the 16-code window (2*BITS bytes, at a 2-byte aligned offset)
  constexpr int kWinDw = (2 * BITS + 2 + 3) / 4;

  __shared__ __attribute__((aligned(16))) uint16_t xs[2][kQtM * kQtLd];
  __shared__ __attribute__((aligned(16))) uint16_t wsl[2][NB][kQtN * kQtLd];
  __shared__ __attribute__((aligned(16))) uint8_t raw[kQtK * kRowBytes + 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * kQtM, n0 = blockIdx.x * kQtN;
  const int nk = (K + kQtK - 1) / kQtK;
  const int sk = blockIdx.z;                           // K split: steps [t0, t1)
  const int t0 = sk * ksteps, t1 = t0 + ksteps < nk ? t0 + ksteps : nk;
  const int G = N >> gs_log2;
  const uint32_t row_bytes = (uint32_t)N * BITS / 8;

  const __amdgpu_buffer_rsrc_t xr =
      make_rsrc(x + (int64_t)m0 * K, (uint32_t)((int64_t)(M - m0 < kQtM ? M - m0 : kQtM) * K * 2));
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(wq, (uint32_t)((int64_t)K * row_bytes));
  constexpr int ES = kFp ? 1 : 2;                       // bytes per scale
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(scales, (uint32_t)((int64_t)K * G * ES));
  const __amdgpu_buffer_rsrc_t br = make_rsrc(kFp ? scales : biases, (uint32_t)((int64_t)K * G * ES));

  // dequantization role: rows 2p, 2p+1 of the step, columns 32c + 16h + [0, 16)
  const int p = tid & 31, c = (tid >> 5) & 3, h = tid >> 7;
  const int grp = (n0 + 32 * c + 16 * h) >> gs_log2;   // the thread's group
  const int wbyte = (4 * c + 2 * h) * BITS;            // window start in a raw row
  const int wshift = 8 * (wbyte & 3);                  // 0 or 16 (uniform per wavefront)

  // ---- global loads of step t into registers
  uint4 xreg[kXPer], rreg[kRawPer];
  uint32_t snext[4], scur[4];   // (scale, bias) of rows 2p, 2p+1: next step, this step
  auto load = [&](int t) QMM_INLINE {
    const int k0 = t * kQtK;
#pragma unroll
    for (int i = 0; i < kXPer; i++) {
      const int u = tid + kQtThreads * i;              // row u / 8, k unit u % 8
      const int m = u >> 3, k = k0 + 8 * (u & 7);
      const uint32_t off = k < K ? (uint32_t)(m * K + k) * 2 : kOob;
      xreg[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < kRawPer; i++) {
      const int u = tid + kQtThreads * i;              // row u / BITS, part u % BITS
      const int r = u / BITS, part = u - r * BITS;
      const uint32_t off = (u < kRawUnits && k0 + r < K)
                               ? (uint32_t)(k0 + r) * row_bytes + (uint32_t)(n0 * BITS / 8 + 16 * part)
                               : kOob;
      rreg[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, 0));
    }
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int k = k0 + 2 * p + j;
      const uint32_t off = k < K ? (uint32_t)(k * G + grp) * ES : kOob;
      if constexpr (kFp) {
        snext[2 * j] = __builtin_amdgcn_raw_buffer_load_b8(sr, off, 0, 0);
        snext[2 * j + 1] = 0;
      } else {
        snext[2 * j] = __builtin_amdgcn_raw_buffer_load_b16(sr, off, 0, 0);
        snext[2 * j + 1] = __builtin_amdgcn_raw_buffer_load_b16(br, off, 0, 0);
      }
    }
  };
  // ---- registers into the LDS x slot b and the raw code tile (and the
  // scales into scur)
  auto store = [&](int b) QMM_INLINE {
#pragma unroll
    for (int i = 0; i < 4; i++) scur[i] = snext[i];
#pragma unroll
    for (int i = 0; i < kXPer; i++) {
      const int u = tid + kQtThreads * i;
      *reinterpret_cast<uint4*>(&xs[b][(u >> 3) * kQtLd + 8 * (u & 7)]) = xreg[i];
    }
#pragma unroll
    for (int i = 0; i < kRawPer; i++) {
      const int u = tid + kQtThreads * i;
      if (u < kRawUnits) {
        const int r = u / BITS, part = u - r * BITS;
        *reinterpret_cast<uint4*>(&raw[r * kRowBytes + 16 * part]) = rreg[i];
      }
    }
  };

  // ---- dequantize the raw tile (scales in scur) into W slot b
  auto dequant = [&](int b) QMM_INLINE {
    float sf[2], bf[2];
#pragma unroll
    for (int j = 0; j < 2; j++) {
      sf[j] = to_f32(T{}, (uint16_t)scur[2 * j]);
      bf[j] = to_f32(T{}, (uint16_t)scur[2 * j + 1]);
    }
    uint32_t win[2][kWinDw];
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const uint32_t* rp =
          reinterpret_cast<const uint32_t*>(&raw[(2 * p + j) * kRowBytes + (wbyte & ~3)]);
      uint32_t d[kWinDw + 1];
#pragma unroll
      for (int i = 0; i <= kWinDw; i++) d[i] = i < kWinDw ? rp[i] : 0u;
#pragma unroll
      for (int i = 0; i < kWinDw; i++) win[j][i] = __builtin_amdgcn_alignbit(d[i + 1], d[i], wshift);
    }
    constexpr uint32_t mask = (1u << BITS) - 1;
    auto code = [&](int j, int e) QMM_INLINE -> uint32_t {
      const int pos = e * BITS, wd = pos >> 5, of = pos & 31;
      if (of + BITS <= 32) return (win[j][wd] >> of) & mask;
      return __builtin_amdgcn_alignbit(win[j][wd + 1], win[j][wd], of) & mask;
    };
    uint16_t* wlo = wsl[b][0];
    if constexpr (kFp) {
      // w = scale_T * code value (exact in T within its range)
      float v[2][16];
#pragma unroll
      for (int j = 0; j < 2; j++)
#pragma unroll
        for (int q = 0; q < BITS / 2; q++) fp_decode_word<FPM>(win[j][q], &v[j][q * 32 / BITS]);
      float sc[2];
#pragma unroll
      for (int j = 0; j < 2; j++)
        sc[j] = __builtin_bit_cast(float, fp_scale_t_bits<T, FPM>(scur[2 * j]));
#pragma unroll
      for (int e = 0; e < 16; e++) {
        const int n = 32 * c + 16 * h + e;
        *reinterpret_cast<uint32_t*>(&wlo[n * kQtLd + 2 * p]) =
            (uint32_t)from_f32(T{}, sc[0] * v[0][e]) | ((uint32_t)from_f32(T{}, sc[1] * v[1][e]) << 16);
      }
      return;
    }
#pragma unroll
    for (int e = 0; e < 16; e++) {
      const int n = 32 * c + 16 * h + e;
      const float w0 = fmaf(sf[0], (float)code(0, e), bf[0]);
      const float w1 = fmaf(sf[1], (float)code(1, e), bf[1]);
      uint32_t* dst = reinterpret_cast<uint32_t*>(&wlo[n * kQtLd + 2 * p]);
      if constexpr (kSplit) {
        const uint32_t hu = (uint32_t)from_f32(BF16{}, w0) | ((uint32_t)from_f32(BF16{}, w1) << 16);
        *dst = hu;
        const float r0 = w0 - __builtin_bit_cast(float, hu << 16);
        const float r1 = w1 - __builtin_bit_cast(float, hu & 0xffff0000u);
        *reinterpret_cast<uint32_t*>(&wsl[b][1][n * kQtLd + 2 * p]) =
            (uint32_t)from_f32(BF16{}, r0) | ((uint32_t)from_f32(BF16{}, r1) << 16);
      } else {
        *dst = (uint32_t)from_f32(F16{}, w0) | ((uint32_t)from_f32(F16{}, w1) << 16);
      }
    }
  };

  float16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

  const int rr = lane & 31, kg = lane >> 5;
  auto multiply = [&](int b) QMM_INLINE {
#pragma unroll
    for (int ks = 0; ks < kQtK / 16; ks++) {
      uint4 a[2], bq[2][NB];
#pragma unroll
      for (int i = 0; i < 2; i++)
        a[i] = *reinterpret_cast<const uint4*>(
            &xs[b][(wm * 64 + 32 * i + rr) * kQtLd + 16 * ks + 8 * kg]);
#pragma unroll
      for (int j = 0; j < 2; j++)
#pragma unroll
        for (int e = 0; e < NB; e++)
          bq[j][e] = *reinterpret_cast<const uint4*>(
              &wsl[b][e][(wn * 64 + 32 * j + rr) * kQtLd + 16 * ks + 8 * kg]);
#pragma unroll
      for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
          for (int e = 0; e < NB; e++) acc[i][j] = mfma32(T{}, a[i], bq[j][e], acc[i][j]);
    }
  };

  // ---- prologue: the first step into x slot 0 and the raw tile
  load(t0);
  store(0);
  __syncthreads();
  for (int t = t0; t < t1; t++) {
    const int b = (t - t0) & 1;
    if (t + 1 < t1) load(t + 1);          // in flight during this step
    dequant(b);                           // reads the raw tile and this step's scales
    __syncthreads();                      // W slot b complete; raw tile free
    multiply(b);
    if (t + 1 < t1) store(b ^ 1);         // x slot b^1 was last read before the previous barrier
    __syncthreads();
  }

  if (ksplit > 1) {
    // partial tile of split sk: plane [M][N] of fp32
    const int64_t plane = (int64_t)M * N;
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
      for (int j = 0; j < 2; j++) {
        const int n = n0 + wn * 64 + 32 * j + rr;
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int m = m0 + wm * 64 + 32 * i + 8 * (r >> 2) + 4 * kg + (r & 3);
          if (m < M && n < N)
            __hip_atomic_store(ws + sk * plane + (int64_t)m * N + n, acc[i][j][r], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    __builtin_amdgcn_s_waitcnt(0);   // the stores have completed
    __syncthreads();
    __shared__ unsigned last;
    if (tid == 0)
      last = __builtin_amdgcn_atomic_inc32(cnt + blockIdx.y * gridDim.x + blockIdx.x,
                                           (unsigned)(ksplit - 1), __ATOMIC_RELAXED,
                                           "agent") == (unsigned)(ksplit - 1);
    __syncthreads();
    if (!last) return;
    // the tile's partial sums as 16-byte units (N % 32 == 0: whole units),
    // added in split order
    const __amdgpu_buffer_rsrc_t pr = make_rsrc(ws, 0x7fffffffu);
    auto finish = [&]<int KS>() QMM_INLINE {
#pragma unroll
      for (int i = 0; i < kQtM * kQtN / 4 / kQtThreads; i++) {
        const int u = tid + kQtThreads * i;
        const int m = m0 + u / (kQtN / 4), n = n0 + 4 * (u % (kQtN / 4));
        const bool in = m < M && n < N;
        float4_t v[KS];
#pragma unroll
        for (int sp = 0; sp < KS; sp++) {
          const uint32_t off = in ? (uint32_t)(((int64_t)sp * plane + (int64_t)m * N + n) * 4) : kOob;
          v[sp] = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(pr, off, 0, 16));
        }
        float4_t t = v[0];
#pragma unroll
        for (int sp = 1; sp < KS; sp++) t += v[sp];
        if (in) {
          uint2 o;
          o.x = (uint32_t)from_f32(T{}, t[0]) | ((uint32_t)from_f32(T{}, t[1]) << 16);
          o.y = (uint32_t)from_f32(T{}, t[2]) | ((uint32_t)from_f32(T{}, t[3]) << 16);
          *reinterpret_cast<uint2*>(y + (int64_t)m * N + n) = o;
        }
      }
    };
    switch (ksplit) {
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

  // ---- epilogue: lane holds column 32j + lane%32 of rows 8(r/4) + 4(lane/32) + r%4
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int n = n0 + wn * 64 + 32 * j + rr;
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int m = m0 + wm * 64 + 32 * i + 8 * (r >> 2) + 4 * kg + (r & 3);
        if (m < M && n < N) y[(int64_t)m * N + n] = from_f32(T{}, acc[i][j][r]);
      }
    }
}

// K splits: enough workgroups for one wave over the 256 CUs, at most 8 per
// tile, each split at least 4 steps, one counter per tile, the partial sums
// within the workspace
int qmn_splits(int64_t M, int64_t N, int64_t K, int* ksteps) {
  const int64_t tiles = ((N + kQtN - 1) / kQtN) * ((M + kQtM - 1) / kQtM);
  const int nk = (int)((K + kQtK - 1) / kQtK);
  int s = tiles >= 256 ? 1 : (int)(256 / tiles);
  if (s > 8) s = 8;
  if (s > nk / 4) s = nk / 4;
  if (tiles > kTileCntMax) s = 1;
  while (s > 1 && (int64_t)s * M * N > kSplitWsFloats) s--;
  if (s < 1) s = 1;
  const int per = (nk + s - 1) / s;
  *ksteps = per;
  return (nk + per - 1) / per;
}

template <class T, int BITS, int FPM = 0>
hipError_t launch_bits(const void* x, const uint32_t* wq, const void* s, const void* b,
                       int64_t M, int64_t N, int64_t K, int gs, void* y, float* ws,
                       unsigned* cnt, hipStream_t st) {
  int ksteps = 0;
  const int ks = qmn_splits(M, N, K, &ksteps);
  const dim3 grid((unsigned)((N + kQtN - 1) / kQtN), (unsigned)((M + kQtM - 1) / kQtM),
                  (unsigned)ks);
  hipLaunchKernelGGL((qmn_tile_kernel<T, BITS, FPM>), grid, dim3(kQtThreads), 0, st,
                     static_cast<const uint16_t*>(x), reinterpret_cast<const uint8_t*>(wq),
                     static_cast<const uint16_t*>(s), static_cast<const uint16_t*>(b),
                     static_cast<uint16_t*>(y), (int)M, (int)N, (int)K, ilog2(gs), ks, ksteps,
                     ws, cnt);
  return hipGetLastError();
}

template <class T>
hipError_t launch_t(int bits, const void* x, const uint32_t* wq, const void* s, const void* b,
                    int64_t M, int64_t N, int64_t K, int gs, void* y, float* ws, unsigned* cnt,
                    hipStream_t st) {
  switch (bits) {
    case 2: return launch_bits<T, 2>(x, wq, s, b, M, N, K, gs, y, ws, cnt, st);
    case 3: return launch_bits<T, 3>(x, wq, s, b, M, N, K, gs, y, ws, cnt, st);
    case 4: return launch_bits<T, 4>(x, wq, s, b, M, N, K, gs, y, ws, cnt, st);
    case 5: return launch_bits<T, 5>(x, wq, s, b, M, N, K, gs, y, ws, cnt, st);
    case 6: return launch_bits<T, 6>(x, wq, s, b, M, N, K, gs, y, ws, cnt, st);
    default: return launch_bits<T, 8>(x, wq, s, b, M, N, K, gs, y, ws, cnt, st);
  }
}

}  // namespace

hipError_t launch_qmm_n_tile(int dt, int bits, int gs, const void* x, const uint32_t* wq,
                             const void* s, const void* b, int64_t M, int64_t N, int64_t K,
                             void* y, hipStream_t st) {
  float* ws = splitk_workspace();
  unsigned* cnt = tile_counters();
  if (!ws || !cnt) return hipErrorInvalidSymbol;
  if (dt == 0) return launch_t<F16>(bits, x, wq, s, b, M, N, K, gs, y, ws, cnt, st);
  return launch_t<BF16>(bits, x, wq, s, b, M, N, K, gs, y, ws, cnt, st);
}

hipError_t launch_fp_qmm_n_tile(int dt, int bits, int gs, const void* x, const uint32_t* wq,
                                const uint8_t* scales, int64_t M, int64_t N, int64_t K, void* y,
                                hipStream_t st) {
  float* ws = splitk_workspace();
  unsigned* cnt = tile_counters();
  if (!ws || !cnt) return hipErrorInvalidSymbol;
  const void* s = scales;
  if (dt == 0) {
    if (bits == 8) return launch_bits<F16, 8, 3>(x, wq, s, s, M, N, K, gs, y, ws, cnt, st);
    if (gs == 16) return launch_bits<F16, 4, 2>(x, wq, s, s, M, N, K, gs, y, ws, cnt, st);
    return launch_bits<F16, 4, 1>(x, wq, s, s, M, N, K, gs, y, ws, cnt, st);
  }
  if (bits == 8) return launch_bits<BF16, 8, 3>(x, wq, s, s, M, N, K, gs, y, ws, cnt, st);
  if (gs == 16) return launch_bits<BF16, 4, 2>(x, wq, s, s, M, N, K, gs, y, ws, cnt, st);
  return launch_bits<BF16, 4, 1>(x, wq, s, s, M, N, K, gs, y, ws, cnt, st);
}

}  // namespace qmm
