// Quantized GEMV on the matrix cores for a few rows of x (M <= 16), f16 and
// bf16 (kernel template; instantiated by qmv_mfma_f16.hip, qmv_mfma_bf16.hip):
//   y[m, n] = sum_k x[m, k] * (s[n, g(k)] * q[n, k] + b[n, g(k)]),
// the product the quantized matmul computes (mlx affine_qmv / qmm_t, "Add the
// 3bit packed qmm_t"), with fp32 accumulation as the Metal qmv does (mlx PR
// 1061 item 2).
//
// MI355X design (wave64, gfx950):
//  * One workgroup = 16 wavefronts = 16 rows of W over the whole of K. A K
//    step is 4 consecutive 32-code chunks of each of the 16 rows; wavefront w
//    takes steps w, w+16, w+32, ... so that the 16 wavefronts stream one
//    contiguous run of every row at a time.
//  * Lane (n, g) = (lane % 16, lane / 16) loads chunk g of the step of row n
//    and dequantizes it into four 8-code B fragments of
//    v_mfma_f32_16x16x32_{f16,bf16}: MFMA i takes codes 8i..8i+7 of the four
//    chunks, so A lane (m, g) holds the matching 8 elements of row m of x in
//    natural order (rows m >= M repeat row M - 1 and feed only output rows
//    that are never stored). f16: magic pairs and packed f16
//    FMAs, one rounding of s*q+b. bf16 with 2, 3, 5 or 6 bits: s*q+b in
//    fp32 split into hi = bf16(w) and lo = bf16(w - hi), both multiplied (a
//    single bf16 rounding of the weights would cost ~1e-3 relative error).
//  * bf16 with 4- or 8-bit codes (exact codes): the MFMA multiplies the
//    codes themselves, which bf16 holds exactly, and the affine map is
//    applied per group to the fp32 result, sum_k x (s q + b) = s sum_k x q +
//    b sum_k x. For that every MFMA must stay inside one group: the four
//    lanes of a row exchange their chunks' 8-code pieces (a 4 x 4 transpose
//    across the wavefront's 16-lane rows with v_permlane32_swap and
//    v_permlane16_swap), so that MFMA i takes chunk i of the step. 4-bit
//    codes become bf16 128 + q by or-ing them into the mantissa of 128 (two
//    per instruction, codes k and k + 4 of the piece, so x is staged with
//    each 8-element piece in that order), 8-bit codes go through fp32; the
//    128 is taken back with b - 128 s. The group sums of x are formed once
//    per workgroup in LDS.
//  * The workgroup copies x[0:M] and the scales and biases of its 16 rows
//    into LDS once, with coalesced loads issued ahead of the weight loads; A
//    fragments, scales and biases are read from there. The number of vector
//    memory instructions per CU (and the cache lines each one touches) is
//    what limits a kernel this short, so none of these is loaded per
//    wavefront and step.
//  * Every weight load of a wavefront (W chunk, scale, bias) is issued before
//    any arithmetic: for K <= 8192 all of them are in flight at once (one
//    round, no filler loads); longer rows run as a ring of 3 steps. Loads go
//    through buffer resources, so that out-of-range elements (ragged N,
//    chunks past the row end) read zero without a branch or a memory access.
//    Byte offsets stay below 2^31 for K < kQmvMfmaMaxK; x[0:M] must fit in
//    LDS (qmv_mfma_fits).
//  * The 16 partial 16x16 tiles are summed through LDS and written as T.
//  * Layers with fewer than 256 row blocks split K over up to 8 workgroups
//    per row block (contiguous K ranges, so each copies only its part of x);
//    the last workgroup of a row block to finish adds the partial tiles.
#pragma once
#include "common.hpp"
#include "kernels.hpp"
#include "mfma_common.hpp"

namespace qmm {

// arguments of one MFMA GEMV call (shared by the f16 and bf16 units)
struct MvLaunch {
  const void *x, *s, *b;
  const uint32_t* wq;
  void* y;
  int M, N, K, gs;
  float* ws;        // split-K partial tiles and arrival counters
  unsigned* cnt;
};

namespace {

constexpr int kMvWaves = 16;                  // wavefronts per workgroup
constexpr int kMvThreads = kMvWaves * 64;
constexpr int kMvMaxXu = 8;                   // 16-byte x units per thread
constexpr int kMvMaxSb = 2;                   // 16-byte scale (and bias) units per thread

// Compiler fence between groups of loads: memory operations are not moved
// across it, so the groups issue in program order and a wait for one group
// leaves the later ones in flight.
__device__ __forceinline__ void load_fence() { asm volatile("; load fence" ::: "memory"); }

// W chunk of one lane (4*BITS bytes) from the buffer at byte offset off
template <int BITS>
__device__ __forceinline__ void load_wchunk_buf(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                                uint32_t w[BITS]) {
  if constexpr (BITS == 4 || BITS == 8) {
#pragma unroll
    for (int h = 0; h < BITS / 4; h++) {
      const u32x4_t u = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * h, 0, 0));
      w[4 * h] = u.x; w[4 * h + 1] = u.y; w[4 * h + 2] = u.z; w[4 * h + 3] = u.w;
    }
  } else if constexpr (BITS == 2 || BITS == 6) {
#pragma unroll
    for (int h = 0; h < BITS / 2; h++) {
      typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
      const u32x2_t u = __builtin_bit_cast(
          u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off + 8 * h, 0, 0));
      w[2 * h] = u.x; w[2 * h + 1] = u.y;
    }
  } else if constexpr (BITS == 3) {   // 12-byte chunks, 4-byte aligned: one 12-byte load
    typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));
    const u32x3_t u = __builtin_bit_cast(u32x3_t, __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, 0));
    w[0] = u.x; w[1] = u.y; w[2] = u.z;
  } else {   // 5 bits: 20-byte chunks, 4-byte aligned: a 16-byte and a 4-byte load
    const u32x4_t u = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
    w[4] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 16, 0, 0);
  }
}

// Round structure: DEPTH steps of a wavefront are in flight at once. With
// RING = false the kernel runs one round (every wavefront has at most DEPTH
// steps); with RING = true slot d is refilled with the step one round later
// right after it is consumed.
// vector-memory instructions of one W chunk load (load_wchunk_buf). Each is
// already the widest load of its bytes, so the compiler cannot merge them
// into fewer instructions: the x copy's vmcnt wait below counts on that (a
// count above the real one would let older x copies still be landing when
// the barrier passes).
template <int BITS>
constexpr int wchunk_loads() {
  return (BITS == 4 || BITS == 8) ? BITS / 4 : (BITS == 2 || BITS == 6) ? BITS / 2 : BITS == 3 ? 1 : 2;
}

typedef __attribute__((address_space(3))) void mv_lds_t;

// MT: 16-row tiles of x (1 or 2): with 2, rows 16..31 of x take a second A
// fragment and accumulator per MFMA, sharing the dequantized W fragment.
// XDMA: x is copied into LDS by buffer loads that write LDS directly (no
// register round trip, no LDS store instructions), in blocks of 512 elements
// of one row: the split's range is a power-of-two number of whole blocks
// (xb_log2 = log2 of blocks per row). x then stays in natural order, and the
// exact 4-bit path permutes each A fragment in registers instead.
template <class T, int BITS, int DEPTH, bool RING, bool XDMA, int MT>
__global__ __launch_bounds__(kMvThreads) void qmv_mfma_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wq,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases,
    uint16_t* __restrict__ y, int M, int N, int K, int gs_log2, uint32_t m2, int xu, int sbu,
    int ks, int sps, float* __restrict__ ws, unsigned* __restrict__ cnt, int xb_log2) {
  // x rows [M][klen + 8] (8 elements of padding per row spread the rows over
  // the LDS banks), then scales [16][G] and biases [16][G]; afterwards the
  // cross-wavefront reduction buffer
  extern __shared__ uint4 smem4[];
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem4);
  float* red = reinterpret_cast<float*>(smem4);

  constexpr bool kExact = __is_same(T, BF16) && (BITS == 4 || BITS == 8);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int rows = N - n0 < 16 ? N - n0 : 16;
  // split blockIdx.y of ks takes chunks [c0, c1): sps whole 4-chunk steps
  const int nch = K >> 5;
  const int split = blockIdx.y;
  const int c0 = 4 * sps * split;
  const int c1 = c0 + 4 * sps < nch ? c0 + 4 * sps : nch;
  const int nsteps = (c1 - c0 + 3) >> 2;
  const int nsw = wave < nsteps ? (nsteps - wave + kMvWaves - 1) / kMvWaves : 0;
  const int G = K >> gs_log2;
  const int klen = (c1 - c0) * 32;
  const int ldx = klen + 8;
  const uint32_t row_bytes = (uint32_t)K * BITS / 8;

  // Buffers over this workgroup's rows of W / scales / biases and over x:
  // offsets past their ends read zeros without a branch, which covers rows
  // n >= N of the last row block and chunks past the row end (weight 0 from
  // zero codes, scale and bias).
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(wq + (int64_t)n0 * row_bytes, rows * row_bytes);
  // scales and biases of the 16 rows: 16*G contiguous halfs each, read as
  // aligned 16-byte units that cover them (the range is widened to 16-byte
  // boundaries at both ends; the extra bytes lie in the aligned blocks of
  // the first and the last scale, so in mapped pages, and only feed rows or
  // groups that are never used). The LDS copy keeps the offset sd / bd of
  // the first scale / bias within its unit.
  const uintptr_t sp = reinterpret_cast<uintptr_t>(scales + (int64_t)n0 * G);
  const uintptr_t bp = reinterpret_cast<uintptr_t>(biases + (int64_t)n0 * G);
  const uint32_t sd = sp & 15, bd = bp & 15;
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(reinterpret_cast<const void*>(sp - sd),
                                              (sd + rows * G * 2 + 15) & ~15u);
  const __amdgpu_buffer_rsrc_t br = make_rsrc(reinterpret_cast<const void*>(bp - bd),
                                              (bd + rows * G * 2 + 15) & ~15u);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)M * K * 2);
  const uint32_t wbase = n * row_bytes;
  const int sbun = (15 + 32 * G + 15) >> 4;   // 16-byte units per array
  uint4* ss4 = smem4 + (((size_t)M * ldx + 7) >> 3);
  uint4* bs4 = ss4 + sbun;
  const uint8_t* ssb = reinterpret_cast<const uint8_t*>(ss4) + sd;
  const uint8_t* bsb = reinterpret_cast<const uint8_t*>(bs4) + bd;

  // ---- x loads first (the weight loads queue behind them): 16-byte units
  // u = tid + 1024 i for i < xu of the split's K range of every row
  // (row m and unit kk of unit u stepped from one division: u grows by 1024)
  const int xrow_units = klen >> 3, xunits = M * xrow_units;
  const int dq = kMvThreads / xrow_units, dr = kMvThreads - dq * xrow_units;
  uint4 xl[XDMA ? 1 : kMvMaxXu];
  uint32_t xoff[XDMA ? 1 : kMvMaxXu], xlds[XDMA ? 1 : kMvMaxXu];
  if constexpr (XDMA) {
    // block b = wave + 16 i: part b % bpr of row b / bpr (uniform per
    // wavefront), 64 lanes x 16 bytes
    const int nxb = M << xb_log2;
    const int wu = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
    for (int i = 0; i < kMvMaxXu; i++) {
      const int b = wu + kMvWaves * i;
      if (b < nxb) {
        const int m = b >> xb_log2, p = b & ((1 << xb_log2) - 1);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            xr, (mv_lds_t*)(xs + m * ldx + p * 512), 16, lane * 16,
            (int)(((uint32_t)m * K + c0 * 32 + p * 512) * 2), 0, 0);
      }
    }
  } else {
    int m = tid / xrow_units, kk = tid - m * xrow_units;
#pragma unroll
    for (int i = 0; i < kMvMaxXu; i++) {
      const int u = tid + kMvThreads * i;
      xoff[i] = u < xunits ? ((uint32_t)m * K + c0 * 32 + kk * 8) * 2 : kOob;
      xlds[i] = (uint32_t)(m * ldx + kk * 8);
      m += dq;
      kk += dr;
      if (kk >= xrow_units) { kk -= xrow_units; m++; }
    }
#pragma unroll
    for (int i = 0; i < kMvMaxXu; i++) {
      if (i < xu) {
        const u32x4_t v = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(xr, xoff[i], 0, 0));
        xl[i] = make_uint4(v.x, v.y, v.z, v.w);
      }
    }
  }
  // scale and bias units (rows past N read zero), sbu per thread
  uint4 sl[kMvMaxSb], bl[kMvMaxSb];
  uint32_t soff[kMvMaxSb];
#pragma unroll
  for (int i = 0; i < kMvMaxSb; i++) {
    const int u = tid + kMvThreads * i;
    soff[i] = u < sbun ? (uint32_t)u * 16 : kOob;
  }
#pragma unroll
  for (int i = 0; i < kMvMaxSb; i++) {
    if (i < sbu) {
      const u32x4_t v =
          __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(sr, soff[i], 0, 0));
      const u32x4_t w =
          __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(br, soff[i], 0, 0));
      sl[i] = make_uint4(v.x, v.y, v.z, v.w);
      bl[i] = make_uint4(w.x, w.y, w.z, w.w);
    }
  }
  load_fence();
  __builtin_amdgcn_sched_barrier(0);

  uint32_t wv[DEPTH][BITS];

  auto issue = [&](int j, int d) QMM_INLINE {
    const int c = c0 + 4 * (wave + kMvWaves * j) + g;
    // kOob when c >= c1, else 0 (a mask, not a select: the compiler would
    // turn a select of two offsets into a branch around two loads)
    const uint32_t oob = (uint32_t)((c1 - 1 - c) >> 31) & kOob;
    load_wchunk_buf<BITS>(wr, (wbase + c * (4 * BITS)) | oob, wv[d]);
  };

#pragma unroll
  for (int d = 0; d < DEPTH; d++) {
    issue(d, d);
    load_fence();
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- x, scales and biases into LDS (waits for those loads only: they
  // were issued first)
  if constexpr (!XDMA) {
#pragma unroll
    for (int i = 0; i < kMvMaxXu; i++) {
      const int u = tid + kMvThreads * i;
      uint4 v = xl[i];
      if constexpr (kExact && BITS == 4)   // piece order 0 4 1 5 2 6 3 7
        v = make_uint4(__builtin_amdgcn_perm(v.z, v.x, 0x05040100u),
                       __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                       __builtin_amdgcn_perm(v.w, v.y, 0x05040100u),
                       __builtin_amdgcn_perm(v.w, v.y, 0x07060302u));
      if (i < xu && u < xunits) *reinterpret_cast<uint4*>(xs + xlds[i]) = v;
    }
  }
#pragma unroll
  for (int i = 0; i < kMvMaxSb; i++) {
    const int u = tid + kMvThreads * i;
    if (i < sbu && u < sbun) {
      ss4[u] = sl[i];
      bs4[u] = bl[i];
    }
  }
  if constexpr (XDMA) {
    // every copy and load older than the weight loads (the youngest
    // DEPTH * wchunk_loads of this wavefront) has landed, the LDS stores
    // have completed, then the barrier; no fence, which would also wait for
    // the weight loads
    constexpr int kW = DEPTH * wchunk_loads<BITS>();
    static_assert(kW < 64, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((kW & 15) | ((kW >> 4) << 14) | (7 << 4));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  } else {
    __syncthreads();
  }

  // exact codes: xg[gl][m] = sum of x[m] over group gl of the split's range
  // (16 MT rows, rows >= M zero), after the scales and biases
  constexpr int XR = 16 * MT;
  float* xg = reinterpret_cast<float*>(bs4 + sbun);
  if constexpr (kExact) {
    const int ngl = (klen + (1 << gs_log2) - 1) >> gs_log2;
    for (int t = tid; t < ngl * XR; t += kMvThreads) {
      const int m = t & (XR - 1), gl = t / XR;
      // (pairs of x times bf16 (1, 1) by v_dot2: exact products, fp32 sums
      // in four chains)
      float s4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (m < M) {
        const uint4* xp = reinterpret_cast<const uint4*>(xs + m * ldx + (gl << gs_log2));
        for (int u = 0; u < (1 << gs_log2) / 8; u++) {
          const uint4 v = xp[u];
          s4[0] = dot2(BF16{}, v.x, 0x3F803F80u, s4[0]);
          s4[1] = dot2(BF16{}, v.y, 0x3F803F80u, s4[1]);
          s4[2] = dot2(BF16{}, v.z, 0x3F803F80u, s4[2]);
          s4[3] = dot2(BF16{}, v.w, 0x3F803F80u, s4[3]);
        }
      }
      xg[t] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    }
    __syncthreads();
  }

  float4_t acc[MT];
#pragma unroll
  for (int h = 0; h < MT; h++) acc[h] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  // exact codes: chunk i of the step on MFMA i (see the header), groups of
  // gs codes applied to the fp32 sums as s * D + (b - 128 s) * sum(x)
  uint32_t magic_x = 0x43004300u;   // bf16 (128, 128)
  if constexpr (__is_same(T, BF16)) asm volatile("v_mov_b32 %0, %1" : "=v"(magic_x) : "i"(0x43004300));
  auto compute_exact = [&](int j, int d) QMM_INLINE {
    const int cs = c0 + 4 * (wave + kMvWaves * j);   // the step's first chunk
    uint32_t t[BITS];
#pragma unroll
    for (int q = 0; q < BITS; q++) t[q] = wv[d][q];
    // 4 x 4 transpose of 8-code pieces across the 16-lane rows g: row g held
    // chunk g's pieces 0..3, it gets piece g of chunks 0..3 (per word of a
    // piece: W = BITS / 4 words)
    constexpr int W = BITS / 4;
#pragma unroll
    for (int w = 0; w < W; w++) {
      auto r = __builtin_amdgcn_permlane32_swap(t[w], t[2 * W + w], false, false);
      t[w] = r[0]; t[2 * W + w] = r[1];
      r = __builtin_amdgcn_permlane32_swap(t[W + w], t[3 * W + w], false, false);
      t[W + w] = r[0]; t[3 * W + w] = r[1];
      r = __builtin_amdgcn_permlane16_swap(t[w], t[W + w], false, false);
      t[w] = r[0]; t[W + w] = r[1];
      r = __builtin_amdgcn_permlane16_swap(t[2 * W + w], t[3 * W + w], false, false);
      t[2 * W + w] = r[0]; t[3 * W + w] = r[1];
    }
    // chunks per group (1, 2 or 4) as a compile-time count, so that the
    // group ends are fixed places in the unrolled chunk loop
    auto chunks = [&]<int CPG>() QMM_INLINE {
      float4_t dsum[MT];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int c = cs + i;
        const int cx = c < c1 ? c : c1 - 1;
        uint4 a[MT];
#pragma unroll
        for (int h = 0; h < MT; h++) {
          // (rows m >= M repeat row M - 1: they only feed output rows that
          // are never stored)
          const int mr = n + 16 * h < M ? n + 16 * h : M - 1;
          a[h] = *reinterpret_cast<const uint4*>(xs + mr * ldx + (cx - c0) * 32 + 8 * g);
          if constexpr (XDMA && BITS == 4)   // copied in natural order: piece order 0 4 1 5 2 6 3 7
            a[h] = make_uint4(__builtin_amdgcn_perm(a[h].z, a[h].x, 0x05040100u),
                              __builtin_amdgcn_perm(a[h].z, a[h].x, 0x07060302u),
                              __builtin_amdgcn_perm(a[h].w, a[h].y, 0x05040100u),
                              __builtin_amdgcn_perm(a[h].w, a[h].y, 0x07060302u));
        }
        uint4 b;
        if constexpr (BITS == 4) {
          // 128 + q: each code pair or-ed into the mantissas of bf16 (128, 128)
          // (mask in an SGPR, pattern in a VGPR: one v_and_or_b32 per pair)
          const uint32_t w = t[i];
          b = make_uint4((w & m2) | magic_x, ((w >> 4) & m2) | magic_x,
                         ((w >> 8) & m2) | magic_x, ((w >> 12) & m2) | magic_x);
        } else {
          uint32_t p[4];
#pragma unroll
          for (int h = 0; h < 2; h++) {
            const uint32_t w = t[2 * i + h];
            const float f0 = (float)(w & 0xff), f1 = (float)((w >> 8) & 0xff),
                        f2 = (float)((w >> 16) & 0xff), f3 = (float)(w >> 24);
            p[2 * h] = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, f1),
                                             __builtin_bit_cast(uint32_t, f0), 0x07060302u);
            p[2 * h + 1] = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, f3),
                                                 __builtin_bit_cast(uint32_t, f2), 0x07060302u);
          }
          b = make_uint4(p[0], p[1], p[2], p[3]);
        }
#pragma unroll
        for (int h = 0; h < MT; h++)
          dsum[h] = mfma16(BF16{}, a[h], b, i % CPG == 0 ? float4_t{0.0f, 0.0f, 0.0f, 0.0f} : dsum[h]);
        if ((i + 1) % CPG == 0) {
          // end of a group: its scale and bias (zero past the split's end)
          const uint32_t keep = ~(uint32_t)((c1 - 1 - c) >> 31);
          const int gi = 2 * (n * G + ((cx << 5) >> gs_log2));
          const float sf = to_f32(BF16{}, (uint16_t)(*reinterpret_cast<const uint16_t*>(ssb + gi) & keep));
          const float bfl = to_f32(BF16{}, (uint16_t)(*reinterpret_cast<const uint16_t*>(bsb + gi) & keep));
          const float bq = bfl - 128.0f * sf * (BITS == 4 ? 1.0f : 0.0f);
#pragma unroll
          for (int h = 0; h < MT; h++) {
            const float4_t xsum = *reinterpret_cast<const float4_t*>(
                xg + (((cx - c0) << 5) >> gs_log2) * XR + 16 * h + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; e++) acc[h][e] = fmaf(bq, xsum[e], fmaf(sf, dsum[h][e], acc[h][e]));
          }
        }
      }
    };
    if (gs_log2 == 5) chunks.template operator()<1>();
    else if (gs_log2 == 6) chunks.template operator()<2>();
    else chunks.template operator()<4>();
  };

  // The magic pattern lives in a VGPR so that each magic pair is one
  // v_and_or_b32 (with the mask in an SGPR; a VOP3 reads one SGPR at most
  // and no literal on gfx9, so a literal pattern costs an and and an or).
  uint32_t magic_v = F16::kMagic;
  if constexpr (__is_same(T, F16)) asm volatile("v_mov_b32 %0, %1" : "=v"(magic_v) : "i"(F16::kMagic));
  auto compute = [&](int j, int d) QMM_INLINE {
    // A fragments: lane (m, g) = (n, g) takes 8 elements of row m of x
    // (rows m >= M stay zero); the chunk is clamped into the row (a chunk
    // past the end has zero weights)
    // (scale and bias are zeroed too: the chunk's codes read zero, and
    // s*0 + b must be 0 as well)
    const int c = c0 + 4 * (wave + kMvWaves * j) + g;
    const int cx = c < c1 ? c : c1 - 1;
    const uint32_t keep = ~(uint32_t)((c1 - 1 - c) >> 31);   // 0 past the split's end
    const int gi = 2 * (n * G + ((cx << 5) >> gs_log2));
    const uint32_t sh = *reinterpret_cast<const uint16_t*>(ssb + gi) & keep;
    const uint32_t bh = *reinterpret_cast<const uint16_t*>(bsb + gi) & keep;
    // (rows m >= M of the A fragment repeat row M - 1: they only feed
    // output rows that are never stored)
    uint4 a[MT][4];
#pragma unroll
    for (int h = 0; h < MT; h++) {
      const int mr = n + 16 * h < M ? n + 16 * h : M - 1;
      const uint4* xp = reinterpret_cast<const uint4*>(xs + mr * ldx + (cx - c0) * 32);
#pragma unroll
      for (int i = 0; i < 4; i++) a[h][i] = xp[i];
    }
    if constexpr (__is_same(T, F16)) {
      uint32_t bf[16];
      [&]<int... C>(std::integer_sequence<int, C...>) QMM_INLINE {
        (dequant_piece_f16_pk<BITS, C * piece_codes<BITS>(), piece_codes<BITS>()>(
             wv[d], sh * 0x10001u, bh * 0x10001u, m2, magic_v, bf),
         ...);
      }(std::make_integer_sequence<int, 32 / piece_codes<BITS>()>{});
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const uint4 b = make_uint4(bf[4 * i], bf[4 * i + 1], bf[4 * i + 2], bf[4 * i + 3]);
#pragma unroll
        for (int h = 0; h < MT; h++) acc[h] = mfma16(F16{}, a[h][i], b, acc[h]);
      }
    } else {
      const float sf = to_f32(BF16{}, (uint16_t)sh), bfl = to_f32(BF16{}, (uint16_t)bh);
      uint32_t hi[16], lo[16];
      dequant_piece_bf16<BITS, 0>(wv[d], sf, bfl, hi, lo);
      dequant_piece_bf16<BITS, 8>(wv[d], sf, bfl, hi, lo);
      dequant_piece_bf16<BITS, 16>(wv[d], sf, bfl, hi, lo);
      dequant_piece_bf16<BITS, 24>(wv[d], sf, bfl, hi, lo);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const uint4 bh = make_uint4(hi[4 * i], hi[4 * i + 1], hi[4 * i + 2], hi[4 * i + 3]);
        const uint4 bl = make_uint4(lo[4 * i], lo[4 * i + 1], lo[4 * i + 2], lo[4 * i + 3]);
#pragma unroll
        for (int h = 0; h < MT; h++) {
          acc[h] = mfma16(BF16{}, a[h][i], bh, acc[h]);
          acc[h] = mfma16(BF16{}, a[h][i], bl, acc[h]);
        }
      }
    }
  };

  auto step = [&](int j, int d) QMM_INLINE {
    if constexpr (kExact) compute_exact(j, d);
    else compute(j, d);
  };
  if constexpr (!RING) {
#pragma unroll
    for (int d = 0; d < DEPTH; d++) {
      step(d, d);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    // at least one round runs (a wavefront without steps multiplies zeros),
    // so that no branch precedes the loop
    const int nr = nsw > DEPTH ? (nsw + DEPTH - 1) / DEPTH : 1;
    int r = 0;
    do {
#pragma unroll
      for (int d = 0; d < DEPTH; d++) {
        step(r * DEPTH + d, d);
        __builtin_amdgcn_sched_barrier(0);
        issue((r + 1) * DEPTH + d, d);
        load_fence();
        __builtin_amdgcn_sched_barrier(0);
      }
    } while (++r < nr);
  }

  // ---- sum the 16 wavefront tiles (the buffer overlays x: barrier first);
  // tile h holds D[m][n] with m = 16 h + 4*(lane/16) + e; thread t < 256 MT
  // sums element t % 256 of tile t / 256
  __syncthreads();
#pragma unroll
  for (int h = 0; h < MT; h++)
#pragma unroll
    for (int e = 0; e < 4; e++) red[h * kMvThreads * 4 + (wave * 64 + lane) * 4 + e] = acc[h][e];
  __syncthreads();
  constexpr int kOut = 256 * MT;   // outputs of the workgroup's tiles
  const int th = tid >> 8, tl = tid & 255;
  const int ln = tl >> 2, e = tl & 3;
  const int m = 16 * th + 4 * (ln >> 4) + e, col = n0 + (ln & 15);
  float v = 0.0f;
  if (tid < kOut) {
#pragma unroll
    for (int w = 0; w < kMvWaves; w++) v += red[th * kMvThreads * 4 + w * 256 + tl];
  }
  if (ks == 1) {
    if (tid < kOut && m < M && col < N) y[(int64_t)m * N + col] = from_f32(T{}, v);
    return;
  }
  // ---- K split over ks workgroups: each writes its 16 x 16 partial tile to
  // the workspace; the last one to arrive at its row block's counter adds
  // the ks tiles in split order and writes y. The counter update is a
  // wrapping increment with limit ks - 1 (0, 1, ..., ks - 1, then back to 0),
  // so the last arrival itself leaves the counter at zero for the next call:
  // there is no separate reset store for an overlapping call to race with.
  // Tiles and counter use device-scope atomic accesses, which are
  // coherent across the per-XCD L2 caches (so no fence has to write back a
  // whole L2): every thread's stores have completed before the barrier that
  // precedes the counter update, and the last workgroup reads the tiles only
  // after its update has returned.
  __shared__ unsigned last;
  float* wsb = ws + (int64_t)blockIdx.x * ks * kOut;
  if (tid < kOut) __hip_atomic_store(wsb + split * kOut + tid, v, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0);   // vmcnt(0): the stores have completed
  __syncthreads();
  if (tid == 0)
    last = __builtin_amdgcn_atomic_inc32(cnt + blockIdx.x, (unsigned)(ks - 1), __ATOMIC_RELAXED,
                                         "agent") == (unsigned)(ks - 1);
  __syncthreads();
  if (!last) return;
  if (tid < kOut) {
    float t = 0.0f;
    for (int sp = 0; sp < ks; sp++)
      t += __hip_atomic_load(wsb + sp * kOut + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (m < M && col < N) y[(int64_t)m * N + col] = from_f32(T{}, t);
  }
}

template <class T, int BITS, int DEPTH, bool RING>
hipError_t launch_depth(const MvLaunch& L, const QmvMfmaPlan& p, hipStream_t st) {
  constexpr bool kExact = __is_same(T, BF16) && (BITS == 4 || BITS == 8);
  const uint32_t m2 = Pack<BITS>::kMask | (Pack<BITS>::kMask << 16);
  const int xu = (L.M * (p.klen / 8) + kMvThreads - 1) / kMvThreads;
  const int sbu = ((15 + 32 * (L.K / L.gs) + 15) / 16 + kMvThreads - 1) / kMvThreads;
  const size_t lds = qmv_mfma_lds(L.M, p.klen, L.K, L.gs, kExact);
  // direct x copies: every split's range (all of the same length) is whole
  // 512-element blocks, a power of two of them per row, at most 8 per
  // wavefront
  const int bpr = p.klen / 512;
  const bool xdma = p.klen % 512 == 0 && (int64_t)p.ks * p.klen == L.K &&
                    (bpr & (bpr - 1)) == 0 && L.M * bpr <= kMvWaves * kMvMaxXu;
  auto go = [&]<bool XD, int MT>() {
    hipLaunchKernelGGL((qmv_mfma_kernel<T, BITS, DEPTH, RING, XD, MT>), dim3((L.N + 15) / 16, p.ks),
                       dim3(kMvThreads), lds, st, static_cast<const uint16_t*>(L.x),
                       reinterpret_cast<const uint8_t*>(L.wq), static_cast<const uint16_t*>(L.s),
                       static_cast<const uint16_t*>(L.b), static_cast<uint16_t*>(L.y), L.M, L.N,
                       L.K, ilog2(L.gs), m2, xu, sbu, p.ks, p.sps, L.ws, L.cnt,
                       xdma ? ilog2(bpr) : 0);
  };
  if (L.M > 16) {
    if (xdma) go.template operator()<true, 2>();
    else go.template operator()<false, 2>();
  } else {
    if (xdma) go.template operator()<true, 1>();
    else go.template operator()<false, 1>();
  }
  return hipGetLastError();
}

// one round when every wavefront has at most 4 steps of its split, else a
// ring of 3 steps
template <class T, int BITS>
hipError_t launch_bits(const MvLaunch& L, hipStream_t st) {
  const QmvMfmaPlan p = qmv_mfma_plan(L.N, L.K, L.M);
  const int nsw = (p.sps + kMvWaves - 1) / kMvWaves;
  if (nsw <= 1) return launch_depth<T, BITS, 1, false>(L, p, st);
  if (nsw <= 2) return launch_depth<T, BITS, 2, false>(L, p, st);
  if (nsw <= 4) return launch_depth<T, BITS, 4, false>(L, p, st);
  return launch_depth<T, BITS, 3, true>(L, p, st);
}

// all widths, one element type
template <class T>
hipError_t launch_qmv_mfma_t(int bits, const MvLaunch& L, hipStream_t st) {
  switch (bits) {
    case 2: return launch_bits<T, 2>(L, st);
    case 3: return launch_bits<T, 3>(L, st);
    case 4: return launch_bits<T, 4>(L, st);
    case 5: return launch_bits<T, 5>(L, st);
    case 6: return launch_bits<T, 6>(L, st);
    default: return launch_bits<T, 8>(L, st);
  }
}

}  // namespace
}  // namespace qmm
