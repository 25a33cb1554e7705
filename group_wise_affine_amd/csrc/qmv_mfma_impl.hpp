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
//    natural order (rows m >= M stay zero). f16: magic pairs and packed f16
//    FMAs, one rounding of s*q+b. bf16: s*q+b in fp32 split into
//    hi = bf16(w) and lo = bf16(w - hi), both multiplied (a single bf16
//    rounding of the weights would cost ~1e-3 relative error).
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
  } else {  // 3 and 5 bits: 4-byte aligned chunks
#pragma unroll
    for (int i = 0; i < BITS; i++) w[i] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 4 * i, 0, 0);
  }
}

// Round structure: DEPTH steps of a wavefront are in flight at once. With
// RING = false the kernel runs one round (every wavefront has at most DEPTH
// steps); with RING = true slot d is refilled with the step one round later
// right after it is consumed.
template <class T, int BITS, int DEPTH, bool RING>
__global__ __launch_bounds__(kMvThreads) void qmv_mfma_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wq,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases,
    uint16_t* __restrict__ y, int M, int N, int K, int gs_log2, uint32_t m2, int xu, int sbu,
    int ks, int sps, float* __restrict__ ws, unsigned* __restrict__ cnt) {
  // x rows [M][klen + 8] (8 elements of padding per row spread the rows over
  // the LDS banks), then scales [16][G] and biases [16][G]; afterwards the
  // cross-wavefront reduction buffer
  extern __shared__ uint4 smem4[];
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem4);
  float* red = reinterpret_cast<float*>(smem4);

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
  uint4 xl[kMvMaxXu];
  uint32_t xoff[kMvMaxXu], xlds[kMvMaxXu];
  {
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
  }
#pragma unroll
  for (int i = 0; i < kMvMaxXu; i++) {
    if (i < xu) {
      const u32x4_t v =
          __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(xr, xoff[i], 0, 0));
      xl[i] = make_uint4(v.x, v.y, v.z, v.w);
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
#pragma unroll
  for (int i = 0; i < kMvMaxXu; i++) {
    const int u = tid + kMvThreads * i;
    if (i < xu && u < xunits) *reinterpret_cast<uint4*>(xs + xlds[i]) = xl[i];
  }
#pragma unroll
  for (int i = 0; i < kMvMaxSb; i++) {
    const int u = tid + kMvThreads * i;
    if (i < sbu && u < sbun) {
      ss4[u] = sl[i];
      bs4[u] = bl[i];
    }
  }
  __syncthreads();

  float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
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
    uint4 a[4];
#pragma unroll
    for (int i = 0; i < 4; i++) a[i] = make_uint4(0, 0, 0, 0);
    if (n < M) {
      const uint4* xp = reinterpret_cast<const uint4*>(xs + n * ldx + (cx - c0) * 32);
#pragma unroll
      for (int i = 0; i < 4; i++) a[i] = xp[i];
    }
    if constexpr (__is_same(T, F16)) {
      uint32_t bf[16];
      [&]<int... C>(std::integer_sequence<int, C...>) QMM_INLINE {
        (dequant_piece_f16_pk<BITS, C * piece_codes<BITS>(), piece_codes<BITS>()>(
             wv[d], sh * 0x10001u, bh * 0x10001u, m2, F16::kMagic, bf),
         ...);
      }(std::make_integer_sequence<int, 32 / piece_codes<BITS>()>{});
#pragma unroll
      for (int i = 0; i < 4; i++)
        acc = mfma16(F16{}, a[i],
                     make_uint4(bf[4 * i], bf[4 * i + 1], bf[4 * i + 2], bf[4 * i + 3]), acc);
    } else {
      const float sf = to_f32(BF16{}, (uint16_t)sh), bfl = to_f32(BF16{}, (uint16_t)bh);
      uint32_t hi[16], lo[16];
      dequant_piece_bf16<BITS, 0>(wv[d], sf, bfl, hi, lo);
      dequant_piece_bf16<BITS, 8>(wv[d], sf, bfl, hi, lo);
      dequant_piece_bf16<BITS, 16>(wv[d], sf, bfl, hi, lo);
      dequant_piece_bf16<BITS, 24>(wv[d], sf, bfl, hi, lo);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        acc = mfma16(BF16{}, a[i],
                     make_uint4(hi[4 * i], hi[4 * i + 1], hi[4 * i + 2], hi[4 * i + 3]), acc);
        acc = mfma16(BF16{}, a[i],
                     make_uint4(lo[4 * i], lo[4 * i + 1], lo[4 * i + 2], lo[4 * i + 3]), acc);
      }
    }
  };

  if constexpr (!RING) {
#pragma unroll
    for (int d = 0; d < DEPTH; d++) {
      compute(d, d);
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
        compute(r * DEPTH + d, d);
        __builtin_amdgcn_sched_barrier(0);
        issue((r + 1) * DEPTH + d, d);
        load_fence();
        __builtin_amdgcn_sched_barrier(0);
      }
    } while (++r < nr);
  }

  // ---- sum the 16 wavefront tiles (the buffer overlays x: barrier first);
  // D[m][n] with m = 4*(lane/16) + e
  __syncthreads();
#pragma unroll
  for (int e = 0; e < 4; e++) red[(wave * 64 + lane) * 4 + e] = acc[e];
  __syncthreads();
  const int ln = tid >> 2, e = tid & 3;
  const int m = 4 * (ln >> 4) + e, col = n0 + (ln & 15);
  float v = 0.0f;
  if (tid < 256) {
#pragma unroll
    for (int w = 0; w < kMvWaves; w++) v += red[w * 256 + tid];
  }
  if (ks == 1) {
    if (tid < 256 && m < M && col < N) y[(int64_t)m * N + col] = from_f32(T{}, v);
    return;
  }
  // ---- K split over ks workgroups: each writes its 16 x 16 partial tile to
  // the workspace; the last one to arrive at its row block's counter adds
  // the ks tiles in split order, writes y and resets the counter for the
  // next call. Tiles and counter use device-scope atomic accesses, which are
  // coherent across the per-XCD L2 caches (so no fence has to write back a
  // whole L2): every thread's stores have completed before the barrier that
  // precedes the counter update, and the last workgroup reads the tiles only
  // after its update has returned.
  __shared__ unsigned last;
  float* wsb = ws + (int64_t)blockIdx.x * ks * 256;
  if (tid < 256) __hip_atomic_store(wsb + split * 256 + tid, v, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0);   // vmcnt(0): the stores have completed
  __syncthreads();
  if (tid == 0)
    last = __hip_atomic_fetch_add(cnt + blockIdx.x, 1u, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(ks - 1);
  __syncthreads();
  if (!last) return;
  if (tid < 256) {
    float t = 0.0f;
    for (int sp = 0; sp < ks; sp++)
      t += __hip_atomic_load(wsb + sp * 256 + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (m < M && col < N) y[(int64_t)m * N + col] = from_f32(T{}, t);
  }
  if (tid == 0) __hip_atomic_store(cnt + blockIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class T, int BITS, int DEPTH, bool RING>
hipError_t launch_depth(const MvLaunch& L, const QmvMfmaPlan& p, hipStream_t st) {
  const uint32_t m2 = Pack<BITS>::kMask | (Pack<BITS>::kMask << 16);
  const int xu = (L.M * (p.klen / 8) + kMvThreads - 1) / kMvThreads;
  const int sbu = ((15 + 32 * (L.K / L.gs) + 15) / 16 + kMvThreads - 1) / kMvThreads;
  hipLaunchKernelGGL((qmv_mfma_kernel<T, BITS, DEPTH, RING>), dim3((L.N + 15) / 16, p.ks),
                     dim3(kMvThreads), qmv_mfma_lds(L.M, p.klen, L.K, L.gs), st,
                     static_cast<const uint16_t*>(L.x), reinterpret_cast<const uint8_t*>(L.wq),
                     static_cast<const uint16_t*>(L.s), static_cast<const uint16_t*>(L.b),
                     static_cast<uint16_t*>(L.y), L.M, L.N, L.K, ilog2(L.gs), m2, xu, sbu, p.ks,
                     p.sps, L.ws, L.cnt);
  return hipGetLastError();
}

// one round when every wavefront has at most 4 steps of its split, else a
// ring of 3 steps
template <class T, int BITS>
hipError_t launch_bits(const MvLaunch& L, hipStream_t st) {
  const QmvMfmaPlan p = qmv_mfma_plan(L.N, L.K);
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
