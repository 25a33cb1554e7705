// Streaming quantized GEMV for small M (decode):
//   y[m, n] = sum_g ( s[n,g] * sum_{k in g} x[m,k] q[n,k]
//                   + b[n,g] * sum_{k in g} x[m,k] ),
// the group factorisation of y = x . (s*q + b)^T used by the Metal qmv in
// "Add the 3bit packed qmm_t" (affine_packed_qmv_fast_impl: result += s*accum
// + b*sum) with fp32 accumulation ("everything is float32" in qmv, mlx PR
// 1061 item 2).
//
// MI355X design (wave64):
//  * Each workgroup first stages up to MB rows of x into LDS, already
//    permuted into the pair order the weight unpacker produces (see
//    common.hpp), together with the fp32 sum of every 32-element chunk.
//    When a row fits one batch of lane loads (K <= 16384) and scales and
//    biases are 16-byte aligned, the scales and biases of the workgroup's
//    rows (one contiguous run of each array) are staged too, with 16-byte
//    loads; the W wavefronts then issue nothing but their weight loads.
//  * A row of W is split over TPR lanes of one wavefront (64/TPR rows per
//    wavefront); a lane walks the row in 32-code chunks (4*bits bytes,
//    16 bytes at 4 bits) with stride TPR chunks, so a wavefront load covers
//    64/TPR contiguous row segments of TPR*4*bits bytes each.
//  * Codes become exact f16/bf16 values MAGIC + q*2^o with at most one
//    shift and one and-or per pair, and v_dot2_f32_{f16,bf16} multiplies
//    them with the unscaled activation pairs in fp32, one set of partial
//    sums per field offset o, each scaled by 2^-o in fp32 (exact). The MAGIC
//    offset is removed through a per-chunk constant: sum(x*(MAGIC*2^-o + q))
//    - MAGIC*sum(x*2^-o) = sum(x*q). Activations are never rounded again, so
//    small f16 inputs keep every bit.
//  * Every W byte is read once per MB rows of x; one pass serves all of them.
//  * Lanes of a row reduce with DPP moves inside a 16-lane row and lane
//    shuffles across rows; lane 0 writes y.
//  * Gathered products (a compile-time variant): a third grid dimension over
//    products, each with its own batch of x and of W (scales, biases) and y.
#include <utility>

#include "common.hpp"
#include "kernels.hpp"

namespace qmm {

template <class T, int BITS>
struct QmvCfg {
  // bf16 cannot hold 128 + q exactly for 8-bit codes: that case runs in fp32
  static constexpr bool kF32 = (BITS == 8) && __is_same(T, BF16);
  static constexpr int kXWords = kF32 ? 32 : 16;  // LDS words per x chunk
  // LDS record of a chunk: its activations, then the chunk sum and the magic
  // offset (padded to 16 bytes), so that one address serves all of them
  static constexpr int kXRec = kXWords + 4;
};

// Weight chunks are read exactly once per call: nontemporal loads stream
// them past the caches, which keeps x, scales and biases resident in L2.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <int BITS>
__device__ __forceinline__ void load_chunk(const uint8_t* p, uint32_t w[BITS]) {
  if constexpr (BITS == 4 || BITS == 8) {
#pragma unroll
    for (int h = 0; h < BITS / 4; h++) {
      const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + h);
      w[4 * h] = u.x; w[4 * h + 1] = u.y; w[4 * h + 2] = u.z; w[4 * h + 3] = u.w;
    }
  } else if constexpr (BITS == 2 || BITS == 6) {
#pragma unroll
    for (int h = 0; h < BITS / 2; h++) {
      const u32x2 u = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p) + h);
      w[2 * h] = u.x; w[2 * h + 1] = u.y;
    }
  } else {  // 3 and 5 bits: 4-byte aligned chunks
#pragma unroll
    for (int i = 0; i < BITS; i++)
      w[i] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p) + i);
  }
}

// d[r] = sum over the chunk of x_pair . (MAGIC + q*2^o)_pair * 2^-o for each
// of the R rows of a lane, in fp32. The products of each offset class are
// summed apart (dot2 sums of unscaled activations) and the class sums are
// scaled by 2^-o in fp32, which is exact, so no activation is ever rounded
// again. One wavefront per SIMD runs this, so the dot2 instructions form at
// least NP independent chains per row (split over the classes) rather than
// one dependent chain.
template <class T, int BITS, int R, int NP>
__device__ __forceinline__ void chunk_dot_rows(const uint32_t (*pairs)[16], const uint32_t* xp,
                                               float* d) {
  constexpr int NC = n_off_classes<T, BITS>();
  constexpr int NPC = NP / NC >= 1 ? NP / NC : 1;  // chains per class
  float part[R][NC][NPC];
#pragma unroll
  for (int r = 0; r < R; r++)
#pragma unroll
    for (int c = 0; c < NC; c++)
#pragma unroll
      for (int j = 0; j < NPC; j++) part[r][c][j] = 0.0f;
  [&]<int... P>(std::integer_sequence<int, P...>) {
    ([&]() {
       constexpr int c = off_class<T, BITS>(P), j = rank_in_class<T, BITS>(P) % NPC;
#pragma unroll
       for (int r = 0; r < R; r++) part[r][c][j] = dot2(T{}, pairs[r][P], xp[P], part[r][c][j]);
     }(),
     ...);
  }(std::make_integer_sequence<int, 16>{});
#pragma unroll
  for (int r = 0; r < R; r++) {
    float v = part[r][0][0];
#pragma unroll
    for (int j = 1; j < NPC; j++) v += part[r][0][j];
#pragma unroll
    for (int c = 1; c < NC; c++) {
      float u = part[r][c][0];
#pragma unroll
      for (int j = 1; j < NPC; j++) u += part[r][c][j];
      v = fmaf(u, __builtin_bit_cast(float, (uint32_t)(127 - class_off<T, BITS>(c)) << 23), v);
    }
    d[r] = v;
  }
}

// v + (v of the lane that the DPP control selects), all lanes active
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  const int o = __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false);
  return v + __builtin_bit_cast(float, o);
}

// Sum over each aligned group of tpr lanes (a power of two up to 64),
// returned in every lane of the group. Within a row of 16 lanes, DPP moves
// (quad permutes 1-0-3-2 and 2-3-0-1, then the half-row and row mirrors,
// each of which pairs lanes that hold the same partial sum) avoid the LDS
// round trip of a lane shuffle; groups of 32 and 64 add the other rows.
__device__ __forceinline__ float group_sum(float v, int tpr) {
  if (tpr >= 2) v = dpp_add<0xb1>(v);    // quad_perm [1,0,3,2]
  if (tpr >= 4) v = dpp_add<0x4e>(v);    // quad_perm [2,3,0,1]
  if (tpr >= 8) v = dpp_add<0x141>(v);   // row_half_mirror
  if (tpr >= 16) v = dpp_add<0x140>(v);  // row_mirror
  if (tpr >= 32) v += __shfl_xor(v, 16);
  if (tpr >= 64) v += __shfl_xor(v, 32);
  return v;
}

template <class T, int BITS, int P = 0>
__device__ __forceinline__ void unpack_pairs(const uint32_t* w, uint32_t m2,
                                             uint32_t magic, uint32_t* pr) {
  if constexpr (P < 16) {
    pr[P] = magic_pair<T, BITS, P>(w, m2, magic);
    unpack_pairs<T, BITS, P + 1>(w, m2, magic, pr);
  }
}

// x staging helpers. T pair (1, 1).
template <class T>
__host__ __device__ constexpr uint32_t unit_pair() {
  return __is_same(T, F16) ? 0x3C003C00u : 0x3F803F80u;
}
// T bits of 2^-o (o at most 7: a normal value in both types)
template <class T>
__host__ __device__ constexpr uint32_t inv_pow2_bits(int o) {
  return __is_same(T, F16) ? (uint32_t)(15 - o) << 10 : (uint32_t)(127 - o) << 7;
}
// T pair (2^-o(2j), 2^-o(2j+1)) for the activations of loaded word j
// (elements 2j and 2j+1 of a chunk)
template <class T, int BITS>
__host__ __device__ constexpr uint32_t inv_off_pair(int j) {
  return inv_pow2_bits<T>(pair_off<T, BITS>(2 * j)) |
         (inv_pow2_bits<T>(pair_off<T, BITS>(2 * j + 1)) << 16);
}
// code of the high half of pair p
template <int BITS>
__host__ __device__ constexpr int pair_partner(int p) {
  int r = 0;
  for (int k = 0; k < 32; k++)
    if (pair_index<BITS>(k) == p && pair_half<BITS>(k) == 1) r = k;
  return r;
}
// v_perm_b32 selector: low half = half lo of the second source word, high
// half = half hi of the first
__host__ __device__ constexpr uint32_t pair_perm_sel(int lo, int hi) {
  return (uint32_t)(2 * lo) | (uint32_t)(2 * lo + 1) << 8 | (uint32_t)(4 + 2 * hi) << 16 |
         (uint32_t)(5 + 2 * hi) << 24;
}

constexpr int kXWaves = 2;                        // wavefronts staging x

// One workgroup = WW W wavefronts (4 or 8) + 2 x wavefronts.
//  x wavefronts: issue the x loads of their first staging task (and the
//    scale / bias loads when staged), barrier 1, then permute /
//    sum into LDS, barrier 2.
//  W wavefronts: barrier 1 (so that the x loads are ahead of them in the
//    CU's memory queue), issue every weight load of the lane in the order
//    the chunks are multiplied, barrier 2 (which does not wait for those
//    loads), then multiply chunk by chunk as the weight data arrives.
// Staged scales / biases: at most kSbUnits 16-byte units per x lane.
constexpr int kSbUnits = 4;

// Compiler fence between groups of loads: memory operations are not moved
// across it, so the loads issue in program order and the wait for one
// chunk leaves the later chunks in flight.
__device__ __forceinline__ void chunk_fence() { asm volatile("; chunk fence" ::: "memory"); }

// Lane work: R rows x CPL chunks; lane t of a row group handles chunks
// c = t + TPR*i (i < CPL) of each of its R rows, so an x chunk read from LDS
// serves R rows.
// PK: scales and biases in the affine-packed layout of 3/5/6-bit weights
// ("Add the 3bit packed qmm_t", ops.cpp quantize with AffinePacked): one
// array, rows in pairs, per pair and group the two scales then the two
// biases (scale of row n at ((n/2)*G + g)*4 + n%2, its bias 2 further); the
// biases argument is unused.
template <class T, int BITS, int MB, int CPL, int R, bool SBL, int WW, bool GATHER,
          bool PK = false>
__global__ __launch_bounds__((WW + kXWaves) * 64) void qmv_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wq,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases,
    uint16_t* __restrict__ y, int M, int N, int K, int gs_log2, int tpr_log2,
    uint32_t m2, uint32_t magic, const int32_t* __restrict__ lidx,
    const int32_t* __restrict__ ridx, int nxb, int nwb) {
  using Cfg = QmvCfg<T, BITS>;
  constexpr int XW = Cfg::kXWords, XR = Cfg::kXRec;
  extern __shared__ uint32_t smem[];
  const int nch = K >> 5;
  // Batch z (gathered products): x batch lidx[z] and weight batch ridx[z]
  // (z itself where an index array is absent), clamped into range so that
  // no index can move an access outside the arrays; output batch z. (A
  // compile-time switch: the plain GEMV starts without these dependent
  // scalar loads.)
  if constexpr (GATHER) {
    const int z = blockIdx.z;
    int li = lidx ? lidx[z] : z, ri = ridx ? ridx[z] : z;
    li = li < 0 ? 0 : (li >= nxb ? nxb - 1 : li);
    ri = ri < 0 ? 0 : (ri >= nwb ? nwb - 1 : ri);
    x += (int64_t)li * M * K;
    wq += (int64_t)ri * N * ((int64_t)K * BITS / 8);
    scales += (int64_t)ri * N * (K >> gs_log2);
    biases += (int64_t)ri * N * (K >> gs_log2);
    y += (int64_t)z * M * N;
  }
  const int ntask = MB * nch;
  uint32_t* xs = smem;                                            // [MB*nch][XR]
  const int m0 = blockIdx.y * MB;

  const int tpr = 1 << tpr_log2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool w_wave = wave < WW;
  const int slot = lane >> tpr_log2, t = lane & (tpr - 1);
  const int slots = 64 >> tpr_log2;  // row groups per wavefront
  const int rows_blk = WW * slots * R;
  const int row0 = ((blockIdx.x * WW + wave) * slots + slot) * R;

  const int64_t row_bytes = (int64_t)K * BITS / 8;
  const int G = K >> gs_log2;
  // staged scales then biases of the workgroup's rows, [2][rows_blk][G]
  // (16-byte aligned after the x region)
  uint16_t* sbl = reinterpret_cast<uint16_t*>(smem + ntask * XR);
  const int sb_units = SBL ? rows_blk * G / 8 : 0;  // 16-byte units per array
  const int batch = tpr * CPL;  // chunks of a row covered by one batch
  uint32_t wv[R][CPL][BITS];
  uint16_t sw[R][CPL], bw[R][CPL];  // raw scale / bias words
  // Branch-free: out-of-range chunks read a clamped valid address, so all
  // loads issue back to back; chunks past the row end are skipped when
  // multiplying, and rows past N only feed sums that are never stored.
  // Chunk-major, so that chunk i of every row is in before chunk i + 1.
  auto load_batch = [&](int cb) {
#pragma unroll
    for (int i = 0; i < CPL; i++) {
#pragma unroll
      for (int r = 0; r < R; r++) {
        const int row = row0 + r;
        const int rowc = row < N ? row : N - 1;
        const int c = cb + t + i * tpr;
        const int cc = c < nch ? c : nch - 1;
        load_chunk<BITS>(wq + (int64_t)rowc * row_bytes + (int64_t)cc * (4 * BITS), wv[r][i]);
        if constexpr (!SBL) {
          const int g = (cc << 5) >> gs_log2;
          if constexpr (PK) {
            const int64_t e = ((int64_t)(rowc >> 1) * G + g) * 4 + (rowc & 1);
            sw[r][i] = scales[e];
            bw[r][i] = scales[e + 2];
          } else {
            sw[r][i] = scales[(int64_t)rowc * G + g];
            bw[r][i] = biases[(int64_t)rowc * G + g];
          }
        }
      }
      chunk_fence();
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // staged scales / biases of this lane's chunks, read from LDS
  auto read_sb = [&]() {
    const int lr0 = (wave * slots + slot) * R;  // row of the workgroup
#pragma unroll
    for (int i = 0; i < CPL; i++) {
      const int c = t + i * tpr;
      const int cc = c < nch ? c : nch - 1;
      const int g = (cc << 5) >> gs_log2;
#pragma unroll
      for (int r = 0; r < R; r++) {
        if constexpr (PK) {
          // the staged run is the packed rows of the workgroup (rows_blk even)
          const int lr = lr0 + r, e = ((lr >> 1) * G + g) * 4 + (lr & 1);
          sw[r][i] = sbl[e];
          bw[r][i] = sbl[e + 2];
        } else {
          sw[r][i] = sbl[(lr0 + r) * G + g];
          bw[r][i] = sbl[(rows_blk + lr0 + r) * G + g];
        }
      }
    }
  };
  // x lanes: 16-byte unit u of the staged scales (u < sb_units) or biases;
  // a unit that crosses the end of the array is read element by element
  auto sb_load = [&](int u) -> uint4 {
    const bool bias = u >= sb_units;
    const int uu = bias ? u - sb_units : u;
    const uint16_t* src = bias ? biases : scales;
    int64_t e0 = (int64_t)blockIdx.x * rows_blk * G + 8 * (int64_t)uu;
    int64_t total = (int64_t)N * G;
    if constexpr (PK) {   // one run of 2 * rows_blk * G values
      src = scales;
      e0 = (int64_t)blockIdx.x * rows_blk * 2 * G + 8 * (int64_t)u;
      total = (int64_t)N * 2 * G;
    }
    if (e0 + 8 <= total) return *reinterpret_cast<const uint4*>(src + e0);
    uint32_t h[4] = {0, 0, 0, 0};
    for (int e = 0; e < 8; e++)
      if (e0 + e < total) h[e / 2] |= (uint32_t)src[e0 + e] << (16 * (e % 2));
    return make_uint4(h[0], h[1], h[2], h[3]);
  };

  // x staging: task = (row of x, chunk); activations permuted into pair
  // order, plus the chunk's sum and magic offset
  auto x_load = [&](int task, uint4* raw4) {
    const int tk = task < ntask ? task : ntask - 1;
    const int m = tk / nch, c = tk - m * nch;
    const int mr = m0 + m < M ? m0 + m : M - 1;
    const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)mr * K + c * 32);
#pragma unroll
    for (int q = 0; q < 4; q++) raw4[q] = src[q];
  };
  auto stage = [&](int task, const uint4* raw4) {
    const int m = task / nch;
    uint32_t raw[16];
#pragma unroll
    for (int q = 0; q < 4; q++) {
      raw[4 * q] = raw4[q].x; raw[4 * q + 1] = raw4[q].y;
      raw[4 * q + 2] = raw4[q].z; raw[4 * q + 3] = raw4[q].w;
    }
    const bool live = m0 + m < M;
    uint32_t px[XW];
    float sum = 0.0f, d0 = 0.0f;
    if constexpr (Cfg::kF32) {
#pragma unroll
      for (int k = 0; k < 32; k++) {
        const float f = live ? to_f32(T{}, (uint16_t)(raw[k / 2] >> (16 * (k % 2)))) : 0.0f;
        px[k] = __builtin_bit_cast(uint32_t, f);
        sum += f;
      }
    } else {
      // activations keep their own bits (permuted into pair order, one byte
      // permute per pair); the chunk's sum and the magic offset
      // sum(x * MAGIC * 2^-o) come from dot2 of the pairs as loaded with
      // (1, 1) and with (2^-o, 2^-o') (exact products, fp32 sums, two
      // chains each)
      if (!live) {
#pragma unroll
        for (int q = 0; q < 16; q++) raw[q] = 0;
      }
      float s2[2] = {0.0f, 0.0f}, d2[2] = {0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < 16; j++) {
        s2[j & 1] = dot2(T{}, raw[j], unit_pair<T>(), s2[j & 1]);
        d2[j & 1] = dot2(T{}, raw[j], inv_off_pair<T, BITS>(j), d2[j & 1]);
      }
      sum = s2[0] + s2[1];
      d0 = (d2[0] + d2[1]) * T::kMagicF;
#pragma unroll
      for (int p = 0; p < 16; p++) {
        const int klo = pair_code<BITS>(p), khi = pair_partner<BITS>(p);
        px[p] = __builtin_amdgcn_perm(raw[khi / 2], raw[klo / 2], pair_perm_sel(klo & 1, khi & 1));
      }
    }
    uint4* dst = reinterpret_cast<uint4*>(xs + (int64_t)task * XR);
#pragma unroll
    for (int q = 0; q < XW / 4; q++)
      dst[q] = make_uint4(px[4 * q], px[4 * q + 1], px[4 * q + 2], px[4 * q + 3]);
    dst[XW / 4] = make_uint4(__builtin_bit_cast(uint32_t, sum), __builtin_bit_cast(uint32_t, d0),
                             0u, 0u);
  };

  if (w_wave) {
    __syncthreads();  // 1: the x loads of this workgroup are queued first
    load_batch(0);
    __syncthreads();  // 2: x staged (does not wait for the weight loads)
    if constexpr (SBL) read_sb();
  } else {
    const int xl = (wave - WW) * 64 + lane;
    uint4 raw4[4];
    x_load(xl, raw4);
    uint4 sbu[SBL ? kSbUnits : 1];
    if constexpr (SBL) {
#pragma unroll
      for (int j = 0; j < kSbUnits; j++) {
        const int u = xl + j * kXWaves * 64;
        if (u < 2 * sb_units) sbu[j] = sb_load(u);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();  // 1
    if (xl < ntask) stage(xl, raw4);
    if constexpr (SBL) {
#pragma unroll
      for (int j = 0; j < kSbUnits; j++) {
        const int u = xl + j * kXWaves * 64;
        if (u < 2 * sb_units) reinterpret_cast<uint4*>(sbl)[u] = sbu[j];
      }
    }
    for (int task = xl + kXWaves * 64; task < ntask; task += kXWaves * 64) {
      x_load(task, raw4);
      stage(task, raw4);
    }
    __syncthreads();  // 2
    return;
  }

  // ---- multiply
  // The magic pattern lives in a VGPR and the mask in an SGPR, so that
  // mask-and-or is one v_and_or_b32 (a VOP3 reads one SGPR at most and no
  // literal on gfx9).
  uint32_t magic_v;
  asm volatile("v_mov_b32 %0, %1" : "=v"(magic_v) : "s"(magic));
  float acc[R][MB];
#pragma unroll
  for (int r = 0; r < R; r++)
#pragma unroll
    for (int m = 0; m < MB; m++) acc[r][m] = 0.0f;

  for (int cb = 0;;) {
#pragma unroll
    for (int i = 0; i < CPL; i++) {
      const int c = cb + t + i * tpr;
      if (c < nch) {
        float sf[R], bf[R];
#pragma unroll
        for (int r = 0; r < R; r++) {
          sf[r] = to_f32(T{}, sw[r][i]);
          bf[r] = to_f32(T{}, bw[r][i]);
        }
        if constexpr (Cfg::kF32) {
#pragma unroll
          for (int m = 0; m < MB; m++) {
            const float* xp = reinterpret_cast<const float*>(xs + (int64_t)(m * nch + c) * XR);
            float xv[32];
#pragma unroll
            for (int k = 0; k < 32; k++) xv[k] = xp[k];
            const float xsm = xp[XW];
#pragma unroll
            for (int r = 0; r < R; r++) {
              float d = 0.0f;
#pragma unroll
              for (int w = 0; w < 8; w++)
#pragma unroll
                for (int bb = 0; bb < 4; bb++)
                  d = fmaf(xv[4 * w + bb], (float)((wv[r][i][w] >> (8 * bb)) & 0xffu), d);
              acc[r][m] = fmaf(sf[r], d, fmaf(bf[r], xsm, acc[r][m]));
            }
          }
        } else {
          uint32_t pr[R][16];
#pragma unroll
          for (int r = 0; r < R; r++) unpack_pairs<T, BITS>(wv[r][i], m2, magic_v, pr[r]);
#pragma unroll
          for (int m = 0; m < MB; m++) {
            const uint4* xp4 = reinterpret_cast<const uint4*>(xs + (int64_t)(m * nch + c) * XR);
            uint32_t xp[16];
#pragma unroll
            for (int q = 0; q < 4; q++) {
              const uint4 u = xp4[q];
              xp[4 * q] = u.x; xp[4 * q + 1] = u.y; xp[4 * q + 2] = u.z; xp[4 * q + 3] = u.w;
            }
            const uint2 sd = *reinterpret_cast<const uint2*>(xp4 + 4);
            const float xsm = __builtin_bit_cast(float, sd.x);
            const float d0 = __builtin_bit_cast(float, sd.y);
            // partial sums per row: rows x partials >= 4 (rows of x give
            // independent chains as well)
            constexpr int NP = R * MB >= 4 ? 1 : 4 / (R * MB);
            float d[R];
            chunk_dot_rows<T, BITS, R, NP>(pr, xp, d);
#pragma unroll
            for (int r = 0; r < R; r++)
              acc[r][m] = fmaf(sf[r], d[r] - d0, fmaf(bf[r], xsm, acc[r][m]));
          }
        }
      }
    }
    cb += batch;
    if (cb >= nch) break;
    load_batch(cb);  // rows longer than one batch (very large K; never staged)
  }

  // ---- reduce the TPR partial sums of each row
#pragma unroll
  for (int r = 0; r < R; r++)
#pragma unroll
    for (int m = 0; m < MB; m++) acc[r][m] = group_sum(acc[r][m], tpr);
  if (t == 0) {
#pragma unroll
    for (int r = 0; r < R; r++) {
      const int row = row0 + r;
#pragma unroll
      for (int m = 0; m < MB; m++)
        if (row < N && m0 + m < M)
          y[(int64_t)(m0 + m) * N + row] = from_f32(T{}, acc[r][m]);
    }
  }
}

// ----------------------------------------------------------------- launch

// Batches of a gathered GEMV: output batch z of B multiplies x batch
// lidx[z] (of nxb) by weight batch ridx[z] (of nwb); null index arrays mean
// z. One plain GEMV is the single batch with no index arrays.
struct QmvBatch {
  const int32_t* lidx;
  const int32_t* ridx;
  int nxb, nwb, B;
  bool pk = false;   // scales / biases in the affine-packed layout (3/5/6 bits)
};
static constexpr QmvBatch kOneBatch{nullptr, nullptr, 1, 1, 1};
static bool gathered(const QmvBatch& bt) {
  return bt.lidx || bt.ridx || bt.B != 1 || bt.nxb != 1 || bt.nwb != 1;
}

static constexpr int kMaxLds = 64 * 1024;

// Lane work shapes (chunks per lane, rows per lane, W wavefronts) compiled in.
struct Shape {
  int cpl, r, ww;
};
static constexpr Shape kShapes[] = {{2, 1, 4}, {4, 1, 4}, {4, 2, 4}, {8, 1, 4}, {4, 1, 8}};

// Threads per row for a lane shape: enough lanes that CPL chunks each cover
// the row (a power of two, at most 64).
static int tpr_for(int nch, int cpl) {
  int tpr = 1;
  while (tpr < 64 && tpr * cpl < nch) tpr *= 2;
  return tpr;
}

template <class T, int BITS, int MB, int CPL, int R, int WW>
static hipError_t launch_shape(const void* x, const uint32_t* wq, const void* s,
                               const void* b, int M, int N, int K, int gs,
                               int tpr, void* y, hipStream_t st, const QmvBatch& bt) {
  using Cfg = QmvCfg<T, BITS>;
  const int nch = K / 32, G = K / gs;
  const int rows_per_block = WW * (64 / tpr) * R;
  const dim3 block((WW + kXWaves) * 64);
  const dim3 grid((N + rows_per_block - 1) / rows_per_block, (M + MB - 1) / MB, bt.B);
  const size_t lds_x = (size_t)MB * nch * Cfg::kXRec * 4;
  // staged scales / biases: one batch covers a row, the block's run of each
  // array is whole 16-byte units at 16-byte aligned addresses, the x lanes
  // copy it with kSbUnits loads each and it fits in LDS
  const size_t lds_sb = ((lds_x + 15) & ~(size_t)15) + (size_t)rows_per_block * G * 4;
  const bool sbl = tpr * CPL >= nch && ((int64_t)rows_per_block * G) % 8 == 0 &&
                   (int64_t)rows_per_block * G / 4 <= (int64_t)kSbUnits * kXWaves * 64 &&
                   ((reinterpret_cast<uintptr_t>(s) | reinterpret_cast<uintptr_t>(b)) & 15) == 0 &&
                   (bt.nwb == 1 || ((int64_t)N * G) % 8 == 0) &&   // every weight batch aligned
                   lds_sb <= (size_t)kMaxLds;
  const uint32_t m2 = Pack<BITS>::kMask | (Pack<BITS>::kMask << 16);
  uint32_t magic = 0;
  if constexpr (!Cfg::kF32) magic = T::kMagic;
  const auto xp = static_cast<const uint16_t*>(x);
  const auto wp = reinterpret_cast<const uint8_t*>(wq);
  const auto sp = static_cast<const uint16_t*>(s);
  const auto bp = static_cast<const uint16_t*>(b);
  const auto yp = static_cast<uint16_t*>(y);
  auto go = [&]<bool S, bool GA, bool PK = false>() {
    hipLaunchKernelGGL((qmv_kernel<T, BITS, MB, CPL, R, S, WW, GA, PK>), grid, block,
                       S ? lds_sb : lds_x, st, xp, wp, sp, bp, yp, M, N, K, ilog2(gs),
                       ilog2(tpr), m2, magic, bt.lidx, bt.ridx, bt.nxb, bt.nwb);
  };
  // affine-packed scales (3/5/6 bits only; one packed run, N even)
  if constexpr (!Pack<BITS>::kPow2) {
    if (bt.pk) {
      if (sbl) go.template operator()<true, false, true>();
      else go.template operator()<false, false, true>();
      return hipGetLastError();
    }
  }
  // gathered launches come with one row of x per pass (launch_t)
  if constexpr (MB == 1) {
    if (gathered(bt)) {
      if (sbl) go.template operator()<true, true>();
      else go.template operator()<false, true>();
      return hipGetLastError();
    }
  }
  if (sbl) go.template operator()<true, false>();
  else go.template operator()<false, false>();
  return hipGetLastError();
}

// One row of x, one product: does the layer take the 8-wavefront lane shape
// (4 chunks of one row per lane making one round of 256 to 320 workgroups),
// and, for 5-, 6- and 8-bit codes, its 2-chunk form (2 chunks per lane in
// twice the workgroups, while one batch covers the row)?
static bool one_round_8w(int64_t N, int64_t K) {
  const int nch = (int)(K / 32);
  const int64_t rows = 8 * (64 / tpr_for(nch, 4));
  const int64_t b8 = (N + rows - 1) / rows;
  return b8 >= 256 && b8 <= 320;
}
bool qmv_two_chunk_shape(int64_t N, int64_t K, int bits) {
  return bits >= 5 && one_round_8w(N, K) && K / 32 <= 2 * 64;
}

template <class T, int BITS, int MB>
static hipError_t launch_mb(const void* x, const uint32_t* wq, const void* s,
                            const void* b, int M, int N, int K, int gs,
                            void* y, hipStream_t st, const QmvBatch& bt) {
  const int nch = K / 32;
  auto blocks_of = [&](const Shape& sh) {
    const int rows_per_block = sh.ww * (64 / tpr_for(nch, sh.cpl)) * sh.r;
    return (int64_t)((N + rows_per_block - 1) / rows_per_block) * ((M + MB - 1) / MB) * bt.B;
  };
  // One row of x: 8 W wavefronts with 4 chunks of one row per lane, so that
  // two wavefronts per SIMD share the arithmetic that follows the weight
  // data, when that makes one round of 256 to 320 workgroups (such a
  // workgroup fills a CU's registers: more would run in a second round).
  // Two rows of x on the same layers: 2 chunks per lane in 8 W wavefronts
  // (same-box timings of the forced streaming GEMV at M = 2: f16 4096 x 4096
  // 4-bit 6.18 -> 5.69 us, 2-bit 5.70 -> 5.27, 8-bit 8.85 -> 6.80; bf16
  // 8192 x 2048 6-bit 6.19 -> 5.45; 4-bit rows of 2048 codes measured 4.80 ->
  // 4.90 us, so rows that short keep this only for 5- to 8-bit codes)
  if constexpr (MB == 2) {
    const int64_t b8 = blocks_of(kShapes[4]);
    if (b8 >= 256 && b8 <= 320 && nch <= 2 * 64 && (nch > 64 || BITS >= 5))
      return launch_shape<T, BITS, MB, 2, 1, 8>(x, wq, s, b, M, N, K, gs, tpr_for(nch, 2), y,
                                                st, bt);
  }
  if (MB == 1) {
    const int64_t b8 = blocks_of(kShapes[4]);
    if (b8 >= 256 && b8 <= 320) {
      // 5-, 6- and 8-bit codes (20- to 32-byte chunks): 2 chunks per lane in
      // twice the workgroups, while one batch covers the row (same-box
      // timings, 4096 x 4096 M = 1: 8-bit 6.09 -> 5.57 us, 6-bit 5.22 ->
      // 5.04, 5-bit 4.94 -> 4.83; the narrower codes are faster with 4)
      if constexpr (MB == 1 && BITS >= 5) {
        if (nch <= 2 * 64)
          return launch_shape<T, BITS, MB, 2, 1, 8>(x, wq, s, b, M, N, K, gs,
                                                    tpr_for(nch, 2), y, st, bt);
      }
      if constexpr (MB == 1)
        return launch_shape<T, BITS, MB, 4, 1, 8>(x, wq, s, b, M, N, K, gs,
                                                  tpr_for(nch, 4), y, st, bt);
    }
  }
  // Otherwise the first 4-wavefront shape in order of preference that gives
  // at least 256 workgroups (one per CU), else the one with the most: 4
  // chunks x 2 rows per lane first (measured best for several rows of x and
  // for layers of many row blocks).
  static constexpr int kOrder[] = {2, 1, 3, 0};
  int best = -1;
  int64_t best_blocks = -1;
  for (int oi = 0; oi < 4; oi++) {
    const int i = kOrder[oi];
    const int64_t blocks = blocks_of(kShapes[i]);
    if (blocks >= 256) { best = i; break; }
    if (blocks > best_blocks) { best_blocks = blocks; best = i; }
  }
  if (best < 0) best = 3;
  const Shape sh = kShapes[best];
  const int tpr = tpr_for(nch, sh.cpl);
  switch (best) {
    case 0: return launch_shape<T, BITS, MB, 2, 1, 4>(x, wq, s, b, M, N, K, gs, tpr, y, st, bt);
    case 1: return launch_shape<T, BITS, MB, 4, 1, 4>(x, wq, s, b, M, N, K, gs, tpr, y, st, bt);
    case 2: return launch_shape<T, BITS, MB, 4, 2, 4>(x, wq, s, b, M, N, K, gs, tpr, y, st, bt);
    default: return launch_shape<T, BITS, MB, 8, 1, 4>(x, wq, s, b, M, N, K, gs, tpr, y, st, bt);
  }
}

template <class T, int BITS>
static hipError_t launch_t(const void* x, const uint32_t* wq, const void* s,
                           const void* b, int M, int N, int K, int gs, void* y,
                           hipStream_t st, const QmvBatch& bt) {
  using Cfg = QmvCfg<T, BITS>;
  const int64_t per_row = (int64_t)(K / 32) * Cfg::kXRec * 4;
  int mb_max = (int)(kMaxLds / per_row);
  int want = 1;  // smallest of 1, 2, 4 covering M (4 at most)
  while (want < M && want < 4) want *= 2;
  while (want > 1 && want > mb_max) want /= 2;
  if (gathered(bt)) want = 1;  // gathered products: one row of x per pass
  switch (want) {
    case 4: return launch_mb<T, BITS, 4>(x, wq, s, b, M, N, K, gs, y, st, bt);
    case 2: return launch_mb<T, BITS, 2>(x, wq, s, b, M, N, K, gs, y, st, bt);
    default: return launch_mb<T, BITS, 1>(x, wq, s, b, M, N, K, gs, y, st, bt);
  }
}

template <class T>
static hipError_t launch_bits(int bits, const void* x, const uint32_t* wq,
                              const void* s, const void* b, int M, int N,
                              int K, int gs, void* y, hipStream_t st, const QmvBatch& bt) {
  switch (bits) {
    case 2: return launch_t<T, 2>(x, wq, s, b, M, N, K, gs, y, st, bt);
    case 3: return launch_t<T, 3>(x, wq, s, b, M, N, K, gs, y, st, bt);
    case 4: return launch_t<T, 4>(x, wq, s, b, M, N, K, gs, y, st, bt);
    case 5: return launch_t<T, 5>(x, wq, s, b, M, N, K, gs, y, st, bt);
    case 6: return launch_t<T, 6>(x, wq, s, b, M, N, K, gs, y, st, bt);
    default: return launch_t<T, 8>(x, wq, s, b, M, N, K, gs, y, st, bt);
  }
}

hipError_t launch_qmv(int dt, int bits, int gs, const void* x,
                      const uint32_t* wq, const void* s, const void* b,
                      int64_t M, int64_t N, int64_t K, void* y,
                      hipStream_t st) {
  if (route(dt, bits, gs, M, N, K, false) == kRouteQmvMfma)
    return launch_qmv_mfma(dt, bits, gs, x, wq, s, b, M, N, K, y, st);
  if (dt == 0)
    return launch_bits<F16>(bits, x, wq, s, b, (int)M, (int)N, (int)K, gs, y, st, kOneBatch);
  return launch_bits<BF16>(bits, x, wq, s, b, (int)M, (int)N, (int)K, gs, y, st, kOneBatch);
}

// GEMV on the affine-packed layout of 3/5/6-bit weights: standard packed
// words, scales and biases interleaved in pairs of rows (N even)
hipError_t launch_qmv_packed_sb(int dt, int bits, int gs, const void* x, const uint32_t* wq,
                                const void* sbp, int64_t M, int64_t N, int64_t K, void* y,
                                hipStream_t st) {
  QmvBatch bt = kOneBatch;
  bt.pk = true;
  if (dt == 0)
    return launch_bits<F16>(bits, x, wq, sbp, sbp, (int)M, (int)N, (int)K, gs, y, st, bt);
  return launch_bits<BF16>(bits, x, wq, sbp, sbp, (int)M, (int)N, (int)K, gs, y, st, bt);
}

hipError_t launch_gather_qmv(int dt, int bits, int gs, const void* x, int64_t nxb,
                             const int32_t* lidx, const uint32_t* wq, const void* s,
                             const void* b, int64_t nwb, const int32_t* ridx, int64_t B,
                             int64_t M, int64_t N, int64_t K, void* y, hipStream_t st) {
  const QmvBatch bt{lidx, ridx, (int)nxb, (int)nwb, (int)B};
  if (dt == 0)
    return launch_bits<F16>(bits, x, wq, s, b, (int)M, (int)N, (int)K, gs, y, st, bt);
  return launch_bits<BF16>(bits, x, wq, s, b, (int)M, (int)N, (int)K, gs, y, st, bt);
}

}  // namespace qmm
