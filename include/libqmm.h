/*
 * libqmm -- affine group-wise quantized matrix multiply for MI355X (gfx950).
 *
 * y = x . dequant(Wq)^T, where each row of W is split into groups of
 * group_size consecutive elements along K and every group carries one scale
 * and one bias: w ~ scale * q + bias with an unsigned code q of `bits` bits.
 * The quantizer, the packing and the operation follow:
 *  - "Improvements in the quantizer and dequantization kernel" (mlx PR 1061),
 *    item 1 a-c: the bias is the group extreme of larger magnitude, the scale
 *    runs from it to the other extreme and is adjusted so 0 is on the grid;
 *  - "mlx 1.0.0 backend/cpu/quantized.cpp", functions quantize,
 *    get_pack_factor, get_bytes_per_pack, extract_bits and _qmm_t: the
 *    per-group steps, the packed layout and y[m,n] = sum_k x[m,k] *
 *    (scale[n,k/gs] * q[n,k] + bias[n,k/gs]);
 *  - "Add the 3bit packed qmm_t" (mlx compare sdpa-test...packed-quants),
 *    ops.cpp extract_quantized_matmul_dims / quantized_matmul: the argument
 *    checks, one element type for x, scales, biases and y, and the
 *    small-M / large-M split between a GEMV and a tiled GEMM;
 *  - "[Feature] Quantized Convolution 2D - Possible PR?" (mlx issue 2714):
 *    the conv weight reshape with K zero-padded to a multiple of group_size,
 *    and the im2col patch order (dy, dx, c) over NHWC input.
 *
 * Conventions for every call:
 *  - All array pointers are DEVICE pointers, allocated and owned by the
 *    caller; the library never allocates, frees or keeps them.
 *  - Arrays are row-major and contiguous. x, wq, w_out and y must be 16-byte
 *    aligned; scales and biases 2-byte aligned (4-byte for QMM_F32).
 *  - Packed weights wq hold K*bits/8 bytes per row (K*bits/32 uint32 words):
 *    code k of a row sits at bit k*bits of the row's little-endian byte
 *    stream. For bits 2, 4, 8 that is 32/bits codes per uint32 word, low
 *    bits first; for bits 3 and 6 it is 8 (resp. 4) codes per 3 bytes and
 *    for bits 5 eight codes per 5 bytes.
 *  - scales and biases are [rows, K/group_size] of the element type.
 *  - Each call validates its arguments synchronously, before any launch, and
 *    returns a status; on error nothing is launched or written and
 *    qmm_last_error() describes the problem. On success the work is queued
 *    asynchronously on `stream` (a hipStream_t passed as void*; NULL is the
 *    default stream), which must belong to the current HIP device (QMM_E_ARG
 *    otherwise); every pointer is memory of that device. No call synchronizes the host. Device faults surface at
 *    the caller's next synchronization.
 *  - Supported: bits in {2,3,4,5,6,8}; group_size in {32,64,128};
 *    K a positive multiple of group_size.
 *  - Several entry points split K over workgroups and keep fp32 partial sums
 *    in library-owned workspaces: static device arrays, one set per GPU,
 *    holding their last call's contents (nothing is allocated per call):
 *      * the tile-kernel workspace (64 MiB) and 256 per-tile arrival
 *        counters: qmm_t, qmm_t_batched, qmm_gather_qmm, qconv2d_nhwc,
 *        qmm_fp_t, qmm_fp_n, qmm_t_affine_packed and qmm_n when they split K;
 *      * the MFMA GEMV's partial tiles (2 MiB) and its 256 arrival counters:
 *        qmm_t, qmv and qmm_t_batched when they route up to 32 rows of x to
 *        the MFMA GEMV on a narrow layer.
 *    Calls queued on one stream are ordered by the stream. Calls of these
 *    entry points queued on different streams of one GPU, from one host
 *    thread or several, are ordered by the library (except calls that run on
 *    the streaming GEMV, which uses no scratch): each waits (on
 *    the device, hipStreamWaitEvent) for the previous such call's work when
 *    that call was queued on another stream, through one event per GPU
 *    recorded after each call's launches. Calls made while their stream is
 *    being captured into a graph wait for and record nothing: the capturing
 *    caller must order the graph's launches against concurrent calls on other
 *    streams (an overlap makes the overlapping calls' outputs undefined; the
 *    counters wrap back to zero on each call's last arrival, so later calls
 *    are exact again).
 */
#ifndef LIBQMM_H
#define LIBQMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QMM_F16 = 0,  /* IEEE binary16 */
  QMM_BF16 = 1, /* bfloat16 */
  QMM_F32 = 2   /* binary32: accepted by qmm_quantize / qmm_dequantize only */
} qmm_dtype;

typedef enum {
  QMM_OK = 0,
  QMM_E_NULL = 1,   /* a required pointer is NULL */
  QMM_E_BITS = 2,   /* bits not in {2,3,4,5,6,8} */
  QMM_E_GROUP = 3,  /* group_size not in {32,64,128} */
  QMM_E_SHAPE = 4,  /* a size < 1, K % group_size != 0, or bad conv geometry */
  QMM_E_DTYPE = 5,  /* element type not supported by this call */
  QMM_E_ALIGN = 6,  /* a pointer violates the alignment rules above */
  QMM_E_LAUNCH = 7, /* the kernel launch itself failed (hipGetLastError) */
  QMM_E_ARG = 8     /* an argument outside its documented set of values */
} qmm_status;

/*
 * Quantize w[rows, K] (element type dt: f16, bf16 or f32) group by group.
 * Per group: min/max in fp32; the bias candidate is the extreme of larger
 * magnitude (max on a tie); scale = +-max((max-min)/(2^bits-1), 1e-7) pointing
 * from that extreme to the other; q0 = rint(edge/scale); if q0 != 0 then
 * scale = edge/q0 and bias = edge, else bias = 0; code = clamp(rint((w -
 * bias)/scale), 0, 2^bits-1). All in IEEE fp32 with correctly rounded
 * division and ties-to-even rounding; scale and bias are stored rounded to
 * nearest even in dt. (Source: mlx PR 1061 item 1; mlx 1.0.0 CPU backend,
 * function quantize.)
 * Outputs: wq [rows, K*bits/32] uint32, scales [rows, K/gs], biases [rows,
 * K/gs] in dt.
 */
qmm_status qmm_quantize(const void* w, qmm_dtype dt, int64_t rows, int64_t K,
                        int group_size, int bits, uint32_t* wq, void* scales,
                        void* biases, void* stream);

/*
 * Dequantize: w_out[n,k] = dt(fl32(fl32(scale*q) + bias)) with the stored
 * scale and bias widened to fp32 (scale*q is exact for f16/bf16 scales).
 * (Source: mlx 1.0.0 CPU backend, functions extract_bits and _qmm_t_simd.)
 */
qmm_status qmm_dequantize(const uint32_t* wq, const void* scales,
                          const void* biases, qmm_dtype dt, int64_t rows,
                          int64_t K, int group_size, int bits, void* w_out,
                          void* stream);

/*
 * y[M,N] = x[M,K] . dequant(wq, scales, biases)[N,K]^T, fp32 accumulation,
 * y rounded to nearest even in dt (f16 or bf16). Routes small M to the GEMV
 * kernels of qmv (the MFMA GEMV up to 32 rows, the streaming GEMV for a
 * few rows) and larger M to the MFMA tile kernel; qmm_route names the
 * kernel for a shape and qmm_crossover_m the first M on the tile kernel. (Source: mlx 1.0.0 CPU backend, _qmm_t;
 * the packed-quants compare, the qmv/qmm_t split in the Metal dispatch.)
 */
qmm_status qmm_t(const void* x, const uint32_t* wq, const void* scales,
                 const void* biases, qmm_dtype dt, int64_t M, int64_t N,
                 int64_t K, int group_size, int bits, void* y, void* stream);

/*
 * Same operation and arguments as qmm_t, always on the GEMV kernels: the
 * MFMA GEMV (up to 32 rows of x that fit in LDS; every packed weight read
 * once) or the streaming GEMV (one pass over W per up to 4 rows of x).
 * Meant for M <= 16 (decode); correct for any M. QMM_E_SHAPE when K exceeds
 * both kernels' limits.
 */
qmm_status qmv(const void* x, const uint32_t* wq, const void* scales,
               const void* biases, qmm_dtype dt, int64_t M, int64_t N,
               int64_t K, int group_size, int bits, void* y, void* stream);

/*
 * Batched qmm_t: for b in [0, batches),
 *   y[b] = x[b] . dequant(W[w_batches == 1 ? 0 : b])^T,
 * with x [batches, M, K], wq [w_batches, N, K*bits/32], scales and biases
 * [w_batches, N, K/group_size], y [batches, M, N], all contiguous, and
 * w_batches either 1 (one weight for every batch: the batches' rows form
 * one product of batches*M rows, as qmm_t) or batches (QMM_E_SHAPE
 * otherwise). Every product is the qmm_t product above. With one weight per
 * batch, by the qmm_t route for M rows: the streaming GEMV's rows run as
 * one gathered GEMV launch (qmm_gather_qmv with no index arrays), the MFMA
 * tile kernel's as one launch over all batches (its K split, if any, keeps
 * the partial sums of every batch in the split-K workspace), the MFMA
 * GEMV's as one launch per batch. The last two need the per-batch sizes of
 * x (M*K), y (M*N) and wq (N*K*bits/8 bytes) to be multiples of 16 bytes
 * (QMM_E_ALIGN otherwise). batches <= 65535; the other rules are those of
 * qmm_t.
 * (Source: "Add the 3bit packed qmm_t", the batched adjust_matrix_offsets
 * in quantized.h and the dispatch in quantized.cpp: a weight with batch
 * dimensions selects one weight per batch, a 2-D weight takes every row of
 * x as one product.)
 */
qmm_status qmm_t_batched(const void* x, const uint32_t* wq, const void* scales,
                         const void* biases, int64_t batches, int64_t w_batches,
                         qmm_dtype dt, int64_t M, int64_t N, int64_t K,
                         int group_size, int bits, void* y, void* stream);

/*
 * Floating-point modes (no bias; one scale byte per group): (bits,
 * group_size) = (4, 32) mxfp4: E2M1 codes, e8m0 scale 2^(s-127);
 * (4, 16) nvfp4: E2M1 codes, E4M3 scale; (8, 32) mxfp8: E4M3 codes (OCP,
 * no infinities), e8m0 scale. Other pairs: QMM_E_BITS / QMM_E_GROUP.
 * Quantize w[rows, K] (f16, bf16 or f32) per group of group_size: scale =
 * max|w| / (6 for E2M1, 448 for E4M3) encoded in one byte (e8m0: n =
 * round(log2 scale), exact, clamped to [-127, 127]; E4M3: round to nearest
 * even, saturating at 448), then each w divided by the decoded scale and
 * encoded (E2M1: nearest value, ties to the even code, beyond 6 -> 6;
 * E4M3: nearest even, saturating at 448). All fp32, IEEE division.
 * Outputs: wq [rows, K*bits/32] uint32 (the row's bytes; 4-bit codes two per
 * byte, code k in the low nibble of byte k/2 when k is even), scales
 * [rows, K/group_size] uint8 (any alignment). K % group_size == 0.
 * (Source: "mlx 1.0.0 backend/cpu/quantized.cpp": FP4_LUT, to_fp4_e2m1,
 * to_fp8_e8m0, dequantize_scale and the per-group steps of
 * fp_quantize_dequantize.)
 */
qmm_status qmm_fp_quantize(const void* w, qmm_dtype dt, int64_t rows, int64_t K,
                           int group_size, int bits, uint32_t* wq,
                           uint8_t* scales, void* stream);

/*
 * Dequantize a floating-point mode: w_out[n,k] = dt(scale_T * value), where
 * scale_T is the decoded scale rounded to dt (for f16, e8m0 scales below
 * 2^-24 become 0 and above 2^15 infinity; every other case is exact) and
 * the product is exact. (Source: as qmm_fp_quantize; dequantize_scale<T>.)
 */
qmm_status qmm_fp_dequantize(const uint32_t* wq, const uint8_t* scales,
                             qmm_dtype dt, int64_t rows, int64_t K,
                             int group_size, int bits, void* w_out,
                             void* stream);

/*
 * y[M,N] = x[M,K] . dequant(W)^T for a floating-point mode: y[m,n] =
 * sum over groups g of scale_T[n,g] * sum_{k in g} x[m,k] * value[n,k],
 * fp32 accumulation, y rounded to nearest even in dt (f16 or bf16). A GEMV
 * (one pass over W per row of x): K a multiple of 32 up to 16384, M <=
 * 65535. (Source: "mlx 1.0.0 backend/cpu/quantized.cpp", fp_qmm_t and
 * fp_qmm_t_simd.)
 */
qmm_status qmm_fp_qmv(const void* x, const uint32_t* wq, const uint8_t* scales,
                      qmm_dtype dt, int64_t M, int64_t N, int64_t K,
                      int group_size, int bits, void* y, void* stream);

/*
 * The same product for any M: the qmm_fp_qmv GEMV for a few rows of x (up
 * to 2-8 by mode and shape, from timings of both kernels), the MFMA tile
 * kernel beyond (W dequantized on chip to dt: scale_T * value is
 * exact in dt whenever it lies in dt's range, which always holds for bf16
 * and for f16 scales from 2^-14 to 2^14; fp32 accumulation). K a positive
 * multiple of 32 (below 2^22 on the tile kernel, up to 16384 on the GEMV);
 * x, wq and y 16-byte aligned; scales any alignment. The tile kernel may
 * split K and use the library's tile-kernel workspace (see above).
 * (Source: "mlx 1.0.0 backend/cpu/quantized.cpp", fp_qmm_t and
 * fp_qmm_t_simd, which serve any number of rows.)
 */
qmm_status qmm_fp_t(const void* x, const uint32_t* wq, const uint8_t* scales,
                    qmm_dtype dt, int64_t M, int64_t N, int64_t K,
                    int group_size, int bits, void* y, void* stream);

/*
 * Non-transposed product in an fp mode: y[M,N] = x[M,K] . dequant(W)[K,N],
 * where W [K, N] is quantized along N by qmm_fp_quantize of its K rows:
 *   y[m,n] = sum_k x[m,k] * scale_T(scales[k, n/gs]) * value(code[k,n]),
 * fp32 accumulation, y rounded to nearest even in dt. wq is [K, N*bits/32]
 * uint32 (the rows' code bytes), scales [K, N/group_size] uint8; modes as
 * qmm_fp_quantize ((4, 32) mxfp4, (4, 16) nvfp4, (8, 32) mxfp8). N must be a
 * multiple of 32 and K of 8 (QMM_E_SHAPE), x, wq and y 16-byte aligned. Runs
 * the non-transposed MFMA tile kernel for any M (K split over workgroups
 * when the output has few tiles: the tile-kernel workspace and counters,
 * shared as described above). (Source: "mlx 1.0.0 backend/cpu/quantized.cpp",
 * fp_qmm.)
 */
qmm_status qmm_fp_n(const void* x, const uint32_t* wq, const uint8_t* scales, qmm_dtype dt,
                    int64_t M, int64_t N, int64_t K, int group_size, int bits, void* y,
                    void* stream);

/*
 * Gathered product in a floating-point mode (e.g. mixture-of-experts decode
 * with mxfp4 experts): for z in [0, batches),
 *   y[z] = x[lhs_indices[z]] . dequant(W[rhs_indices[z]])^T,
 * x [x_batches, M, K], wq [w_batches, N, K*bits/32], scales [w_batches, N,
 * K/group_size] bytes, y [batches, M, N]; index arrays, their defaults and
 * the clamping of out-of-range values as for qmm_gather_qmv; every product
 * is the qmm_fp_qmv product (same limits on K and M). batches <= 65535.
 * (Source: "Add the 3bit packed qmm_t", ops.cpp gather_qmm, which takes the
 * quantization mode like quantized_matmul; "mlx 1.0.0 backend/cpu/
 * quantized.cpp", fp_qmm_t.)
 */
qmm_status qmm_fp_gather_qmv(const void* x, int64_t x_batches,
                             const int32_t* lhs_indices, const uint32_t* wq,
                             const uint8_t* scales, int64_t w_batches,
                             const int32_t* rhs_indices, int64_t batches,
                             qmm_dtype dt, int64_t M, int64_t N, int64_t K,
                             int group_size, int bits, void* y, void* stream);

/*
 * Affine-packed layout of an affine-quantized weight (wq [N, K*bits/32],
 * scales and biases [N, K/group_size] as qmm_quantize writes them): rows in
 * blocks of RP = 4 (bits 2, 4, 8) or 2 (bits 3, 5, 6), N % RP == 0.
 * sb_packed [N/RP, (K/group_size)*2*RP] in dt: per block and group, the RP
 * scales then the RP biases. For bits 2, 4, 8, wq_packed [N/4, 4*K*bits/32]
 * uint32: word w of row 4i+r at [i, 4w + r]; for 3, 5, 6 the weight rows
 * keep their layout and wq_packed is not written (may be NULL).
 * (Source: "Add the 3bit packed qmm_t", ops.cpp quantize with
 * QuantizationType::AffinePacked.)
 */
qmm_status qmm_affine_pack(const uint32_t* wq, const void* scales,
                           const void* biases, qmm_dtype dt, int64_t N,
                           int64_t K, int group_size, int bits,
                           uint32_t* wq_packed, void* sb_packed, void* stream);

/*
 * y[M,N] = x[M,K] . dequant(W)^T read from the affine-packed layout, on a
 * GEMV (meant for a few rows of x): the same product as qmv, y[m,n] = sum
 * over groups of s * sum x*q + b * sum x in fp32. Bits 2, 4, 8: wq_packed
 * the interleaved words, N % 4 == 0, K <= 16384, one pass over W per row of
 * x. Bits 3, 5, 6: wq_packed the plain packed rows (as qmm_quantize writes
 * them), N % 2 == 0, K up to the streaming GEMV's limit (29120 at 4 bits
 * f16, less for wider codes), one pass over W per 4 rows of x. f16 / bf16,
 * M <= 65535; x, wq_packed, sb_packed and y 16-byte aligned. (Source: "Add
 * the 3bit packed qmm_t", affine_packed_qmv_fast_impl and
 * affine_packed_byte_qmv_fast_impl.)
 */
qmm_status qmv_affine_packed(const void* x, const uint32_t* wq_packed,
                             const void* sb_packed, qmm_dtype dt, int64_t M,
                             int64_t N, int64_t K, int group_size, int bits,
                             void* y, void* stream);

/*
 * The same product for any M: the GEMV above for a few rows of x, the MFMA
 * tile kernel beyond, which reads the packed layout directly (the
 * interleaved rows are separated as they are copied to LDS). Same layout
 * and alignment rules; K below 2^22 on the tile kernel; the tile kernel may
 * split K and use the library's tile-kernel workspace. (Source: "Add the
 * 3bit packed qmm_t", affine_packed_qmm_op: qmv for few rows, otherwise
 * affine_packed_qmm_t.)
 */
qmm_status qmm_t_affine_packed(const void* x, const uint32_t* wq_packed,
                               const void* sb_packed, qmm_dtype dt, int64_t M,
                               int64_t N, int64_t K, int group_size, int bits,
                               void* y, void* stream);

/*
 * Non-transposed product: y[M,N] = x[M,K] . dequant(W)[K,N], where the
 * weight W [K, N] is quantized along N (qmm_quantize of the K rows):
 *   y[m,n] = sum_k x[m,k] * (scale[k,n/gs] * q[k,n] + bias[k,n/gs]),
 * fp32 accumulation, y rounded to nearest even in dt. wq is [K, N*bits/32]
 * uint32, scales and biases [K, N/group_size]; N must be a multiple of
 * group_size (QMM_E_SHAPE otherwise). From 5 rows of x (f16) or 7 (bf16),
 * when K % 8 == 0 and W is below 2 GiB, an MFMA tile kernel (W read once
 * per 128 rows; with few output tiles K is split over workgroups, whose
 * fp32 partial tiles go to the library's split-K workspace and the tile
 * counters, the last split of each tile adding them). Otherwise the GEMV:
 * one pass over W per row of x, K split over workgroups; when K > 128 the
 * fp32 partial sums of the ceil(K/128) K ranges go to the split-K
 * workspace, so the rows of x are taken in blocks of at most
 * floor(16M / (ceil(K/128) * N)) (and 65535) rows, one launch pair each;
 * QMM_E_SHAPE when a single row does not fit, QMM_E_ALIGN when a block's x
 * or y would not start 16-byte aligned (K or N not a multiple of 8 with
 * more rows than one block). Both share the workspace with qmm_t on the
 * device: calls that overlap on one device race.
 * (Source: "mlx 1.0.0 backend/cpu/quantized.cpp", _qmm, the non-transposed
 * branch of quantized_matmul.)
 */
qmm_status qmm_n(const void* x, const uint32_t* wq, const void* scales,
                 const void* biases, qmm_dtype dt, int64_t M, int64_t N,
                 int64_t K, int group_size, int bits, void* y, void* stream);

/*
 * Gathered GEMV (one quantized weight per product, e.g. the experts of a
 * mixture-of-experts layer at decode): for z in [0, batches),
 *   y[z] = x[lhs_indices[z]] . dequant(W[rhs_indices[z]])^T,
 * where x is [x_batches, M, K], wq [w_batches, N, K*bits/32], scales and
 * biases [w_batches, N, K/group_size], y [batches, M, N]; every product is
 * the qmv/qmm_t product above with fp32 accumulation. lhs_indices and
 * rhs_indices are DEVICE arrays of `batches` int32 (4-byte aligned); a NULL
 * array means index z (then x, resp. W, needs at least `batches` batches).
 * Index values are read on the device, so they cannot be checked here: a
 * value outside [0, x_batches) or [0, w_batches) is clamped into range (no
 * access leaves the arrays; that product then uses the clamped batch).
 * Runs on the streaming GEMV (one pass over each selected W per row of x),
 * so K must be within its limit (QMM_E_SHAPE otherwise); meant
 * for small M. batches <= 65535.
 * (Source: "Add the 3bit packed qmm_t", ops.cpp gather_qmm: optional
 * lhs_indices / rhs_indices, defaulting to the batch position, one product
 * per index pair, one element type for x, scales, biases and y.)
 */
qmm_status qmm_gather_qmv(const void* x, int64_t x_batches,
                          const int32_t* lhs_indices, const uint32_t* wq,
                          const void* scales, const void* biases,
                          int64_t w_batches, const int32_t* rhs_indices,
                          int64_t batches, qmm_dtype dt, int64_t M, int64_t N,
                          int64_t K, int group_size, int bits, void* y,
                          void* stream);

/*
 * Gathered product for any M (e.g. the experts of a mixture-of-experts
 * layer with many tokens per expert): same operation, arguments, index
 * rules and clamping as qmm_gather_qmv. Few rows per product (the qmm_t
 * route's streaming GEMV rows) run on the gathered streaming GEMV; the rest
 * on the MFMA tile kernel in one launch, which needs K below its limit and
 * the per-batch sizes of x (M*K), y (M*N) and wq (N*K*bits/8 bytes) to be
 * multiples of 16 bytes (QMM_E_SHAPE / QMM_E_ALIGN otherwise); a K split
 * keeps the partial sums of all products in the split-K workspace.
 * batches <= 65535 and batches*M < 2^31.
 * (Source: "Add the 3bit packed qmm_t", ops.cpp gather_qmm, as for
 * qmm_gather_qmv; the per-batch offsets of the batched
 * adjust_matrix_offsets in quantized.h.)
 */
qmm_status qmm_gather_qmm(const void* x, int64_t x_batches,
                          const int32_t* lhs_indices, const uint32_t* wq,
                          const void* scales, const void* biases,
                          int64_t w_batches, const int32_t* rhs_indices,
                          int64_t batches, qmm_dtype dt, int64_t M, int64_t N,
                          int64_t K, int group_size, int bits, void* y,
                          void* stream);

/*
 * Quantized 2-D convolution, NHWC, dilation 1, no bias:
 *   x [B,H,W,C] (dt), y [B,OH,OW,O] (dt), OH = (H + 2*pad_h - kh)/stride_h + 1,
 *   OW likewise. The weight [O, kh, kw, C/groups] is reshaped to
 *   [O, K_true = kh*kw*C/groups] in (dy, dx, c) order, zero-padded on the
 *   right to K_pad = ceil(K_true/group_size)*group_size and quantized with
 *   qmm_quantize: wq [O, K_pad*bits/32], scales/biases [O, K_pad/gs].
 *   Output channel o belongs to conv group o / (O/groups), which reads input
 *   channels [g*C/groups, (g+1)*C/groups). Computed as an implicit-im2col
 *   GEMM (rows = output pixels, columns = output channels), with patch
 *   elements outside the image and k >= K_true contributing zero.
 *   (Source: mlx issue 2714, quantize_weights / img2col / forward.)
 */
qmm_status qconv2d_nhwc(const void* x, int64_t B, int64_t H, int64_t W,
                        int64_t C, const uint32_t* wq, const void* scales,
                        const void* biases, int64_t O, int kh, int kw,
                        int stride_h, int stride_w, int pad_h, int pad_w,
                        int groups, qmm_dtype dt, int group_size, int bits,
                        void* y, void* stream);

/*
 * Kernels of the affine products (qmm_t, qmv, qmm_t_batched, the packed
 * layout's entry points): which one runs is a function of (dt, bits,
 * group_size, M, N, K) only. (Source: the qmv / qmm_t split of "Add the
 * 3bit packed qmm_t", affine_packed_qmm_op, which switches at a fixed row
 * count; here the switch points come from measured kernel times.)
 */
#define QMM_KERNEL_NONE 0       /* no kernel takes the shape */
#define QMM_KERNEL_GEMV 1       /* streaming dot2 GEMV (x staged in LDS) */
#define QMM_KERNEL_MFMA_GEMV 2  /* MFMA GEMV, at most 32 rows of x */
#define QMM_KERNEL_TILE 3       /* MFMA tile GEMM */

/*
 * The kernel qmm_t runs for this shape (QMM_KERNEL_*; QMM_KERNEL_NONE for
 * invalid bits/group sizes or non-positive sizes). Host only, no GPU call.
 */
int qmm_route(qmm_dtype dt, int bits, int group_size, int64_t M, int64_t N, int64_t K);

/*
 * Smallest M (>= 1) at which qmm_t runs the MFMA tile kernel for an [N, K]
 * layer, i.e. where it leaves the GEMV kernels (0 when it never does below
 * 2^20 rows). Host only.
 */
int64_t qmm_crossover_m(qmm_dtype dt, int bits, int group_size, int64_t N, int64_t K);

/*
 * For measurement: from now on, in this process, qmm_t, qmv and
 * qmm_t_batched run `kernel` (QMM_KERNEL_GEMV, _MFMA_GEMV or _TILE) for every
 * shape that kernel takes (qmv never runs the tile kernel), and qmm_fp_t its
 * GEMV for QMM_KERNEL_GEMV and its tile kernel for QMM_KERNEL_TILE; the
 * automatic choice otherwise. QMM_KERNEL_NONE restores the automatic choice
 * everywhere. Not synchronised with calls in flight on other threads.
 * Returns QMM_E_ARG for other values.
 */
qmm_status qmm_force_kernel(int kernel);

/* Message for the last non-OK status returned on the calling thread. */
const char* qmm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif
