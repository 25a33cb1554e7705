"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on
the same seeded inputs.

Gates: quantize / pack / dequantize bit-exact; qmv, qmm_t and qconv2d against
the oracle's fp32 result y32 within relative Frobenius error 1e-3 (beyond the
oracle's own rounding of y32 to the element type) and max error
1e-2 * max|y32| (tests/helpers.py). Sizes span several tiles with ragged tails in M, N and K; the
full-size workloads are checked whole where the oracle is fast enough and on
sampled rows otherwise.
"""
import numpy as np
import pytest
import torch

from group_wise_affine_amd import qmm as Q
from group_wise_affine_amd import synth
from tests.helpers import (assert_parity, bytes_to_words_dev, from_dev, orc_code,
                           to_dev, words_dev_to_bytes)

pytestmark = pytest.mark.gpu

BITS = [2, 3, 4, 5, 6, 8]
GS = [32, 64, 128]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    Q.lib()


def _quantized(orc, dt, N, K, gs, bits, seed=2, sigma=1.0, structured=False):
    """Seeded normal weights, quantized by the oracle; with ``structured`` the
    first rows (up to 9, at most a quarter of the rows) hold the quantizer's
    special groups (zeros, constants, ramps, exact zeros, symmetric extremes,
    an outlier, tiny values) at the same spread."""
    code = orc_code(orc, dt)
    w = synth.normal((N, K), seed=seed, sigma=sigma, dt=dt)
    if structured:
        ns = min(9, max(N // 4, 1))
        w[:ns] = synth.structured_rows(ns, K, gs, seed=seed + 1, dt=dt, sigma=sigma)
    wq, s, b = orc.quantize(w, code, gs, bits)
    return w, wq, s, b


# ------------------------------------------------------------ quantize

@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("gs", GS)
@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
def test_quantize_bit_exact(orc, dt, gs, bits):
    rows, K = 37, gs * 5
    w = synth.normal((rows, K), seed=10 + bits, sigma=2.0, dt=dt)
    w[:18] = synth.structured_rows(18, K, gs, seed=4, dt=dt)
    wq_o, s_o, b_o = orc.quantize(w, orc_code(orc, dt), gs, bits)
    wq, s, b = Q.qmm_quantize(to_dev(w, dt), gs, bits)
    torch.cuda.synchronize()
    assert np.array_equal(words_dev_to_bytes(wq), wq_o)
    assert np.array_equal(from_dev(s), s_o)
    assert np.array_equal(from_dev(b), b_o)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
def test_dequantize_bit_exact(orc, dt, bits):
    gs, rows, K = 64, 29, 448
    w, wq, s, b = _quantized(orc, dt, rows, K, gs, bits, structured=True)
    _, w_o = orc.dequantize(wq, s, b, orc_code(orc, dt), K, gs, bits)
    out = Q.qmm_dequantize(bytes_to_words_dev(wq), to_dev(s, dt), to_dev(b, dt), gs, bits)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(out), w_o)


def test_quantize_large_rows(orc):
    """A full-size decode weight (4096 x 4096, 4-bit g64 f16), bit-exact."""
    w = synth.normal((4096, 4096), seed=1)
    wq_o, s_o, b_o = orc.quantize(w, orc.F16, 64, 4)
    wq, s, b = Q.qmm_quantize(to_dev(w, "f16"), 64, 4)
    torch.cuda.synchronize()
    assert np.array_equal(words_dev_to_bytes(wq), wq_o)
    assert np.array_equal(from_dev(s), s_o) and np.array_equal(from_dev(b), b_o)


# ------------------------------------------------------------ qmv

def _run_mm(fn, orc, dt, M, N, K, gs, bits, seed=0, sigma_w=1.0, rows=None, x=None,
            structured=True):
    """fn (qmv / qmm_t) against the oracle on seeded x (N(0,1) unless given)
    and seeded weights with structured rows."""
    code = orc_code(orc, dt)
    if x is None:
        x = synth.normal((M, K), seed=seed, dt=dt)
    w, wq, s, b = _quantized(orc, dt, N, K, gs, bits, seed=seed + 1, sigma=sigma_w,
                             structured=structured)
    y = fn(to_dev(x, dt), bytes_to_words_dev(wq), to_dev(s, dt), to_dev(b, dt), gs, bits)
    torch.cuda.synchronize()
    yg = from_dev(y)
    if rows is not None:
        yo, _ = orc.qmm_t(x, wq, s, b, code, gs, bits, nthreads=8, rows=rows)
        yg = yg[rows[0]:rows[1]]
    else:
        yo, _ = orc.qmm_t(x, wq, s, b, code, gs, bits, nthreads=8)
    return assert_parity(yg, yo, dt, f"{fn.__name__} {dt} M{M} N{N} K{K} g{gs} b{bits}")


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("gs", GS)
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_qmv_parity(orc, dt, gs, bits):
    # K = 640: 20 chunks of 32 codes (ragged against the lanes per row);
    # N = 70: ragged against the rows per workgroup
    for M in (1, 3, 8):
        _run_mm(Q.qmv, orc, dt, M, 70, 640, gs, bits, seed=M)


@pytest.mark.parametrize("M", [2, 5, 11, 16, 20])
def test_qmv_multi_m_blocks(orc, M):
    _run_mm(Q.qmv, orc, "f16", M, 130, 1024, 64, 4, seed=M)
    _run_mm(Q.qmv, orc, "bf16", M, 33, 2048, 128, 3, seed=M)


@pytest.mark.parametrize("N,K", [(1, 32), (5, 64), (257, 96), (64, 8192), (3, 15360)])
def test_qmv_edge_shapes(orc, N, K):
    gs = 32
    _run_mm(Q.qmv, orc, "f16", 1, N, K, gs, 4, seed=N)
    _run_mm(Q.qmv, orc, "bf16", 2, N, K, gs, 8, seed=N)


@pytest.mark.parametrize("M,N,K,gs,bits", [
    (3, 17, 352, 32, 4),        # one ragged row block, K % 128 == 96: partial steps
    (16, 200, 4160, 64, 4),     # 33 steps: one round of 4 with empty slots
    (5, 300, 2080, 32, 3),      # one round of 2
    (12, 64, 6144, 64, 5),
    (9, 96, 2048, 128, 6),      # one step per wavefront
    (7, 40, 4096, 32, 8),
    (4, 130, 11008, 128, 2),    # ring of 3 steps, uneven steps per wavefront
    (1, 4096, 8704, 64, 4),     # M = 1 on the MFMA GEMV: long rows, wide layer
    (2, 4100, 12288, 64, 4),    # ring with whole rounds, ragged N
    (6, 72, 9216, 32, 5),       # ring, 5-bit
    (8, 40, 8704, 64, 8),       # ring, 8-bit
])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_qmv_mfma(orc, dt, M, N, K, gs, bits):
    """The MFMA GEMV (up to 16 rows of x), through qmv and qmm_t."""
    _run_mm(Q.qmv, orc, dt, M, N, K, gs, bits, seed=K + M)
    _run_mm(Q.qmm_t, orc, dt, M, N, K, gs, bits, seed=K + M + 1)


@pytest.mark.parametrize("M,N,K,gs,bits", [
    (17, 200, 4160, 64, 4),     # two row tiles, 3 K ranges of 11 steps (x through registers)
    (24, 4096, 4096, 64, 4),    # 256 row blocks, 2 K ranges of 2048 (direct x copy)
    (32, 96, 2048, 128, 6),     # one range, 128 x blocks of 512 (the direct copy's limit)
    (20, 40, 8704, 32, 8),      # 5 ranges of 14 steps
    (32, 130, 4096, 32, 5),     # ragged row block
    (29, 72, 2048, 64, 3),
    (25, 64, 2048, 32, 2),
])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_qmv_mfma_two_row_tiles(orc, dt, M, N, K, gs, bits):
    """The MFMA GEMV with 17..32 rows of x (two 16-row tiles sharing each
    dequantized W fragment), forced through qmm_t and qmv."""
    try:
        Q.force_kernel(Q.KERNEL_MFMA_GEMV)
        _run_mm(Q.qmm_t, orc, dt, M, N, K, gs, bits, seed=K + M)
        _run_mm(Q.qmv, orc, dt, M, N, K, gs, bits, seed=K + M + 1)
    finally:
        Q.force_kernel(Q.KERNEL_NONE)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_qmv_mfma_split_k_repeat(orc, dt):
    """Narrow layers split K over workgroups; the last one to finish adds the
    partial tiles and resets its row block's counter. Calls in a row (same
    shape, then another, then the first again) must all be exact."""
    code = orc_code(orc, dt)
    cases = []
    for (M, N, K, gs, bits, seed) in [(8, 512, 8192, 64, 4, 1), (5, 96, 4160, 32, 3, 2)]:
        x = synth.normal((M, K), seed=seed, dt=dt)
        w = synth.normal((N, K), seed=seed + 1, dt=dt)
        wq, s, b = orc.quantize(w, code, gs, bits)
        yo, _ = orc.qmm_t(x, wq, s, b, code, gs, bits, nthreads=8)
        dev = (to_dev(x, dt), bytes_to_words_dev(wq), to_dev(s, dt), to_dev(b, dt), gs, bits)
        cases.append((dev, yo, (M, N, K)))
    outs = []
    for i in (0, 0, 1, 0, 1, 1):
        outs.append((Q.qmv(*cases[i][0]), i))
    torch.cuda.synchronize()
    for y, i in outs:
        assert_parity(from_dev(y), cases[i][1], dt, f"split-K GEMV repeat {cases[i][2]}")


@pytest.mark.parametrize("dt,M", [("f16", 5), ("f16", 1), ("bf16", 2)])
def test_qmv_unaligned_scales(orc, dt, M):
    """Scales and biases only 2-byte aligned (views at an odd element offset).
    The MFMA GEMV (f16, 5 rows) reads them as aligned 16-byte units around
    the block; the streaming GEMV (1 and 2 rows) cannot stage them with
    16-byte loads and reads them per lane."""
    code = orc_code(orc, dt)
    N, K, gs, bits = 70, 1024, 32, 4
    x = synth.normal((M, K), seed=3, dt=dt)
    w = synth.normal((N, K), seed=4, dt=dt)
    wq, s, b = orc.quantize(w, code, gs, bits)
    yo, _ = orc.qmm_t(x, wq, s, b, code, gs, bits, nthreads=8)
    sd, bd = to_dev(s, dt), to_dev(b, dt)
    s_big = torch.zeros(sd.numel() + 1, dtype=sd.dtype, device=sd.device)
    b_big = torch.zeros(bd.numel() + 3, dtype=bd.dtype, device=bd.device)
    s_big[1:].copy_(sd.reshape(-1))
    b_big[3:].copy_(bd.reshape(-1))
    y = Q.qmv(to_dev(x, dt), bytes_to_words_dev(wq), s_big[1:].view(sd.shape),
              b_big[3:].view(bd.shape), gs, bits)
    torch.cuda.synchronize()
    assert_parity(from_dev(y), yo, dt, "qmv unaligned scales")


@pytest.mark.parametrize("dt,N,K,gs,bits", [
    ("bf16", 4100, 4096, 32, 3),    # ragged last workgroup (4 of 16 rows)
    ("f16", 8192, 2048, 128, 5),
    ("bf16", 4096, 4096, 64, 6),
    ("f16", 2560, 4160, 64, 4),     # 64 lanes per row, the last chunks past the row end
])
def test_qmv_decode_wide(orc, dt, N, K, gs, bits):
    """One row of x over layers that make one round of 256 to 320 workgroups
    in the 8-wavefront lane shape (one W row per lane), with staged scales
    and biases."""
    _run_mm(Q.qmv, orc, dt, 1, N, K, gs, bits, seed=N + bits)


def test_qmv_max_k(orc):
    """The largest K the streaming kernel accepts (f16 4-bit, g32)."""
    _run_mm(Q.qmv, orc, "f16", 1, 3, 29120, 32, 4, seed=3)


# ------------------------------------------------------------ small activations

def _x_of(kind, M, K, seed, dt):
    """Activations that f16 holds only as small normals or subnormals:
    N(0, 1e-4), N(0, 3e-5), and rows mixing 1e-5 and 1e2 magnitudes."""
    if kind == "mixed":
        return synth.mixed_magnitude((M, K), seed=seed, dt=dt)
    return synth.normal((M, K), seed=seed, sigma={"n1e-4": 1e-4, "n3e-5": 3e-5}[kind], dt=dt)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("kind", ["n1e-4", "n3e-5", "mixed"])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_small_activations(orc, dt, kind, bits):
    """Every kernel that takes x: the streaming GEMV (M = 1, 2), the MFMA GEMV
    (M = 5), the tile kernel (M = 100), through qmv and qmm_t."""
    N, K, gs = 96, 1024, 64
    for M in (1, 2, 5, 100):
        x = _x_of(kind, M, K, seed=M + bits, dt=dt)
        fns = (Q.qmv, Q.qmm_t) if M <= 16 else (Q.qmm_t,)
        for fn in fns:
            _run_mm(fn, orc, dt, M, N, K, gs, bits, seed=M + 7, x=x)


@pytest.mark.parametrize("kind", ["n1e-4", "n3e-5", "mixed"])
@pytest.mark.parametrize("bits", [2, 4, 8])
def test_small_activations_decode_shape(orc, kind, bits):
    """x f16 [1, 4096] of small magnitude on the 4096 x 4096 decode layer
    (the 8-wavefront lane shape of the streaming GEMV)."""
    x = _x_of(kind, 1, 4096, seed=bits, dt="f16")
    _run_mm(Q.qmm_t, orc, "f16", 1, 4096, 4096, 64, bits, seed=0, x=x)


@pytest.mark.parametrize("kind", ["n1e-4", "n3e-5", "mixed"])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_small_activations_gather_batched(orc, dt, kind):
    """Gathered GEMV and batched weights at M = 1 with small activations and
    structured weight rows."""
    code = orc_code(orc, dt)
    Bx, E, M, N, K, gs, bits = 3, 4, 1, 72, 1024, 64, 4
    x = np.stack([_x_of(kind, M, K, seed=20 + i, dt=dt) for i in range(Bx)])
    parts = [_quantized(orc, dt, N, K, gs, bits, seed=30 + e, structured=True)[1:]
             for e in range(E)]
    wq = np.stack([p[0] for p in parts])
    s = np.stack([p[1] for p in parts])
    b = np.stack([p[2] for p in parts])
    lhs, rhs = [2, 0, 1, 1], [3, 1, 0, 2]
    yo, _ = orc.gather_qmm(x, wq, s, b, lhs, rhs, code, gs, bits, nthreads=8)
    y = Q.gather_qmv(to_dev(x, dt), bytes_to_words_dev(wq), to_dev(s, dt), to_dev(b, dt),
                     _idx_dev(lhs), _idx_dev(rhs), gs, bits)
    torch.cuda.synchronize()
    for z in range(len(lhs)):
        assert_parity(from_dev(y[z]), yo[z], dt, f"gather_qmv small x batch {z}")
    yo, _ = orc.gather_qmm(x, wq[:Bx], s[:Bx], b[:Bx], None, None, code, gs, bits, nthreads=8)
    y = Q.qmm_t_batched(to_dev(x, dt), bytes_to_words_dev(wq[:Bx]), to_dev(s[:Bx], dt),
                        to_dev(b[:Bx], dt), gs, bits)
    torch.cuda.synchronize()
    for z in range(Bx):
        assert_parity(from_dev(y[z]), yo[z], dt, f"qmm_t_batched small x batch {z}")


# ------------------------------------------------------------ qmm_t (MFMA)

@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("gs", GS)
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_qmm_t_mfma_parity(orc, dt, gs, bits):
    # M >= crossover routes to the MFMA kernel; ragged M, N and a K with a
    # half K-step tail (K % 64 == 32 when gs == 32)
    K = 384 if gs != 32 else 352
    _run_mm(Q.qmm_t, orc, dt, 100, 72, K, gs, bits, seed=bits)


@pytest.mark.parametrize("M,N,K", [(16, 16, 64), (129, 200, 640), (300, 520, 256),
                                   (1, 128, 128), (513, 33, 1024)])
def test_qmm_t_shapes(orc, M, N, K):
    _run_mm(Q.qmm_t, orc, "f16", M, N, K, 64, 4, seed=M)
    _run_mm(Q.qmm_t, orc, "bf16", M, N, K, 64, 6, seed=M)


@pytest.mark.parametrize("M,N,K,gs,bits", [
    (130, 200, 1536, 64, 4),    # 24 steps: too few to split (unsplit 64 x 64 tiles)
    (200, 300, 4096, 32, 3),    # split 4 ways
    (64, 64, 2080, 32, 4),      # 33 steps: last split a single step, K % 64 == 32
    (257, 130, 4160, 64, 8),    # ragged M and N, K not a multiple of a stage
    (40, 300, 4096, 128, 2),
    (100, 96, 2560, 32, 3),
    (72, 136, 3072, 64, 5),
    (33, 64, 2048, 128, 6),
])
def test_qmm_t_split_k(orc, M, N, K, gs, bits):
    """Few output tiles: K is split over workgroups (fp32 partial sums in the
    library's workspace, then a reduction)."""
    _run_mm(Q.qmm_t, orc, "f16", M, N, K, gs, bits, seed=K)
    _run_mm(Q.qmm_t, orc, "bf16", M, N, K, gs, bits, seed=K + 1)


@pytest.mark.parametrize("M,N,K,gs,bits", [
    (2, 200, 384, 64, 4),       # one split, ragged N
    (9, 130, 1088, 32, 4),      # K % 64 == 0, 17 steps over splits
    (17, 300, 2080, 32, 2),     # K % 64 == 32
    (32, 256, 4096, 64, 8),
    (24, 96, 1536, 128, 3),
    (31, 136, 3072, 64, 5),
    (20, 64, 2048, 128, 6),
])
def test_qmm_t_skinny(orc, M, N, K, gs, bits):
    """At most 32 rows above the crossover: 32-row tiles, K split over
    workgroups when the output has few tiles."""
    M = max(M, Q.crossover_m(bits, torch.float16, N, K, gs))
    _run_mm(Q.qmm_t, orc, "f16", M, N, K, gs, bits, seed=K + M)
    M = max(M, Q.crossover_m(bits, torch.bfloat16, N, K, gs))
    _run_mm(Q.qmm_t, orc, "bf16", M, N, K, gs, bits, seed=K + M + 1)


def test_qmm_t_split_k_back_to_back(orc):
    """Two split-K calls in a row on one stream reuse the workspace: the second
    (smaller) result must not see the first one's partial sums."""
    code = orc_code(orc, "f16")
    outs = []
    for (M, N, K, seed) in [(96, 256, 4096, 5), (40, 64, 2048, 6)]:
        x = synth.normal((M, K), seed=seed, dt="f16")
        w = synth.normal((N, K), seed=seed + 1, dt="f16")
        wq, s, b = orc.quantize(w, code, 64, 4)
        yo, _ = orc.qmm_t(x, wq, s, b, code, 64, 4, nthreads=8)
        y = Q.qmm_t(to_dev(x, "f16"), bytes_to_words_dev(wq), to_dev(s, "f16"),
                    to_dev(b, "f16"), 64, 4)
        outs.append((y, yo, (M, N, K)))
    torch.cuda.synchronize()
    for y, yo, shape in outs:
        assert_parity(from_dev(y), yo, "f16", f"split-K back to back {shape}")


@pytest.mark.parametrize("M,N,K,bits", [
    (31, 136, 3072, 5),     # 32-row tiles, K split 6 ways
    (200, 160, 1472, 4),    # 64 x 64 tiles, two wavefronts per slice
    (1024, 3072, 512, 4),   # 128 x 128 tiles (192 of them)
])
def test_tile_reads_only_landed_copies(orc, M, N, K, bits):
    """Regression: each workgroup of the tile kernel must read a ring slot
    only after its copies have landed (the first step builds the second
    step's state). Launches on NaN activations leave NaN in the LDS slots of
    the CUs; a read of a slot before its copy lands then shows as NaN or a
    parity failure in the following launch on finite inputs."""
    gs, dt = 64, "f16"
    _, wq, s, b = _quantized(orc, dt, N, K, gs, bits, seed=N + K)
    x = synth.normal((M, K), seed=M, dt=dt)
    yo, _ = orc.qmm_t(x, wq, s, b, orc.F16, gs, bits, nthreads=8)
    wd, sd, bd = bytes_to_words_dev(wq), to_dev(s, dt), to_dev(b, dt)
    xd = to_dev(x, dt)
    xnan = torch.full((M, K), float("nan"), dtype=torch.float16, device="cuda")
    for it in range(8):
        Q.qmm_t(xnan, wd, sd, bd, gs, bits)
        y = Q.qmm_t(xd, wd, sd, bd, gs, bits)
        torch.cuda.synchronize()
        assert_parity(from_dev(y), yo, dt, f"tile after NaN launch {it} M{M} N{N} K{K} b{bits}")


@pytest.mark.parametrize("M,N,K,gs,bits", [
    (12, 64, 6144, 64, 5),      # K split, one step per wavefront: 16 + 4 byte chunk loads
    (6, 96, 4096, 64, 3),       # 12-byte chunk loads
    (16, 4096, 4096, 64, 5),    # 256 row blocks, two steps per wavefront
    (8, 512, 8192, 32, 3),
    (4, 256, 4096, 64, 4),
])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_mfma_gemv_reads_only_landed_x(orc, dt, M, N, K, gs, bits):
    """Regression: the MFMA GEMV's direct x copy into LDS ends with a wait
    that must leave only the weight loads in flight. When the compiler merged
    the 3- and 5-bit chunk loads into fewer instructions than the wait
    counted, the barrier could pass with x copies still landing. Launches on
    NaN activations leave NaN in the x region of LDS; a read before the copy
    lands then shows as NaN or a parity failure in the next launch."""
    code = orc_code(orc, dt)
    _, wq, s, b = _quantized(orc, dt, N, K, gs, bits, seed=N + K + bits)
    x = synth.normal((M, K), seed=M + bits, dt=dt)
    yo, _ = orc.qmm_t(x, wq, s, b, code, gs, bits, nthreads=8)
    wd, sd, bd = bytes_to_words_dev(wq), to_dev(s, dt), to_dev(b, dt)
    xd = to_dev(x, dt)
    xnan = torch.full((M, K), float("nan"), dtype=xd.dtype, device="cuda")
    try:
        Q.force_kernel(Q.KERNEL_MFMA_GEMV)
        for it in range(8):
            Q.qmm_t(xnan, wd, sd, bd, gs, bits)
            y = Q.qmm_t(xd, wd, sd, bd, gs, bits)
            torch.cuda.synchronize()
            assert_parity(from_dev(y), yo, dt, f"MFMA GEMV after NaN launch {it} {dt} M{M} N{N} K{K} b{bits}")
    finally:
        Q.force_kernel(Q.KERNEL_NONE)


def test_scratch_calls_on_two_streams(orc):
    """Calls that use the shared split-K scratch, queued alternately on two
    streams without any ordering by the caller: the library orders them (an
    event per device), so every result stays exact."""
    code = orc_code(orc, "f16")
    cases = []
    for (M, N, K, seed) in [(96, 256, 4096, 21), (40, 64, 2048, 22), (8, 512, 8192, 23),
                            (64, 256, 4096, 24)]:
        x = synth.normal((M, K), seed=seed, dt="f16")
        w = synth.normal((N, K), seed=seed + 1, dt="f16")
        wq, s, b = orc.quantize(w, code, 64, 4)
        yo, _ = orc.qmm_t(x, wq, s, b, code, 64, 4, nthreads=8)
        dev = (to_dev(x, "f16"), bytes_to_words_dev(wq), to_dev(s, "f16"), to_dev(b, "f16"))
        cases.append((dev, yo, (M, N, K)))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    outs = []
    for rep in range(3):
        for i, (dev, yo, shape) in enumerate(cases):
            st = streams[(i + rep) % 2]
            with torch.cuda.stream(st):
                y = torch.empty((shape[0], shape[1]), dtype=torch.float16, device="cuda")
                outs.append((Q.qmm_t(*dev, 64, 4, out=y), yo, shape))
    torch.cuda.synchronize()
    for y, yo, shape in outs:
        assert_parity(from_dev(y), yo, "f16", f"two streams {shape}")


def test_qmm_t_routes_consistently(orc):
    """Around the crossover both kernels agree with the oracle."""
    mx = Q.crossover_m(4, torch.float16, 96, 512, 64)
    for M in (mx - 1, mx, mx + 1):
        if M >= 1:
            _run_mm(Q.qmm_t, orc, "f16", M, 96, 512, 64, 4, seed=M)


# ------------------------------------------------------------ qconv2d

CONV = [
    # B, H, W, C, O, kh, kw, stride, pad, groups, gs, bits
    (1, 9, 7, 16, 24, 3, 3, (1, 1), (1, 1), 1, 32, 4),
    (2, 8, 8, 16, 8, 3, 3, (2, 1), (1, 0), 2, 32, 4),
    (1, 10, 6, 8, 6, 5, 3, (1, 2), (2, 1), 1, 64, 3),
    (1, 6, 6, 32, 16, 1, 1, (1, 1), (0, 0), 1, 32, 8),
    (1, 7, 5, 20, 10, 3, 2, (1, 1), (0, 1), 5, 32, 6),   # Cg = 4: scalar im2col
    (1, 5, 5, 24, 12, 3, 3, (1, 1), (1, 1), 3, 128, 5),
    (2, 17, 19, 64, 96, 3, 3, (1, 1), (1, 1), 1, 64, 2),
    (1, 12, 12, 48, 40, 3, 3, (2, 2), (0, 0), 2, 64, 4),
    (1, 16, 16, 128, 64, 3, 3, (1, 1), (1, 1), 1, 64, 4),  # 18 K steps: split K
    (1, 14, 14, 256, 32, 3, 3, (1, 1), (1, 1), 2, 128, 4),  # split K per group
]


@pytest.mark.parametrize("case", CONV)
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_qconv2d_parity(orc, dt, case):
    B, H, W, C, O, kh, kw, stride, pad, groups, gs, bits = case
    code = orc_code(orc, dt)
    x = synth.normal((B, H, W, C), seed=12, dt=dt)
    wconv = synth.normal((O, kh, kw, C // groups), seed=13, sigma=0.5, dt=dt)
    # structured groups in the first output channels (along the flattened taps)
    ns, kt = min(9, max(O // 4, 1)), kh * kw * (C // groups)
    wconv[:ns] = synth.structured_rows(ns, kt, gs, seed=14, dt=dt, sigma=0.5).reshape(
        ns, kh, kw, C // groups)
    wm = orc.conv_weight_matrix(wconv, groups, gs)
    wq, s, b = orc.quantize(wm, code, gs, bits)
    yo, _ = orc.qconv2d_nhwc(x, wq, s, b, code, O, kh, kw, stride, pad, groups, gs, bits,
                             nthreads=8)
    y = Q.qconv2d_nhwc(to_dev(x, dt), bytes_to_words_dev(wq), to_dev(s, dt), to_dev(b, dt),
                       O, kh, kw, stride, pad, groups, gs, bits)
    torch.cuda.synchronize()
    assert_parity(from_dev(y), yo, dt, f"conv {case} {dt}")


def test_conv_weight_prep_matches_oracle(orc):
    """The binding's reshape + zero pad + GPU quantize equals the oracle's."""
    wconv = synth.normal((20, 3, 3, 30), seed=3)
    wm_o = orc.conv_weight_matrix(wconv, 1, 64)
    wq_o, s_o, b_o = orc.quantize(wm_o, orc.F16, 64, 4)
    wq, s, b = Q.quantize_conv_weight(to_dev(wconv, "f16"), 64, 4)
    torch.cuda.synchronize()
    assert np.array_equal(words_dev_to_bytes(wq), wq_o)
    assert np.array_equal(from_dev(s), s_o) and np.array_equal(from_dev(b), b_o)


# ------------------------------------------------------------ full-size workloads

def test_tiny_qmm_t_config(orc):
    """x f16 [8,512], W [512,512] 4-bit g64, seed 0."""
    _run_mm(Q.qmm_t, orc, "f16", 8, 512, 512, 64, 4, seed=0)


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("M", [1, 16])
def test_decode_qmv_config(orc, bits, M):
    """x f16 [M,4096], W [4096,4096] g64, full output against the oracle."""
    _run_mm(Q.qmv, orc, "f16", M, 4096, 4096, 64, bits, seed=0)
    _run_mm(Q.qmm_t, orc, "f16", M, 4096, 4096, 64, bits, seed=0)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_chained_qmm_config(orc, bits):
    """First loop of x = qmm(qmm(x, W1), W2), x [1024,1024], W1 [4096,1024],
    W2 [1024,4096], g64 f16: checked on sampled rows (the oracle recomputes
    rows 0..15 and 1000..1023 of each product)."""
    gs = 64
    x = synth.normal((1024, 1024), seed=0)
    _, wq1, s1, b1 = _quantized(orc, "f16", 4096, 1024, gs, bits, seed=1)
    _, wq2, s2, b2 = _quantized(orc, "f16", 1024, 4096, gs, bits, seed=2)
    xd = to_dev(x, "f16")
    h = Q.qmm_t(xd, bytes_to_words_dev(wq1), to_dev(s1, "f16"), to_dev(b1, "f16"), gs, bits)
    y = Q.qmm_t(h, bytes_to_words_dev(wq2), to_dev(s2, "f16"), to_dev(b2, "f16"), gs, bits)
    torch.cuda.synchronize()
    hg, yg = from_dev(h), from_dev(y)
    for rows in [(0, 16), (1000, 1024)]:
        ho, _ = orc.qmm_t(x, wq1, s1, b1, orc.F16, gs, bits, nthreads=8, rows=rows)
        assert_parity(hg[rows[0]:rows[1]], ho, "f16", f"chained h bits{bits}")
        # second product on the GPU's own h rows (isolates the second kernel)
        yo, _ = orc.qmm_t(hg, wq2, s2, b2, orc.F16, gs, bits, nthreads=8, rows=rows)
        assert_parity(yg[rows[0]:rows[1]], yo, "f16", f"chained y bits{bits}")


SWEEP_NK = [(2048, 2048), (512, 2048), (8192, 2048), (2048, 8192)]


@pytest.mark.parametrize("N,K", SWEEP_NK)
@pytest.mark.parametrize("bits", [4, 3, 6])
def test_small_m_sweep_config(orc, N, K, bits):
    """bf16 Llama-3.2-1B-shaped layers, W ~ N(0, 0.02), g64; every M of the
    sweep, sampled rows for the large M."""
    for M in (1, 2, 4, 8, 16, 32, 64, 512):
        rows = (0, M) if M <= 64 else (M - 24, M)
        _run_mm(Q.qmm_t, orc, "bf16", M, N, K, 64, bits, seed=M, sigma_w=0.02, rows=rows)


@pytest.mark.parametrize("groups", [1, 2])
def test_conv_config(orc, groups):
    """x f16 [1,64,64,320], W [320,3,3,320/groups] ~ N(0, 0.05), 4-bit g64,
    stride 1, pad 1: full output against the oracle."""
    dt, gs, bits = "f16", 64, 4
    x = synth.normal((1, 64, 64, 320), seed=0)
    wconv = synth.normal((320, 3, 3, 320 // groups), seed=1, sigma=0.05)
    wm = orc.conv_weight_matrix(wconv, groups, gs)
    wq, s, b = orc.quantize(wm, orc.F16, gs, bits)
    yo, _ = orc.qconv2d_nhwc(x, wq, s, b, orc.F16, 320, 3, 3, (1, 1), (1, 1), groups, gs,
                             bits, nthreads=16)
    y = Q.qconv2d_nhwc(to_dev(x, dt), bytes_to_words_dev(wq), to_dev(s, dt), to_dev(b, dt),
                       320, 3, 3, (1, 1), (1, 1), groups, gs, bits)
    torch.cuda.synchronize()
    assert_parity(from_dev(y), yo, dt, f"conv config groups={groups}")


# ------------------------------------------------------------ gathered GEMV

def _gather_inputs(orc, dt, Bx, E, M, N, K, gs, bits, seed):
    code = orc_code(orc, dt)
    x = np.stack([synth.normal((M, K), seed=seed + i, dt=dt) for i in range(Bx)])
    parts = [_quantized(orc, dt, N, K, gs, bits, seed=seed + 100 + e, structured=True)[1:]
             for e in range(E)]
    wq = np.stack([p[0] for p in parts])
    s = np.stack([p[1] for p in parts])
    b = np.stack([p[2] for p in parts])
    return code, x, wq, s, b


def _idx_dev(v):
    return None if v is None else torch.tensor(v, dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("dt,Bx,E,M,N,K,gs,bits,lhs,rhs", [
    ("f16", 4, 6, 1, 70, 640, 32, 4, [3, 0, 2, 2, 1], [5, 1, 1, 0, 4]),   # ragged N
    ("bf16", 3, 3, 2, 96, 1024, 64, 3, None, None),                     # identity
    ("f16", 1, 8, 3, 200, 2048, 128, 6, [0] * 6, [7, 3, 3, 0, 6, 1]),     # one token, 6 experts
    ("bf16", 2, 4, 5, 33, 4160, 32, 2, [1, 0, 1, 0], [3, 2, 1, 0]),      # 2 row blocks of x;
                                                                         # N*G % 8 != 0
    ("f16", 1, 2, 1, 4096, 4096, 64, 4, [0, 0], [1, 0]),                 # 8-wavefront shape
    ("f16", 2, 2, 1, 64, 11008, 64, 4, [1, 0], None),                    # rows over 1 batch
    ("bf16", 2, 3, 1, 48, 512, 32, 8, [0, 1, 1], [2, 0, 2]),             # 8-bit bf16 (fp32)
])
def test_gather_qmv(orc, dt, Bx, E, M, N, K, gs, bits, lhs, rhs):
    code, x, wq, s, b = _gather_inputs(orc, dt, Bx, E, M, N, K, gs, bits, seed=K + E)
    yo, _ = orc.gather_qmm(x, wq, s, b, lhs, rhs, code, gs, bits, nthreads=8)
    y = Q.gather_qmv(to_dev(x, dt), bytes_to_words_dev(wq), to_dev(s, dt), to_dev(b, dt),
                     _idx_dev(lhs), _idx_dev(rhs), gs, bits)
    torch.cuda.synchronize()
    assert tuple(y.shape) == yo.shape
    for z in range(yo.shape[0]):
        assert_parity(from_dev(y[z]), yo[z], dt, f"gather_qmv batch {z}")


def test_gather_qmv_clamps_indices(orc):
    """Index values outside the batch ranges are clamped on the device."""
    dt, Bx, E, M, N, K, gs, bits = "f16", 2, 3, 1, 40, 256, 32, 4
    code, x, wq, s, b = _gather_inputs(orc, dt, Bx, E, M, N, K, gs, bits, seed=5)
    lhs, rhs = [-4, 1, 9], [2, 7, -1]
    yo, _ = orc.gather_qmm(x, wq, s, b, [0, 1, 1], [2, 2, 0], code, gs, bits)
    y = Q.gather_qmv(to_dev(x, dt), bytes_to_words_dev(wq), to_dev(s, dt), to_dev(b, dt),
                     _idx_dev(lhs), _idx_dev(rhs), gs, bits)
    torch.cuda.synchronize()
    assert_parity(from_dev(y), yo, dt, "gather_qmv clamped")


def test_gather_max_batches(orc):
    """65535 products (the largest batch count) on the GEMV and on the tile kernel,
    random routing; every product checked against the oracle on a sample."""
    dt, Bx, E, gs, bits, B = "f16", 7, 5, 32, 4, 65535
    rng = np.random.default_rng(9)
    lhs = rng.integers(0, Bx, B).tolist()
    rhs = rng.integers(0, E, B).tolist()
    for M, N, K, fn in ((1, 32, 64, Q.gather_qmv), (32, 128, 64, Q.gather_qmm)):
        code, x, wq, s, b = _gather_inputs(orc, dt, Bx, E, M, N, K, gs, bits, seed=M + 3)
        y = fn(to_dev(x, dt), bytes_to_words_dev(wq), to_dev(s, dt), to_dev(b, dt),
               _idx_dev(lhs), _idx_dev(rhs), gs, bits)
        torch.cuda.synchronize()
        yg = from_dev(y)
        # every (x batch, expert) pair's product, then each output against its pair
        pairs = {}
        for lz in range(Bx):
            for rz in range(E):
                pairs[lz, rz], _ = orc.qmm_t(x[lz], wq[rz], s[rz], b[rz], code, gs, bits)
        for z in list(range(0, B, 97)) + [B - 1]:
            assert_parity(yg[z], pairs[lhs[z], rhs[z]], dt, f"{fn.__name__} batch {z}")


def test_gather_qmv_rejects_bad_arguments():
    x = torch.zeros((2, 1, 64), dtype=torch.float16, device="cuda")
    wq = torch.zeros((3, 8, 8), dtype=torch.int32, device="cuda")
    s = torch.zeros((3, 8, 2), dtype=torch.float16, device="cuda")
    with pytest.raises(Q.QmmError) as e:        # 3 outputs without lhs need 3 x batches
        Q.gather_qmv(x, wq, s, s, None, _idx_dev([0, 1, 2]), 32, 4)
    assert e.value.status == Q.QMM_E_SHAPE
    with pytest.raises(Q.QmmError) as e:        # K beyond the streaming GEMV's limit
        big = torch.zeros((1, 1, 65536), dtype=torch.float16, device="cuda")
        wb = torch.zeros((1, 8, 65536 // 8), dtype=torch.int32, device="cuda")
        sb = torch.zeros((1, 8, 2048), dtype=torch.float16, device="cuda")
        Q.gather_qmv(big, wb, sb, sb, None, None, 32, 4)
    assert e.value.status == Q.QMM_E_SHAPE


@pytest.mark.parametrize("dt,Bx,E,M,N,K,gs,bits,lhs,rhs", [
    ("f16", 4, 6, 64, 256, 512, 64, 4, [3, 0, 2, 2, 1], [5, 1, 1, 0, 4]),  # tile kernel
    ("bf16", 2, 3, 40, 320, 1024, 32, 3, [1, 0, 1], [2, 2, 0]),          # ragged M, bf16
    ("f16", 1, 8, 16, 512, 2048, 128, 6, [0] * 4, [7, 3, 3, 0]),         # 32-row tiles, K split
    ("f16", 3, 4, 128, 384, 4096, 64, 4, [2, 1, 0, 2], [3, 2, 1, 0]),    # K split 4 ways
    ("bf16", 2, 2, 200, 128, 256, 32, 8, None, [1, 0]),                  # 8-bit, rhs only
    ("f16", 2, 3, 2, 96, 512, 32, 5, [1, 0], [2, 2]),                    # gathered GEMV rows
])
def test_gather_qmm(orc, dt, Bx, E, M, N, K, gs, bits, lhs, rhs):
    code, x, wq, s, b = _gather_inputs(orc, dt, Bx, E, M, N, K, gs, bits, seed=M + K + E)
    yo, _ = orc.gather_qmm(x, wq, s, b, lhs, rhs, code, gs, bits, nthreads=8)
    y = Q.gather_qmm(to_dev(x, dt), bytes_to_words_dev(wq), to_dev(s, dt), to_dev(b, dt),
                     _idx_dev(lhs), _idx_dev(rhs), gs, bits)
    torch.cuda.synchronize()
    assert tuple(y.shape) == yo.shape
    for z in range(yo.shape[0]):
        assert_parity(from_dev(y[z]), yo[z], dt, f"gather_qmm batch {z}")


def test_gather_qmm_clamps_indices(orc):
    """Index values outside the batch ranges are clamped in the tile kernel."""
    dt, Bx, E, M, N, K, gs, bits = "f16", 2, 3, 48, 128, 512, 64, 4
    code, x, wq, s, b = _gather_inputs(orc, dt, Bx, E, M, N, K, gs, bits, seed=15)
    lhs, rhs = [-3, 1, 5], [9, 0, -1]
    yo, _ = orc.gather_qmm(x, wq, s, b, [0, 1, 1], [2, 0, 0], code, gs, bits)
    y = Q.gather_qmm(to_dev(x, dt), bytes_to_words_dev(wq), to_dev(s, dt), to_dev(b, dt),
                     _idx_dev(lhs), _idx_dev(rhs), gs, bits)
    torch.cuda.synchronize()
    assert_parity(from_dev(y), yo, dt, "gather_qmm clamped")


# ------------------------------------------------------------ affine-packed layout

@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
def test_affine_pack_bit_exact(orc, dt, bits):
    N, K, gs = 24, 256, 64
    w = synth.normal((N, K), seed=bits, dt=dt)
    wq, s, b = orc.quantize(w, orc_code(orc, dt), gs, bits)
    wp_o, sbp_o = orc.affine_pack(wq, s, b, bits)
    wp, sbp = Q.affine_pack(bytes_to_words_dev(wq), to_dev(s, dt), to_dev(b, dt), gs, bits)
    torch.cuda.synchronize()
    assert np.array_equal(words_dev_to_bytes(wp), wp_o)
    assert np.array_equal(from_dev(sbp), sbp_o)


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("dt,M,N,K,gs", [
    ("f16", 1, 4096, 4096, 64),
    ("bf16", 1, 4096, 4096, 64),
    ("f16", 3, 72, 640, 32),       # 18 row blocks: a partial workgroup; few words per lane
    ("bf16", 2, 8, 16384, 128),    # the largest K of the interleaved-row GEMV
    ("f16", 5, 130, 1024, 64),     # 3/5/6 bits: rows of x in blocks of 4, N % 4 == 2
])
def test_qmv_affine_packed(orc, dt, M, N, K, gs, bits):
    if N % (4 if bits in (2, 4, 8) else 2):
        pytest.skip("the packed layout takes whole row blocks")
    code = orc_code(orc, dt)
    x = synth.normal((M, K), seed=M + N, dt=dt)
    w = synth.normal((N, K), seed=N + K, dt=dt)
    w[: min(N, 8)] = synth.structured_rows(min(N, 8), K, gs, seed=N, dt=dt)
    wq, s, b = orc.quantize(w, code, gs, bits)
    yo, _ = orc.qmm_t(x, wq, s, b, code, gs, bits, nthreads=8)
    wp, sbp = Q.affine_pack(bytes_to_words_dev(wq), to_dev(s, dt), to_dev(b, dt), gs, bits)
    y = Q.qmv_affine_packed(to_dev(x, dt), wp, sbp, N, gs, bits)
    torch.cuda.synchronize()
    assert_parity(from_dev(y), yo, dt, f"qmv_affine_packed {dt} M{M} N{N} K{K} b{bits}")


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("dt,M,N,K,gs", [
    ("f16", 64, 256, 512, 64),      # 32-row-free tiles, K split
    ("bf16", 100, 200, 1024, 32),   # ragged M; N % 128 == 72
    ("f16", 256, 384, 2080, 32),    # K % 64 == 32, split K
    ("bf16", 1024, 256, 1024, 128),
    ("f16", 20, 136, 4096, 64),     # 32-row tiles, K split
    ("f16", 2, 96, 640, 64),        # the GEMV
])
def test_qmm_t_affine_packed(orc, dt, M, N, K, gs, bits):
    """The product on the affine-packed layout for any M (the MFMA tile kernel
    reading the interleaved rows and packed scales beyond a few rows) against
    the oracle's qmm_t on the plain layout, with structured weight rows."""
    code = orc_code(orc, dt)
    x = synth.normal((M, K), seed=M + K, dt=dt)
    _, wq, s, b = _quantized(orc, dt, N, K, gs, bits, seed=N + bits, structured=True)
    yo, _ = orc.qmm_t(x, wq, s, b, code, gs, bits, nthreads=8)
    wp, sbp = Q.affine_pack(bytes_to_words_dev(wq), to_dev(s, dt), to_dev(b, dt), gs, bits)
    y = Q.qmm_t_affine_packed(to_dev(x, dt), wp, sbp, N, gs, bits)
    torch.cuda.synchronize()
    assert_parity(from_dev(y), yo, dt, f"qmm_t_affine_packed {dt} M{M} N{N} K{K} b{bits}")


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_chained_affine_packed_config(orc, bits):
    """The packed half of the chained bench: x f16 [1024,1024], W1 [4096,1024],
    W2 [1024,4096] in the affine-packed layout, first loop, sampled rows."""
    gs = 64
    x = synth.normal((1024, 1024), seed=0)
    _, wq1, s1, b1 = _quantized(orc, "f16", 4096, 1024, gs, bits, seed=1)
    _, wq2, s2, b2 = _quantized(orc, "f16", 1024, 4096, gs, bits, seed=2)
    p1 = Q.affine_pack(bytes_to_words_dev(wq1), to_dev(s1, "f16"), to_dev(b1, "f16"), gs, bits)
    p2 = Q.affine_pack(bytes_to_words_dev(wq2), to_dev(s2, "f16"), to_dev(b2, "f16"), gs, bits)
    h = Q.qmm_t_affine_packed(to_dev(x, "f16"), *p1, 4096, gs, bits)
    y = Q.qmm_t_affine_packed(h, *p2, 1024, gs, bits)
    torch.cuda.synchronize()
    hg, yg = from_dev(h), from_dev(y)
    for rows in [(0, 16), (1000, 1024)]:
        ho, _ = orc.qmm_t(x, wq1, s1, b1, orc.F16, gs, bits, nthreads=8, rows=rows)
        assert_parity(hg[rows[0]:rows[1]], ho, "f16", f"packed chained h bits{bits}")
        yo, _ = orc.qmm_t(hg, wq2, s2, b2, orc.F16, gs, bits, nthreads=8, rows=rows)
        assert_parity(yg[rows[0]:rows[1]], yo, "f16", f"packed chained y bits{bits}")


# ------------------------------------------------------------ batched weights

@pytest.mark.parametrize("dt,B,E,M,N,K,gs,bits", [
    ("f16", 3, 3, 1, 520, 1024, 64, 4),      # per-batch W, streaming GEMV (one launch)
    ("bf16", 4, 4, 2, 256, 512, 32, 3),      # per-batch W, bf16 streaming GEMV
    ("f16", 3, 3, 8, 512, 2048, 128, 5),     # per-batch W, MFMA GEMV per batch
    ("f16", 2, 2, 96, 384, 512, 64, 4),      # per-batch W, one tile launch (z = batch)
    ("bf16", 3, 3, 200, 256, 1024, 32, 8),   # per-batch W, ragged M tiles, 8-bit
    ("f16", 2, 2, 64, 512, 4096, 64, 4),     # per-batch W, tile kernel, K split 4 ways
    ("f16", 3, 3, 20, 256, 2048, 32, 3),     # 32-row tiles, K split, 3 batches
    ("bf16", 2, 2, 24, 320, 1024, 128, 6),   # bf16 32-row tiles, N % 128 = 64
    ("f16", 4, 1, 5, 256, 512, 64, 6),       # one W for every batch: 20 rows, tile kernel
    ("bf16", 3, 1, 1, 136, 768, 64, 2),      # one W for every batch: 3 rows, GEMV
])
def test_qmm_t_batched(orc, dt, B, E, M, N, K, gs, bits):
    code, x, wq, s, b = _gather_inputs(orc, dt, B, E, M, N, K, gs, bits, seed=M + N + E)
    yo, _ = orc.gather_qmm(x, wq, s, b, None, None if E == B else [0] * B, code, gs, bits,
                           nthreads=8)
    y = Q.qmm_t_batched(to_dev(x, dt), bytes_to_words_dev(wq), to_dev(s, dt), to_dev(b, dt),
                        gs, bits)
    torch.cuda.synchronize()
    assert tuple(y.shape) == yo.shape
    for z in range(B):
        assert_parity(from_dev(y[z]), yo[z], dt, f"qmm_t_batched batch {z}")


def test_qmm_t_batched_rejects_unaligned_batches():
    x = torch.zeros((2, 3, 64), dtype=torch.float16, device="cuda")
    wq = torch.zeros((2, 7, 8), dtype=torch.int32, device="cuda")
    s = torch.zeros((2, 7, 1), dtype=torch.float16, device="cuda")
    with pytest.raises(Q.QmmError) as e:        # y batches of 3 x 7 halves: 42 bytes
        Q.qmm_t_batched(x, wq, s, s, 64, 4)
    assert e.value.status == Q.QMM_E_ALIGN


# ------------------------------------------------------------ non-transposed GEMV

@pytest.mark.parametrize("dt,M,K,N,gs,bits", [
    ("f16", 1, 4096, 4096, 64, 4),
    ("bf16", 2, 640, 96, 32, 3),        # 3 chunks: a partial block of columns
    ("f16", 3, 30, 256, 128, 5),        # one K range (direct write), K % 4 != 0
    ("bf16", 1, 1000, 2112, 64, 6),     # 66 chunks: the second block holds 2
    ("f16", 4, 2048, 512, 32, 2),
    ("f16", 1, 11008, 4096, 64, 8),     # 344 K ranges
    ("bf16", 1, 4096, 4096, 128, 8),
    ("f16", 300, 2048, 8192, 64, 4),    # rows taken 128 at a time (workspace): 3 launches
    ("bf16", 150, 8192, 2048, 32, 3),   # 128 + 22 rows
])
def test_qmm_n(orc, dt, M, K, N, gs, bits):
    """y = x . dequant(W), W [K, N] quantized along N, against the oracle."""
    code = orc_code(orc, dt)
    x = synth.normal((M, K), seed=K + N, dt=dt)
    w = synth.normal((K, N), seed=K + N + 1, dt=dt)
    wq, s, b = orc.quantize(w, code, gs, bits)
    yo, _ = orc.qmm_n(x, wq, s, b, code, gs, bits, nthreads=8)
    y = Q.qmm_n(to_dev(x, dt), bytes_to_words_dev(wq), to_dev(s, dt), to_dev(b, dt), gs, bits)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (M, N)
    assert_parity(from_dev(y), yo, dt, f"qmm_n {M}x{K}x{N}")


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("dt,M,K,N,gs", [
    ("f16", 8, 256, 128, 32),       # the first M on the tile kernel
    ("bf16", 200, 1000, 160, 32),   # ragged M, K (a partial 64-row step) and N (a partial tile)
    ("f16", 130, 4096, 384, 128),
    ("bf16", 64, 512, 2048, 64),
])
def test_qmm_n_tile(orc, dt, M, K, N, gs, bits):
    """Many rows of x on the MFMA tile kernel for the non-transposed product,
    with structured weight rows."""
    code = orc_code(orc, dt)
    x = synth.normal((M, K), seed=M + K, dt=dt)
    w = synth.normal((K, N), seed=K + N + bits, dt=dt)
    w[:8] = synth.structured_rows(8, N, gs, seed=bits, dt=dt)
    wq, s, b = orc.quantize(w, code, gs, bits)
    yo, _ = orc.qmm_n(x, wq, s, b, code, gs, bits, nthreads=8)
    y = Q.qmm_n(to_dev(x, dt), bytes_to_words_dev(wq), to_dev(s, dt), to_dev(b, dt), gs, bits)
    torch.cuda.synchronize()
    assert_parity(from_dev(y), yo, dt, f"qmm_n tile {dt} {M}x{K}x{N} g{gs} b{bits}")


def test_qmm_n_tile_large(orc):
    """x f16 [1024, 2048] . dequant(W [2048, 2048] 4-bit g64 along N)."""
    x = synth.normal((1024, 2048), seed=3)
    w = synth.normal((2048, 2048), seed=4)
    wq, s, b = orc.quantize(w, orc.F16, 64, 4)
    yo, _ = orc.qmm_n(x, wq, s, b, orc.F16, 64, 4, nthreads=16)
    y = Q.qmm_n(to_dev(x, "f16"), bytes_to_words_dev(wq), to_dev(s, "f16"), to_dev(b, "f16"), 64, 4)
    torch.cuda.synchronize()
    assert_parity(from_dev(y), yo, "f16", "qmm_n tile 1024x2048x2048")


def test_qmm_n_repeat(orc):
    """Calls in a row reuse the split-K workspace: a larger then a smaller
    problem, both exact."""
    code = orc_code(orc, "f16")
    outs = []
    for (M, K, N, seed) in [(2, 4096, 2048, 1), (1, 1024, 512, 2)]:
        x = synth.normal((M, K), seed=seed, dt="f16")
        w = synth.normal((K, N), seed=seed + 1, dt="f16")
        wq, s, b = orc.quantize(w, code, 64, 4)
        yo, _ = orc.qmm_n(x, wq, s, b, code, 64, 4, nthreads=8)
        y = Q.qmm_n(to_dev(x, "f16"), bytes_to_words_dev(wq), to_dev(s, "f16"),
                    to_dev(b, "f16"), 64, 4)
        outs.append((y, yo, (M, K, N)))
    torch.cuda.synchronize()
    for y, yo, shape in outs:
        assert_parity(from_dev(y), yo, "f16", f"qmm_n repeat {shape}")
