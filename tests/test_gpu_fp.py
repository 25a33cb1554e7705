"""GPU parity of the floating-point modes (mxfp4, nvfp4, mxfp8) against the
oracle ("mlx 1.0.0 backend/cpu/quantized.cpp": to_fp4_e2m1, to_fp8_e8m0,
dequantize_scale, fp_quantize_dequantize, fp_qmm_t, fp_qmm): quantize and
dequantize bit-exact, the GEMV, the any-M product (MFMA tile kernel) and the
non-transposed product within the floating-point gate."""
import numpy as np
import pytest
import torch

from group_wise_affine_amd import qmm as Q
from group_wise_affine_amd import synth
from tests.helpers import (assert_parity, bytes_to_words_dev, from_dev, orc_code, to_dev,
                           words_dev_to_bytes)

pytestmark = pytest.mark.gpu

MODES = [("mxfp4", 4, 32), ("nvfp4", 4, 16), ("mxfp8", 8, 32)]


def _weights(rows, K, gs, dt, seed, big=2.0 ** 8):
    """Normal rows, plus structured groups (zeros, constants, ramps, outliers,
    tiny values) and rows scaled far down (2^-12) and up (big)."""
    w = synth.normal((rows, K), seed=seed, sigma=2.0, dt=dt)
    n = min(rows, 12)
    w[:n] = synth.structured_rows(n, K, gs, seed=seed + 1, dt=dt)
    f = synth.words_to_f32(w, dt)
    if rows > n + 2:
        f[n] *= 2.0 ** -12      # tiny groups: small e8m0 / E4M3 scales, E4M3 subnormals
        f[n + 1] *= big         # large groups
    return synth.to_words(f, dt)


@pytest.mark.parametrize("name,bits,gs", MODES)
@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
def test_fp_quantize_bit_exact(orc, name, bits, gs, dt):
    rows, K = 33, gs * 6
    w = _weights(rows, K, gs, dt, seed=20 + bits + gs)
    wq_o, sc_o = orc.fp_quantize(w, orc_code(orc, dt), gs, bits)
    wq, sc = Q.fp_quantize(to_dev(w, dt), gs, bits)
    torch.cuda.synchronize()
    assert np.array_equal(words_dev_to_bytes(wq), wq_o)
    assert np.array_equal(sc.cpu().numpy(), sc_o)


@pytest.mark.parametrize("name,bits,gs", MODES)
def test_fp_quantize_large(orc, name, bits, gs):
    """A 4096 x 4096 f16 weight, bit-exact."""
    w = synth.normal((4096, 4096), seed=1)
    wq_o, sc_o = orc.fp_quantize(w, orc.F16, gs, bits)
    wq, sc = Q.fp_quantize(to_dev(w, "f16"), gs, bits)
    torch.cuda.synchronize()
    assert np.array_equal(words_dev_to_bytes(wq), wq_o)
    assert np.array_equal(sc.cpu().numpy(), sc_o)


@pytest.mark.parametrize("name,bits,gs", MODES)
@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
def test_fp_dequantize_bit_exact(orc, name, bits, gs, dt):
    """Every code value and a wide range of scale bytes (for f16, e8m0 scales
    below 2^-24 round to 0; bytes whose scale leaves f16 are left out, their
    zero codes would give NaN)."""
    rows, K = 24, gs * 8
    rng = np.random.default_rng(bits + gs)
    if bits == 4:
        wq = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    else:
        wq = rng.integers(0, 256, (rows, K), dtype=np.uint8)
        wq[(wq & 0x7f) == 0x7f] = 0x11                   # no NaN codes
    if gs == 16:
        sc = rng.integers(0, 256, (rows, K // gs), dtype=np.uint8)
        sc[(sc & 0x7f) == 0x7f] = 0x30
        sc &= 0x7f                                        # positive E4M3 scales
    else:
        top = 142 if dt == "f16" else 254
        sc = rng.integers(0, top + 1, (rows, K // gs), dtype=np.uint8)
        sc[0, :3] = [0, 102, 103]                          # 2^-127, 2^-25, 2^-24
    _, w_o = orc.fp_dequantize(wq, sc, orc_code(orc, dt), K, gs, bits)
    out = Q.fp_dequantize(bytes_to_words_dev(wq), torch.from_numpy(sc).cuda(), synth_dt(dt), gs,
                          bits)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(out), w_o)


def synth_dt(dt):
    return {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[dt]


@pytest.mark.parametrize("name,bits,gs", MODES)
@pytest.mark.parametrize("dt,M,N,K", [
    ("f16", 1, 4096, 4096),      # decode layer
    ("bf16", 1, 4096, 4096),
    ("f16", 4, 4096, 1024),      # 4 rows of W per wavefront, 8 wavefronts (4-bit)
    ("bf16", 2, 4096, 512),      # 4 rows of W per wavefront, 4 wavefronts (4-bit)
    ("f16", 3, 70, 1024),        # N % 16 != 0: a partial block of rows
    ("bf16", 2, 257, 96),        # 3 units of 32 codes: most lanes idle
    ("f16", 1, 64, 16384),       # the largest K (x in 64 KB of LDS)
    ("bf16", 5, 200, 2080),      # K % 64 == 32
])
def test_fp_qmv(orc, name, bits, gs, dt, M, N, K):
    code = orc_code(orc, dt)
    x = synth.normal((M, K), seed=M + K, dt=dt)
    w = _weights(N, K, gs, dt, seed=N + bits, big=16.0)   # keeps y within f16 at K = 16384
    wq, sc = orc.fp_quantize(w, code, gs, bits)
    yo, _ = orc.fp_qmm_t(x, wq, sc, code, gs, bits, nthreads=8)
    y = Q.fp_qmv(to_dev(x, dt), bytes_to_words_dev(wq), torch.from_numpy(sc).cuda(), gs, bits)
    torch.cuda.synchronize()
    assert_parity(from_dev(y), yo, dt, f"fp_qmv {name} {dt} M{M} N{N} K{K}")


@pytest.mark.parametrize("name,bits,gs", MODES)
@pytest.mark.parametrize("dt,M,N,K", [
    ("f16", 64, 256, 512),       # 64 rows: K split over 32-row-free tiles
    ("bf16", 256, 384, 1024),    # 128 x 128 tiles, split K
    ("f16", 1024, 512, 1024),    # 128 x 128 tiles, whole K
    ("bf16", 1024, 256, 2048),
    ("f16", 100, 200, 2080),     # ragged M and N, K % 64 == 32
    ("bf16", 20, 136, 4096),     # 32-row tiles, K split
    ("f16", 9, 64, 512),         # just above the GEMV's rows
    ("bf16", 3, 96, 640),        # the GEMV
])
def test_fp_qmm_t(orc, name, bits, gs, dt, M, N, K):
    """The fp-mode product for any M (the tile kernel beyond a few rows)
    against the oracle's fp_qmm_t, with structured groups and rows of small
    (2^-12) and large (x16) scales."""
    code = orc_code(orc, dt)
    x = synth.normal((M, K), seed=M + K + 1, dt=dt)
    w = _weights(N, K, gs, dt, seed=N + K + bits, big=16.0)
    wq, sc = orc.fp_quantize(w, code, gs, bits)
    yo, _ = orc.fp_qmm_t(x, wq, sc, code, gs, bits, nthreads=8)
    y = Q.fp_qmm_t(to_dev(x, dt), bytes_to_words_dev(wq), torch.from_numpy(sc).cuda(), gs, bits)
    torch.cuda.synchronize()
    assert_parity(from_dev(y), yo, dt, f"fp_qmm_t {name} {dt} M{M} N{N} K{K}")


@pytest.mark.parametrize("name,bits,gs", MODES)
@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("M,K,N", [
    (1, 64, 64),         # one row of x, one tile
    (37, 1000, 160),     # ragged M, K (a partial 64-row step) and N (a partial tile), K split
    (256, 4096, 384),    # K split 8 ways
    (300, 512, 2048),    # 48 tiles over 3 row blocks
])
def test_fp_qmm_n(orc, name, bits, gs, dt, M, K, N):
    """The non-transposed fp-mode product (W [K, N] quantized along N) on the
    tile kernel against the oracle's fp_qmm_n, with structured groups and rows
    of small (2^-12) and large (x16) scales."""
    code = orc_code(orc, dt)
    x = synth.normal((M, K), seed=M + K + 2, dt=dt)
    w = _weights(K, N, gs, dt, seed=N + K + bits + 1, big=16.0)
    wq, sc = orc.fp_quantize(w, code, gs, bits)
    yo, _ = orc.fp_qmm_n(x, wq, sc, code, gs, bits, nthreads=8)
    y = Q.fp_qmm_n(to_dev(x, dt), bytes_to_words_dev(wq), torch.from_numpy(sc).cuda(), gs, bits)
    torch.cuda.synchronize()
    assert_parity(from_dev(y), yo, dt, f"fp_qmm_n {name} {dt} M{M} K{K} N{N}")


@pytest.mark.parametrize("name,bits,gs", MODES)
def test_fp_qmm_t_full_size(orc, name, bits, gs):
    """x f16 [1024, 4096] . W [4096, 4096] quantized on the GPU, checked on
    sampled rows (the oracle recomputes rows 0..15 and 1000..1023)."""
    x = synth.normal((1024, 4096), seed=0)
    w = synth.normal((4096, 4096), seed=1)
    wq, sc = Q.fp_quantize(to_dev(w, "f16"), gs, bits)
    y = Q.fp_qmm_t(to_dev(x, "f16"), wq, sc, gs, bits)
    torch.cuda.synchronize()
    yg = from_dev(y)
    wq_o, sc_o = words_dev_to_bytes(wq), sc.cpu().numpy()
    for r0, r1 in [(0, 16), (1000, 1024)]:
        yo, _ = orc.fp_qmm_t(x[r0:r1], wq_o, sc_o, orc.F16, gs, bits, nthreads=8)
        assert_parity(yg[r0:r1], yo, "f16", f"fp_qmm_t {name} 1024x4096x4096 rows {r0}..{r1}")


@pytest.mark.parametrize("name,bits,gs", MODES)
def test_fp_qmm_t_routes_consistently(orc, name, bits, gs):
    """Around the GEMV / tile crossover both kernels (each forced, then the
    automatic choice) agree with the oracle."""
    dt, N, K = "f16", 96, 512
    w = _weights(N, K, gs, dt, seed=5, big=16.0)
    wq, sc = orc.fp_quantize(w, orc.F16, gs, bits)
    try:
        for M in (2, 3, 4, 5, 9, 33):
            x = synth.normal((M, K), seed=M, dt=dt)
            yo, _ = orc.fp_qmm_t(x, wq, sc, orc.F16, gs, bits, nthreads=8)
            for kern in (Q.KERNEL_GEMV, Q.KERNEL_TILE, Q.KERNEL_NONE):
                Q.force_kernel(kern)
                y = Q.fp_qmm_t(to_dev(x, dt), bytes_to_words_dev(wq), torch.from_numpy(sc).cuda(),
                               gs, bits)
                torch.cuda.synchronize()
                assert_parity(from_dev(y), yo, dt, f"fp_qmm_t {name} M{M} kernel {kern}")
    finally:
        Q.force_kernel(Q.KERNEL_NONE)


def _idx(v):
    return None if v is None else torch.tensor(v, dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("name,bits,gs", MODES)
@pytest.mark.parametrize("dt,Bx,E,M,N,K,lhs,rhs", [
    ("f16", 4, 8, 1, 512, 1024, [3, 0, 2, 2, 1, 0], [5, 1, 1, 0, 7, 6]),   # MoE decode routing
    ("bf16", 2, 2, 3, 70, 256, None, None),                               # identity, ragged N
    ("f16", 1, 3, 2, 4096, 2048, [0, 0, 0], [2, 0, 1]),                    # one token, 3 experts
])
def test_fp_gather_qmv(orc, name, bits, gs, dt, Bx, E, M, N, K, lhs, rhs):
    code = orc_code(orc, dt)
    x = np.stack([synth.normal((M, K), seed=30 + i, dt=dt) for i in range(Bx)])
    parts = [orc.fp_quantize(synth.normal((N, K), seed=40 + e, dt=dt), code, gs, bits)
             for e in range(E)]
    wq = np.stack([p[0] for p in parts])
    sc = np.stack([p[1] for p in parts])
    y = Q.fp_gather_qmv(to_dev(x, dt), bytes_to_words_dev(wq), torch.from_numpy(sc).cuda(),
                        _idx(lhs), _idx(rhs), gs, bits)
    torch.cuda.synchronize()
    B = len(lhs) if lhs is not None else (len(rhs) if rhs is not None else Bx)
    assert tuple(y.shape) == (B, M, N)
    yg = from_dev(y)
    for z in range(B):
        lz = lhs[z] if lhs is not None else z
        rz = rhs[z] if rhs is not None else z
        yo, _ = orc.fp_qmm_t(x[lz], wq[rz], sc[rz], code, gs, bits, nthreads=8)
        assert_parity(yg[z], yo, dt, f"fp_gather {name} batch {z}")


def test_fp_gather_max_batches(orc):
    """65535 products (the largest batch count), random routing, sampled."""
    dt, gs, bits, M, N, K, Bx, E, B = "f16", 32, 4, 1, 32, 64, 5, 6, 65535
    rng = np.random.default_rng(11)
    lhs = rng.integers(0, Bx, B).tolist()
    rhs = rng.integers(0, E, B).tolist()
    x = np.stack([synth.normal((M, K), seed=70 + i, dt=dt) for i in range(Bx)])
    parts = [orc.fp_quantize(synth.normal((N, K), seed=80 + e, dt=dt), orc.F16, gs, bits)
             for e in range(E)]
    wq = np.stack([p[0] for p in parts])
    sc = np.stack([p[1] for p in parts])
    y = Q.fp_gather_qmv(to_dev(x, dt), bytes_to_words_dev(wq), torch.from_numpy(sc).cuda(),
                        _idx(lhs), _idx(rhs), gs, bits)
    torch.cuda.synchronize()
    yg = from_dev(y)
    for z in list(range(0, B, 97)) + [B - 1]:
        yo, _ = orc.fp_qmm_t(x[lhs[z]], wq[rhs[z]], sc[rhs[z]], orc.F16, gs, bits)
        assert_parity(yg[z], yo, dt, f"fp_gather batch {z}")


def test_fp_gather_qmv_clamps_indices(orc):
    dt, gs, bits, M, N, K = "f16", 32, 4, 1, 96, 512
    x = np.stack([synth.normal((M, K), seed=50 + i, dt=dt) for i in range(2)])
    parts = [orc.fp_quantize(synth.normal((N, K), seed=60 + e, dt=dt), orc.F16, gs, bits)
             for e in range(3)]
    wq = np.stack([p[0] for p in parts])
    sc = np.stack([p[1] for p in parts])
    y = Q.fp_gather_qmv(to_dev(x, dt), bytes_to_words_dev(wq), torch.from_numpy(sc).cuda(),
                        _idx([-2, 1, 7]), _idx([5, 0, -1]), gs, bits)
    torch.cuda.synchronize()
    yg = from_dev(y)
    for z, (lz, rz) in enumerate([(0, 2), (1, 0), (1, 0)]):
        yo, _ = orc.fp_qmm_t(x[lz], wq[rz], sc[rz], orc.F16, gs, bits)
        assert_parity(yg[z], yo, dt, f"fp_gather clamped {z}")


def test_fp_quantize_then_qmv_end_to_end(orc):
    """Quantize on the GPU, multiply on the GPU, compare with the oracle's
    product over the oracle's codes (identical by the bit-exact quantizer)."""
    dt, M, N, K, gs, bits = "f16", 2, 512, 2048, 32, 4
    x = synth.normal((M, K), seed=3, dt=dt)
    w = synth.normal((N, K), seed=4, dt=dt)
    wq, sc = Q.fp_quantize(to_dev(w, dt), gs, bits)
    y = Q.fp_qmv(to_dev(x, dt), wq, sc, gs, bits)
    wq_o, sc_o = orc.fp_quantize(w, orc.F16, gs, bits)
    yo, _ = orc.fp_qmm_t(x, wq_o, sc_o, orc.F16, gs, bits, nthreads=8)
    torch.cuda.synchronize()
    assert_parity(from_dev(y), yo, dt, "fp quantize + qmv")


def test_fp_rejects_bad_arguments():
    x = torch.zeros((1, 64), dtype=torch.float16, device="cuda")
    wq = torch.zeros((8, 8), dtype=torch.int32, device="cuda")
    sc = torch.zeros((8, 2), dtype=torch.uint8, device="cuda")
    with pytest.raises(Q.QmmError) as e:          # nvfp4 takes bits 4 only
        Q.fp_qmv(x, torch.zeros((8, 16), dtype=torch.int32, device="cuda"), sc, 16, 8)
    assert e.value.status == Q.QMM_E_GROUP
    with pytest.raises(Q.QmmError) as e:          # K beyond the LDS-staged row
        big = torch.zeros((1, 32768), dtype=torch.float16, device="cuda")
        Q.fp_qmv(big, torch.zeros((8, 4096), dtype=torch.int32, device="cuda"),
                 torch.zeros((8, 1024), dtype=torch.uint8, device="cuda"), 32, 4)
    assert e.value.status == Q.QMM_E_SHAPE
    with pytest.raises(Q.QmmError) as e:
        Q.fp_qmv(x, wq, sc, 32, 3)
    assert e.value.status == Q.QMM_E_BITS
