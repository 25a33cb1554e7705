"""Pins for the oracle's floating-point modes (mxfp4, nvfp4, mxfp8; "mlx 1.0.0
backend/cpu/quantized.cpp": FP4_LUT, to_fp4_e2m1, to_fp8_e8m0,
dequantize_scale, fp_quantize_dequantize, fp_qmm_t).

* E2M1 encoding against a brute-force nearest-value search (ties to the even
  code, saturation at 6), on random values and on every midpoint;
* E4M3 decoding of all 256 bytes and encoding of random values and of every
  midpoint against torch's float8_e4m3fn (round to nearest even), and the
  saturation at 448;
* the e8m0 exponent against round(log2 x) in double precision, and closed forms
  around sqrt(2), at the clamps and for zero;
* quantization: groups built on the code grid come back exactly; on random data
  each code is the grid point nearest to w / scale (float64 search) and the
  scale byte follows the rule;
* the product (transposed and non-transposed) against a float64 matmul of the
  dequantized weights within the forward error bound, and pure-Python loops on
  tiny cases; one-hot rows of x pick rows of the dequantized weight exactly.
"""
import math

import numpy as np
import pytest
import torch

from group_wise_affine_amd import synth

U32 = 2.0 ** -24
GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
MODES = [("mxfp4", 4, 32), ("nvfp4", 4, 16), ("mxfp8", 8, 32)]


def _code(orc, dt):
    return {"f16": orc.F16, "bf16": orc.BF16, "f32": orc.F32}[dt]


def _e2m1_brute(x):
    """Nearest magnitude in GRID, ties to the even index, above 6 -> 6."""
    a = min(abs(x), 6.0)
    best = min(range(8), key=lambda i: (abs(a - GRID[i]), i % 2))
    return best | (8 if math.copysign(1.0, x) < 0 else 0)


def test_fp4_values(orc):
    assert [orc.fp4_value(c) for c in range(8)] == GRID
    assert [orc.fp4_value(c + 8) for c in range(8)] == [-v for v in GRID]


def test_fp4_encode_vs_brute_force(orc):
    rng = np.random.default_rng(0)
    xs = list(rng.uniform(-8, 8, 4000).astype(np.float32))
    mids = [(GRID[i] + GRID[i + 1]) / 2 for i in range(7)]
    for m in mids:
        for v in (m, np.nextafter(np.float32(m), np.float32(0)), np.nextafter(np.float32(m), np.float32(9))):
            xs += [np.float32(v), -np.float32(v)]
    xs += [np.float32(v) for v in (0.0, -0.0, 6.0, 7.9, 100.0, -1e30)]
    for x in xs:
        assert orc.fp4_encode(float(x)) == _e2m1_brute(float(x)), x


def test_e4m3_decode_all_bytes(orc):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    for b in range(256):
        v = orc.e4m3_value(b)
        if np.isnan(ref[b]):
            assert math.isnan(v), b
        else:
            assert v == ref[b], b


def test_e4m3_encode_vs_torch(orc):
    rng = np.random.default_rng(1)
    mags = np.exp2(rng.uniform(-12, math.log2(447.9), 6000)).astype(np.float32)
    xs = np.concatenate([mags, -mags[:3000]])
    vals = torch.arange(0, 0x7f, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)  # exact in f32
    xs = np.concatenate([xs, mids, -mids, np.array([0.0, -0.0, 2.0 ** -10, 2.0 ** -9 * 0.5],
                                                    np.float32)])
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.e4m3_encode(float(x)) for x in xs], np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(xs[i]), int(got[i]), int(ref[i])) for i in bad[:5]]


def test_e4m3_saturates(orc):
    for x in (448.0, 449.0, 463.9, 464.0, 480.0, 1e6, float("inf")):
        assert orc.e4m3_encode(x) == 0x7e
        assert orc.e4m3_encode(-x) == 0xfe
    assert orc.e4m3_value(0x7e) == 448.0


def test_e8m0_closed_forms(orc):
    for k in (-100, -20, -1, 0, 1, 7, 100):
        assert orc.e8m0_encode(2.0 ** k) == k + 127
        assert orc.e8m0_encode(2.0 ** k * 1.4142135) == k + 127      # just below sqrt 2
        assert orc.e8m0_encode(2.0 ** k * 1.4142137) == k + 128      # just above
    assert orc.e8m0_encode(0.0) == 0
    assert orc.e8m0_encode(1e-45) == 0           # 2^-149: clamped to -127
    assert orc.e8m0_encode(2.0 ** 127 * 1.9) == 254    # 128 clamped to 127
    assert orc.e8m0_encode(float("inf")) == 255


def test_e8m0_vs_log2(orc):
    rng = np.random.default_rng(2)
    xs = np.exp2(rng.uniform(-140, 127, 5000)).astype(np.float32)
    for x in xs:
        if x == 0:
            continue
        n = math.floor(math.log2(float(x)) + 0.5)
        n = min(max(n, -127), 127)
        assert orc.e8m0_encode(float(x)) == n + 127, x


@pytest.mark.parametrize("name,bits,gs", MODES)
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_fp_quantize_grid_roundtrip(orc, name, bits, gs, dt):
    """Groups made of code values times a representable scale come back exactly."""
    code = _code(orc, dt)
    rng = np.random.default_rng(3)
    rows, G = 4, 3
    K = G * gs
    w = np.zeros((rows, K), np.float32)
    if bits == 8:
        grid = torch.arange(0, 0x7f, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
        top = 448.0
    else:
        grid, top = np.array(GRID, np.float32), 6.0
    for r in range(rows):
        for g in range(G):
            # mx modes: power-of-two scales; nvfp4: E4M3 scales
            s = 2.0 ** int(rng.integers(-6, 4)) if gs == 32 else [0.625, 0.1875, 1.5, 3.25][(r + g) % 4]
            v = rng.choice(grid, gs) * rng.choice([-1.0, 1.0], gs)
            v[rng.integers(gs)] = top * rng.choice([-1.0, 1.0])
            w[r, g * gs:(g + 1) * gs] = v * s
    wt = synth.to_words(w, dt)
    assert np.array_equal(synth.words_to_f32(wt, dt), w)   # exact in T
    wq, sc = orc.fp_quantize(wt, code, gs, bits)
    w32, _ = orc.fp_dequantize(wq, sc, code, K, gs, bits)
    assert np.array_equal(w32, w)


@pytest.mark.parametrize("name,bits,gs", MODES)
def test_fp_quantize_nearest_code(orc, name, bits, gs):
    """Each code is the nearest grid point to w / scale (float64 search,
    saturating at the top code); the scale byte follows the rule."""
    dt = "f16"
    code = _code(orc, dt)
    rows, K = 6, 4 * gs
    wt = synth.normal((rows, K), seed=4, dt=dt)
    w = synth.words_to_f32(wt, dt).astype(np.float64)
    wq, sc = orc.fp_quantize(wt, code, gs, bits)
    if bits == 8:
        grid = torch.arange(0, 0x7f, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
        codes = wq.astype(np.int64)
        vals = torch.from_numpy(wq.copy()).view(torch.float8_e4m3fn).double().numpy()
    else:
        grid = np.array(GRID)
        lo, hi = wq & 15, wq >> 4
        codes = np.stack([lo, hi], -1).reshape(rows, K).astype(np.int64)
        vals = np.array([orc.fp4_value(c) for c in codes.ravel()]).reshape(rows, K)
    for r in range(rows):
        for g in range(K // gs):
            amax = np.max(np.abs(w[r, g * gs:(g + 1) * gs]))
            s_byte = int(sc[r, g])
            if gs == 32:
                s = 2.0 ** (s_byte - 127)
                ratio = (np.float32(amax) / np.float32(6.0 if bits == 4 else 448.0)) / s
                assert 2 ** -0.5 <= ratio <= 2 ** 0.5
            else:
                s = orc.e4m3_value(s_byte)
                assert s == torch.tensor([np.float32(amax) / np.float32(6.0)]).to(
                    torch.float8_e4m3fn).float().item()
            for k in range(g * gs, (g + 1) * gs):
                t = w[r, k] / s
                d = np.abs(np.abs(t) - grid)
                got = abs(vals[r, k])
                assert np.abs(np.abs(t) - got) <= d.min() + 1e-12 * max(1.0, abs(t)), (r, k)
                if t != 0:
                    assert math.copysign(1, vals[r, k]) == math.copysign(1, t)


@pytest.mark.parametrize("name,bits,gs", MODES)
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_fp_qmm_t_vs_float64(orc, name, bits, gs, dt):
    code = _code(orc, dt)
    M, N, K = 3, 40, 4 * gs + 64
    x = synth.normal((M, K), seed=5, dt=dt)
    w = synth.normal((N, K), seed=6, dt=dt)
    wq, sc = orc.fp_quantize(w, code, gs, bits)
    w32, _ = orc.fp_dequantize(wq, sc, code, K, gs, bits)
    y32, yt = orc.fp_qmm_t(x, wq, sc, code, gs, bits)
    xf = synth.words_to_f32(x, dt).astype(np.float64)
    wf = w32.astype(np.float64)
    ref = xf @ wf.T
    gamma = (K + 2) * U32 / (1 - (K + 2) * U32)
    assert np.all(np.abs(y32 - ref) <= gamma * (np.abs(xf) @ np.abs(wf).T))
    assert np.array_equal(yt, synth.to_words(y32, dt))


def test_fp_qmm_t_tiny_bruteforce(orc):
    M, N, K, gs, bits = 2, 3, 32, 16, 4
    x = synth.normal((M, K), seed=7, dt="f16")
    w = synth.normal((N, K), seed=8, dt="f16")
    wq, sc = orc.fp_quantize(w, orc.F16, gs, bits)
    y32, _ = orc.fp_qmm_t(x, wq, sc, orc.F16, gs, bits)
    xf = synth.words_to_f32(x, "f16")
    for m in range(M):
        for n in range(N):
            acc = mag = 0.0
            for k in range(K):
                byte = int(wq[n, k // 2])
                c = (byte >> 4) if k % 2 else (byte & 15)
                s = orc.e4m3_value(int(sc[n, k // gs]))
                v = GRID[c & 7] * (-1 if c & 8 else 1) * s
                acc += float(xf[m, k]) * v
                mag += abs(float(xf[m, k]) * v)
            assert abs(y32[m, n] - acc) <= (K + 2) * U32 * mag * 1.01 + 1e-30


# ---------------------------------------------------- the non-transposed product
# "mlx 1.0.0 backend/cpu/quantized.cpp", fp_qmm: W [K, N] quantized along N
# (one scale byte per group of N), y[m, n] = sum_k x[m, k] * scale * code value.

@pytest.mark.parametrize("name,bits,gs", MODES)
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_fp_qmm_n_vs_float64(orc, name, bits, gs, dt):
    """Against a float64 matmul of x and the dequantized [K, N] weight within
    the forward error bound (K != N: a transposed weight fails)."""
    code = _code(orc, dt)
    M, K, N = 3, 72, 4 * gs
    x = synth.normal((M, K), seed=15, dt=dt)
    w = synth.normal((K, N), seed=16, dt=dt)
    wq, sc = orc.fp_quantize(w, code, gs, bits)
    w32, _ = orc.fp_dequantize(wq, sc, code, N, gs, bits)
    y32, yt = orc.fp_qmm_n(x, wq, sc, code, gs, bits)
    xf = synth.words_to_f32(x, dt).astype(np.float64)
    wf = w32.astype(np.float64)
    ref = xf @ wf
    gamma = (K + 2) * U32 / (1 - (K + 2) * U32)
    assert np.all(np.abs(y32 - ref) <= gamma * (np.abs(xf) @ np.abs(wf)))
    assert np.array_equal(yt, synth.to_words(y32, dt))


@pytest.mark.parametrize("name,bits,gs", MODES)
def test_fp_qmm_n_one_hot_rows(orc, name, bits, gs):
    """x = e_k picks row k of the dequantized weight exactly."""
    K, N = 40, 2 * gs
    w = synth.normal((K, N), seed=17)
    wq, sc = orc.fp_quantize(w, orc.F16, gs, bits)
    w32, _ = orc.fp_dequantize(wq, sc, orc.F16, N, gs, bits)
    x = synth.to_words(np.eye(K, dtype=np.float32), "f16")
    y32, _ = orc.fp_qmm_n(x, wq, sc, orc.F16, gs, bits)
    assert np.array_equal(y32, w32)


def test_fp_qmm_n_tiny_bruteforce(orc):
    """mxfp4, pure-Python decoding of codes and e8m0 scales."""
    M, K, N, gs, bits = 2, 5, 64, 32, 4
    x = synth.normal((M, K), seed=18, dt="f16")
    w = synth.normal((K, N), seed=19, dt="f16")
    wq, sc = orc.fp_quantize(w, orc.F16, gs, bits)
    y32, _ = orc.fp_qmm_n(x, wq, sc, orc.F16, gs, bits)
    xf = synth.words_to_f32(x, "f16")
    for m in range(M):
        for n in range(N):
            acc = mag = 0.0
            for k in range(K):
                byte = int(wq[k, n // 2])
                c = (byte >> 4) if n % 2 else (byte & 15)
                b = int(sc[k, n // gs])
                s = 2.0 ** (b - 127) if b else 2.0 ** -127
                s = float(np.float64(s).astype(np.float16))   # the scale rounded to f16
                v = GRID[c & 7] * (-1 if c & 8 else 1) * s
                acc += float(xf[m, k]) * v
                mag += abs(float(xf[m, k]) * v)
            assert abs(y32[m, n] - acc) <= (K + 2) * U32 * mag * 1.01 + 1e-30


# ---------------------------------------------------- the scale as the product uses it
# "mlx 1.0.0 backend/cpu/quantized.cpp", dequantize_scale<T>: the decoded
# group scale is converted to the element type T before it multiplies the
# codes. Expected values come from numpy / torch casts of the exact scale.

E8M0_BYTES = [0, 1, 100, 101, 102, 103, 104, 112, 113, 127, 141, 142, 143, 144, 200, 254]


def _cast_scale(v, dt):
    """Exact scale (a Python float) rounded to T by numpy / torch, as float."""
    if dt == "f16":
        with np.errstate(over="ignore"):
            return float(np.float64(v).astype(np.float16))
    if dt == "bf16":
        return float(torch.tensor(v, dtype=torch.float64).to(torch.bfloat16).double())
    return float(np.float32(v))


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
def test_fp_scale_e8m0_rounded_to_t(orc, dt):
    """2^(s-127) rounded to T: f16 flushes bytes <= 102 to 0 (2^-25 ties to
    even, down to 0), keeps 2^-24 (byte 103) as a subnormal and overflows from
    byte 143 (2^16); bf16 and f32 hold every byte exactly."""
    for s in E8M0_BYTES:
        want = _cast_scale(math.ldexp(1.0, s - 127), dt)
        got = orc.fp_scale(s, 32, _code(orc, dt))
        assert got == want, (dt, s, got, want)
    if dt == "f16":
        assert orc.fp_scale(102, 32, orc.F16) == 0.0
        assert orc.fp_scale(103, 32, orc.F16) == 2.0 ** -24
        assert orc.fp_scale(142, 32, orc.F16) == 32768.0
        assert math.isinf(orc.fp_scale(143, 32, orc.F16))


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
def test_fp_scale_e4m3(orc, dt):
    """Group size 16 (nvfp4): the scale byte is an E4M3 value (torch's
    float8_e4m3fn), which f16, bf16 and f32 all hold exactly."""
    vals = torch.arange(128, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for s in range(127):          # 0x7f is NaN, outside the contract
        want = _cast_scale(float(vals[s]), dt)
        assert want == float(vals[s])
        assert orc.fp_scale(s, 16, _code(orc, dt)) == want, (dt, s)


def test_fp_dequantize_uses_rounded_scale(orc):
    """Dequantization with the E2M1 code for 1.0 returns the scale as T holds
    it: byte 102 gives 0 in f16 (2^-25 rounds to 0) but 2^-25 in bf16; byte 143
    gives inf in f16 and 65536 in bf16."""
    K, gs = 32, 32
    wq = np.full((2, K // 2), 0x22, np.uint8)         # every code 0b0010 = 1.0
    sc = np.array([[102], [143]], np.uint8)
    w16, _ = orc.fp_dequantize(wq, sc, orc.F16, K, gs, 4)
    wbf, _ = orc.fp_dequantize(wq, sc, orc.BF16, K, gs, 4)
    assert np.all(w16[0] == 0.0) and np.all(np.isinf(w16[1]))
    assert np.all(wbf[0] == 2.0 ** -25) and np.all(wbf[1] == 65536.0)
