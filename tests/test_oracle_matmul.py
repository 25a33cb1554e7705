"""Pins for the oracle's qmm_t and qconv2d.

* qmm_t against a float64 matmul (numpy, a library routine) of the widened
  activations and the oracle's dequantized weights (pinned separately in
  test_oracle_quantize.py), within the classical forward error bound of a
  length-K fp32 dot product, |err| <= gamma_K * sum |x| |w|;
* qmm_t row subsets equal the full product;
* qconv2d against torch.nn.functional.conv2d in float64 on the dequantized
  weight (the conv issue's claim that im2col + matmul reproduces a direct
  convolution), for strides, paddings and groups;
* a 1x1, stride-1, pad-0 conv is exactly qmm_t on the [B*H*W, C] view;
* groups=G equals G independent convolutions on channel slices.
"""
import numpy as np
import pytest
import torch

from group_wise_affine_amd import synth

U32 = 2.0 ** -24


def _gamma(K):
    return K * U32 / (1 - K * U32)


def _code(orc, dt):
    return {"f16": orc.F16, "bf16": orc.BF16, "f32": orc.F32}[dt]


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("gs", [32, 64, 128])
@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
def test_qmm_t_vs_float64(orc, bits, gs, dt):
    M, N, K = 5, 24, 256
    code = _code(orc, dt)
    x = synth.normal((M, K), seed=1, dt=dt)
    w = synth.normal((N, K), seed=2, dt=dt)
    wq, s, b = orc.quantize(w, code, gs, bits)
    w32, _ = orc.dequantize(wq, s, b, code, K, gs, bits)
    y32, yt = orc.qmm_t(x, wq, s, b, code, gs, bits)
    xf = synth.words_to_f32(x, dt).astype(np.float64)
    wf = w32.astype(np.float64)
    ref = xf @ wf.T
    bound = _gamma(K) * (np.abs(xf) @ np.abs(wf).T)
    assert np.all(np.abs(y32 - ref) <= bound)
    assert np.array_equal(yt, synth.to_words(y32, dt))


def test_qmm_t_planted_error_is_caught(orc):
    """Sanity of the bound itself: a one-ulp-of-a-weight perturbation of the
    dequantized weights moves the float64 reference outside it somewhere."""
    M, N, K = 4, 16, 256
    x = synth.normal((M, K), seed=1, dt="f32")
    w = synth.normal((N, K), seed=2, dt="f32")
    wq, s, b = orc.quantize(w, orc.F32, 64, 4)
    w32, _ = orc.dequantize(wq, s, b, orc.F32, K, 64, 4)
    y32, _ = orc.qmm_t(x, wq, s, b, orc.F32, 64, 4)
    wf = w32.astype(np.float64)
    wf[3, 17] += 0.01  # a dropped/perturbed term
    ref = x.astype(np.float64) @ wf.T
    bound = _gamma(K) * (np.abs(x.astype(np.float64)) @ np.abs(wf).T)
    assert np.any(np.abs(y32 - ref) > bound)


def test_qmm_t_row_subset(orc):
    M, N, K = 9, 40, 512
    x = synth.normal((M, K), seed=3)
    w = synth.normal((N, K), seed=4)
    wq, s, b = orc.quantize(w, orc.F16, 64, 4)
    y_all, t_all = orc.qmm_t(x, wq, s, b, orc.F16, 64, 4)
    y_sub, t_sub = orc.qmm_t(x, wq, s, b, orc.F16, 64, 4, rows=(3, 7))
    assert np.array_equal(y_all[3:7], y_sub) and np.array_equal(t_all[3:7], t_sub)
    y_mt, _ = orc.qmm_t(x, wq, s, b, orc.F16, 64, 4, nthreads=4)
    assert np.array_equal(y_mt, y_all)


def test_qmm_t_tiny_bruteforce(orc):
    """Pure-Python loops over codes, scales and biases on a 2x3x32 case."""
    M, N, K, gs, bits = 2, 3, 32, 32, 3
    x = synth.normal((M, K), seed=8, dt="f32")
    w = synth.normal((N, K), seed=9, dt="f32")
    wq, s, b = orc.quantize(w, orc.F32, gs, bits)
    q = orc.unpack(wq, K, bits)
    y32, _ = orc.qmm_t(x, wq, s, b, orc.F32, gs, bits)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            mag = 0.0
            for k in range(K):
                wv = float(s[n, k // gs]) * int(q[n, k]) + float(b[n, k // gs])
                acc += float(x[m, k]) * wv
                mag += abs(float(x[m, k]) * wv)
            assert abs(y32[m, n] - acc) <= _gamma(K) * mag + 2 * U32 * mag


def _conv_ref_f64(xw, dt, w32_rows, O, kh, kw, Cg, stride, pad, groups, K_true):
    xf = torch.from_numpy(synth.words_to_f32(xw, dt).astype(np.float64))
    xf = xf.permute(0, 3, 1, 2)  # NCHW
    wt = torch.from_numpy(w32_rows[:, :K_true].astype(np.float64))
    wt = wt.reshape(O, kh, kw, Cg).permute(0, 3, 1, 2).contiguous()  # OIHW
    y = torch.nn.functional.conv2d(xf, wt, stride=stride, padding=pad, groups=groups)
    ya = torch.nn.functional.conv2d(xf.abs(), wt.abs(), stride=stride, padding=pad,
                                    groups=groups)
    return y.permute(0, 2, 3, 1).numpy(), ya.permute(0, 2, 3, 1).numpy()


CONV_CASES = [
    # B, H, W, C, O, kh, kw, stride, pad, groups, gs, bits
    (1, 9, 7, 16, 24, 3, 3, (1, 1), (1, 1), 1, 32, 4),
    (2, 8, 8, 12, 8, 3, 3, (2, 1), (1, 0), 2, 32, 4),
    (1, 10, 6, 8, 6, 5, 3, (1, 2), (2, 1), 1, 64, 3),
    (1, 6, 6, 32, 16, 1, 1, (1, 1), (0, 0), 1, 32, 8),
    (1, 7, 5, 20, 10, 3, 2, (1, 1), (0, 1), 5, 32, 6),
    (1, 5, 5, 24, 12, 3, 3, (1, 1), (1, 1), 3, 128, 5),
]


@pytest.mark.parametrize("case", CONV_CASES)
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_qconv2d_vs_torch_float64(orc, case, dt):
    B, H, W, C, O, kh, kw, stride, pad, groups, gs, bits = case
    code = _code(orc, dt)
    Cg = C // groups
    x = synth.normal((B, H, W, C), seed=12, dt=dt)
    wconv = synth.normal((O, kh, kw, Cg), seed=13, sigma=0.5, dt=dt)
    wmat = orc.conv_weight_matrix(wconv, groups, gs)
    K_true, K_pad = kh * kw * Cg, wmat.shape[1]
    assert K_pad % gs == 0 and K_pad - K_true < gs
    wq, s, b = orc.quantize(wmat, code, gs, bits)
    w32, _ = orc.dequantize(wq, s, b, code, K_pad, gs, bits)
    y32, yt = orc.qconv2d_nhwc(x, wq, s, b, code, O, kh, kw, stride, pad, groups, gs, bits)
    ref, mag = _conv_ref_f64(x, dt, w32, O, kh, kw, Cg, stride, pad, groups, K_true)
    assert y32.shape == ref.shape
    assert np.all(np.abs(y32 - ref) <= _gamma(K_true) * mag)
    assert np.array_equal(yt, synth.to_words(y32, dt))


def test_qconv2d_1x1_is_qmm_t(orc):
    B, H, W, C, O = 2, 5, 6, 64, 24
    x = synth.normal((B, H, W, C), seed=14)
    wconv = synth.normal((O, 1, 1, C), seed=15)
    wmat = orc.conv_weight_matrix(wconv, 1, 64)
    wq, s, b = orc.quantize(wmat, orc.F16, 64, 4)
    y32, _ = orc.qconv2d_nhwc(x, wq, s, b, orc.F16, O, 1, 1, (1, 1), (0, 0), 1, 64, 4)
    ym, _ = orc.qmm_t(x.reshape(B * H * W, C), wq, s, b, orc.F16, 64, 4)
    assert np.array_equal(y32.reshape(B * H * W, O), ym)


def test_qconv2d_groups_are_independent_convs(orc):
    B, H, W, C, O, G, gs = 1, 6, 5, 16, 12, 2, 32
    x = synth.normal((B, H, W, C), seed=16)
    wconv = synth.normal((O, 3, 3, C // G), seed=17)
    wmat = orc.conv_weight_matrix(wconv, G, gs)
    wq, s, b = orc.quantize(wmat, orc.F16, gs, 4)
    y32, _ = orc.qconv2d_nhwc(x, wq, s, b, orc.F16, O, 3, 3, (1, 1), (1, 1), G, gs, 4)
    Og, Cg = O // G, C // G
    for g in range(G):
        xg = np.ascontiguousarray(x[..., g * Cg:(g + 1) * Cg])
        rs = slice(g * Og, (g + 1) * Og)
        yg, _ = orc.qconv2d_nhwc(xg, wq[rs], s[rs], b[rs], orc.F16, Og, 3, 3, (1, 1),
                                 (1, 1), 1, gs, 4)
        assert np.array_equal(yg, y32[..., rs])
