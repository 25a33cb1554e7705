"""Pins for the oracle's gathered product (gather_qmm: output z is
x[lhs[z]] . dequant(W[rhs[z]])^T, "Add the 3bit packed qmm_t", ops.cpp).

* one-hot activations: every output element is then one dequantized weight
  (from the dequantizer, pinned in test_oracle_quantize.py) times 1, exactly,
  so an index applied to the wrong operand, a wrong batch stride or a
  transposed selection fails;
* each output batch against a float64 matmul of its selected batches, within
  the forward error bound of a length-K fp32 dot product;
* permuting the weight stack and remapping rhs leaves the output unchanged;
* absent index arrays mean the batch position; out-of-range indices raise.
"""
import numpy as np
import pytest

from group_wise_affine_amd import synth

U32 = 2.0 ** -24


def _stack(orc, dt, E, N, K, gs, bits, seed):
    code = {"f16": orc.F16, "bf16": orc.BF16, "f32": orc.F32}[dt]
    parts = [orc.quantize(synth.normal((N, K), seed=seed + e, dt=dt), code, gs, bits)
             for e in range(E)]
    wq = np.stack([p[0] for p in parts])
    s = np.stack([p[1] for p in parts])
    b = np.stack([p[2] for p in parts])
    return code, wq, s, b


def test_gather_one_hot_selects_weights(orc):
    Bx, E, M, N, K, gs, bits = 4, 4, 2, 8, 64, 32, 4
    code, wq, s, b = _stack(orc, "f16", E, N, K, gs, bits, seed=10)
    kpos = lambda bx, m: 7 * bx + 3 * m + 1  # distinct column per (batch, row)
    x = np.zeros((Bx, M, K), np.float32)
    for bx in range(Bx):
        for m in range(M):
            x[bx, m, kpos(bx, m)] = 1.0
    xw = synth.to_words(x, "f16")
    lhs, rhs = [2, 0, 1, 3, 1], [3, 3, 0, 1, 2]
    y32, _ = orc.gather_qmm(xw, wq, s, b, lhs, rhs, code, gs, bits)
    assert y32.shape == (5, M, N)
    for z in range(5):
        w32, _ = orc.dequantize(wq[rhs[z]], s[rhs[z]], b[rhs[z]], code, K, gs, bits)
        for m in range(M):
            assert np.array_equal(y32[z, m], w32[:, kpos(lhs[z], m)])


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_gather_vs_float64(orc, dt):
    Bx, E, M, N, K, gs, bits = 3, 5, 3, 16, 256, 64, 3
    code, wq, s, b = _stack(orc, dt, E, N, K, gs, bits, seed=20)
    x = np.stack([synth.normal((M, K), seed=30 + i, dt=dt) for i in range(Bx)])
    lhs, rhs = [1, 1, 0, 2, 2, 0], [4, 0, 0, 2, 3, 1]
    y32, yt = orc.gather_qmm(x, wq, s, b, lhs, rhs, code, gs, bits)
    gamma = K * U32 / (1 - K * U32)
    for z in range(len(lhs)):
        xf = synth.words_to_f32(x[lhs[z]], dt).astype(np.float64)
        w32, _ = orc.dequantize(wq[rhs[z]], s[rhs[z]], b[rhs[z]], code, K, gs, bits)
        wf = w32.astype(np.float64)
        ref = xf @ wf.T
        assert np.all(np.abs(y32[z] - ref) <= gamma * (np.abs(xf) @ np.abs(wf).T))
    assert np.array_equal(yt, synth.to_words(y32, dt))


def test_gather_expert_permutation_invariance(orc):
    Bx, E, M, N, K, gs, bits = 2, 6, 1, 12, 128, 32, 5
    code, wq, s, b = _stack(orc, "f16", E, N, K, gs, bits, seed=40)
    x = np.stack([synth.normal((M, K), seed=50 + i) for i in range(Bx)])
    lhs, rhs = [0, 1, 1, 0], [5, 2, 0, 5]
    y, _ = orc.gather_qmm(x, wq, s, b, lhs, rhs, code, gs, bits)
    perm = np.array([3, 5, 0, 1, 4, 2])           # new stack position i holds old perm[i]
    inv = np.argsort(perm)
    yp, _ = orc.gather_qmm(x, wq[perm], s[perm], b[perm], lhs, [int(inv[r]) for r in rhs],
                           code, gs, bits)
    assert np.array_equal(y, yp)
    assert np.array_equal(y[0], y[3])              # same index pair, same output


def test_gather_default_indices_and_range(orc):
    B, M, N, K, gs, bits = 3, 2, 8, 64, 64, 2
    code, wq, s, b = _stack(orc, "f16", B, N, K, gs, bits, seed=60)
    x = np.stack([synth.normal((M, K), seed=70 + i) for i in range(B)])
    y_none, _ = orc.gather_qmm(x, wq, s, b, None, None, code, gs, bits)
    y_id, _ = orc.gather_qmm(x, wq, s, b, [0, 1, 2], [0, 1, 2], code, gs, bits)
    assert np.array_equal(y_none, y_id)
    with pytest.raises(IndexError):
        orc.gather_qmm(x, wq, s, b, [0, 3], [0, 1], code, gs, bits)
    with pytest.raises(IndexError):
        orc.gather_qmm(x, wq, s, b, [0, 1], [-1, 1], code, gs, bits)
