"""Pins for the oracle's affine-packed layout ("Add the 3bit packed qmm_t",
ops.cpp quantize, QuantizationType::AffinePacked): element-by-element index
maps written out with loops on small cases, for power-of-two and other widths."""
import numpy as np
import pytest

from group_wise_affine_amd import synth


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
def test_affine_pack_index_maps(orc, bits):
    N, K, gs = 8, 128, 32
    w = synth.normal((N, K), seed=bits, dt="f16")
    wq, s, b = orc.quantize(w, orc.F16, gs, bits)
    wp, sbp = orc.affine_pack(wq, s, b, bits)
    rp = 4 if bits in (2, 4, 8) else 2
    G = K // gs
    assert sbp.shape == (N // rp, G * 2 * rp)
    for i in range(N // rp):
        for g in range(G):
            for r in range(rp):
                assert sbp[i, g * 2 * rp + r] == s[i * rp + r, g]
                assert sbp[i, g * 2 * rp + rp + r] == b[i * rp + r, g]
    words = wq.view(np.uint32)
    if rp == 4:
        pw = wp.view(np.uint32)
        Kw = K * bits // 32
        assert pw.shape == (N // 4, Kw * 4)
        for i in range(N // 4):
            for wd in range(Kw):
                for r in range(4):
                    assert pw[i, wd * 4 + r] == words[i * 4 + r, wd]
    else:
        assert np.array_equal(wp, wq)


def test_affine_pack_rejects_ragged_rows(orc):
    wq = np.zeros((6, 16), np.uint8)
    s = np.zeros((6, 1), np.uint16)
    with pytest.raises(ValueError):
        orc.affine_pack(wq, s, s, 4)          # 6 rows, blocks of 4
    orc.affine_pack(wq, s, s, 3)              # blocks of 2: fine
