"""Pins for the oracle's hand-written f16/bf16 converters against numpy's and
torch's casts (library routines), exhaustively over 16-bit patterns and on
round-to-nearest-even tie cases."""
import numpy as np
import pytest
import torch


def test_f16_to_f32_exhaustive(orc):
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.f16_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _f16_test_values():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = h.view(np.float16).astype(np.float64)
    fin = np.isfinite(f)
    f = np.sort(np.unique(f[fin]))
    mids = (f[:-1] + f[1:]) / 2  # exact ties in f64; exact in f32 too
    vals = [f, mids]
    m32 = mids.astype(np.float32)
    vals.append(np.nextafter(m32, np.float32(np.inf)).astype(np.float64))
    vals.append(np.nextafter(m32, np.float32(-np.inf)).astype(np.float64))
    vals.append(np.array([65504.0, 65519.99, 65520.0, 65536.0, 1e6, -65520.0,
                          2.0 ** -25, 2.0 ** -26, 3 * 2.0 ** -26, 1e-7, -1e-7,
                          1e-30, 0.0, -0.0]))
    rng = np.random.default_rng(1)
    vals.append(rng.standard_normal(200000) * 10.0 ** rng.uniform(-9, 5, 200000))
    return np.concatenate(vals).astype(np.float32)


def test_f32_to_f16_ties_and_random(orc):
    a = _f16_test_values()
    # the midpoints must survive the float32 cast exactly for the tie check
    got = orc.f32_to_f16(a)
    ref = a.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_f32_to_f16_nan_inf(orc):
    a = np.array([np.inf, -np.inf, np.nan], np.float32)
    got = orc.f32_to_f16(a)
    assert got[0] == 0x7C00 and got[1] == 0xFC00
    assert (got[2] & 0x7C00) == 0x7C00 and (got[2] & 0x3FF) != 0


def test_bf16_to_f32_exhaustive(orc):
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.bf16_to_f32(h)
    ref = torch.from_numpy(h.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f32_to_bf16_ties_and_random(orc):
    h = np.arange(1 << 16, dtype=np.uint32)
    base = (h << 16).view(np.float32)
    base = base[np.isfinite(base)]
    u = base.view(np.uint32)
    ties = (u + 0x8000).view(np.float32)  # exact halfway to the next bf16
    rng = np.random.default_rng(2)
    rnd = (rng.standard_normal(300000) * 10.0 ** rng.uniform(-30, 30, 300000)).astype(np.float32)
    a = np.concatenate([base, ties, rnd, (u + 0x7FFF).view(np.float32),
                        (u + 0x8001).view(np.float32)])
    a = a[np.isfinite(a)]
    got = orc.f32_to_bf16(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_synth_words_roundtrip(orc, dt):
    """The shared input generator's casts agree with the oracle's."""
    from group_wise_affine_amd import synth
    w = synth.normal((64, 64), seed=5, sigma=3.0, dt=dt)
    code = orc.F16 if dt == "f16" else orc.BF16
    f = orc.to_f32(w, code)
    assert np.array_equal(f.view(np.uint32), synth.words_to_f32(w, dt).view(np.uint32))
    assert np.array_equal(orc.from_f32(f, code), w)
