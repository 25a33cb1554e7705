"""CPU checks of the parity gate used by the GPU tests (tests/helpers.py):
it must accept an exact fp32 result rounded to T, and a result a few fp32
ulps away whose rounding flips at midpoints, and reject a relative
perturbation above what T can show (2e-3 for f16, 1e-2 for bf16) and a
single wrong element."""
import numpy as np
import pytest

from group_wise_affine_amd import synth
from tests.helpers import parity, REL_FRO, MAX_REL


def _y32(n=70, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(n) * 25).astype(np.float32)[None, :]


def _ok(rel, mrel):
    return rel <= REL_FRO and mrel <= MAX_REL


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_gate_accepts_exact_and_near_exact(dt):
    y = _y32()
    assert _ok(*parity(synth.to_words(y, dt), y, dt))
    # a few ulps of fp32 away: bf16/f16 roundings may flip at midpoints
    y2 = (y * np.float32(1 + 3e-7)).astype(np.float32)
    y2[0, 0] = np.float32(-101.24999)
    y[0, 0] = np.float32(-101.25001)
    assert _ok(*parity(synth.to_words(y2, dt), y, dt))


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_gate_rejects_perturbations(dt):
    y = _y32(n=4096)
    f = np.float32(1.002 if dt == "f16" else 1.01)
    assert not _ok(*parity(synth.to_words(y * f, dt), y, dt))
    bad = y.copy()
    bad[0, 7] += np.float32(0.05) * np.abs(y).max()
    assert not _ok(*parity(synth.to_words(bad, dt), y, dt))


def test_bf16_interval_contains_its_value():
    rng = np.random.default_rng(3)
    y = (rng.standard_normal(10000) * 10.0 ** rng.uniform(-3, 3, 10000)).astype(np.float32)
    y = np.concatenate([y, np.float32([0.0, -0.0, 1.0, -1.0, 2.0, 0.5])])
    w = synth.to_words(y, "bf16")
    from tests.helpers import _bf16_interval
    lo, hi = _bf16_interval(w)
    v = synth.words_to_f32(w, "bf16")
    assert np.all(lo <= v) and np.all(v <= hi)
    assert np.all(lo <= y) and np.all(y <= hi)  # RNE lands inside
