"""No device allocation per call: the library's scratch (the split-K
workspace, the tile kernel's per-tile counters, the MFMA GEMV's partial tiles
and counters) is static device arrays, looked up once per device. Across
calls that use every one of them, the device's free memory does not change,
and calls in a row that reuse them (each case followed by a smaller one) stay
exact. Collected last: it runs after the other tests in one process, and
alone in a fresh one."""
import pytest
import torch

from group_wise_affine_amd import qmm as Q
from group_wise_affine_amd import synth
from tests.helpers import assert_parity, bytes_to_words_dev, from_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    Q.lib()


def _case(orc, fn, M, N, K, seed, gs=64, bits=4):
    """(launch, oracle y) for qmm_t (W [N, K]) or qmm_n (W [K, N]), f16."""
    x = synth.normal((M, K), seed=seed)
    if fn == "qmm_n":
        w = synth.normal((K, N), seed=seed + 1)
        wq, s, b = orc.quantize(w, orc.F16, gs, bits)
        yo, _ = orc.qmm_n(x, wq, s, b, orc.F16, gs, bits, nthreads=8)
    else:
        w = synth.normal((N, K), seed=seed + 1)
        wq, s, b = orc.quantize(w, orc.F16, gs, bits)
        yo, _ = orc.qmm_t(x, wq, s, b, orc.F16, gs, bits, nthreads=8)
    dev = (to_dev(x, "f16"), bytes_to_words_dev(wq), to_dev(s, "f16"), to_dev(b, "f16"))
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    f = getattr(Q, fn)
    return (lambda: f(*dev, gs, bits, out=y)), y, yo, (fn, M, N, K)


def test_calls_allocate_no_device_memory(orc):
    cases = [
        _case(orc, "qmm_t", 96, 256, 4096, 5),    # tile kernel, K split 4 ways
        _case(orc, "qmm_t", 40, 64, 2048, 6),     # smaller, K split 2 ways
        _case(orc, "qmm_t", 8, 512, 8192, 7),     # MFMA GEMV, K split 8 ways
        _case(orc, "qmm_t", 5, 96, 4160, 8),      # smaller, K split 2 ways
        _case(orc, "qmm_n", 2, 2048, 4096, 9),    # K ranges through the workspace
        _case(orc, "qmm_n", 1, 512, 1024, 10),    # smaller
        _case(orc, "qmm_n", 64, 256, 4096, 11),   # tile kernel, K split 8 ways
        _case(orc, "qmm_n", 16, 128, 2048, 12),   # smaller, K split 8 ways
    ]
    for launch, _, _, _ in cases:   # first calls: module load, scratch lookup
        launch()
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(2):
        for launch, _, _, _ in cases:
            launch()
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0, f"device free memory changed by {free0 - free1} bytes"
    for _, y, yo, what in cases:
        assert_parity(from_dev(y), yo, "f16", f"no-alloc {what}")
