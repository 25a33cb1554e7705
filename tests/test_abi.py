"""CPU checks of the C ABI: the library loads, exports every function that
include/libqmm.h declares, and rejects each kind of bad argument with the
documented status before anything is launched (no valid call is made here,
so no GPU is needed). The rejected cases follow the argument errors of the
mlx ops on the pages (bits / group size / dtype switches, K a multiple of
the group size, conv geometry)."""
import ctypes
import os
import re
import subprocess

import pytest

from group_wise_affine_amd import qmm as Q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libqmm.h")

# aligned, non-NULL placeholders: validation never dereferences pointers
P = ctypes.c_void_p(0x10000)
P2 = ctypes.c_void_p(0x10002)  # 2-byte but not 16-byte aligned


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(Q.LIB_PATH):
        from group_wise_affine_amd import build
        build.build()
    return Q.lib()


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert set(names) == set(Q.EXPORTS), names
    out = subprocess.run(["nm", "-D", "--defined-only", Q.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for n in names:
        assert n in exported, n
        assert hasattr(L, n)


def _st(L, fn, *args):
    return getattr(L, fn)(*args)


BAD_BITS = [1, 7, 9, 16, 0, -4]
BAD_GS = [16, 48, 256, 0, -64]


@pytest.mark.parametrize("bits", BAD_BITS)
def test_bad_bits(L, bits):
    assert _st(L, "qmm_quantize", P, 0, 4, 64, 64, bits, P, P, P, None) == Q.QMM_E_BITS
    assert _st(L, "qmm_dequantize", P, P, P, 0, 4, 64, 64, bits, P, None) == Q.QMM_E_BITS
    for fn in ("qmm_t", "qmv"):
        assert _st(L, fn, P, P, P, P, 0, 1, 8, 64, 64, bits, P, None) == Q.QMM_E_BITS
    assert _st(L, "qconv2d_nhwc", P, 1, 8, 8, 8, P, P, P, 8, 3, 3, 1, 1, 1, 1, 1,
               0, 64, bits, P, None) == Q.QMM_E_BITS
    assert b"bits" in L.qmm_last_error()


@pytest.mark.parametrize("gs", BAD_GS)
def test_bad_group_size(L, gs):
    assert _st(L, "qmm_quantize", P, 0, 4, 256, gs, 4, P, P, P, None) == Q.QMM_E_GROUP
    assert _st(L, "qmm_dequantize", P, P, P, 1, 4, 256, gs, 4, P, None) == Q.QMM_E_GROUP
    for fn in ("qmm_t", "qmv"):
        assert _st(L, fn, P, P, P, P, 0, 1, 8, 256, gs, 4, P, None) == Q.QMM_E_GROUP
    assert b"group_size" in L.qmm_last_error()


def test_null_pointers(L):
    for i in range(4):
        args = [P, P, P, P]
        args[i] = None
        st = _st(L, "qmm_quantize", args[0], 0, 4, 64, 64, 4, args[1], args[2], args[3], None)
        assert st == Q.QMM_E_NULL
    for fn in ("qmm_t", "qmv"):
        for i in range(5):
            a = [P, P, P, P, P]
            a[i] = None
            assert _st(L, fn, a[0], a[1], a[2], a[3], 0, 1, 8, 64, 64, 4, a[4], None) == Q.QMM_E_NULL
    assert _st(L, "qmm_dequantize", None, P, P, 0, 4, 64, 64, 4, P, None) == Q.QMM_E_NULL
    assert _st(L, "qconv2d_nhwc", None, 1, 8, 8, 8, P, P, P, 8, 3, 3, 1, 1, 1, 1, 1,
               0, 64, 4, P, None) == Q.QMM_E_NULL


@pytest.mark.parametrize("K", [0, -64, 96, 100, 65])
def test_k_not_multiple_of_group(L, K):
    assert _st(L, "qmm_quantize", P, 0, 4, K, 64, 4, P, P, P, None) == Q.QMM_E_SHAPE
    assert _st(L, "qmm_dequantize", P, P, P, 0, 4, K, 64, 4, P, None) == Q.QMM_E_SHAPE
    for fn in ("qmm_t", "qmv"):
        assert _st(L, fn, P, P, P, P, 0, 2, 8, K, 64, 4, P, None) == Q.QMM_E_SHAPE


def test_bad_sizes(L):
    for fn in ("qmm_t", "qmv"):
        assert _st(L, fn, P, P, P, P, 0, 0, 8, 64, 64, 4, P, None) == Q.QMM_E_SHAPE
        assert _st(L, fn, P, P, P, P, 0, 4, 0, 64, 64, 4, P, None) == Q.QMM_E_SHAPE
        assert _st(L, fn, P, P, P, P, 0, -1, 8, 64, 64, 4, P, None) == Q.QMM_E_SHAPE
    assert _st(L, "qmm_quantize", P, 0, 0, 64, 64, 4, P, P, P, None) == Q.QMM_E_SHAPE
    # the streaming kernel's K limit is reported, qmm_t is not limited by it
    assert _st(L, "qmv", P, P, P, P, 0, 1, 8, 1 << 20, 64, 4, P, None) == Q.QMM_E_SHAPE
    assert b"K" in L.qmm_last_error()
    # the tile kernel keeps lane offsets inside a tile in 32 bits: K < 2^24
    assert _st(L, "qmm_t", P, P, P, P, 0, 64, 8, 1 << 24, 64, 4, P, None) == Q.QMM_E_SHAPE
    assert b"K" in L.qmm_last_error()


def test_bad_dtype(L):
    for fn in ("qmm_t", "qmv"):
        assert _st(L, fn, P, P, P, P, 2, 1, 8, 64, 64, 4, P, None) == Q.QMM_E_DTYPE
        assert _st(L, fn, P, P, P, P, 7, 1, 8, 64, 64, 4, P, None) == Q.QMM_E_DTYPE
    assert _st(L, "qmm_quantize", P, 3, 4, 64, 64, 4, P, P, P, None) == Q.QMM_E_DTYPE
    assert _st(L, "qmm_dequantize", P, P, P, -1, 4, 64, 64, 4, P, None) == Q.QMM_E_DTYPE
    assert _st(L, "qconv2d_nhwc", P, 1, 8, 8, 8, P, P, P, 8, 3, 3, 1, 1, 1, 1, 1,
               2, 64, 4, P, None) == Q.QMM_E_DTYPE


def test_alignment(L):
    for fn in ("qmm_t", "qmv"):
        assert _st(L, fn, P2, P, P, P, 0, 1, 8, 64, 64, 4, P, None) == Q.QMM_E_ALIGN
        assert _st(L, fn, P, P2, P, P, 0, 1, 8, 64, 64, 4, P, None) == Q.QMM_E_ALIGN
        assert _st(L, fn, P, P, P, P, 0, 1, 8, 64, 64, 4, P2, None) == Q.QMM_E_ALIGN
        odd = ctypes.c_void_p(0x10001)
        assert _st(L, fn, P, P, odd, P, 0, 1, 8, 64, 64, 4, P, None) == Q.QMM_E_ALIGN
    assert _st(L, "qmm_quantize", P2, 0, 4, 64, 64, 4, P, P, P, None) == Q.QMM_E_ALIGN
    assert _st(L, "qmm_quantize", P, 2, 4, 64, 64, 4, P, P2, P, None) == Q.QMM_E_ALIGN


def test_conv_geometry(L):
    def conv(B=1, H=8, W=8, C=8, O=8, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, g=1):
        return _st(L, "qconv2d_nhwc", P, B, H, W, C, P, P, P, O, kh, kw, sh, sw, ph, pw,
                   g, 0, 64, 4, P, None)
    assert conv(C=9, g=2) == Q.QMM_E_SHAPE
    assert conv(O=9, g=2) == Q.QMM_E_SHAPE
    assert conv(kh=11, ph=1) == Q.QMM_E_SHAPE  # kernel larger than padded input
    assert conv(sh=0) == Q.QMM_E_SHAPE
    assert conv(ph=-1) == Q.QMM_E_SHAPE
    assert conv(g=0) == Q.QMM_E_SHAPE
    assert conv(B=0) == Q.QMM_E_SHAPE


SHAPES = [(4096, 4096), (2048, 8192), (8192, 2048), (512, 2048), (4096, 11008), (64, 16384),
          (4096, 32768)]


def test_route_is_a_step_function_of_m(L):
    """Host-only routing: for a fixed layer, qmm_t runs GEMV kernels up to
    some M and the tile kernel from there on; qmm_crossover_m reports that M."""
    for dt in (0, 1):
        for bits in (2, 3, 4, 5, 6, 8):
            for gs in (32, 64, 128):
                for (N, K) in SHAPES:
                    rs = [L.qmm_route(dt, bits, gs, M, N, K) for M in range(1, 129)]
                    assert all(r in (Q.KERNEL_GEMV, Q.KERNEL_MFMA_GEMV, Q.KERNEL_TILE) for r in rs)
                    first = rs.index(Q.KERNEL_TILE) + 1 if Q.KERNEL_TILE in rs else None
                    assert first is not None, (dt, bits, gs, N, K)
                    assert all(r == Q.KERNEL_TILE for r in rs[first - 1:]), (dt, bits, gs, N, K)
                    assert L.qmm_crossover_m(dt, bits, gs, N, K) == first
                    # the MFMA GEMV never takes more than 32 rows
                    assert all(r != Q.KERNEL_MFMA_GEMV for r in rs[32:])


def test_route_rejects_invalid_arguments(L):
    assert L.qmm_route(0, 7, 64, 1, 64, 64) == Q.KERNEL_NONE
    assert L.qmm_route(0, 4, 48, 1, 64, 96) == Q.KERNEL_NONE
    assert L.qmm_route(2, 4, 64, 1, 64, 64) == Q.KERNEL_NONE   # f32 products do not exist
    assert L.qmm_route(0, 4, 64, 0, 64, 64) == Q.KERNEL_NONE
    assert L.qmm_route(0, 4, 64, 1, 64, 96) == Q.KERNEL_NONE   # K % group_size
    assert L.qmm_crossover_m(0, 7, 64, 64, 64) == 0


def test_force_kernel(L):
    try:
        assert L.qmm_force_kernel(4) == Q.QMM_E_ARG
        assert L.qmm_force_kernel(-1) == Q.QMM_E_ARG
        assert L.qmm_force_kernel(Q.KERNEL_TILE) == Q.QMM_OK
        assert L.qmm_route(0, 4, 64, 1, 4096, 4096) == Q.KERNEL_TILE
        assert L.qmm_force_kernel(Q.KERNEL_MFMA_GEMV) == Q.QMM_OK
        assert L.qmm_route(0, 4, 64, 1, 4096, 4096) == Q.KERNEL_MFMA_GEMV
        assert L.qmm_route(0, 4, 64, 33, 4096, 4096) == Q.KERNEL_TILE   # does not fit: automatic
        assert L.qmm_force_kernel(Q.KERNEL_GEMV) == Q.QMM_OK
        assert L.qmm_route(0, 4, 64, 64, 4096, 4096) == Q.KERNEL_GEMV
    finally:
        assert L.qmm_force_kernel(Q.KERNEL_NONE) == Q.QMM_OK
    assert L.qmm_route(0, 4, 64, 64, 4096, 4096) == Q.KERNEL_TILE


def test_route_measured_switch_points(L):
    """Host-only: switch points that the committed route table (kernel-only
    times of the three kernels forced at M = 1..32) fixes."""
    G, M_, T = Q.KERNEL_GEMV, Q.KERNEL_MFMA_GEMV, Q.KERNEL_TILE
    # f16 4096 x 4096 4-bit: streaming GEMV at M = 1, MFMA GEMV 2..16, tile from 24
    assert [L.qmm_route(0, 4, 64, M, 4096, 4096) for M in (1, 2, 16, 24)] == [G, M_, M_, T]
    # bf16 with 8-bit codes: the streaming GEMV keeps M = 1 where it runs its
    # 2-chunk lane shape (4096 x 4096), not where it does not (rows of 8192
    # codes need two batches of 2 chunks per lane)
    assert L.qmm_route(1, 8, 64, 1, 4096, 4096) == G
    assert L.qmm_route(1, 8, 64, 2, 4096, 4096) == M_
    assert L.qmm_route(1, 8, 64, 1, 2048, 8192) == M_
    # bf16 layers of at most 2^20 weights: streaming GEMV above 8 rows
    assert [L.qmm_route(1, 4, 64, M, 512, 2048) for M in (1, 4, 8, 12, 32)] == [G, M_, M_, G, G]
    assert [L.qmm_route(1, 4, 64, M, 2048, 2048) for M in (2, 3, 12, 32)] == [G, M_, M_, M_]


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(Q, "_lib", None)
    monkeypatch.setattr(Q, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        Q.lib()


def test_gather_arguments(L):
    def g(x=P, nxb=2, li=None, wq=P, s=P, b=P, nwb=3, ri=None, B=2, dt=0, M=1, N=8, K=64,
          gs=64, bits=4, y=P):
        return _st(L, "qmm_gather_qmv", x, nxb, li, wq, s, b, nwb, ri, B, dt, M, N, K, gs,
                   bits, y, None)
    assert g(x=None) == Q.QMM_E_NULL
    assert g(y=None) == Q.QMM_E_NULL
    assert g(bits=7) == Q.QMM_E_BITS
    assert g(gs=16) == Q.QMM_E_GROUP
    assert g(dt=2) == Q.QMM_E_DTYPE
    assert g(B=0) == Q.QMM_E_SHAPE
    assert g(B=65536, li=P, ri=P) == Q.QMM_E_SHAPE
    assert g(nxb=0) == Q.QMM_E_SHAPE
    assert g(nwb=0, ri=P) == Q.QMM_E_SHAPE
    assert g(nxb=1) == Q.QMM_E_SHAPE          # no lhs_indices: one x batch per output
    assert g(nwb=1) == Q.QMM_E_SHAPE          # no rhs_indices: one W batch per output
    assert b"batch" in L.qmm_last_error()
    assert g(li=ctypes.c_void_p(0x10002)) == Q.QMM_E_ALIGN
    assert g(ri=ctypes.c_void_p(0x10001)) == Q.QMM_E_ALIGN
    assert g(x=P2) == Q.QMM_E_ALIGN
    assert g(K=1 << 20) == Q.QMM_E_SHAPE      # beyond the streaming GEMV's K limit
    assert b"K" in L.qmm_last_error()


def test_gather_qmm_arguments(L):
    def g(x=P, nxb=2, li=None, wq=P, s=P, b=P, nwb=3, ri=None, B=2, dt=0, M=3, N=8, K=64,
          gs=64, bits=4, y=P):
        return _st(L, "qmm_gather_qmm", x, nxb, li, wq, s, b, nwb, ri, B, dt, M, N, K, gs,
                   bits, y, None)
    assert g(x=None) == Q.QMM_E_NULL
    assert g(bits=7) == Q.QMM_E_BITS
    assert g(gs=16) == Q.QMM_E_GROUP
    assert g(dt=2) == Q.QMM_E_DTYPE
    assert g(B=0) == Q.QMM_E_SHAPE
    assert g(B=65536, li=P, ri=P) == Q.QMM_E_SHAPE
    assert g(nxb=1) == Q.QMM_E_SHAPE          # no lhs_indices: one x batch per output
    assert g(nwb=1) == Q.QMM_E_SHAPE          # no rhs_indices: one W batch per output
    assert g(li=ctypes.c_void_p(0x10002)) == Q.QMM_E_ALIGN
    assert g(B=65535, li=P, ri=P, M=65535) == Q.QMM_E_SHAPE   # batches * M beyond int32
    assert g(x=P2) == Q.QMM_E_ALIGN
    assert g(N=7) == Q.QMM_E_ALIGN            # tile kernel: y batches of 42 bytes
    assert b"16 bytes" in L.qmm_last_error()
    assert g(M=100, K=1 << 22) == Q.QMM_E_SHAPE   # beyond the tile kernel's K
    assert b"K" in L.qmm_last_error()


def test_fp_arguments(L):
    def q(w=P, dt=0, rows=4, K=64, gs=32, bits=4, wq=P, sc=P):
        return _st(L, "qmm_fp_quantize", w, dt, rows, K, gs, bits, wq, sc, None)

    def d(wq=P, sc=P, dt=0, rows=4, K=64, gs=32, bits=4, out=P):
        return _st(L, "qmm_fp_dequantize", wq, sc, dt, rows, K, gs, bits, out, None)

    def v(x=P, wq=P, sc=P, dt=0, M=1, N=8, K=64, gs=32, bits=4, y=P):
        return _st(L, "qmm_fp_qmv", x, wq, sc, dt, M, N, K, gs, bits, y, None)
    for f in (q, d, v):
        assert f(bits=3) == Q.QMM_E_BITS
        assert f(bits=2) == Q.QMM_E_BITS
        assert f(gs=64) == Q.QMM_E_GROUP
        assert f(bits=8, gs=16) == Q.QMM_E_GROUP    # nvfp4 is 4-bit only
        assert f(K=48) == Q.QMM_E_SHAPE             # not a multiple of the group size
    assert q(w=None) == Q.QMM_E_NULL and q(sc=None) == Q.QMM_E_NULL
    assert q(dt=5) == Q.QMM_E_DTYPE
    assert q(rows=0) == Q.QMM_E_SHAPE
    assert q(w=P2) == Q.QMM_E_ALIGN
    assert d(out=None) == Q.QMM_E_NULL
    assert d(out=P2) == Q.QMM_E_ALIGN
    assert v(y=None) == Q.QMM_E_NULL
    assert v(dt=2) == Q.QMM_E_DTYPE             # the GEMV takes f16 / bf16
    assert v(K=16, gs=16) == Q.QMM_E_SHAPE      # K must be a multiple of 32
    assert v(K=32768) == Q.QMM_E_SHAPE          # beyond the LDS-staged row of x
    assert v(M=65536) == Q.QMM_E_SHAPE
    assert v(x=P2) == Q.QMM_E_ALIGN


def test_fp_t_arguments(L):
    def t(x=P, wq=P, sc=P, dt=0, M=64, N=8, K=64, gs=32, bits=4, y=P):
        return _st(L, "qmm_fp_t", x, wq, sc, dt, M, N, K, gs, bits, y, None)
    assert t(bits=3) == Q.QMM_E_BITS
    assert t(gs=64) == Q.QMM_E_GROUP
    assert t(bits=8, gs=16) == Q.QMM_E_GROUP
    assert t(x=None) == Q.QMM_E_NULL and t(sc=None) == Q.QMM_E_NULL
    assert t(dt=2) == Q.QMM_E_DTYPE
    assert t(K=48) == Q.QMM_E_SHAPE             # not a multiple of 32
    assert t(M=0) == Q.QMM_E_SHAPE and t(N=0) == Q.QMM_E_SHAPE
    assert t(K=1 << 22) == Q.QMM_E_SHAPE        # beyond the tile kernel's K
    assert t(y=P2) == Q.QMM_E_ALIGN and t(wq=P2) == Q.QMM_E_ALIGN


def test_fp_n_arguments(L):
    def t(x=P, wq=P, sc=P, dt=0, M=64, N=64, K=64, gs=32, bits=4, y=P):
        return _st(L, "qmm_fp_n", x, wq, sc, dt, M, N, K, gs, bits, y, None)
    assert t(bits=3) == Q.QMM_E_BITS
    assert t(gs=64) == Q.QMM_E_GROUP
    assert t(x=None) == Q.QMM_E_NULL and t(sc=None) == Q.QMM_E_NULL
    assert t(dt=2) == Q.QMM_E_DTYPE
    assert t(N=48) == Q.QMM_E_SHAPE             # the quantized dimension: a multiple of 32
    assert t(K=12) == Q.QMM_E_SHAPE             # rows of x: a multiple of 8
    assert t(M=0) == Q.QMM_E_SHAPE and t(K=0) == Q.QMM_E_SHAPE
    assert t(N=1 << 16, K=1 << 16) == Q.QMM_E_SHAPE   # weight beyond 2 GiB
    assert t(y=P2) == Q.QMM_E_ALIGN and t(x=P2) == Q.QMM_E_ALIGN


def test_fp_gather_arguments(L):
    def g(x=P, nxb=2, li=None, wq=P, sc=P, nwb=3, ri=None, B=2, dt=0, M=1, N=8, K=64, gs=32,
          bits=4, y=P):
        return _st(L, "qmm_fp_gather_qmv", x, nxb, li, wq, sc, nwb, ri, B, dt, M, N, K, gs, bits,
                   y, None)
    assert g(x=None) == Q.QMM_E_NULL
    assert g(bits=3) == Q.QMM_E_BITS
    assert g(gs=64) == Q.QMM_E_GROUP
    assert g(dt=2) == Q.QMM_E_DTYPE
    assert g(K=48) == Q.QMM_E_SHAPE
    assert g(K=32768) == Q.QMM_E_SHAPE
    assert g(B=0) == Q.QMM_E_SHAPE
    assert g(B=65536, li=P, ri=P) == Q.QMM_E_SHAPE
    assert g(nxb=1) == Q.QMM_E_SHAPE          # no lhs_indices: one x batch per output
    assert g(nwb=1) == Q.QMM_E_SHAPE          # no rhs_indices: one W batch per output
    assert g(li=ctypes.c_void_p(0x10002)) == Q.QMM_E_ALIGN
    assert g(y=P2) == Q.QMM_E_ALIGN


def test_affine_packed_arguments(L):
    def pk(wq=P, s=P, b=P, dt=0, N=8, K=64, gs=64, bits=4, wp=P, sbp=P):
        return _st(L, "qmm_affine_pack", wq, s, b, dt, N, K, gs, bits, wp, sbp, None)

    def mv(x=P, wp=P, sbp=P, dt=0, M=1, N=8, K=64, gs=64, bits=4, y=P):
        return _st(L, "qmv_affine_packed", x, wp, sbp, dt, M, N, K, gs, bits, y, None)
    assert pk(wq=None) == Q.QMM_E_NULL
    assert pk(wp=None) == Q.QMM_E_NULL          # needed for power-of-two bits
    assert pk(bits=7) == Q.QMM_E_BITS
    assert pk(gs=16) == Q.QMM_E_GROUP
    assert pk(dt=5) == Q.QMM_E_DTYPE
    assert pk(N=6) == Q.QMM_E_SHAPE             # blocks of 4 rows
    assert pk(N=5, bits=3, wp=None) == Q.QMM_E_SHAPE   # blocks of 2 rows
    assert pk(K=48) == Q.QMM_E_SHAPE
    assert pk(wq=P2) == Q.QMM_E_ALIGN
    def mt(x=P, wp=P, sbp=P, dt=0, M=64, N=8, K=64, gs=64, bits=4, y=P):
        return _st(L, "qmm_t_affine_packed", x, wp, sbp, dt, M, N, K, gs, bits, y, None)
    for f in (mv, mt):
        assert f(x=None) == Q.QMM_E_NULL and f(sbp=None) == Q.QMM_E_NULL
        assert f(bits=7) == Q.QMM_E_BITS
        assert f(gs=16) == Q.QMM_E_GROUP
        assert f(dt=2) == Q.QMM_E_DTYPE
        assert f(N=6) == Q.QMM_E_SHAPE              # blocks of 4 rows (bits 2, 4, 8)
        assert f(N=5, bits=3) == Q.QMM_E_SHAPE      # blocks of 2 rows (bits 3, 5, 6)
        assert f(K=48) == Q.QMM_E_SHAPE
        assert f(M=0) == Q.QMM_E_SHAPE
        assert f(sbp=P2) == Q.QMM_E_ALIGN and f(y=P2) == Q.QMM_E_ALIGN
    assert mv(K=32768) == Q.QMM_E_SHAPE          # beyond the interleaved-row GEMV's x row
    assert mv(K=65536, bits=3) == Q.QMM_E_SHAPE  # beyond the streaming GEMV's x row
    assert mv(M=65536) == Q.QMM_E_SHAPE
    assert mt(K=1 << 22) == Q.QMM_E_SHAPE        # beyond the tile kernel


def test_batched_arguments(L):
    def f(x=P, wq=P, s=P, b=P, B=2, E=2, dt=0, M=1, N=8, K=64, gs=64, bits=4, y=P):
        return _st(L, "qmm_t_batched", x, wq, s, b, B, E, dt, M, N, K, gs, bits, y, None)
    assert f(x=None) == Q.QMM_E_NULL
    assert f(bits=7) == Q.QMM_E_BITS
    assert f(gs=16) == Q.QMM_E_GROUP
    assert f(dt=2) == Q.QMM_E_DTYPE
    assert f(B=0) == Q.QMM_E_SHAPE
    assert f(B=65536, E=65536) == Q.QMM_E_SHAPE
    assert f(E=3) == Q.QMM_E_SHAPE            # one weight, or one per batch
    assert b"w_batches" in L.qmm_last_error()
    assert f(E=0) == Q.QMM_E_SHAPE
    assert f(B=65535, E=1, M=65535) == Q.QMM_E_SHAPE   # batches * M rows beyond int32
    assert f(x=P2) == Q.QMM_E_ALIGN
    assert f(M=3, N=7) == Q.QMM_E_ALIGN       # MFMA GEMV per batch: y batch of 42 bytes
    assert b"16 bytes" in L.qmm_last_error()
    assert f(M=100, N=7) == Q.QMM_E_ALIGN     # tile kernel per batch: y batch of 1400 bytes
    assert f(M=100, K=1 << 22) == Q.QMM_E_SHAPE   # beyond the tile kernel's K


def test_qmm_n_arguments(L):
    def f(x=P, wq=P, s=P, b=P, dt=0, M=1, N=64, K=64, gs=64, bits=4, y=P):
        return _st(L, "qmm_n", x, wq, s, b, dt, M, N, K, gs, bits, y, None)
    assert f(x=None) == Q.QMM_E_NULL
    assert f(bits=7) == Q.QMM_E_BITS
    assert f(gs=48) == Q.QMM_E_GROUP
    assert f(dt=2) == Q.QMM_E_DTYPE
    assert f(N=96) == Q.QMM_E_SHAPE           # W [K, N] is quantized along N
    assert b"N" in L.qmm_last_error()
    assert f(M=0) == Q.QMM_E_SHAPE
    assert f(K=0) == Q.QMM_E_SHAPE
    assert f(M=1, N=262208, K=8192) == Q.QMM_E_SHAPE  # one row: 64 K ranges x N > 16M floats
    assert b"workspace" in L.qmm_last_error()
    assert f(M=300, N=4160, K=2047) == Q.QMM_E_ALIGN  # x blocks of 252 rows x 2047 halves
    assert f(x=P2) == Q.QMM_E_ALIGN
    assert f(s=ctypes.c_void_p(0x10001)) == Q.QMM_E_ALIGN
