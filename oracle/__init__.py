"""Python access to the plain CPU oracle (oracle/qmm_oracle.c).

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package; the HIP library and its
binding never do.

Arrays are numpy. Activations, scales, biases and outputs are passed as raw
storage words: uint16 for f16/bf16, float32 for f32 (see ``DTYPES``).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F16, BF16, F32 = 0, 1, 2
DTYPES = {"f16": F16, "bf16": BF16, "f32": F32}

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        _lib = ctypes.CDLL(_LIB_PATH)
        _declare(_lib)
    return _lib


def _declare(L):
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.orc_f32_to_f16.argtypes = [ctypes.c_float]
    L.orc_f32_to_f16.restype = ctypes.c_uint16
    L.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
    L.orc_f16_to_f32.restype = ctypes.c_float
    L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
    L.orc_f32_to_bf16.restype = ctypes.c_uint16
    L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
    L.orc_bf16_to_f32.restype = ctypes.c_float
    L.orc_to_f32.argtypes = [vp, i32, i64, vp]
    L.orc_to_f32.restype = None
    L.orc_from_f32.argtypes = [vp, i32, i64, vp]
    L.orc_from_f32.restype = None
    L.orc_row_bytes.argtypes = [i64, i32]
    L.orc_row_bytes.restype = i64
    L.orc_quantize.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp, vp, vp, vp]
    L.orc_quantize.restype = i32
    L.orc_unpack_code.argtypes = [vp, i64, i32]
    L.orc_unpack_code.restype = ctypes.c_uint32
    L.orc_unpack.argtypes = [vp, i64, i64, i32, vp]
    L.orc_unpack.restype = i32
    L.orc_dequantize.argtypes = [vp, vp, vp, i32, i64, i64, i32, i32, vp, vp]
    L.orc_dequantize.restype = i32
    L.orc_qmm_t.argtypes = [vp, vp, vp, vp, i32, i64, i64, i64, i32, i32, vp, vp, i32]
    L.orc_qmm_t.restype = i32
    L.orc_qmm_t_rows.argtypes = [vp, vp, vp, vp, i32, i64, i64, i64, i32, i32,
                                 i64, i64, vp, vp, i32]
    L.orc_qmm_t_rows.restype = i32
    L.orc_qmm_n.argtypes = [vp, vp, vp, vp, i32, i64, i64, i64, i32, i32, vp, vp, i32]
    L.orc_qmm_n.restype = i32
    L.orc_qconv2d_nhwc.argtypes = [vp, i64, i64, i64, i64, vp, vp, vp, i64, i32,
                                   i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                   vp, vp, i32]
    L.orc_qconv2d_nhwc.restype = i32
    u8, f32 = ctypes.c_uint8, ctypes.c_float
    L.orc_fp4_value.argtypes = [u8]
    L.orc_fp4_value.restype = f32
    L.orc_fp4_encode.argtypes = [f32]
    L.orc_fp4_encode.restype = u8
    L.orc_fp8_e4m3_value.argtypes = [u8]
    L.orc_fp8_e4m3_value.restype = f32
    L.orc_fp8_e4m3_encode.argtypes = [f32]
    L.orc_fp8_e4m3_encode.restype = u8
    L.orc_e8m0_encode.argtypes = [f32]
    L.orc_e8m0_encode.restype = u8
    L.orc_fp_scale.argtypes = [u8, i32, i32]
    L.orc_fp_scale.restype = f32
    L.orc_fp_quantize.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp]
    L.orc_fp_quantize.restype = i32
    L.orc_fp_dequantize.argtypes = [vp, vp, i32, i64, i64, i32, i32, vp, vp]
    L.orc_fp_dequantize.restype = i32
    L.orc_fp_qmm_t.argtypes = [vp, vp, vp, i32, i64, i64, i64, i32, i32, vp, vp, i32]
    L.orc_fp_qmm_t.restype = i32
    L.orc_fp_qmm_n.argtypes = [vp, vp, vp, i32, i64, i64, i64, i32, i32, vp, vp, i32]
    L.orc_fp_qmm_n.restype = i32


class OracleError(RuntimeError):
    pass


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _chk(rc, what):
    if rc != 0:
        raise OracleError(f"{what} returned {rc}")


def storage_dtype(dt):
    return np.float32 if dt == F32 else np.uint16


def _words(a, dt):
    """Contiguous storage words for dtype ``dt``."""
    a = np.ascontiguousarray(a)
    if a.dtype != storage_dtype(dt):
        raise TypeError(f"expected {storage_dtype(dt)} storage, got {a.dtype}")
    return a


# ---------------------------------------------------------------- converters

def f32_to_f16(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, np.uint16)
    lib().orc_from_f32(_p(a), F16, a.size, _p(out))
    return out


def f16_to_f32(h):
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().orc_to_f32(_p(h), F16, h.size, _p(out))
    return out


def f32_to_bf16(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, np.uint16)
    lib().orc_from_f32(_p(a), BF16, a.size, _p(out))
    return out


def bf16_to_f32(h):
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().orc_to_f32(_p(h), BF16, h.size, _p(out))
    return out


def to_f32(words, dt):
    words = _words(words, dt)
    out = np.empty(words.shape, np.float32)
    lib().orc_to_f32(_p(words), dt, words.size, _p(out))
    return out


def from_f32(a, dt):
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, storage_dtype(dt))
    lib().orc_from_f32(_p(a), dt, a.size, _p(out))
    return out


# ---------------------------------------------------------------- method

def row_bytes(K, bits):
    return K * bits // 8


def quantize(w, dt, group_size=64, bits=4, with_f32=False):
    """w: [rows, K] storage words of dtype dt.

    Returns (wq bytes [rows, K*bits/8] uint8, scales [rows, K/gs], biases
    [rows, K/gs]) in storage words; with ``with_f32`` also the fp32 scale and
    bias before rounding to T."""
    w = _words(w, dt)
    rows, K = w.shape
    G = K // group_size if group_size else 0
    wq = np.zeros((rows, row_bytes(K, bits)), np.uint8)
    s = np.zeros((rows, max(G, 1)), storage_dtype(dt))
    b = np.zeros((rows, max(G, 1)), storage_dtype(dt))
    s32 = np.zeros((rows, max(G, 1)), np.float32)
    b32 = np.zeros((rows, max(G, 1)), np.float32)
    rc = lib().orc_quantize(_p(w), dt, rows, K, group_size, bits, _p(wq), _p(s),
                            _p(b), _p(s32), _p(b32))
    _chk(rc, "orc_quantize")
    if with_f32:
        return wq, s, b, s32, b32
    return wq, s, b


def unpack(wq, K, bits):
    wq = np.ascontiguousarray(wq, dtype=np.uint8)
    rows = wq.shape[0]
    codes = np.zeros((rows, K), np.uint8)
    _chk(lib().orc_unpack(_p(wq), rows, K, bits, _p(codes)), "orc_unpack")
    return codes


def dequantize(wq, scales, biases, dt, K, group_size=64, bits=4):
    """Returns (w32 [rows,K] float32, w_out [rows,K] storage words)."""
    wq = np.ascontiguousarray(wq, dtype=np.uint8)
    scales, biases = _words(scales, dt), _words(biases, dt)
    rows = wq.shape[0]
    w32 = np.zeros((rows, K), np.float32)
    wo = np.zeros((rows, K), storage_dtype(dt))
    rc = lib().orc_dequantize(_p(wq), _p(scales), _p(biases), dt, rows, K,
                              group_size, bits, _p(w32), _p(wo))
    _chk(rc, "orc_dequantize")
    return w32, wo


def qmm_t(x, wq, scales, biases, dt, group_size=64, bits=4, nthreads=1,
          rows=None):
    """y = x . dequant(W)^T. x: [M,K] words. Returns (y32, y_T).

    ``rows=(m0, m1)`` computes only rows m0..m1-1 of y."""
    x = _words(x, dt)
    wq = np.ascontiguousarray(wq, dtype=np.uint8)
    scales, biases = _words(scales, dt), _words(biases, dt)
    M, K = x.shape
    N = wq.shape[0]
    m0, m1 = (0, M) if rows is None else rows
    y32 = np.zeros((m1 - m0, N), np.float32)
    yo = np.zeros((m1 - m0, N), storage_dtype(dt))
    rc = lib().orc_qmm_t_rows(_p(x), _p(wq), _p(scales), _p(biases), dt, M, N,
                              K, group_size, bits, m0, m1, _p(y32), _p(yo),
                              nthreads)
    _chk(rc, "orc_qmm_t")
    return y32, yo


def qmm_n(x, wq, scales, biases, dt, group_size=64, bits=4, nthreads=1):
    """Non-transposed product (mlx CPU backend _qmm): y = x . dequant(W)
    with W [K, N] quantized along N. x: [M,K] words; wq: [K, N*bits/8]
    bytes; scales, biases: [K, N/gs] words. Returns (y32, y_T)."""
    x = _words(x, dt)
    wq = np.ascontiguousarray(wq, dtype=np.uint8)
    scales, biases = _words(scales, dt), _words(biases, dt)
    M, K = x.shape
    N = wq.shape[1] * 8 // bits
    if wq.shape[0] != K:
        raise ValueError("qmm_n: W must have K rows")
    y32 = np.zeros((M, N), np.float32)
    yo = np.zeros((M, N), storage_dtype(dt))
    rc = lib().orc_qmm_n(_p(x), _p(wq), _p(scales), _p(biases), dt, M, N, K,
                         group_size, bits, _p(y32), _p(yo), nthreads)
    _chk(rc, "orc_qmm_n")
    return y32, yo


def gather_qmm(x, wq, scales, biases, lhs, rhs, dt, group_size=64, bits=4,
               nthreads=1):
    """Gathered products, "Add the 3bit packed qmm_t", ops.cpp gather_qmm:
    one product per index pair, output z = x[lhs[z]] . dequant(W[rhs[z]])^T,
    each computed by qmm_t above. A missing index array (None) means z.

    x: [Bx, M, K] words; wq: [E, N, row bytes]; scales, biases: [E, N, K/gs]
    words; lhs, rhs: int sequences (or None) of one length B. Indices must
    lie in range. Returns (y32 [B,M,N], y_T [B,M,N])."""
    x = np.asarray(x)
    wq = np.asarray(wq)
    Bx, M, _ = x.shape
    E, N = wq.shape[0], wq.shape[1]
    B = len(lhs) if lhs is not None else (len(rhs) if rhs is not None else Bx)
    lhs = list(range(B)) if lhs is None else [int(v) for v in lhs]
    rhs = list(range(B)) if rhs is None else [int(v) for v in rhs]
    if len(lhs) != B or len(rhs) != B:
        raise ValueError("gather_qmm: index arrays of different lengths")
    y32 = np.zeros((B, M, N), np.float32)
    yo = np.zeros((B, M, N), storage_dtype(dt))
    for z in range(B):
        if not (0 <= lhs[z] < Bx and 0 <= rhs[z] < E):
            raise IndexError(f"gather_qmm: index pair ({lhs[z]}, {rhs[z]}) out of range")
        y32[z], yo[z] = qmm_t(x[lhs[z]], wq[rhs[z]], scales[rhs[z]], biases[rhs[z]], dt,
                              group_size, bits, nthreads)
    return y32, yo


def conv_out_hw(H, W, kh, kw, stride, pad):
    return ((H + 2 * pad[0] - kh) // stride[0] + 1,
            (W + 2 * pad[1] - kw) // stride[1] + 1)


def qconv2d_nhwc(x, wq, scales, biases, dt, O, kh, kw, stride=(1, 1),
                 pad=(0, 0), groups=1, group_size=64, bits=4, nthreads=1):
    """x: [B,H,W,C] words; wq: [O, K_pad*bits/8] bytes. Returns (y32, y_T)
    with shape [B,OH,OW,O]."""
    x = _words(x, dt)
    wq = np.ascontiguousarray(wq, dtype=np.uint8)
    scales, biases = _words(scales, dt), _words(biases, dt)
    B, H, W, C = x.shape
    OH, OW = conv_out_hw(H, W, kh, kw, stride, pad)
    y32 = np.zeros((B, OH, OW, O), np.float32)
    yo = np.zeros((B, OH, OW, O), storage_dtype(dt))
    rc = lib().orc_qconv2d_nhwc(_p(x), B, H, W, C, _p(wq), _p(scales),
                                _p(biases), O, kh, kw, stride[0], stride[1],
                                pad[0], pad[1], groups, dt, group_size, bits,
                                _p(y32), _p(yo), nthreads)
    _chk(rc, "orc_qconv2d_nhwc")
    return y32, yo


def conv_weight_matrix(w, groups, group_size):
    """Weight [O, kh, kw, C/groups] (storage words) -> [O, K_pad] words:
    each row flattened in (dy, dx, c) order and zero-padded on the right to a
    multiple of the group size (the quantize_weights step of the conv issue).
    """
    O = w.shape[0]
    K_true = int(np.prod(w.shape[1:]))
    K_pad = -(-K_true // group_size) * group_size
    out = np.zeros((O, K_pad), w.dtype)
    out[:, :K_true] = w.reshape(O, K_true)
    return out


# ------------------------------------------------- floating-point modes
# (bits, group size): (4, 32) mxfp4, (4, 16) nvfp4, (8, 32) mxfp8; see
# fp_oracle.c ("mlx 1.0.0 backend/cpu/quantized.cpp": FP4_LUT, to_fp4_e2m1,
# to_fp8_e8m0, dequantize_scale, fp_quantize_dequantize, fp_qmm_t).

FP_MODES = {"mxfp4": (4, 32), "nvfp4": (4, 16), "mxfp8": (8, 32)}


def fp4_value(code):
    return lib().orc_fp4_value(int(code))


def fp4_encode(x):
    return lib().orc_fp4_encode(float(x))


def e4m3_value(b):
    return lib().orc_fp8_e4m3_value(int(b))


def e4m3_encode(x):
    return lib().orc_fp8_e4m3_encode(float(x))


def e8m0_encode(x):
    return lib().orc_e8m0_encode(float(x))


def fp_scale(s, group_size, dt):
    return lib().orc_fp_scale(int(s), group_size, dt)


def fp_quantize(w, dt, group_size=32, bits=4):
    """w: [rows, K] storage words. Returns (wq bytes [rows, K*bits/8],
    scales uint8 [rows, K/gs])."""
    w = _words(w, dt)
    rows, K = w.shape
    wq = np.zeros((rows, row_bytes(K, bits)), np.uint8)
    sc = np.zeros((rows, max(K // group_size, 1)), np.uint8)
    _chk(lib().orc_fp_quantize(_p(w), dt, rows, K, group_size, bits, _p(wq), _p(sc)),
         "orc_fp_quantize")
    return wq, sc


def fp_dequantize(wq, scales, dt, K, group_size=32, bits=4):
    """Returns (w32 [rows,K] float32, w_out [rows,K] storage words)."""
    wq = np.ascontiguousarray(wq, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows = wq.shape[0]
    w32 = np.zeros((rows, K), np.float32)
    wo = np.zeros((rows, K), storage_dtype(dt))
    _chk(lib().orc_fp_dequantize(_p(wq), _p(scales), dt, rows, K, group_size, bits, _p(w32),
                                 _p(wo)), "orc_fp_dequantize")
    return w32, wo


def fp_qmm_t(x, wq, scales, dt, group_size=32, bits=4, nthreads=1):
    """y = x . dequant(W)^T in an fp mode. x: [M,K] words. Returns (y32, y_T)."""
    x = _words(x, dt)
    wq = np.ascontiguousarray(wq, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    M, K = x.shape
    N = wq.shape[0]
    y32 = np.zeros((M, N), np.float32)
    yo = np.zeros((M, N), storage_dtype(dt))
    _chk(lib().orc_fp_qmm_t(_p(x), _p(wq), _p(scales), dt, M, N, K, group_size, bits, _p(y32),
                            _p(yo), nthreads), "orc_fp_qmm_t")
    return y32, yo


def fp_qmm_n(x, wq, scales, dt, group_size=32, bits=4, nthreads=1):
    """Non-transposed product in an fp mode ("mlx 1.0.0 backend/cpu/
    quantized.cpp", fp_qmm): y = x . dequant(W), W [K, N] quantized along N.
    x: [M,K] words; wq: [K, N*bits/8] bytes; scales: uint8 [K, N/gs].
    Returns (y32, y_T)."""
    x = _words(x, dt)
    wq = np.ascontiguousarray(wq, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    M, K = x.shape
    N = wq.shape[1] * 8 // bits
    if wq.shape[0] != K:
        raise ValueError("fp_qmm_n: W must have K rows")
    y32 = np.zeros((M, N), np.float32)
    yo = np.zeros((M, N), storage_dtype(dt))
    _chk(lib().orc_fp_qmm_n(_p(x), _p(wq), _p(scales), dt, M, N, K, group_size, bits, _p(y32),
                            _p(yo), nthreads), "orc_fp_qmm_n")
    return y32, yo


# ---------------------------------------------------- affine-packed layout
# "Add the 3bit packed qmm_t", ops.cpp quantize with QuantizationType::
# AffinePacked: after the affine quantizer, rows are taken in blocks of RP =
# 4 (power-of-two bits) or 2 (3, 5, 6 bits); each block's scales and biases
# become one row holding, per group, the RP scales then the RP biases; for
# power-of-two bits the block's weight words are interleaved (word w of row r
# at position w*RP + r). The steps below follow the page's order: unflatten
# the row axis, concatenate scales and biases, move the block axis last,
# flatten.

def affine_pack(wq, scales, biases, bits):
    """wq: [N, K*bits/8] bytes; scales, biases: [N, G] words. Returns
    (wq_packed bytes [N/RP, RP*K*bits/8] for power-of-two bits, else wq
    unchanged; sb_packed words [N/RP, G*2*RP])."""
    wq = np.ascontiguousarray(wq, dtype=np.uint8)
    N = wq.shape[0]
    pow2 = (bits & (bits - 1)) == 0
    rp = 4 if pow2 else 2
    if N % rp:
        raise ValueError(f"affine_pack: rows ({N}) must be a multiple of {rp}")
    s = scales.reshape(N // rp, rp, -1)                  # unflatten(-2, {-1, rp})
    b = biases.reshape(N // rp, rp, -1)
    sb = np.concatenate([s, b], axis=-2)                 # [N/rp, 2rp, G]
    sb = np.moveaxis(sb, -2, -1)                         # [N/rp, G, 2rp]
    sb = np.ascontiguousarray(sb).reshape(N // rp, -1)   # flatten(-2, -1)
    if pow2:
        words = wq.view(np.uint32).reshape(N // rp, rp, -1)
        words = np.ascontiguousarray(np.moveaxis(words, -2, -1))   # [N/rp, Kw, rp]
        wq = words.reshape(N // rp, -1).view(np.uint8)
    return wq, sb
