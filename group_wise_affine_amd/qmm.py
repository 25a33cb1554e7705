"""Python binding of libqmm (ctypes). Argument marshalling only: every step of
the computation runs in the HIP kernels of libqmm.so. PyTorch supplies device
memory and the current stream.

Functions carry the C names: qmm_quantize, qmm_dequantize, qmm_t, qmv,
qconv2d_nhwc. Tensors must be contiguous and on a ROCm device; packed weights
are int32 tensors holding the uint32 words. Raises QmmError on a non-OK
status and RuntimeError if the library has not been built.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqmm.so")

QMM_OK, QMM_E_NULL, QMM_E_BITS, QMM_E_GROUP, QMM_E_SHAPE, QMM_E_DTYPE, \
    QMM_E_ALIGN, QMM_E_LAUNCH = range(8)
STATUS_NAMES = ["QMM_OK", "QMM_E_NULL", "QMM_E_BITS", "QMM_E_GROUP",
                "QMM_E_SHAPE", "QMM_E_DTYPE", "QMM_E_ALIGN", "QMM_E_LAUNCH"]
EXPORTS = ["qmm_quantize", "qmm_dequantize", "qmm_t", "qmv", "qmm_n", "qconv2d_nhwc",
           "qmm_gather_qmv", "qmm_gather_qmm", "qmm_t_batched",
           "qmm_fp_quantize", "qmm_fp_dequantize", "qmm_fp_qmv", "qmm_fp_gather_qmv",
           "qmm_affine_pack", "qmv_affine_packed",
           "qmm_crossover_m", "qmm_last_error"]

_DT = {torch.float16: 0, torch.bfloat16: 1, torch.float32: 2}

_lib = None


class QmmError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS_NAMES[status] if 0 <= status < 8 else status}: {msg}")
        self.status = status


def lib():
    """Load libqmm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -c 'import "
                f"__graft_entry__ as g; g.build()'` (or group_wise_affine_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.qmm_quantize.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp, vp, vp]
        L.qmm_dequantize.argtypes = [vp, vp, vp, i32, i64, i64, i32, i32, vp, vp]
        L.qmm_t.argtypes = [vp, vp, vp, vp, i32, i64, i64, i64, i32, i32, vp, vp]
        L.qmv.argtypes = [vp, vp, vp, vp, i32, i64, i64, i64, i32, i32, vp, vp]
        L.qconv2d_nhwc.argtypes = [vp, i64, i64, i64, i64, vp, vp, vp, i64, i32,
                                   i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                   vp, vp]
        L.qmm_n.argtypes = [vp, vp, vp, vp, i32, i64, i64, i64, i32, i32, vp, vp]
        L.qmm_gather_qmv.argtypes = [vp, i64, vp, vp, vp, vp, i64, vp, i64, i32, i64,
                                     i64, i64, i32, i32, vp, vp]
        L.qmm_gather_qmm.argtypes = L.qmm_gather_qmv.argtypes
        L.qmm_affine_pack.argtypes = [vp, vp, vp, i32, i64, i64, i32, i32, vp, vp, vp]
        L.qmv_affine_packed.argtypes = [vp, vp, vp, i32, i64, i64, i64, i32, i32, vp, vp]
        L.qmm_t_batched.argtypes = [vp, vp, vp, vp, i64, i64, i32, i64, i64, i64, i32, i32,
                                    vp, vp]
        L.qmm_fp_quantize.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp, vp]
        L.qmm_fp_dequantize.argtypes = [vp, vp, i32, i64, i64, i32, i32, vp, vp]
        L.qmm_fp_qmv.argtypes = [vp, vp, vp, i32, i64, i64, i64, i32, i32, vp, vp]
        L.qmm_fp_gather_qmv.argtypes = [vp, i64, vp, vp, vp, i64, vp, i64, i32, i64, i64, i64,
                                        i32, i32, vp, vp]
        for f in ("qmm_quantize", "qmm_dequantize", "qmm_t", "qmv", "qmm_n", "qconv2d_nhwc",
                  "qmm_gather_qmv", "qmm_gather_qmm", "qmm_t_batched", "qmm_fp_quantize",
                  "qmm_fp_dequantize", "qmm_fp_qmv", "qmm_fp_gather_qmv",
                  "qmm_affine_pack", "qmv_affine_packed"):
            getattr(L, f).restype = i32
        L.qmm_crossover_m.argtypes = [i32, i32]
        L.qmm_crossover_m.restype = i32
        L.qmm_last_error.argtypes = []
        L.qmm_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(st):
    if st != QMM_OK:
        raise QmmError(st, lib().qmm_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libqmm must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dt(dtype):
    if dtype not in _DT:
        raise QmmError(QMM_E_DTYPE, f"unsupported dtype {dtype}")
    return _DT[dtype]


def packed_words(K, bits):
    return K * bits // 32


def qmm_quantize(w, group_size=64, bits=4, out=None, stream=None):
    """w [rows, K] -> (wq int32 [rows, K*bits/32], scales, biases [rows, K/gs])."""
    rows, K = w.shape
    if out is None:
        G = max(K // group_size, 1) if group_size > 0 else 1
        out = (torch.empty((rows, max(packed_words(K, bits), 1)), dtype=torch.int32, device=w.device),
               torch.empty((rows, G), dtype=w.dtype, device=w.device),
               torch.empty((rows, G), dtype=w.dtype, device=w.device))
    wq, s, b = out
    _check(lib().qmm_quantize(_ptr(w), _dt(w.dtype), rows, K, group_size, bits,
                              _ptr(wq), _ptr(s), _ptr(b), _stream(stream)))
    return wq, s, b


def qmm_dequantize(wq, scales, biases, group_size=64, bits=4, out=None, stream=None):
    rows = wq.shape[0]
    K = wq.shape[1] * 32 // bits
    if out is None:
        out = torch.empty((rows, K), dtype=scales.dtype, device=wq.device)
    _check(lib().qmm_dequantize(_ptr(wq), _ptr(scales), _ptr(biases), _dt(scales.dtype),
                                rows, K, group_size, bits, _ptr(out), _stream(stream)))
    return out


def _matmul(fn, x, wq, scales, biases, group_size, bits, out, stream):
    M, K = x.shape
    N = wq.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    _check(fn(_ptr(x), _ptr(wq), _ptr(scales), _ptr(biases), _dt(x.dtype), M, N, K,
              group_size, bits, _ptr(out), _stream(stream)))
    return out


def qmm_t(x, wq, scales, biases, group_size=64, bits=4, out=None, stream=None):
    """y [M,N] = x [M,K] . dequant(wq)^T (routes small M to qmv)."""
    return _matmul(lib().qmm_t, x, wq, scales, biases, group_size, bits, out, stream)


def qmv(x, wq, scales, biases, group_size=64, bits=4, out=None, stream=None):
    """Same as qmm_t, always on the streaming GEMV."""
    return _matmul(lib().qmv, x, wq, scales, biases, group_size, bits, out, stream)


def qmm_n(x, wq, scales, biases, group_size=64, bits=4, out=None, stream=None):
    """y = x . dequant(W) with W [K, N] quantized along N: x [M, K], wq
    [K, N*bits/32] (uint32 words), scales, biases [K, N/group_size]."""
    M, K = x.shape
    if wq.shape[0] != K:
        raise ValueError("qmm_n: W must have K rows")
    N = wq.shape[1] * 32 // bits
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    _check(lib().qmm_n(_ptr(x), _ptr(wq), _ptr(scales), _ptr(biases), _dt(x.dtype), M, N, K,
                       group_size, bits, _ptr(out), _stream(stream)))
    return out


def gather_qmv(x, wq, scales, biases, lhs_indices=None, rhs_indices=None, group_size=64,
               bits=4, out=None, stream=None, _fn="qmm_gather_qmv"):
    """y[z] = x[lhs_indices[z]] . dequant(W[rhs_indices[z]])^T on the
    gathered streaming GEMV (small M).

    x [Bx, M, K]; wq [E, N, K*bits/32] (uint32 words); scales, biases
    [E, N, K/group_size]; indices int32 device tensors of one length B (None:
    z itself). Returns y [B, M, N]."""
    Bx, M, K = x.shape
    E, N = wq.shape[0], wq.shape[1]
    if lhs_indices is not None:
        B = lhs_indices.numel()
    elif rhs_indices is not None:
        B = rhs_indices.numel()
    else:
        B = Bx
    for t in (lhs_indices, rhs_indices):
        if t is not None and (t.dtype != torch.int32 or t.numel() != B):
            raise ValueError("indices must be int32 tensors of one length")
    if out is None:
        out = torch.empty((B, M, N), dtype=x.dtype, device=x.device)
    _check(getattr(lib(), _fn)(_ptr(x), Bx, _ptr(lhs_indices), _ptr(wq), _ptr(scales),
                               _ptr(biases), E, _ptr(rhs_indices), B, _dt(x.dtype), M, N, K,
                               group_size, bits, _ptr(out), _stream(stream)))
    return out


def gather_qmm(x, wq, scales, biases, lhs_indices=None, rhs_indices=None, group_size=64,
               bits=4, out=None, stream=None):
    """Same as gather_qmv for any M (the MFMA tile kernel beyond a few rows)."""
    return gather_qmv(x, wq, scales, biases, lhs_indices, rhs_indices, group_size, bits, out,
                      stream, _fn="qmm_gather_qmm")


def qmm_t_batched(x, wq, scales, biases, group_size=64, bits=4, out=None, stream=None):
    """y[b] = x[b] . dequant(W[b])^T, or the one W for every b: x [B, M, K];
    wq [B or 1, N, K*bits/32] (uint32 words); scales, biases [B or 1, N,
    K/group_size]. Returns y [B, M, N]."""
    B, M, K = x.shape
    E, N = wq.shape[0], wq.shape[1]
    if out is None:
        out = torch.empty((B, M, N), dtype=x.dtype, device=x.device)
    _check(lib().qmm_t_batched(_ptr(x), _ptr(wq), _ptr(scales), _ptr(biases), B, E,
                               _dt(x.dtype), M, N, K, group_size, bits, _ptr(out),
                               _stream(stream)))
    return out


def fp_quantize(w, group_size=32, bits=4, stream=None):
    """Floating-point mode ((4, 32) mxfp4, (4, 16) nvfp4, (8, 32) mxfp8):
    w [rows, K] -> (wq int32 [rows, K*bits/32], scales uint8 [rows, K/gs])."""
    rows, K = w.shape
    wq = torch.empty((rows, max(K * bits // 32, 1)), dtype=torch.int32, device=w.device)
    sc = torch.empty((rows, max(K // group_size, 1)), dtype=torch.uint8, device=w.device)
    _check(lib().qmm_fp_quantize(_ptr(w), _dt(w.dtype), rows, K, group_size, bits, _ptr(wq),
                                 _ptr(sc), _stream(stream)))
    return wq, sc


def fp_dequantize(wq, scales, dtype=torch.float16, group_size=32, bits=4, stream=None):
    rows = wq.shape[0]
    K = wq.shape[1] * 32 // bits
    out = torch.empty((rows, K), dtype=dtype, device=wq.device)
    _check(lib().qmm_fp_dequantize(_ptr(wq), _ptr(scales), _dt(dtype), rows, K, group_size,
                                   bits, _ptr(out), _stream(stream)))
    return out


def fp_qmv(x, wq, scales, group_size=32, bits=4, out=None, stream=None):
    """y [M,N] = x [M,K] . dequant(W)^T for a floating-point mode."""
    M, K = x.shape
    N = wq.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    _check(lib().qmm_fp_qmv(_ptr(x), _ptr(wq), _ptr(scales), _dt(x.dtype), M, N, K, group_size,
                            bits, _ptr(out), _stream(stream)))
    return out


def fp_gather_qmv(x, wq, scales, lhs_indices=None, rhs_indices=None, group_size=32, bits=4,
                  out=None, stream=None):
    """y[z] = x[lhs_indices[z]] . dequant(W[rhs_indices[z]])^T in a floating-point
    mode: x [Bx, M, K]; wq [E, N, K*bits/32]; scales uint8 [E, N, K/gs]."""
    Bx, M, K = x.shape
    E, N = wq.shape[0], wq.shape[1]
    B = (lhs_indices.numel() if lhs_indices is not None else
         rhs_indices.numel() if rhs_indices is not None else Bx)
    for t in (lhs_indices, rhs_indices):
        if t is not None and (t.dtype != torch.int32 or t.numel() != B):
            raise ValueError("indices must be int32 tensors of one length")
    if out is None:
        out = torch.empty((B, M, N), dtype=x.dtype, device=x.device)
    _check(lib().qmm_fp_gather_qmv(_ptr(x), Bx, _ptr(lhs_indices), _ptr(wq), _ptr(scales), E,
                                   _ptr(rhs_indices), B, _dt(x.dtype), M, N, K, group_size, bits,
                                   _ptr(out), _stream(stream)))
    return out


def affine_pack(wq, scales, biases, group_size=64, bits=4, stream=None):
    """Affine-packed layout of (wq [N, K*bits/32], scales, biases [N, K/gs]):
    returns (wq_packed [N/4, 4*K*bits/32] for bits 2/4/8, else wq itself;
    sb_packed [N/RP, K/gs*2*RP])."""
    N = wq.shape[0]
    K = wq.shape[1] * 32 // bits
    pow2 = (bits & (bits - 1)) == 0
    rp = 4 if pow2 else 2
    wp = torch.empty((N // rp, rp * wq.shape[1]), dtype=torch.int32,
                     device=wq.device) if pow2 else None
    sbp = torch.empty((N // rp, scales.shape[1] * 2 * rp), dtype=scales.dtype, device=wq.device)
    _check(lib().qmm_affine_pack(_ptr(wq), _ptr(scales), _ptr(biases), _dt(scales.dtype), N, K,
                                 group_size, bits, _ptr(wp), _ptr(sbp), _stream(stream)))
    return (wp if pow2 else wq), sbp


def qmv_affine_packed(x, wq_packed, sb_packed, N, group_size=64, bits=4, out=None, stream=None):
    """y [M,N] = x [M,K] . dequant(W)^T from the affine-packed layout."""
    M, K = x.shape
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    _check(lib().qmv_affine_packed(_ptr(x), _ptr(wq_packed), _ptr(sb_packed), _dt(x.dtype), M, N,
                                   K, group_size, bits, _ptr(out), _stream(stream)))
    return out


def conv_out_hw(H, W, kh, kw, stride, padding):
    return ((H + 2 * padding[0] - kh) // stride[0] + 1,
            (W + 2 * padding[1] - kw) // stride[1] + 1)


def qconv2d_nhwc(x, wq, scales, biases, O, kh, kw, stride=(1, 1), padding=(0, 0),
                 groups=1, group_size=64, bits=4, out=None, stream=None):
    """x [B,H,W,C] -> y [B,OH,OW,O]; wq from quantize_conv_weight."""
    B, H, W, C = x.shape
    OH, OW = conv_out_hw(H, W, kh, kw, stride, padding)
    if out is None:
        out = torch.empty((B, OH, OW, O), dtype=x.dtype, device=x.device)
    _check(lib().qconv2d_nhwc(_ptr(x), B, H, W, C, _ptr(wq), _ptr(scales), _ptr(biases),
                              O, kh, kw, stride[0], stride[1], padding[0], padding[1],
                              groups, _dt(x.dtype), group_size, bits, _ptr(out),
                              _stream(stream)))
    return out


def conv_weight_matrix(w, group_size):
    """Conv weight [O, kh, kw, C/groups] -> [O, K_pad]: flattened in (dy, dx, c)
    order and zero-padded to a multiple of the group size (layout only)."""
    O = w.shape[0]
    K_true = w[0].numel()
    K_pad = -(-K_true // group_size) * group_size
    wm = torch.zeros((O, K_pad), dtype=w.dtype, device=w.device)
    wm[:, :K_true] = w.reshape(O, K_true)
    return wm


def quantize_conv_weight(w, group_size=64, bits=4, stream=None):
    """Quantize a conv weight [O, kh, kw, C/groups] for qconv2d_nhwc."""
    return qmm_quantize(conv_weight_matrix(w, group_size), group_size, bits, stream=stream)


def crossover_m(bits, dtype=torch.float16):
    return lib().qmm_crossover_m(bits, _dt(dtype))
