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
    QMM_E_ALIGN, QMM_E_LAUNCH, QMM_E_ARG = range(9)
STATUS_NAMES = ["QMM_OK", "QMM_E_NULL", "QMM_E_BITS", "QMM_E_GROUP",
                "QMM_E_SHAPE", "QMM_E_DTYPE", "QMM_E_ALIGN", "QMM_E_LAUNCH", "QMM_E_ARG"]
# kernels of the affine products (qmm_route, force_kernel)
KERNEL_NONE, KERNEL_GEMV, KERNEL_MFMA_GEMV, KERNEL_TILE = range(4)
EXPORTS = ["qmm_quantize", "qmm_dequantize", "qmm_t", "qmv", "qmm_n", "qconv2d_nhwc",
           "qmm_gather_qmv", "qmm_gather_qmm", "qmm_t_batched",
           "qmm_fp_quantize", "qmm_fp_dequantize", "qmm_fp_qmv", "qmm_fp_t", "qmm_fp_n", "qmm_fp_gather_qmv",
           "qmm_affine_pack", "qmv_affine_packed", "qmm_t_affine_packed",
           "qmm_crossover_m", "qmm_route", "qmm_force_kernel", "qmm_last_error"]

_DT = {torch.float16: 0, torch.bfloat16: 1, torch.float32: 2}

_lib = None


class QmmError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else status}: {msg}")
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
        L.qmm_t_affine_packed.argtypes = L.qmv_affine_packed.argtypes
        L.qmm_t_batched.argtypes = [vp, vp, vp, vp, i64, i64, i32, i64, i64, i64, i32, i32,
                                    vp, vp]
        L.qmm_fp_quantize.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp, vp]
        L.qmm_fp_dequantize.argtypes = [vp, vp, i32, i64, i64, i32, i32, vp, vp]
        L.qmm_fp_qmv.argtypes = [vp, vp, vp, i32, i64, i64, i64, i32, i32, vp, vp]
        L.qmm_fp_t.argtypes = L.qmm_fp_qmv.argtypes
        L.qmm_fp_n.argtypes = L.qmm_fp_qmv.argtypes
        L.qmm_fp_gather_qmv.argtypes = [vp, i64, vp, vp, vp, i64, vp, i64, i32, i64, i64, i64,
                                        i32, i32, vp, vp]
        for f in ("qmm_quantize", "qmm_dequantize", "qmm_t", "qmv", "qmm_n", "qconv2d_nhwc",
                  "qmm_gather_qmv", "qmm_gather_qmm", "qmm_t_batched", "qmm_fp_quantize",
                  "qmm_fp_dequantize", "qmm_fp_qmv", "qmm_fp_t", "qmm_fp_n", "qmm_fp_gather_qmv",
                  "qmm_affine_pack", "qmv_affine_packed", "qmm_t_affine_packed"):
            getattr(L, f).restype = i32
        L.qmm_crossover_m.argtypes = [i32, i32, i32, i64, i64]
        L.qmm_crossover_m.restype = i64
        L.qmm_route.argtypes = [i32, i32, i32, i64, i64, i64]
        L.qmm_route.restype = i32
        L.qmm_force_kernel.argtypes = [i32]
        L.qmm_force_kernel.restype = i32
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
    elif stream.device.index != torch.cuda.current_device():
        raise ValueError(f"stream is on {stream.device} but the current device is "
                         f"cuda:{torch.cuda.current_device()}")
    return ctypes.c_void_p(stream.cuda_stream)


def _dt(dtype):
    if dtype not in _DT:
        raise QmmError(QMM_E_DTYPE, f"unsupported dtype {dtype}")
    return _DT[dtype]


def packed_words(K, bits):
    return K * bits // 32


# ---------------------------------------------------------------- validation
# The C ABI takes plain pointers and sizes, so it cannot see a tensor's
# extent: the binding checks every tensor's shape, element type, layout and
# device against the sizes it passes before anything is launched ("Add the
# 3bit packed qmm_t", ops.cpp extract_quantized_matmul_dims: the packed
# width, scales and biases of one shape, the inner dimension of x). Sizes the
# library itself rejects (bits, group size, K not a multiple of the group)
# are left to its status codes.

_BITS = (2, 3, 4, 5, 6, 8)
_GS = (32, 64, 128)


def _sizes_ok(K, group_size, bits):
    """True when the packed shapes below are defined (else the library rejects
    the call with its own status)."""
    return bits in _BITS and group_size in _GS and K >= 1 and K % group_size == 0


def _check_tensor(t, name, shape=None, dtype=None, dims=None):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dimensions, got shape {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_device(*named):
    """Every given tensor on one ROCm device."""
    dev = None
    for name, t in named:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a ROCm device, got {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")
    # the library launches on the current device (its memory, its static
    # scratch, its streams)
    if dev is not None and dev.index is not None and dev.index != torch.cuda.current_device():
        raise ValueError(f"the tensors are on {dev} but the current device is "
                         f"cuda:{torch.cuda.current_device()}; call under torch.cuda.device({dev})")


def _check_indices(t, name, B):
    if t is None:
        return
    _check_tensor(t, name, shape=(B,), dtype=torch.int32)


def qmm_quantize(w, group_size=64, bits=4, out=None, stream=None):
    """w [rows, K] -> (wq int32 [rows, K*bits/32], scales, biases [rows, K/gs])."""
    _check_tensor(w, "w", dims=2)
    rows, K = w.shape
    if out is None:
        G = max(K // group_size, 1) if group_size > 0 else 1
        out = (torch.empty((rows, max(packed_words(K, bits), 1)), dtype=torch.int32, device=w.device),
               torch.empty((rows, G), dtype=w.dtype, device=w.device),
               torch.empty((rows, G), dtype=w.dtype, device=w.device))
    wq, s, b = out
    if _sizes_ok(K, group_size, bits):
        _check_tensor(wq, "wq", (rows, packed_words(K, bits)), torch.int32)
        _check_tensor(s, "scales", (rows, K // group_size), w.dtype)
        _check_tensor(b, "biases", (rows, K // group_size), w.dtype)
    _check_device(("w", w), ("wq", wq), ("scales", s), ("biases", b))
    _check(lib().qmm_quantize(_ptr(w), _dt(w.dtype), rows, K, group_size, bits,
                              _ptr(wq), _ptr(s), _ptr(b), _stream(stream)))
    return wq, s, b


def qmm_dequantize(wq, scales, biases, group_size=64, bits=4, out=None, stream=None):
    _check_tensor(wq, "wq", dims=2, dtype=torch.int32)
    rows = wq.shape[0]
    K = wq.shape[1] * 32 // bits if bits in _BITS else 0
    if out is None:
        out = torch.empty((rows, K), dtype=scales.dtype, device=wq.device)
    if _sizes_ok(K, group_size, bits):
        _check_tensor(scales, "scales", (rows, K // group_size))
        _check_tensor(biases, "biases", (rows, K // group_size), scales.dtype)
        _check_tensor(out, "out", (rows, K), scales.dtype)
    _check_device(("wq", wq), ("scales", scales), ("biases", biases), ("out", out))
    _check(lib().qmm_dequantize(_ptr(wq), _ptr(scales), _ptr(biases), _dt(scales.dtype),
                                rows, K, group_size, bits, _ptr(out), _stream(stream)))
    return out


def _check_mm(x, wq, scales, biases, out, lead, M, N, K, group_size, bits, nw=None):
    """x [*lead, M, K]; wq [*nw, N, K*bits/32]; scales, biases [*nw, N, K/gs];
    out [*lead, M, N]; one element type for x, scales, biases and out."""
    nw = lead if nw is None else nw
    if _sizes_ok(K, group_size, bits):
        _check_tensor(wq, "wq", (*nw, N, packed_words(K, bits)), torch.int32)
        _check_tensor(scales, "scales", (*nw, N, K // group_size), x.dtype)
        _check_tensor(biases, "biases", (*nw, N, K // group_size), x.dtype)
    _check_tensor(out, "out", (*lead, M, N), x.dtype)
    _check_device(("x", x), ("wq", wq), ("scales", scales), ("biases", biases), ("out", out))


def _matmul(fn, x, wq, scales, biases, group_size, bits, out, stream):
    _check_tensor(x, "x", dims=2)
    _check_tensor(wq, "wq", dims=2)
    M, K = x.shape
    N = wq.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    _check_mm(x, wq, scales, biases, out, (), M, N, K, group_size, bits)
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
    _check_tensor(x, "x", dims=2)
    _check_tensor(wq, "wq", dims=2, dtype=torch.int32)
    M, K = x.shape
    if wq.shape[0] != K:
        raise ValueError("qmm_n: W must have K rows")
    N = wq.shape[1] * 32 // bits if bits in _BITS else 0
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    if _sizes_ok(N, group_size, bits):
        _check_tensor(scales, "scales", (K, N // group_size), x.dtype)
        _check_tensor(biases, "biases", (K, N // group_size), x.dtype)
    _check_tensor(out, "out", (M, N), x.dtype)
    _check_device(("x", x), ("wq", wq), ("scales", scales), ("biases", biases), ("out", out))
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
    _check_tensor(x, "x", dims=3)
    _check_tensor(wq, "wq", dims=3)
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
    _check_indices(lhs_indices, "lhs_indices", B)
    _check_indices(rhs_indices, "rhs_indices", B)
    if out is None:
        out = torch.empty((B, M, N), dtype=x.dtype, device=x.device)
    _check_mm(x, wq, scales, biases, out, (B,), M, N, K, group_size, bits, nw=(E,))
    _check_device(("x", x), ("lhs_indices", lhs_indices), ("rhs_indices", rhs_indices))
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
    _check_tensor(x, "x", dims=3)
    _check_tensor(wq, "wq", dims=3)
    B, M, K = x.shape
    E, N = wq.shape[0], wq.shape[1]
    if out is None:
        out = torch.empty((B, M, N), dtype=x.dtype, device=x.device)
    _check_mm(x, wq, scales, biases, out, (B,), M, N, K, group_size, bits, nw=(E,))
    _check(lib().qmm_t_batched(_ptr(x), _ptr(wq), _ptr(scales), _ptr(biases), B, E,
                               _dt(x.dtype), M, N, K, group_size, bits, _ptr(out),
                               _stream(stream)))
    return out


def fp_quantize(w, group_size=32, bits=4, stream=None):
    """Floating-point mode ((4, 32) mxfp4, (4, 16) nvfp4, (8, 32) mxfp8):
    w [rows, K] -> (wq int32 [rows, K*bits/32], scales uint8 [rows, K/gs])."""
    _check_tensor(w, "w", dims=2)
    _check_device(("w", w))
    rows, K = w.shape
    wq = torch.empty((rows, max(K * bits // 32, 1)), dtype=torch.int32, device=w.device)
    sc = torch.empty((rows, max(K // group_size, 1)), dtype=torch.uint8, device=w.device)
    _check(lib().qmm_fp_quantize(_ptr(w), _dt(w.dtype), rows, K, group_size, bits, _ptr(wq),
                                 _ptr(sc), _stream(stream)))
    return wq, sc


def _fp_sizes_ok(K, group_size, bits):
    return (bits, group_size) in ((4, 32), (4, 16), (8, 32)) and K >= 1 and K % group_size == 0


def fp_dequantize(wq, scales, dtype=torch.float16, group_size=32, bits=4, stream=None):
    _check_tensor(wq, "wq", dims=2, dtype=torch.int32)
    rows = wq.shape[0]
    K = wq.shape[1] * 32 // bits if bits in (4, 8) else 0
    if _fp_sizes_ok(K, group_size, bits):
        _check_tensor(scales, "scales", (rows, K // group_size), torch.uint8)
    _check_device(("wq", wq), ("scales", scales))
    out = torch.empty((rows, K), dtype=dtype, device=wq.device)
    _check(lib().qmm_fp_dequantize(_ptr(wq), _ptr(scales), _dt(dtype), rows, K, group_size,
                                   bits, _ptr(out), _stream(stream)))
    return out


def fp_qmv(x, wq, scales, group_size=32, bits=4, out=None, stream=None, _fn="qmm_fp_qmv"):
    """y [M,N] = x [M,K] . dequant(W)^T for a floating-point mode (the GEMV)."""
    _check_tensor(x, "x", dims=2)
    _check_tensor(wq, "wq", dims=2, dtype=torch.int32)
    M, K = x.shape
    N = wq.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    if _fp_sizes_ok(K, group_size, bits):
        _check_tensor(wq, "wq", (N, K * bits // 32), torch.int32)
        _check_tensor(scales, "scales", (N, K // group_size), torch.uint8)
    _check_tensor(out, "out", (M, N), x.dtype)
    _check_device(("x", x), ("wq", wq), ("scales", scales), ("out", out))
    _check(getattr(lib(), _fn)(_ptr(x), _ptr(wq), _ptr(scales), _dt(x.dtype), M, N, K,
                               group_size, bits, _ptr(out), _stream(stream)))
    return out


def fp_qmm_t(x, wq, scales, group_size=32, bits=4, out=None, stream=None):
    """Same as fp_qmv for any M: the GEMV for a few rows, the MFMA tile kernel
    beyond."""
    return fp_qmv(x, wq, scales, group_size, bits, out, stream, _fn="qmm_fp_t")


def fp_qmm_n(x, wq, scales, group_size=32, bits=4, out=None, stream=None):
    """y [M,N] = x [M,K] . dequant(W) for a floating-point mode, W [K, N]
    quantized along N: wq [K, N*bits/32], scales uint8 [K, N/gs]."""
    _check_tensor(x, "x", dims=2)
    _check_tensor(wq, "wq", dims=2, dtype=torch.int32)
    M, K = x.shape
    if wq.shape[0] != K:
        raise ValueError(f"fp_qmm_n: wq has {wq.shape[0]} rows, x has K = {K}")
    N = wq.shape[1] * 32 // bits if bits in (4, 8) else 0
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    if N >= group_size and group_size in (16, 32) and N % group_size == 0:
        _check_tensor(scales, "scales", (K, N // group_size), torch.uint8)
    _check_tensor(out, "out", (M, N), x.dtype)
    _check_device(("x", x), ("wq", wq), ("scales", scales), ("out", out))
    _check(lib().qmm_fp_n(_ptr(x), _ptr(wq), _ptr(scales), _dt(x.dtype), M, N, K, group_size,
                          bits, _ptr(out), _stream(stream)))
    return out


def fp_gather_qmv(x, wq, scales, lhs_indices=None, rhs_indices=None, group_size=32, bits=4,
                  out=None, stream=None):
    """y[z] = x[lhs_indices[z]] . dequant(W[rhs_indices[z]])^T in a floating-point
    mode: x [Bx, M, K]; wq [E, N, K*bits/32]; scales uint8 [E, N, K/gs]."""
    _check_tensor(x, "x", dims=3)
    _check_tensor(wq, "wq", dims=3, dtype=torch.int32)
    Bx, M, K = x.shape
    E, N = wq.shape[0], wq.shape[1]
    B = (lhs_indices.numel() if lhs_indices is not None else
         rhs_indices.numel() if rhs_indices is not None else Bx)
    for t in (lhs_indices, rhs_indices):
        if t is not None and (t.dtype != torch.int32 or t.numel() != B):
            raise ValueError("indices must be int32 tensors of one length")
    _check_indices(lhs_indices, "lhs_indices", B)
    _check_indices(rhs_indices, "rhs_indices", B)
    if out is None:
        out = torch.empty((B, M, N), dtype=x.dtype, device=x.device)
    if _fp_sizes_ok(K, group_size, bits):
        _check_tensor(wq, "wq", (E, N, K * bits // 32), torch.int32)
        _check_tensor(scales, "scales", (E, N, K // group_size), torch.uint8)
    _check_tensor(out, "out", (B, M, N), x.dtype)
    _check_device(("x", x), ("wq", wq), ("scales", scales), ("out", out),
                  ("lhs_indices", lhs_indices), ("rhs_indices", rhs_indices))
    _check(lib().qmm_fp_gather_qmv(_ptr(x), Bx, _ptr(lhs_indices), _ptr(wq), _ptr(scales), E,
                                   _ptr(rhs_indices), B, _dt(x.dtype), M, N, K, group_size, bits,
                                   _ptr(out), _stream(stream)))
    return out


def affine_pack(wq, scales, biases, group_size=64, bits=4, stream=None):
    """Affine-packed layout of (wq [N, K*bits/32], scales, biases [N, K/gs]):
    returns (wq_packed [N/4, 4*K*bits/32] for bits 2/4/8, else wq itself;
    sb_packed [N/RP, K/gs*2*RP])."""
    _check_tensor(wq, "wq", dims=2, dtype=torch.int32)
    N = wq.shape[0]
    K = wq.shape[1] * 32 // bits if bits in _BITS else 0
    pow2 = (bits & (bits - 1)) == 0
    rp = 4 if pow2 else 2
    if _sizes_ok(K, group_size, bits):
        _check_tensor(scales, "scales", (N, K // group_size))
        _check_tensor(biases, "biases", (N, K // group_size), scales.dtype)
    _check_device(("wq", wq), ("scales", scales), ("biases", biases))
    wp = torch.empty((N // rp, rp * wq.shape[1]), dtype=torch.int32,
                     device=wq.device) if pow2 else None
    sbp = torch.empty((N // rp, scales.shape[1] * 2 * rp), dtype=scales.dtype, device=wq.device)
    _check(lib().qmm_affine_pack(_ptr(wq), _ptr(scales), _ptr(biases), _dt(scales.dtype), N, K,
                                 group_size, bits, _ptr(wp), _ptr(sbp), _stream(stream)))
    return (wp if pow2 else wq), sbp


def qmv_affine_packed(x, wq_packed, sb_packed, N, group_size=64, bits=4, out=None, stream=None,
                      _fn="qmv_affine_packed"):
    """y [M,N] = x [M,K] . dequant(W)^T from the affine-packed layout (GEMV)."""
    _check_tensor(x, "x", dims=2)
    M, K = x.shape
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    if _sizes_ok(K, group_size, bits):
        rp = 4 if (bits & (bits - 1)) == 0 else 2
        if N % rp == 0:
            _check_tensor(wq_packed, "wq_packed", (N // rp, rp * packed_words(K, bits))
                          if rp == 4 else (N, packed_words(K, bits)), torch.int32)
            _check_tensor(sb_packed, "sb_packed", (N // rp, K // group_size * 2 * rp), x.dtype)
    _check_tensor(out, "out", (M, N), x.dtype)
    _check_device(("x", x), ("wq_packed", wq_packed), ("sb_packed", sb_packed), ("out", out))
    _check(getattr(lib(), _fn)(_ptr(x), _ptr(wq_packed), _ptr(sb_packed), _dt(x.dtype), M, N,
                               K, group_size, bits, _ptr(out), _stream(stream)))
    return out


def qmm_t_affine_packed(x, wq_packed, sb_packed, N, group_size=64, bits=4, out=None,
                        stream=None):
    """Same as qmv_affine_packed for any M (the MFMA tile kernel beyond a few
    rows)."""
    return qmv_affine_packed(x, wq_packed, sb_packed, N, group_size, bits, out, stream,
                             _fn="qmm_t_affine_packed")


def conv_out_hw(H, W, kh, kw, stride, padding):
    return ((H + 2 * padding[0] - kh) // stride[0] + 1,
            (W + 2 * padding[1] - kw) // stride[1] + 1)


def qconv2d_nhwc(x, wq, scales, biases, O, kh, kw, stride=(1, 1), padding=(0, 0),
                 groups=1, group_size=64, bits=4, out=None, stream=None):
    """x [B,H,W,C] -> y [B,OH,OW,O]; wq from quantize_conv_weight."""
    _check_tensor(x, "x", dims=4)
    B, H, W, C = x.shape
    OH, OW = conv_out_hw(H, W, kh, kw, stride, padding)
    if out is None:
        out = torch.empty((B, OH, OW, O), dtype=x.dtype, device=x.device)
    if groups >= 1 and C % groups == 0 and bits in _BITS and group_size in _GS:
        k_true = kh * kw * (C // groups)
        k_pad = -(-k_true // group_size) * group_size
        _check_tensor(wq, "wq", (O, packed_words(k_pad, bits)), torch.int32)
        _check_tensor(scales, "scales", (O, k_pad // group_size), x.dtype)
        _check_tensor(biases, "biases", (O, k_pad // group_size), x.dtype)
    _check_tensor(out, "out", (B, OH, OW, O), x.dtype)
    _check_device(("x", x), ("wq", wq), ("scales", scales), ("biases", biases), ("out", out))
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


def crossover_m(bits, dtype=torch.float16, N=4096, K=4096, group_size=64):
    """Smallest M at which qmm_t runs the MFMA tile kernel for an [N, K] layer."""
    return lib().qmm_crossover_m(_dt(dtype), bits, group_size, N, K)


def route(M, N, K, bits=4, dtype=torch.float16, group_size=64):
    """Kernel qmm_t runs for the shape: KERNEL_GEMV, KERNEL_MFMA_GEMV or KERNEL_TILE."""
    return lib().qmm_route(_dt(dtype), bits, group_size, M, N, K)


def force_kernel(kernel):
    """Measurement: run `kernel` wherever the shape fits it (KERNEL_NONE: automatic)."""
    _check(lib().qmm_force_kernel(kernel))
