"""CPU checks of the Python binding's argument validation: a packed weight,
scale, bias or output tensor whose shape, element type, layout or device does
not match the sizes passed to the C ABI raises ValueError before anything is
launched (the C ABI sees only pointers and sizes, so an undersized buffer
would otherwise be read or written past its end). The tensors here live on
the CPU, which the binding also rejects, so no call can reach a GPU."""
import pytest
import torch

from group_wise_affine_amd import qmm as Q

F16, I32, U8 = torch.float16, torch.int32, torch.uint8


def z(*shape, dtype=F16):
    return torch.zeros(shape, dtype=dtype)


def _mm_args(M=4, N=8, K=128, gs=64, bits=4):
    return (z(M, K), z(N, K * bits // 32, dtype=I32), z(N, K // gs), z(N, K // gs))


@pytest.mark.parametrize("fn", [Q.qmm_t, Q.qmv])
def test_matmul_shape_mismatches(fn):
    x, wq, s, b = _mm_args()
    bad = [
        (x, z(8, 15, dtype=I32), s, b),          # packed width != K*bits/32
        (x, wq, z(8, 3), b),                     # scales not [N, K/gs]
        (x, wq, s, z(7, 2)),                     # biases not [N, K/gs]
        (x, wq.to(torch.int64), s, b),           # packed words not int32
        (x, wq, s.to(torch.bfloat16), b),        # scales of another dtype
        (z(4, 128, 1), wq, s, b),                # x not 2-D
        (x, wq, s, b.t().contiguous().t()),      # non-contiguous view
    ]
    for args in bad:
        with pytest.raises(ValueError):
            fn(*args, group_size=64, bits=4)
    with pytest.raises(ValueError):              # bits does not match the packed width
        fn(x, wq, s, b, group_size=64, bits=8)
    with pytest.raises(ValueError):              # group size does not match the scales
        fn(x, wq, s, b, group_size=32, bits=4)
    with pytest.raises(ValueError):              # short output
        fn(x, wq, s, b, group_size=64, bits=4, out=z(4, 7))
    with pytest.raises(ValueError):              # output of another dtype
        fn(x, wq, s, b, group_size=64, bits=4, out=z(4, 8, dtype=torch.float32))


def test_matmul_requires_device_tensors():
    with pytest.raises(ValueError, match="ROCm device"):
        Q.qmm_t(*_mm_args(), group_size=64, bits=4)


def test_quantize_dequantize_shapes():
    w = z(8, 128)
    with pytest.raises(ValueError):
        Q.qmm_quantize(w, 64, 4, out=(z(8, 15, dtype=I32), z(8, 2), z(8, 2)))
    with pytest.raises(ValueError):
        Q.qmm_quantize(w, 64, 4, out=(z(8, 16, dtype=I32), z(8, 3), z(8, 2)))
    with pytest.raises(ValueError):
        Q.qmm_dequantize(z(8, 16, dtype=I32), z(8, 2), z(8, 2), 64, 4, out=z(8, 127))
    with pytest.raises(ValueError):
        Q.qmm_dequantize(z(8, 16, dtype=I32), z(8, 4), z(8, 2), 64, 4)


def test_gather_and_batched_shapes():
    x = z(2, 1, 128)
    wq, s = z(3, 8, 16, dtype=I32), z(3, 8, 2)
    idx = torch.zeros(4, dtype=I32)
    with pytest.raises(ValueError):              # scales of another expert count
        Q.gather_qmv(x, wq, z(2, 8, 2), s, idx, idx, 64, 4)
    with pytest.raises(ValueError):              # output not [B, M, N]
        Q.gather_qmv(x, wq, s, s, idx, idx, 64, 4, out=z(3, 1, 8))
    with pytest.raises(ValueError):              # indices of another dtype
        Q.gather_qmm(x, wq, s, s, idx.long(), None, 64, 4)
    with pytest.raises(ValueError):              # packed width
        Q.qmm_t_batched(x, z(2, 8, 15, dtype=I32), z(2, 8, 2), z(2, 8, 2), 64, 4)
    with pytest.raises(ValueError):
        Q.qmm_t_batched(x, z(2, 8, 16, dtype=I32), z(2, 8, 2), z(2, 8, 2), 64, 4,
                        out=z(2, 1, 9))


def test_qmm_n_shapes():
    x = z(2, 64)
    with pytest.raises(ValueError):              # scales not [K, N/gs]
        Q.qmm_n(x, z(64, 16, dtype=I32), z(64, 1), z(64, 2), 64, 4)
    with pytest.raises(ValueError):
        Q.qmm_n(x, z(64, 16, dtype=I32), z(64, 2), z(64, 2), 64, 4, out=z(2, 64))


def test_fp_and_packed_shapes():
    x = z(1, 64)
    with pytest.raises(ValueError):              # mxfp4 scale bytes of the wrong shape
        Q.fp_qmv(x, z(8, 8, dtype=I32), z(8, 1, dtype=U8), 32, 4)
    with pytest.raises(ValueError):              # scale bytes not uint8
        Q.fp_qmv(x, z(8, 8, dtype=I32), z(8, 2), 32, 4)
    with pytest.raises(ValueError):
        Q.fp_gather_qmv(z(1, 1, 64), z(2, 8, 8, dtype=I32), z(2, 8, 2, dtype=U8), None,
                        torch.zeros(3, dtype=I32), 32, 4, out=z(3, 1, 7))
    with pytest.raises(ValueError):              # packed words of 4 rows per block
        Q.qmv_affine_packed(z(1, 128), z(8, 16, dtype=I32), z(2, 16), 8, 64, 4)
    with pytest.raises(ValueError):
        Q.qmv_affine_packed(z(1, 128), z(2, 64, dtype=I32), z(2, 15), 8, 64, 4)


def test_conv_shapes():
    x = z(1, 6, 6, 32)
    k_pad = 320                                   # 3*3*32 = 288 -> 320 at gs 64
    good = (z(16, k_pad * 4 // 32, dtype=I32), z(16, k_pad // 64), z(16, k_pad // 64))
    with pytest.raises(ValueError):               # unpadded packed width
        Q.qconv2d_nhwc(x, z(16, 288 * 4 // 32, dtype=I32), good[1], good[2], 16, 3, 3,
                       (1, 1), (1, 1), 1, 64, 4)
    with pytest.raises(ValueError):               # output of the wrong spatial size
        Q.qconv2d_nhwc(x, *good, 16, 3, 3, (1, 1), (1, 1), 1, 64, 4, out=z(1, 4, 4, 16))
    with pytest.raises(ValueError, match="ROCm device"):
        Q.qconv2d_nhwc(x, *good, 16, 3, 3, (1, 1), (1, 1), 1, 64, 4)
