"""Moving seeded storage words between numpy and device tensors (plumbing for
the tests, the smoke check and the benchmark; no method arithmetic)."""
import numpy as np
import torch

TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def to_dev(words, dt, dev="cuda"):
    """Storage words (numpy) -> torch tensor of the element type on dev."""
    if dt == "f32":
        return torch.from_numpy(np.ascontiguousarray(words, np.float32)).to(dev)
    t = torch.from_numpy(np.ascontiguousarray(words).view(np.int16))
    return t.view(TORCH_DT[dt]).to(dev)


def from_dev(t):
    """torch tensor -> storage words (numpy)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def bytes_to_words_dev(wq_bytes, dev="cuda"):
    """Packed row bytes [..., K*bits/8] -> int32 tensor [..., K*bits/32]."""
    b = np.ascontiguousarray(wq_bytes, np.uint8)
    return torch.from_numpy(b.view(np.int32).copy()).to(dev)


def from_dev_i32(t):
    return t.detach().cpu().contiguous().numpy().view(np.uint32)


def words_dev_to_bytes(wq):
    return from_dev_i32(wq).view(np.uint8).reshape(wq.shape[0], -1)
