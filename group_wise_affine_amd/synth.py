"""Seeded synthetic inputs, shared by the tests, the smoke check and the bench.

This module only draws numbers and stores them in the element type; it holds
none of the quantization or matmul arithmetic, so both the HIP path and the
oracle can take their inputs from it.

Recipe: numpy PCG64 ``default_rng(seed)``, ``standard_normal`` in float32,
times sigma (one float32 multiply), then rounded to nearest-even into the
storage type (f16 through numpy, bf16 through torch). Arrays are returned as
storage words: uint16 for f16/bf16, float32 for f32.
"""
import numpy as np

DT_NAMES = ("f16", "bf16", "f32")


def to_words(a, dt):
    """float32 array -> storage words of ``dt`` (round to nearest even)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dt == "f32":
        return a
    if dt == "f16":
        return a.astype(np.float16).view(np.uint16)
    if dt == "bf16":
        import torch
        t = torch.from_numpy(a).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(dt)


def words_to_f32(w, dt):
    """Storage words -> float32 (exact widening)."""
    if dt == "f32":
        return np.asarray(w, np.float32)
    if dt == "f16":
        return np.asarray(w, np.uint16).view(np.float16).astype(np.float32)
    if dt == "bf16":
        return (np.asarray(w, np.uint16).astype(np.uint32) << 16).view(np.float32)
    raise ValueError(dt)


def normal(shape, seed, sigma=1.0, dt="f16"):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        a = a * np.float32(sigma)
    return to_words(a, dt)


def mixed_magnitude(shape, seed, lo=1e-5, hi=1e2, block=16, dt="f16"):
    """Normal values whose magnitude alternates between ``lo`` and ``hi`` in
    blocks of ``block`` consecutive elements along the last axis (one float32
    multiply per element, then rounded into the storage type)."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(size=shape, dtype=np.float32)
    k = np.arange(shape[-1])
    mag = np.where((k // block) % 2 == 0, np.float32(lo), np.float32(hi)).astype(np.float32)
    return to_words(a * mag, dt)


def structured_rows(rows, K, group_size, seed, dt="f16", sigma=1.0):
    """Weight rows whose groups cover the quantizer's special cases: all-zero
    groups, constant groups, integer ramps, groups holding exact zeros among
    normal values, sign-symmetric extremes (|min| == |max|), a single
    outlier, tiny magnitudes, and plain normal groups. ``sigma`` scales every
    row (one float32 multiply) so that they sit among weights of that
    spread."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(size=(rows, K), dtype=np.float32)
    G = K // group_size
    kinds = 9
    for r in range(rows):
        for g in range(G):
            sl = slice(g * group_size, (g + 1) * group_size)
            kind = (r * G + g) % kinds
            if kind == 0:
                a[r, sl] = 0.0
            elif kind == 1:
                a[r, sl] = np.float32(rng.standard_normal())
            elif kind == 2:
                a[r, sl] = (np.arange(group_size) % 16).astype(np.float32)
            elif kind == 3:
                a[r, sl] = (np.arange(group_size) % 16).astype(np.float32) - 8
            elif kind == 4:
                idx = rng.choice(group_size, size=group_size // 4, replace=False)
                a[r, g * group_size + idx] = 0.0
            elif kind == 5:
                m = np.float32(abs(rng.standard_normal()) + 0.5)
                a[r, g * group_size] = m
                a[r, g * group_size + 1] = -m
                a[r, g * group_size + 2:(g + 1) * group_size] = np.clip(
                    a[r, g * group_size + 2:(g + 1) * group_size], -m * 0.9, m * 0.9)
            elif kind == 6:
                a[r, g * group_size + group_size // 2] = np.float32(40.0)
            elif kind == 7:
                a[r, sl] = a[r, sl] * np.float32(1e-3)
            # kind 8: plain normal
    if sigma != 1.0:
        a = a * np.float32(sigma)
    return to_words(a, dt)
