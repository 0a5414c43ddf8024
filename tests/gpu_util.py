"""Helpers for the GPU tests: move seeded numpy inputs to the device and results back.

bf16 tensors travel as their uint16 bit patterns, so the device sees exactly the values
the oracle reads (bf16 -> fp32 widening is exact)."""
from __future__ import annotations

import numpy as np


def torch():
    import torch as _t
    return _t


def dev_bf16(bits: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(t.bfloat16)


def dev_f32(x: np.ndarray):
    return torch().from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")


def dev_i32(x: np.ndarray):
    return torch().from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to("cuda")


def host(t) -> np.ndarray:
    """Device tensor -> float64 numpy (exact for bf16 and fp32)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def max_abs(a, b) -> float:
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    return float(np.max(np.abs(a - b), initial=0.0))


def bits_to_f64(bits: np.ndarray) -> np.ndarray:
    from synth import f32_from_bf16_bits
    return f32_from_bf16_bits(bits).astype(np.float64)
