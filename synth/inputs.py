"""Seeded, per-slice synthetic tensors.

Every (tensor, batch, head) slice is drawn from its own numpy generator seeded
with ``[seed, tensor_id, b, h]``, as i.i.d. standard normals in float32. For
bf16 workloads the float32 samples are rounded once to bf16 with
round-to-nearest-even and kept as uint16 bit patterns; widening those bits back
to float32 (a 16-bit shift) is exact, so the oracle and the GPU see the same
values. Per-slice seeding lets a checker regenerate any single slice of a large
tensor without holding the whole tensor.

Layouts: dense tensors are [B, N, H, d]; packed variable-length tensors are
[total_tokens, H, d]; a decode query is [B, H, d].
"""
from __future__ import annotations

import numpy as np

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_DO = 0, 1, 2, 3


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return uint16 bits.

    Inputs are finite samples; NaN/Inf handling is not needed here.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding_bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding_bias) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_slice(seed: int, tensor_id: int, b: int, h: int, shape) -> np.ndarray:
    """float32 N(0,1) samples for one (tensor, batch, head) slice."""
    rng = np.random.default_rng([seed, tensor_id, b, h])
    return rng.standard_normal(shape, dtype=np.float32)


def _finish(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return bf16_bits_from_f32(x32)
    raise ValueError(f"unknown dtype {dtype!r}")


def bnhd_tensor(seed, tensor_id, B, N, H, d, dtype="bf16", head_scale=None):
    """A [B, N, H, d] tensor built slice by slice.

    ``head_scale`` optionally maps a head index to a multiplier applied to the
    float32 samples before rounding (used to stress the online-softmax rescaling
    with larger scores on some heads).
    Returns float32 values (dtype "f32") or uint16 bf16 bits (dtype "bf16").
    """
    out = np.empty((B, N, H, d), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            x = normal_slice(seed, tensor_id, b, h, (N, d))
            if head_scale is not None:
                x = x * np.float32(head_scale(h))
            out[b, :, h, :] = x
    return _finish(out, dtype)


def varlen_lengths(seed: int, n: int, lo: int, hi: int) -> np.ndarray:
    """``n`` integer lengths drawn uniformly from [lo, hi] inclusive."""
    rng = np.random.default_rng([seed, 99])
    return rng.integers(lo, hi + 1, n).astype(np.int64)


def cu_seqlens_from_lengths(lengths) -> np.ndarray:
    """Cumulative offsets [0, L1, L1+L2, ...] as int32 of length len(lengths)+1."""
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    if cu[-1] > np.iinfo(np.int32).max:
        raise ValueError("total tokens exceed int32")
    return cu.astype(np.int32)


def varlen_tensor(seed, tensor_id, lengths, H, d, dtype="bf16", head_scale=None):
    """Packed [total_tokens, H, d] tensor; sequence s and head h form one slice."""
    cu = cu_seqlens_from_lengths(lengths)
    out = np.empty((int(cu[-1]), H, d), dtype=np.float32)
    for s, L in enumerate(lengths):
        for h in range(H):
            x = normal_slice(seed, tensor_id, s, h, (int(L), d))
            if head_scale is not None:
                x = x * np.float32(head_scale(h))
            out[cu[s]:cu[s + 1], h, :] = x
    return _finish(out, dtype)


def decode_query(seed, B, H, d, dtype="bf16"):
    """A [B, H, d] single-token query, one slice per (b, h)."""
    out = np.empty((B, H, d), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            out[b, h, :] = normal_slice(seed, TENSOR_Q, b, h, (d,))
    return _finish(out, dtype)


def paged_layout(seed, seqlens, page_size, extra_pages=0):
    """Block table for a paged cache: sequence b owns ceil(L_b / page_size) pages, listed in
    row b of a [B, max_pages] int32 table; the physical pages are a seeded permutation of
    the pool (plus `extra_pages` never referenced). Unused table entries point at random
    valid pages. Returns (block_table, num_pages)."""
    seqlens = [int(x) for x in seqlens]
    need = [(L + page_size - 1) // page_size for L in seqlens]
    max_pages = max(1, max(need) if need else 1)
    num_pages = max(1, sum(need) + int(extra_pages))
    rng = np.random.default_rng([seed, 77])
    perm = rng.permutation(num_pages).astype(np.int32)
    table = rng.integers(0, num_pages, size=(len(seqlens), max_pages)).astype(np.int32)
    pos = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[pos:pos + n]
        pos += n
    return table, num_pages


def paged_tensor(seed, tensor_id, seqlens, block_table, num_pages, page_size, H, d, dtype="bf16"):
    """Page pool [num_pages, page_size, H, d]: token t of sequence b (slice (b, h) of the
    seeded normal draw, as in a contiguous cache) sits in page block_table[b, t // page_size]
    at slot t % page_size. Every other slot holds seeded noise of its own."""
    rng = np.random.default_rng([seed, tensor_id, 991])
    pool = rng.standard_normal((num_pages, page_size, H, d)).astype(np.float32) * np.float32(3.0)
    for b, L in enumerate(seqlens):
        L = int(L)
        for h in range(H):
            x = normal_slice(seed, tensor_id, b, h, (L, d))
            t = np.arange(L)
            pool[block_table[b, t // page_size], t % page_size, h, :] = x
    return _finish(pool, dtype)


def rademacher_signs(seed: int, d: int) -> np.ndarray:
    """d independent +-1 values (float32), the random diagonal of an incoherence rotation."""
    rng = np.random.default_rng([seed, 4711])
    return np.where(rng.integers(0, 2, d) == 1, 1.0, -1.0).astype(np.float32)


def outlier_tensor(seed, tensor_id, B, N, H, d, dtype="bf16", rate=1e-3, outlier_std=10.0):
    """A [B, N, H, d] tensor whose entries are N(0, 1) plus, on a `rate` fraction of entries
    chosen independently, an extra N(0, outlier_std^2) term (the FP8 outlier test:
    N(0, 100) on 0.1% of entries)."""
    out = np.empty((B, N, H, d), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            x = normal_slice(seed, tensor_id, b, h, (N, d))
            rng = np.random.default_rng([seed, tensor_id, b, h, 313])
            hit = rng.random((N, d)) < rate
            x = x + np.where(hit, rng.standard_normal((N, d)).astype(np.float32) * np.float32(outlier_std), 0)
            out[b, :, h, :] = x
    return _finish(out, dtype)
