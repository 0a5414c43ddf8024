"""MI355X-native exact attention: tiled online-softmax HIP kernels behind a C ABI.

Python entry points with the same names as the C calls. They only marshal
arguments (device pointers, sizes, the current HIP stream); every step of the
computation runs in the HIP kernels of ``libfa.so``. PyTorch provides device
memory and streams. Tensors must be contiguous device tensors:

    fwd(q, k, v, scale=None, causal=False) -> (o, lse)          q [B, N, H, d], k,v [B, N, Hkv, d]
    fwd_window(q, k, v, scale=None, causal=False, window=(-1, -1)) -> (o, lse)
                                                 q [B, Nq, H, d], k,v [B, Nk, Hkv, d]
    fwd_fp8(q, k, v, signs=None, scale=None, causal=False) -> (o, lse)   FP8 e4m3 compute
    fwd_varlen(q, k, v, cu_seqlens, max_seqlen, ...) -> (o, lse) q [T, H, d], k,v [T, Hkv, d]
    bwd(q, k, v, o, lse, do, scale=None, causal=False) -> (dq, dk, dv)   fp32 grads (dk, dv: Hkv heads)
    decode(q, k_cache, v_cache, scale=None, num_splits=64) -> (o, lse)   q [B, H, d]
    decode_paged(q, k_pages, v_pages, block_table, seqlens, ...) -> (o, lse)

``scale`` defaults to 1/sqrt(d). K and V may have fewer heads than Q (Hkv dividing H,
grouped-query attention: query head h reads key-value head h // (H // Hkv)); the number
is taken from their shapes (the backward returns dK, dV with Hkv heads).
"""
from __future__ import annotations

import math

from ._clib import (  # noqa: F401
    FAError, FA_DTYPE_BF16, FA_DTYPE_F32, check, lib, strerror,
)

__all__ = ["fwd", "fwd_window", "fwd_fp8", "fwd_varlen", "check_cu_seqlens", "bwd", "decode", "decode_noalloc", "decode_paged", "FAError", "lib"]


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return FA_DTYPE_BF16
    if t.dtype == torch.float32:
        return FA_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _require(tensors, names):
    for t, n in zip(tensors, names):
        if not t.is_cuda:
            raise ValueError(f"{n} must be a GPU tensor (no CPU path exists)")
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")


def _stream(device):
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _scale(scale, d):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def fwd(q, k, v, scale=None, causal=False, out=None):
    """Dense forward. Returns O (q's dtype, [B, N, H, d]) and fp32 LSE [B, H, N].
    ``out=(o, lse)`` writes into preallocated tensors of those shapes."""
    torch = _torch()
    _require((q, k, v), ("q", "k", "v"))
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape or k.shape[:2] != q.shape[:2] or k.shape[3] != q.shape[3]:
        raise ValueError("q must be [B, N, H, d] and k, v [B, N, Hkv, d]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    B, N, H, d = q.shape
    Hkv = k.shape[2]
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        _require((o, lse), ("o", "lse"))
        if o.shape != q.shape or o.dtype != q.dtype or lse.shape != (B, H, N) or lse.dtype != torch.float32:
            raise ValueError("out must be (o [B, N, H, d] like q, lse fp32 [B, H, N])")
    st = lib().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                      B, H, Hkv, N, d, _scale(scale, d), int(bool(causal)), _dtype_code(q), _stream(q.device))
    check(st, "fa_fwd")
    return o, lse


def fwd_window(q, k, v, scale=None, causal=False, window=(-1, -1), out=None):
    """Forward with Nq queries against Nk keys, bottom-right aligned, and an optional
    sliding window ``(left, right)`` around each query's key position i + Nk - Nq (-1: no
    bound; causal fixes right = 0). q [B, Nq, H, d], k, v [B, Nk, Hkv, d].
    Returns O [B, Nq, H, d] and fp32 LSE [B, H, Nq]."""
    torch = _torch()
    _require((q, k, v), ("q", "k", "v"))
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape or k.shape[0] != q.shape[0] or k.shape[3] != q.shape[3]:
        raise ValueError("q must be [B, Nq, H, d] and k, v [B, Nk, Hkv, d]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    B, Nq, H, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    left, right = (int(w) for w in window)
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        _require((o, lse), ("o", "lse"))
        if o.shape != q.shape or o.dtype != q.dtype or lse.shape != (B, H, Nq) or lse.dtype != torch.float32:
            raise ValueError("out must be (o [B, Nq, H, d] like q, lse fp32 [B, H, Nq])")
    st = lib().fa_fwd_window(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                             B, H, Hkv, Nq, Nk, d, _scale(scale, d), int(bool(causal)), left, right,
                             _dtype_code(q), _stream(q.device))
    check(st, "fa_fwd_window")
    return o, lse


def fwd_fp8(q, k, v, signs=None, scale=None, causal=False, out=None, workspace=None):
    """Forward computed in FP8 e4m3 with block quantization, and incoherent processing when
    ``signs`` (a device fp32 [d] tensor of +-1) is given. q [B, N, H, d], k, v [B, N, Hkv, d],
    all bf16. Returns O [B, N, H, d] bf16 and fp32 LSE [B, H, N]."""
    torch = _torch()
    _require((q, k, v), ("q", "k", "v"))
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape or k.shape[:2] != q.shape[:2] or k.shape[3] != q.shape[3]:
        raise ValueError("q must be [B, N, H, d] and k, v [B, N, Hkv, d]")
    if q.dtype != torch.bfloat16 or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("fwd_fp8 takes bfloat16 q, k, v")
    B, N, H, d = q.shape
    Hkv = k.shape[2]
    if signs is not None:
        _require((signs,), ("signs",))
        if signs.dtype != torch.float32 or signs.shape != (d,):
            raise ValueError("signs must be a float32 [d] tensor")
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        _require((o, lse), ("o", "lse"))
        if o.shape != q.shape or o.dtype != q.dtype or lse.shape != (B, H, N) or lse.dtype != torch.float32:
            raise ValueError("out must be (o [B, N, H, d] like q, lse fp32 [B, H, N])")
    nbytes = lib().fa_fwd_fp8_workspace_bytes(B, H, Hkv, N, d)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    st = lib().fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), None if signs is None else signs.data_ptr(),
                          o.data_ptr(), lse.data_ptr(), B, H, Hkv, N, d, _scale(scale, d), int(bool(causal)),
                          workspace.data_ptr(), workspace.numel(), _stream(q.device))
    check(st, "fa_fwd_fp8")
    return o, lse


def check_cu_seqlens(cu, total_tokens, max_seqlen=None):
    """Validate packed-sequence offsets on the host (a 1-D integer sequence or array):
    cu[0] = 0, nondecreasing, cu[-1] = total_tokens, and no sequence longer than max_seqlen
    (when given). Returns the longest sequence length; raises ValueError otherwise."""
    import numpy as np
    cu = np.asarray(cu, dtype=np.int64).reshape(-1)
    if cu.size < 1 or cu[0] != 0:
        raise ValueError("cu_seqlens must start with 0")
    lengths = np.diff(cu)
    if lengths.size and lengths.min() < 0:
        raise ValueError("cu_seqlens must be nondecreasing")
    if cu[-1] != total_tokens:
        raise ValueError(f"cu_seqlens must end at total_tokens ({total_tokens}), got {int(cu[-1])}")
    longest = int(lengths.max()) if lengths.size else 0
    if max_seqlen is not None and longest > max_seqlen:
        raise ValueError(f"a sequence of {longest} tokens exceeds max_seqlen = {max_seqlen}")
    return longest


def fwd_varlen(q, k, v, cu_seqlens, max_seqlen=None, scale=None, causal=False, validate=True):
    """Packed forward over sequences laid end to end. q: [T, H, d], k, v: [T, Hkv, d];
    cu_seqlens: int32 offsets [num_seqs + 1], a device tensor or host data (uploaded here);
    max_seqlen: the longest sequence length (host int; computed from the offsets if None).
    With validate (the default) the offsets are checked on the host first (check_cu_seqlens;
    a device tensor is copied back for it, which waits for the stream). The kernels clamp the
    offsets into the tensor and compute every row whatever max_seqlen says, so validate=False
    is memory-safe; rows outside every [cu[s], cu[s+1]) range are then left unwritten.
    Returns O [T, H, d] and fp32 LSE [H, T]."""
    torch = _torch()
    _require((q, k, v), ("q", "k", "v"))
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape or k.shape[0] != q.shape[0] or k.shape[2] != q.shape[2]:
        raise ValueError("q must be [total_tokens, H, d] and k, v [total_tokens, Hkv, d]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    T, H, d = q.shape
    on_device = isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.is_cuda
    if validate or max_seqlen is None:
        host_cu = cu_seqlens.cpu() if isinstance(cu_seqlens, torch.Tensor) else cu_seqlens
        longest = check_cu_seqlens(host_cu, T, max_seqlen)
        if max_seqlen is None:
            max_seqlen = max(longest, 1 if T > 0 else 0)
    if on_device:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
            raise TypeError("cu_seqlens must be a 1-D int32 tensor")
        _require((cu_seqlens,), ("cu_seqlens",))
    else:
        cu_seqlens = torch.as_tensor(cu_seqlens, dtype=torch.int32).reshape(-1).to(q.device)
    o = torch.empty_like(q)
    lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
    st = lib().fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                             cu_seqlens.data_ptr(), cu_seqlens.numel() - 1, T, int(max_seqlen), H, k.shape[1], d,
                             _scale(scale, d), int(bool(causal)), _dtype_code(q), _stream(q.device))
    check(st, "fa_fwd_varlen")
    return o, lse


def bwd(q, k, v, o, lse, do, scale=None, causal=False, out=None, workspace=None):
    """Backward from the forward's O and LSE. Returns fp32 dq [B, N, H, d] and dk, dv
    [B, N, Hkv, d]. ``out=(dq, dk, dv)`` and ``workspace`` may be preallocated."""
    torch = _torch()
    _require((q, k, v, o, lse, do), ("q", "k", "v", "o", "lse", "do"))
    B, N, H, d = q.shape
    for t, n in ((o, "o"), (do, "do")):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{n} must match q in shape and dtype")
    if k.dim() != 4 or k.shape[:2] != q.shape[:2] or k.shape[3] != d or v.shape != k.shape:
        raise ValueError("k, v must be [B, N, Hkv, d] matching q")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("k, v must match q in dtype")
    Hkv = k.shape[2]
    if lse.shape != (B, H, N) or lse.dtype != torch.float32:
        raise ValueError("lse must be fp32 [B, H, N]")
    if out is None:
        dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        dk = torch.empty(k.shape, dtype=torch.float32, device=q.device)
        dv = torch.empty_like(dk)
    else:
        dq, dk, dv = out
        _require((dq, dk, dv), ("dq", "dk", "dv"))
        if dq.shape != q.shape or dk.shape != k.shape or dv.shape != k.shape or any(
                t.dtype != torch.float32 for t in (dq, dk, dv)):
            raise ValueError("out gradients must be fp32, dq shaped like q and dk, dv like k")
    nbytes = lib().fa_bwd_workspace_bytes(B, H, N)
    ws = workspace
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    st = lib().fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                      dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Hkv, N, d, _scale(scale, d),
                      int(bool(causal)), _dtype_code(q), ws.data_ptr(), ws.numel(), _stream(q.device))
    check(st, "fa_bwd")
    return dq, dk, dv


def decode(q, k_cache, v_cache, scale=None, num_splits=64, workspace=None, out=None):
    """Single-token decode. q [B, H, d]; caches [B, L, Hkv, d]. Returns O [B, H, d], LSE [B, H]."""
    torch = _torch()
    _require((q, k_cache, v_cache), ("q", "k_cache", "v_cache"))
    B, H, d = q.shape
    if k_cache.dim() != 4:
        raise ValueError("caches must be [B, L, Hkv, d]")
    L, Hkv = k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape != (B, L, Hkv, d) or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [B, L, Hkv, d] matching q")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q and the caches must share a dtype")
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        _require((o, lse), ("o", "lse"))
        if o.shape != q.shape or o.dtype != q.dtype or lse.shape != (B, H) or lse.dtype != torch.float32:
            raise ValueError("out must be (o [B, H, d] like q, lse fp32 [B, H])")
    nbytes = lib().fa_decode_workspace_bytes(B, H, d, num_splits)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    st = lib().fa_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), o.data_ptr(), lse.data_ptr(),
                         B, H, Hkv, L, d, _scale(scale, d), num_splits, _dtype_code(q),
                         workspace.data_ptr(), workspace.numel(), _stream(q.device))
    check(st, "fa_decode")
    return o, lse


def decode_noalloc(q, k_cache, v_cache, out, scale=None, num_splits=64):
    """decode() without a workspace and without allocating: the chunk partials go to the
    library's fixed scratch (fa_decode_noalloc). `out` = (o [B, H, d] like q, lse fp32
    [B, H]) is required. Calls that overlap on one GPU race on the scratch."""
    torch = _torch()
    _require((q, k_cache, v_cache), ("q", "k_cache", "v_cache"))
    B, H, d = q.shape
    if k_cache.dim() != 4:
        raise ValueError("caches must be [B, L, Hkv, d]")
    L, Hkv = k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape != (B, L, Hkv, d) or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [B, L, Hkv, d] matching q")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q and the caches must share a dtype")
    o, lse = out
    _require((o, lse), ("o", "lse"))
    if o.shape != q.shape or o.dtype != q.dtype or lse.shape != (B, H) or lse.dtype != torch.float32:
        raise ValueError("out must be (o [B, H, d] like q, lse fp32 [B, H])")
    st = lib().fa_decode_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                 B, H, Hkv, L, d, _scale(scale, d), num_splits, _dtype_code(q), _stream(q.device))
    check(st, "fa_decode_noalloc")
    return o, lse


def decode_paged(q, k_pages, v_pages, block_table, seqlens, scale=None, num_splits=64, workspace=None, out=None):
    """Single-token decode over a paged cache. q [B, H, d]; pages [num_pages, page_size, Hkv, d];
    block_table int32 [B, max_pages]; seqlens int32 [B]. Returns O [B, H, d], LSE [B, H]."""
    torch = _torch()
    _require((q, k_pages, v_pages, block_table, seqlens), ("q", "k_pages", "v_pages", "block_table", "seqlens"))
    B, H, d = q.shape
    if k_pages.dim() != 4:
        raise ValueError("pages must be [num_pages, page_size, Hkv, d]")
    num_pages, page_size, Hkv = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    if k_pages.shape != (num_pages, page_size, Hkv, d) or v_pages.shape != k_pages.shape:
        raise ValueError("pages must be [num_pages, page_size, Hkv, d] matching q")
    if k_pages.dtype != q.dtype or v_pages.dtype != q.dtype:
        raise TypeError("q and the pages must share a dtype")
    if block_table.dtype != torch.int32 or seqlens.dtype != torch.int32:
        raise TypeError("block_table and seqlens must be int32")
    if block_table.dim() != 2 or block_table.shape[0] != B or seqlens.shape != (B,):
        raise ValueError("block_table must be [B, max_pages] and seqlens [B]")
    max_pages = block_table.shape[1]
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        _require((o, lse), ("o", "lse"))
        if o.shape != q.shape or o.dtype != q.dtype or lse.shape != (B, H) or lse.dtype != torch.float32:
            raise ValueError("out must be (o [B, H, d] like q, lse fp32 [B, H])")
    nbytes = lib().fa_decode_workspace_bytes(B, H, d, num_splits)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    st = lib().fa_decode_paged(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), block_table.data_ptr(),
                               seqlens.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, Hkv, d, page_size, num_pages,
                               max_pages, _scale(scale, d), num_splits, _dtype_code(q),
                               workspace.data_ptr(), workspace.numel(), _stream(q.device))
    check(st, "fa_decode_paged")
    return o, lse
