"""Exact attention written out from its definition, in float64 (test infrastructure only).

Definition (FlashAttention: IO-aware exact attention, opening section, and
"Flash Attention and the Online-Softmax Trick", §1): for one (batch, head)
slice with queries q [Nq, d], keys k [Nk, d] and values v [Nk, dv],

    S = scale * q k^T                       (Nq x Nk, materialised)
    S[i, j] = -inf where masked             (causal: key j > query i)
    m_i = max_j S_ij,  l_i = sum_j exp(S_ij - m_i)
    P = exp(S - m) / l                      (rows sum to one)
    O = P v,           LSE_i = m_i + ln l_i (natural log)

The log-sum-exp output is the statistic FlashAttention-2 keeps for the backward
pass ("FlashAttention-2 and -3" page, section "Fewer non-matmul FLOPs").

Readings taken where the pages are silent (each is listed in the design notes):
* ``scale`` multiplies q k^T before the softmax; LSE is the natural log of the
  sum of exponentials of the *scaled* scores.
* causal keeps key j for query i when j <= i, counted from the top-left
  corner (the PyTorch ``is_causal`` alignment the "Using it, the real way"
  section describes). For the square shapes used here top-left and
  bottom-right coincide.
* a row with every key masked has O = 0 and LSE = -inf.
* rectangular causal (Nq queries, Nk keys, Nq != Nk) is aligned bottom-right, the
  flash-attn convention the same section recommends for chunked prefill and decoding
  with a cache: query i stands at key position i + Nk - Nq and sees keys up to it. A
  sliding window (the same section: kernels support sliding windows natively) follows
  flash-attn's (left, right) form around that position: key j is visible when
  i + Nk - Nq - left <= j <= i + Nk - Nq + right, a negative bound meaning none and
  causal meaning right = 0. With a 64-token causal window each query sees itself and the
  64 keys before it.
* grouped-query attention ("FlashAttention-2 and -3", "Using it, the real way":
  fewer key-value heads than query heads, shared in groups without copying K
  and V): with H query heads and Hkv key-value heads, the query heads form Hkv
  consecutive groups of H / Hkv and group j reads key-value head j. Hkv = H is
  ordinary multi-head attention. In the backward a shared key-value head gets the sum of
  its group's gradients.
* the backward pass is the exact gradient of O(q, k, v) for an upstream dO,
  derived by calculus from the definition above; the pages state only that it
  recomputes the tiles from the saved LSE.
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _causal_keep(nq: int, nk: int) -> np.ndarray:
    """Boolean [nq, nk] mask: key j is visible to query i when j <= i (top-left)."""
    return np.arange(nk)[None, :] <= np.arange(nq)[:, None]


def kv_head(h: int, H: int, Hkv: int) -> int:
    """Key-value head read by query head h: query heads come in Hkv consecutive groups of
    H / Hkv, group j sharing key-value head j (grouped-query attention)."""
    if Hkv <= 0 or H % Hkv != 0:
        raise ValueError(f"{H} query heads cannot be grouped over {Hkv} key-value heads")
    return h // (H // Hkv)


def band_keep(nq: int, nk: int, causal: bool, window_left: int = -1, window_right: int = -1) -> np.ndarray:
    """Boolean [nq, nk] visibility with the bottom-right alignment: query i stands at key
    position i + nk - nq; key j is visible when it lies within `window_left` keys before and
    `window_right` keys after that position (a negative bound: unlimited; causal: right 0)."""
    pos = np.arange(nq)[:, None] + (nk - nq)
    j = np.arange(nk)[None, :]
    keep = np.ones((nq, nk), dtype=bool)
    right = 0 if causal else window_right
    if right >= 0:
        keep &= j <= pos + right
    if window_left >= 0:
        keep &= j >= pos - window_left
    return keep


def attention_head(q, k, v, scale, causal=False, return_p=False, keep=None):
    """Forward attention for one (batch, head) slice; returns (O, LSE[, P]).
    ``causal`` applies the top-left mask; ``keep`` (boolean [Nq, Nk]) any other."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    S = float(scale) * (q @ k.T)
    if causal:
        S = np.where(_causal_keep(q.shape[0], k.shape[0]), S, -np.inf)
    if keep is not None:
        S = np.where(keep, S, -np.inf)
    m = S.max(axis=1) if S.shape[1] else np.full(S.shape[0], -np.inf)
    has_key = np.isfinite(m)
    m_ref = np.where(has_key, m, 0.0)
    E = np.exp(S - m_ref[:, None])          # exp(-inf) = 0 on masked entries
    l = E.sum(axis=1)
    P = E / np.where(l > 0, l, 1.0)[:, None]
    O = P @ v
    lse = np.where(l > 0, m_ref + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    if return_p:
        return O, lse, P
    return O, lse


def attn_fwd(q, k, v, scale, causal=False):
    """Dense forward. q: [B, N, H, d]; k, v: [B, N, Hkv, d] (Hkv divides H; Hkv = H for
    multi-head attention). Returns O [B, N, H, d], LSE [B, H, N]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, N, H, _ = q.shape
    Hkv = k.shape[2]
    O = np.empty(q.shape[:3] + (v.shape[3],))
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            j = kv_head(h, H, Hkv)
            O[b, :, h, :], lse[b, h, :] = attention_head(q[b, :, h], k[b, :, j], v[b, :, j],
                                                         scale, causal)
    return O, lse


def attn_fwd_window(q, k, v, scale, causal=False, window_left=-1, window_right=-1):
    """Forward with Nq queries against Nk keys, bottom-right aligned, with an optional
    sliding window (see band_keep). q: [B, Nq, H, d]; k, v: [B, Nk, Hkv, d].
    Returns O [B, Nq, H, d], LSE [B, H, Nq]; a query with no visible key gets O = 0,
    LSE = -inf."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Nq, H, _ = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    keep = band_keep(Nq, Nk, causal, window_left, window_right)
    O = np.empty(q.shape[:3] + (v.shape[3],))
    lse = np.empty((B, H, Nq))
    for b in range(B):
        for h in range(H):
            j = kv_head(h, H, Hkv)
            O[b, :, h, :], lse[b, h, :] = attention_head(q[b, :, h], k[b, :, j], v[b, :, j], scale, keep=keep)
    return O, lse


def attn_fwd_varlen(q, k, v, cu_seqlens, scale, causal=False):
    """Packed variable-length forward ("Variable-length batches without padding").

    q: [total_tokens, H, d], k, v: [total_tokens, Hkv, d] (grouped as in attn_fwd);
    sequence s occupies rows cu_seqlens[s] to
    cu_seqlens[s+1]. Attention never crosses a sequence boundary (block-diagonal
    document mask); causal is counted within each sequence.
    Returns O [total_tokens, H, d] and LSE [H, total_tokens].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu.ndim != 1 or cu[0] != 0 or np.any(np.diff(cu) < 0) or cu[-1] != q.shape[0]:
        raise ValueError("cu_seqlens must start at 0, be nondecreasing and end at total_tokens")
    T, H, _ = q.shape
    Hkv = k.shape[1]
    O = np.zeros((T, H, v.shape[2]))
    lse = np.full((H, T), -np.inf)
    for s in range(len(cu) - 1):
        a, e = int(cu[s]), int(cu[s + 1])
        if e == a:
            continue
        for h in range(H):
            j = kv_head(h, H, Hkv)
            O[a:e, h, :], lse[h, a:e] = attention_head(q[a:e, h], k[a:e, j], v[a:e, j],
                                                       scale, causal)
    return O, lse


def attn_bwd_head(q, k, v, do, scale, causal=False):
    """Exact gradients for one slice. Returns dict with dq, dk, dv, o, lse, delta.

    With P the forward probabilities and dO the upstream gradient of O:
        dV = P^T dO
        dP = dO v^T
        D_i = sum_j P_ij dP_ij          (equals sum_c dO_ic O_ic)
        dS = P * (dP - D)               (softmax Jacobian, row by row)
        dQ = scale * dS k
        dK = scale * dS^T q
    Masked entries have P = 0 and contribute nothing.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    o, lse, P = attention_head(q, k, v, scale, causal, return_p=True)
    dv = P.T @ do
    dP = do @ v.T
    delta = (P * dP).sum(axis=1)
    dS = P * (dP - delta[:, None])
    dq = float(scale) * (dS @ k)
    dk = float(scale) * (dS.T @ q)
    return {"dq": dq, "dk": dk, "dv": dv, "o": o, "lse": lse, "delta": delta}


def attn_bwd(q, k, v, do, scale, causal=False):
    """Dense backward. q, do: [B, N, H, d]; k, v: [B, N, Hkv, d] (grouped as in attn_fwd).
    Returns (dq [B, N, H, d], dk, dv [B, N, Hkv, d]) in float64. A key-value head shared by
    a group of query heads receives the sum of the group's gradients (the chain rule through
    every use of it)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, N, H, _ = q.shape
    Hkv = k.shape[2]
    dq, dk, dv = np.empty(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    for b in range(B):
        for h in range(H):
            j = kv_head(h, H, Hkv)
            g = attn_bwd_head(q[b, :, h], k[b, :, j], v[b, :, j], do[b, :, h], scale, causal)
            dq[b, :, h] = g["dq"]
            dk[b, :, j] += g["dk"]
            dv[b, :, j] += g["dv"]
    return dq, dk, dv


def attn_decode_slice(q_vec, k_rows, v_rows, scale):
    """One decode step for one (batch, head): a single query against L cached keys.

    The newest token sees every cached key, so there is no mask. Not split into
    chunks: the split-and-merge of Flash-Decoding is checked separately.
    Returns (o [dv], lse scalar).
    """
    o, lse = attention_head(_f64(q_vec)[None, :], k_rows, v_rows, scale, causal=False)
    return o[0], float(lse[0])


def attn_decode(q, k_cache, v_cache, scale):
    """Decode for a batch. q [B, H, d]; caches [B, L, Hkv, d] (grouped as in attn_fwd).
    Returns O [B, H, d], LSE [B, H]."""
    q, kc, vc = _f64(q), _f64(k_cache), _f64(v_cache)
    B, H, _ = q.shape
    Hkv = kc.shape[2]
    O = np.empty((B, H, vc.shape[3]))
    lse = np.empty((B, H))
    for b in range(B):
        for h in range(H):
            j = kv_head(h, H, Hkv)
            O[b, h], lse[b, h] = attn_decode_slice(q[b, h], kc[b, :, j], vc[b, :, j], scale)
    return O, lse


def attn_decode_paged(q, k_pages, v_pages, block_table, seqlens, scale):
    """Decode against a paged cache ("FlashAttention-2 and -3", "Paged KV caches, a preview
    of serving"): the cache is a pool of fixed-size pages [num_pages, P, H, d] and row b of
    the block table maps sequence b's logical blocks (tokens 0..P-1, P..2P-1, ...) to
    physical pages. Token t of sequence b is page block_table[b, t // P], slot t % P.
    Exactly seqlens[b] tokens are gathered (the slots past the end of the last page are not
    part of the sequence), then the contiguous decode runs. An empty sequence gives O = 0,
    LSE = -inf (a row with no visible key). q [B, H, d]; pages [num_pages, P, Hkv, d]
    (grouped as in attn_fwd); returns O [B, H, d], LSE [B, H]."""
    q, kp, vp = _f64(q), _f64(k_pages), _f64(v_pages)
    P = kp.shape[1]
    B, H, _ = q.shape
    Hkv = kp.shape[2]
    O = np.zeros((B, H, vp.shape[3]))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        L = int(seqlens[b])
        if L == 0:
            continue
        t = np.arange(L)
        pg, slot = block_table[b, t // P], t % P
        k_rows, v_rows = kp[pg, slot], vp[pg, slot]  # [L, H, d]
        for h in range(H):
            j = kv_head(h, H, Hkv)
            O[b, h], lse[b, h] = attn_decode_slice(q[b, h], k_rows[:, j], v_rows[:, j], scale)
    return O, lse
