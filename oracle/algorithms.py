"""The pages' algorithms, step by step in float64 (test infrastructure only).

These exist to pin ``oracle.attention`` and the claims the pages make about
it. None of them is compared with the GPU.
"""
from __future__ import annotations

import math

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def tiled_online_attention_head(q, k, v, scale, causal=False, block_cols=64,
                                stale_threshold=None):
    """Tiled attention with the online softmax, for one (batch, head) slice.

    Follows "FlashAttention: IO-aware exact attention", sections "Tile
    decomposition" and "Online softmax", and the unnormalised accumulator of
    "FlashAttention-2 and -3", section "Fewer non-matmul FLOPs":

    for each key/value block j (block_cols keys):
        S_j     = scale * q K_j^T            (masked entries -inf)
        m~      = row max of S_j
        m_new   = max(m, m~)
        alpha   = exp(m - m_new)             (change of pivot)
        P_j     = exp(S_j - m_new)
        l       = alpha * l + row sum of P_j
        O~      = alpha * O~ + P_j V_j
    then O = O~ / l and LSE = m + ln l.

    ``stale_threshold`` (optional) keeps the old pivot unless the block maximum
    exceeds it by more than the threshold — the conditional rescaling of
    "And on Blackwell": any pivot shared by l and O~ gives the same result.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    nq, nk = q.shape[0], k.shape[0]
    m = np.full(nq, -np.inf)
    l = np.zeros(nq)
    acc = np.zeros((nq, v.shape[1]))
    rows = np.arange(nq)[:, None]
    for j0 in range(0, nk, block_cols):
        j1 = min(j0 + block_cols, nk)
        S = float(scale) * (q @ k[j0:j1].T)
        if causal:
            S = np.where(np.arange(j0, j1)[None, :] <= rows, S, -np.inf)
        m_blk = S.max(axis=1)
        m_new = np.maximum(m, m_blk)
        if stale_threshold is not None:
            keep_old = np.isfinite(m) & (m_blk <= m + stale_threshold)
            m_new = np.where(keep_old, m, m_new)
        m_ref = np.where(np.isfinite(m_new), m_new, 0.0)
        alpha = np.where(np.isfinite(m), np.exp(m - m_ref), 0.0)
        P = np.exp(S - m_ref[:, None])
        l = alpha * l + P.sum(axis=1)
        acc = alpha[:, None] * acc + P @ v[j0:j1]
        m = m_new
    out = acc / np.where(l > 0, l, 1.0)[:, None]
    lse = np.where(l > 0, np.where(np.isfinite(m), m, 0.0) + np.log(np.where(l > 0, l, 1.0)),
                   -np.inf)
    return out, lse


def softmax_two_pass(x):
    """Row softmax in two passes ("Online softmax" section): first the max, then the sum."""
    x = _f64(x)
    m = x.max(axis=-1, keepdims=True)          # pass 1
    e = np.exp(x - m)                          # pass 2
    return e / e.sum(axis=-1, keepdims=True)


def softmax_online(x, chunk):
    """Row softmax in one streaming pass over chunks, carrying (running max, running sum).

    "Flash Attention and the Online-Softmax Trick", §3: when a chunk raises the
    maximum, the old sum is multiplied by exp(m_old - m_new).
    """
    x = _f64(x)
    m = np.full(x.shape[:-1], -np.inf)
    s = np.zeros(x.shape[:-1])
    n = x.shape[-1]
    for c0 in range(0, n, chunk):
        xc = x[..., c0:c0 + chunk]
        m_new = np.maximum(m, xc.max(axis=-1))
        s = s * np.exp(m - m_new) + np.exp(xc - m_new[..., None]).sum(axis=-1)
        m = m_new
    return np.exp(x - m[..., None]) / s[..., None]


def decode_chunk_partials(q_vec, k_rows, v_rows, scale, n_chunks):
    """Flash-Decoding's split ("Decoding needs a different split"): cut the L keys
    into ``n_chunks`` contiguous chunks; each yields its normalised output and
    its log-sum-exp. An empty chunk yields (0, -inf)."""
    q_vec, k_rows, v_rows = _f64(q_vec), _f64(k_rows), _f64(v_rows)
    L = k_rows.shape[0]
    csize = -(-L // n_chunks)
    outs, lses = [], []
    for c in range(n_chunks):
        a, e = c * csize, min((c + 1) * csize, L)
        if a >= e:
            outs.append(np.zeros(v_rows.shape[1]))
            lses.append(-np.inf)
            continue
        s = float(scale) * (k_rows[a:e] @ q_vec)
        m = s.max()
        w = np.exp(s - m)
        outs.append(w @ v_rows[a:e] / w.sum())
        lses.append(m + math.log(w.sum()))
    return np.array(outs), np.array(lses)


def merge_partials(outs, lses):
    """Merge chunk partials with log-sum-exp weights: each chunk's output is weighted by
    its softmax mass, lse = log sum_c exp(lse_c), O = sum_c exp(lse_c - lse) O_c."""
    outs, lses = _f64(outs), _f64(lses)
    M = lses.max()
    w = np.exp(lses - M)                        # empty chunks have weight 0
    total = w.sum()
    return (w[:, None] * outs).sum(axis=0) / total, M + math.log(total)


def brute_force_attention(q, k, v, scale, causal=False):
    """Scalar pure-Python attention for tiny inputs (math.exp, math.fsum).

    Written independently of the numpy definitions: for every query i and key j
    the score is scale * sum_c q[i][c] k[j][c]; visible keys are j <= i when
    causal. Returns (O as nested lists, LSE list).
    """
    q = [[float(x) for x in row] for row in q]
    k = [[float(x) for x in row] for row in k]
    v = [[float(x) for x in row] for row in v]
    O, LSE = [], []
    for i, qi in enumerate(q):
        keys = [j for j in range(len(k)) if (not causal or j <= i)]
        if not keys:
            O.append([0.0] * len(v[0]))
            LSE.append(-math.inf)
            continue
        s = {j: scale * math.fsum(a * b for a, b in zip(qi, k[j])) for j in keys}
        mx = max(s.values())
        e = {j: math.exp(s[j] - mx) for j in keys}
        tot = math.fsum(e.values())
        O.append([math.fsum(e[j] * v[j][c] for j in keys) / tot for c in range(len(v[0]))])
        LSE.append(mx + math.log(tot))
    return O, LSE
