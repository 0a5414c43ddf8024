"""Pins of grouped-query attention in the oracle ("FlashAttention-2 and -3", "Using it, the
real way": fewer key-value heads than query heads, shared in groups): with H query heads
and Hkv key-value heads, query head h reads key-value head h // (H / Hkv).

The closed forms below are built so that every key-value head gives a different, known
answer: a mapping that sends a query head to the wrong key-value head (interleaved groups,
say) fails them. A planted mistake of that kind is checked to be caught."""
import math

import numpy as np
import pytest

import oracle
import synth


def heads_values(Hkv, d):
    """A distinct constant value vector per key-value head."""
    return np.stack([(j + 1.0) * (1.0 + np.arange(d) / d) for j in range(Hkv)])  # [Hkv, d]


def rand(seed, *shape):
    return np.random.default_rng([seed, 5150]).standard_normal(shape)


@pytest.mark.parametrize("H,Hkv", [(8, 2), (6, 3), (4, 1), (4, 4)])
@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_identify_the_group(H, Hkv, causal):
    """V constant per key-value head: every output row of query head h is that head's
    constant, whatever the scores are (the softmax weights sum to one)."""
    B, N, d = 2, 7, 8
    c = heads_values(Hkv, d)
    q, k = rand(1, B, N, H, d), rand(2, B, N, Hkv, d)
    v = np.broadcast_to(c[None, None], (B, N, Hkv, d)).copy()
    O, _ = oracle.attn_fwd(q, k, v, 0.5, causal)
    for h in range(H):
        np.testing.assert_allclose(O[:, :, h], np.broadcast_to(c[h * Hkv // H], (B, N, d)), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_closed_form(causal):
    """K[n, j] = u_j for every position: each visible key scores scale * q_i . u_j, so
    LSE_i = scale * q_i . u_j + ln(#visible) and O_i is the mean of the visible values."""
    B, N, H, Hkv, d, scale = 1, 6, 6, 2, 4, 0.7
    u = rand(3, Hkv, d)
    q, v = rand(4, B, N, H, d), rand(5, B, N, Hkv, d)
    k = np.broadcast_to(u[None, None], (B, N, Hkv, d)).copy()
    O, lse = oracle.attn_fwd(q, k, v, scale, causal)
    count = np.arange(1, N + 1) if causal else np.full(N, N)
    for h in range(H):
        j = h // (H // Hkv)
        expect_lse = scale * q[0, :, h] @ u[j] + np.log(count)
        np.testing.assert_allclose(lse[0, h], expect_lse, rtol=0, atol=1e-12)
        mean = np.cumsum(v[0, :, j], axis=0) / count[:, None] if causal else np.broadcast_to(v[0, :, j].mean(0), (N, d))
        np.testing.assert_allclose(O[0, :, h], mean, rtol=0, atol=1e-12)


def test_equals_multi_head_on_repeated_keys_and_values():
    """Sharing a key-value head equals giving each query head its own copy of it: expand K
    and V by repeating each head H / Hkv times along the head axis."""
    B, N, H, Hkv, d = 2, 9, 8, 2, 16
    q, k, v = rand(6, B, N, H, d), rand(7, B, N, Hkv, d), rand(8, B, N, Hkv, d)
    g = H // Hkv
    for causal in (False, True):
        O, lse = oracle.attn_fwd(q, k, v, 0.25, causal)
        O2, lse2 = oracle.attn_fwd(q, np.repeat(k, g, axis=2), np.repeat(v, g, axis=2), 0.25, causal)
        np.testing.assert_array_equal(O, O2)
        np.testing.assert_array_equal(lse, lse2)


def test_varlen_and_decode_share_the_grouping():
    H, Hkv, d = 6, 3, 8
    c = heads_values(Hkv, d)
    # packed forward: two sequences
    T = 11
    q, k = rand(9, T, H, d), rand(10, T, Hkv, d)
    v = np.broadcast_to(c[None], (T, Hkv, d)).copy()
    O, _ = oracle.attn_fwd_varlen(q, k, v, [0, 4, 11], 0.3, causal=True)
    for h in range(H):
        np.testing.assert_allclose(O[:, h], np.broadcast_to(c[h // 2], (T, d)), rtol=0, atol=1e-12)
    # contiguous decode
    B, L = 2, 5
    qd, kc = rand(11, B, H, d), rand(12, B, L, Hkv, d)
    vc = np.broadcast_to(c[None, None], (B, L, Hkv, d)).copy()
    Od, _ = oracle.attn_decode(qd, kc, vc, 0.3)
    for h in range(H):
        np.testing.assert_allclose(Od[:, h], np.broadcast_to(c[h // 2], (B, d)), rtol=0, atol=1e-12)
    # paged decode: identical keys per head give a closed-form LSE
    seqlens, P = [7, 3], 4
    table, npg = synth.paged_layout(3, seqlens, P, 2)
    u = rand(13, Hkv, d)
    kp = np.broadcast_to(u[None, None], (npg, P, Hkv, d)).copy()
    vp = np.broadcast_to(c[None, None], (npg, P, Hkv, d)).copy()
    Op, lsep = oracle.attn_decode_paged(qd, kp, vp, table, seqlens, 0.3)
    for b in range(B):
        for h in range(H):
            np.testing.assert_allclose(Op[b, h], c[h // 2], rtol=0, atol=1e-12)
            assert abs(lsep[b, h] - (0.3 * qd[b, h] @ u[h // 2] + math.log(seqlens[b]))) < 1e-12


def test_heads_must_divide():
    q, k = rand(1, 1, 3, 6, 4), rand(2, 1, 3, 4, 4)
    with pytest.raises(ValueError):
        oracle.attn_fwd(q, k, k, 0.5)
    with pytest.raises(ValueError):
        oracle.attn_bwd(q, k, k, q, 0.5)


def _grouped_loss(q, k, v, do, scale, causal):
    """sum(O * dO) of the grouped forward, through the scalar brute force per query head."""
    from oracle.algorithms import brute_force_attention
    H, Hkv = q.shape[2], k.shape[2]
    total = 0.0
    for h in range(H):
        j = h // (H // Hkv)
        o, _ = brute_force_attention(q[0, :, h], k[0, :, j], v[0, :, j], scale, causal)
        total += float(np.sum(np.asarray(o) * do[0, :, h]))
    return total


@pytest.mark.parametrize("causal", [False, True])
def test_grouped_backward_finite_differences(causal):
    """dK, dV of a shared head by central differences of sum(O * dO) through the scalar
    brute force: the shared head's gradient is the sum over its group."""
    B, N, H, Hkv, d, scale, step = 1, 5, 4, 2, 3, 0.7, 1e-6
    q, k, v, do = rand(30, B, N, H, d), rand(31, B, N, Hkv, d), rand(32, B, N, Hkv, d), rand(33, B, N, H, d)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, scale, causal)
    for name, x, g in (("k", k, dk), ("v", v, dv), ("q", q, dq)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += step
            xm[idx] -= step
            args_p, args_m = {"q": q, "k": k, "v": v}, {"q": q, "k": k, "v": v}
            args_p[name], args_m[name] = xp, xm
            num[idx] = (_grouped_loss(args_p["q"], args_p["k"], args_p["v"], do, scale, causal)
                        - _grouped_loss(args_m["q"], args_m["k"], args_m["v"], do, scale, causal)) / (2 * step)
        assert np.max(np.abs(g - num)) / max(1.0, np.max(np.abs(num))) <= 1e-6, name


def test_grouped_backward_is_multi_head_on_repeated_heads_summed():
    B, N, H, Hkv, d = 2, 7, 6, 3, 4
    q, k, v, do = rand(34, B, N, H, d), rand(35, B, N, Hkv, d), rand(36, B, N, Hkv, d), rand(37, B, N, H, d)
    g = H // Hkv
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, 0.4, True)
    dq2, dk2, dv2 = oracle.attn_bwd(q, np.repeat(k, g, axis=2), np.repeat(v, g, axis=2), do, 0.4, True)
    np.testing.assert_allclose(dq, dq2, atol=1e-13)
    np.testing.assert_allclose(dk, dk2.reshape(B, N, Hkv, g, d).sum(axis=3), atol=1e-13)
    np.testing.assert_allclose(dv, dv2.reshape(B, N, Hkv, g, d).sum(axis=3), atol=1e-13)


def _fwd_interleaved(q, k, v, scale, causal=False):
    """Planted mistake: query head h reads key-value head h % Hkv (interleaved groups)."""
    B, N, H, _ = q.shape
    Hkv = k.shape[2]
    O, lse = np.empty(q.shape), np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            O[b, :, h], lse[b, h] = oracle.attention_head(q[b, :, h], k[b, :, h % Hkv], v[b, :, h % Hkv], scale, causal)
    return O, lse


def test_interleaved_grouping_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "attn_fwd", _fwd_interleaved)
    with pytest.raises(AssertionError):
        test_constant_values_identify_the_group(8, 2, False)
    with pytest.raises(AssertionError):
        test_identical_keys_closed_form(True)
