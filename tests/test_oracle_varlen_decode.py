"""CPU pins for the packed variable-length forward and the single-token decode."""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


# ------------------------------------------------------------------ varlen

def test_cu_seqlens_form_from_page():
    """Offsets start at 0 and have length B+1 ('Variable-length batches without padding')."""
    g = GOLDEN["cu_seqlens_form"]
    assert synth.cu_seqlens_from_lengths(g["lengths"]).tolist() == g["cu_seqlens"]


def test_offsets_without_leading_zero_are_rejected():
    """Negative control: plain cumulative sums (no leading 0) are not valid offsets."""
    lengths = [5, 3, 4]
    bad = np.cumsum(lengths).astype(np.int32)
    q = np.zeros((12, 1, 2))
    with pytest.raises(ValueError):
        oracle.attn_fwd_varlen(q, q, q, bad, 1.0)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_matches_brute_force_per_sequence(causal):
    rng = np.random.default_rng(31)
    lengths = [3, 1, 0, 6, 4]
    cu = synth.cu_seqlens_from_lengths(lengths)
    T, H, d = int(cu[-1]), 2, 3
    q, k, v = (rng.standard_normal((T, H, d)) for _ in range(3))
    o, lse = oracle.attn_fwd_varlen(q, k, v, cu, 0.9, causal)
    assert lse.shape == (H, T)
    for s in range(len(lengths)):
        a, e = cu[s], cu[s + 1]
        for h in range(H):
            if e == a:
                continue
            ob, lb = oracle.brute_force_attention(q[a:e, h], k[a:e, h], v[a:e, h], 0.9, causal)
            np.testing.assert_allclose(o[a:e, h], ob, atol=1e-12)
            np.testing.assert_allclose(lse[h, a:e], lb, atol=1e-12)


def test_cross_sequence_attention_is_caught():
    """Negative control: attending over the whole packed tensor (ignoring the offsets)
    differs from the block-diagonal definition."""
    rng = np.random.default_rng(32)
    lengths = [4, 5]
    cu = synth.cu_seqlens_from_lengths(lengths)
    q, k, v = (rng.standard_normal((9, 1, 4)) for _ in range(3))
    o, _ = oracle.attn_fwd_varlen(q, k, v, cu, 0.5, False)
    wrong, _ = oracle.attention_head(q[:, 0], k[:, 0], v[:, 0], 0.5, False)
    assert np.max(np.abs(wrong - o[:, 0])) > 1e-3


# ------------------------------------------------------------------ decode

def test_decode_matches_brute_force():
    rng = np.random.default_rng(41)
    L, d = 7, 4
    qv, kr, vr = rng.standard_normal(d), rng.standard_normal((L, d)), rng.standard_normal((L, 5))
    o, lse = oracle.attn_decode_slice(qv, kr, vr, 0.5)
    ob, lb = oracle.brute_force_attention(qv[None, :], kr, vr, 0.5, False)
    np.testing.assert_allclose(o, ob[0], atol=1e-13)
    assert abs(lse - lb[0]) < 1e-13


@pytest.mark.parametrize("n_chunks", [1, 2, 8, 64, 512, 1000])
def test_split_and_merge_equals_unsplit(n_chunks):
    """Flash-Decoding: each chunk's (output, log-sum-exp) merged with log-sum-exp weights
    reproduces unsplit attention ('Decoding needs a different split'). 1000 chunks of
    L=1024 leaves empty chunks, which must carry zero weight."""
    rng = np.random.default_rng([42, n_chunks])
    L, d = 1024, 16
    qv = rng.standard_normal(d) * 2
    kr, vr = rng.standard_normal((L, d)), rng.standard_normal((L, d))
    o_ref, lse_ref = oracle.attn_decode_slice(qv, kr, vr, 0.25)
    outs, lses = oracle.decode_chunk_partials(qv, kr, vr, 0.25, n_chunks)
    o, lse = oracle.merge_partials(outs, lses)
    np.testing.assert_allclose(o, o_ref, atol=1e-12)
    assert abs(lse - lse_ref) < 1e-12


def test_equal_weight_merge_is_caught():
    """Negative control: averaging chunk outputs with equal weights (and taking the largest
    chunk log-sum-exp) is not the merge; it must differ from unsplit attention."""
    g = GOLDEN["decode_eight_chunks"]
    rng = np.random.default_rng(43)
    L, d = 512, 8
    qv = rng.standard_normal(d) * 3
    kr, vr = rng.standard_normal((L, d)), rng.standard_normal((L, d))
    o_ref, lse_ref = oracle.attn_decode_slice(qv, kr, vr, 0.5)
    outs, lses = oracle.decode_chunk_partials(qv, kr, vr, 0.5, g["n_chunks"])
    wrong_o, wrong_lse = outs.mean(axis=0), lses.max()
    assert np.max(np.abs(wrong_o - o_ref)) > 1e-3
    assert abs(wrong_lse - lse_ref) > 1e-3
    o, lse = oracle.merge_partials(outs, lses)
    np.testing.assert_allclose(o, o_ref, atol=1e-12)


def test_decode_batch_layout():
    rng = np.random.default_rng(44)
    q = rng.standard_normal((2, 3, 4))
    kc, vc = rng.standard_normal((2, 10, 3, 4)), rng.standard_normal((2, 10, 3, 4))
    o, lse = oracle.attn_decode(q, kc, vc, 0.5)
    for b in range(2):
        for h in range(3):
            ob, lb = oracle.brute_force_attention(q[b, h][None], kc[b, :, h], vc[b, :, h], 0.5)
            np.testing.assert_allclose(o[b, h], ob[0], atol=1e-13)
            assert abs(lse[b, h] - lb[0]) < 1e-13


def test_decode_is_last_row_of_causal_prefill():
    """The newest token sees every cached key: decoding query L-1 equals row L-1 of causal
    attention over the same L tokens (bottom-right reading of the decode step)."""
    rng = np.random.default_rng(45)
    L, d = 33, 8
    q, k, v = (rng.standard_normal((L, d)) for _ in range(3))
    o_full, lse_full = oracle.attention_head(q, k, v, 0.3, causal=True)
    o, lse = oracle.attn_decode_slice(q[-1], k, v, 0.3)
    np.testing.assert_allclose(o, o_full[-1], atol=1e-13)
    assert abs(lse - lse_full[-1]) < 1e-13
