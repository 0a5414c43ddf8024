"""Pins of the paged-cache decode oracle ("FlashAttention-2 and -3", "Paged KV caches, a
preview of serving"): gathering a sequence's tokens through its block table must give the
contiguous decode of those tokens, pages may sit anywhere in the pool, slots past a
sequence's end are not part of it, and an empty sequence has no visible key."""
import math

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def make(seed, seqlens, H, d, P, extra=3):
    table, npg = synth.paged_layout(seed, seqlens, P, extra)
    kp = synth.f32_from_bf16_bits(synth.paged_tensor(seed, synth.TENSOR_K, seqlens, table, npg, P, H, d))
    vp = synth.f32_from_bf16_bits(synth.paged_tensor(seed, synth.TENSOR_V, seqlens, table, npg, P, H, d))
    q = synth.f32_from_bf16_bits(synth.decode_query(seed, len(seqlens), H, d))
    return q, kp, vp, table


def contiguous(seed, b, L, H, d, tensor_id):
    """Sequence b's cache as the generator draws it: slice (b, h) for every head."""
    x = np.stack([synth.normal_slice(seed, tensor_id, b, h, (L, d)) for h in range(H)], axis=1)
    return synth.f32_from_bf16_bits(synth.bf16_bits_from_f32(x))


@pytest.mark.parametrize("P", [1, 4, 16])
def test_paged_equals_contiguous_decode(P):
    seqlens = [1, 16, 17, 40, 0, 33]
    H, d = 2, 8
    q, kp, vp, table = make(5, seqlens, H, d, P)
    O, lse = oracle.attn_decode_paged(q, kp, vp, table, seqlens, 1 / math.sqrt(d))
    for b, L in enumerate(seqlens):
        if L == 0:
            assert np.all(O[b] == 0) and np.all(np.isneginf(lse[b]))
            continue
        kc = contiguous(5, b, L, H, d, synth.TENSOR_K)[None]
        vc = contiguous(5, b, L, H, d, synth.TENSOR_V)[None]
        Oc, lc = oracle.attn_decode(q[b:b + 1], kc, vc, 1 / math.sqrt(d))
        np.testing.assert_allclose(O[b], Oc[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b], lc[0], rtol=0, atol=1e-12)


def test_page_placement_does_not_matter():
    seqlens = [23, 9]
    H, d, P = 1, 4, 4
    q, kp, vp, table = make(6, seqlens, H, d, P, extra=0)
    O, lse = oracle.attn_decode_paged(q, kp, vp, table, seqlens, 0.5)
    # move every page to a new physical slot and rewrite the table accordingly
    perm = np.random.default_rng(1).permutation(kp.shape[0])
    inv = np.argsort(perm)
    O2, lse2 = oracle.attn_decode_paged(q, kp[perm], vp[perm], inv[table], seqlens, 0.5)
    np.testing.assert_allclose(O2, O, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-12)


def gather_whole_pages(pages, block_table, seq_len):
    """The planted mistake: read every slot of the listed pages, including the ones past
    the end of the sequence."""
    n = (seq_len + pages.shape[1] - 1) // pages.shape[1]
    return pages[block_table[:n]].reshape(-1, *pages.shape[2:])


def test_garbage_slots_are_rejected():
    seqlens = [21]  # six 4-slot pages: the last one holds 1 token and 3 slots of noise
    H, d, P = 1, 8, 4
    q, kp, vp, table = make(7, seqlens, H, d, P)
    O, lse = oracle.attn_decode_paged(q, kp, vp, table, seqlens, 1 / math.sqrt(d))
    k_bad = gather_whole_pages(kp, table[0], seqlens[0])
    v_bad = gather_whole_pages(vp, table[0], seqlens[0])
    assert k_bad.shape[0] > seqlens[0]
    Ob, lb = oracle.attn_decode(q[:1], k_bad[None], v_bad[None], 1 / math.sqrt(d))
    assert np.max(np.abs(Ob[0] - O[0])) > 1e-3 or np.max(np.abs(lb[0] - lse[0])) > 1e-3
