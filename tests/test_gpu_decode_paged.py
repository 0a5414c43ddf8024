"""GPU parity of the paged-cache decode against the float64 oracle.

Bounds as for the contiguous decode: O max-abs <= 2e-2, LSE <= 1e-3. The block tables put
each sequence's pages at seeded random places in the pool, the last page of a sequence is
partly filled, and every slot that is not part of a sequence holds noise of its own, so a
kernel that reads a wrong page, a wrong slot or past the end of a sequence fails."""
import math

import numpy as np
import pytest

import oracle
import synth
from gpu_util import bits_to_f64, dev_bf16, dev_i32, host, max_abs

pytestmark = pytest.mark.gpu

TOL_O, TOL_LSE = 2e-2, 1e-3


def fa():
    import io_aware_softmax_03_amd as m
    return m


def gen_paged(seed, seqlens, page_size, H, d, extra_pages=3):
    table, num_pages = synth.paged_layout(seed, seqlens, page_size, extra_pages)
    q = synth.decode_query(seed, len(seqlens), H, d)
    kp = synth.paged_tensor(seed, synth.TENSOR_K, seqlens, table, num_pages, page_size, H, d)
    vp = synth.paged_tensor(seed, synth.TENSOR_V, seqlens, table, num_pages, page_size, H, d)
    return q, kp, vp, table


def run_paged(q, kp, vp, table, seqlens, splits):
    return fa().decode_paged(dev_bf16(q), dev_bf16(kp), dev_bf16(vp), dev_i32(table), dev_i32(seqlens),
                             num_splits=splits)


@pytest.mark.parametrize("seqlens,page_size,H,d,splits", [
    ([100, 37, 16, 1], 16, 4, 128, 8),             # partial last pages, a one-token sequence
    ([300, 0, 129], 16, 2, 128, 4),                 # an empty sequence
    ([257, 64, 5], 1, 2, 64, 16),                   # one token per page
    ([1000, 999, 1001], 64, 2, 128, 64),
    ([5000, 17], 256, 2, 64, 1024),                 # more splits than keys in the short sequence
    ([4500, 3000], 16, 2, 128, 3),                  # chunks longer than one 256-page window
    ([2048], 1024, 3, 128, 1),                      # largest page size, one chunk
])
def test_decode_paged(seqlens, page_size, H, d, splits):
    q, kp, vp, table = gen_paged(11, seqlens, page_size, H, d)
    o, lse = run_paged(q, kp, vp, table, seqlens, splits)
    o_ref, lse_ref = oracle.attn_decode_paged(bits_to_f64(q), bits_to_f64(kp), bits_to_f64(vp), table,
                                              seqlens, 1 / math.sqrt(d))
    o, lse = host(o), host(lse)
    assert max_abs(o, o_ref) <= TOL_O
    empty = np.array(seqlens) == 0
    assert np.all(np.isneginf(lse[empty])) and np.all(o[empty] == 0)
    assert max_abs(lse[~empty], lse_ref[~empty]) <= TOL_LSE


def test_decode_paged_matches_contiguous_decode():
    """With equal lengths, the paged gather visits the same keys in the same chunks and
    batches as the contiguous decode over the gathered cache: the results agree to rounding."""
    torch = pytest.importorskip("torch")
    B, H, L, d, P = 3, 4, 3000, 128, 16
    seqlens = [L] * B
    q, kp, vp, table = gen_paged(12, seqlens, P, H, d)
    o_p, lse_p = run_paged(q, kp, vp, table, seqlens, 16)
    t = np.arange(L)
    kc = np.stack([kp[table[b, t // P], t % P] for b in range(B)])   # [B, L, H, d]
    vc = np.stack([vp[table[b, t // P], t % P] for b in range(B)])
    o_c, lse_c = fa().decode(dev_bf16(q), dev_bf16(kc), dev_bf16(vc), num_splits=16)
    assert max_abs(host(o_p), host(o_c)) <= 2 ** -8
    assert max_abs(host(lse_p), host(lse_c)) <= 1e-5


def test_decode_paged_clamps_bad_tables():
    """Lengths past the table's capacity and page ids outside the pool are clamped on the
    device (to max_pages * page_size tokens and to [0, num_pages - 1]), never read through."""
    seqlens = [90, 40]
    P, H, d = 16, 2, 64
    q, kp, vp, table = gen_paged(13, seqlens, P, H, d)
    num_pages = kp.shape[0]
    bad_table = table.copy()
    bad_table[1, 0] = -5                  # -> page 0
    bad_table[1, 2] = num_pages + 1000    # -> last page
    bad_len = [10 ** 6, 40]               # -> max_pages * P
    o, lse = run_paged(q, kp, vp, bad_table, bad_len, 4)
    eff_table = np.clip(bad_table, 0, num_pages - 1)
    eff_len = [min(bad_len[0], table.shape[1] * P), 40]
    o_ref, lse_ref = oracle.attn_decode_paged(bits_to_f64(q), bits_to_f64(kp), bits_to_f64(vp), eff_table,
                                              eff_len, 1 / math.sqrt(d))
    assert max_abs(host(o), o_ref) <= TOL_O
    assert max_abs(host(lse), lse_ref) <= TOL_LSE


def test_decode_paged_full_size_every_element():
    """B=64, H=32, d=128, page size 16, lengths uniform in [16384, 32768], 32 splits, as the
    bench runs it (about 26 GB of pages drawn on the device); each sequence's tokens are
    gathered through its block table on the device and copied back: every (b, h) against
    the oracle."""
    torch = pytest.importorskip("torch")
    B, H, d, P = 64, 32, 128, 16
    seqlens = synth.varlen_lengths(8, B, 16384, 32768).tolist()
    table, num_pages = synth.paged_layout(8, seqlens, P, 0)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(8)
    q = torch.randn((B, H, d), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    kp = torch.randn((num_pages, P, H, d), generator=gen, device="cuda", dtype=torch.bfloat16)
    vp = torch.randn((num_pages, P, H, d), generator=gen, device="cuda", dtype=torch.bfloat16)
    tab, sl = dev_i32(table), dev_i32(seqlens)
    o, lse = fa().decode_paged(q, kp, vp, tab, sl, num_splits=32)
    o, lse = host(o), host(lse)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    scale = 1 / math.sqrt(d)
    qh = host(q)
    worst_o = worst_l = 0.0
    for b in range(B):
        L = seqlens[b]
        t = torch.arange(L, device="cuda")
        pages = tab[b].long()[t // P]
        kb, vb = host(kp[pages, t % P]), host(vp[pages, t % P])   # [L, H, d]
        for h in range(H):
            o_ref, lse_ref = oracle.attn_decode_slice(qh[b, h], kb[:, h], vb[:, h], scale)
            worst_o = max(worst_o, max_abs(o[b, h], o_ref))
            worst_l = max(worst_l, abs(lse[b, h] - lse_ref))
    assert worst_o <= TOL_O, worst_o
    assert worst_l <= TOL_LSE, worst_l
    del kp, vp
    torch.cuda.empty_cache()
