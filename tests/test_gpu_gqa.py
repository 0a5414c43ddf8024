"""GPU parity of grouped-query attention (Hkv < H key-value heads, query head h reading
key-value head h // (H // Hkv)) against the float64 oracle, for the forward, the packed
forward and both decodes. Bounds as elsewhere: bf16 O <= 2e-2, LSE <= 1e-3; fp32 1e-5."""
import math

import numpy as np
import pytest

import oracle
import synth
from gpu_util import bits_to_f64, dev_bf16, dev_f32, dev_i32, host, max_abs

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_O, TOL_LSE = 2e-2, 1e-3


def fa():
    import io_aware_softmax_03_amd as m
    return m


def gen(seed, B, N, H, Hkv, d, dtype):
    q = synth.bnhd_tensor(seed, synth.TENSOR_Q, B, N, H, d, dtype)
    k = synth.bnhd_tensor(seed, synth.TENSOR_K, B, N, Hkv, d, dtype)
    v = synth.bnhd_tensor(seed, synth.TENSOR_V, B, N, Hkv, d, dtype)
    return q, k, v


@pytest.mark.parametrize("B,N,H,Hkv,d,causal", [
    (1, 600, 8, 2, 128, True),
    (2, 300, 6, 3, 64, False),
    (1, 520, 16, 8, 128, True),    # key-value heads divisible by 8: XCD-grouped launch order
    (1, 257, 32, 8, 128, False),
    (1, 100, 4, 1, 64, True),      # one key-value head (multi-query)
    (2, 777, 16, 2, 128, True),
])
def test_fwd_bf16_gqa(B, N, H, Hkv, d, causal):
    q, k, v = gen(21, B, N, H, Hkv, d, "bf16")
    o, lse = fa().fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), causal=causal)
    o_ref, lse_ref = oracle.attn_fwd(bits_to_f64(q), bits_to_f64(k), bits_to_f64(v), 1 / math.sqrt(d), causal)
    assert max_abs(host(o), o_ref) <= TOL_O
    assert max_abs(host(lse), lse_ref) <= TOL_LSE


@pytest.mark.parametrize("B,N,H,Hkv,d,causal", [
    (1, 256, 4, 2, 64, False), (2, 100, 6, 3, 128, True),
    (1, 1024, 8, 2, 128, True),   # eight-row query blocks (larger grid) with grouped heads
])
def test_fwd_f32_gqa(B, N, H, Hkv, d, causal):
    q, k, v = gen(22, B, N, H, Hkv, d, "f32")
    o, lse = fa().fwd(dev_f32(q), dev_f32(k), dev_f32(v), causal=causal)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, 1 / math.sqrt(d), causal)
    assert max_abs(host(o), o_ref) <= TOL_F32
    assert max_abs(host(lse), lse_ref) <= TOL_F32


def test_fwd_gqa_equals_multi_head_on_repeated_heads():
    """The grouped read gives what multi-head attention gives on K and V repeated per query
    head: same kernel arithmetic, only the key-value addresses differ."""
    torch = pytest.importorskip("torch")
    B, N, H, Hkv, d = 2, 700, 16, 4, 128
    q, k, v = (dev_bf16(x) for x in gen(23, B, N, H, Hkv, d, "bf16"))
    o, lse = fa().fwd(q, k, v, causal=True)
    g = H // Hkv
    o2, lse2 = fa().fwd(q, k.repeat_interleave(g, dim=2).contiguous(), v.repeat_interleave(g, dim=2).contiguous(),
                        causal=True)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("d", [64, 128])
def test_varlen_gqa(d):
    lengths = [5, 0, 200, 129, 64]
    H, Hkv = 4, 2
    cu = synth.cu_seqlens_from_lengths(lengths)
    q = synth.varlen_tensor(24, synth.TENSOR_Q, lengths, H, d)
    k = synth.varlen_tensor(24, synth.TENSOR_K, lengths, Hkv, d)
    v = synth.varlen_tensor(24, synth.TENSOR_V, lengths, Hkv, d)
    o, lse = fa().fwd_varlen(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_i32(cu), max(lengths), causal=True)
    o_ref, lse_ref = oracle.attn_fwd_varlen(bits_to_f64(q), bits_to_f64(k), bits_to_f64(v), cu, 1 / math.sqrt(d),
                                            True)
    assert max_abs(host(o), o_ref) <= TOL_O
    assert max_abs(host(lse), lse_ref) <= TOL_LSE


# ------------------------------------------------------------------------------ decode

def gen_decode(seed, B, H, Hkv, L, d):
    q = synth.decode_query(seed, B, H, d)
    kc = synth.bnhd_tensor(seed, synth.TENSOR_K, B, L, Hkv, d)
    vc = synth.bnhd_tensor(seed, synth.TENSOR_V, B, L, Hkv, d)
    return q, kc, vc


@pytest.mark.parametrize("B,H,Hkv,L,d,splits", [
    (2, 8, 2, 1000, 128, 8),
    (3, 32, 8, 4097, 128, 64),
    (1, 4, 1, 1, 128, 1),
    (2, 6, 3, 77, 64, 16),
    (1, 32, 1, 5000, 64, 1024),    # 32 query heads per key-value head: two waves per group
    (2, 40, 2, 300, 128, 4),       # groups of 20: a full and a partial block of 16
    (1, 16, 8, 33, 128, 2),
])
def test_decode_gqa(B, H, Hkv, L, d, splits):
    qb, kb, vb = gen_decode(25, B, H, Hkv, L, d)
    o, lse = fa().decode(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), num_splits=splits)
    o_ref, lse_ref = oracle.attn_decode(bits_to_f64(qb), bits_to_f64(kb), bits_to_f64(vb), 1 / math.sqrt(d))
    assert max_abs(host(o), o_ref) <= TOL_O
    assert max_abs(host(lse), lse_ref) <= TOL_LSE


def test_decode_gqa_split_invariance():
    B, H, Hkv, L, d = 2, 8, 2, 6000, 128
    q, k, v = (dev_bf16(x) for x in gen_decode(26, B, H, Hkv, L, d))
    outs = [fa().decode(q, k, v, num_splits=s) for s in (1, 8, 64, 512)]
    for o, lse in outs[1:]:
        assert max_abs(host(o), host(outs[0][0])) <= 2 ** -7
        assert max_abs(host(lse), host(outs[0][1])) <= 1e-5


@pytest.mark.parametrize("seqlens,page_size,H,Hkv,d,splits", [
    ([100, 37, 0, 1], 16, 8, 2, 128, 8),
    ([257, 64, 5], 1, 4, 1, 64, 16),
    ([4500, 3000], 16, 16, 1, 128, 3),     # chunks longer than one 256-page window
    ([1000, 999], 64, 12, 4, 64, 64),
])
def test_decode_paged_gqa(seqlens, page_size, H, Hkv, d, splits):
    table, num_pages = synth.paged_layout(27, seqlens, page_size, 3)
    q = synth.decode_query(27, len(seqlens), H, d)
    kp = synth.paged_tensor(27, synth.TENSOR_K, seqlens, table, num_pages, page_size, Hkv, d)
    vp = synth.paged_tensor(27, synth.TENSOR_V, seqlens, table, num_pages, page_size, Hkv, d)
    o, lse = fa().decode_paged(dev_bf16(q), dev_bf16(kp), dev_bf16(vp), dev_i32(table), dev_i32(seqlens),
                               num_splits=splits)
    o_ref, lse_ref = oracle.attn_decode_paged(bits_to_f64(q), bits_to_f64(kp), bits_to_f64(vp), table, seqlens,
                                              1 / math.sqrt(d))
    o, lse = host(o), host(lse)
    assert max_abs(o, o_ref) <= TOL_O
    empty = np.array(seqlens) == 0
    assert np.all(np.isneginf(lse[empty])) and np.all(o[empty] == 0)
    assert max_abs(lse[~empty], lse_ref[~empty]) <= TOL_LSE


def test_decode_gqa_full_size_every_element():
    """B=64, H=32 query heads over Hkv=8 key-value heads, L=32768, d=128, 32 splits (8.6 GB
    of cache drawn on the device, copied back one batch row at a time): every (b, h)
    against the oracle."""
    torch = pytest.importorskip("torch")
    B, H, Hkv, L, d = 64, 32, 8, 32768, 128
    gen = torch.Generator(device="cuda")
    gen.manual_seed(9)
    q = torch.randn((B, H, d), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    kc = torch.randn((B, L, Hkv, d), generator=gen, device="cuda", dtype=torch.bfloat16)
    vc = torch.randn((B, L, Hkv, d), generator=gen, device="cuda", dtype=torch.bfloat16)
    o, lse = fa().decode(q, kc, vc, num_splits=32)
    o, lse = host(o), host(lse)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    scale = 1 / math.sqrt(d)
    qh = host(q)
    worst_o = worst_l = 0.0
    for b in range(B):
        kb, vb = host(kc[b]), host(vc[b])
        for h in range(H):
            j = h // (H // Hkv)
            o_ref, lse_ref = oracle.attn_decode_slice(qh[b, h], kb[:, j], vb[:, j], scale)
            worst_o = max(worst_o, max_abs(o[b, h], o_ref))
            worst_l = max(worst_l, abs(lse[b, h] - lse_ref))
    assert worst_o <= TOL_O, worst_o
    assert worst_l <= TOL_LSE, worst_l
    del kc, vc
    torch.cuda.empty_cache()


# ------------------------------------------------------------------------------ backward

TOL_GRAD = 2e-2


@pytest.mark.parametrize("B,N,H,Hkv,d,causal", [
    (1, 256, 4, 2, 128, True),
    (2, 300, 6, 3, 64, False),
    (1, 200, 8, 1, 128, True),     # one key-value head for all eight query heads
    (1, 513, 4, 2, 64, True),
])
def test_bwd_gqa(B, N, H, Hkv, d, causal):
    q, k, v = gen(28, B, N, H, Hkv, d, "bf16")
    g = synth.bnhd_tensor(28, synth.TENSOR_DO, B, N, H, d)
    qd, kd, vd, gd = (dev_bf16(x) for x in (q, k, v, g))
    o, lse = fa().fwd(qd, kd, vd, causal=causal)
    dq, dk, dv = fa().bwd(qd, kd, vd, o, lse, gd, causal=causal)
    ref = oracle.attn_bwd(bits_to_f64(q), bits_to_f64(k), bits_to_f64(v), bits_to_f64(g), 1 / math.sqrt(d), causal)
    for got, want in zip((dq, dk, dv), ref):
        assert got.shape == want.shape
        assert max_abs(host(got), want) <= TOL_GRAD


def test_bwd_gqa_equals_multi_head_on_repeated_heads_summed():
    """dK, dV of a shared head equal the multi-head gradients of its repeated copies, summed
    over the group (to the order of the fp32 additions); dQ is the same."""
    torch = pytest.importorskip("torch")
    B, N, H, Hkv, d = 1, 600, 8, 2, 128
    q, k, v = (dev_bf16(x) for x in gen(29, B, N, H, Hkv, d, "bf16"))
    g = dev_bf16(synth.bnhd_tensor(29, synth.TENSOR_DO, B, N, H, d))
    grp = H // Hkv
    kr, vr = k.repeat_interleave(grp, dim=2).contiguous(), v.repeat_interleave(grp, dim=2).contiguous()
    o, lse = fa().fwd(q, k, v, causal=True)
    dq, dk, dv = fa().bwd(q, k, v, o, lse, g, causal=True)
    dq2, dk2, dv2 = fa().bwd(q, kr, vr, o, lse, g, causal=True)
    assert max_abs(host(dq), host(dq2)) <= 1e-5
    assert max_abs(host(dk), host(dk2.view(B, N, Hkv, grp, d).sum(dim=3))) <= 1e-4
    assert max_abs(host(dv), host(dv2.view(B, N, Hkv, grp, d).sum(dim=3))) <= 1e-4


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_row_terms_identical_on_both_launch_paths(d):
    """D = rowsum(dO * O) and the base-2 LSE that the backward leaves in its workspace depend
    on O, dO and the LSE only. The multi-head backward forms them in the dQ kernel, the
    grouped one in a separate preprocessing launch, in the same order of additions: the
    two workspaces agree bit for bit (so dS, and dQ, round the same on both paths)."""
    torch = pytest.importorskip("torch")
    B, N, H = 2, 333, 4
    q, k, v = (dev_bf16(x) for x in gen(41, B, N, H, H, d, "bf16"))
    _, k2, v2 = (dev_bf16(x) for x in gen(42, B, N, H, 2, d, "bf16"))
    g = dev_bf16(synth.bnhd_tensor(41, synth.TENSOR_DO, B, N, H, d))
    o, lse = fa().fwd(q, k, v, causal=True)
    nbytes = fa().lib().fa_bwd_workspace_bytes(B, H, N)
    rows = B * H * N
    terms = []
    for kk, vv in ((k, v), (k2, v2)):
        ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
        fa().bwd(q, kk, vv, o, lse, g, causal=True, workspace=ws)
        terms.append(ws.view(torch.int32)[:2 * rows].cpu().numpy())
    assert np.array_equal(terms[0], terms[1])
    dref = (host(g).astype(np.float64) * host(o).astype(np.float64)).sum(-1).transpose(0, 2, 1).reshape(-1)
    assert np.abs(terms[0][:rows].view(np.float32) - dref).max() <= 1e-4 * max(1.0, np.abs(dref).max())
