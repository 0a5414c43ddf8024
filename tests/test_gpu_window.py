"""GPU parity of fa_fwd_window (Nq queries against Nk keys, bottom-right aligned, optional
sliding window) against the float64 oracle. bf16 O <= 2e-2, LSE <= 1e-3; fp32 1e-5. Rows
with no visible key must come out as O = 0, LSE = -inf exactly."""
import math

import numpy as np
import pytest

import oracle
import synth
from gpu_util import bits_to_f64, dev_bf16, dev_f32, host, max_abs

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_O, TOL_LSE = 2e-2, 1e-3


def fa():
    import io_aware_softmax_03_amd as m
    return m


def gen(seed, B, Nq, Nk, H, Hkv, d, dtype):
    q = synth.bnhd_tensor(seed, synth.TENSOR_Q, B, Nq, H, d, dtype)
    k = synth.bnhd_tensor(seed, synth.TENSOR_K, B, Nk, Hkv, d, dtype)
    v = synth.bnhd_tensor(seed, synth.TENSOR_V, B, Nk, Hkv, d, dtype)
    return q, k, v


def check(o, lse, o_ref, lse_ref, tol_o, tol_lse):
    o, lse = host(o), host(lse)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty)
    assert np.all(o.transpose(0, 2, 1, 3)[empty] == 0)
    assert max_abs(o, o_ref) <= tol_o
    assert max_abs(lse[~empty], lse_ref[~empty]) <= tol_lse


CASES = [
    # B, Nq, Nk, H, Hkv, d, causal, left, right
    (1, 300, 1000, 2, 2, 128, True, -1, -1),     # chunked prefill: 300 new queries on a 700-key cache
    (2, 4, 128, 2, 1, 64, True, -1, -1),         # the pages' four queries against 128 keys
    (1, 700, 300, 2, 2, 128, True, -1, -1),      # more queries than keys: the first 400 see nothing
    (1, 1000, 1000, 2, 2, 128, True, 64, -1),    # 64-key sliding window
    (1, 1500, 1500, 2, 1, 64, True, 300, -1),
    (1, 600, 600, 2, 2, 128, False, 40, 70),     # two-sided window, not causal
    (1, 257, 900, 4, 2, 128, False, -1, 5),      # upper bound only
    (2, 520, 2000, 4, 4, 128, True, 700, -1),    # prefill with a window
    (1, 1, 777, 2, 2, 128, True, 10, -1),        # a single query
    (1, 33, 0, 2, 2, 64, False, -1, -1),         # no keys at all
    (1, 1100, 1100, 2, 2, 64, False, 0, 0),      # each query sees only its own key
    (1, 700, 700, 2, 2, 128, True, 90, -1),      # waves whose first block is odd (near the start)
    (1, 600, 600, 2, 1, 64, True, 90, -1),
    (2, 300, 330, 2, 2, 128, True, 60, -1),
]


@pytest.mark.parametrize("B,Nq,Nk,H,Hkv,d,causal,left,right", CASES)
def test_fwd_window_bf16(B, Nq, Nk, H, Hkv, d, causal, left, right):
    q, k, v = gen(31, B, Nq, Nk, H, Hkv, d, "bf16")
    if Nk == 0:
        # through the C ABI: an empty key tensor has no storage to point at
        import torch
        qd = dev_bf16(q)
        kd = torch.zeros((1, 1, Hkv, d), dtype=torch.bfloat16, device="cuda")
        o = torch.full_like(qd, 7.0)
        lse = torch.zeros((B, H, Nq), dtype=torch.float32, device="cuda")
        st = fa().lib().fa_fwd_window(qd.data_ptr(), kd.data_ptr(), kd.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                      B, H, Hkv, Nq, 0, d, 1 / math.sqrt(d), int(causal), left, right,
                                      fa().FA_DTYPE_BF16, torch.cuda.current_stream().cuda_stream)
        assert st == 0
        assert np.all(host(o) == 0) and np.all(np.isneginf(host(lse)))
        return
    o, lse = fa().fwd_window(dev_bf16(q), dev_bf16(k), dev_bf16(v), causal=causal, window=(left, right))
    o_ref, lse_ref = oracle.attn_fwd_window(bits_to_f64(q), bits_to_f64(k), bits_to_f64(v), 1 / math.sqrt(d),
                                            causal, left, right)
    check(o, lse, o_ref, lse_ref, TOL_O, TOL_LSE)


@pytest.mark.parametrize("B,Nq,Nk,H,Hkv,d,causal,left,right", [
    (1, 100, 400, 2, 2, 64, True, -1, -1), (1, 300, 300, 2, 1, 128, True, 50, -1),
    (1, 200, 150, 2, 2, 64, True, 20, -1), (1, 128, 128, 2, 2, 128, False, 3, 9),
    (1, 1000, 2000, 4, 2, 64, True, 300, -1),      # four-row query blocks, several 256-key blocks
    (1, 2048, 2048, 2, 2, 128, False, 100, 50),    # eight-row query blocks, two-sided window
])
def test_fwd_window_f32(B, Nq, Nk, H, Hkv, d, causal, left, right):
    q, k, v = gen(32, B, Nq, Nk, H, Hkv, d, "f32")
    o, lse = fa().fwd_window(dev_f32(q), dev_f32(k), dev_f32(v), causal=causal, window=(left, right))
    o_ref, lse_ref = oracle.attn_fwd_window(q, k, v, 1 / math.sqrt(d), causal, left, right)
    check(o, lse, o_ref, lse_ref, TOL_F32, TOL_F32)


def test_square_without_window_is_fa_fwd():
    torch = pytest.importorskip("torch")
    q, k, v = (dev_bf16(x) for x in gen(33, 2, 900, 900, 4, 2, 128, "bf16"))
    for causal in (False, True):
        a = fa().fwd(q, k, v, causal=causal)
        b = fa().fwd_window(q, k, v, causal=causal)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_chunked_prefill_matches_the_tail_of_the_full_prefill():
    """Processing the last 512 tokens as a chunk against the 4096-key cache gives the last
    512 rows of the full causal prefill (same kernel arithmetic, up to where the row's keys
    fall in the 256-row query blocks)."""
    torch = pytest.importorskip("torch")
    Nk, Nq = 4096, 512
    q, k, v = (dev_bf16(x) for x in gen(34, 1, Nk, Nk, 2, 2, 128, "bf16"))
    o_full, lse_full = fa().fwd(q, k, v, causal=True)
    o, lse = fa().fwd_window(q[:, Nk - Nq:].contiguous(), k, v, causal=True)
    assert max_abs(host(o), host(o_full[:, Nk - Nq:])) <= 2 ** -8
    assert max_abs(host(lse), host(lse_full[:, :, Nk - Nq:])) <= 1e-5


@pytest.mark.parametrize("name,B,Nq,Nk,H,left", [
    ("chunked prefill", 4, 2048, 16384, 16, -1),
    ("sliding window", 2, 8192, 8192, 16, 1024),
])
def test_fwd_window_full_size_every_element(name, B, Nq, Nk, H, left):
    """The bench's banded workloads (d=128, causal, bf16), drawn on the device: every row of
    every head against the oracle. The oracle runs on blocks of 512 rows against the keys
    between the block's first row's lowest and last row's highest visible key, with the
    band mask on that rectangle, so each row still sees exactly its visible keys."""
    torch = pytest.importorskip("torch")
    d = 128
    gen_t = torch.Generator(device="cuda")
    gen_t.manual_seed(10)
    q = torch.randn((B, Nq, H, d), generator=gen_t, device="cuda", dtype=torch.bfloat16)
    k = torch.randn((B, Nk, H, d), generator=gen_t, device="cuda", dtype=torch.bfloat16)
    v = torch.randn((B, Nk, H, d), generator=gen_t, device="cuda", dtype=torch.bfloat16)
    o, lse = fa().fwd_window(q, k, v, causal=True, window=(left, -1))
    o, lse = host(o), host(lse)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    scale = 1 / math.sqrt(d)
    keep = oracle.band_keep(Nq, Nk, True, left, -1)
    rows = 512
    worst_o = worst_l = 0.0
    for b in range(B):
        for h in range(H):
            qh, kh, vh = host(q[b, :, h]), host(k[b, :, h]), host(v[b, :, h])
            for i0 in range(0, Nq, rows):
                i1 = min(Nq, i0 + rows)
                j0 = 0 if left < 0 else max(0, i0 + Nk - Nq - left)
                j1 = i1 - 1 + Nk - Nq + 1
                o_ref, lse_ref = oracle.attention_head(qh[i0:i1], kh[j0:j1], vh[j0:j1], scale,
                                                       keep=keep[i0:i1, j0:j1])
                worst_o = max(worst_o, max_abs(o[b, i0:i1, h], o_ref))
                worst_l = max(worst_l, max_abs(lse[b, h, i0:i1], lse_ref))
    assert worst_o <= TOL_O, (name, worst_o)
    assert worst_l <= TOL_LSE, (name, worst_l)
