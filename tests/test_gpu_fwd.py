"""GPU parity of the forward entry points against the float64 oracle.

Tolerances: fp32 inputs max-abs <= 1e-5 on O and LSE; bf16 inputs (fp32 accumulation)
max-abs <= 2e-2 on O and <= 1e-3 on LSE."""
import math

import numpy as np
import pytest

import oracle
import synth
from gpu_util import bits_to_f64, dev_bf16, dev_f32, dev_i32, host, max_abs

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_O_BF16, TOL_LSE_BF16 = 2e-2, 1e-3


def fa():
    import io_aware_softmax_03_amd as m
    return m


def gen_dense(seed, B, N, H, d, dtype):
    return [synth.bnhd_tensor(seed, t, B, N, H, d, dtype) for t in (synth.TENSOR_Q, synth.TENSOR_K, synth.TENSOR_V)]


# ----------------------------------------------------------------------------- fp32

@pytest.mark.parametrize("B,N,H,d,causal", [
    (1, 256, 1, 64, False),     # the exact-precision configuration
    (1, 256, 1, 64, True),
    (2, 100, 3, 128, True),
    (1, 257, 2, 64, False),
    (1, 1, 1, 128, True),
    (1, 1000, 4, 64, True),     # several 256-key blocks, ragged tail, four-row query blocks
    (1, 600, 4, 128, True),     # four-row query blocks at d = 128
    (2, 1024, 4, 128, False),   # eight-row query blocks (the larger grid), four key blocks
    (1, 2048, 2, 64, True),     # eight-row query blocks, causal over eight key blocks
])
def test_fwd_f32(B, N, H, d, causal):
    q, k, v = gen_dense(1, B, N, H, d, "f32")
    o, lse = fa().fwd(dev_f32(q), dev_f32(k), dev_f32(v), scale=1 / math.sqrt(d), causal=causal)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, 1 / math.sqrt(d), causal)
    assert max_abs(host(o), o_ref) <= TOL_F32
    assert max_abs(host(lse), lse_ref) <= TOL_F32


# ----------------------------------------------------------------------------- bf16

@pytest.mark.parametrize("B,N,H,d,causal", [
    (1, 1024, 2, 128, True),    # reduced causal prefill
    (1, 1024, 2, 128, False),
    (2, 129, 2, 128, True),     # one row past a block
    (1, 300, 3, 64, False),
    (1, 300, 3, 64, True),
    (1, 1, 1, 64, True),
    (1, 17, 1, 128, False),
    (3, 64, 2, 128, True),
    (1, 2000, 1, 64, True),
    (1, 600, 2, 128, True),     # three 256-row blocks: one causal workgroup takes a single block
    (1, 600, 1, 64, False),
    (1, 260, 1, 128, True),     # last block holds 4 rows: three of its waves have no rows
    (2, 1500, 1, 128, True),    # six blocks, ragged last key tile
    (1, 300, 8, 64, True),      # head count divisible by 8: heads interleaved across XCDs
    (2, 520, 8, 128, True),
    (1, 777, 16, 128, False),
])
def test_fwd_bf16(B, N, H, d, causal):
    qb, kb, vb = gen_dense(2, B, N, H, d, "bf16")
    o, lse = fa().fwd(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), causal=causal)
    o_ref, lse_ref = oracle.attn_fwd(bits_to_f64(qb), bits_to_f64(kb), bits_to_f64(vb), 1 / math.sqrt(d), causal)
    assert max_abs(host(o), o_ref) <= TOL_O_BF16
    assert max_abs(host(lse), lse_ref) <= TOL_LSE_BF16


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [33, 80, 100, 150, 192, 224, 250])
def test_fwd_bf16_few_key_blocks(N, causal, d):
    """One query block over 2 to 8 key blocks of 32: the key loop runs a whole pass of six
    steps or none, then a tail of up to five steps, and the last block's P V is taken from
    each of the six step phases (its buffer and P registers). The prologue's copies past the
    last block repeat it."""
    qb, kb, vb = gen_dense(11, 1, N, 2, d, "bf16")
    o, lse = fa().fwd(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), causal=causal)
    o_ref, lse_ref = oracle.attn_fwd(bits_to_f64(qb), bits_to_f64(kb), bits_to_f64(vb), 1 / math.sqrt(d), causal)
    assert max_abs(host(o), o_ref) <= TOL_O_BF16
    assert max_abs(host(lse), lse_ref) <= TOL_LSE_BF16


def test_fwd_bf16_large_scores_rescale():
    """Scores of tens of units force the running maximum (and the rescale) to move often."""
    B, N, H, d = 1, 777, 2, 128
    qb, kb, vb = gen_dense(7, B, N, H, d, "bf16")
    q = bits_to_f64(qb) * 8.0   # exact in bf16
    qb8 = synth.bf16_bits_from_f32(q.astype(np.float32))
    for causal in (False, True):
        o, lse = fa().fwd(dev_bf16(qb8), dev_bf16(kb), dev_bf16(vb), causal=causal)
        o_ref, lse_ref = oracle.attn_fwd(q, bits_to_f64(kb), bits_to_f64(vb), 1 / math.sqrt(d), causal)
        assert max_abs(host(o), o_ref) <= TOL_O_BF16
        assert max_abs(host(lse), lse_ref) <= TOL_LSE_BF16


@pytest.mark.parametrize("spikes", [
    (4.0, 8.0),     # scores about 90.5 and 181 (130 and 260 base-2 units above the rest):
                    # exp2 against the old pivot overflows fp32
    (0.75, 1.5),    # about 17 and 34 (24.5 and 49 base-2 units): against a pivot placed
                    # 16 units above a first block's maximum (about 6), the first stays under
                    # the kernel's bound on P (P about 2^3, no rescue), the second goes past
                    # it (P about 2^27, no inf)
])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_bf16_score_spikes_past_overflow(causal, spikes):
    """Keys whose scores jump far above every earlier score: the block holding each spike
    must be redone against a new maximum, or carried with large P where no accumulator can
    overflow. Values are exact in bf16."""
    B, N, H, d = 1, 900, 2, 128
    rng = np.random.default_rng(11)
    q = np.full((B, N, H, d), 2.0)
    k = np.round(rng.standard_normal((B, N, H, d)) * 8) / 8
    v = np.round(rng.standard_normal((B, N, H, d)) * 8) / 8
    k[:, 300] = spikes[0]    # score 2*c*128/sqrt(128)
    k[:, 650] = spikes[1]
    k[:, 651] = -spikes[1]   # a large negative score right after
    to = lambda x: dev_bf16(synth.bf16_bits_from_f32(x.astype(np.float32)))  # noqa: E731
    o, lse = fa().fwd(to(q), to(k), to(v), causal=causal)
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, 1 / math.sqrt(d), causal)
    o, lse = host(o), host(lse)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    assert max_abs(o, o_ref) <= TOL_O_BF16
    assert max_abs(lse, lse_ref) <= TOL_LSE_BF16


def test_fwd_bf16_full_size_every_element():
    """Causal B=2, H=16, N=8192, d=128 in the launch configuration the bench times: every
    element of O and LSE, head by head, against the float64 oracle (which materialises the
    8192 x 8192 S and P of each head)."""
    B, N, H, d = 2, 8192, 16, 128
    qb, kb, vb = gen_dense(2, B, N, H, d, "bf16")
    o, lse = fa().fwd(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), causal=True)
    o, lse = host(o), host(lse)
    scale = 1 / math.sqrt(d)
    worst_o = worst_l = 0.0
    for b in range(B):
        for h in range(H):
            o_ref, lse_ref = oracle.attention_head(bits_to_f64(qb[b, :, h]), bits_to_f64(kb[b, :, h]),
                                                   bits_to_f64(vb[b, :, h]), scale, causal=True)
            eo, el = max_abs(o[b, :, h], o_ref), max_abs(lse[b, h], lse_ref)
            assert eo <= TOL_O_BF16 and el <= TOL_LSE_BF16, (b, h, eo, el)
            worst_o, worst_l = max(worst_o, eo), max(worst_l, el)
    print(f"full-size causal forward, all {B * H} heads: max |O err| {worst_o:.2e}, max |LSE err| {worst_l:.2e}")


@pytest.mark.parametrize("causal", [True, False])
def test_fwd_bf16_identical_keys(causal):
    """All keys equal: every visible key gets the same weight, so O_i is the mean of the
    visible values (the prefix mean when causal) and LSE_i = scale q_i.k + ln(#visible)."""
    B, N, H, d = 1, 1000, 2, 128
    q, _, v = gen_dense(8, B, N, H, d, "bf16")
    k1 = synth.bnhd_tensor(8, synth.TENSOR_K, 1, 1, H, d)
    k = np.ascontiguousarray(np.broadcast_to(k1, (B, N, H, d)))
    o, lse = fa().fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), causal=causal)
    o, lse = host(o), host(lse)
    qf, kf, vf = bits_to_f64(q), bits_to_f64(k1)[0, 0], bits_to_f64(v)
    count = np.arange(1, N + 1) if causal else np.full(N, N)
    mean = np.cumsum(vf, axis=1) / count[None, :, None, None] if causal else \
        np.broadcast_to(vf.mean(axis=1, keepdims=True), vf.shape)
    lse_ref = np.einsum("bnhd,hd->bhn", qf, kf) / math.sqrt(d) + np.log(count)[None, None, :]
    assert max_abs(o, mean) <= TOL_O_BF16
    assert max_abs(lse, lse_ref) <= TOL_LSE_BF16


def test_fwd_bf16_deterministic():
    B, N, H, d = 1, 1000, 2, 128
    q, k, v = (dev_bf16(x) for x in gen_dense(3, B, N, H, d, "bf16"))
    o1, l1 = fa().fwd(q, k, v, causal=True)
    o2, l2 = fa().fwd(q, k, v, causal=True)
    import torch
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fwd_bf16_values_one_and_shift():
    """V = 1 gives O = 1; adding u to every key leaves O unchanged and moves LSE by scale*q.u
    (inputs on a 1/16 grid so that K + u is exact in bf16)."""
    torch = pytest.importorskip("torch")
    B, N, H, d = 1, 500, 2, 128
    rng = np.random.default_rng(5)
    q = np.round(rng.standard_normal((B, N, H, d)) * 16) / 16
    k = np.round(rng.standard_normal((B, N, H, d)) * 16) / 16
    u = np.round(rng.standard_normal(d) * 16) / 16
    v = np.round(rng.standard_normal((B, N, H, d)) * 16) / 16
    to = lambda x: dev_bf16(synth.bf16_bits_from_f32(x.astype(np.float32)))  # noqa: E731
    ones = torch.ones((B, N, H, d), dtype=torch.bfloat16, device="cuda")
    o1, _ = fa().fwd(to(q), to(k), ones, causal=True)
    assert max_abs(host(o1), np.ones((B, N, H, d))) <= 2 ** -8
    oa, la = fa().fwd(to(q), to(k), to(v), causal=True)
    ob, lb = fa().fwd(to(q), to(k + u), to(v), causal=True)
    scale = 1 / math.sqrt(d)
    assert max_abs(host(oa), host(ob)) <= TOL_O_BF16
    shift = scale * np.einsum("bnhd,d->bhn", q, u)
    assert max_abs(host(lb) - host(la), shift) <= 2 * TOL_LSE_BF16


# ----------------------------------------------------------------------------- varlen

def run_varlen(lengths, H, d, causal, dtype, seed, head_scale=None):
    cu = synth.cu_seqlens_from_lengths(lengths)
    q, k, v = (synth.varlen_tensor(seed, t, lengths, H, d, dtype, head_scale if t == synth.TENSOR_Q else None)
               for t in (synth.TENSOR_Q, synth.TENSOR_K, synth.TENSOR_V))
    to = dev_bf16 if dtype == "bf16" else dev_f32
    o, lse = fa().fwd_varlen(to(q), to(k), to(v), dev_i32(cu), max(lengths), causal=causal)
    f64 = bits_to_f64 if dtype == "bf16" else (lambda x: x.astype(np.float64))
    return cu, f64(q), f64(k), f64(v), host(o), host(lse)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_small_full_check(d, causal):
    lengths = [5, 0, 1, 63, 64, 65, 200, 129]
    cu, q, k, v, o, lse = run_varlen(lengths, 2, d, causal, "bf16", 3)
    o_ref, lse_ref = oracle.attn_fwd_varlen(q, k, v, cu, 1 / math.sqrt(d), causal)
    assert max_abs(o, o_ref) <= TOL_O_BF16
    assert max_abs(lse, lse_ref) <= TOL_LSE_BF16


@pytest.mark.parametrize("d", [64, 128])
def test_varlen_equal_lengths_each_sequence_once(d):
    """Sequences are visited longest first, ties by index: repeated lengths (zeros among
    them) must still map every sequence to exactly one set of workgroups. The output starts
    as NaN, so a sequence left out or computed twice into the wrong rows would show."""
    torch = pytest.importorskip("torch")
    lengths = [300, 0, 300, 47, 0, 300, 47, 600, 1]
    H = 4
    cu = synth.cu_seqlens_from_lengths(lengths)
    q, k, v = (synth.varlen_tensor(9, t, lengths, H, d, "bf16") for t in (synth.TENSOR_Q, synth.TENSOR_K, synth.TENSOR_V))
    T = sum(lengths)
    o = torch.full((T, H, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((H, T), float("nan"), dtype=torch.float32, device="cuda")
    qd, kd, vd, cud = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_i32(cu)
    st = fa().lib().fa_fwd_varlen(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                  cud.data_ptr(), len(lengths), T, max(lengths), H, H, d, 1 / math.sqrt(d), 1,
                                  fa().FA_DTYPE_BF16, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    o_ref, lse_ref = oracle.attn_fwd_varlen(bits_to_f64(q), bits_to_f64(k), bits_to_f64(v), cu, 1 / math.sqrt(d), True)
    assert max_abs(host(o), o_ref) <= TOL_O_BF16
    assert max_abs(host(lse), lse_ref) <= TOL_LSE_BF16


def test_varlen_f32():
    lengths = [7, 100, 33]
    cu, q, k, v, o, lse = run_varlen(lengths, 2, 64, True, "f32", 3)
    o_ref, lse_ref = oracle.attn_fwd_varlen(q, k, v, cu, 1 / 8, True)
    assert max_abs(o, o_ref) <= TOL_F32
    assert max_abs(lse, lse_ref) <= TOL_F32


def test_varlen_matches_dense_per_sequence():
    """Each packed sequence gives what the dense entry point gives for it alone."""
    lengths = [300, 77, 512]
    H, d = 2, 128
    cu, q, k, v, o, lse = run_varlen(lengths, H, d, True, "bf16", 4)
    for s, L in enumerate(lengths):
        a, e = cu[s], cu[s + 1]
        to = lambda x: dev_bf16(synth.bf16_bits_from_f32(x[a:e][None].astype(np.float32)))  # noqa: E731
        od, ld = fa().fwd(to(q), to(k), to(v), causal=True)
        assert max_abs(host(od)[0], o[a:e]) <= 1e-6
        assert max_abs(host(ld)[0], lse[:, a:e]) <= 1e-6


def test_varlen_full_size_every_element():
    """16 sequences of uniform lengths in [128, 4096], H=32, d=64, causal, Q x4 on heads
    16-31 (the bench's packed workload): every row of every sequence and head against the
    oracle."""
    lengths = synth.varlen_lengths(3, 16, 128, 4096).tolist()
    H, d = 32, 64
    cu, q, k, v, o, lse = run_varlen(lengths, H, d, True, "bf16", 3, head_scale=lambda h: 4.0 if h >= 16 else 1.0)
    o_ref, lse_ref = oracle.attn_fwd_varlen(q, k, v, cu, 1 / math.sqrt(d), True)
    eo, el = max_abs(o, o_ref), max_abs(lse, lse_ref)
    print(f"full-size packed forward ({sum(lengths)} tokens x {H} heads): max |O err| {eo:.2e}, max |LSE err| {el:.2e}")
    assert eo <= TOL_O_BF16 and el <= TOL_LSE_BF16
