"""GPU edge cases beyond the configured workloads: very long sequences (offsets past 2^31
bytes per tensor would show here), a million-token decode cache, thousands of tiny packed
sequences, and empty inputs through the binding. Bounds as elsewhere: bf16 O <= 2e-2,
LSE <= 1e-3."""
import math

import numpy as np
import pytest

import oracle
import synth
from gpu_util import bits_to_f64, dev_bf16, dev_f32, dev_i32, host, max_abs

pytestmark = pytest.mark.gpu

TOL_O, TOL_LSE = 2e-2, 1e-3


def fa():
    import io_aware_softmax_03_amd as m
    return m


def test_fwd_long_sequence_sampled_rows():
    """B=1, H=1, N=131072, d=128, causal: 2.2e12 FLOP on 64 K query blocks x 4 K key blocks
    of one head; sampled rows against the oracle over their visible keys."""
    torch = pytest.importorskip("torch")
    N, d = 131072, 128
    gen = torch.Generator(device="cuda")
    gen.manual_seed(21)
    q, k, v = (torch.randn((1, N, 1, d), generator=gen, device="cuda", dtype=torch.bfloat16) for _ in range(3))
    o, lse = fa().fwd(q, k, v, causal=True)
    o, lse = host(o), host(lse)
    kh, vh = host(k[0, :, 0]), host(v[0, :, 0])
    for i in (0, 1, 255, 256, 65535, 65536, 100000, N - 1):
        o_ref, lse_ref = oracle.attention_head(host(q[0, i:i + 1, 0]), kh[:i + 1], vh[:i + 1], 1 / math.sqrt(d))
        assert max_abs(o[0, i, 0], o_ref[0]) <= TOL_O, i
        assert abs(lse[0, 0, i] - lse_ref[0]) <= TOL_LSE, i
    assert np.isfinite(o).all() and np.isfinite(lse).all()


def test_decode_million_token_cache():
    """One query per head against L = 2^20 cached keys (B=1, H=2, d=128, 1024 splits):
    each chunk holds 1024 keys; both heads checked in full."""
    torch = pytest.importorskip("torch")
    L, H, d = 1 << 20, 2, 128
    gen = torch.Generator(device="cuda")
    gen.manual_seed(22)
    q = torch.randn((1, H, d), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    kc, vc = (torch.randn((1, L, H, d), generator=gen, device="cuda", dtype=torch.bfloat16) for _ in range(2))
    o, lse = fa().decode(q, kc, vc, num_splits=1024)
    o, lse = host(o), host(lse)
    for h in range(H):
        o_ref, lse_ref = oracle.attn_decode_slice(host(q[0, h]), host(kc[0, :, h]), host(vc[0, :, h]), 1 / math.sqrt(d))
        assert max_abs(o[0, h], o_ref) <= TOL_O
        assert abs(lse[0, h] - lse_ref) <= TOL_LSE


def test_varlen_thousands_of_tiny_sequences():
    """2000 sequences of 0 to 3 tokens and one of 3000 (H=2, d=64, causal): most query
    blocks hold a single short sequence; checked in full."""
    rng = np.random.default_rng(23)
    lengths = rng.integers(0, 4, 2000).tolist() + [3000]
    H, d = 2, 64
    cu = synth.cu_seqlens_from_lengths(lengths)
    q, k, v = (synth.varlen_tensor(23, t, lengths, H, d) for t in (synth.TENSOR_Q, synth.TENSOR_K, synth.TENSOR_V))
    o, lse = fa().fwd_varlen(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_i32(cu), max(lengths), causal=True)
    o_ref, lse_ref = oracle.attn_fwd_varlen(bits_to_f64(q), bits_to_f64(k), bits_to_f64(v), cu, 1 / math.sqrt(d),
                                            True)
    assert max_abs(host(o), o_ref) <= TOL_O
    assert max_abs(host(lse), lse_ref) <= TOL_LSE


def test_empty_inputs_through_the_binding():
    torch = pytest.importorskip("torch")
    z = torch.empty((1, 0, 2, 128), dtype=torch.bfloat16, device="cuda")
    o, lse = fa().fwd(z, z, z, causal=True)
    assert o.shape == (1, 0, 2, 128) and lse.shape == (1, 2, 0)
    zb = torch.empty((0, 16, 2, 64), dtype=torch.bfloat16, device="cuda")
    o, lse = fa().fwd(zb, zb, zb)
    assert o.shape == zb.shape
    qd = torch.empty((0, 2, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.empty((0, 5, 2, 128), dtype=torch.bfloat16, device="cuda")
    o, lse = fa().decode(qd, kc, kc, num_splits=4)
    assert o.shape == (0, 2, 128) and lse.shape == (0, 2)


# ------------------------------------------------------------------ packed-sequence contract

def _varlen_inputs(lengths, H, d, dtype, seed):
    return [synth.varlen_tensor(seed, t, lengths, H, d, dtype) for t in (synth.TENSOR_Q, synth.TENSOR_K, synth.TENSOR_V)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [True, False])
def test_varlen_understated_max_seqlen_computes_every_row(dtype, causal):
    """max_seqlen only sizes the grid: with it far below the longest sequence, the
    workgroups take the extra query blocks and every row still matches the oracle."""
    lengths = [700, 50, 1300]
    H, d = 2, 64
    q, k, v = _varlen_inputs(lengths, H, d, dtype, 21)
    cu = synth.cu_seqlens_from_lengths(lengths)
    to = dev_bf16 if dtype == "bf16" else dev_f32
    o, lse = fa().fwd_varlen(to(q), to(k), to(v), dev_i32(cu), 100, causal=causal, validate=False)
    f64 = bits_to_f64 if dtype == "bf16" else (lambda x: x.astype(np.float64))
    o_ref, lse_ref = oracle.attn_fwd_varlen(f64(q), f64(k), f64(v), cu, 1 / math.sqrt(d), causal)
    tol_o, tol_l = (2e-2, 1e-3) if dtype == "bf16" else (1e-5, 1e-5)
    assert max_abs(host(o), o_ref) <= tol_o
    assert max_abs(host(lse), lse_ref) <= tol_l


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_varlen_clamps_offsets_outside_the_tensor(dtype):
    """Offsets that break the contract (a negative start, a sequence running past
    total_tokens) are clamped into the tensor: the rows of the clamped sequences match the
    oracle on the clamped offsets, and nothing is written past row T (guard rows keep their
    sentinel)."""
    import ctypes
    import torch
    from io_aware_softmax_03_amd import _clib
    T, G, H, d = 800, 64, 2, 64
    bad = np.array([-5, 300, 300, 900], dtype=np.int32)       # sequences [0,300), [300,300), [300,800)
    clamped = np.array([0, 300, 300, 800], dtype=np.int32)
    q, k, v = _varlen_inputs([T], H, d, dtype, 22)
    to = dev_bf16 if dtype == "bf16" else dev_f32
    tq, tk, tv = to(q), to(k), to(v)
    sentinel = 7.0
    o_buf = torch.full((T + G, H, d), sentinel, dtype=tq.dtype, device="cuda")
    lse_buf = torch.full((H * T + G,), sentinel, dtype=torch.float32, device="cuda")
    cu = dev_i32(bad)
    code = _clib.FA_DTYPE_BF16 if dtype == "bf16" else _clib.FA_DTYPE_F32
    st = _clib.lib().fa_fwd_varlen(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o_buf.data_ptr(), lse_buf.data_ptr(),
                                   cu.data_ptr(), 3, T, 500, H, H, d, 1 / math.sqrt(d), 1, code,
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == _clib.FA_OK
    torch.cuda.synchronize()
    o, lse = host(o_buf[:T]), host(lse_buf[:H * T]).reshape(H, T)
    assert np.all(host(o_buf[T:]) == sentinel) and np.all(host(lse_buf[H * T:]) == sentinel)
    f64 = bits_to_f64 if dtype == "bf16" else (lambda x: x.astype(np.float64))
    o_ref, lse_ref = oracle.attn_fwd_varlen(f64(q), f64(k), f64(v), clamped, 1 / math.sqrt(d), True)
    tol_o, tol_l = (2e-2, 1e-3) if dtype == "bf16" else (1e-5, 1e-5)
    assert max_abs(o, o_ref) <= tol_o
    assert max_abs(lse, lse_ref) <= tol_l
