"""CPU pins for the oracle's forward definition and the pages' softmax claims."""
import math

import numpy as np
import pytest

import oracle
import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.FORWARD_PINS, ids=lambda p: p.__name__)
def test_forward_pin(pin):
    pin(oracle.attention_head)


def test_dense_layout_matches_per_head():
    """attn_fwd walks [B, N, H, d] slices and writes LSE as [B, H, N]."""
    rng = np.random.default_rng(11)
    q, k, v = (rng.standard_normal((2, 9, 3, 4)) for _ in range(3))
    o, lse = oracle.attn_fwd(q, k, v, 0.5, True)
    for b in range(2):
        for h in range(3):
            ob, lb = oracle.brute_force_attention(q[b, :, h], k[b, :, h], v[b, :, h], 0.5, True)
            np.testing.assert_allclose(o[b, :, h], ob, atol=1e-12)
            np.testing.assert_allclose(lse[b, h], lb, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bc", [1, 7, 64, 200])
def test_tiled_online_equals_batch(causal, bc):
    """Online softmax over key blocks gives the batch softmax result up to summation order
    (FlashAttention: IO-aware exact attention, 'Online softmax')."""
    rng = np.random.default_rng([12, bc])
    n, d = 200, 16
    q, k, v = rng.standard_normal((n, d)) * 2, rng.standard_normal((n, d)) * 2, rng.standard_normal((n, 8))
    o1, l1 = oracle.attention_head(q, k, v, 0.25, causal)
    o2, l2 = oracle.tiled_online_attention_head(q, k, v, 0.25, causal, block_cols=bc)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-12)


@pytest.mark.parametrize("threshold", [0.0, 2.0, 8.0 * math.log(2)])
def test_stale_pivot_is_exact(threshold):
    """Keeping an old maximum as the pivot unless the new one exceeds it by a threshold
    leaves the result unchanged ('And on Blackwell': any pivot shared by l and O works)."""
    rng = np.random.default_rng(13)
    n, d = 300, 32
    q, k, v = rng.standard_normal((n, d)) * 3, rng.standard_normal((n, d)), rng.standard_normal((n, 8))
    for causal in (False, True):
        o1, l1 = oracle.attention_head(q, k, v, 1 / math.sqrt(d), causal)
        o2, l2 = oracle.tiled_online_attention_head(q, k, v, 1 / math.sqrt(d), causal,
                                                    block_cols=32, stale_threshold=threshold)
        np.testing.assert_allclose(o2, o1, atol=1e-12)
        np.testing.assert_allclose(l2, l1, atol=1e-12)


def test_two_pass_online_and_batch_softmax_agree():
    """Two-pass softmax, one-pass online softmax and the direct definition agree, and
    softmax(x - c) = softmax(x) ('Flash Attention and the Online-Softmax Trick', §3)."""
    rng = np.random.default_rng(14)
    x = rng.standard_normal((10, 257)) * 20
    direct = np.exp(x - x.max(1, keepdims=True))
    direct /= direct.sum(1, keepdims=True)
    np.testing.assert_allclose(oracle.softmax_two_pass(x), direct, atol=1e-15)
    for chunk in (1, 16, 100, 257):
        np.testing.assert_allclose(oracle.softmax_online(x, chunk), direct, atol=1e-14)
    c = rng.standard_normal((10, 1)) * 50
    np.testing.assert_allclose(oracle.softmax_two_pass(x - c), direct, atol=1e-14)
    np.testing.assert_allclose(direct.sum(1), 1.0, atol=1e-15)


def test_unstabilised_softmax_overflows():
    """Negative control: exponentiating scores without subtracting the maximum overflows in
    float64 once scores pass ~710, while the oracle stays finite."""
    s = np.array([[800.0, 1.0, -3.0]])
    with np.errstate(over="ignore", invalid="ignore"):
        w = np.exp(s)
        naive = w / w.sum()
    assert not np.all(np.isfinite(naive))
    q = np.array([[800.0, 0.0]])
    k = np.array([[1.0, 0.0], [0.0, 1.0], [0.0, 0.0]])
    v = np.eye(3)
    o, lse = oracle.attention_head(q, k, v, 1.0)
    assert np.all(np.isfinite(o)) and np.isfinite(lse).all()
    np.testing.assert_allclose(o[0], [1.0, 0.0, 0.0], atol=1e-300)


def test_fully_masked_row_convention():
    """A query with no visible key (no keys at all) has O = 0 and LSE = -inf."""
    q = np.ones((2, 4))
    k = np.zeros((0, 4))
    v = np.zeros((0, 3))
    o, lse = oracle.attention_head(q, k, v, 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
