"""CPU pins for the oracle's backward pass."""
import numpy as np
import pytest

import oracle
import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.BACKWARD_PINS, ids=lambda p: p.__name__)
def test_backward_pin(pin):
    pin(oracle.attn_bwd_head)


def test_delta_identity():
    """D_i = sum_j P_ij dP_ij equals sum_c dO_ic O_ic (so a kernel may form D from O)."""
    rng = np.random.default_rng(21)
    q, k, v, do = (rng.standard_normal((40, 8)) for _ in range(4))
    for causal in (False, True):
        g = oracle.attn_bwd_head(q, k, v, do, 0.3, causal)
        np.testing.assert_allclose(g["delta"], (do * g["o"]).sum(1), atol=1e-13)


def test_dense_backward_layout():
    rng = np.random.default_rng(22)
    q, k, v, do = (rng.standard_normal((2, 6, 2, 3)) for _ in range(4))
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, 0.6, True)
    for b in range(2):
        for h in range(2):
            g = oracle.attn_bwd_head(q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h], 0.6, True)
            np.testing.assert_array_equal(dq[b, :, h], g["dq"])
            np.testing.assert_array_equal(dk[b, :, h], g["dk"])
            np.testing.assert_array_equal(dv[b, :, h], g["dv"])
