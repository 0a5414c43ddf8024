"""Pins for the CPU oracle: checks that do not go through the oracle's own formulas.

Each pin takes the function under test as an argument so the same checks can be
run against deliberately broken variants (tests/test_oracle_mutants.py) and
shown to catch them. A pin raises AssertionError when violated.

Forward functions have the signature  f(q, k, v, scale, causal) -> (O, LSE)
for one (batch, head) slice; backward functions
g(q, k, v, do, scale, causal) -> dict(dq=, dk=, dv=).
"""
from __future__ import annotations

import math

import numpy as np

from oracle.algorithms import brute_force_attention


def _close(a, b, tol, what):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    err = np.where(both_inf, 0.0, np.abs(a - b))
    assert np.all(np.isfinite(err)), f"{what}: non-finite mismatch"
    scale = max(1.0, float(np.max(np.abs(np.where(np.isfinite(b), b, 0.0)))))
    assert float(np.max(err, initial=0.0)) <= tol * scale, \
        f"{what}: max err {float(np.max(err)):.3e} > {tol:.1e}"


# ---------------------------------------------------------------- forward pins

def pin_brute_force(f, seed=0):
    """Scalar brute force (pure Python, math.fsum) on tiny shapes, causal on and off."""
    rng = np.random.default_rng([seed, 1])
    for n, d in [(1, 1), (3, 2), (5, 4), (8, 3), (7, 4)]:
        for causal in (False, True):
            q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
            scale = 1.0 / math.sqrt(d) * rng.uniform(0.5, 2.0)
            o, lse = f(q, k, v, scale, causal)
            ob, lseb = brute_force_attention(q, k, v, scale, causal)
            _close(o, ob, 1e-12, f"O n={n} d={d} causal={causal}")
            _close(lse, lseb, 1e-12, f"LSE n={n} d={d} causal={causal}")


def pin_rows_sum_to_one(f, seed=0):
    """With every value row equal to 1, O = sum_j P_ij = 1 exactly (rows of P sum to one)."""
    rng = np.random.default_rng([seed, 2])
    for causal in (False, True):
        q, k = rng.standard_normal((33, 16)) * 3, rng.standard_normal((33, 16)) * 3
        v = np.ones((33, 5))
        o, _ = f(q, k, v, 0.25, causal)
        _close(o, np.ones_like(o), 1e-14, f"V=1 causal={causal}")


def pin_identical_keys(f, seed=0):
    """All keys equal: P is uniform over the visible keys, so O_i is the mean of the visible
    values and LSE_i = scale*q_i.k + ln(#visible)."""
    rng = np.random.default_rng([seed, 3])
    n, d = 19, 8
    q, v = rng.standard_normal((n, d)), rng.standard_normal((n, 6))
    kvec = rng.standard_normal(d)
    k = np.tile(kvec, (n, 1))
    scale = 0.7
    for causal in (False, True):
        o, lse = f(q, k, v, scale, causal)
        counts = np.arange(1, n + 1) if causal else np.full(n, n)
        if causal:
            mean_v = np.cumsum(v, axis=0) / counts[:, None]
        else:
            mean_v = np.tile(v.mean(axis=0), (n, 1))
        _close(o, mean_v, 1e-13, f"identical keys O causal={causal}")
        _close(lse, scale * (q @ kvec) + np.log(counts), 1e-13, f"identical keys LSE causal={causal}")


def pin_zero_queries(f, seed=0):
    """q = 0: every visible score is 0, O_i is the (prefix) mean of v and LSE_i = ln(#visible)."""
    rng = np.random.default_rng([seed, 4])
    n, d = 23, 4
    q = np.zeros((n, d))
    k, v = rng.standard_normal((n, d)), rng.standard_normal((n, 3))
    for causal in (False, True):
        o, lse = f(q, k, v, 1.3, causal)
        counts = np.arange(1, n + 1) if causal else np.full(n, n)
        mean_v = np.cumsum(v, axis=0) / counts[:, None] if causal else np.tile(v.mean(0), (n, 1))
        _close(o, mean_v, 1e-13, "zero queries O")
        _close(lse, np.log(counts), 1e-13, "zero queries LSE")


def pin_one_hot(f, seed=0):
    """Orthonormal keys and q_i = t * k_pi(i): the score is a = scale*t on key pi(i) and 0 on
    every other key, so O_i = (e^a v_pi(i) + sum_{j != pi(i)} v_j) / (e^a + n - 1) and
    LSE_i = ln(e^a + n - 1). A random permutation pi exposes transposed or swapped operands.
    The causal case uses pi = identity, where key i is the last visible key of query i.
    Large a (above 700) also exposes a softmax without the max subtraction."""
    rng = np.random.default_rng([seed, 5])
    n, d = 12, 16
    basis, _ = np.linalg.qr(rng.standard_normal((d, d)))
    k = basis[:n]
    v = rng.standard_normal((n, 5))
    for a in (3.0, 40.0, 800.0):
        scale = 0.5
        t = a / scale
        perm = rng.permutation(n)
        q = t * k[perm]
        o, lse = f(q, k, v, scale, False)
        ea = math.exp(min(a, 700.0))
        if a > 700:      # e^a dominates: O_i = v_pi(i), LSE = a + ln(1 + (n-1) e^-a)
            exp_o = v[perm]
            exp_lse = np.full(n, a)
        else:
            exp_o = (ea * v[perm] + (v.sum(0)[None, :] - v[perm])) / (ea + n - 1)
            exp_lse = np.full(n, math.log(ea + n - 1))
        _close(o, exp_o, 1e-12, f"one-hot O a={a}")
        _close(lse, exp_lse, 1e-12, f"one-hot LSE a={a}")
        q = t * k
        o, lse = f(q, k, v, scale, True)
        cnt = np.arange(n)                  # visible keys other than key i
        prefix = np.cumsum(v, axis=0) - v   # sum of v_j for j < i
        if a > 700:
            exp_o, exp_lse = v, np.full(n, a)
        else:
            exp_o = (ea * v + prefix) / (ea + cnt)[:, None]
            exp_lse = np.log(ea + cnt)
        _close(o, exp_o, 1e-12, f"one-hot causal O a={a}")
        _close(lse, exp_lse, 1e-12, f"one-hot causal LSE a={a}")


def pin_shift_invariance(f, seed=0):
    """Adding u to every key shifts row i of the scores by scale*q_i.u: softmax(x - c) =
    softmax(x), so O is unchanged and LSE_i moves by exactly scale*q_i.u."""
    rng = np.random.default_rng([seed, 6])
    n, d = 29, 8
    q, k, v = rng.standard_normal((n, d)), rng.standard_normal((n, d)), rng.standard_normal((n, 7))
    u = rng.standard_normal(d) * 2
    for causal in (False, True):
        o1, l1 = f(q, k, v, 0.4, causal)
        o2, l2 = f(q, k + u[None, :], v, 0.4, causal)
        _close(o2, o1, 1e-12, "shift O")
        _close(l2, l1 + 0.4 * (q @ u), 1e-12, "shift LSE")


def pin_top_left_causal(f):
    """Four queries against 128 keys with the top-left causal mask: the first query sees only
    key 0 (its output is v_0 exactly), query i sees keys 0..i."""
    rng = np.random.default_rng(7)
    q, k, v = rng.standard_normal((4, 8)), rng.standard_normal((128, 8)), rng.standard_normal((128, 3))
    o, lse = f(q, k, v, 0.3, True)
    _close(o[0], v[0], 1e-15, "first query output")
    _close(lse[0], 0.3 * float(q[0] @ k[0]), 1e-14, "first query LSE")
    ob, lb = brute_force_attention(q, k[:4], v[:4], 0.3, True)
    _close(o, ob, 1e-12, "top-left rows")


FORWARD_PINS = [pin_brute_force, pin_rows_sum_to_one, pin_identical_keys, pin_zero_queries,
                pin_one_hot, pin_shift_invariance, pin_top_left_causal]


# --------------------------------------------------------------- backward pins

def _loss_brute(q, k, v, do, scale, causal):
    o, _ = brute_force_attention(q, k, v, scale, causal)
    return math.fsum(float(a) * float(b) for ro, rd in zip(o, do) for a, b in zip(ro, rd))


def pin_finite_differences(g, seed=0):
    """Central differences of L = sum(O * dO) through the scalar brute-force forward."""
    rng = np.random.default_rng([seed, 8])
    hstep = 1e-6
    for n, d, causal in [(4, 3, False), (5, 2, True), (6, 4, True)]:
        q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
        scale = 0.8
        grads = g(q, k, v, do, scale, causal)
        for name, x in (("dq", q), ("dk", k), ("dv", v)):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += hstep
                xm[idx] -= hstep
                args_p = {"q": q, "k": k, "v": v}
                args_m = dict(args_p)
                key = name[1]
                args_p[key], args_m[key] = xp, xm
                num[idx] = (_loss_brute(args_p["q"], args_p["k"], args_p["v"], do, scale, causal)
                            - _loss_brute(args_m["q"], args_m["k"], args_m["v"], do, scale, causal)
                            ) / (2 * hstep)
            err = np.max(np.abs(grads[name] - num)) / max(1.0, np.max(np.abs(num)))
            assert err <= 1e-6, f"{name} n={n} causal={causal}: finite-difference rel err {err:.2e}"


def pin_gradient_sums(g, seed=0):
    """Rows of P sum to one, so sum_j dV_j = sum_i dO_i; shift invariance in K makes the
    loss independent of adding u to every key, so sum_j dK_j = 0."""
    rng = np.random.default_rng([seed, 9])
    n, d = 37, 8
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    for causal in (False, True):
        gr = g(q, k, v, do, 0.35, causal)
        _close(gr["dv"].sum(0), do.sum(0), 1e-12, "sum dV")
        _close(gr["dk"].sum(0), np.zeros(d), 1e-12, "sum dK")


BACKWARD_PINS = [pin_finite_differences, pin_gradient_sums]
