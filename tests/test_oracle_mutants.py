"""The pins must catch plausible mistakes: each planted mistake below is a broken copy of
the oracle's arithmetic (on the CPU), and at least one pin has to reject it."""
import numpy as np
import pytest

import oracle
import oracle_pins as pins


def _mask(S, causal, keep):
    if not causal:
        return S
    nq, nk = S.shape
    i, j = np.arange(nq)[:, None], np.arange(nk)[None, :]
    return np.where(keep(i, j), S, -np.inf)


def _fwd(q, k, v, scale, causal, *, score=None, keep=lambda i, j: j <= i, subtract_max=True,
         normalise=True, lse_form="ln", out=None):
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    S = score(q, k, scale) if score else scale * (q @ k.T)
    S = _mask(S, causal, keep)
    m = S.max(axis=1)
    mr = np.where(np.isfinite(m), m, 0.0) if subtract_max else np.zeros_like(m)
    with np.errstate(over="ignore", invalid="ignore"):
        E = np.exp(S - mr[:, None])
        l = E.sum(axis=1)
        P = E / l[:, None] if normalise else E
        O = out(P, v, k) if out else P @ v
        if lse_form == "ln":
            lse = mr + np.log(l)
        elif lse_form == "log2":
            lse = mr + np.log2(l)
        else:
            lse = np.log(l)
    return O, lse


FWD_MUTANTS = {
    "scale_dropped": lambda q, k, v, s, c: _fwd(q, k, v, s, c, score=lambda q, k, s: q @ k.T),
    "scale_squared": lambda q, k, v, s, c: _fwd(q, k, v, s, c, score=lambda q, k, s: s * s * (q @ k.T)),
    "scores_transposed": lambda q, k, v, s, c: _fwd(
        q, k, v, s, c, score=lambda q, k, s: (s * (k @ q.T)) if k.shape[0] == q.shape[0] else s * (q @ k.T)),
    "causal_reversed": lambda q, k, v, s, c: _fwd(q, k, v, s, c, keep=lambda i, j: j >= i),
    "causal_strict": lambda q, k, v, s, c: _fwd(q, k, v, s, c, keep=lambda i, j: j < i),
    "no_max_subtraction": lambda q, k, v, s, c: _fwd(q, k, v, s, c, subtract_max=False),
    "unnormalised_output": lambda q, k, v, s, c: _fwd(q, k, v, s, c, normalise=False),
    "lse_base2": lambda q, k, v, s, c: _fwd(q, k, v, s, c, lse_form="log2"),
    "lse_without_max": lambda q, k, v, s, c: _fwd(q, k, v, s, c, lse_form="nomax"),
    "p_transposed": lambda q, k, v, s, c: _fwd(
        q, k, v, s, c, out=lambda P, v, k: (P.T @ v) if P.shape[0] == P.shape[1] else P @ v),
    "values_are_keys": lambda q, k, v, s, c: _fwd(
        q, k, v, s, c, out=lambda P, v, k: P @ k if k.shape[1] == v.shape[1] else P @ v[:, ::-1]),
}


@pytest.mark.parametrize("name", sorted(FWD_MUTANTS))
def test_forward_mutant_is_caught(name):
    mutant = FWD_MUTANTS[name]
    failures = []
    for pin in pins.FORWARD_PINS:
        try:
            pin(mutant)
        except (AssertionError, ValueError, FloatingPointError):
            failures.append(pin.__name__)
    assert failures, f"no forward pin rejects the mutant {name}"


def _bwd(q, k, v, do, scale, causal, *, mutate):
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    _, _, P = oracle.attention_head(q, k, v, scale, causal, return_p=True)
    dv = P.T @ do
    dP = do @ v.T
    delta = (P * dP).sum(1)
    dS = P * (dP - delta[:, None])
    dq, dk = scale * (dS @ k), scale * (dS.T @ q)
    if mutate == "dk_scale_dropped":
        dk = dS.T @ q
    elif mutate == "ds_sign":
        dS2 = P * (dP + delta[:, None])
        dq, dk = scale * (dS2 @ k), scale * (dS2.T @ q)
    elif mutate == "dv_untransposed":
        dv = P @ do
    elif mutate == "dq_transposed_ds":
        dq = scale * (dS.T @ k)
    elif mutate == "delta_dropped":
        dS2 = P * dP
        dq, dk = scale * (dS2 @ k), scale * (dS2.T @ q)
    elif mutate == "dk_uses_k":
        dk = scale * (dS.T @ k)
    return {"dq": dq, "dk": dk, "dv": dv}


BWD_MUTANTS = ["dk_scale_dropped", "ds_sign", "dv_untransposed", "dq_transposed_ds",
               "delta_dropped", "dk_uses_k"]


@pytest.mark.parametrize("name", BWD_MUTANTS)
def test_backward_mutant_is_caught(name):
    mutant = lambda q, k, v, do, s, c: _bwd(q, k, v, do, s, c, mutate=name)  # noqa: E731
    failures = []
    for pin in pins.BACKWARD_PINS:
        try:
            pin(mutant)
        except AssertionError:
            failures.append(pin.__name__)
    assert failures, f"no backward pin rejects the mutant {name}"


def test_reference_passes_all_pins():
    for pin in pins.FORWARD_PINS:
        pin(oracle.attention_head)
    for pin in pins.BACKWARD_PINS:
        pin(oracle.attn_bwd_head)
