"""Pins of the backward oracle (``oracle/backward.py``), CPU only.

The pages give no backward formulas, so the backward oracle is pinned by the
definition of a gradient: central finite differences, in fp64, of the C
forward oracle (itself pinned by ``tests/test_oracle_pins.py``) for every
element of every input, on tiny shapes, for per-channel and scalar decay,
with and without A, B, and with an initial state and a final-state
cotangent.  A dropped term, a transposed operand or a wrong sign in any
gradient fails it.
"""
import numpy as np
import pytest

import oracle
from oracle import backward as bwd_oracle


def _inputs(T, dk, dv, r_ab, r_kv, scalar, seed):
    rng = np.random.default_rng(seed)
    x = dict(
        q=rng.standard_normal((1, 2, T, dk)),
        K=rng.standard_normal((1, 2, T, r_kv, dk)) * 0.5,
        V=rng.standard_normal((1, 2, T, r_kv, dv)) * 0.5,
        log_decay=-np.abs(rng.standard_normal((1, 2, T) if scalar else (1, 2, T, dk))) * 0.3,
        A=None if r_ab == 0 else rng.standard_normal((1, 2, T, r_ab, dk)) * 0.3,
        B=None if r_ab == 0 else rng.standard_normal((1, 2, T, r_ab, dk)) * 0.3,
        S0=rng.standard_normal((1, 2, dk, dv)) * 0.5,
    )
    dout = rng.standard_normal((1, 2, T, dv))
    dfin = rng.standard_normal((1, 2, dk, dv))
    return x, dout, dfin


def _loss(x, dout, dfin):
    out, S = oracle.generic(x["q"], x["K"], x["V"], x["log_decay"], x["A"], x["B"], initial_state=x["S0"])
    return float(np.sum(out * dout) + np.sum(S * dfin))


@pytest.mark.parametrize("T,dk,dv,r_ab,r_kv,scalar", [(6, 3, 2, 2, 1, False), (5, 3, 3, 1, 2, True),
                                                      (4, 2, 3, 0, 1, False)])
def test_backward_matches_finite_differences(T, dk, dv, r_ab, r_kv, scalar):
    x, dout, dfin = _inputs(T, dk, dv, r_ab, r_kv, scalar, seed=T * 10 + dk)
    g = bwd_oracle.backward(x["q"], x["K"], x["V"], x["log_decay"], x["A"], x["B"], dout, dfin, x["S0"])
    names = {"q": "dq", "K": "dK", "V": "dV", "log_decay": "dlog_decay", "A": "dA", "B": "dB", "S0": "dS0"}
    h = 1e-6
    for n, gn in names.items():
        if x[n] is None:
            assert g[gn] is None
            continue
        fd = np.zeros_like(x[n])
        it = np.nditer(x[n], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = {k: (None if v is None else v.copy()) for k, v in x.items()}
            xm = {k: (None if v is None else v.copy()) for k, v in x.items()}
            xp[n][idx] += h
            xm[n][idx] -= h
            fd[idx] = (_loss(xp, dout, dfin) - _loss(xm, dout, dfin)) / (2 * h)
        err = np.abs(g[gn] - fd).max() / max(1e-12, np.abs(fd).max())
        assert err < 1e-6, (n, err)


def test_backward_without_state_terms():
    """No initial state and no final-state cotangent: the same as zero ones."""
    x, dout, _ = _inputs(5, 3, 2, 2, 1, False, seed=3)
    a = bwd_oracle.backward(x["q"], x["K"], x["V"], x["log_decay"], x["A"], x["B"], dout)
    b = bwd_oracle.backward(x["q"], x["K"], x["V"], x["log_decay"], x["A"], x["B"], dout,
                            np.zeros((1, 2, 3, 2)), np.zeros((1, 2, 3, 2)))
    for n in a:
        assert np.array_equal(a[n], b[n]), n
