"""Pins of the log-linear lift oracle (``oracle/loglinear.py``), CPU only.

The pages print no worked numbers for the lift, so the pins are what the
Log-Linear note fixes:
* the Fenwick split: the bucket of level l >= 1 holds 2^(l-1) positions and
  exists exactly when that power of two is in the binary expansion of t, and
  the level of s relative to t equals the highest differing bit of t and s,
  plus one ("Key design" 1; the closed form is the one the kernels use);
* equal weights at every level give the plain recurrence ("Key design" 2:
  the lift reduces to linear attention when the lambdas agree);
* weights equal across levels but varying over t scale the plain output;
* for linear attention (no decay, no A, B) the output is (Q K^T (.) M^H) V
  with M^H[t, s] = lam[t, level(t, s)] ("Key design" 3, the parallel form),
  computed by brute force;
* weight only on level 0 keeps the current token alone: o_t = (k_t . q_t) v_t.
"""
import numpy as np
import pytest

import oracle
from oracle import loglinear as ll_oracle
import workloads


def _raw(T, dk, dv, r_ab, r_kv, decay="channel", seed=0):
    return workloads.generic_raw(1, 2, T, dk, dv, r_ab, r_kv, "fp32", decay, seed=seed)


def _run(raw, lam):
    return ll_oracle.loglinear(raw["q"], raw["K"], raw["V"], raw["log_decay"], raw["A"], raw["B"], lam)


def test_fenwick_split_structure():
    for t in range(0, 300):
        lev = ll_oracle.fenwick_levels(t)
        assert lev[t] == 0
        for l in range(1, 12):
            n = int(np.sum(lev[:t] == l))
            assert n == ((1 << (l - 1)) if (t >> (l - 1)) & 1 else 0), (t, l)
        # closed form used by the chunked kernels: highest differing bit + 1
        for s in range(t):
            assert lev[s] == (t ^ s).bit_length(), (t, s)
        # the nearest keys sit in the finest buckets
        assert np.all(np.diff(lev[:t][::-1]) >= 0)
    assert ll_oracle.num_levels(4096) == 13 and ll_oracle.num_levels(1) == 1 and ll_oracle.num_levels(4097) == 14


@pytest.mark.parametrize("T,r_ab,r_kv,decay", [(40, 2, 1, "channel"), (33, 1, 2, "scalar"), (20, 0, 1, "channel")])
def test_equal_weights_are_plain_recurrence(T, r_ab, r_kv, decay):
    raw = _raw(T, 6, 5, r_ab, r_kv, decay, seed=T)
    L = ll_oracle.num_levels(T)
    out = _run(raw, np.ones((1, 2, T, L)))
    ref, _ = oracle.generic(raw["q"], raw["K"], raw["V"], raw["log_decay"], raw["A"], raw["B"])
    assert np.abs(out - ref).max() <= 1e-12 * np.abs(ref).max()
    c = np.random.default_rng(1).uniform(0.5, 2.0, size=(1, 2, T))
    out_c = _run(raw, np.repeat(c[..., None], L, axis=-1))
    assert np.abs(out_c - c[..., None] * ref).max() <= 1e-12 * np.abs(ref).max()


def test_linear_attention_parallel_form():
    T, dk, dv = 37, 5, 4
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 1, T, dk))
    k = rng.standard_normal((1, 1, T, dk))
    v = rng.standard_normal((1, 1, T, dv))
    L = ll_oracle.num_levels(T)
    lam = rng.uniform(0.0, 2.0, size=(1, 1, T, L))
    out = ll_oracle.loglinear(q, k[..., None, :], v[..., None, :], np.zeros((1, 1, T, dk)), None, None, lam)
    MH = np.zeros((T, T))
    for t in range(T):
        for s in range(t + 1):
            MH[t, s] = lam[0, 0, t, (t ^ s).bit_length()]
    ref = ((q[0, 0] @ k[0, 0].T) * MH) @ v[0, 0]
    assert np.abs(out[0, 0] - ref).max() <= 1e-12 * np.abs(ref).max()


def test_level_zero_only_is_current_token():
    T = 25
    raw = _raw(T, 6, 5, 2, 1, seed=7)
    L = ll_oracle.num_levels(T)
    lam = np.zeros((1, 2, T, L))
    lam[..., 0] = 1.0
    out = _run(raw, lam)
    k, v, q = raw["K"][..., 0, :].astype(np.float64), raw["V"][..., 0, :].astype(np.float64), raw["q"].astype(np.float64)
    ref = np.sum(k * q, axis=-1, keepdims=True) * v
    assert np.abs(out - ref).max() <= 1e-12 * np.abs(ref).max()


@pytest.mark.parametrize("T,dk,dv,r_ab,r_kv,decay", [(70, 6, 5, 2, 1, "channel"), (129, 4, 3, 1, 2, "scalar"),
                                                     (64, 5, 4, 0, 1, "channel"), (33, 3, 3, 3, 1, "channel")])
def test_recurrent_form_equals_per_query_definition(T, dk, dv, r_ab, r_kv, decay):
    """The note's recurrent form (bucket states merged as t advances) against the
    per-query walk over keys: two independent computations of the lift."""
    raw = _raw(T, dk, dv, r_ab, r_kv, decay, seed=T + dk)
    lam = workloads.loglinear_lambdas(1, 2, T, seed=T)
    a = _run(raw, lam)
    b = ll_oracle.loglinear_recurrent(raw["q"], raw["K"], raw["V"], raw["log_decay"], raw["A"], raw["B"], lam)
    assert np.abs(a - b).max() <= 1e-12 * np.abs(a).max()


def test_recurrent_form_single_level_weights():
    """Weight 1 on one level l only: the output reads exactly the keys at level l
    of each query (brute force over the closed-form level), for every l in use."""
    T, dk, dv = 45, 4, 3
    raw = _raw(T, dk, dv, 0, 1, "channel", seed=3)
    L = ll_oracle.num_levels(T)
    K = raw["K"][0, 0, :, 0].astype(np.float64)
    V = raw["V"][0, 0, :, 0].astype(np.float64)
    q = raw["q"][0, 0].astype(np.float64)
    G = np.cumsum(raw["log_decay"][0, 0].astype(np.float64), axis=0)   # diagonal decay: Phi(t, s) = exp(G_t - G_s)
    for l in range(L):
        lam = np.zeros((1, 2, T, L))
        lam[..., l] = 1.0
        got = ll_oracle.loglinear_recurrent(raw["q"], raw["K"], raw["V"], raw["log_decay"], None, None, lam)[0, 0]
        ref = np.zeros((T, dv))
        for t in range(T):
            for s in range(t + 1):
                if (0 if s == t else (t ^ s).bit_length()) == l:
                    ref[t] += (q[t] * np.exp(G[t] - G[s])) @ K[s] * V[s]
        assert np.abs(got - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max()), l
