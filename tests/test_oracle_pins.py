"""Pins for the fp64 oracle: closed forms, brute force and special cases.

Each test checks the oracle against something other than itself: a
different formula for the same quantity (masked-matrix parallel form,
unrolled transition products, Householder algebra), or a special case whose
answer is fixed by the pages or by linear algebra.  The pages print no worked
numerical example, so there are no stored golden values.
"""
import numpy as np
import pytest

import oracle
import workloads


def _rng(seed=0):
    return np.random.default_rng(seed)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _causal(T):
    return np.tril(np.ones((T, T)))


# ---------------------------------------------------------------------------
# Linear attention and diagonal decay: the masked-matrix form O = (Q K^T * M) V
# (Log-linear attention note, "Overall framework": all-ones causal mask gives
# linear attention, a 1-semiseparable mask gives the gated scalar-decay case).


@pytest.mark.parametrize("r_kv", [1, 2])
def test_linear_attention_masked_form(r_kv):
    rng = _rng(1)
    H, T, dk, dv = 2, 23, 5, 4
    q = rng.standard_normal((H, T, dk))
    K = rng.standard_normal((H, T, r_kv, dk))
    V = rng.standard_normal((H, T, r_kv, dv))
    ld = np.zeros((H, T, dk))
    out, S = oracle.generic(q, K, V, ld)
    M = _causal(T)
    ref = np.zeros((H, T, dv))
    for r in range(r_kv):
        ref += ((q @ np.swapaxes(K[:, :, r], -1, -2)) * M) @ V[:, :, r]
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    Sref = sum(np.swapaxes(K[:, :, r], -1, -2) @ V[:, :, r] for r in range(r_kv))
    np.testing.assert_allclose(S, Sref, rtol=0, atol=1e-12)


def test_scalar_decay_semiseparable_mask():
    rng = _rng(2)
    H, T, dk, dv = 3, 31, 6, 5
    q = rng.standard_normal((H, T, dk))
    K = rng.standard_normal((H, T, 1, dk))
    V = rng.standard_normal((H, T, 1, dv))
    g = -rng.uniform(0.0, 0.3, (H, T))
    out, S = oracle.generic(q, K, V, g)
    G = np.cumsum(g, axis=-1)
    Mask = np.exp(G[:, :, None] - G[:, None, :]) * _causal(T)
    ref = ((q @ np.swapaxes(K[:, :, 0], -1, -2)) * Mask) @ V[:, :, 0]
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    wlast = np.exp(G[:, -1:] - G)  # decay from each token to the end
    Sref = np.swapaxes(K[:, :, 0] * wlast[..., None], -1, -2) @ V[:, :, 0]
    np.testing.assert_allclose(S, Sref, rtol=1e-12, atol=1e-12)


def test_diagonal_decay_closed_form():
    # GLA: o_t = sum_{s<=t} sum_i q_t[i] exp(G_t[i]-G_s[i]) k_s[i] v_s with G the
    # inclusive cumulative log decay (HDLA note, "Background": diagonal decay).
    rng = _rng(3)
    H, T, dk, dv = 2, 19, 4, 3
    q = rng.standard_normal((H, T, dk))
    K = rng.standard_normal((H, T, 1, dk))
    V = rng.standard_normal((H, T, 1, dv))
    ld = -rng.uniform(0.0, 0.5, (H, T, dk))
    out, S = oracle.generic(q, K, V, ld)
    G = np.cumsum(ld, axis=1)
    ref = np.zeros((H, T, dv))
    Sref = np.zeros((H, dk, dv))
    for h in range(H):
        for t in range(T):
            for s in range(t + 1):
                w = np.sum(q[h, t] * np.exp(G[h, t] - G[h, s]) * K[h, s, 0])
                ref[h, t] += w * V[h, s, 0]
        for s in range(T):
            Sref[h] += np.outer(np.exp(G[h, -1] - G[h, s]) * K[h, s, 0], V[h, s, 0])
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S, Sref, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------------------
# Arbitrary rank: the unrolled solution of the recurrence
#   S_t = Phi(t,0) S_0 + sum_{s<=t} Phi(t,s) K_s V_s^T,  Phi(t,s) = P_t ... P_{s+1}
# built from explicit transition matrices, independent of the oracle's loop.


def _transitions(ld, A, B):
    T, dk = ld.shape[0], A.shape[-1]
    P = np.zeros((T, dk, dk))
    for t in range(T):
        D = np.diag(np.exp(ld[t])) if ld.ndim == 2 else np.exp(ld[t]) * np.eye(dk)
        P[t] = D - A[t].T @ B[t]
    return P


@pytest.mark.parametrize("r_ab,r_kv,scalar", [(1, 1, False), (2, 1, False), (3, 2, False), (2, 2, True)])
def test_unrolled_transition_products(r_ab, r_kv, scalar):
    rng = _rng(10 + r_ab)
    T, dk, dv = 13, 5, 4
    q = rng.standard_normal((1, T, dk))
    K = rng.standard_normal((1, T, r_kv, dk))
    V = rng.standard_normal((1, T, r_kv, dv))
    ld = -rng.uniform(0, 0.4, (1, T) if scalar else (1, T, dk))
    A = rng.standard_normal((1, T, r_ab, dk)) * 0.4
    B = rng.standard_normal((1, T, r_ab, dk)) * 0.4
    S0 = rng.standard_normal((1, dk, dv))
    out, S = oracle.generic(q, K, V, ld, A, B, initial_state=S0)
    P = _transitions(ld[0], A[0], B[0])
    ref = np.zeros((T, dv))
    for t in range(T):
        Phi = np.eye(dk)
        acc = np.zeros((dk, dv))
        for s in range(t, -1, -1):          # Phi(t, s) accumulated right to left
            acc += Phi @ (K[0, s].T @ V[0, s])
            Phi = Phi @ P[s]
        acc += Phi @ S0[0]
        ref[t] = acc.T @ q[0, t]
        if t == T - 1:
            np.testing.assert_allclose(S[0], acc, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out[0], ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# HDLA decay (HDLA note, "Key design 2" and "Key design 3").


def _householder_P(k, lam, beta):
    H = np.eye(k.size) - beta * np.outer(k, k)
    return H @ np.diag(lam) @ H


def test_hdla_rewrite_equals_householder_congruence():
    rng = _rng(4)
    T, dk = 9, 7
    k = rng.standard_normal((T, dk))  # deliberately not normalised: the identity is algebraic
    v = rng.standard_normal((T, 3))
    ll = np.log(rng.uniform(0.2, 1.0, (T, dk)))
    beta = rng.uniform(0.0, 2.0, T)
    ld, A, B, K, V = oracle.hdla_to_generic(k, v, ll, beta)
    assert A.shape == (T, 2, dk) and B.shape == (T, 2, dk)
    for t in range(T):
        Prw = np.diag(np.exp(ld[t])) - A[t].T @ B[t]
        Ph = _householder_P(k[t], np.exp(ll[t]), beta[t])
        np.testing.assert_allclose(Prw, Ph, rtol=0, atol=1e-13)
        np.testing.assert_allclose(Prw, Prw.T, rtol=0, atol=1e-13)  # congruence keeps P symmetric
    np.testing.assert_allclose(K[:, 0], k)
    np.testing.assert_allclose(V[:, 0], beta[:, None] * v)


def test_gdn_rewrite():
    rng = _rng(5)
    T, dk = 6, 5
    k = _unit(rng.standard_normal((T, dk)))
    v = rng.standard_normal((T, 2))
    g = -rng.uniform(0, 0.5, T)
    beta = rng.uniform(0, 1, T)
    ld, A, B, K, V = oracle.gdn_to_generic(k, v, g, beta)
    for t in range(T):
        P = np.exp(ld[t]) * np.eye(dk) - A[t].T @ B[t]
        Pref = np.exp(g[t]) * (np.eye(dk) - beta[t] * np.outer(k[t], k[t]))
        np.testing.assert_allclose(P, Pref, rtol=0, atol=1e-14)


def test_hdla_reflection_squared_is_identity():
    # Unit k, beta = 2, lambda = 1: H is a reflection, H H = I, so P_t = I and the
    # model is plain causal linear attention with write 2 k v^T.
    rng = _rng(6)
    H_, T, dk, dv = 2, 17, 6, 5
    q = rng.standard_normal((H_, T, dk))
    k = _unit(rng.standard_normal((H_, T, dk)))
    v = rng.standard_normal((H_, T, dv))
    ll = np.zeros((H_, T, dk))
    beta = np.full((H_, T), 2.0)
    ref = 2.0 * ((q @ np.swapaxes(k, -1, -2)) * _causal(T)) @ v
    out_h, _ = oracle.hdla(q, k, v, ll, beta)
    np.testing.assert_allclose(out_h, ref, rtol=1e-12, atol=1e-12)
    ld, A, B, K, V = oracle.hdla_to_generic(k, v, ll, beta)
    out_g, _ = oracle.generic(q, K, V, ld, A, B)
    np.testing.assert_allclose(out_g, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("form", ["hdla", "gdn"])
def test_delta_rule_exact_recall(form):
    # Unit k, beta = 1, q_t = k_t: P_t k_t = 0 (the Householder factor annihilates k_t),
    # so o_t = S_{t-1}^T P_t k_t + v_t (k_t^T k_t) = v_t exactly, whatever the history.
    rng = _rng(7)
    H_, T, dk, dv = 2, 21, 8, 6
    k = _unit(rng.standard_normal((H_, T, dk)))
    v = rng.standard_normal((H_, T, dv))
    beta = np.ones((H_, T))
    S0 = rng.standard_normal((H_, dk, dv))
    if form == "hdla":
        ll = np.log(rng.uniform(0.3, 1.0, (H_, T, dk)))
        out, _ = oracle.hdla(k, k, v, ll, beta, initial_state=S0)
        conv = oracle.hdla_to_generic(k, v, ll, beta)
    else:
        g = -rng.uniform(0, 1.0, (H_, T))
        out, _ = oracle.gdn(k, k, v, g, beta, initial_state=S0)
        conv = oracle.gdn_to_generic(k, v, g, beta)
    np.testing.assert_allclose(out, v, rtol=0, atol=1e-12)
    ld, A, B, K, V = conv
    out_g, _ = oracle.generic(k, K, V, ld, A, B, initial_state=S0)
    np.testing.assert_allclose(out_g, v, rtol=0, atol=1e-12)


def test_three_forms_agree():
    rng = _rng(8)
    Bb, H_, T, dk, dv = 1, 3, 40, 8, 6
    q = rng.standard_normal((Bb, H_, T, dk))
    k = _unit(rng.standard_normal((Bb, H_, T, dk)))
    v = rng.standard_normal((Bb, H_, T, dv))
    S0 = rng.standard_normal((Bb, H_, dk, dv))
    ll = np.log(rng.uniform(0.5, 1.0, (Bb, H_, T, dk)))
    beta = rng.uniform(0, 2, (Bb, H_, T))
    o1, s1 = oracle.hdla(q, k, v, ll, beta, initial_state=S0)
    ld, A, B, K, V = oracle.hdla_to_generic(k, v, ll, beta)
    o2, s2 = oracle.generic(q, K, V, ld, A, B, initial_state=S0)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s1, s2, rtol=1e-12, atol=1e-12)
    g = -rng.uniform(0, 0.2, (Bb, H_, T))
    b1 = rng.uniform(0, 1, (Bb, H_, T))
    o3, s3 = oracle.gdn(q, k, v, g, b1, initial_state=S0)
    ld, A, B, K, V = oracle.gdn_to_generic(k, v, g, b1)
    o4, s4 = oracle.generic(q, K, V, ld, A, B, initial_state=S0)
    np.testing.assert_allclose(o3, o4, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s3, s4, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Chunk summaries (HLA note, "Affine maps and closure under composition").


def test_chunk_summary_is_transition_product_and_zero_state_run():
    rng = _rng(9)
    T, dk, dv, r_ab, r_kv, C = 22, 5, 3, 2, 2, 8      # chunks of 8, 8, 6 (ragged tail)
    K = rng.standard_normal((1, T, r_kv, dk))
    V = rng.standard_normal((1, T, r_kv, dv))
    ld = -rng.uniform(0, 0.3, (1, T, dk))
    A = rng.standard_normal((1, T, r_ab, dk)) * 0.3
    B = rng.standard_normal((1, T, r_ab, dk)) * 0.3
    sA, sB = oracle.chunk_summaries(K, V, ld, A, B, C)
    assert sA.shape == (1, 3, dk, dk) and sB.shape == (1, 3, dk, dv)
    P = _transitions(ld[0], A[0], B[0])
    for j in range(3):
        t0, t1 = j * C, min(T, (j + 1) * C)
        prod = np.eye(dk)
        for t in range(t0, t1):
            prod = P[t] @ prod
        np.testing.assert_allclose(sA[0, j], prod, rtol=1e-12, atol=1e-13)
        q = np.zeros((1, t1 - t0, dk))
        _, Sz = oracle.generic(q, K[:, t0:t1], V[:, t0:t1], ld[:, t0:t1], A[:, t0:t1], B[:, t0:t1])
        np.testing.assert_allclose(sB[0, j], Sz[0], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("C", [1, 3, 7, 16, 64, 100])
def test_composition_equals_sequential_run(C):
    rng = _rng(11)
    H_, T, dk, dv = 2, 50, 6, 4
    q = rng.standard_normal((H_, T, dk))
    K = rng.standard_normal((H_, T, 1, dk))
    V = rng.standard_normal((H_, T, 1, dv))
    k = _unit(K[:, :, 0])
    ll = np.log(rng.uniform(0.6, 1.0, (H_, T, dk)))
    beta = rng.uniform(0, 2, (H_, T))
    ld, A, B, K, V = oracle.hdla_to_generic(k, V[:, :, 0], ll, beta)
    S0 = rng.standard_normal((H_, dk, dv))
    sA, sB = oracle.chunk_summaries(K, V, ld, A, B, C)
    starts, Sf = oracle.compose(sA, sB, initial_state=S0)
    _, Sref = oracle.generic(q, K, V, ld, A, B, initial_state=S0)
    np.testing.assert_allclose(Sf, Sref, rtol=1e-11, atol=1e-12)
    for j in range(starts.shape[1]):
        t = j * C
        _, Sp = oracle.generic(q[:, :t], K[:, :t], V[:, :t], ld[:, :t], A[:, :t], B[:, :t], initial_state=S0)
        np.testing.assert_allclose(starts[:, j], Sp, rtol=1e-11, atol=1e-12)


def test_state_passing_split():
    rng = _rng(12)
    H_, T, dk, dv, r_ab = 2, 30, 5, 4, 2
    q = rng.standard_normal((H_, T, dk))
    K = rng.standard_normal((H_, T, 1, dk))
    V = rng.standard_normal((H_, T, 1, dv))
    ld = -rng.uniform(0, 0.3, (H_, T, dk))
    A = rng.standard_normal((H_, T, r_ab, dk)) * 0.3
    B = rng.standard_normal((H_, T, r_ab, dk)) * 0.3
    o, S = oracle.generic(q, K, V, ld, A, B)
    t1 = 11
    o1, S1 = oracle.generic(q[:, :t1], K[:, :t1], V[:, :t1], ld[:, :t1], A[:, :t1], B[:, :t1])
    o2, S2 = oracle.generic(q[:, t1:], K[:, t1:], V[:, t1:], ld[:, t1:], A[:, t1:], B[:, t1:], initial_state=S1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S2, S, rtol=1e-12, atol=1e-12)


def test_threads_do_not_change_results():
    rng = _rng(13)
    q = rng.standard_normal((5, 20, 4))
    K = rng.standard_normal((5, 20, 1, 4))
    V = rng.standard_normal((5, 20, 1, 3))
    ld = -rng.uniform(0, 0.3, (5, 20, 4))
    A = rng.standard_normal((5, 20, 2, 4)) * 0.3
    B = rng.standard_normal((5, 20, 2, 4)) * 0.3
    o1, s1 = oracle.generic(q, K, V, ld, A, B, nthreads=1)
    o2, s2 = oracle.generic(q, K, V, ld, A, B, nthreads=4)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


# ---------------------------------------------------------------------------
# Input recipe: bf16 rounding agrees with torch's round-to-nearest-even cast.


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 10
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 3.0e-39]  # ties and a subnormal
    ours = workloads.round_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(ours, ref)


def test_workload_shapes_and_determinism():
    spec = workloads.CONFIGS["hdla_fp32_small"]
    a = workloads.raw_for(spec)
    b = workloads.raw_for(spec)
    assert a["q"].shape == (1, 2, 512, 64) and a["beta"].shape == (1, 2, 512)
    assert all(np.array_equal(a[k], b[k]) for k in a)
    assert np.all(a["beta"] > 0) and np.all(a["beta"] < 2)
    assert np.all(a["log_lambda"] < 0)
    nrm = np.linalg.norm(a["k"].astype(np.float64), axis=-1)
    np.testing.assert_allclose(nrm, 1.0, atol=1e-6)
