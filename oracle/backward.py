"""Plain fp64 CPU oracle of the backward pass of the recurrence.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: it shares no code
with the HIP path, and only ``tests/`` uses it.

The pages train these models but print no backward formulas; this is the
chain rule applied to the token recurrence of the HDLA note ("Key design 3"),
written out token by token in reverse (backpropagation through time):

    forward   P_t = D_t - A_t B_t^T,  S_t = P_t S_{t-1} + K_t V_t^T,  o_t = S_t^T q_t
    loss      sum_t <do_t, o_t> + <dS_T, S_T>   (the given output and final-state cotangents)
    backward  G <- dS_T;  for t = T-1 .. 0:
                G   += q_t do_t^T                       (o_t reads S_t)
                dq_t = S_t do_t
                dK_t = G V_t,  dV_t = G^T K_t            (the write K_t V_t^T)
                dP_t = G S_{t-1}^T
                dA_t = -dP_t B_t,  dB_t = -dP_t^T A_t,  dlog_decay_t = diag(dP_t) (.) exp(log_decay_t)
                       (scalar decay: the sum of that diagonal times exp(g_t))
                G    = P_t^T G                          (becomes dS_{t-1})
              dS_init = G

with A_t, B_t the d_k x r_ab matrices whose columns are the rank rows of the
stored [.., r_ab, d_k] arrays (likewise K_t, V_t).  Pins:
``tests/test_backward_oracle_pins.py`` (central finite differences of the C
forward oracle in every input).
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def backward(q, K, V, log_decay, A, B, dout, dfinal=None, initial_state=None):
    """Gradients of sum <dout, out> + <dfinal, final_state> with respect to every
    input.  Shapes as the forward oracle (``lead`` = batch/head dims); dout
    [*lead, T, dv]; dfinal and initial_state [*lead, dk, dv] or None.
    Returns a dict of fp64 arrays: dq, dK, dV, dlog_decay, dA, dB (None when
    r_ab = 0) and dS0 (the initial state's gradient)."""
    q, K, V, ld, A, B, dout = (_f64(x) for x in (q, K, V, log_decay, A, B, dout))
    dfinal, S0 = _f64(dfinal), _f64(initial_state)
    lead = q.shape[:-2]
    T, dk = q.shape[-2:]
    dv = V.shape[-1]
    scalar = ld.shape == lead + (T,)
    flat = int(np.prod(lead)) if lead else 1
    rs = lambda x, tail: None if x is None else x.reshape((flat,) + tail)
    qf, Kf, Vf = rs(q, (T, dk)), rs(K, K.shape[-3:]), rs(V, V.shape[-3:])
    ldf = rs(ld, (T,) if scalar else (T, dk))
    Af, Bf = rs(A, A.shape[-3:]) if A is not None else None, rs(B, B.shape[-3:]) if B is not None else None
    dof = rs(dout, (T, dv))
    dff, S0f = rs(dfinal, (dk, dv)), rs(S0, (dk, dv))
    g = {n: np.zeros_like(x) for n, x in (("dq", qf), ("dK", Kf), ("dV", Vf), ("dlog_decay", ldf))}
    g["dA"] = None if Af is None else np.zeros_like(Af)
    g["dB"] = None if Bf is None else np.zeros_like(Bf)
    g["dS0"] = np.zeros((flat, dk, dv))
    for h in range(flat):
        # forward, keeping every state (S[t + 1] is the state after token t)
        S = np.zeros((T + 1, dk, dv))
        S[0] = 0.0 if S0f is None else S0f[h]
        P = np.empty((T, dk, dk))
        for t in range(T):
            lam = np.exp(ldf[h, t])
            D = lam * np.eye(dk) if scalar else np.diag(lam)
            P[t] = D if Af is None else D - Af[h, t].T @ Bf[h, t]
            S[t + 1] = P[t] @ S[t] + Kf[h, t].T @ Vf[h, t]
        G = np.zeros((dk, dv)) if dff is None else dff[h].copy()
        for t in range(T - 1, -1, -1):
            G += np.outer(qf[h, t], dof[h, t])
            g["dq"][h, t] = S[t + 1] @ dof[h, t]
            g["dK"][h, t] = (G @ Vf[h, t].T).T
            g["dV"][h, t] = (G.T @ Kf[h, t].T).T
            dP = G @ S[t].T
            lam = np.exp(ldf[h, t])
            g["dlog_decay"][h, t] = np.sum(np.diag(dP)) * lam if scalar else np.diag(dP) * lam
            if Af is not None:
                g["dA"][h, t] = -(dP @ Bf[h, t].T).T
                g["dB"][h, t] = -(dP.T @ Af[h, t].T).T
            G = P[t].T @ G
        g["dS0"][h] = G
    out = {}
    for n, x in g.items():
        if x is None:
            out[n] = None
        else:
            out[n] = x.reshape(lead + x.shape[1:])
    return out
