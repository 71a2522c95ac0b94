"""Plain fp64 CPU oracle of the query-conditioned chunk composition (HLA).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: it shares no code
with the HIP path, and only ``tests/`` and ``bench.py``'s ``cpu_baseline``
leg use it.

What it computes (HLA note, "Core method" and "Method steps", steps 2, 5
and 7), for one recurrence S_t = P_t S_{t-1} + K_t V_t^T with
P_t = D_t - A_t B_t^T (HDLA note, "Key design 3"):

* the exact affine pair (A_j, B_j) of every chunk of ``chunk`` tokens, by
  composing the token maps of the chunk in time order (step 2);
* for every query token i in chunk c = i // chunk, starting from a zero state,
  each earlier chunk j = 0 .. c-1 in time order applied with the query's gate
  w = gates[i, j] as  S <- ((1 - w) I + w A_j) S + w B_j  (step 5), where a
  gate below ``theta`` counts as zero (step 7: thresholded to zero, no
  renormalisation);
* then the current chunk's own tokens up to and including i, each as
  S <- P_t S + K_t V_t^T (the causal prefix of step 5, gate fixed at 1);
* the readout o_i = S^T q_i (no 1/sqrt(d_k) scale: the caller scales q, as
  for the base path).

Every step is the definition written out with one matrix product per token
or chunk; nothing is blocked, fused or reordered.  Pins:
``tests/test_hla_oracle_pins.py``.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def _token_maps(K, V, log_decay, A, B):
    """Per token: P_t (d_k x d_k) and the write K_t V_t^T (d_k x d_v), fp64."""
    T, r_kv, dk = K.shape
    P = np.empty((T, dk, dk))
    W = np.empty((T, dk, V.shape[-1]))
    for t in range(T):
        lam = np.exp(log_decay[t])
        D = np.diag(lam) if np.ndim(lam) == 1 else lam * np.eye(dk)
        P[t] = D if A is None else D - A[t].T @ B[t]
        W[t] = K[t].T @ V[t]
    return P, W


def hla(q, K, V, log_decay, A, B, gates, chunk: int, theta: float = 0.0, queries=None):
    """Query-conditioned composition of exact chunk transitions.

    Shapes (``lead`` = batch/head dims): q [*lead, T, dk]; K [*lead, T, r_kv, dk];
    V [*lead, T, r_kv, dv]; log_decay [*lead, T, dk] or [*lead, T]; A, B
    [*lead, T, r_ab, dk] or None; gates [*lead, T, N] with N = ceil(T / chunk)
    (entry [i, j] is query i's gate for chunk j; entries j >= i // chunk are
    not used).  ``queries``: token indices to evaluate (default all; the other
    rows of the result stay zero).  Returns out [*lead, T, dv] in fp64.
    """
    q, K, V, ld, A, B, gates = (_f64(x) for x in (q, K, V, log_decay, A, B, gates))
    lead = q.shape[:-2]
    T, dk = q.shape[-2:]
    dv = V.shape[-1]
    N = -(-T // chunk)
    assert gates.shape == lead + (T, N)
    flat = int(np.prod(lead)) if lead else 1
    qf, Kf, Vf = q.reshape(flat, T, dk), K.reshape((flat,) + K.shape[-3:]), V.reshape((flat,) + V.shape[-3:])
    ldf = ld.reshape((flat,) + ld.shape[len(lead):])
    Af = None if A is None else A.reshape((flat,) + A.shape[-3:])
    Bf = None if B is None else B.reshape((flat,) + B.shape[-3:])
    gf = gates.reshape(flat, T, N)
    out = np.zeros((flat, T, dv))
    I = np.eye(dk)
    for h in range(flat):
        P, W = _token_maps(Kf[h], Vf[h], ldf[h], None if Af is None else Af[h], None if Bf is None else Bf[h])
        # step 2: exact pair of each chunk, composing its token maps in order
        sumA = np.empty((N, dk, dk))
        sumB = np.empty((N, dk, dv))
        for j in range(N):
            Aj, Bj = I.copy(), np.zeros((dk, dv))
            for t in range(j * chunk, min(T, (j + 1) * chunk)):
                Aj = P[t] @ Aj
                Bj = P[t] @ Bj + W[t]
            sumA[j], sumB[j] = Aj, Bj
        for i in (range(T) if queries is None else queries):
            c = i // chunk
            S = np.zeros((dk, dv))
            # step 5: gated history chunks in time order (step 7: gates below theta are zero)
            for j in range(c):
                w = gf[h, i, j]
                if w < theta:
                    w = 0.0
                S = ((1.0 - w) * I + w * sumA[j]) @ S + w * sumB[j]
            # the current chunk's causal prefix, gate 1
            for t in range(c * chunk, i + 1):
                S = P[t] @ S + W[t]
            out[h, i] = S.T @ qf[h, i]
    return out.reshape(lead + (T, dv))
