"""Plain fp64 CPU oracle of the log-linear lift of the recurrence.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: it shares no code
with the HIP path, and only ``tests/`` uses it.

What it computes (Log-Linear note, "Key design" 1-3):

* the Fenwick split of the prefix of position t (positions counted from 0):
  the current token is a bucket of its own at level 0; the rest [0, t) is cut
  greedily from the right, each time taking off the lowest set bit of the
  remaining length r as a bucket [r - lssb(r), r) at level log2(lssb(r)) + 1
  (``fenwick_levels``, written from that greedy description);
* the lifted output, every key weighted by the query's weight for the key's
  bucket level, with the recurrence's own transport between them:
      o_t = sum_{s <= t} lam[t, level(t, s)] (Phi(t, s) K_s V_s^T)^T q_t,
      Phi(t, s) = P_t P_{t-1} ... P_{s+1},   P_t = D_t - A_t B_t^T,
  i.e. the bucket states S_t^(l) = sum_{s in bucket l} Phi(t, s) K_s V_s^T
  read out as o_t = sum_l lam[t, l] S_t^(l)^T q_t (the note's recurrent form,
  with the transport of the HDLA note's "Key design 3" recurrence in place of
  plain accumulation; with D = I and no A, B it is the note's linear-attention
  case).

Nothing is blocked or reordered: per query, the keys are walked from t down
to 0, carrying Phi(t, s) as a running product.

``loglinear_recurrent`` computes the same output a second, independent way,
from the note's recurrent form ("Key design" 1-2): one state per bucket level,
advanced token by token.  At every step each bucket state is transported by
P_t; when t - 1 ends in z one-bits, the buckets of levels 0 .. z of t - 1
together make up the single bucket of level z + 1 of t, so their states are
summed into it (the Fenwick merge), and the new token's write K_t V_t^T
starts level 0.  Its cost is O(T log T) state products, so it reaches every
level of long sequences.  The two are pinned against each other (and each
against the plain recurrence) by ``tests/test_loglinear_oracle_pins.py``.
"""
from __future__ import annotations

import numpy as np


def fenwick_levels(t: int) -> np.ndarray:
    """Bucket level of every position s <= t in the Fenwick split of [0, t]."""
    lev = np.empty(t + 1, dtype=np.int64)
    lev[t] = 0                      # the current token: the size-1 bucket
    r = t
    while r > 0:
        size = r & -r               # lowest set bit of the remaining length
        lev[r - size:r] = size.bit_length()   # log2(size) + 1
        r -= size
    return lev


def num_levels(T: int) -> int:
    """Levels a sequence of T tokens can use: 0 .. highest level of position T-1."""
    return 1 + int(T - 1).bit_length() if T > 0 else 0


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def loglinear(q, K, V, log_decay, A, B, lam):
    """Lifted output.  Shapes as the base oracle (``lead`` = batch/head dims);
    lam [*lead, T, L] with L >= num_levels(T).  Returns out [*lead, T, dv] fp64."""
    q, K, V, ld, A, B, lam = (_f64(x) for x in (q, K, V, log_decay, A, B, lam))
    lead = q.shape[:-2]
    T, dk = q.shape[-2:]
    dv = V.shape[-1]
    flat = int(np.prod(lead)) if lead else 1
    qf = q.reshape(flat, T, dk)
    Kf = K.reshape((flat,) + K.shape[-3:])
    Vf = V.reshape((flat,) + V.shape[-3:])
    ldf = ld.reshape((flat,) + ld.shape[len(lead):])
    Af = None if A is None else A.reshape((flat,) + A.shape[-3:])
    Bf = None if B is None else B.reshape((flat,) + B.shape[-3:])
    lf = lam.reshape(flat, T, lam.shape[-1])
    out = np.zeros((flat, T, dv))
    for h in range(flat):
        P = np.empty((T, dk, dk))
        for t in range(T):
            d = np.exp(ldf[h, t])
            D = np.diag(d) if np.ndim(d) == 1 else d * np.eye(dk)
            P[t] = D if Af is None else D - Af[h, t].T @ Bf[h, t]
        for t in range(T):
            lev = fenwick_levels(t)
            S = np.zeros((dk, dv))
            Phi = np.eye(dk)        # Phi(t, s), starting at s = t
            for s in range(t, -1, -1):
                S += lf[h, t, lev[s]] * (Phi @ (Kf[h, s].T @ Vf[h, s]))
                Phi = Phi @ P[s]    # Phi(t, s - 1) = Phi(t, s) P_s
            out[h, t] = S.T @ qf[h, t]
    return out.reshape(lead + (T, dv))


def loglinear_recurrent(q, K, V, log_decay, A, B, lam):
    """Lifted output from per-level bucket states (the recurrent form).  Same
    arguments and result as :func:`loglinear`."""
    q, K, V, ld, A, B, lam = (_f64(x) for x in (q, K, V, log_decay, A, B, lam))
    lead = q.shape[:-2]
    T, dk = q.shape[-2:]
    dv = V.shape[-1]
    flat = int(np.prod(lead)) if lead else 1
    qf = q.reshape(flat, T, dk)
    Kf = K.reshape((flat,) + K.shape[-3:])
    Vf = V.reshape((flat,) + V.shape[-3:])
    ldf = ld.reshape((flat,) + ld.shape[len(lead):])
    Af = None if A is None else A.reshape((flat,) + A.shape[-3:])
    Bf = None if B is None else B.reshape((flat,) + B.shape[-3:])
    lf = lam.reshape(flat, T, lam.shape[-1])
    out = np.zeros((flat, T, dv))
    for h in range(flat):
        states = {}                                   # level -> bucket state (d_k x d_v)
        for t in range(T):
            if t > 0:
                z = 0                                 # trailing one-bits of t - 1
                while ((t - 1) >> z) & 1:
                    z += 1
                merged = np.zeros((dk, dv))
                for l in range(z + 1):
                    if l in states:
                        merged += states.pop(l)
                states[z + 1] = merged
                d = np.exp(ldf[h, t])
                P = np.diag(d) if np.ndim(d) == 1 else d * np.eye(dk)
                if Af is not None:
                    P = P - Af[h, t].T @ Bf[h, t]
                levels = sorted(states)
                moved = np.matmul(P, np.stack([states[l] for l in levels]))
                for i, l in enumerate(levels):
                    states[l] = moved[i]
            states[0] = Kf[h, t].T @ Vf[h, t]
            o = np.zeros(dv)
            for l, S in states.items():
                o += lf[h, t, l] * (S.T @ qf[h, t])
            out[h, t] = o
    return out.reshape(lead + (T, dv))
