"""Plain fp64 CPU oracle for the generalized linear-attention recurrence.

TEST INFRASTRUCTURE ONLY.  This package is the correctness reference the HIP
path is checked against.  It shares no code with that path and imports
nothing from it; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.

What it computes (pages cited by title and section):

* ``generic``      -- S_t = (D_t - A_t B_t^T) S_{t-1} + K_t V_t^T, o_t = S_t^T q_t,
                      with P_t formed explicitly (HDLA note, "Key design 3").
* ``hdla``         -- P_t = (I - b k k^T) Diag(lambda) (I - b k k^T), write b k v^T
                      (HDLA note, "Key design 2"); never touches A, B.
* ``gdn``          -- P_t = exp(g)(I - b k k^T), write b k v^T (HLA note,
                      "Prerequisites: Gated DeltaNet").
* ``chunk_summaries`` -- exact per-chunk affine pair (A_j, B_j) from the state
                      [0 | I] with values [V | 0] (HLA note, "Affine maps and
                      closure under composition").
* ``compose``      -- S_j = A_j S_{j-1} + B_j over the chunk pairs.
* ``hdla_to_generic`` / ``gdn_to_generic`` -- the diagonal-minus-low-rank
                      rewrite P_t = D_t - A_t B_t^T of each decay (HDLA note,
                      "Key design 3" states the rank-2 form exists; the
                      factor pair used here is derived in the function).

Parity pins: every function above is pinned by ``tests/test_oracle_pins.py``
against closed forms, brute force and special cases fixed by the pages and
by linear algebra.  No function here is "parity unpinned".

The C core (``oracle.c``) is built with gcc by :func:`build` into
``oracle/liboracle.so``; OpenMP threads over (batch, head).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` with gcc (fp64, no fast-math) into ``liboracle.so``."""
    global _lib
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
        _lib = None
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int
        lib.oracle_generic.argtypes = [i64, i64, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P, i32]
        lib.oracle_hdla.argtypes = [i64, i64, i32, i32, P, P, P, P, P, P, P, P, i32]
        lib.oracle_gdn.argtypes = [i64, i64, i32, i32, P, P, P, P, P, P, P, P, i32]
        lib.oracle_chunk_summaries.argtypes = [i64, i64, i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, i32]
        for f in (lib.oracle_generic, lib.oracle_hdla, lib.oracle_gdn, lib.oracle_chunk_summaries):
            f.restype = ctypes.c_int
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = []
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, name: str):
    if rc != 0:
        raise RuntimeError(f"{name} failed with code {rc}")


def generic(q, K, V, log_decay, A=None, B=None, initial_state=None, nthreads: int = 0,
            want_out: bool = True) -> Tuple[Optional[np.ndarray], np.ndarray]:
    """Token-by-token recurrence with explicit P_t = D_t - A_t B_t^T.

    Shapes (leading dims ``lead`` are any batch/head dims, flattened inside):
      q [*lead, T, dk]; K [*lead, T, r_kv, dk]; V [*lead, T, r_kv, dv];
      log_decay [*lead, T, dk] (per channel) or [*lead, T] (scalar);
      A, B [*lead, T, r_ab, dk] or None (r_ab = 0);
      initial_state [*lead, dk, dv] or None (zero).
    Returns (out [*lead, T, dv] or None, final_state [*lead, dk, dv]).
    """
    q, K, V, ld = _f64(q), _f64(K), _f64(V), _f64(log_decay)
    lead = q.shape[:-2]
    T, dk = q.shape[-2], q.shape[-1]
    r_kv, dv = K.shape[-2], V.shape[-1]
    assert K.shape == lead + (T, r_kv, dk) and V.shape == lead + (T, r_kv, dv)
    scalar = ld.shape == lead + (T,)
    assert scalar or ld.shape == lead + (T, dk)
    if A is None:
        r_ab = 0
        A_ = B_ = None
    else:
        A_, B_ = _f64(A), _f64(B)
        r_ab = A_.shape[-2]
        assert A_.shape == lead + (T, r_ab, dk) and B_.shape == A_.shape
    BH = int(np.prod(lead)) if lead else 1
    S0 = _f64(initial_state)
    if S0 is not None:
        assert S0.shape == lead + (dk, dv)
    out = np.empty(lead + (T, dv)) if want_out else None
    Sf = np.empty(lead + (dk, dv))
    rc = _load().oracle_generic(BH, T, dk, dv, r_ab, r_kv, int(scalar), _ptr(q), _ptr(K), _ptr(V),
                                _ptr(ld), _ptr(A_), _ptr(B_), _ptr(S0), _ptr(out), _ptr(Sf), nthreads)
    _check(rc, "oracle_generic")
    return out, Sf


def hdla(q, k, v, log_lambda, beta, initial_state=None, nthreads: int = 0):
    """HDLA in Householder form: P_t = H_t Diag(lambda_t) H_t, H_t = I - beta_t k_t k_t^T,
    write beta_t k_t v_t^T.  q, k [*lead,T,dk]; v [*lead,T,dv]; log_lambda [*lead,T,dk];
    beta [*lead,T].  Returns (out, final_state)."""
    q, k, v, ll, b = _f64(q), _f64(k), _f64(v), _f64(log_lambda), _f64(beta)
    lead = q.shape[:-2]
    T, dk = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    assert k.shape == q.shape and ll.shape == q.shape and b.shape == lead + (T,)
    BH = int(np.prod(lead)) if lead else 1
    S0 = _f64(initial_state)
    out = np.empty(lead + (T, dv))
    Sf = np.empty(lead + (dk, dv))
    rc = _load().oracle_hdla(BH, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(ll), _ptr(b),
                             _ptr(S0), _ptr(out), _ptr(Sf), nthreads)
    _check(rc, "oracle_hdla")
    return out, Sf


def gdn(q, k, v, g, beta, initial_state=None, nthreads: int = 0):
    """Gated DeltaNet: P_t = exp(g_t)(I - beta_t k_t k_t^T), write beta_t k_t v_t^T.
    g, beta [*lead,T].  Returns (out, final_state)."""
    q, k, v, g, b = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta)
    lead = q.shape[:-2]
    T, dk = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    assert k.shape == q.shape and g.shape == lead + (T,) and b.shape == g.shape
    BH = int(np.prod(lead)) if lead else 1
    S0 = _f64(initial_state)
    out = np.empty(lead + (T, dv))
    Sf = np.empty(lead + (dk, dv))
    rc = _load().oracle_gdn(BH, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b),
                            _ptr(S0), _ptr(out), _ptr(Sf), nthreads)
    _check(rc, "oracle_gdn")
    return out, Sf


def chunk_summaries(K, V, log_decay, A, B, chunk: int, nthreads: int = 0):
    """Exact affine pair of each chunk: returns (sumA [*lead,N,dk,dk], sumB [*lead,N,dk,dv])."""
    K, V, ld = _f64(K), _f64(V), _f64(log_decay)
    lead = K.shape[:-3]
    T, r_kv, dk = K.shape[-3:]
    dv = V.shape[-1]
    scalar = ld.shape == lead + (T,)
    if A is None:
        r_ab, A_, B_ = 0, None, None
    else:
        A_, B_ = _f64(A), _f64(B)
        r_ab = A_.shape[-2]
    BH = int(np.prod(lead)) if lead else 1
    N = -(-T // chunk)
    sA = np.empty(lead + (N, dk, dk))
    sB = np.empty(lead + (N, dk, dv))
    rc = _load().oracle_chunk_summaries(BH, T, dk, dv, r_ab, r_kv, int(scalar), chunk, _ptr(K),
                                        _ptr(V), _ptr(ld), _ptr(A_), _ptr(B_), _ptr(sA), _ptr(sB),
                                        nthreads)
    _check(rc, "oracle_chunk_summaries")
    return sA, sB


def compose(sumA, sumB, initial_state=None):
    """Scan S_j = A_j S_{j-1} + B_j over chunks (axis -3).  Returns the states
    entering each chunk [*lead,N,dk,dv] and the final state [*lead,dk,dv]."""
    sumA, sumB = _f64(sumA), _f64(sumB)
    lead = sumA.shape[:-3]
    N, dk, dv = sumB.shape[-3:]
    S = np.zeros(lead + (dk, dv)) if initial_state is None else _f64(initial_state).copy()
    starts = np.empty(lead + (N, dk, dv))
    for j in range(N):
        starts[..., j, :, :] = S
        S = np.matmul(sumA[..., j, :, :], S) + sumB[..., j, :, :]
    return starts, S


def hdla_to_generic(k, v, log_lambda, beta):
    """Rewrite of the HDLA decay as diagonal minus rank 2 (HDLA note, "Key design 3").

    With u = lambda * k and c = k^T u:
      (I - b k k^T) Diag(lambda) (I - b k k^T)
        = Diag(lambda) - b k u^T - b u k^T + b^2 c k k^T
        = Diag(lambda) - [b k, b u] [u - b c k, k]^T,
    so A_t = [b k, b u], B_t = [u - b c k, k] (columns stacked on the rank axis),
    D_t = Diag(lambda_t), and the write is K_t = k_t, V_t = b_t v_t.
    Returns fp64 (log_decay, A, B, K, V) in the generic layouts.
    """
    k, v, ll, b = _f64(k), _f64(v), _f64(log_lambda), _f64(beta)
    lam = np.exp(ll)
    u = lam * k
    c = np.sum(k * u, axis=-1, keepdims=True)
    bb = b[..., None]
    A = np.stack([bb * k, bb * u], axis=-2)
    B = np.stack([u - bb * c * k, k], axis=-2)
    return ll, A, B, k[..., None, :], (bb * v)[..., None, :]


def gdn_to_generic(k, v, g, beta):
    """Gated DeltaNet as diagonal minus rank 1: exp(g)(I - b k k^T) = exp(g) I - (exp(g) b k) k^T.
    Returns fp64 (scalar log_decay g, A, B, K, V)."""
    k, v, g, b = _f64(k), _f64(v), _f64(g), _f64(beta)
    coef = (np.exp(g) * b)[..., None]
    A = (coef * k)[..., None, :]
    B = k[..., None, :]
    return g, A, B, k[..., None, :], (b[..., None] * v)[..., None, :]
