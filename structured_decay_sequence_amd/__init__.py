"""MI355X-native chunk-wise forward of the generalized linear-attention recurrence.

    S_t = (D_t - A_t B_t^T) S_{t-1} + K_t V_t^T,   o_t = S_t^T q_t

Thin Python binding over ``liblattn.so`` (C ABI in ``include/lattn.h``).
Torch tensors supply device memory and the current HIP stream; every step of
the computation runs in the library's HIP kernels.  The functions below only
check shapes/dtypes, allocate outputs and marshal pointers.
"""
from __future__ import annotations

import ctypes
from typing import Dict, Optional, Tuple

import torch

from . import _lib
from ._lib import LattnError, LATTN_BF16, LATTN_FP32, LATTN_DECAY_PER_CHANNEL, LATTN_DECAY_SCALAR

__all__ = [
    "chunk_fwd", "chunk_summaries", "step", "hdla_params", "gdn_params", "decay_range",
    "check_decay_range", "workspace_size", "make_dims", "LattnError", "version", "ChunkPlan",
    "hdla_chunk_fwd", "gdn_chunk_fwd", "FamilyPlan", "hla_fwd", "loglinear_fwd", "loglinear_levels", "chunk_bwd",
    "chunk_fwd_train", "chunk_bwd_saved", "train_saved_size", "TrainPlan", "chunk_attention",
]


def version() -> str:
    return _lib.load().lattn_version().decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return LATTN_BF16
    if t.dtype == torch.float32:
        return LATTN_FP32
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.float32 or torch.bfloat16")


def make_dims(batch, heads, seqlen, d_k, d_v, dtype_code, scalar_decay) -> _lib.lattn_dims:
    return _lib.lattn_dims(int(batch), int(heads), int(seqlen), int(d_k), int(d_v), int(dtype_code),
                           LATTN_DECAY_SCALAR if scalar_decay else LATTN_DECAY_PER_CHANNEL)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to lattn must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, dtype, shape, name):
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def _workspace(device, nbytes: int) -> Optional[torch.Tensor]:
    """A fresh workspace for one call, from torch's caching allocator on the
    current stream.  The tensor lives until the caller drops it; the allocator
    hands its memory to a later request only in stream order, so calls on
    different streams never share a buffer that one of them still uses."""
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _ranked(x: torch.Tensor, lead, T, d):
    """Accept [*lead, T, d] as rank 1 or [*lead, T, r, d]."""
    if x.dim() == len(lead) + 2:
        return x.unsqueeze(-2)
    return x


def workspace_size(batch, heads, seqlen, d_k, d_v, r_ab, r_kv, chunk, dtype=torch.bfloat16,
                   scalar_decay=False) -> int:
    code = LATTN_BF16 if dtype == torch.bfloat16 else LATTN_FP32
    dims = make_dims(batch, heads, seqlen, d_k, d_v, code, scalar_decay)
    return int(_lib.load().lattn_chunk_fwd_workspace_size(ctypes.byref(dims), r_ab, r_kv, chunk))


def chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_decay: torch.Tensor,
              A: Optional[torch.Tensor] = None, B: Optional[torch.Tensor] = None, chunk: int = 64,
              initial_state: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
              final_state: Optional[torch.Tensor] = None, return_final_state: bool = True,
              workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunk-wise forward.  q [B,H,T,dk]; k [B,H,T,(r_kv,)dk]; v [B,H,T,(r_kv,)dv];
    log_decay fp32 [B,H,T,dk] or [B,H,T]; A, B [B,H,T,r_ab,dk] or None.
    Returns (out [B,H,T,dv], final_state [B,H,dk,dv] fp32 or None)."""
    Bb, H, T, dk = q.shape
    dt = q.dtype
    lead = (Bb, H)
    k = _ranked(k, lead, T, dk)
    v = _ranked(v, lead, T, None)
    r_kv, dv = k.shape[-2], v.shape[-1]
    _need(q, dt, (Bb, H, T, dk), "q")
    _need(k, dt, (Bb, H, T, r_kv, dk), "k")
    _need(v, dt, (Bb, H, T, r_kv, dv), "v")
    scalar = log_decay.dim() == 3
    _need(log_decay, torch.float32, (Bb, H, T) if scalar else (Bb, H, T, dk), "log_decay")
    r_ab = 0
    if A is not None:
        r_ab = A.shape[-2]
        _need(A, dt, (Bb, H, T, r_ab, dk), "A")
        _need(B, dt, (Bb, H, T, r_ab, dk), "B")
    if initial_state is not None:
        _need(initial_state, torch.float32, (Bb, H, dk, dv), "initial_state")
    if out is None:
        out = torch.empty((Bb, H, T, dv), dtype=dt, device=q.device)
    _need(out, dt, (Bb, H, T, dv), "out")
    if final_state is None and return_final_state:
        final_state = torch.empty((Bb, H, dk, dv), dtype=torch.float32, device=q.device)
    if final_state is not None:
        _need(final_state, torch.float32, (Bb, H, dk, dv), "final_state")
    lib = _lib.load()
    dims = make_dims(Bb, H, T, dk, dv, _dtype_code(q), scalar)
    ws_bytes = int(lib.lattn_chunk_fwd_workspace_size(ctypes.byref(dims), r_ab, r_kv, chunk))
    if workspace is None:
        workspace = _workspace(q.device, ws_bytes)
    rc = lib.lattn_chunk_fwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(log_decay), _ptr(A),
                             _ptr(B), r_ab, r_kv, chunk, _ptr(out), _ptr(final_state),
                             _ptr(initial_state), _ptr(workspace),
                             0 if workspace is None else workspace.numel(), _stream(q.device))
    _lib.check(rc, "lattn_chunk_fwd")
    return out, final_state


def _family_fwd(name: str, q, k, v, decay, beta, chunk, initial_state, out, final_state,
                return_final_state, workspace):
    Bb, H, T, dk = q.shape
    dt = q.dtype
    dv = v.shape[-1]
    scalar = name == "gdn"
    _need(q, dt, (Bb, H, T, dk), "q")
    _need(k, dt, (Bb, H, T, dk), "k")
    _need(v, dt, (Bb, H, T, dv), "v")
    _need(decay, torch.float32, (Bb, H, T) if scalar else (Bb, H, T, dk), "g" if scalar else "log_lambda")
    _need(beta, torch.float32, (Bb, H, T), "beta")
    if initial_state is not None:
        _need(initial_state, torch.float32, (Bb, H, dk, dv), "initial_state")
    if out is None:
        out = torch.empty((Bb, H, T, dv), dtype=dt, device=q.device)
    _need(out, dt, (Bb, H, T, dv), "out")
    if final_state is None and return_final_state:
        final_state = torch.empty((Bb, H, dk, dv), dtype=torch.float32, device=q.device)
    if final_state is not None:
        _need(final_state, torch.float32, (Bb, H, dk, dv), "final_state")
    lib = _lib.load()
    dims = make_dims(Bb, H, T, dk, dv, _dtype_code(q), scalar)
    ws_bytes = int(getattr(lib, f"lattn_{name}_chunk_fwd_workspace_size")(ctypes.byref(dims), chunk))
    if workspace is None:
        workspace = _workspace(q.device, ws_bytes)
    rc = getattr(lib, f"lattn_{name}_chunk_fwd")(
        ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(beta), chunk, _ptr(out),
        _ptr(final_state), _ptr(initial_state), _ptr(workspace), 0 if workspace is None else workspace.numel(),
        _stream(q.device))
    _lib.check(rc, f"lattn_{name}_chunk_fwd")
    return out, final_state


def hdla_chunk_fwd(q, k, v, log_lambda, beta, chunk: int = 64, initial_state=None, out=None,
                   final_state=None, return_final_state: bool = True, workspace=None):
    """HDLA forward from its raw parameters (decay operands formed in the kernel).
    q, k [B,H,T,dk]; v [B,H,T,dv]; log_lambda fp32 [B,H,T,dk]; beta fp32 [B,H,T].
    Returns (out [B,H,T,dv], final_state [B,H,dk,dv] fp32 or None)."""
    return _family_fwd("hdla", q, k, v, log_lambda, beta, chunk, initial_state, out, final_state,
                       return_final_state, workspace)


def gdn_chunk_fwd(q, k, v, g, beta, chunk: int = 64, initial_state=None, out=None, final_state=None,
                  return_final_state: bool = True, workspace=None):
    """Gated DeltaNet forward from its raw parameters.  q, k [B,H,T,dk]; v [B,H,T,dv];
    g, beta fp32 [B,H,T].  Returns (out, final_state)."""
    return _family_fwd("gdn", q, k, v, g, beta, chunk, initial_state, out, final_state,
                       return_final_state, workspace)


def chunk_summaries(k, v, log_decay, A=None, B=None, chunk: int = 64):
    """Exact affine pair of every chunk: (sum_A [B,H,N,dk,dk], sum_B [B,H,N,dk,dv]) fp32."""
    Bb, H, T = k.shape[:3]
    dk = k.shape[-1]
    k = _ranked(k, (Bb, H), T, dk)
    v = _ranked(v, (Bb, H), T, None)
    r_kv, dv = k.shape[-2], v.shape[-1]
    dt = k.dtype
    _need(v, dt, (Bb, H, T, r_kv, dv), "v")
    scalar = log_decay.dim() == 3
    _need(log_decay, torch.float32, (Bb, H, T) if scalar else (Bb, H, T, dk), "log_decay")
    r_ab = 0 if A is None else A.shape[-2]
    N = -(-T // chunk)
    sA = torch.empty((Bb, H, N, dk, dk), dtype=torch.float32, device=k.device)
    sB = torch.empty((Bb, H, N, dk, dv), dtype=torch.float32, device=k.device)
    lib = _lib.load()
    dims = make_dims(Bb, H, T, dk, dv, _dtype_code(k), scalar)
    ws_bytes = int(lib.lattn_chunk_summaries_workspace_size(ctypes.byref(dims), r_ab, r_kv, chunk))
    ws = _workspace(k.device, ws_bytes)
    rc = lib.lattn_chunk_summaries(ctypes.byref(dims), _ptr(k), _ptr(v), _ptr(log_decay), _ptr(A),
                                   _ptr(B), r_ab, r_kv, chunk, _ptr(sA), _ptr(sB), _ptr(ws),
                                   0 if ws is None else ws.numel(), _stream(k.device))
    _lib.check(rc, "lattn_chunk_summaries")
    return sA, sB


def hla_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_decay: torch.Tensor,
            A: Optional[torch.Tensor], B: Optional[torch.Tensor], gates: torch.Tensor, chunk: int = 64,
            theta: float = 0.1, out: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Query-conditioned composition of the exact chunk transitions (lattn_hla_fwd).
    Inputs as chunk_fwd, plus gates fp32 [B,H,T,ceil(T/chunk)] (query i's gate for
    chunk j) and the threshold below which a gate counts as 0.  Returns out [B,H,T,dv]."""
    Bb, H, T, dk = q.shape
    dt = q.dtype
    lead = (Bb, H)
    k = _ranked(k, lead, T, dk)
    v = _ranked(v, lead, T, None)
    r_kv, dv = k.shape[-2], v.shape[-1]
    _need(q, dt, (Bb, H, T, dk), "q")
    _need(k, dt, (Bb, H, T, r_kv, dk), "k")
    _need(v, dt, (Bb, H, T, r_kv, dv), "v")
    scalar = log_decay.dim() == 3
    _need(log_decay, torch.float32, (Bb, H, T) if scalar else (Bb, H, T, dk), "log_decay")
    r_ab = 0
    if A is not None:
        r_ab = A.shape[-2]
        _need(A, dt, (Bb, H, T, r_ab, dk), "A")
        _need(B, dt, (Bb, H, T, r_ab, dk), "B")
    _need(gates, torch.float32, (Bb, H, T, -(-T // chunk)), "gates")
    if out is None:
        out = torch.empty((Bb, H, T, dv), dtype=dt, device=q.device)
    _need(out, dt, (Bb, H, T, dv), "out")
    lib = _lib.load()
    dims = make_dims(Bb, H, T, dk, dv, _dtype_code(q), scalar)
    if workspace is None:
        workspace = _workspace(q.device, int(lib.lattn_hla_fwd_workspace_size(ctypes.byref(dims), r_ab, r_kv, chunk)))
    rc = lib.lattn_hla_fwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(log_decay), _ptr(A), _ptr(B),
                           r_ab, r_kv, chunk, _ptr(gates), float(theta), _ptr(out), _ptr(workspace),
                           0 if workspace is None else workspace.numel(), _stream(q.device))
    _lib.check(rc, "lattn_hla_fwd")
    return out


def loglinear_levels(seqlen: int) -> int:
    """Levels L of the log-linear lift for a sequence of ``seqlen`` tokens."""
    return int(_lib.load().lattn_loglinear_levels(int(seqlen)))


def loglinear_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_decay: torch.Tensor,
                  A: Optional[torch.Tensor], B: Optional[torch.Tensor], lam: torch.Tensor, chunk: int = 64,
                  out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Log-linear lift of the recurrence (lattn_loglinear_fwd).  Inputs as chunk_fwd,
    plus lam fp32 [B,H,T,loglinear_levels(T)] (per-token weight of each Fenwick
    level).  Returns out [B,H,T,dv]."""
    Bb, H, T, dk = q.shape
    dt = q.dtype
    lead = (Bb, H)
    k = _ranked(k, lead, T, dk)
    v = _ranked(v, lead, T, None)
    r_kv, dv = k.shape[-2], v.shape[-1]
    _need(q, dt, (Bb, H, T, dk), "q")
    _need(k, dt, (Bb, H, T, r_kv, dk), "k")
    _need(v, dt, (Bb, H, T, r_kv, dv), "v")
    scalar = log_decay.dim() == 3
    _need(log_decay, torch.float32, (Bb, H, T) if scalar else (Bb, H, T, dk), "log_decay")
    r_ab = 0
    if A is not None:
        r_ab = A.shape[-2]
        _need(A, dt, (Bb, H, T, r_ab, dk), "A")
        _need(B, dt, (Bb, H, T, r_ab, dk), "B")
    _need(lam, torch.float32, (Bb, H, T, loglinear_levels(T)), "lam")
    if out is None:
        out = torch.empty((Bb, H, T, dv), dtype=dt, device=q.device)
    _need(out, dt, (Bb, H, T, dv), "out")
    lib = _lib.load()
    dims = make_dims(Bb, H, T, dk, dv, _dtype_code(q), scalar)
    if workspace is None:
        workspace = _workspace(q.device, int(lib.lattn_loglinear_fwd_workspace_size(ctypes.byref(dims), r_ab, r_kv,
                                                                                        chunk)))
    rc = lib.lattn_loglinear_fwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(log_decay), _ptr(A), _ptr(B),
                                 r_ab, r_kv, chunk, _ptr(lam), _ptr(out), _ptr(workspace),
                                 0 if workspace is None else workspace.numel(), _stream(q.device))
    _lib.check(rc, "lattn_loglinear_fwd")
    return out


def _bwd_inputs(q, k, v, log_decay, A, B, dout, dfinal, initial_state):
    """Checks chunk_bwd's inputs; returns (k, v with the rank axis, r_ab, r_kv,
    the fp32 gradient tensors)."""
    Bb, H, T, dk = q.shape
    dt = q.dtype
    lead = (Bb, H)
    k = _ranked(k, lead, T, dk)
    v = _ranked(v, lead, T, None)
    r_kv, dv = k.shape[-2], v.shape[-1]
    _need(q, dt, (Bb, H, T, dk), "q")
    _need(k, dt, (Bb, H, T, r_kv, dk), "k")
    _need(v, dt, (Bb, H, T, r_kv, dv), "v")
    _need(dout, dt, (Bb, H, T, dv), "dout")
    scalar = log_decay.dim() == 3
    _need(log_decay, torch.float32, (Bb, H, T) if scalar else (Bb, H, T, dk), "log_decay")
    r_ab = 0
    if A is not None:
        r_ab = A.shape[-2]
        _need(A, dt, (Bb, H, T, r_ab, dk), "A")
        _need(B, dt, (Bb, H, T, r_ab, dk), "B")
    for t, n in ((dfinal, "dfinal"), (initial_state, "initial_state")):
        if t is not None:
            _need(t, torch.float32, (Bb, H, dk, dv), n)
    f32 = dict(dtype=torch.float32, device=q.device)
    g = dict(dq=torch.empty((Bb, H, T, dk), **f32), dk=torch.empty((Bb, H, T, r_kv, dk), **f32),
             dv=torch.empty((Bb, H, T, r_kv, dv), **f32), dlog_decay=torch.empty(tuple(log_decay.shape), **f32),
             dA=None if A is None else torch.empty(tuple(A.shape), **f32),
             dB=None if A is None else torch.empty(tuple(A.shape), **f32),
             dinitial_state=torch.empty((Bb, H, dk, dv), **f32))
    return k, v, r_ab, r_kv, g


def chunk_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_decay: torch.Tensor,
              A: Optional[torch.Tensor], B: Optional[torch.Tensor], dout: torch.Tensor, chunk: int = 64,
              dfinal: Optional[torch.Tensor] = None, initial_state: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None) -> Dict[str, Optional[torch.Tensor]]:
    """Backward pass of chunk_fwd (lattn_chunk_bwd): gradients of
    sum <dout, out> + <dfinal, final_state>.  Inputs as chunk_fwd plus dout
    [B,H,T,dv] (dtype of q) and dfinal [B,H,dk,dv] fp32 or None.  Returns fp32
    tensors dq, dk, dv, dlog_decay, dA, dB (None when A is None), dinitial_state,
    each shaped like its input (k, v with the rank axis)."""
    k, v, r_ab, r_kv, g = _bwd_inputs(q, k, v, log_decay, A, B, dout, dfinal, initial_state)
    Bb, H, T, dk = q.shape
    lib = _lib.load()
    dims = make_dims(Bb, H, T, dk, v.shape[-1], _dtype_code(q), log_decay.dim() == 3)
    if workspace is None:
        workspace = _workspace(q.device, int(lib.lattn_chunk_bwd_workspace_size(ctypes.byref(dims), r_ab, r_kv, chunk)))
    rc = lib.lattn_chunk_bwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(log_decay), _ptr(A), _ptr(B), r_ab,
                             r_kv, chunk, _ptr(dout), _ptr(dfinal), _ptr(initial_state), _ptr(g["dq"]), _ptr(g["dk"]),
                             _ptr(g["dv"]), _ptr(g["dlog_decay"]), _ptr(g["dA"]), _ptr(g["dB"]),
                             _ptr(g["dinitial_state"]), _ptr(workspace), 0 if workspace is None else workspace.numel(),
                             _stream(q.device))
    _lib.check(rc, "lattn_chunk_bwd")
    return g


def train_saved_size(batch, heads, seqlen, d_k, d_v, r_ab, r_kv, chunk=64, dtype=torch.bfloat16,
                     scalar_decay=False) -> int:
    """Bytes of the buffer chunk_fwd_train keeps for chunk_bwd_saved (0 where the
    shape is off the training pair's route: then use chunk_fwd and chunk_bwd)."""
    code = LATTN_BF16 if dtype == torch.bfloat16 else LATTN_FP32
    dims = make_dims(batch, heads, seqlen, d_k, d_v, code, scalar_decay)
    return int(_lib.load().lattn_chunk_fwd_train_saved_size(ctypes.byref(dims), r_ab, r_kv, chunk))


def chunk_fwd_train(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_decay: torch.Tensor,
                    A: Optional[torch.Tensor] = None, B: Optional[torch.Tensor] = None, chunk: int = 64,
                    initial_state: Optional[torch.Tensor] = None, saved: Optional[torch.Tensor] = None
                    ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """The training forward (lattn_chunk_fwd_train): chunk_fwd's results, plus
    the uint8 buffer `saved` that chunk_bwd_saved reads instead of forming the
    chunk operators and the decay-scaled operands again.  Returns (out,
    final_state, saved)."""
    Bb, H, T, dk = q.shape
    dt = q.dtype
    lead = (Bb, H)
    k = _ranked(k, lead, T, dk)
    v = _ranked(v, lead, T, None)
    r_kv, dv = k.shape[-2], v.shape[-1]
    _need(q, dt, (Bb, H, T, dk), "q")
    _need(k, dt, (Bb, H, T, r_kv, dk), "k")
    _need(v, dt, (Bb, H, T, r_kv, dv), "v")
    scalar = log_decay.dim() == 3
    _need(log_decay, torch.float32, (Bb, H, T) if scalar else (Bb, H, T, dk), "log_decay")
    r_ab = 0
    if A is not None:
        r_ab = A.shape[-2]
        _need(A, dt, (Bb, H, T, r_ab, dk), "A")
        _need(B, dt, (Bb, H, T, r_ab, dk), "B")
    if initial_state is not None:
        _need(initial_state, torch.float32, (Bb, H, dk, dv), "initial_state")
    out = torch.empty((Bb, H, T, dv), dtype=dt, device=q.device)
    final_state = torch.empty((Bb, H, dk, dv), dtype=torch.float32, device=q.device)
    lib = _lib.load()
    dims = make_dims(Bb, H, T, dk, dv, _dtype_code(q), scalar)
    if saved is None:
        saved = _workspace(q.device, int(lib.lattn_chunk_fwd_train_saved_size(ctypes.byref(dims), r_ab, r_kv,
                                                                               chunk)))
    rc = lib.lattn_chunk_fwd_train(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(log_decay), _ptr(A), _ptr(B),
                                   r_ab, r_kv, chunk, _ptr(out), _ptr(final_state), _ptr(initial_state), _ptr(saved),
                                   0 if saved is None else saved.numel(), _stream(q.device))
    _lib.check(rc, "lattn_chunk_fwd_train")
    return out, final_state, saved


def chunk_bwd_saved(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_decay: torch.Tensor,
                    A: Optional[torch.Tensor], B: Optional[torch.Tensor], dout: torch.Tensor, saved: torch.Tensor,
                    chunk: int = 64, dfinal: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None) -> Dict[str, Optional[torch.Tensor]]:
    """The training backward (lattn_chunk_bwd_saved): chunk_bwd's gradients,
    reading what chunk_fwd_train left in `saved` for the same inputs (the
    initial state among them)."""
    k, v, r_ab, r_kv, g = _bwd_inputs(q, k, v, log_decay, A, B, dout, dfinal, None)
    Bb, H, T, dk = q.shape
    lib = _lib.load()
    dims = make_dims(Bb, H, T, dk, v.shape[-1], _dtype_code(q), log_decay.dim() == 3)
    if workspace is None:
        workspace = _workspace(q.device, int(lib.lattn_chunk_bwd_saved_workspace_size(ctypes.byref(dims), r_ab, r_kv,
                                                                                        chunk)))
    rc = lib.lattn_chunk_bwd_saved(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(log_decay), _ptr(A), _ptr(B),
                                   r_ab, r_kv, chunk, _ptr(dout), _ptr(dfinal), _ptr(saved),
                                   0 if saved is None else saved.numel(), _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]),
                                   _ptr(g["dlog_decay"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dinitial_state"]),
                                   _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(q.device))
    _lib.check(rc, "lattn_chunk_bwd_saved")
    return g


def step(q, k, v, log_decay, A, B, state, out=None):
    """One recurrent token.  q [B,H,dk]; k [B,H,(r_kv,)dk]; v [B,H,(r_kv,)dv];
    log_decay [B,H,dk] or [B,H]; A, B [B,H,r_ab,dk] or None; state [B,H,dk,dv]
    fp32 updated in place.  Returns out [B,H,dv]."""
    Bb, H, dk = q.shape
    if k.dim() == 3:
        k = k.unsqueeze(-2)
    if v.dim() == 3:
        v = v.unsqueeze(-2)
    r_kv, dv = k.shape[-2], v.shape[-1]
    scalar = log_decay.dim() == 2
    _need(log_decay, torch.float32, (Bb, H) if scalar else (Bb, H, dk), "log_decay")
    _need(state, torch.float32, (Bb, H, dk, dv), "state")
    r_ab = 0 if A is None else A.shape[-2]
    if out is None:
        out = torch.empty((Bb, H, dv), dtype=q.dtype, device=q.device)
    lib = _lib.load()
    dims = make_dims(Bb, H, 1, dk, dv, _dtype_code(q), scalar)
    rc = lib.lattn_step(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(log_decay), _ptr(A),
                        _ptr(B), r_ab, r_kv, _ptr(state), _ptr(out), _stream(q.device))
    _lib.check(rc, "lattn_step")
    return out


def hdla_params(k, v, log_lambda, beta):
    """HDLA decay operands on the device: returns (A, B [B,H,T,2,dk], V [B,H,T,1,dv])."""
    Bb, H, T, dk = k.shape
    dv = v.shape[-1]
    A = torch.empty((Bb, H, T, 2, dk), dtype=k.dtype, device=k.device)
    Bm = torch.empty_like(A)
    V = torch.empty((Bb, H, T, 1, dv), dtype=k.dtype, device=k.device)
    _need(log_lambda, torch.float32, (Bb, H, T, dk), "log_lambda")
    _need(beta, torch.float32, (Bb, H, T), "beta")
    lib = _lib.load()
    dims = make_dims(Bb, H, T, dk, dv, _dtype_code(k), False)
    rc = lib.lattn_hdla_params(ctypes.byref(dims), _ptr(k), _ptr(v), _ptr(log_lambda), _ptr(beta),
                               _ptr(A), _ptr(Bm), _ptr(V), _stream(k.device))
    _lib.check(rc, "lattn_hdla_params")
    return A, Bm, V


def gdn_params(k, v, g, beta):
    """Gated DeltaNet decay operands: returns (A, B [B,H,T,1,dk], V [B,H,T,1,dv])."""
    Bb, H, T, dk = k.shape
    dv = v.shape[-1]
    A = torch.empty((Bb, H, T, 1, dk), dtype=k.dtype, device=k.device)
    Bm = torch.empty_like(A)
    V = torch.empty((Bb, H, T, 1, dv), dtype=k.dtype, device=k.device)
    _need(g, torch.float32, (Bb, H, T), "g")
    _need(beta, torch.float32, (Bb, H, T), "beta")
    lib = _lib.load()
    dims = make_dims(Bb, H, T, dk, dv, _dtype_code(k), True)
    rc = lib.lattn_gdn_params(ctypes.byref(dims), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(A),
                              _ptr(Bm), _ptr(V), _stream(k.device))
    _lib.check(rc, "lattn_gdn_params")
    return A, Bm, V


def decay_range(log_decay, chunk: int, d_k: Optional[int] = None):
    """Per chunk, the largest -G (chunk-local inclusive cumulative log-decay): [B,H,N] fp32."""
    scalar = log_decay.dim() == 3
    Bb, H, T = log_decay.shape[:3]
    dk = d_k if scalar else log_decay.shape[-1]
    dk = 16 if dk is None else dk
    N = -(-T // chunk)
    res = torch.empty((Bb, H, N), dtype=torch.float32, device=log_decay.device)
    lib = _lib.load()
    dims = make_dims(Bb, H, T, dk, 16, LATTN_FP32, scalar)
    rc = lib.lattn_decay_range(ctypes.byref(dims), _ptr(log_decay), chunk, _ptr(res),
                               _stream(log_decay.device))
    _lib.check(rc, "lattn_decay_range")
    return res


def check_decay_range(log_decay, chunk: int, d_k: Optional[int] = None) -> None:
    """Raise LattnError(LATTN_EDECAY_RANGE) if any chunk's -G exceeds the supported limit."""
    scalar = log_decay.dim() == 3
    Bb, H, T = log_decay.shape[:3]
    dk = d_k if scalar else log_decay.shape[-1]
    dk = 16 if dk is None else dk
    N = -(-T // chunk)
    scratch = torch.empty((max(1, Bb * H * N),), dtype=torch.float32, device=log_decay.device)
    lib = _lib.load()
    dims = make_dims(Bb, H, T, dk, 16, LATTN_FP32, scalar)
    rc = lib.lattn_check_decay_range(ctypes.byref(dims), _ptr(log_decay), chunk, _ptr(scratch),
                                     _stream(log_decay.device))
    _lib.check(rc, "lattn_check_decay_range")


class ChunkPlan:
    """Pre-marshalled arguments of one chunk-wise forward, for calling its two
    stages (prepare, scan) repeatedly with no per-call Python shape work.

    ``prepare()`` + ``scan()`` on one stream is exactly ``chunk_fwd``.
    """

    def __init__(self, q, k, v, log_decay, A=None, B=None, chunk=64, initial_state=None,
                 return_final_state=True):
        Bb, H, T, dk = q.shape
        k = _ranked(k, (Bb, H), T, dk)
        v = _ranked(v, (Bb, H), T, None)
        self.r_kv, dv = k.shape[-2], v.shape[-1]
        self.r_ab = 0 if A is None else A.shape[-2]
        self.chunk = chunk
        scalar = log_decay.dim() == 3
        self.dims = make_dims(Bb, H, T, dk, dv, _dtype_code(q), scalar)
        self.lib = _lib.load()
        self.ws_bytes = int(self.lib.lattn_chunk_fwd_workspace_size(ctypes.byref(self.dims), self.r_ab,
                                                                   self.r_kv, chunk))
        self.workspace = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=q.device)
        self.out = torch.empty((Bb, H, T, dv), dtype=q.dtype, device=q.device)
        self.final_state = (torch.empty((Bb, H, dk, dv), dtype=torch.float32, device=q.device)
                            if return_final_state else None)
        self._keep = (q, k, v, log_decay, A, B, initial_state)
        self.p = dict(q=_ptr(q), k=_ptr(k), v=_ptr(v), ld=_ptr(log_decay), A=_ptr(A), B=_ptr(B),
                      S0=_ptr(initial_state), out=_ptr(self.out), Sf=_ptr(self.final_state),
                      ws=_ptr(self.workspace))
        self.device = q.device

    def prepare(self):
        p = self.p
        rc = self.lib.lattn_chunk_prepare(ctypes.byref(self.dims), p["q"], p["k"], p["ld"], p["A"], p["B"],
                                          self.r_ab, self.r_kv, self.chunk, p["ws"], self.ws_bytes,
                                          _stream(self.device))
        _lib.check(rc, "lattn_chunk_prepare")

    def scan(self):
        p = self.p
        rc = self.lib.lattn_chunk_scan(ctypes.byref(self.dims), p["v"], self.r_ab, self.r_kv, self.chunk,
                                       p["out"], p["Sf"], p["S0"], p["ws"], self.ws_bytes,
                                       _stream(self.device))
        _lib.check(rc, "lattn_chunk_scan")

    def forward(self):
        p = self.p
        rc = self.lib.lattn_chunk_fwd(ctypes.byref(self.dims), p["q"], p["k"], p["v"], p["ld"], p["A"], p["B"],
                                      self.r_ab, self.r_kv, self.chunk, p["out"], p["Sf"], p["S0"], p["ws"],
                                      self.ws_bytes, _stream(self.device))
        _lib.check(rc, "lattn_chunk_fwd")
        return self.out, self.final_state


class TrainPlan:
    """Pre-marshalled arguments of the backward and of the training pair on one
    set of inputs and cotangents, for repeated calls with no per-call Python
    work (outputs, gradients, workspaces and the saved buffer allocated once).

    ``backward()`` is ``chunk_bwd``; ``forward_train()`` then
    ``backward_saved()`` is ``chunk_fwd_train`` then ``chunk_bwd_saved`` (on
    the shapes the training pair takes: ``self.saved`` is None elsewhere).
    """

    def __init__(self, q, k, v, log_decay, A, B, dout, chunk=64, dfinal=None, initial_state=None):
        Bb, H, T, dk = q.shape
        k, v, self.r_ab, self.r_kv, self.grads = _bwd_inputs(q, k, v, log_decay, A, B, dout, dfinal, initial_state)
        dv = v.shape[-1]
        self.chunk = chunk
        self.dims = make_dims(Bb, H, T, dk, dv, _dtype_code(q), log_decay.dim() == 3)
        self.lib = _lib.load()
        d = ctypes.byref(self.dims)
        size = lambda fn: int(getattr(self.lib, fn)(d, self.r_ab, self.r_kv, chunk))
        self.ws_bytes = size("lattn_chunk_bwd_workspace_size")
        self.saved_bytes = size("lattn_chunk_fwd_train_saved_size")
        self.sws_bytes = size("lattn_chunk_bwd_saved_workspace_size")
        self.workspace = _workspace(q.device, self.ws_bytes)
        self.saved = _workspace(q.device, self.saved_bytes)
        self.saved_workspace = _workspace(q.device, self.sws_bytes)
        self.out = torch.empty((Bb, H, T, dv), dtype=q.dtype, device=q.device)
        self.final_state = torch.empty((Bb, H, dk, dv), dtype=torch.float32, device=q.device)
        self._keep = (q, k, v, log_decay, A, B, dout, dfinal, initial_state)
        g = self.grads
        self.p = dict(q=_ptr(q), k=_ptr(k), v=_ptr(v), ld=_ptr(log_decay), A=_ptr(A), B=_ptr(B), do=_ptr(dout),
                      df=_ptr(dfinal), S0=_ptr(initial_state), ws=_ptr(self.workspace), sv=_ptr(self.saved),
                      sws=_ptr(self.saved_workspace), out=_ptr(self.out), Sf=_ptr(self.final_state),
                      g=[_ptr(g[n]) for n in ("dq", "dk", "dv", "dlog_decay", "dA", "dB", "dinitial_state")])
        self.device = q.device

    def backward(self):
        p = self.p
        rc = self.lib.lattn_chunk_bwd(ctypes.byref(self.dims), p["q"], p["k"], p["v"], p["ld"], p["A"], p["B"],
                                      self.r_ab, self.r_kv, self.chunk, p["do"], p["df"], p["S0"], *p["g"],
                                      p["ws"], self.ws_bytes, _stream(self.device))
        _lib.check(rc, "lattn_chunk_bwd")
        return self.grads

    def forward_train(self):
        p = self.p
        rc = self.lib.lattn_chunk_fwd_train(ctypes.byref(self.dims), p["q"], p["k"], p["v"], p["ld"], p["A"],
                                            p["B"], self.r_ab, self.r_kv, self.chunk, p["out"], p["Sf"], p["S0"],
                                            p["sv"], self.saved_bytes, _stream(self.device))
        _lib.check(rc, "lattn_chunk_fwd_train")
        return self.out, self.final_state

    def backward_saved(self):
        p = self.p
        rc = self.lib.lattn_chunk_bwd_saved(ctypes.byref(self.dims), p["q"], p["k"], p["v"], p["ld"], p["A"],
                                            p["B"], self.r_ab, self.r_kv, self.chunk, p["do"], p["df"], p["sv"],
                                            self.saved_bytes, *p["g"], p["sws"], self.sws_bytes,
                                            _stream(self.device))
        _lib.check(rc, "lattn_chunk_bwd_saved")
        return self.grads


class FamilyPlan:
    """Pre-marshalled arguments of one fused family forward (``"hdla"``: decay
    ``log_lambda`` [B,H,T,dk]; ``"gdn"``: decay ``g`` [B,H,T]), for repeated
    timed calls.  ``forward()`` is exactly ``hdla_chunk_fwd`` / ``gdn_chunk_fwd``."""

    def __init__(self, family, q, k, v, decay, beta, chunk=64, initial_state=None, return_final_state=True):
        assert family in ("hdla", "gdn")
        Bb, H, T, dk = q.shape
        dv = v.shape[-1]
        self.name = family
        self.chunk = chunk
        self.dims = make_dims(Bb, H, T, dk, dv, _dtype_code(q), family == "gdn")
        self.lib = _lib.load()
        self.fn = getattr(self.lib, f"lattn_{family}_chunk_fwd")
        self.ws_bytes = int(getattr(self.lib, f"lattn_{family}_chunk_fwd_workspace_size")(ctypes.byref(self.dims),
                                                                                            chunk))
        self.workspace = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=q.device)
        self.out = torch.empty((Bb, H, T, dv), dtype=q.dtype, device=q.device)
        self.final_state = (torch.empty((Bb, H, dk, dv), dtype=torch.float32, device=q.device)
                            if return_final_state else None)
        self._keep = (q, k, v, decay, beta, initial_state)
        self.args = (_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(beta), chunk, _ptr(self.out),
                     _ptr(self.final_state), _ptr(initial_state), _ptr(self.workspace), self.ws_bytes)
        self.device = q.device

    def forward(self):
        rc = self.fn(ctypes.byref(self.dims), *self.args, _stream(self.device))
        _lib.check(rc, f"lattn_{self.name}_chunk_fwd")
        return self.out, self.final_state


class _ChunkAttention(torch.autograd.Function):
    """chunk_fwd as an autograd function: the forward keeps what the backward
    needs (the training pair's saved buffer on its shapes, else the inputs),
    the backward returns the gradients of every tensor input in its dtype."""

    @staticmethod
    def forward(ctx, q, k, v, log_decay, A, B, initial_state, chunk):
        Bb, H, T, dk = q.shape
        r_ab = 0 if A is None else A.shape[-2]
        r_kv = 1 if k.dim() == 4 else k.shape[-2]
        saved = None
        if train_saved_size(Bb, H, T, dk, v.shape[-1], r_ab, r_kv, chunk, q.dtype, log_decay.dim() == 3) > 0:
            out, final_state, saved = chunk_fwd_train(q, k, v, log_decay, A, B, chunk=chunk,
                                                      initial_state=initial_state)
        else:
            out, final_state = chunk_fwd(q, k, v, log_decay, A, B, chunk=chunk, initial_state=initial_state)
        ctx.chunk = chunk
        ctx.has_ab = A is not None
        ctx.has_s0 = initial_state is not None
        ctx.k_dim = k.dim()
        ctx.v_dim = v.dim()
        ctx.save_for_backward(q, k, v, log_decay, A, B, initial_state, saved)
        return out, final_state

    @staticmethod
    def backward(ctx, dout, dfinal):
        q, k, v, log_decay, A, B, initial_state, saved = ctx.saved_tensors
        dout = (torch.zeros_like(q[..., :1]).expand(*q.shape[:-1], v.shape[-1]) if dout is None else dout)
        dout = dout.to(q.dtype).contiguous()
        dfinal = None if dfinal is None else dfinal.float().contiguous()
        if saved is not None:
            g = chunk_bwd_saved(q, k, v, log_decay, A, B, dout, saved, chunk=ctx.chunk, dfinal=dfinal)
        else:
            g = chunk_bwd(q, k, v, log_decay, A, B, dout, chunk=ctx.chunk, dfinal=dfinal,
                          initial_state=initial_state)
        cast = lambda t, like: None if t is None else t.reshape(like.shape).to(like.dtype)
        return (cast(g["dq"], q), cast(g["dk"], k), cast(g["dv"], v), cast(g["dlog_decay"], log_decay),
                cast(g["dA"], A) if ctx.has_ab else None, cast(g["dB"], B) if ctx.has_ab else None,
                g["dinitial_state"] if ctx.has_s0 else None, None)


def chunk_attention(q, k, v, log_decay, A=None, B=None, chunk: int = 64, initial_state=None):
    """chunk_fwd with gradients through torch.autograd: returns (out,
    final_state); out.backward(...) runs lattn_chunk_bwd_saved on the training
    pair's shapes (bf16, chunk 64, r_kv 1, r_ab <= 2, d_k and d_v in {64, 128}),
    lattn_chunk_bwd elsewhere.  Gradients come back in each input's dtype
    (the library forms them in fp32)."""
    return _ChunkAttention.apply(q, k, v, log_decay, A, B, initial_state, chunk)
