"""Seeded synthetic inputs for the chunk-wise linear-attention forward.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the method's arithmetic (no decay products, no low-rank
rewrite, no recurrence): both the CPU oracle's callers and the HIP path's
callers take their inputs from here, and nothing else is shared between them.

Distributions follow the workload descriptions: queries, keys and values are
standard normal, keys (and for Gated DeltaNet also queries) are l2-normalised
per token, the HDLA forget gate is lambda = sigmoid(x) with x ~ N(mu, 1) per
channel (HDLA note, "Key design 2": sigmoid-gated diagonal eigenvalues), the
Householder coefficient is beta = 2 sigmoid(N(0,1)) in (0, 2), the Gated
DeltaNet gate is g = -softplus(N(0,1)) * 0.1 per head-token with
beta = sigmoid(N(0,1)).  The decay is handed over as its logarithm, as the
library takes it.

Every array is drawn in full, in a fixed order, from one
``numpy.random.default_rng(seed)`` stream in float32, so any (batch, head)
slice of a large workload is reproducible by slicing.
"""
from __future__ import annotations

import dataclasses
from typing import Dict

import numpy as np


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(a.shape)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    return round_bf16(x) if dtype == "bf16" else x


def _log_sigmoid(x: np.ndarray) -> np.ndarray:
    # log(sigmoid(x)) = -log(1 + exp(-x)), evaluated stably in float64, stored as float32.
    x64 = x.astype(np.float64)
    return (-np.logaddexp(0.0, -x64)).astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    x64 = x.astype(np.float64)
    return (1.0 / (1.0 + np.exp(-x64))).astype(np.float32)


def _l2n(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return (x / n).astype(np.float32)


@dataclasses.dataclass(frozen=True)
class Spec:
    """One synthetic workload."""
    name: str
    family: str          # "hdla" | "gdn" | "generic"
    B: int
    H: int
    T: int
    dk: int
    dv: int
    chunk: int
    r_ab: int
    r_kv: int
    dtype: str           # "fp32" | "bf16"  (storage of q, K, V, A, B and out)
    lam_mu: float = 3.0  # mean of the pre-sigmoid forget-gate logit
    seed: int = 0

    @property
    def scalar_decay(self) -> bool:
        return self.family == "gdn"

    @property
    def tokens(self) -> int:
        return self.B * self.T

    @property
    def head_tokens(self) -> int:
        return self.B * self.H * self.T

    def describe(self) -> str:
        return (f"{self.family} B={self.B} H={self.H} T={self.T} dk={self.dk} dv={self.dv} "
                f"C={self.chunk} r_ab={self.r_ab} r_kv={self.r_kv} {self.dtype}")


# The five workloads: the small fp32 HDLA case, Gated DeltaNet rank 1, HDLA rank 2
# (the headline shape), long-context HDLA with slow decay, and a generic
# rank-(4, 2) recurrence.
CONFIGS: Dict[str, Spec] = {
    "hdla_fp32_small": Spec("hdla_fp32_small", "hdla", 1, 2, 512, 64, 64, 64, 2, 1, "fp32", 3.0),
    "gdn_bf16": Spec("gdn_bf16", "gdn", 4, 16, 4096, 128, 128, 64, 1, 1, "bf16"),
    "hdla_bf16": Spec("hdla_bf16", "hdla", 8, 16, 4096, 128, 128, 64, 2, 1, "bf16", 3.0),
    "hdla_long_bf16": Spec("hdla_long_bf16", "hdla", 1, 48, 32768, 64, 64, 64, 2, 1, "bf16", 4.0),
    "generic_fp32": Spec("generic_fp32", "generic", 2, 16, 16384, 128, 128, 64, 4, 2, "fp32"),
}
CONFIG_ORDER = ["hdla_fp32_small", "gdn_bf16", "hdla_bf16", "hdla_long_bf16", "generic_fp32"]
HEADLINE = "hdla_bf16"


def hdla_raw(B, H, T, dk, dv, dtype="fp32", lam_mu=3.0, seed=0) -> Dict[str, np.ndarray]:
    """HDLA inputs.  Draw order: q, k, v, x_lambda, x_beta.

    Returns q, k [B,H,T,dk]; v [B,H,T,dv] (rounded to ``dtype``);
    log_lambda [B,H,T,dk] float32 = log(sigmoid(x_lambda)); beta [B,H,T] float32
    = 2 sigmoid(x_beta).
    """
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, T, dk), dtype=np.float32)
    k = _l2n(rng.standard_normal((B, H, T, dk), dtype=np.float32))
    v = rng.standard_normal((B, H, T, dv), dtype=np.float32)
    xl = rng.standard_normal((B, H, T, dk), dtype=np.float32) + np.float32(lam_mu)
    xb = rng.standard_normal((B, H, T), dtype=np.float32)
    return dict(q=_store(q, dtype), k=_store(k, dtype), v=_store(v, dtype),
                log_lambda=_log_sigmoid(xl), beta=(2.0 * _sigmoid(xb)).astype(np.float32))


def gdn_raw(B, H, T, dk, dv, dtype="bf16", seed=0) -> Dict[str, np.ndarray]:
    """Gated DeltaNet inputs.  Draw order: q, k, v, x_g, x_beta.

    Returns q, k (both l2-normalised) [B,H,T,dk]; v [B,H,T,dv]; g [B,H,T] float32
    = -softplus(x_g) * 0.1; beta [B,H,T] float32 = sigmoid(x_beta).
    """
    rng = np.random.default_rng(seed)
    q = _l2n(rng.standard_normal((B, H, T, dk), dtype=np.float32))
    k = _l2n(rng.standard_normal((B, H, T, dk), dtype=np.float32))
    v = rng.standard_normal((B, H, T, dv), dtype=np.float32)
    xg = rng.standard_normal((B, H, T), dtype=np.float32)
    xb = rng.standard_normal((B, H, T), dtype=np.float32)
    g = (0.1 * _log_sigmoid(-xg).astype(np.float64)).astype(np.float32)  # -softplus(x) = log sigmoid(-x)
    return dict(q=_store(q, dtype), k=_store(k, dtype), v=_store(v, dtype),
                g=g, beta=_sigmoid(xb))


def generic_raw(B, H, T, dk, dv, r_ab, r_kv, dtype="fp32", decay="channel", lam_mu=3.0,
                ab_scale=0.5, seed=0) -> Dict[str, np.ndarray]:
    """Arbitrary-rank inputs.  Draw order: q, x_decay, A, B, K, V.

    q ~ N(0,1) [B,H,T,dk]; log_decay = log(sigmoid(N(lam_mu,1))) [B,H,T,dk]
    (or [B,H,T] when ``decay == "scalar"``); A, B ~ N(0,1)/sqrt(dk)*ab_scale
    [B,H,T,r_ab,dk]; K ~ N(0,1)/sqrt(dk) [B,H,T,r_kv,dk]; V ~ N(0,1)/sqrt(dk)
    [B,H,T,r_kv,dv].  A and B are None when r_ab == 0.
    """
    rng = np.random.default_rng(seed)
    s = np.float32(1.0 / np.sqrt(dk))
    q = rng.standard_normal((B, H, T, dk), dtype=np.float32)
    dshape = (B, H, T, dk) if decay == "channel" else (B, H, T)
    ld = _log_sigmoid(rng.standard_normal(dshape, dtype=np.float32) + np.float32(lam_mu))
    if r_ab > 0:
        A = rng.standard_normal((B, H, T, r_ab, dk), dtype=np.float32) * (s * np.float32(ab_scale))
        Bm = rng.standard_normal((B, H, T, r_ab, dk), dtype=np.float32) * (s * np.float32(ab_scale))
    else:
        A = Bm = None
    K = rng.standard_normal((B, H, T, r_kv, dk), dtype=np.float32) * s
    V = rng.standard_normal((B, H, T, r_kv, dv), dtype=np.float32) * s
    return dict(q=_store(q, dtype), log_decay=ld,
                A=None if A is None else _store(A, dtype), B=None if Bm is None else _store(Bm, dtype),
                K=_store(K, dtype), V=_store(V, dtype))


def raw_for(spec: Spec, B=None, H=None, T=None) -> Dict[str, np.ndarray]:
    """Raw inputs of a workload (optionally with a smaller B/H/T, same recipe and seed)."""
    B = spec.B if B is None else B
    H = spec.H if H is None else H
    T = spec.T if T is None else T
    if spec.family == "hdla":
        return hdla_raw(B, H, T, spec.dk, spec.dv, spec.dtype, spec.lam_mu, spec.seed)
    if spec.family == "gdn":
        return gdn_raw(B, H, T, spec.dk, spec.dv, spec.dtype, spec.seed)
    return generic_raw(B, H, T, spec.dk, spec.dv, spec.r_ab, spec.r_kv, spec.dtype, "channel",
                       spec.lam_mu, 0.5, spec.seed)


def hla_gates(B, H, T, chunk, mu=-4.0, sd=1.5, seed=0) -> np.ndarray:
    """Per (query token, chunk) routing gates w = sigmoid(s), s ~ N(mu, sd), float32
    [B, H, T, ceil(T / chunk)].  The HLA note ("Method steps", step 4) forms each gate
    as a sigmoid of a query-to-chunk score and keeps about three history chunks per
    query active (its routing budget, step 6); with mu = -4, sd = 1.5 about one gate
    in nine is at or above the inference threshold 0.1 (step 7)."""
    rng = np.random.default_rng(seed)
    N = -(-T // chunk)
    s = rng.standard_normal((B, H, T, N), dtype=np.float32) * np.float32(sd) + np.float32(mu)
    return _sigmoid(s)


def loglinear_lambdas(B, H, T, seed=0) -> np.ndarray:
    """Per (token, level) non-negative weights lam = softplus(N(0, 1)), float32
    [B, H, T, 1 + bit_length(T - 1)] (levels 0 .. that of position T - 1).  The
    Log-Linear note ("Key design" 2) makes each level's weight a non-negative
    function of the token's input; here they are drawn independently."""
    rng = np.random.default_rng(seed)
    L = 1 + int(T - 1).bit_length() if T > 0 else 0
    x = rng.standard_normal((B, H, T, L), dtype=np.float32)
    return (-_log_sigmoid(-x).astype(np.float64)).astype(np.float32)   # softplus(x) = -log sigmoid(-x)


def device_raw(spec: Spec, torch, device, seed: int = 0):
    """The same distributions as :func:`raw_for`, drawn on the device with a seeded
    torch generator (used where only timing needs the inputs: the values differ
    from the numpy stream, the shapes and distributions do not).  Returns a dict
    of device tensors in the storage dtype (decay, beta in float32)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    td = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
    B, H, T, dk, dv = spec.B, spec.H, spec.T, spec.dk, spec.dv
    f32 = dict(dtype=torch.float32, device=device, generator=g)
    normal = lambda *shape: torch.randn(shape, **f32)
    l2n = lambda x: x / x.norm(dim=-1, keepdim=True)
    logsig = torch.nn.functional.logsigmoid
    if spec.family == "hdla":
        q, k, v = normal(B, H, T, dk), l2n(normal(B, H, T, dk)), normal(B, H, T, dv)
        ll = logsig(normal(B, H, T, dk) + spec.lam_mu)
        beta = 2.0 * torch.sigmoid(normal(B, H, T))
        return dict(q=q.to(td), k=k.to(td), v=v.to(td), log_lambda=ll, beta=beta)
    if spec.family == "gdn":
        q, k, v = l2n(normal(B, H, T, dk)), l2n(normal(B, H, T, dk)), normal(B, H, T, dv)
        gg = 0.1 * logsig(-normal(B, H, T))
        beta = torch.sigmoid(normal(B, H, T))
        return dict(q=q.to(td), k=k.to(td), v=v.to(td), g=gg, beta=beta)
    s = 1.0 / float(np.sqrt(dk))
    q = normal(B, H, T, dk)
    ld = logsig(normal(B, H, T, dk) + spec.lam_mu)
    A = normal(B, H, T, spec.r_ab, dk) * (s * 0.5) if spec.r_ab > 0 else None
    Bm = normal(B, H, T, spec.r_ab, dk) * (s * 0.5) if spec.r_ab > 0 else None
    K = normal(B, H, T, spec.r_kv, dk) * s
    V = normal(B, H, T, spec.r_kv, dv) * s
    return dict(q=q.to(td), log_decay=ld, A=None if A is None else A.to(td), B=None if Bm is None else Bm.to(td),
                K=K.to(td), V=V.to(td))
