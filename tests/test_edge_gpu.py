"""GPU edge cases of the chunk-wise forward, through the C ABI.

* Strong decay: the chunk-wise form scales operands by exp(+-G) with G the
  chunk-local cumulative log-decay, so a chunk whose -G approaches the guard
  LATTN_MAX_CHUNK_LOG_DECAY (80) puts bf16 and fp32 operands near exp(+-80).
  Cases at -G of 40, 60 and 79.5 on half the channels, and chunks holding
  tokens with lambda ~ 1e-13 (near-zero forget gate), on the bf16 MFMA path
  (generic and fused HDLA / Gated DeltaNet entry points) and the general fp32
  path, each against the fp64 oracle on the same stored inputs.
* Exact special cases with a closed form that needs no oracle (HDLA note,
  "Key design 2"; HLA note, "Prerequisites: Gated DeltaNet"):
  - unit k, beta = 2, lambda = 1: each transition is a Householder reflection
    squared, P_t = I, so the output is causal linear attention with write
    2 k v^T and the final state is sum_t 2 k_t v_t^T;
  - unit k, beta = 1, q_t = k_t: P_t k_t = 0 for HDLA and Gated DeltaNet
    (delta-rule exact recall), so o_t = v_t for every token.
  The unit keys have 16 entries of +-1/4 (d_k = 128), exactly representable
  in bf16, so the stored keys are exactly unit vectors.
* NaN: the decay-range check reports a NaN log-decay.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.helpers import TOL, dev, host, rel_err, store_like, torch_dtype

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

lattn = pytest.importorskip("structured_decay_sequence_amd")


def _strong_decay(shape_tok, dk, level, seed):
    """log-decay [*shape_tok, dk]: channels 0 .. dk/2-1 decay at -level/64 per token
    (so a full 64-token chunk reaches -G = level), the rest ~ log sigmoid(N(3, 1))."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape_tok + (dk,)).astype(np.float32) + np.float32(3.0)
    ld = (-np.logaddexp(0.0, -x.astype(np.float64))).astype(np.float32)
    ld[..., : dk // 2] = np.float32(-level / 64.0)
    return ld


def _near_zero_gate(shape_tok, dk, seed, chunk=64):
    """log-decay with two tokens per chunk at log lambda = -30 on every channel
    (lambda ~ 9e-14); the rest ~ log sigmoid(N(3, 1)).  Per chunk -G stays below 80."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape_tok + (dk,)).astype(np.float32) + np.float32(3.0)
    ld = (-np.logaddexp(0.0, -x.astype(np.float64))).astype(np.float32)
    T = shape_tok[-1]
    for j0 in range(0, T, chunk):
        n = min(chunk, T - j0)
        picks = rng.choice(n, size=min(2, n), replace=False)
        ld[..., j0 + picks, :] = np.float32(-30.0)
    return ld


def _check_in_range(ld):
    lattn.check_decay_range(dev(ld), 64)   # raises LattnError beyond the guard
    return float(host(lattn.decay_range(dev(ld), 64)).max())


DECAY_CASES = ["level40", "level60", "level79.5", "near_zero"]


def _decay(kind, shape_tok, dk, seed):
    if kind == "near_zero":
        return _near_zero_gate(shape_tok, dk, seed)
    return _strong_decay(shape_tok, dk, float(kind[5:]), seed)


@pytest.mark.parametrize("kind", DECAY_CASES)
@pytest.mark.parametrize("path", ["mfma_bf16", "general_fp32"])
def test_strong_decay_generic(kind, path):
    Bb, H, T = 1, 2, 200
    dk = dv = 128 if path == "mfma_bf16" else 64
    dtype = "bf16" if path == "mfma_bf16" else "fp32"
    raw = workloads.generic_raw(Bb, H, T, dk, dv, 2, 1, dtype, "channel", seed=21)
    raw["log_decay"] = _decay(kind, (Bb, H, T), dk, seed=22)
    gmax = _check_in_range(raw["log_decay"])
    td = torch_dtype(dtype)
    dims = lattn.make_dims(Bb, H, T, dk, dv, 1 if dtype == "bf16" else 0, False)
    import ctypes
    assert lattn._lib.load().lattn_chunk_fwd_kernels(ctypes.byref(dims), 2, 1, 64).decode() == path
    S0 = (np.random.default_rng(23).standard_normal((Bb, H, dk, dv)) * 0.1).astype(np.float32)
    out, S = lattn.chunk_fwd(dev(raw["q"], td), dev(raw["K"], td), dev(raw["V"], td), dev(raw["log_decay"]),
                             dev(raw["A"], td), dev(raw["B"], td), chunk=64, initial_state=dev(S0))
    torch.cuda.synchronize()
    ref_out, ref_S = oracle.generic(raw["q"], raw["K"], raw["V"], raw["log_decay"], raw["A"], raw["B"],
                                    initial_state=S0)
    e_o, e_s = rel_err(host(out), ref_out), rel_err(host(S), ref_S)
    print(f"{path} {kind}: max chunk -G {gmax:.2f}  out {e_o:.2e} state {e_s:.2e}", flush=True)
    assert np.all(np.isfinite(host(out)))
    assert e_o <= TOL[dtype] and e_s <= TOL[dtype]


@pytest.mark.parametrize("kind", DECAY_CASES)
def test_strong_decay_fused_hdla(kind):
    Bb, H, T, d = 1, 2, 200, 128
    raw = workloads.hdla_raw(Bb, H, T, d, d, "bf16", 3.0, seed=24)
    raw["log_lambda"] = _decay(kind, (Bb, H, T), d, seed=25)
    gmax = _check_in_range(raw["log_lambda"])
    td = torch.bfloat16
    out, S = lattn.hdla_chunk_fwd(dev(raw["q"], td), dev(raw["k"], td), dev(raw["v"], td), dev(raw["log_lambda"]),
                                  dev(raw["beta"]), chunk=64)
    torch.cuda.synchronize()
    ref_out, ref_S = oracle.hdla(raw["q"], raw["k"], raw["v"], raw["log_lambda"], raw["beta"])
    e_o, e_s = rel_err(host(out), ref_out), rel_err(host(S), ref_S)
    print(f"fused hdla {kind}: max chunk -G {gmax:.2f}  out {e_o:.2e} state {e_s:.2e}", flush=True)
    assert e_o <= TOL["bf16"] and e_s <= TOL["bf16"]


@pytest.mark.parametrize("level", [40.0, 79.5])
@pytest.mark.parametrize("entry", ["generic", "fused"])
def test_strong_decay_gdn(level, entry):
    """Scalar decay g = -level/64 per token: every chunk reaches -G = level."""
    Bb, H, T, d = 1, 2, 200, 128
    raw = workloads.gdn_raw(Bb, H, T, d, d, "bf16", seed=26)
    raw["g"] = np.full((Bb, H, T), -level / 64.0, dtype=np.float32)
    gmax = _check_in_range(raw["g"])
    td = torch.bfloat16
    q, k, v = dev(raw["q"], td), dev(raw["k"], td), dev(raw["v"], td)
    g, beta = dev(raw["g"]), dev(raw["beta"])
    if entry == "generic":
        A, B, V = lattn.gdn_params(k, v, g, beta)
        out, S = lattn.chunk_fwd(q, k, V, g, A, B, chunk=64)
    else:
        out, S = lattn.gdn_chunk_fwd(q, k, v, g, beta, chunk=64)
    torch.cuda.synchronize()
    ref_out, ref_S = oracle.gdn(raw["q"], raw["k"], raw["v"], raw["g"], raw["beta"])
    e_o, e_s = rel_err(host(out), ref_out), rel_err(host(S), ref_S)
    print(f"gdn {entry} level {level}: max chunk -G {gmax:.2f}  out {e_o:.2e} state {e_s:.2e}", flush=True)
    assert e_o <= TOL["bf16"] and e_s <= TOL["bf16"]


def _unit_keys(Bb, H, T, d, seed, nnz=16):
    """Keys with nnz entries of +-1/sqrt(nnz) (1/4 for nnz = 16): exact unit vectors in bf16."""
    rng = np.random.default_rng(seed)
    k = np.zeros((Bb, H, T, d), dtype=np.float32)
    for idx in np.ndindex(Bb, H, T):
        ch = rng.choice(d, size=nnz, replace=False)
        k[idx + (ch,)] = rng.choice([-1.0, 1.0], size=nnz).astype(np.float32) / np.float32(np.sqrt(nnz))
    return k


@pytest.mark.parametrize("entry", ["generic", "fused"])
def test_reflection_squared_is_linear_attention(entry):
    """beta = 2, lambda = 1, unit k: P_t = (I - 2kk^T)^2 = I, write 2 k v^T."""
    Bb, H, T, d = 1, 2, 200, 128
    rng = np.random.default_rng(27)
    q = workloads.round_bf16(rng.standard_normal((Bb, H, T, d)).astype(np.float32))
    k = _unit_keys(Bb, H, T, d, seed=28)
    v = workloads.round_bf16(rng.standard_normal((Bb, H, T, d)).astype(np.float32))
    ll = np.zeros((Bb, H, T, d), dtype=np.float32)
    beta = np.full((Bb, H, T), 2.0, dtype=np.float32)
    td = torch.bfloat16
    qd, kd, vd, lld, bd = dev(q, td), dev(k, td), dev(v, td), dev(ll), dev(beta)
    if entry == "generic":
        A, B, V = lattn.hdla_params(kd, vd, lld, bd)
        out, S = lattn.chunk_fwd(qd, kd, V, lld, A, B, chunk=64)
    else:
        out, S = lattn.hdla_chunk_fwd(qd, kd, vd, lld, bd, chunk=64)
    torch.cuda.synchronize()
    q64, k64, v64 = (x.astype(np.float64) for x in (q, k, v))
    mask = np.tril(np.ones((T, T)))
    ref_out = np.matmul(np.matmul(q64, np.swapaxes(k64, -1, -2)) * mask, 2.0 * v64)
    ref_S = np.matmul(np.swapaxes(k64, -1, -2), 2.0 * v64)
    e_o, e_s = rel_err(host(out), ref_out), rel_err(host(S), ref_S)
    print(f"P = I ({entry}): out {e_o:.2e} state {e_s:.2e}", flush=True)
    assert e_o <= TOL["bf16"] and e_s <= TOL["bf16"]


@pytest.mark.parametrize("family,entry", [("hdla", "generic"), ("hdla", "fused"), ("gdn", "generic"), ("gdn", "fused")])
def test_exact_recall(family, entry):
    """Unit k, beta = 1, q_t = k_t: P_t k_t = 0, so o_t = v_t exactly."""
    Bb, H, T, d = 1, 2, 200, 128
    rng = np.random.default_rng(29)
    k = _unit_keys(Bb, H, T, d, seed=30)
    v = workloads.round_bf16(rng.standard_normal((Bb, H, T, d)).astype(np.float32))
    beta = np.ones((Bb, H, T), dtype=np.float32)
    td = torch.bfloat16
    kd, vd, bd = dev(k, td), dev(v, td), dev(beta)
    if family == "hdla":
        decay = workloads.hdla_raw(Bb, H, T, d, d, "bf16", 3.0, seed=31)["log_lambda"]
    else:
        decay = workloads.gdn_raw(Bb, H, T, d, d, "bf16", seed=31)["g"]
    dd = dev(decay)
    if entry == "generic":
        params = lattn.hdla_params if family == "hdla" else lattn.gdn_params
        A, B, V = params(kd, vd, dd, bd)
        out, _ = lattn.chunk_fwd(kd, kd, V, dd, A, B, chunk=64)
    else:
        fwd = lattn.hdla_chunk_fwd if family == "hdla" else lattn.gdn_chunk_fwd
        out, _ = fwd(kd, kd, vd, dd, bd, chunk=64)
    torch.cuda.synchronize()
    e = rel_err(host(out), v)
    print(f"exact recall {family} {entry}: out vs v {e:.2e}", flush=True)
    assert e <= TOL["bf16"]


def test_decay_range_reports_nan():
    ld = workloads.hdla_raw(1, 1, 130, 32, 32, "fp32", 3.0, seed=32)["log_lambda"]
    ld[0, 0, 70, 5] = np.nan
    got = host(lattn.decay_range(dev(ld), 64))
    assert np.isfinite(got[0, 0, 0]) and np.isnan(got[0, 0, 1]) and np.isfinite(got[0, 0, 2])
    with pytest.raises(lattn.LattnError) as ei:
        lattn.check_decay_range(dev(ld), 64)
    assert ei.value.status == -5
