"""Full-size parity on the five workloads, in the launch configuration the
benchmark times, on EVERY (batch, head).

The GPU runs the whole workload; the fp64 oracle (OpenMP over (batch, head)
on all host cores) runs every (batch, head) on the same stored inputs.  The
gate is the global one, max|gpu - ref| / max|ref| over the whole tensor, for
out and the final state separately; the worst (batch, head) by its own
relative error is reported beside it.  For HDLA and Gated DeltaNet the
generic entry point is compared with the generic oracle on the oracle's own
low-rank rewrite of the raw parameters (rounded to the stored dtype), and the
fused family entry point with the structured (Householder / GDN) oracle, which
sees only the raw parameters.

Set LATTN_PARITY_LOG to a file path to append one JSON line of margins per
workload and entry point.
"""
import json
import os

import numpy as np
import pytest

import oracle
import workloads
from tests.helpers import TOL, dev, host, rel_err, store_like, torch_dtype

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu, pytest.mark.slow]
lattn = pytest.importorskip("structured_decay_sequence_amd")


def _per_head(got, ref):
    """Worst relative error of one (batch, head) against its own max|ref|, and where."""
    BH = got.shape[0] * got.shape[1]
    g = got.reshape(BH, -1).astype(np.float64)
    r = ref.reshape(BH, -1)
    scale = np.maximum(np.abs(r).max(axis=1), 1e-300)
    e = np.abs(g - r).max(axis=1) / scale
    i = int(np.argmax(e))
    return float(e[i]), (i // got.shape[1], i % got.shape[1])


def _log(rec):
    path = os.environ.get("LATTN_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")


def _compare(name, entry, spec, out, S, ref_out, ref_S, extra=None):
    g_out, g_S = host(out), host(S)
    tol = TOL[spec.dtype]
    e_o, e_s = rel_err(g_out, ref_out), rel_err(g_S, ref_S)
    h_o, at_o = _per_head(g_out, ref_out)
    h_s, at_s = _per_head(g_S, ref_S)
    rec = dict(workload=name, entry=entry, heads=spec.B * spec.H, tol=tol, out=e_o, state=e_s,
               worst_head_out=h_o, worst_head_out_at=at_o, worst_head_state=h_s, worst_head_state_at=at_s)
    if extra:
        rec.update(extra)
    msg = (f"{name} [{entry}] all {spec.B * spec.H} heads: out {e_o:.2e} state {e_s:.2e} (tol {tol:g}); "
           f"worst head out {h_o:.2e} at {at_o}, state {h_s:.2e} at {at_s}")
    print(msg, flush=True)
    _log(rec)
    assert np.all(np.isfinite(g_out)) and np.all(np.isfinite(g_S)), msg
    assert e_o <= tol and e_s <= tol, msg


def _oracle_inputs(spec, raw):
    """Generic-form oracle inputs on the same stored values the GPU receives."""
    if spec.family == "hdla":
        ll, A, B, K, V = oracle.hdla_to_generic(raw["k"], raw["v"], raw["log_lambda"], raw["beta"])
        return raw["q"], raw["k"][..., None, :], store_like(V, spec.dtype), raw["log_lambda"], \
            store_like(A, spec.dtype), store_like(B, spec.dtype)
    if spec.family == "gdn":
        g, A, B, K, V = oracle.gdn_to_generic(raw["k"], raw["v"], raw["g"], raw["beta"])
        return raw["q"], raw["k"][..., None, :], store_like(V, spec.dtype), raw["g"], \
            store_like(A, spec.dtype), store_like(B, spec.dtype)
    return raw["q"], raw["K"], raw["V"], raw["log_decay"], raw["A"], raw["B"]


def _gpu_generic(spec, raw):
    td = torch_dtype(spec.dtype)
    if spec.family in ("hdla", "gdn"):
        k, v = dev(raw["k"], td), dev(raw["v"], td)
        ld = dev(raw["log_lambda"] if spec.family == "hdla" else raw["g"])
        params = lattn.hdla_params if spec.family == "hdla" else lattn.gdn_params
        A, B, V = params(k, v, ld, dev(raw["beta"]))
        K = k
    else:
        K, V, ld = dev(raw["K"], td), dev(raw["V"], td), dev(raw["log_decay"])
        A, B = dev(raw["A"], td), dev(raw["B"], td)
    q = dev(raw["q"], td)
    out, S = lattn.chunk_fwd(q, K, V, ld, A, B, chunk=spec.chunk)
    torch.cuda.synchronize()
    return out, S, (q, K, V, ld, A, B)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", workloads.CONFIG_ORDER)
def test_workload_every_head(name):
    spec = workloads.CONFIGS[name]
    print(f"workload {name}: {spec.describe()} ({oracle.max_threads()} oracle threads)", flush=True)
    raw = workloads.raw_for(spec)
    out, S, inputs = _gpu_generic(spec, raw)
    if name == workloads.HEADLINE:
        # bitwise repeatability at the benchmark's shape and launch configuration
        out2, S2 = lattn.chunk_fwd(*inputs, chunk=spec.chunk)
        torch.cuda.synchronize()
        assert torch.equal(out, out2) and torch.equal(S, S2), "headline forward is not bitwise repeatable"
        print(f"{name}: two calls bitwise equal", flush=True)
        del out2, S2
    del inputs
    ref_out, ref_S = oracle.generic(*_oracle_inputs(spec, raw))
    _compare(name, "lattn_chunk_fwd", spec, out, S, ref_out, ref_S)
    del ref_out, ref_S
    if spec.family not in ("hdla", "gdn"):
        return
    if spec.family == "hdla":
        st_out, st_S = oracle.hdla(raw["q"], raw["k"], raw["v"], raw["log_lambda"], raw["beta"])
    else:
        st_out, st_S = oracle.gdn(raw["q"], raw["k"], raw["v"], raw["g"], raw["beta"])
    # distance of the generic entry point from the structured form (includes the
    # rounding of A, B to the stored dtype): reported, not gated
    print(f"{name}: generic entry vs structured oracle: out {rel_err(host(out), st_out):.2e} "
          f"state {rel_err(host(S), st_S):.2e}", flush=True)
    del out, S
    td = torch_dtype(spec.dtype)
    q, k, v = dev(raw["q"], td), dev(raw["k"], td), dev(raw["v"], td)
    if spec.family == "hdla":
        f_out, f_S = lattn.hdla_chunk_fwd(q, k, v, dev(raw["log_lambda"]), dev(raw["beta"]), chunk=spec.chunk)
        entry = "lattn_hdla_chunk_fwd"
    else:
        f_out, f_S = lattn.gdn_chunk_fwd(q, k, v, dev(raw["g"]), dev(raw["beta"]), chunk=spec.chunk)
        entry = "lattn_gdn_chunk_fwd"
    torch.cuda.synchronize()
    _compare(name, entry, spec, f_out, f_S, st_out, st_S)
