"""Full-size parity on the five workloads, in the launch configuration the
benchmark times.  The GPU runs every (batch, head); the fp64 oracle checks a
sample of (batch, head) pairs one by one (first, middle, last), which covers
every output and state element of those heads."""
import numpy as np
import pytest

import oracle
import workloads
from tests.helpers import TOL, dev, host, rel_err, store_like, torch_dtype

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu, pytest.mark.slow]
lattn = pytest.importorskip("structured_decay_sequence_amd")


def _sample_heads(spec):
    BH = spec.B * spec.H
    idx = sorted({0, BH // 2, BH - 1})
    return [(i // spec.H, i % spec.H) for i in idx]


def _run_gpu(spec, raw):
    td = torch_dtype(spec.dtype)
    if spec.family == "hdla":
        k, v = dev(raw["k"], td), dev(raw["v"], td)
        ld = dev(raw["log_lambda"])
        A, B, V = lattn.hdla_params(k, v, ld, dev(raw["beta"]))
        K = k
    elif spec.family == "gdn":
        k, v = dev(raw["k"], td), dev(raw["v"], td)
        ld = dev(raw["g"])
        A, B, V = lattn.gdn_params(k, v, ld, dev(raw["beta"]))
        K = k
    else:
        K, V, ld = dev(raw["K"], td), dev(raw["V"], td), dev(raw["log_decay"])
        A, B = dev(raw["A"], td), dev(raw["B"], td)
    out, S = lattn.chunk_fwd(dev(raw["q"], td), K, V, ld, A, B, chunk=spec.chunk)
    torch.cuda.synchronize()
    return out, S


def _oracle_head(spec, raw, b, h):
    sl = lambda x: x[b:b + 1, h:h + 1]
    if spec.family == "hdla":
        ll, A, B, K, V = oracle.hdla_to_generic(sl(raw["k"]), sl(raw["v"]), sl(raw["log_lambda"]), sl(raw["beta"]))
        gen = oracle.generic(sl(raw["q"]), sl(raw["k"])[..., None, :], store_like(V, spec.dtype), sl(raw["log_lambda"]),
                             store_like(A, spec.dtype), store_like(B, spec.dtype))
        struct = oracle.hdla(sl(raw["q"]), sl(raw["k"]), sl(raw["v"]), sl(raw["log_lambda"]), sl(raw["beta"]))
        return gen, struct
    if spec.family == "gdn":
        g, A, B, K, V = oracle.gdn_to_generic(sl(raw["k"]), sl(raw["v"]), sl(raw["g"]), sl(raw["beta"]))
        gen = oracle.generic(sl(raw["q"]), sl(raw["k"])[..., None, :], store_like(V, spec.dtype), sl(raw["g"]),
                             store_like(A, spec.dtype), store_like(B, spec.dtype))
        struct = oracle.gdn(sl(raw["q"]), sl(raw["k"]), sl(raw["v"]), sl(raw["g"]), sl(raw["beta"]))
        return gen, struct
    gen = oracle.generic(sl(raw["q"]), sl(raw["K"]), sl(raw["V"]), sl(raw["log_decay"]), sl(raw["A"]), sl(raw["B"]))
    return gen, None


@pytest.mark.parametrize("name", workloads.CONFIG_ORDER)
def test_workload_full_size(name):
    spec = workloads.CONFIGS[name]
    print(f"workload {name}: {spec.describe()}", flush=True)
    raw = workloads.raw_for(spec)
    out, S = _run_gpu(spec, raw)
    tol = TOL[spec.dtype]
    for b, h in _sample_heads(spec):
        (r_out, r_S), struct = _oracle_head(spec, raw, b, h)
        g_out = host(out[b:b + 1, h:h + 1])
        g_S = host(S[b:b + 1, h:h + 1])
        e_o, e_s = rel_err(g_out, r_out), rel_err(g_S, r_S)
        msg = f"{name} head ({b},{h}): out {e_o:.2e} state {e_s:.2e}"
        if struct is not None:
            msg += f" | structured-form distance out {rel_err(g_out, struct[0]):.2e} state {rel_err(g_S, struct[1]):.2e}"
        print(msg, flush=True)
        assert e_o <= tol and e_s <= tol, msg
        assert np.all(np.isfinite(g_out))


@pytest.mark.parametrize("name", [n for n in workloads.CONFIG_ORDER if workloads.CONFIGS[n].family != "generic"])
def test_workload_full_size_fused(name):
    """The fused family forward on the same full-size workloads, sampled heads
    against the structured oracle (which sees only the raw parameters)."""
    spec = workloads.CONFIGS[name]
    print(f"workload {name} (fused): {spec.describe()}", flush=True)
    raw = workloads.raw_for(spec)
    td = torch_dtype(spec.dtype)
    q, k, v = dev(raw["q"], td), dev(raw["k"], td), dev(raw["v"], td)
    if spec.family == "hdla":
        out, S = lattn.hdla_chunk_fwd(q, k, v, dev(raw["log_lambda"]), dev(raw["beta"]), chunk=spec.chunk)
    else:
        out, S = lattn.gdn_chunk_fwd(q, k, v, dev(raw["g"]), dev(raw["beta"]), chunk=spec.chunk)
    torch.cuda.synchronize()
    tol = TOL[spec.dtype]
    for b, h in _sample_heads(spec):
        _, (r_out, r_S) = _oracle_head(spec, raw, b, h)
        e_o = rel_err(host(out[b:b + 1, h:h + 1]), r_out)
        e_s = rel_err(host(S[b:b + 1, h:h + 1]), r_S)
        msg = f"{name} fused head ({b},{h}): out {e_o:.2e} state {e_s:.2e}"
        print(msg, flush=True)
        assert e_o <= tol and e_s <= tol, msg
