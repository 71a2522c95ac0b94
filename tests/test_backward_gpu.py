"""GPU parity of the backward pass (lattn_chunk_bwd) against the fp64 BPTT oracle
(itself pinned by finite differences), through the C ABI.

Gate per gradient tensor: max|gpu - ref| / max|ref| <= 1e-4 for fp32 storage and
<= 2e-2 for bf16 storage (fp32 arithmetic and fp32 gradients in both).
"""
import numpy as np
import pytest

import oracle
from oracle import backward as bwd_oracle
import workloads
from tests.helpers import TOL, dev, host, rel_err, store_like, torch_dtype

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

lattn = pytest.importorskip("structured_decay_sequence_amd")

CASES = [
    # B, H, T, dk, dv, r_ab, r_kv, C, dtype, decay, state terms
    (1, 2, 100, 32, 32, 2, 1, 32, "fp32", "channel", True),
    (1, 1, 77, 64, 48, 1, 2, 16, "fp32", "scalar", True),
    (2, 1, 64, 16, 16, 0, 1, 64, "fp32", "channel", False),
    (1, 1, 90, 48, 64, 4, 2, 64, "fp32", "channel", True),
    (1, 1, 130, 128, 128, 2, 1, 64, "fp32", "channel", True),
    (1, 2, 70, 64, 64, 2, 1, 32, "bf16", "channel", True),
    (1, 1, 1, 32, 32, 1, 1, 16, "fp32", "channel", True),
    # more (batch, head, chunk) jobs than resident workgroups (276 > 256)
    (1, 4, 1100, 32, 32, 2, 1, 16, "fp32", "channel", True),
    # bf16 storage at C 64, r_kv 1, d_k, d_v in {64, 128}: the chunked route on
    # bf16 MFMAs (65 chunks per head with a 4-token tail here)
    (2, 3, 4100, 64, 64, 1, 1, 64, "bf16", "scalar", True),
    (1, 2, 150, 64, 64, 2, 1, 64, "bf16", "channel", True),
    (1, 1, 200, 128, 128, 2, 1, 64, "bf16", "channel", True),
    (2, 1, 100, 64, 128, 0, 1, 64, "bf16", "channel", False),
    (1, 1, 130, 128, 64, 1, 1, 64, "bf16", "scalar", True),
    (1, 1, 1, 64, 64, 2, 1, 64, "bf16", "channel", True),
    (1, 1, 64, 128, 128, 2, 1, 64, "bf16", "scalar", False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}T{}dk{}dv{}r{}-{}C{}{}{}s{}".format(*c))
def test_backward_parity(case):
    Bb, H, T, dk, dv, r_ab, r_kv, C, dtype, decay, state = case
    print(f"backward case {case}", flush=True)
    raw = workloads.generic_raw(Bb, H, T, dk, dv, r_ab, r_kv, dtype, decay, seed=T + dk)
    rng = np.random.default_rng(T)
    dout = workloads.round_bf16(rng.standard_normal((Bb, H, T, dv)).astype(np.float32)) if dtype == "bf16" \
        else rng.standard_normal((Bb, H, T, dv)).astype(np.float32)
    S0 = (rng.standard_normal((Bb, H, dk, dv)) * 0.1).astype(np.float32) if state else None
    dfin = rng.standard_normal((Bb, H, dk, dv)).astype(np.float32) if state else None
    td = torch_dtype(dtype)
    g = lattn.chunk_bwd(dev(raw["q"], td), dev(raw["K"], td), dev(raw["V"], td), dev(raw["log_decay"]),
                        dev(raw["A"], td), dev(raw["B"], td), dev(dout, td), chunk=C, dfinal=dev(dfin),
                        initial_state=dev(S0))
    torch.cuda.synchronize()
    ref = bwd_oracle.backward(raw["q"], raw["K"], raw["V"], raw["log_decay"], raw["A"], raw["B"], dout, dfin, S0)
    pairs = [("dq", "dq"), ("dk", "dK"), ("dv", "dV"), ("dlog_decay", "dlog_decay"), ("dA", "dA"), ("dB", "dB"),
             ("dinitial_state", "dS0")]
    for gn, rn in pairs:
        if ref[rn] is None:
            assert g[gn] is None
            continue
        e = rel_err(host(g[gn]), ref[rn])
        print(f"{gn} {e:.2e}", flush=True)
        assert e <= TOL[dtype], gn


def test_backward_rejects_unsupported():
    raw = workloads.generic_raw(1, 1, 16, 256, 64, 1, 1, "fp32", "channel", seed=0)
    with pytest.raises(lattn.LattnError):
        lattn.chunk_bwd(dev(raw["q"]), dev(raw["K"]), dev(raw["V"]), dev(raw["log_decay"]), dev(raw["A"]),
                        dev(raw["B"]), dev(np.zeros((1, 1, 16, 64), np.float32)), chunk=16)


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_backward_headline_workload_full_heads():
    """The headline HDLA workload (B8 H16 T4096 d128, C 64, bf16) through
    lattn_chunk_bwd as bench.py calls it (output cotangents on every token and a
    final-state cotangent); every gradient of two whole (batch, head) rows against
    the oracle on its own decay operands (the fp64 HDLA rewrite rounded to bf16)."""
    spec = workloads.CONFIGS[workloads.HEADLINE]
    raw = workloads.raw_for(spec)
    td = torch.bfloat16
    k, v = dev(raw["k"], td), dev(raw["v"], td)
    ll = dev(raw["log_lambda"])
    A, B, V = lattn.hdla_params(k, v, ll, dev(raw["beta"]))
    rng = np.random.default_rng(2)
    dout = workloads.round_bf16(rng.standard_normal((spec.B, spec.H, spec.T, spec.dv)).astype(np.float32))
    dfin = rng.standard_normal((spec.B, spec.H, spec.dk, spec.dv)).astype(np.float32)
    g = lattn.chunk_bwd(dev(raw["q"], td), k, V, ll, A, B, dev(dout, td), chunk=spec.chunk, dfinal=dev(dfin))
    torch.cuda.synchronize()
    del A, B, V
    pairs = [("dq", "dq"), ("dk", "dK"), ("dv", "dV"), ("dlog_decay", "dlog_decay"), ("dA", "dA"), ("dB", "dB")]
    for b, h in ((0, 0), (spec.B - 1, spec.H - 1)):
        sl = lambda x: x[b:b + 1, h:h + 1]
        lld, rA, rB, rK, rV = oracle.hdla_to_generic(sl(raw["k"]), sl(raw["v"]), sl(raw["log_lambda"]),
                                                     sl(raw["beta"]))
        ref = bwd_oracle.backward(sl(raw["q"]), sl(raw["k"])[..., None, :], store_like(rV, "bf16"),
                                  sl(raw["log_lambda"]), store_like(rA, "bf16"), store_like(rB, "bf16"), sl(dout),
                                  dfinal=sl(dfin))
        for gn, rn in pairs + [("dinitial_state", "dS0")]:
            got = host(g[gn][b:b + 1, h:h + 1])
            e = rel_err(got, ref[rn])
            print(f"(b {b}, h {h}) {gn} all {spec.T} tokens: {e:.2e}", flush=True)
            assert e <= TOL["bf16"], gn


def test_backward_empty_sequence_passes_the_state_gradient():
    """T = 0: no token, so the initial state's gradient is the final state's cotangent."""
    raw = workloads.generic_raw(1, 2, 0, 32, 32, 1, 1, "fp32", "channel", seed=0)
    dfin = np.random.default_rng(0).standard_normal((1, 2, 32, 32)).astype(np.float32)
    g = lattn.chunk_bwd(dev(raw["q"]), dev(raw["K"]), dev(raw["V"]), dev(raw["log_decay"]), dev(raw["A"]),
                        dev(raw["B"]), dev(np.zeros((1, 2, 0, 32), np.float32)), chunk=16, dfinal=dev(dfin))
    torch.cuda.synchronize()
    assert np.array_equal(host(g["dinitial_state"]), dfin)


@pytest.mark.parametrize("chunk", [32, 64])
def test_backward_repeatable(chunk):
    """Two calls give bitwise equal gradients (chunk 64: the chunked route)."""
    raw = workloads.generic_raw(1, 2, 90, 64, 64, 2, 1, "bf16", "channel", seed=4)
    dout = workloads.round_bf16(np.random.default_rng(4).standard_normal((1, 2, 90, 64)).astype(np.float32))
    run = lambda: lattn.chunk_bwd(dev(raw["q"], torch.bfloat16), dev(raw["K"], torch.bfloat16),
                                  dev(raw["V"], torch.bfloat16), dev(raw["log_decay"]), dev(raw["A"], torch.bfloat16),
                                  dev(raw["B"], torch.bfloat16), dev(dout, torch.bfloat16), chunk=chunk)
    a, b = run(), run()
    torch.cuda.synchronize()
    for n in a:
        if a[n] is not None:
            assert torch.equal(a[n], b[n]), n
