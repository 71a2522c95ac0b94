"""GPU parity of the query-conditioned chunk composition (lattn_hla_fwd) against
the fp64 HLA oracle, through the C ABI.

Gate as for the base path: max|gpu - ref| / max|ref| <= 1e-4 for fp32 storage
and <= 2e-2 for bf16 storage (the arithmetic is fp32 in both).  Inputs are the
seeded generic recurrence inputs and seeded sigmoid gates; the oracle runs on
the same stored values.
"""
import numpy as np
import pytest

import oracle
from oracle import hla as hla_oracle
import workloads
from tests.helpers import TOL, dev, host, rel_err, store_like, torch_dtype

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

lattn = pytest.importorskip("structured_decay_sequence_amd")


def _gpu(raw, gates, dtype, chunk, theta):
    td = torch_dtype(dtype)
    out = lattn.hla_fwd(dev(raw["q"], td), dev(raw["K"], td), dev(raw["V"], td), dev(raw["log_decay"]),
                        dev(raw["A"], td), dev(raw["B"], td), dev(gates), chunk=chunk, theta=theta)
    torch.cuda.synchronize()
    return host(out)


CASES = [
    # B, H, T, dk, dv, r_ab, r_kv, C, dtype, decay, gate mean
    (1, 2, 200, 64, 64, 2, 1, 64, "fp32", "channel", -2.0),
    (1, 2, 300, 32, 32, 1, 1, 32, "fp32", "scalar", -4.0),
    (2, 1, 77, 48, 32, 2, 2, 16, "fp32", "channel", -1.0),
    (1, 1, 300, 32, 64, 0, 1, 128, "fp32", "channel", -2.0),
    (1, 1, 40, 16, 16, 1, 1, 64, "fp32", "channel", 0.0),
    (1, 2, 130, 64, 64, 2, 1, 64, "bf16", "channel", -2.0),      # operators from the bf16 MFMA prepare
    (1, 1, 200, 128, 128, 2, 1, 64, "bf16", "channel", -2.0),    # the same at d_k = 128
    (1, 1, 161, 32, 128, 1, 1, 32, "bf16", "scalar", -3.0),
    # gating chunks of 128 and 256 tokens on the bf16 path: composed from 2 or 4
    # 64-token operators (the HLA note's length is 256), ragged tails
    (1, 2, 600, 128, 128, 2, 1, 256, "bf16", "channel", -2.0),
    (1, 1, 300, 64, 64, 1, 1, 256, "bf16", "scalar", -3.0),
    (2, 1, 330, 64, 128, 2, 1, 128, "bf16", "channel", -1.0),
    (1, 1, 200, 128, 64, 0, 1, 128, "bf16", "channel", -2.0),
    (1, 1, 100, 64, 64, 2, 1, 256, "bf16", "channel", 0.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}T{}dk{}dv{}r{}-{}C{}{}{}mu{}".format(*c))
def test_hla_parity(case):
    Bb, H, T, dk, dv, r_ab, r_kv, C, dtype, decay, mu = case
    print(f"hla case {case}", flush=True)
    raw = workloads.generic_raw(Bb, H, T, dk, dv, r_ab, r_kv, dtype, decay, seed=T + dk)
    gates = workloads.hla_gates(Bb, H, T, C, mu=mu, seed=T)
    out = _gpu(raw, gates, dtype, C, 0.1)
    ref = hla_oracle.hla(raw["q"], raw["K"], raw["V"], raw["log_decay"], raw["A"], raw["B"], gates, C, 0.1)
    e = rel_err(out, ref)
    print(f"out {e:.2e}", flush=True)
    assert e <= TOL[dtype]


def test_hla_all_gates_one_is_base_forward():
    Bb, H, T, dk, dv, C = 1, 2, 200, 64, 64, 32
    raw = workloads.generic_raw(Bb, H, T, dk, dv, 2, 1, "fp32", "channel", seed=1)
    gates = np.ones((Bb, H, T, -(-T // C)), dtype=np.float32)
    out = _gpu(raw, gates, "fp32", C, 0.1)
    ref, _ = oracle.generic(raw["q"], raw["K"], raw["V"], raw["log_decay"], raw["A"], raw["B"])
    assert rel_err(out, ref) <= TOL["fp32"]


def test_hla_gates_below_threshold_are_chunk_local():
    Bb, H, T, dk, dv, C = 1, 1, 150, 32, 32, 64
    raw = workloads.generic_raw(Bb, H, T, dk, dv, 1, 1, "fp32", "channel", seed=2)
    gates = np.full((Bb, H, T, -(-T // C)), 0.09, dtype=np.float32)
    out = _gpu(raw, gates, "fp32", C, 0.1)
    zero = hla_oracle.hla(raw["q"], raw["K"], raw["V"], raw["log_decay"], raw["A"], raw["B"],
                          np.zeros_like(gates), C, 0.0)
    assert rel_err(out, zero) <= TOL["fp32"]


def test_hla_256_token_chunks_need_the_bf16_path():
    raw = workloads.generic_raw(1, 1, 300, 64, 64, 1, 1, "fp32", "channel", seed=0)
    gates = workloads.hla_gates(1, 1, 300, 256, seed=0)
    with pytest.raises(lattn.LattnError) as ei:
        _gpu(raw, gates, "fp32", 256, 0.1)
    assert ei.value.status == -2


def test_hla_rejects_wide_heads():
    raw = workloads.generic_raw(1, 1, 32, 256, 64, 1, 1, "fp32", "channel", seed=0)
    gates = workloads.hla_gates(1, 1, 32, 16, seed=0)
    with pytest.raises(lattn.LattnError):
        _gpu(raw, gates, "fp32", 16, 0.1)


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_hla_bench_workload_two_heads():
    """The bench's HLA workload (Gated DeltaNet, B1 H16 T4096 d128, 256-token gating
    chunks, bf16) in the launch configuration bench.py times.  On the first and
    last head: every query of four whole gating chunks (the first, the second, a
    middle and the last) and every 16th query elsewhere, against the oracle on
    its own decay operands (the fp64 Gated DeltaNet rewrite rounded to bf16)."""
    import bench
    w = bench.HLA_WORKLOAD
    Bb, H, T, dk, dv, C = w["B"], w["H"], w["T"], w["dk"], w["dv"], w["chunk"]
    raw = workloads.gdn_raw(Bb, H, T, dk, dv, "bf16", seed=0)
    gates = workloads.hla_gates(Bb, H, T, C, mu=w["mu"], seed=0)
    td = torch.bfloat16
    k, v = dev(raw["k"], td), dev(raw["v"], td)
    A, B, V = lattn.gdn_params(k, v, dev(raw["g"]), dev(raw["beta"]))
    out = lattn.hla_fwd(dev(raw["q"], td), k, V, dev(raw["g"]), A, B, dev(gates), chunk=C, theta=w["theta"])
    torch.cuda.synchronize()
    out = host(out)
    N = T // C
    qs = sorted(set(range(0, C)) | set(range(C, 2 * C)) | set(range((N // 2) * C, (N // 2 + 1) * C))
                | set(range((N - 1) * C, T)) | set(range(0, T, 16)))
    for h in (0, H - 1):
        sl = lambda x: x[:, h:h + 1]
        g, rA, rB, rK, rV = oracle.gdn_to_generic(sl(raw["k"]), sl(raw["v"]), sl(raw["g"]), sl(raw["beta"]))
        ref = hla_oracle.hla(sl(raw["q"]), sl(raw["k"])[..., None, :], store_like(rV, "bf16"), g,
                             store_like(rA, "bf16"), store_like(rB, "bf16"), sl(gates), C, w["theta"], queries=qs)
        e = rel_err(out[:, h:h + 1][:, :, qs], ref[:, :, qs])
        print(f"head {h}: {len(qs)} queries: out {e:.2e}", flush=True)
        assert e <= TOL["bf16"]


def test_hla_empty_and_repeatable():
    raw = workloads.generic_raw(1, 2, 0, 32, 32, 1, 1, "fp32", "channel", seed=0)
    gates = np.zeros((1, 2, 0, 0), np.float32)
    assert _gpu(raw, gates, "fp32", 32, 0.1).shape == (1, 2, 0, 32)
    raw = workloads.generic_raw(1, 2, 150, 64, 64, 2, 1, "bf16", "channel", seed=9)
    gates = workloads.hla_gates(1, 2, 150, 64, mu=-1.0, seed=9)
    a = _gpu(raw, gates, "bf16", 64, 0.1)
    b = _gpu(raw, gates, "bf16", 64, 0.1)
    assert np.array_equal(a, b)


def test_hla_nan_gate_propagates_like_the_oracle():
    """A NaN gate is not below the threshold, so it is applied (and poisons only
    its own query's row), as in the oracle; every other row stays finite and
    matches."""
    Bb, H, T, dk, dv, C = 1, 1, 150, 32, 32, 32
    raw = workloads.generic_raw(Bb, H, T, dk, dv, 1, 1, "fp32", "channel", seed=12)
    gates = workloads.hla_gates(Bb, H, T, C, mu=-1.0, seed=12)
    gates[0, 0, 100, 1] = np.nan       # query 100 (chunk 3), history chunk 1
    out = _gpu(raw, gates, "fp32", C, 0.1)
    ref = hla_oracle.hla(raw["q"], raw["K"], raw["V"], raw["log_decay"], raw["A"], raw["B"], gates, C, 0.1)
    assert np.array_equal(np.isnan(out), np.isnan(ref))
    assert np.isnan(out[0, 0, 100]).all()
    keep = ~np.isnan(ref)
    assert rel_err(out[keep], ref[keep]) <= TOL["fp32"]


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64)])
def test_hla_bf16_all_gates_one_over_many_gating_chunks(dk, dv):
    """Gates all 1 over eight 256-token gating chunks on the bf16 path: every query's
    history is the full exact prefix, so the output is the plain recurrence (the
    C oracle).  This stresses the composition's carried R over seven history
    chunks, each step a bf16 product with fp32 accumulation."""
    Bb, H, T, C = 1, 2, 2048, 256
    raw = workloads.generic_raw(Bb, H, T, dk, dv, 2, 1, "bf16", "channel", seed=13)
    gates = np.ones((Bb, H, T, T // C), dtype=np.float32)
    out = _gpu(raw, gates, "bf16", C, 0.1)
    ref, _ = oracle.generic(raw["q"], raw["K"], raw["V"], raw["log_decay"], raw["A"], raw["B"])
    e = rel_err(out, ref)
    print(f"all gates 1, d_k {dk}: out {e:.2e}", flush=True)
    assert e <= TOL["bf16"]
