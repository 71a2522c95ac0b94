"""GPU parity of the log-linear lift (lattn_loglinear_fwd) against the fp64
oracle, through the C ABI.

Gate as for the base path: max|gpu - ref| / max|ref| <= 1e-4 for fp32 storage
and <= 2e-2 for bf16 storage.  Inputs: the seeded generic recurrence inputs and
seeded per-level weights softplus(N(0, 1)).

Two routes are exercised: fp32 arithmetic on row-major fp32 chunk operators
(fp32 storage, and bf16 storage at d_k = 128), and, for bf16 storage at the
bf16 MFMA prepare's shapes with d_k = 64, the scan on that prepare's bf16
operators with bf16 MFMAs (cases marked "bf16 route").
"""
import numpy as np
import pytest

import oracle
from oracle import loglinear as ll_oracle
import workloads
from tests.helpers import TOL, dev, host, rel_err, store_like, torch_dtype

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

lattn = pytest.importorskip("structured_decay_sequence_amd")


def _gpu(raw, lam, dtype, chunk):
    td = torch_dtype(dtype)
    out = lattn.loglinear_fwd(dev(raw["q"], td), dev(raw["K"], td), dev(raw["V"], td), dev(raw["log_decay"]),
                              dev(raw["A"], td), dev(raw["B"], td), dev(lam), chunk=chunk)
    torch.cuda.synchronize()
    return host(out)


def _ref(raw, lam):
    T = raw["q"].shape[-2]
    # the per-query definition is O(T^2) transports; longer cases use the recurrent form
    f = ll_oracle.loglinear if T <= 400 else ll_oracle.loglinear_recurrent
    return f(raw["q"], raw["K"], raw["V"], raw["log_decay"], raw["A"], raw["B"], lam)


CASES = [
    # B, H, T, dk, dv, r_ab, r_kv, C, dtype, decay
    (1, 2, 200, 32, 32, 2, 1, 16, "fp32", "channel"),
    (1, 1, 300, 64, 64, 1, 1, 32, "fp32", "scalar"),
    (1, 1, 257, 64, 48, 2, 2, 64, "fp32", "channel"),
    (2, 1, 100, 16, 32, 0, 1, 16, "fp32", "channel"),
    (1, 1, 40, 32, 32, 1, 1, 64, "fp32", "channel"),
    (1, 1, 1, 16, 16, 1, 1, 16, "fp32", "channel"),
    (1, 2, 130, 64, 64, 2, 1, 32, "bf16", "channel"),
    (1, 1, 200, 128, 128, 2, 1, 64, "bf16", "channel"),   # operators from the bf16 MFMA prepare
    (1, 2, 150, 64, 64, 1, 1, 64, "bf16", "scalar"),      # bf16 route
    (1, 1, 160, 64, 128, 1, 1, 128, "bf16", "scalar"),
    # bf16 route: rank 0, 6 (batch, head) slices (not a multiple of 8), ragged tail
    (2, 3, 1000, 64, 64, 0, 1, 64, "bf16", "channel"),
    # bf16 route: rank 2, d_v 128 (eight column slices), 38 chunks (6 inter-chunk levels)
    (1, 2, 2373, 64, 128, 2, 1, 64, "bf16", "channel"),
    # bf16 route: one token, one exact chunk, one chunk and one token
    (1, 1, 1, 64, 64, 1, 1, 64, "bf16", "scalar"),
    (1, 1, 64, 64, 64, 1, 1, 64, "bf16", "channel"),
    (1, 1, 65, 64, 64, 2, 1, 64, "bf16", "channel"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}T{}dk{}dv{}r{}-{}C{}{}{}".format(*c))
def test_loglinear_parity(case):
    Bb, H, T, dk, dv, r_ab, r_kv, C, dtype, decay = case
    print(f"log-linear case {case}", flush=True)
    raw = workloads.generic_raw(Bb, H, T, dk, dv, r_ab, r_kv, dtype, decay, seed=T + dk)
    lam = workloads.loglinear_lambdas(Bb, H, T, seed=T)
    out = _gpu(raw, lam, dtype, C)
    e = rel_err(out, _ref(raw, lam))
    print(f"out {e:.2e}", flush=True)
    assert e <= TOL[dtype]


def test_loglinear_equal_weights_is_base_forward():
    Bb, H, T, dk, dv = 1, 2, 200, 64, 64
    raw = workloads.generic_raw(Bb, H, T, dk, dv, 2, 1, "fp32", "channel", seed=4)
    lam = np.ones((Bb, H, T, lattn.loglinear_levels(T)), dtype=np.float32)
    out = _gpu(raw, lam, "fp32", 16)
    ref, _ = oracle.generic(raw["q"], raw["K"], raw["V"], raw["log_decay"], raw["A"], raw["B"])
    assert rel_err(out, ref) <= TOL["fp32"]


def test_loglinear_chunk_size_invariance():
    Bb, H, T, dk, dv = 1, 1, 230, 32, 32
    raw = workloads.generic_raw(Bb, H, T, dk, dv, 1, 1, "fp32", "channel", seed=6)
    lam = workloads.loglinear_lambdas(Bb, H, T, seed=6)
    outs = [_gpu(raw, lam, "fp32", C) for C in (16, 32, 64, 128)]
    for o in outs[1:]:
        assert rel_err(o, outs[0]) <= TOL["fp32"]


def test_loglinear_long_sequence_one_and_two_state_copies():
    """d_k 128 over 8300 tokens.  At C 16 (519 chunks, 10 inter-chunk levels)
    two copies of the level states would need 169 KB of LDS, so the scan keeps
    one and orders each level's reads before its writes; at C 64 (130 chunks,
    8 levels, 135 KB) it keeps two and alternates them by chunk parity.  The
    outputs must agree."""
    Bb, H, T, dk, dv = 1, 1, 8300, 128, 16
    raw = workloads.generic_raw(Bb, H, T, dk, dv, 1, 1, "fp32", "channel", seed=8)
    lam = workloads.loglinear_lambdas(Bb, H, T, seed=8)
    a, b = _gpu(raw, lam, "fp32", 16), _gpu(raw, lam, "fp32", 64)
    e = rel_err(b, a)
    print(f"C 16 vs C 64 over {T} tokens: {e:.2e}", flush=True)
    assert e <= TOL["fp32"]


def test_loglinear_levels_and_rejects():
    assert lattn.loglinear_levels(4096) == ll_oracle.num_levels(4096) == 13
    assert lattn.loglinear_levels(1) == 1 and lattn.loglinear_levels(5) == 4
    raw = workloads.generic_raw(1, 1, 32, 256, 64, 1, 1, "fp32", "channel", seed=0)
    lam = workloads.loglinear_lambdas(1, 1, 32, seed=0)
    with pytest.raises(lattn.LattnError):
        _gpu(raw, lam, "fp32", 16)


def test_loglinear_every_level_small_head():
    """d_k 32, C 16 over 2100 tokens (132 chunks): inter-chunk levels m = 0 .. 7
    with distinct per-level weights, the whole sequence against the recurrent
    oracle (bucket states per level)."""
    Bb, H, T, dk, dv, C = 1, 2, 2100, 32, 32, 16
    raw = workloads.generic_raw(Bb, H, T, dk, dv, 2, 1, "fp32", "channel", seed=10)
    lam = workloads.loglinear_lambdas(Bb, H, T, seed=10)
    out = _gpu(raw, lam, "fp32", C)
    ref = ll_oracle.loglinear_recurrent(raw["q"], raw["K"], raw["V"], raw["log_decay"], raw["A"], raw["B"], lam)
    e = rel_err(out, ref)
    print(f"{T} tokens, {-(-T // C)} chunks, {lattn.loglinear_levels(T)} levels: out {e:.2e}", flush=True)
    assert e <= TOL["fp32"]


def test_loglinear_single_state_copy_against_oracle():
    """d_k 128, C 16 over 8300 tokens (519 chunks): two copies of the level states
    would not fit in LDS, so the scan runs its single-copy mode; checked against
    the recurrent oracle on the whole sequence."""
    Bb, H, T, dk, dv, C = 1, 1, 8300, 128, 16, 16
    raw = workloads.generic_raw(Bb, H, T, dk, dv, 1, 1, "fp32", "channel", seed=11)
    lam = workloads.loglinear_lambdas(Bb, H, T, seed=11)
    out = _gpu(raw, lam, "fp32", C)
    ref = ll_oracle.loglinear_recurrent(raw["q"], raw["K"], raw["V"], raw["log_decay"], raw["A"], raw["B"], lam)
    e = rel_err(out, ref)
    print(f"single-copy mode, {T} tokens: out {e:.2e}", flush=True)
    assert e <= TOL["fp32"]


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_loglinear_bench_workload_full_heads():
    """The bench's log-linear workload (Gated DeltaNet B1 H48 T32768 d64, C 64, bf16:
    512 chunks, inter-chunk levels m = 0 .. 8) in the launch configuration bench.py
    times; two whole heads against the recurrent oracle on the oracle's own
    decay operands (its fp64 Gated DeltaNet rewrite rounded to bf16)."""
    import bench
    w = bench.LOGLINEAR_WORKLOAD
    Bb, H, T, dk, dv, C = w["B"], w["H"], w["T"], w["dk"], w["dv"], w["chunk"]
    raw = workloads.gdn_raw(Bb, H, T, dk, dv, "bf16", seed=0)
    lam = workloads.loglinear_lambdas(Bb, H, T, seed=0)
    td = torch.bfloat16
    k, v = dev(raw["k"], td), dev(raw["v"], td)
    A, B, V = lattn.gdn_params(k, v, dev(raw["g"]), dev(raw["beta"]))
    out = host(lattn.loglinear_fwd(dev(raw["q"], td), k, V, dev(raw["g"]), A, B, dev(lam), chunk=C))
    torch.cuda.synchronize()
    for h in (0, H - 1):
        sl = lambda x: x[:, h:h + 1]
        g, rA, rB, rK, rV = oracle.gdn_to_generic(sl(raw["k"]), sl(raw["v"]), sl(raw["g"]), sl(raw["beta"]))
        ref = ll_oracle.loglinear_recurrent(sl(raw["q"]), sl(raw["k"])[..., None, :], store_like(rV, "bf16"), g,
                                            store_like(rA, "bf16"), store_like(rB, "bf16"), sl(lam))
        e = rel_err(out[:, h:h + 1], ref)
        print(f"head {h}, all {T} tokens ({lattn.loglinear_levels(T)} levels): out {e:.2e}", flush=True)
        assert e <= TOL["bf16"]


def test_loglinear_empty_and_repeatable():
    raw = workloads.generic_raw(1, 2, 0, 32, 32, 1, 1, "fp32", "channel", seed=0)
    lam = np.zeros((1, 2, 0, 0), np.float32)
    assert _gpu(raw, lam, "fp32", 16).shape == (1, 2, 0, 32)
    raw = workloads.generic_raw(1, 2, 150, 64, 64, 2, 1, "bf16", "channel", seed=9)
    lam = workloads.loglinear_lambdas(1, 2, 150, seed=9)
    a = _gpu(raw, lam, "bf16", 64)
    b = _gpu(raw, lam, "bf16", 64)
    assert np.array_equal(a, b)


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_loglinear_sixteen_levels_sparse_writes():
    """bf16 route at its largest level count: 2^15 + 1 chunks of 64 tokens plus
    36 (2097252 tokens, 16 inter-chunk levels, 23 in all).  Keys and values are
    zero before H - 256 (H = 2^21), so:
      * outputs before H - 256 are exactly zero;
      * on [H - 256, H) (a 256-aligned block, so levels are those of the block
        taken on its own) the output is the recurrent oracle's on that block;
      * on [H, T) it is the recurrent oracle's on [H, T) plus, at the top level
        (index 22, the bucket [0, H) of every such query), the state of the
        writes on [H - 256, H) carried by the recurrence's transport: the
        oracle's token recurrence over [H - 256, H), then over [H, T) from that
        state with no writes, read out and weighted by lambda[t, 22]."""
    T, H0, W = (1 << 21) + 100, 1 << 21, 256
    dk = dv = 64
    raw = workloads.generic_raw(1, 1, T, dk, dv, 1, 1, "bf16", "scalar", seed=12)
    raw["K"][:, :, :H0 - W] = 0
    raw["V"][:, :, :H0 - W] = 0
    lam = workloads.loglinear_lambdas(1, 1, T, seed=12)
    assert lam.shape[-1] == 23 and lattn.loglinear_levels(T) == 23
    out = _gpu(raw, lam, "bf16", 64)
    assert not np.any(out[:, :, :H0 - W]), "outputs before the first write must be zero"
    sl = lambda d, a, b: {k: (None if v is None else v[:, :, a:b]) for k, v in d.items()}
    blk = sl(raw, H0 - W, H0)
    ref1 = ll_oracle.loglinear_recurrent(blk["q"], blk["K"], blk["V"], blk["log_decay"], blk["A"], blk["B"],
                                         lam[:, :, H0 - W:H0, :9])
    e1 = rel_err(out[:, :, H0 - W:H0], ref1)
    tail = sl(raw, H0, T)
    ref2 = ll_oracle.loglinear_recurrent(tail["q"], tail["K"], tail["V"], tail["log_decay"], tail["A"], tail["B"],
                                         lam[:, :, H0:T, :8])
    _, S = oracle.generic(blk["q"], blk["K"], blk["V"], blk["log_decay"], blk["A"], blk["B"])
    carried, _ = oracle.generic(tail["q"], np.zeros_like(tail["K"]), tail["V"], tail["log_decay"], tail["A"],
                                tail["B"], initial_state=S)
    ref2 = ref2 + lam[:, :, H0:T, 22:23] * carried
    e2 = rel_err(out[:, :, H0:T], ref2)
    print(f"{T} tokens, 16 inter-chunk levels: block before H {e1:.2e}, after H {e2:.2e}", flush=True)
    assert e1 <= TOL["bf16"] and e2 <= TOL["bf16"]
