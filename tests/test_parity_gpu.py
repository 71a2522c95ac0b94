"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Gate (per tensor): max|gpu - ref| / max|ref| <= 1e-4 for fp32 inputs and
<= 2e-2 for bf16 inputs with fp32 accumulation.  The reference is the generic
oracle run on the same stored input values; for HDLA and Gated DeltaNet the
oracle builds its own decay operands (its fp64 low-rank rewrite, rounded to the
stored dtype) and the structured (Householder / GDN) oracles run beside it.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.helpers import TOL, dev, host, rel_err, store_like, torch_dtype

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

lattn = pytest.importorskip("structured_decay_sequence_amd")


def _gpu_generic(raw, dtype, chunk, S0=None):
    td = torch_dtype(dtype)
    out, S = lattn.chunk_fwd(dev(raw["q"], td), dev(raw["K"], td), dev(raw["V"], td), dev(raw["log_decay"]),
                             dev(raw["A"], td), dev(raw["B"], td), chunk=chunk,
                             initial_state=dev(S0))
    torch.cuda.synchronize()
    return host(out), host(S)


GENERIC_CASES = [
    # B, H, T, dk, dv, r_ab, r_kv, C, dtype, decay
    (1, 2, 200, 64, 64, 2, 1, 64, "fp32", "channel"),
    (2, 1, 300, 32, 48, 1, 1, 32, "fp32", "scalar"),
    (1, 2, 130, 128, 128, 2, 1, 64, "bf16", "channel"),
    (1, 1, 257, 64, 64, 4, 2, 64, "fp32", "channel"),
    (1, 2, 100, 16, 16, 0, 1, 16, "fp32", "channel"),
    (1, 1, 90, 32, 32, 0, 2, 128, "bf16", "scalar"),
    (1, 1, 64, 256, 256, 1, 1, 32, "fp32", "channel"),
    (1, 1, 33, 128, 64, 8, 1, 16, "fp32", "channel"),
    (1, 1, 70, 64, 64, 2, 4, 64, "fp32", "channel"),
    (1, 1, 40, 32, 32, 4, 1, 128, "fp32", "channel"),
    (2, 2, 192, 64, 128, 2, 1, 64, "bf16", "channel"),
]


@pytest.mark.parametrize("case", GENERIC_CASES, ids=lambda c: "B{}H{}T{}dk{}dv{}r{}-{}C{}{}{}".format(*c))
def test_generic_parity(case):
    Bb, H, T, dk, dv, r_ab, r_kv, C, dtype, decay = case
    print(f"case {case}", flush=True)
    raw = workloads.generic_raw(Bb, H, T, dk, dv, r_ab, r_kv, dtype, decay, seed=T + dk)
    S0 = (np.random.default_rng(5).standard_normal((Bb, H, dk, dv)) * 0.1).astype(np.float32)
    out, S = _gpu_generic(raw, dtype, C, S0)
    ref_out, ref_S = oracle.generic(raw["q"], raw["K"], raw["V"], raw["log_decay"], raw["A"], raw["B"],
                                    initial_state=S0)
    assert rel_err(out, ref_out) <= TOL[dtype]
    assert rel_err(S, ref_S) <= TOL[dtype]


# Shapes the bf16 MFMA path takes (C = 64, r_kv = 1, r_ab in {1, 2}, d_k in {64, 128},
# d_v a multiple of 64): ragged tails, a sequence shorter than one chunk, both decay
# modes, batch*heads not a multiple of 8, and wide d_v.
FAST_CASES = [
    # B, H, T, dk, dv, r_ab, decay
    (1, 3, 200, 128, 128, 2, "channel"),
    (1, 2, 64, 128, 128, 2, "channel"),
    (2, 1, 37, 128, 64, 2, "channel"),
    (1, 2, 300, 128, 128, 1, "scalar"),
    (1, 2, 150, 128, 128, 1, "channel"),
    (1, 5, 257, 64, 64, 2, "channel"),
    (1, 2, 100, 64, 64, 1, "scalar"),
    (3, 3, 130, 64, 128, 2, "channel"),
    (1, 2, 129, 128, 256, 2, "channel"),
    (1, 9, 128, 128, 192, 1, "channel"),
    # diagonal decay only (GLA, r_ab = 0)
    (1, 2, 200, 128, 128, 0, "channel"),
    (2, 2, 130, 64, 64, 0, "scalar"),
    (1, 3, 64, 128, 192, 0, "channel"),
    # enough (batch, head) rows for the wide d_v slices of the scan (128 rows x 2 slices)
    (2, 64, 130, 128, 128, 2, "channel"),
    (4, 32, 192, 128, 128, 1, "scalar"),
]


# d_k = 64 with few (batch, head) rows: the scan splits the sequence in two
# (from 64 chunks) or three (from 96 chunks) segments, each later one
# corrected with the state entering it (odd chunk counts, ragged tails, exact
# multiples, d_v 64 and 128, ranks 0-2, both decay modes, with and without
# the final state).
SPLIT_CASES = [
    # B, H, T, dk, dv, r_ab, decay, final state returned
    (1, 2, 4133, 64, 64, 2, "channel", True),
    (1, 1, 4096, 64, 128, 0, "channel", True),
    (2, 1, 5000, 64, 64, 1, "scalar", True),
    (1, 3, 8192, 64, 64, 2, "channel", False),
    (1, 2, 6500, 64, 64, 2, "channel", True),
    (1, 1, 7000, 64, 128, 1, "scalar", True),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: "B{}H{}T{}dk{}dv{}r{}{}fin{}".format(*c))
def test_split_scan_parity(case):
    Bb, H, T, dk, dv, r_ab, decay, fin = case
    print(f"split scan case {case}", flush=True)
    raw = workloads.generic_raw(Bb, H, T, dk, dv, r_ab, 1, "bf16", decay, seed=T + dv)
    S0 = (np.random.default_rng(8).standard_normal((Bb, H, dk, dv)) * 0.1).astype(np.float32)
    td = torch.bfloat16
    out, S = lattn.chunk_fwd(dev(raw["q"], td), dev(raw["K"], td), dev(raw["V"], td), dev(raw["log_decay"]),
                             dev(raw["A"], td), dev(raw["B"], td), chunk=64, initial_state=dev(S0),
                             return_final_state=fin)
    torch.cuda.synchronize()
    ref_out, ref_S = oracle.generic(raw["q"], raw["K"], raw["V"], raw["log_decay"], raw["A"], raw["B"],
                                    initial_state=S0)
    e_o = rel_err(host(out), ref_out)
    # the last third alone (corrected rows in every split)
    tail = T - T // 3
    e_h = rel_err(host(out)[:, :, tail:], ref_out[:, :, tail:])
    print(f"out {e_o:.2e} last third {e_h:.2e}", flush=True)
    assert e_o <= TOL["bf16"] and e_h <= TOL["bf16"]
    if fin:
        e_s = rel_err(host(S), ref_S)
        print(f"state {e_s:.2e}", flush=True)
        assert e_s <= TOL["bf16"]
    else:
        assert S is None


@pytest.mark.parametrize("case", FAST_CASES, ids=lambda c: "B{}H{}T{}dk{}dv{}r{}{}".format(*c))
def test_mfma_path_parity(case):
    Bb, H, T, dk, dv, r_ab, decay = case
    print(f"mfma case {case}", flush=True)
    raw = workloads.generic_raw(Bb, H, T, dk, dv, r_ab, 1, "bf16", decay, seed=3 * T + dk)
    dims = lattn.make_dims(Bb, H, T, dk, dv, 1, decay == "scalar")
    import ctypes
    assert lattn._lib.load().lattn_chunk_fwd_kernels(ctypes.byref(dims), r_ab, 1, 64) == b"mfma_bf16"
    S0 = (np.random.default_rng(7).standard_normal((Bb, H, dk, dv)) * 0.1).astype(np.float32)
    out, S = _gpu_generic(raw, "bf16", 64, S0)
    ref_out, ref_S = oracle.generic(raw["q"], raw["K"], raw["V"], raw["log_decay"], raw["A"], raw["B"],
                                    initial_state=S0)
    e_o, e_s = rel_err(out, ref_out), rel_err(S, ref_S)
    print(f"out {e_o:.2e} state {e_s:.2e}", flush=True)
    assert e_o <= TOL["bf16"] and e_s <= TOL["bf16"]


def _hdla_ref_inputs(raw, dtype):
    ll, A, B, K, V = oracle.hdla_to_generic(raw["k"], raw["v"], raw["log_lambda"], raw["beta"])
    return dict(q=raw["q"], log_decay=raw["log_lambda"], A=store_like(A, dtype), B=store_like(B, dtype),
                K=raw["k"][..., None, :], V=store_like(V, dtype))


def _gdn_ref_inputs(raw, dtype):
    g, A, B, K, V = oracle.gdn_to_generic(raw["k"], raw["v"], raw["g"], raw["beta"])
    return dict(q=raw["q"], log_decay=raw["g"], A=store_like(A, dtype), B=store_like(B, dtype),
                K=raw["k"][..., None, :], V=store_like(V, dtype))


def _gpu_hdla(raw, dtype, chunk, S0=None):
    td = torch_dtype(dtype)
    k, v = dev(raw["k"], td), dev(raw["v"], td)
    ll, beta = dev(raw["log_lambda"]), dev(raw["beta"])
    A, B, V = lattn.hdla_params(k, v, ll, beta)
    out, S = lattn.chunk_fwd(dev(raw["q"], td), k, V, ll, A, B, chunk=chunk, initial_state=dev(S0))
    torch.cuda.synchronize()
    return host(out), host(S)


def _gpu_gdn(raw, dtype, chunk, S0=None):
    td = torch_dtype(dtype)
    k, v = dev(raw["k"], td), dev(raw["v"], td)
    g, beta = dev(raw["g"]), dev(raw["beta"])
    A, B, V = lattn.gdn_params(k, v, g, beta)
    out, S = lattn.chunk_fwd(dev(raw["q"], td), k, V, g, A, B, chunk=chunk, initial_state=dev(S0))
    torch.cuda.synchronize()
    return host(out), host(S)


@pytest.mark.parametrize("dtype,d,T,C", [("fp32", 64, 200, 64), ("bf16", 128, 200, 64), ("fp32", 32, 77, 16)])
def test_hdla_parity(dtype, d, T, C):
    raw = workloads.hdla_raw(1, 2, T, d, d, dtype, 3.0, seed=1)
    out, S = _gpu_hdla(raw, dtype, C)
    r = _hdla_ref_inputs(raw, dtype)
    ref_out, ref_S = oracle.generic(r["q"], r["K"], r["V"], r["log_decay"], r["A"], r["B"])
    assert rel_err(out, ref_out) <= TOL[dtype]
    assert rel_err(S, ref_S) <= TOL[dtype]
    h_out, h_S = oracle.hdla(raw["q"], raw["k"], raw["v"], raw["log_lambda"], raw["beta"])
    assert rel_err(out, h_out) <= TOL[dtype]
    assert rel_err(S, h_S) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_gdn_parity(dtype):
    raw = workloads.gdn_raw(1, 2, 300, 128, 128, dtype, seed=2)
    out, S = _gpu_gdn(raw, dtype, 64)
    r = _gdn_ref_inputs(raw, dtype)
    ref_out, ref_S = oracle.generic(r["q"], r["K"], r["V"], r["log_decay"], r["A"], r["B"])
    assert rel_err(out, ref_out) <= TOL[dtype]
    assert rel_err(S, ref_S) <= TOL[dtype]
    g_out, g_S = oracle.gdn(raw["q"], raw["k"], raw["v"], raw["g"], raw["beta"])
    assert rel_err(out, g_out) <= TOL[dtype]
    assert rel_err(S, g_S) <= TOL[dtype]


def test_chunk_size_invariance():
    raw = workloads.hdla_raw(1, 2, 256, 32, 32, "fp32", 3.0, seed=3)
    ref_out, ref_S = oracle.hdla(raw["q"], raw["k"], raw["v"], raw["log_lambda"], raw["beta"])
    outs = []
    for C in (16, 32, 64, 128):
        out, S = _gpu_hdla(raw, "fp32", C)
        assert rel_err(out, ref_out) <= 1e-4, C
        assert rel_err(S, ref_S) <= 1e-4, C
        outs.append(out)
    for o in outs[1:]:
        assert rel_err(o, outs[0]) <= 1e-4


def test_state_passing_split_equals_one_call():
    raw = workloads.generic_raw(1, 2, 300, 64, 64, 2, 1, "fp32", "channel", seed=4)
    full_out, full_S = _gpu_generic(raw, "fp32", 64)
    t1 = 100
    first = {k: (None if v is None else v[:, :, :t1]) for k, v in raw.items()}
    second = {k: (None if v is None else v[:, :, t1:]) for k, v in raw.items()}
    o1, S1 = _gpu_generic(first, "fp32", 64)
    o2, S2 = _gpu_generic(second, "fp32", 64, S0=S1)
    assert rel_err(np.concatenate([o1, o2], axis=2), full_out) <= 1e-5
    assert rel_err(S2, full_S) <= 1e-5


def test_steps_equal_chunk_forward():
    T = 40
    raw = workloads.hdla_raw(1, 2, T, 64, 64, "fp32", 3.0, seed=5)
    out_c, S_c = _gpu_hdla(raw, "fp32", 16)
    k, v = dev(raw["k"]), dev(raw["v"])
    ll, beta = dev(raw["log_lambda"]), dev(raw["beta"])
    A, B, V = lattn.hdla_params(k, v, ll, beta)
    q = dev(raw["q"])
    state = torch.zeros((1, 2, 64, 64), dtype=torch.float32, device="cuda:0")
    outs = []
    for t in range(T):
        sl = lambda x: x[:, :, t].contiguous()
        outs.append(lattn.step(sl(q), sl(k), sl(V), sl(ll), sl(A), sl(B), state))
    out_s = host(torch.stack(outs, dim=2))
    assert rel_err(out_s, out_c) <= 1e-5
    assert rel_err(host(state), S_c) <= 1e-5
    ref_out, ref_S = oracle.hdla(raw["q"], raw["k"], raw["v"], raw["log_lambda"], raw["beta"])
    assert rel_err(out_s, ref_out) <= 1e-4


def test_step_bf16_and_generic_ranks():
    raw = workloads.generic_raw(2, 2, 1, 128, 64, 3, 2, "bf16", "channel", seed=6)
    S0 = (np.random.default_rng(6).standard_normal((2, 2, 128, 64)) * 0.1).astype(np.float32)
    td = torch.bfloat16
    state = dev(S0)
    sl = lambda x: None if x is None else dev(x[:, :, 0], td)
    out = lattn.step(sl(raw["q"]), sl(raw["K"]), sl(raw["V"]), dev(raw["log_decay"][:, :, 0]), sl(raw["A"]),
                     sl(raw["B"]), state)
    torch.cuda.synchronize()
    ref_out, ref_S = oracle.generic(raw["q"], raw["K"], raw["V"], raw["log_decay"], raw["A"], raw["B"],
                                    initial_state=S0)
    assert rel_err(host(out), ref_out[:, :, 0]) <= 2e-2
    assert rel_err(host(state), ref_S) <= 1e-4  # state stays fp32


def test_determinism_bitwise():
    raw = workloads.hdla_raw(1, 2, 200, 128, 128, "bf16", 3.0, seed=7)
    o1, s1 = _gpu_hdla(raw, "bf16", 64)
    o2, s2 = _gpu_hdla(raw, "bf16", 64)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


def test_split_scan_determinism_bitwise():
    """The scan split in three segments (its correction and chained entering
    states included) gives bitwise equal results on a second call."""
    raw = workloads.generic_raw(1, 2, 6500, 64, 64, 2, 1, "bf16", "channel", seed=11)
    S0 = (np.random.default_rng(12).standard_normal((1, 2, 64, 64)) * 0.1).astype(np.float32)
    o1, s1 = _gpu_generic(raw, "bf16", 64, S0)
    o2, s2 = _gpu_generic(raw, "bf16", 64, S0)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


@pytest.mark.parametrize("dtype,r_ab,r_kv,T", [("fp32", 2, 1, 150), ("fp32", 3, 2, 70), ("bf16", 1, 1, 130)])
def test_chunk_summaries(dtype, r_ab, r_kv, T):
    raw = workloads.generic_raw(1, 2, T, 64, 32, r_ab, r_kv, dtype, "channel", seed=8)
    td = torch_dtype(dtype)
    sA, sB = lattn.chunk_summaries(dev(raw["K"], td), dev(raw["V"], td), dev(raw["log_decay"]),
                                   dev(raw["A"], td), dev(raw["B"], td), chunk=32)
    torch.cuda.synchronize()
    rA, rB = oracle.chunk_summaries(raw["K"], raw["V"], raw["log_decay"], raw["A"], raw["B"], 32)
    assert rel_err(host(sA), rA) <= TOL[dtype]
    assert rel_err(host(sB), rB) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_decay_param_kernels(dtype):
    td = torch_dtype(dtype)
    raw = workloads.hdla_raw(1, 2, 50, 64, 32, dtype, 3.0, seed=9)
    A, B, V = lattn.hdla_params(dev(raw["k"], td), dev(raw["v"], td), dev(raw["log_lambda"]), dev(raw["beta"]))
    ll, rA, rB, rK, rV = oracle.hdla_to_generic(raw["k"], raw["v"], raw["log_lambda"], raw["beta"])
    # fp32: computed in fp32 vs fp64; bf16: the stored values may also differ by one
    # rounding step.  The absolute floor covers the cancellation in u - b c k.
    rel = 1e-6 if dtype == "fp32" else 2.0 ** -8

    def close(got, ref):
        g = host(got)
        bound = rel * np.abs(ref) + 1e-6 * np.abs(ref).max()
        worst = float(np.max(np.abs(g - ref) - bound))
        assert worst <= 0, f"{dtype}: exceeds bound by {worst:.3e}"

    for got, ref in [(A, rA), (B, rB), (V, rV)]:
        close(got, ref)
    graw = workloads.gdn_raw(1, 2, 50, 64, 32, dtype, seed=9)
    A, B, V = lattn.gdn_params(dev(graw["k"], td), dev(graw["v"], td), dev(graw["g"]), dev(graw["beta"]))
    g_, rA, rB, rK, rV = oracle.gdn_to_generic(graw["k"], graw["v"], graw["g"], graw["beta"])
    for got, ref in [(A, rA), (B, rB), (V, rV)]:
        close(got, ref)


def test_decay_range_and_guard():
    raw = workloads.hdla_raw(1, 2, 150, 32, 32, "fp32", 3.0, seed=10)
    got = host(lattn.decay_range(dev(raw["log_lambda"]), 64))
    ld = raw["log_lambda"].astype(np.float64)
    ref = np.zeros((1, 2, 3))
    for j in range(3):
        G = np.cumsum(ld[:, :, j * 64:(j + 1) * 64], axis=2)
        ref[:, :, j] = np.maximum(0, (-G).max(axis=(2, 3)))
    np.testing.assert_allclose(got, ref, rtol=1e-5)
    lattn.check_decay_range(dev(raw["log_lambda"]), 64)  # within range
    bad = np.full((1, 1, 64, 16), -2.0, dtype=np.float32)  # -G reaches 128 inside one chunk
    with pytest.raises(lattn.LattnError) as ei:
        lattn.check_decay_range(dev(bad), 64)
    assert ei.value.status == -5


def test_empty_sequence_copies_initial_state():
    S0 = np.random.default_rng(11).standard_normal((1, 2, 32, 32)).astype(np.float32)
    z = np.zeros((1, 2, 0, 32), np.float32)
    out, S = lattn.chunk_fwd(dev(z), dev(z), dev(z), dev(z), None, None, chunk=64, initial_state=dev(S0))
    torch.cuda.synchronize()
    assert out.shape == (1, 2, 0, 32)
    assert np.array_equal(host(S), S0)


def test_invalid_call_raises_before_launch():
    q = torch.zeros((1, 1, 8, 24), device="cuda:0")
    with pytest.raises(lattn.LattnError) as ei:
        lattn.chunk_fwd(q, q, q, q, None, None, chunk=64)
    assert ei.value.status == -1


STEP_CASES = [
    # B, H, dk, dv, r_ab, r_kv, dtype, decay
    (2, 3, 128, 128, 2, 1, "bf16", "channel"),
    (1, 2, 256, 256, 8, 4, "fp32", "channel"),
    (1, 2, 48, 48, 1, 1, "fp32", "scalar"),
    (2, 1, 64, 80, 0, 2, "bf16", "channel"),
    (1, 1, 208, 16, 3, 1, "fp32", "scalar"),
]


@pytest.mark.parametrize("case", STEP_CASES, ids=lambda c: "B{}H{}dk{}dv{}r{}-{}{}{}".format(*c))
def test_step_shapes(case):
    """lattn_step against the oracle over its row buckets (d_k up to 64, 128, 256),
    d_v slices with masked columns, every rank bound and both decay modes; a few
    tokens in a row from a non-zero state."""
    Bb, H, dk, dv, r_ab, r_kv, dtype, decay = case
    T = 3
    raw = workloads.generic_raw(Bb, H, T, dk, dv, r_ab, r_kv, dtype, decay, seed=dk + dv)
    S0 = (np.random.default_rng(12).standard_normal((Bb, H, dk, dv)) * 0.1).astype(np.float32)
    td = torch_dtype(dtype)
    state = dev(S0)
    outs = []
    for t in range(T):
        sl = lambda x: None if x is None else dev(np.ascontiguousarray(x[:, :, t]), td)
        ld = dev(np.ascontiguousarray(raw["log_decay"][:, :, t]))
        outs.append(host(lattn.step(sl(raw["q"]), sl(raw["K"]), sl(raw["V"]), ld, sl(raw["A"]), sl(raw["B"]), state)))
    torch.cuda.synchronize()
    ref_out, ref_S = oracle.generic(raw["q"], raw["K"], raw["V"], raw["log_decay"], raw["A"], raw["B"],
                                    initial_state=S0)
    e_o = rel_err(np.stack(outs, axis=2), ref_out)
    e_s = rel_err(host(state), ref_S)
    print(f"step {case}: out {e_o:.2e} state {e_s:.2e}", flush=True)
    assert e_o <= TOL[dtype]
    assert e_s <= 1e-4   # the state stays fp32 whatever the storage dtype
