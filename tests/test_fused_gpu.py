"""GPU parity of the fused family forwards (HDLA and Gated DeltaNet from their
raw parameters) against the structured fp64 oracles.

The reference is the Householder-form oracle (HDLA) or the Gated DeltaNet
oracle on the same stored q, k, v, decay and beta values; neither touches a
low-rank rewrite, so these tests also check that the kernels form the decay
operands correctly.  Gate as elsewhere: max|gpu - ref| / max|ref| <= 1e-4 for
fp32 storage, <= 2e-2 for bf16.
"""
import ctypes

import numpy as np
import pytest

import oracle
import workloads
from tests.helpers import TOL, dev, host, rel_err, torch_dtype

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

lattn = pytest.importorskip("structured_decay_sequence_amd")


def _kernels(family, Bb, H, T, dk, dv, dtype, chunk):
    dims = lattn.make_dims(Bb, H, T, dk, dv, 1 if dtype == "bf16" else 0, family == "gdn")
    r_ab = 2 if family == "hdla" else 1
    return lattn._lib.load().lattn_chunk_fwd_kernels(ctypes.byref(dims), r_ab, 1, chunk).decode()


FUSED_CASES = [
    # family, B, H, T, dk, dv, dtype, chunk, with initial state
    ("hdla", 1, 2, 200, 128, 128, "bf16", 64, True),
    ("hdla", 1, 3, 257, 64, 64, "bf16", 64, False),
    ("hdla", 2, 1, 129, 128, 192, "bf16", 64, True),
    ("hdla", 2, 64, 130, 128, 128, "bf16", 64, False),   # wide scan slices
    ("hdla", 1, 2, 200, 64, 64, "fp32", 64, True),       # general path
    ("hdla", 1, 2, 77, 32, 32, "bf16", 16, False),       # general path, bf16 storage
    ("gdn", 1, 2, 300, 128, 128, "bf16", 64, True),
    ("gdn", 2, 2, 130, 64, 64, "bf16", 64, False),
    ("gdn", 1, 2, 100, 128, 128, "fp32", 32, True),
    ("gdn", 1, 1, 1, 128, 128, "bf16", 64, False),       # a single token
    ("hdla", 1, 2, 4200, 64, 64, "bf16", 64, True),      # the scan split in two segments
    ("gdn", 1, 1, 4100, 64, 128, "bf16", 64, False),     # the same, d_v 128
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: "{}B{}H{}T{}dk{}dv{}{}C{}S0{}".format(*c))
def test_fused_parity(case):
    family, Bb, H, T, dk, dv, dtype, chunk, with_s0 = case
    print(f"fused case {case} kernels {_kernels(family, Bb, H, T, dk, dv, dtype, chunk)}", flush=True)
    td = torch_dtype(dtype)
    S0 = (np.random.default_rng(11).standard_normal((Bb, H, dk, dv)) * 0.1).astype(np.float32) if with_s0 else None
    if family == "hdla":
        raw = workloads.hdla_raw(Bb, H, T, dk, dv, dtype, 3.0, seed=5 + T)
        decay = raw["log_lambda"]
        out, S = lattn.hdla_chunk_fwd(dev(raw["q"], td), dev(raw["k"], td), dev(raw["v"], td), dev(decay),
                                      dev(raw["beta"]), chunk=chunk, initial_state=dev(S0))
        ref_out, ref_S = oracle.hdla(raw["q"], raw["k"], raw["v"], decay, raw["beta"], initial_state=S0)
    else:
        raw = workloads.gdn_raw(Bb, H, T, dk, dv, dtype, seed=5 + T)
        decay = raw["g"]
        out, S = lattn.gdn_chunk_fwd(dev(raw["q"], td), dev(raw["k"], td), dev(raw["v"], td), dev(decay),
                                     dev(raw["beta"]), chunk=chunk, initial_state=dev(S0))
        ref_out, ref_S = oracle.gdn(raw["q"], raw["k"], raw["v"], decay, raw["beta"], initial_state=S0)
    torch.cuda.synchronize()
    e_o, e_s = rel_err(host(out), ref_out), rel_err(host(S), ref_S)
    print(f"out {e_o:.2e} state {e_s:.2e}", flush=True)
    assert e_o <= TOL[dtype] and e_s <= TOL[dtype]


def test_fused_matches_materialized_path():
    """The fused HDLA forward and parameter kernel + generic forward agree to
    the bf16 rounding of the materialized A, B and beta v."""
    raw = workloads.hdla_raw(1, 4, 192, 128, 128, "bf16", 3.0, seed=21)
    td = torch.bfloat16
    q, k, v = dev(raw["q"], td), dev(raw["k"], td), dev(raw["v"], td)
    ll, beta = dev(raw["log_lambda"]), dev(raw["beta"])
    o1, s1 = lattn.hdla_chunk_fwd(q, k, v, ll, beta)
    A, B, V = lattn.hdla_params(k, v, ll, beta)
    o2, s2 = lattn.chunk_fwd(q, k, V, ll, A, B)
    torch.cuda.synchronize()
    assert rel_err(host(o1), host(o2)) <= TOL["bf16"]
    assert rel_err(host(s1), host(s2)) <= TOL["bf16"]


def test_fused_empty_sequence_copies_state():
    S0 = torch.randn(1, 2, 64, 64, device="cuda")
    z = torch.empty(1, 2, 0, 64, dtype=torch.bfloat16, device="cuda")
    out, S = lattn.hdla_chunk_fwd(z, z, z, torch.empty(1, 2, 0, 64, device="cuda"),
                                  torch.empty(1, 2, 0, device="cuda"), initial_state=S0)
    torch.cuda.synchronize()
    assert out.shape == (1, 2, 0, 64)
    assert torch.equal(S, S0)


def test_fused_rejects_wrong_decay_mode():
    lib = lattn._lib.load()
    dims = lattn.make_dims(1, 1, 64, 64, 64, 1, True)   # scalar decay: not HDLA
    assert lib.lattn_hdla_chunk_fwd_workspace_size(ctypes.byref(dims), 64) == 0
    x = torch.zeros(64 * 64, dtype=torch.bfloat16, device="cuda")
    rc = lib.lattn_hdla_chunk_fwd(ctypes.byref(dims), x.data_ptr(), x.data_ptr(), x.data_ptr(), x.data_ptr(),
                                  x.data_ptr(), 64, x.data_ptr(), None, None, None, 0, None)
    assert rc == lattn._lib.LATTN_EINVAL
