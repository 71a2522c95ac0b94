"""lattn_chunk_fwd_noalloc (the forward for callers that cannot allocate),
through the C ABI, against lattn_chunk_fwd with a caller-owned workspace on
the same inputs: two calls in a row, the second on a smaller problem, on the
bf16 MFMA path and on the general fp32 path.  Gate as for the base path
(1e-4 fp32, 2e-2 bf16, max|got - ref| / max|ref|); the two share their
kernels, so the results are expected to be bitwise equal as well.  A problem
too large for the static scratch is rejected before any launch."""
import ctypes

import numpy as np
import pytest

import workloads
from tests.helpers import TOL, dev, host, rel_err, torch_dtype

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
lattn = pytest.importorskip("structured_decay_sequence_amd")
from structured_decay_sequence_amd import _lib  # noqa: E402

SCRATCH = 64 << 20


def _inputs(Bb, H, T, dk, dv, r_ab, dtype, seed):
    raw = workloads.generic_raw(Bb, H, T, dk, dv, r_ab, 1, dtype, "channel", seed=seed)
    td = torch_dtype(dtype)
    S0 = dev((np.random.default_rng(seed).standard_normal((Bb, H, dk, dv)) * 0.1).astype(np.float32))
    return (dev(raw["q"], td), dev(raw["K"], td), dev(raw["V"], td), dev(raw["log_decay"]),
            dev(raw["A"], td), dev(raw["B"], td), S0)


def _noalloc(q, K, V, ld, A, B, S0, chunk):
    Bb, H, T, dk = q.shape
    dv = V.shape[-1]
    r_ab = 0 if A is None else A.shape[-2]
    out = torch.empty((Bb, H, T, dv), dtype=q.dtype, device=q.device)
    Sf = torch.empty((Bb, H, dk, dv), dtype=torch.float32, device=q.device)
    dims = lattn.make_dims(Bb, H, T, dk, dv, 1 if q.dtype == torch.bfloat16 else 0, False)
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    rc = _lib.load().lattn_chunk_fwd_noalloc(ctypes.byref(dims), p(q), p(K), p(V), p(ld), p(A), p(B), r_ab, 1,
                                             chunk, p(out), p(Sf), p(S0),
                                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    _lib.check(rc, "lattn_chunk_fwd_noalloc")
    return out, Sf


CASES = [
    # first call, then a smaller second call: (B, H, T, dk, dv, r_ab, dtype)
    ((2, 8, 1000, 128, 128, 2, "bf16"), (1, 2, 130, 128, 128, 2, "bf16")),
    ((1, 4, 300, 64, 64, 2, "fp32"), (1, 1, 77, 64, 64, 2, "fp32")),
]


@pytest.mark.parametrize("first,second", CASES, ids=["mfma_bf16", "general_fp32"])
def test_noalloc_matches_workspace_entry(first, second):
    for i, shape in enumerate((first, second)):
        Bb, H, T, dk, dv, r_ab, dtype = shape
        dims = lattn.make_dims(Bb, H, T, dk, dv, 1 if dtype == "bf16" else 0, False)
        need = int(_lib.load().lattn_chunk_fwd_workspace_size(ctypes.byref(dims), r_ab, 1, 64))
        assert 0 < need <= SCRATCH, (shape, need)
        args = _inputs(Bb, H, T, dk, dv, r_ab, dtype, seed=40 + i)
        ref_out, ref_S = lattn.chunk_fwd(*args[:6], chunk=64, initial_state=args[6])
        got_out, got_S = _noalloc(*args, chunk=64)
        torch.cuda.synchronize()
        e_o = rel_err(host(got_out), host(ref_out))
        e_s = rel_err(host(got_S), host(ref_S))
        same = torch.equal(got_out, ref_out) and torch.equal(got_S, ref_S)
        print(f"call {i + 1} {shape}: scratch {need} B, out {e_o:.2e} state {e_s:.2e}, bitwise equal {same}",
              flush=True)
        assert e_o <= TOL[dtype] and e_s <= TOL[dtype]


def test_noalloc_rejects_problems_beyond_the_scratch():
    Bb, H, T, dk, dv = 8, 16, 4096, 128, 128
    dims = lattn.make_dims(Bb, H, T, dk, dv, 1, False)
    need = int(_lib.load().lattn_chunk_fwd_workspace_size(ctypes.byref(dims), 2, 1, 64))
    assert need > SCRATCH
    fake = ctypes.c_void_p(0x100000)   # never dereferenced: the call returns before any launch
    rc = _lib.load().lattn_chunk_fwd_noalloc(ctypes.byref(dims), fake, fake, fake, fake, fake, fake, 2, 1, 64,
                                             fake, None, None, None)
    assert rc == _lib.LATTN_EWORKSPACE
    assert b"scratch" in _lib.load().lattn_last_error()
