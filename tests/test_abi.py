"""C ABI checks that need no GPU: the library loads, exports every declared
entry point, and its host-side validation rejects bad arguments before any
launch (only the pure host functions are called here)."""
import ctypes
import os
import re

import pytest

from structured_decay_sequence_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "lattn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lattn_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ["lattn_chunk_fwd", "lattn_step", "lattn_chunk_fwd_workspace_size", "lattn_status_str",
              "lattn_last_error", "lattn_chunk_summaries", "lattn_hdla_params", "lattn_gdn_params",
              "lattn_check_decay_range", "lattn_decay_range", "lattn_chunk_fwd_check", "lattn_version"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in _declared():
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, f"binding lacks a signature for {name}"


def test_status_strings():
    lib = _lib.load()
    for code in [0, -1, -2, -3, -4, -5]:
        assert lib.lattn_status_str(code)
    assert b"unknown" in lib.lattn_status_str(-99)
    assert lib.lattn_version().startswith(b"lattn")


def _dims(**kw):
    d = dict(batch=1, heads=2, seqlen=128, d_k=64, d_v=64, dtype=_lib.LATTN_BF16,
             decay_mode=_lib.LATTN_DECAY_PER_CHANNEL)
    d.update(kw)
    return _lib.lattn_dims(d["batch"], d["heads"], d["seqlen"], d["d_k"], d["d_v"], d["dtype"],
                           d["decay_mode"])


FAKE = 0x100000  # never dereferenced: validation only tests NULL and alignment


def _check(dims, r_ab=2, r_kv=1, chunk=64, ws_bytes=None, **ptrs):
    lib = _lib.load()
    p = {n: FAKE for n in ["q", "k", "v", "ld", "A", "B", "out", "ws"]}
    if r_ab == 0:
        p["A"] = p["B"] = None
    p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = lib.lattn_chunk_fwd_workspace_size(ctypes.byref(dims), r_ab, r_kv, chunk)
    return lib.lattn_chunk_fwd_check(ctypes.byref(dims), p["q"], p["k"], p["v"], p["ld"], p["A"], p["B"],
                                     r_ab, r_kv, chunk, p["out"], p["ws"], ws_bytes)


def test_valid_arguments_pass():
    assert _check(_dims()) == _lib.LATTN_OK
    assert _check(_dims(dtype=_lib.LATTN_FP32, decay_mode=_lib.LATTN_DECAY_SCALAR), r_ab=1) == _lib.LATTN_OK
    assert _check(_dims(), r_ab=0, r_kv=2, chunk=16) == _lib.LATTN_OK
    assert _check(_dims(seqlen=0), q=None, k=None, v=None, ld=None, A=None, B=None, out=None, ws=None,
                  ws_bytes=0) == _lib.LATTN_OK


@pytest.mark.parametrize("kw,args,code", [
    (dict(d_k=24), {}, _lib.LATTN_EINVAL),
    (dict(d_k=272), {}, _lib.LATTN_EINVAL),
    (dict(d_v=8), {}, _lib.LATTN_EINVAL),
    (dict(batch=0), {}, _lib.LATTN_EINVAL),
    (dict(seqlen=-1), {}, _lib.LATTN_EINVAL),
    (dict(dtype=7), {}, _lib.LATTN_EINVAL),
    (dict(decay_mode=3), {}, _lib.LATTN_EINVAL),
    ({}, dict(chunk=48), _lib.LATTN_EINVAL),
    ({}, dict(r_ab=-1), _lib.LATTN_EINVAL),
    ({}, dict(r_kv=0), _lib.LATTN_EINVAL),
    ({}, dict(r_ab=8, chunk=128), _lib.LATTN_EUNSUPPORTED),
    ({}, dict(r_kv=4, chunk=128), _lib.LATTN_EUNSUPPORTED),
    ({}, dict(q=None), _lib.LATTN_EINVAL),
    ({}, dict(A=None), _lib.LATTN_EINVAL),
    ({}, dict(r_ab=0), _lib.LATTN_OK),
    ({}, dict(v=FAKE + 2), _lib.LATTN_EINVAL),
    ({}, dict(ws=None), _lib.LATTN_EWORKSPACE),
    ({}, dict(ws_bytes=16), _lib.LATTN_EWORKSPACE),
])
def test_invalid_arguments_are_rejected(kw, args, code):
    rc = _check(_dims(**kw), **args)
    assert rc == code, (rc, _lib.last_error())
    if code != _lib.LATTN_OK:
        assert _lib.last_error()


def test_ab_must_be_null_without_decay_rank():
    assert _check(_dims(), r_ab=0, A=FAKE, B=FAKE) == _lib.LATTN_EINVAL


def test_workspace_size_is_zero_for_invalid_and_grows_with_length():
    lib = _lib.load()
    bad = _dims(d_k=20)
    assert lib.lattn_chunk_fwd_workspace_size(ctypes.byref(bad), 2, 1, 64) == 0
    a = lib.lattn_chunk_fwd_workspace_size(ctypes.byref(_dims(seqlen=256)), 2, 1, 64)
    b = lib.lattn_chunk_fwd_workspace_size(ctypes.byref(_dims(seqlen=512)), 2, 1, 64)
    assert 0 < a < b


def test_hla_and_loglinear_entry_points_declared():
    names = _declared()
    for n in ["lattn_hla_fwd", "lattn_hla_fwd_workspace_size", "lattn_loglinear_fwd",
              "lattn_loglinear_fwd_workspace_size", "lattn_loglinear_levels"]:
        assert n in names


def test_loglinear_levels_host():
    lib = _lib.load()
    # 1 + bit length of (T - 1): levels 0 .. that of position T - 1
    for T, L in [(0, 0), (1, 1), (2, 2), (3, 3), (4, 3), (5, 4), (4096, 13), (4097, 14), (32768, 16)]:
        assert lib.lattn_loglinear_levels(T) == L, T


def test_hla_and_loglinear_validation_before_launch():
    lib = _lib.load()
    d = _dims(d_k=256, d_v=64, dtype=_lib.LATTN_FP32)
    F = ctypes.c_void_p(FAKE)
    # d_k = 256 is outside both kernels' register plans: rejected on the host
    rc = lib.lattn_hla_fwd(ctypes.byref(d), F, F, F, F, F, F, 2, 1, 64, F, ctypes.c_float(0.1), F, F, 1 << 40, None)
    assert rc == _lib.LATTN_EUNSUPPORTED
    rc = lib.lattn_loglinear_fwd(ctypes.byref(d), F, F, F, F, F, F, 2, 1, 64, F, F, F, 1 << 40, None)
    assert rc == _lib.LATTN_EUNSUPPORTED
    d = _dims(dtype=_lib.LATTN_FP32)
    # gates / lambda are required
    rc = lib.lattn_hla_fwd(ctypes.byref(d), F, F, F, F, F, F, 2, 1, 64, None, ctypes.c_float(0.1), F, F, 1 << 40, None)
    assert rc == _lib.LATTN_EINVAL and b"gates" in lib.lattn_last_error()
    rc = lib.lattn_loglinear_fwd(ctypes.byref(d), F, F, F, F, F, F, 2, 1, 64, None, F, F, 1 << 40, None)
    assert rc == _lib.LATTN_EINVAL and b"lambda" in lib.lattn_last_error()
    # workspace too small
    rc = lib.lattn_hla_fwd(ctypes.byref(d), F, F, F, F, F, F, 2, 1, 64, F, ctypes.c_float(0.1), F, F, 16, None)
    assert rc == _lib.LATTN_EWORKSPACE
    rc = lib.lattn_loglinear_fwd(ctypes.byref(d), F, F, F, F, F, F, 2, 1, 64, F, F, F, 16, None)
    assert rc == _lib.LATTN_EWORKSPACE
    # d_k + chunk > 192 is outside the log-linear scan's register plan
    d = _dims(d_k=128, d_v=64, dtype=_lib.LATTN_FP32)
    rc = lib.lattn_loglinear_fwd(ctypes.byref(d), F, F, F, F, F, F, 2, 1, 128, F, F, F, 1 << 40, None)
    assert rc == _lib.LATTN_EUNSUPPORTED
    assert lib.lattn_hla_fwd_workspace_size(ctypes.byref(d), 2, 1, 64) > 0
    assert lib.lattn_loglinear_fwd_workspace_size(ctypes.byref(d), 2, 1, 64) > 0


def test_training_pair_sizes_follow_the_chunked_route():
    """lattn_chunk_fwd_train's saved buffer and lattn_chunk_bwd_saved's workspace
    exist only on the chunked backward's route (bf16, chunk 64, r_kv 1,
    r_ab <= 2, d_k and d_v in {64, 128}); the saved-state backward needs less
    workspace than lattn_chunk_bwd, which forms the saved operands itself."""
    lib = _lib.load()
    on = _dims(seqlen=256)
    saved = lib.lattn_chunk_fwd_train_saved_size(ctypes.byref(on), 2, 1, 64)
    ws = lib.lattn_chunk_bwd_saved_workspace_size(ctypes.byref(on), 2, 1, 64)
    assert saved > 0 and ws > 0
    # the saved buffer holds at least the chunk operators the forward needs
    assert saved > lib.lattn_chunk_fwd_workspace_size(ctypes.byref(on), 2, 1, 64)
    assert ws < lib.lattn_chunk_bwd_workspace_size(ctypes.byref(on), 2, 1, 64)
    longer = _dims(seqlen=512)
    assert lib.lattn_chunk_fwd_train_saved_size(ctypes.byref(longer), 2, 1, 64) > saved
    for dims, r_ab, r_kv, chunk in [(_dims(dtype=_lib.LATTN_FP32), 2, 1, 64), (on, 2, 1, 32), (on, 2, 2, 64),
                                    (on, 3, 1, 64), (_dims(d_k=32, d_v=32), 2, 1, 64)]:
        assert lib.lattn_chunk_fwd_train_saved_size(ctypes.byref(dims), r_ab, r_kv, chunk) == 0
        assert lib.lattn_chunk_bwd_saved_workspace_size(ctypes.byref(dims), r_ab, r_kv, chunk) == 0


def test_training_pair_validation_before_launch():
    """Off-route shapes and short buffers are rejected on the host, before any
    device work (the pointers are never dereferenced)."""
    lib = _lib.load()
    f = FAKE
    fp32 = _dims(dtype=_lib.LATTN_FP32)
    rc = lib.lattn_chunk_fwd_train(ctypes.byref(fp32), f, f, f, f, f, f, 2, 1, 64, f, None, None, f, 1 << 30, None)
    assert rc == _lib.LATTN_EUNSUPPORTED
    assert b"lattn_chunk_fwd_train" in lib.lattn_last_error()
    on = _dims()
    need = lib.lattn_chunk_fwd_train_saved_size(ctypes.byref(on), 2, 1, 64)
    rc = lib.lattn_chunk_fwd_train(ctypes.byref(on), f, f, f, f, f, f, 2, 1, 64, f, None, None, f, need - 1, None)
    assert rc == _lib.LATTN_EWORKSPACE
    rc = lib.lattn_chunk_fwd_train(ctypes.byref(on), f, f, f, f, f, f, 2, 1, 64, f, None, None, None, need, None)
    assert rc == _lib.LATTN_EWORKSPACE
    ws = lib.lattn_chunk_bwd_saved_workspace_size(ctypes.byref(on), 2, 1, 64)
    grads = [f] * 7
    rc = lib.lattn_chunk_bwd_saved(ctypes.byref(on), f, f, f, f, f, f, 2, 1, 64, f, None, f, need - 1, *grads,
                                   f, ws, None)
    assert rc == _lib.LATTN_EWORKSPACE
    rc = lib.lattn_chunk_bwd_saved(ctypes.byref(on), f, f, f, f, f, f, 2, 1, 64, f, None, f, need, *grads,
                                   f, ws - 1, None)
    assert rc == _lib.LATTN_EWORKSPACE
    rc = lib.lattn_chunk_bwd_saved(ctypes.byref(fp32), f, f, f, f, f, f, 2, 1, 64, f, None, f, need, *grads,
                                   f, ws, None)
    assert rc == _lib.LATTN_EUNSUPPORTED
    # r_ab == 0 takes no dA, dB
    rc = lib.lattn_chunk_bwd_saved(ctypes.byref(on), f, f, f, f, None, None, 0, 1, 64, f, None, f, need,
                                   f, f, f, f, f, f, f, f, ws, None)
    assert rc == _lib.LATTN_EINVAL


def test_split_scan_workspace():
    """The forward's workspace holds the chunk operators, plus the split scan's
    scratch where the scan splits the sequence (d_k = 64, few heads, at least 64
    chunks): the long-context HDLA shape splits, the headline shape does not."""
    lib = _lib.load()
    ops = lambda B, H, T, dk, dv: B * H * -(-T // 64) * ((dk + 64) // 16) ** 2 * 512
    head = _dims(batch=8, heads=16, seqlen=4096, d_k=128, d_v=128)
    assert lib.lattn_chunk_fwd_workspace_size(ctypes.byref(head), 2, 1, 64) == ops(8, 16, 4096, 128, 128)
    long = _dims(batch=1, heads=48, seqlen=32768, d_k=64, d_v=64)
    assert lib.lattn_chunk_fwd_workspace_size(ctypes.byref(long), 2, 1, 64) > ops(1, 48, 32768, 64, 64)
    short = _dims(batch=1, heads=48, seqlen=4000, d_k=64, d_v=64)   # 63 chunks: not split
    assert lib.lattn_chunk_fwd_workspace_size(ctypes.byref(short), 2, 1, 64) == ops(1, 48, 4000, 64, 64)
