"""ctypes view of liblattn.so (the C ABI declared in include/lattn.h)."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblattn.so")

LATTN_OK = 0
LATTN_EINVAL = -1
LATTN_EUNSUPPORTED = -2
LATTN_EWORKSPACE = -3
LATTN_EHIP = -4
LATTN_EDECAY_RANGE = -5

LATTN_FP32 = 0
LATTN_BF16 = 1
LATTN_DECAY_PER_CHANNEL = 0
LATTN_DECAY_SCALAR = 1


class lattn_dims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64),
        ("heads", ctypes.c_int64),
        ("seqlen", ctypes.c_int64),
        ("d_k", ctypes.c_int32),
        ("d_v", ctypes.c_int32),
        ("dtype", ctypes.c_int),
        ("decay_mode", ctypes.c_int),
    ]


# Every exported entry point with its (restype, argtypes).
_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_D = ctypes.POINTER(lattn_dims)
SIGNATURES = {
    "lattn_chunk_fwd": (_I, [_D, _P, _P, _P, _P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "lattn_chunk_fwd_workspace_size": (_SZ, [_D, _I, _I, _I]),
    "lattn_chunk_fwd_noalloc": (_I, [_D, _P, _P, _P, _P, _P, _P, _I, _I, _I, _P, _P, _P, _P]),
    "lattn_chunk_fwd_check": (_I, [_D, _P, _P, _P, _P, _P, _P, _I, _I, _I, _P, _P, _SZ]),
    "lattn_chunk_prepare": (_I, [_D, _P, _P, _P, _P, _P, _I, _I, _I, _P, _SZ, _P]),
    "lattn_chunk_scan": (_I, [_D, _P, _I, _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "lattn_chunk_summaries_workspace_size": (_SZ, [_D, _I, _I, _I]),
    "lattn_chunk_summaries": (_I, [_D, _P, _P, _P, _P, _P, _I, _I, _I, _P, _P, _P, _SZ, _P]),
    "lattn_hla_fwd": (_I, [_D, _P, _P, _P, _P, _P, _P, _I, _I, _I, _P, ctypes.c_float, _P, _P, _SZ, _P]),
    "lattn_hla_fwd_workspace_size": (_SZ, [_D, _I, _I, _I]),
    "lattn_loglinear_fwd": (_I, [_D, _P, _P, _P, _P, _P, _P, _I, _I, _I, _P, _P, _P, _SZ, _P]),
    "lattn_loglinear_fwd_workspace_size": (_SZ, [_D, _I, _I, _I]),
    "lattn_loglinear_levels": (_I, [ctypes.c_int64]),
    "lattn_chunk_bwd": (_I, [_D, _P, _P, _P, _P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                              _SZ, _P]),
    "lattn_chunk_bwd_workspace_size": (_SZ, [_D, _I, _I, _I]),
    "lattn_chunk_fwd_train": (_I, [_D, _P, _P, _P, _P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "lattn_chunk_fwd_train_saved_size": (_SZ, [_D, _I, _I, _I]),
    "lattn_chunk_bwd_saved": (_I, [_D, _P, _P, _P, _P, _P, _P, _I, _I, _I, _P, _P, _P, _SZ, _P, _P, _P, _P, _P, _P,
                                    _P, _P, _SZ, _P]),
    "lattn_chunk_bwd_saved_workspace_size": (_SZ, [_D, _I, _I, _I]),
    "lattn_step": (_I, [_D, _P, _P, _P, _P, _P, _P, _I, _I, _P, _P, _P]),
    "lattn_hdla_params": (_I, [_D, _P, _P, _P, _P, _P, _P, _P, _P]),
    "lattn_gdn_params": (_I, [_D, _P, _P, _P, _P, _P, _P, _P, _P]),
    "lattn_hdla_chunk_fwd": (_I, [_D, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _SZ, _P]),
    "lattn_hdla_chunk_fwd_workspace_size": (_SZ, [_D, _I]),
    "lattn_gdn_chunk_fwd": (_I, [_D, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _SZ, _P]),
    "lattn_gdn_chunk_fwd_workspace_size": (_SZ, [_D, _I]),
    "lattn_decay_range": (_I, [_D, _P, _I, _P, _P]),
    "lattn_check_decay_range": (_I, [_D, _P, _I, _P, _P]),
    "lattn_chunk_fwd_kernels": (ctypes.c_char_p, [_D, _I, _I, _I]),
    "lattn_status_str": (ctypes.c_char_p, [_I]),
    "lattn_last_error": (ctypes.c_char_p, []),
    "lattn_version": (ctypes.c_char_p, []),
}

_lib = None


class LattnError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str):
        self.status = status
        super().__init__(f"{fn}: {status_str(status)} ({detail})")


def load():
    """Load the in-tree liblattn.so.  Raises if it has not been built: there is no
    fallback implementation."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
                "or `python structured_decay_sequence_amd/build.py`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def status_str(status: int) -> str:
    return load().lattn_status_str(status).decode()


def last_error() -> str:
    return load().lattn_last_error().decode()


def check(status: int, fn: str):
    if status != LATTN_OK:
        raise LattnError(status, fn, last_error())
    return status
