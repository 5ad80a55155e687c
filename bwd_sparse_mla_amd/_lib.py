"""ctypes loader for libsmla.so; declares every C ABI entry point of include/smla.h."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsmla.so")

SMLA_OK = 0
SMLA_DKV_ACCUMULATE = 1
SMLA_DKV_ATOMIC = 2
SMLA_PLAN_READY = 4
SMLA_DKV_STORED_P = 8
SMLA_FP8_POW2_SCALES = 16
SMLA_DTYPE_BF16 = 0
SMLA_DTYPE_F32 = 1
SMLA_NOALLOC_SCRATCH_BYTES = 64 << 20   # smla_fwd_noalloc's per-device scratch

STATUS_NAMES = {0: "SMLA_OK", 1: "SMLA_ERR_NULL", 2: "SMLA_ERR_SHAPE", 3: "SMLA_ERR_ALIGN",
                4: "SMLA_ERR_WORKSPACE", 5: "SMLA_ERR_FLAGS", 6: "SMLA_ERR_HIP",
                7: "SMLA_ERR_DEVICE"}

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t

SIGNATURES = {
    "smla_fwd": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I32, _I32, ctypes.c_float,
                                _P, _P, _P, _SZ, _P]),
    "smla_fwd_ex": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I32, _I32, ctypes.c_float,
                                   _P, _P, ctypes.c_uint32, _P, _SZ, _P]),
    "smla_plan": (ctypes.c_int, [_P, _I64, _I64, _I32, _I32, _P, _SZ, _P]),
    "smla_fwd_workspace_size": (_SZ, [_I64, _I64, _I32, _I32]),
    "smla_fwd_noalloc": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I32, _I32, ctypes.c_float,
                                        _P, _P, _P]),
    "smla_bwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I32, _I32, ctypes.c_float,
                                _P, _P, _P, ctypes.c_uint32, _P, _SZ, _P]),
    "smla_bwd_workspace_size": (_SZ, [_I64, _I64, _I32, _I32, ctypes.c_uint32]),
    "smla_plan_g": (ctypes.c_int, [_P, _I64, _I64, _I32, _I32, _I32, _P, _SZ, _P]),
    "smla_fwd_g": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I32, _I32, _I32, ctypes.c_float,
                                  _P, _P, ctypes.c_uint32, _P, _SZ, _P]),
    "smla_fwd_workspace_size_g": (_SZ, [_I64, _I64, _I32, _I32, _I32]),
    "smla_fwd_fp8": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I32, _I32, _I32, ctypes.c_float,
                                    _P, _P, ctypes.c_uint32, _P, _SZ, _P]),
    "smla_bwd_g": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I32, _I32, _I32,
                                  ctypes.c_float, _P, _P, _P, ctypes.c_uint32, _P, _SZ, _P]),
    "smla_bwd_workspace_size_g": (_SZ, [_I64, _I64, _I32, _I32, _I32, ctypes.c_uint32]),
    "smla_validate_indices": (ctypes.c_int, [_P, _I64, _I32, _I64, _P, _P]),
    "smla_nonfinite_count": (ctypes.c_int, [_P, _I32, _I64, _P, _P]),
    "smla_nonfinite_replace": (ctypes.c_int, [_P, _P, _I32, _I64, _P, _P]),
    "smla_topk_indices": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _P, _I32, _P, _P]),
    "smla_timing_start": (ctypes.c_int, [ctypes.c_int]),
    "smla_timing_stop": (ctypes.c_int, []),
    "smla_timing_read": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_int),
                                        ctypes.POINTER(ctypes.c_double)]),
    "smla_last_error": (ctypes.c_char_p, []),
    "smla_version": (ctypes.c_int, []),
    "smla_device_supported": (ctypes.c_int, [ctypes.c_int]),
}

_lib = None


class SmlaError(RuntimeError):
    """A nonzero status from the C ABI."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libsmla.so (built in-tree).  Raises if it has not been built:
    there is no fallback implementation."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m bwd_sparse_mla_amd.build` "
                "(or __graft_entry__.build()); the HIP library is required")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(status: int) -> None:
    if status != SMLA_OK:
        msg = load().smla_last_error()
        raise SmlaError(status, msg.decode() if msg else "")
