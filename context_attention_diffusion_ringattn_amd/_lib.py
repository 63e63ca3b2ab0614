"""ctypes binding of include/ringattn.h.

Argument marshalling only: every step of the attention path runs in the HIP
library.  Loading fails loudly if ``libringattn.so`` has not been built --
there is no CPU fallback.
"""

from __future__ import annotations

import ctypes
import os
import threading

# RINGATTN_LIB selects another build of the same library (the sanitizer
# build of build.py); by default the in-tree libringattn.so.
LIB_PATH = os.environ.get("RINGATTN_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                          "libringattn.so")

RINGATTN_OK = 0
RINGATTN_EINVAL = -1
RINGATTN_EUNSUPPORTED = -2
RINGATTN_EWORKSPACE = -3
RINGATTN_EHIP = -4
RINGATTN_MAX_CHUNKS = 128

# Every symbol include/ringattn.h declares.
EXPORTED_SYMBOLS = (
    "ringattn_status_string",
    "ringattn_last_error",
    "ringattn_abi_version",
    "ringattn_chunk_offsets",
    "ringattn_acc_init",
    "ringattn_step",
    "ringattn_merge",
    "ringattn_forward_plan",
    "ringattn_forward",
    "ringattn_ring_sweep",
    "ringattn_cp_layout",
    "ringattn_acc_init_bf16",
    "ringattn_step_bf16",
    "ringattn_step_split",
    "ringattn_forward_noalloc",
)


class Shape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("q_len", ctypes.c_int64),
        ("kv_len", ctypes.c_int64),
    ]


class Plan(ctypes.Structure):
    _fields_ = [
        ("n_splits", ctypes.c_int32),
        ("block_m", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_uint64),
    ]


class CpConfig(ctypes.Structure):
    _fields_ = [
        ("seq_len", ctypes.c_int64),
        ("heads", ctypes.c_int32),
        ("ring_degree", ctypes.c_int32),
        ("ulysses_degree", ctypes.c_int32),
        ("ring_anything", ctypes.c_int32),
        ("ulysses_anything", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class CpShare(ctypes.Structure):
    _fields_ = [
        ("ring_index", ctypes.c_int32),
        ("ulysses_index", ctypes.c_int32),
        ("token_begin", ctypes.c_int64),
        ("token_end", ctypes.c_int64),
        ("q_begin", ctypes.c_int64),
        ("q_end", ctypes.c_int64),
        ("head_begin", ctypes.c_int32),
        ("head_end", ctypes.c_int32),
    ]


class RingAttnError(RuntimeError):
    """A library call returned a non-OK status."""

    def __init__(self, status: int, func: str, message: str):
        self.status = status
        self.func = func
        super().__init__(f"{func}: {status_string(status)}: {message}")


_lib = None
_lock = threading.Lock()

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_sz = ctypes.c_size_t
_shape_p = ctypes.POINTER(Shape)
_plan_p = ctypes.POINTER(Plan)
_i64p = ctypes.POINTER(ctypes.c_int64)

_SIGNATURES = {
    "ringattn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "ringattn_last_error": (ctypes.c_char_p, []),
    "ringattn_abi_version": (_i32, []),
    "ringattn_chunk_offsets": (ctypes.c_int, [_i64, _i32, _i32, _i64p]),
    "ringattn_acc_init": (ctypes.c_int, [_vp, _vp, _shape_p, _vp]),
    "ringattn_step": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _f32, _shape_p, _vp]),
    "ringattn_merge": (ctypes.c_int, [_vp, _vp, _vp, _vp, _shape_p, _vp]),
    "ringattn_forward_plan": (ctypes.c_int, [_shape_p, _i64p, _i32, _i64, _plan_p]),
    "ringattn_forward": (ctypes.c_int, [_vp, _vp, _vp, _i64p, _i32, _i64, _vp, _vp, _f32, _shape_p, _plan_p, _vp,
                                        _sz, _vp]),
    "ringattn_ring_sweep": (ctypes.c_int, [_vp, _vp, _vp, _i64p, _i32, _i64, _vp, _vp, _f32, _shape_p, _vp]),
    "ringattn_cp_layout": (ctypes.c_int, [ctypes.POINTER(CpConfig), _i32, ctypes.POINTER(CpShare)]),
    "ringattn_acc_init_bf16": (ctypes.c_int, [_vp, _vp, _shape_p, _vp]),
    "ringattn_step_bf16": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _f32, _shape_p, _vp]),
    "ringattn_step_split": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _f32, _shape_p, _plan_p, _vp, _sz, _vp]),
    "ringattn_forward_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _i64p, _i32, _i64, _vp, _vp, _f32, _shape_p, _plan_p,
                                                _vp]),
}


def lib() -> ctypes.CDLL:
    """The loaded library (loaded on first use)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is not built; run `python -m context_attention_diffusion_ringattn_amd.build` "
                    f"(or __graft_entry__.build()) first -- there is no CPU fallback")
            handle = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in _SIGNATURES.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().ringattn_status_string(status).decode()


def last_error() -> str:
    return lib().ringattn_last_error().decode()


def check(status: int, func: str) -> None:
    if status != RINGATTN_OK:
        raise RingAttnError(status, func, last_error())


def offsets_array(offsets):
    arr = (ctypes.c_int64 * len(offsets))(*[int(x) for x in offsets])
    return arr
