"""ctypes binding of libgdpa.so (include/gdpa.h). Argument marshalling only.

The structures mirror ``gdpa_problem`` and ``gdpa_tensors``; the functions keep the C names.
Every computation runs in the library's HIP kernels; if the library is missing this module
raises instead of falling back to anything else.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdpa.so")

GDPA_OK = 0
GDPA_ERR_INVALID_ARGUMENT = -1
GDPA_ERR_UNSUPPORTED = -2
GDPA_ERR_WORKSPACE = -3
GDPA_ERR_HIP = -4

GDPA_DTYPE_BF16 = 0
GDPA_DTYPE_FP32 = 1

GDPA_ACT_GELU = 0
GDPA_ACT_SILU = 1
GDPA_ACT_SOFTMAX = 2

GDPA_MAX_GROUPS = 16
GDPA_FLAG_PLANNED = 1
GDPA_FLAG_SHARED_Q = 2
GDPA_FLAG_FP32_OUT = 4
GDPA_FLAG_VALIDATE = 8
GDPA_FLAG_SPLIT_OPERANDS = 16

GDPA_WS_ERROR_OFFSET = 0
GDPA_DEVICE_ERR_OFFSETS = 1
GDPA_DEVICE_ERR_LENGTH = 2
GDPA_DEVICE_ERR_SELF = 4
GDPA_DEVICE_ERR_PLAN = 8

EXPORTED = ("gdpa_workspace_size", "gdpa_plan", "gdpa_fwd", "gdpa_bwd", "gdpa_fwd_grouped",
            "gdpa_bwd_grouped", "gdpa_validate_offsets", "gdpa_bwd_noalloc", "gdpa_strerror", "gdpa_version")
GDPA_NOALLOC_SCRATCH_BYTES = 16 << 20


class gdpa_problem(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("act", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("window_left", ctypes.c_int32),
        ("window_right", ctypes.c_int32),
        ("total_q", ctypes.c_int64),
        ("total_kv", ctypes.c_int64),
        ("max_seqlen_q", ctypes.c_int32),
        ("max_seqlen_kv", ctypes.c_int32),
        ("self_attention", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("q_offsets", ctypes.c_void_p),
        ("kv_offsets", ctypes.c_void_p),
        ("head_acts", ctypes.c_void_p),
    ]


class gdpa_tensors(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("g", ctypes.c_void_p),
        ("o", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("dout", ctypes.c_void_p),
        ("dq", ctypes.c_void_p),
        ("dk", ctypes.c_void_p),
        ("dv", ctypes.c_void_p),
        ("dg", ctypes.c_void_p),
    ]


class GdpaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {strerror(status)} (status {status})")
        self.status = status


_lib = None


def load(path: str = LIB_PATH):
    """Load libgdpa.so. Raises if it has not been built (no fallback path exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} not found: build it with `python -m generalized_attention_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    lib.gdpa_workspace_size.argtypes = [P(gdpa_problem), ctypes.c_int32, ctypes.c_int32]
    lib.gdpa_workspace_size.restype = ctypes.c_size_t
    for name in ("gdpa_fwd", "gdpa_bwd"):
        f = getattr(lib, name)
        f.argtypes = [P(gdpa_problem), P(gdpa_tensors), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        f.restype = ctypes.c_int
    for name in ("gdpa_fwd_grouped", "gdpa_bwd_grouped"):
        f = getattr(lib, name)
        f.argtypes = [P(gdpa_problem), P(gdpa_tensors), ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
                      ctypes.c_void_p]
        f.restype = ctypes.c_int
    lib.gdpa_plan.argtypes = [P(gdpa_problem), ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.gdpa_plan.restype = ctypes.c_int
    lib.gdpa_bwd_noalloc.argtypes = [P(gdpa_problem), P(gdpa_tensors), ctypes.c_void_p]
    lib.gdpa_bwd_noalloc.restype = ctypes.c_int
    lib.gdpa_validate_offsets.argtypes = [P(gdpa_problem), ctypes.c_void_p, ctypes.c_void_p]
    lib.gdpa_validate_offsets.restype = ctypes.c_int
    lib.gdpa_strerror.argtypes = [ctypes.c_int]
    lib.gdpa_strerror.restype = ctypes.c_char_p
    lib.gdpa_version.argtypes = []
    lib.gdpa_version.restype = ctypes.c_int
    _lib = lib
    return lib


def strerror(status: int) -> str:
    return load().gdpa_strerror(int(status)).decode()


def gdpa_workspace_size(problems, pass_: int) -> int:
    arr = (gdpa_problem * len(problems))(*problems)
    return int(load().gdpa_workspace_size(arr, len(problems), int(pass_)))


def _call_grouped(fn, problems, tensors, ws, ws_bytes, stream):
    n = len(problems)
    pa = (gdpa_problem * n)(*problems)
    ta = (gdpa_tensors * n)(*tensors)
    return fn(pa, ta, n, ctypes.c_void_p(ws), ctypes.c_size_t(ws_bytes), ctypes.c_void_p(stream))


def gdpa_plan(problems, ws, ws_bytes, stream) -> int:
    n = len(problems)
    pa = (gdpa_problem * n)(*problems)
    return load().gdpa_plan(pa, n, ctypes.c_void_p(ws), ctypes.c_size_t(ws_bytes), ctypes.c_void_p(stream))


def gdpa_validate_offsets(problem, q_offsets_host, kv_offsets_host) -> int:
    """The offsets rules on host int32 arrays (numpy, contiguous): GDPA_DEVICE_ERR_* bits or a
    negative status."""
    return load().gdpa_validate_offsets(ctypes.byref(problem), q_offsets_host.ctypes.data_as(ctypes.c_void_p),
                                        kv_offsets_host.ctypes.data_as(ctypes.c_void_p))


def gdpa_fwd(problem, tensors, ws, ws_bytes, stream) -> int:
    return load().gdpa_fwd(ctypes.byref(problem), ctypes.byref(tensors), ctypes.c_void_p(ws),
                           ctypes.c_size_t(ws_bytes), ctypes.c_void_p(stream))


def gdpa_bwd(problem, tensors, ws, ws_bytes, stream) -> int:
    return load().gdpa_bwd(ctypes.byref(problem), ctypes.byref(tensors), ctypes.c_void_p(ws),
                           ctypes.c_size_t(ws_bytes), ctypes.c_void_p(stream))


def gdpa_bwd_noalloc(problem, tensors, stream) -> int:
    return load().gdpa_bwd_noalloc(ctypes.byref(problem), ctypes.byref(tensors), ctypes.c_void_p(stream))


def gdpa_fwd_grouped(problems, tensors, ws, ws_bytes, stream) -> int:
    return _call_grouped(load().gdpa_fwd_grouped, problems, tensors, ws, ws_bytes, stream)


def gdpa_bwd_grouped(problems, tensors, ws, ws_bytes, stream) -> int:
    return _call_grouped(load().gdpa_bwd_grouped, problems, tensors, ws, ws_bytes, stream)
