"""ctypes front end of the fp64 GDPA oracle (``oracle/gdpa_oracle.cpp``).

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the benchmark's
CPU-baseline leg may import this module; the product path (``generalized_attention_amd``) never
does, and shares no code with it. The oracle computes the plain definition of the operator in
float64 (see the header comment of the C++ source for the formulas and their sources).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdpa_oracle.so")
SRC_PATH = os.path.join(_HERE, "gdpa_oracle.cpp")

ACT_CODES = {"gelu": 0, "silu": 1, "softmax": 2}

_lib = None


def build(src: str = SRC_PATH, out: str = LIB_PATH, extra_flags=()) -> str:
    """Compile the oracle with g++ (plain IEEE arithmetic: no fast-math)."""
    cmd = ["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-pthread", *extra_flags, src, "-o", out]
    subprocess.run(cmd, check=True)
    return out


def load(path: str = LIB_PATH):
    """Load (building first if absent) and declare the oracle's C entry points."""
    global _lib
    if path == LIB_PATH and _lib is not None:
        return _lib
    if not os.path.exists(path):
        build(out=path)
    lib = ctypes.CDLL(path)
    d, i, p = ctypes.c_double, ctypes.c_int, ctypes.c_void_p
    lib.gdpa_oracle_phi.argtypes = [i, d]
    lib.gdpa_oracle_phi.restype = d
    lib.gdpa_oracle_phi_grad.argtypes = [i, d]
    lib.gdpa_oracle_phi_grad.restype = d
    lib.gdpa_oracle_log_sigmoid.argtypes = [d]
    lib.gdpa_oracle_log_sigmoid.restype = d
    lib.gdpa_oracle_fwd.argtypes = [i, i, i, p, p, p, p, p, p, i, d, i, i, p, p, i, p, i]
    lib.gdpa_oracle_fwd.restype = i
    lib.gdpa_oracle_bwd.argtypes = [i, i, i, p, p, p, p, p, p, i, d, i, i, p, p, p, p, p, i, p, i]
    lib.gdpa_oracle_bwd.restype = i
    if path == LIB_PATH:
        _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _acts(act, h):
    """(default code, per-head codes or None) for act = a name or one name per head."""
    if isinstance(act, str):
        return ACT_CODES[act], None
    codes = np.ascontiguousarray([ACT_CODES[a] for a in act], dtype=np.int32)
    if codes.shape != (h,):
        raise ValueError("one activation per head expected")
    return int(codes[0]), codes


def fwd(q, k, v, q_offsets, kv_offsets, *, act, scale: float, g=None,
        window=(-1, -1), shared_q: bool = False, nthreads: int = 0, lib=None) -> Dict[str, np.ndarray]:
    """Forward of the plain definition. Arrays: q [Tq,H,d], k/v [Tk,H,d], g [Tk,H] or None.
    act: an activation name, or a list with one name per head. shared_q: q is one [S,H,d] query
    matrix whose row i is query row i of every sequence (o and lse still have Tq rows)."""
    lib = lib or load()
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    qo = np.ascontiguousarray(q_offsets, dtype=np.int64)
    ko = np.ascontiguousarray(kv_offsets, dtype=np.int64)
    _, h, d = q.shape
    tq = int(qo[-1])
    code, heads = _acts(act, h)
    o = np.zeros((tq, h, d), dtype=np.float64)
    lse = np.zeros((tq, h), dtype=np.float64)
    rc = lib.gdpa_oracle_fwd(len(qo) - 1, h, d, _ptr(qo), _ptr(ko), _ptr(q), _ptr(k), _ptr(v),
                             _ptr(g), code, float(scale), int(window[0]),
                             int(window[1]), _ptr(o), _ptr(lse), int(nthreads), _ptr(heads),
                             q.shape[0] if shared_q else 0)
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    out = {"o": o}
    if (act == "softmax") if isinstance(act, str) else ("softmax" in act):
        out["lse"] = lse  # rows of non-softmax heads hold 0
    return out


def bwd(q, k, v, dout, q_offsets, kv_offsets, *, act, scale: float, g=None,
        window=(-1, -1), want_dg: bool = False, shared_q: bool = False, nthreads: int = 0,
        lib=None) -> Dict[str, np.ndarray]:
    """Gradients of sum(dout * o) with respect to q, k, v (and the gate G if want_dg); with
    shared_q, dq is the [S,H,d] gradient of the shared query matrix."""
    lib = lib or load()
    q, k, v, g, dout = _f64(q), _f64(k), _f64(v), _f64(g), _f64(dout)
    qo = np.ascontiguousarray(q_offsets, dtype=np.int64)
    ko = np.ascontiguousarray(kv_offsets, dtype=np.int64)
    tq, h, d = q.shape
    code, heads = _acts(act, h)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dg = np.zeros((k.shape[0], h), dtype=np.float64) if (want_dg and g is not None) else None
    rc = lib.gdpa_oracle_bwd(len(qo) - 1, h, d, _ptr(qo), _ptr(ko), _ptr(q), _ptr(k), _ptr(v),
                             _ptr(g), code, float(scale), int(window[0]),
                             int(window[1]), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg),
                             int(nthreads), _ptr(heads), q.shape[0] if shared_q else 0)
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    out = {"dq": dq, "dk": dk, "dv": dv}
    if dg is not None:
        out["dg"] = dg
    return out


def group_fwd(group, nthreads: int = 0, **overrides):
    """Forward on a ``gdpa_workloads.Group`` (inputs widened exactly to float64)."""
    from gdpa_workloads import widen
    s = group.spec
    kw = dict(act=s.act, scale=s.scale, window=s.window, shared_q=getattr(s, "shared_q", False))
    kw.update(overrides)
    return fwd(widen(group.q), widen(group.k), widen(group.v), group.q_offsets, group.kv_offsets,
               g=widen(group.g), nthreads=nthreads, **kw)


def group_bwd(group, nthreads: int = 0, want_dg: bool = False, **overrides):
    from gdpa_workloads import widen
    s = group.spec
    kw = dict(act=s.act, scale=s.scale, window=s.window, shared_q=getattr(s, "shared_q", False))
    kw.update(overrides)
    return bwd(widen(group.q), widen(group.k), widen(group.v), widen(group.dout), group.q_offsets,
               group.kv_offsets, g=widen(group.g), want_dg=want_dg, nthreads=nthreads, **kw)
