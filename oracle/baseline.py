"""All-cores CPU baseline for the benchmark -- BENCHMARK INFRASTRUCTURE ONLY.

ctypes wrapper over ``baseline_omp.c``: the oracle's definitions (stable
counting-sort lowering, the two aggregations, the edge gradient, fp64 with the
|term| sums) with one OpenMP loop over owners -- the rows of the oracle's own
CSR for the aggregations, the edges for the edge gradient.  Only the
benchmark's cpu_baseline leg uses it; no test checks against it, and the
checker (``oracle/__init__.py``) never loads it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "baseline_omp.c")
_LIB = os.path.join(_HERE, "libbaseline_omp.so")
_lib = None


def build(force: bool = True) -> str:
    """gcc -O2 -fopenmp baseline_omp.c -> oracle/libbaseline_omp.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-o", tmp,
                        _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        lib.baseline_threads.restype = ctypes.c_int
        lib.baseline_threads.argtypes = []
        lib.baseline_lower.restype = ctypes.c_int
        lib.baseline_lower.argtypes = [i64, i64, vp, vp, vp, vp, vp]
        lib.baseline_aggregate.restype = None
        lib.baseline_aggregate.argtypes = [i64, i64, vp, vp, vp, vp, vp, vp, vp]
        lib.baseline_edge_grad.restype = None
        lib.baseline_edge_grad.argtypes = [i64, i64, vp, vp, vp, vp, vp, vp]
        _lib = lib
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def threads() -> int:
    return int(_load().baseline_threads())


def run_path(n, src, dst, w, x, dy):
    """Lowering of both directions, forward, input gradient and edge gradient on
    all OpenMP threads; returns the wall seconds of each stage."""
    lib = _load()
    src = np.ascontiguousarray(src, dtype=np.int64)
    dst = np.ascontiguousarray(dst, dtype=np.int64)
    w, x, dy = (np.ascontiguousarray(a, dtype=np.float32) for a in (w, x, dy))
    e, h = src.shape[0], x.shape[1]
    secs = {}
    csr = []
    t0 = time.perf_counter()
    for key, other in ((dst, src), (src, dst)):
        rowptr = np.empty(n + 1, np.int64)
        col = np.empty(e, np.int64)
        order = np.empty(e, np.int64)
        if lib.baseline_lower(n, e, _p(key), _p(other), _p(rowptr), _p(col), _p(order)) != 0:
            raise IndexError("edge index outside [0, n)")
        csr.append((rowptr, col, order))
    secs["lowering"] = time.perf_counter() - t0
    out = np.empty((n, h), np.float64)
    s = np.empty((n, h), np.float64)
    for name, (rowptr, col, order), feats in (("forward", csr[0], x), ("input_grad", csr[1], dy)):
        t0 = time.perf_counter()
        lib.baseline_aggregate(n, h, _p(rowptr), _p(col), _p(order), _p(w), _p(feats), _p(out),
                               _p(s))
        secs[name] = time.perf_counter() - t0
    del out, s, csr
    dw = np.empty(e, np.float64)
    sdw = np.empty(e, np.float64)
    t0 = time.perf_counter()
    lib.baseline_edge_grad(e, h, _p(src), _p(dst), _p(x), _p(dy), _p(dw), _p(sdw))
    secs["edge_grad"] = time.perf_counter() - t0
    return secs
