"""Oracle for weighted sparse message passing -- TEST INFRASTRUCTURE ONLY.

A thin numpy/ctypes wrapper over ``oracle.c``, the plain fp64 CPU edge loop
written from the pages (tinymesh "Weighted aggregation experiment": "Decision",
"Edge order is explicit", "Exact witness").  Only the test suite, the smoke
check and the CPU-baseline leg of the benchmark may import this package; the
library under test never does, and the two share no code.

Every function takes plain numpy arrays.  Index arrays are widened to int64,
float inputs must already hold the exact values the device sees (bf16 features
widened to float32 by the caller), and float results come back in float64
together with ``S``, the per-element sum of |term| the parity tolerance is
measured against.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into oracle/liboracle.so (plain -O2, no SIMD flags)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"],
                       check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _bind(lib):
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    sig = {
        "oracle_lower": (ctypes.c_int, [i64, i64, vp, vp, vp, vp, vp]),
        "oracle_forward": (None, [i64, i64, i64, vp, vp, vp, vp, vp, vp]),
        "oracle_input_grad": (None, [i64, i64, i64, vp, vp, vp, vp, vp, vp]),
        "oracle_edge_grad": (None, [i64, i64, vp, vp, vp, vp, vp, vp]),
        "oracle_forward_rows": (ctypes.c_int, [i64, i64, i64, vp, vp, vp, vp, i64, vp, vp, vp]),
        "oracle_input_grad_rows": (ctypes.c_int, [i64, i64, i64, vp, vp, vp, vp, i64, vp, vp, vp]),
        "oracle_edge_grad_edges": (None, [i64, i64, vp, vp, vp, vp, vp, vp, vp]),
        "oracle_degree_plan": (None, [i64, vp, vp, vp]),
        "oracle_edge_softmax": (None, [i64, i64, vp, vp, vp, vp, vp]),
        "oracle_edge_softmax_backward": (None, [i64, i64, vp, vp, vp, vp, vp, vp]),
        "oracle_edge_normalize": (ctypes.c_int, [i64, i64, vp, vp, ctypes.c_int, vp, vp]),
        "oracle_forward_heads": (ctypes.c_int, [i64, i64, i64, i64, vp, vp, vp, vp, i64, vp,
                                                vp, vp]),
        "oracle_input_grad_heads": (ctypes.c_int, [i64, i64, i64, i64, vp, vp, vp, vp, i64, vp,
                                                   vp, vp]),
        "oracle_edge_grad_heads": (ctypes.c_int, [i64, i64, i64, vp, vp, vp, vp, i64, vp, vp,
                                                  vp]),
        "oracle_edge_softmax_heads": (None, [i64, i64, i64, vp, vp, vp, vp, vp]),
        "oracle_edge_softmax_backward_heads": (None, [i64, i64, i64, vp, vp, vp, vp, vp, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


@contextlib.contextmanager
def using_library(path: str):
    """Route every call to another build of oracle.c for the duration (used by
    the mutation tests, which build deliberately broken copies)."""
    global _lib
    saved = _lib
    _lib = _bind(ctypes.CDLL(path))
    try:
        yield
    finally:
        _lib = saved


def _i64(a):
    return np.ascontiguousarray(np.asarray(a), dtype=np.int64)


def _f32(a):
    a = np.asarray(a)
    if a.dtype != np.float32:
        raise TypeError("oracle float inputs must be float32 (exact device values)")
    return np.ascontiguousarray(a)


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def lower(n: int, key, other):
    """Stable COO->CSR keyed on ``key``: returns (rowptr[n+1], col[e], order[e]), int64.

    Forward lowering: ``lower(n, dst, src)`` -> (rowptr, col, edge_order).
    Transpose lowering: ``lower(n, src, dst)`` -> (rowptr_t, col_t, transpose_order).
    """
    key, other = _i64(key), _i64(other)
    e = key.shape[0]
    rowptr = np.empty(n + 1, np.int64)
    col = np.empty(e, np.int64)
    order = np.empty(e, np.int64)
    rc = _load().oracle_lower(n, e, _p(key), _p(other), _p(rowptr), _p(col), _p(order))
    if rc == -1:
        raise IndexError("edge index outside [0, n)")
    if rc != 0:
        raise MemoryError("oracle_lower")
    return rowptr, col, order


def forward(n: int, src, dst, w, x):
    """Y = A_w X and its scale S, both float64 [n, h]."""
    src, dst, w, x = _i64(src), _i64(dst), _f32(w), _f32(x)
    h = x.shape[1]
    y = np.empty((n, h), np.float64)
    s = np.empty((n, h), np.float64)
    _load().oracle_forward(n, src.shape[0], h, _p(src), _p(dst), _p(w), _p(x), _p(y), _p(s))
    return y, s


def input_grad(n: int, src, dst, w, dy):
    """dX = A_w^T dY and its scale S, both float64 [n, h]."""
    src, dst, w, dy = _i64(src), _i64(dst), _f32(w), _f32(dy)
    h = dy.shape[1]
    dx = np.empty((n, h), np.float64)
    s = np.empty((n, h), np.float64)
    _load().oracle_input_grad(n, src.shape[0], h, _p(src), _p(dst), _p(w), _p(dy), _p(dx), _p(s))
    return dx, s


def edge_grad(src, dst, x, dy):
    """dw_e = <X[src_e], dY[dst_e]> in COO order, and its scale S, float64 [e]."""
    src, dst, x, dy = _i64(src), _i64(dst), _f32(x), _f32(dy)
    e, h = src.shape[0], x.shape[1]
    dw = np.empty(e, np.float64)
    s = np.empty(e, np.float64)
    _load().oracle_edge_grad(e, h, _p(src), _p(dst), _p(x), _p(dy), _p(dw), _p(s))
    return dw, s


def forward_rows(n: int, src, dst, w, x, rows):
    """Rows ``rows`` of Y = A_w X (and S), without forming the whole output."""
    src, dst, w, x, rows = _i64(src), _i64(dst), _f32(w), _f32(x), _i64(rows)
    h = x.shape[1]
    y = np.empty((rows.shape[0], h), np.float64)
    s = np.empty_like(y)
    rc = _load().oracle_forward_rows(n, src.shape[0], h, _p(src), _p(dst), _p(w), _p(x),
                                     rows.shape[0], _p(rows), _p(y), _p(s))
    if rc != 0:
        raise MemoryError("oracle_forward_rows")
    return y, s


def input_grad_rows(n: int, src, dst, w, dy, rows):
    """Rows ``rows`` of dX = A_w^T dY (and S)."""
    src, dst, w, dy, rows = _i64(src), _i64(dst), _f32(w), _f32(dy), _i64(rows)
    h = dy.shape[1]
    dx = np.empty((rows.shape[0], h), np.float64)
    s = np.empty_like(dx)
    rc = _load().oracle_input_grad_rows(n, src.shape[0], h, _p(src), _p(dst), _p(w), _p(dy),
                                        rows.shape[0], _p(rows), _p(dx), _p(s))
    if rc != 0:
        raise MemoryError("oracle_input_grad_rows")
    return dx, s


def edge_grad_edges(src, dst, x, dy, edges):
    """dw for the COO ordinals ``edges`` only (and S)."""
    src, dst, x, dy, edges = _i64(src), _i64(dst), _f32(x), _f32(dy), _i64(edges)
    h = x.shape[1]
    dw = np.empty(edges.shape[0], np.float64)
    s = np.empty_like(dw)
    _load().oracle_edge_grad_edges(h, edges.shape[0], _p(edges), _p(src), _p(dst), _p(x),
                                   _p(dy), _p(dw), _p(s))
    return dw, s


def degree_plan(n: int, rowptr):
    """Rows listed by degree class (highest first, ascending id inside), and class counts[33]."""
    rowptr = _i64(rowptr)
    perm = np.empty(n, np.int64)
    counts = np.empty(33, np.int64)
    _load().oracle_degree_plan(n, _p(rowptr), _p(perm), _p(counts))
    return perm, counts


def edge_softmax(n: int, dst, s):
    """alpha_e = softmax of the scores over the incoming edges of dst_e (float64),
    plus the row maxima and row sums (-inf / 0 for rows without edges)."""
    dst, s = _i64(dst), _f32(s)
    e = dst.shape[0]
    alpha = np.empty(e, np.float64)
    rmax = np.empty(n, np.float64)
    rsum = np.empty(n, np.float64)
    _load().oracle_edge_softmax(n, e, _p(dst), _p(s), _p(alpha), _p(rmax), _p(rsum))
    return alpha, rmax, rsum


def edge_softmax_backward(n: int, dst, alpha, dalpha):
    """ds_e = alpha_e (dalpha_e - sum over the row of alpha * dalpha), with the row
    dots and the per-edge scale S (all float64).  alpha, dalpha: float32 inputs."""
    dst, alpha, dalpha = _i64(dst), _f32(alpha), _f32(dalpha)
    e = dst.shape[0]
    ds = np.empty(e, np.float64)
    rdot = np.empty(n, np.float64)
    scale = np.empty(e, np.float64)
    _load().oracle_edge_softmax_backward(n, e, _p(dst), _p(alpha), _p(dalpha), _p(ds),
                                         _p(rdot), _p(scale))
    return ds, rdot, scale


NORM_MEAN, NORM_SYM = 1, 2


def edge_normalize(n: int, src, dst, mode: int, values):
    """out_e = values_e / deg_in(dst_e) (mode 1) or / sqrt(deg_out(src_e) deg_in(dst_e))
    (mode 2), degrees being edge counts; float64."""
    src, dst, values = _i64(src), _i64(dst), _f32(values)
    out = np.empty(src.shape[0], np.float64)
    rc = _load().oracle_edge_normalize(n, src.shape[0], _p(src), _p(dst), int(mode), _p(values),
                                       _p(out))
    if rc != 0:
        raise ValueError(f"unknown normalisation mode {mode}")
    return out


def _heads_w(w, e):
    w = _f32(w)
    if w.ndim != 2 or w.shape[0] != e:
        raise ValueError("multi-head weights must be [e, k]")
    return np.ascontiguousarray(w), w.shape[1]


def _rows_arg(rows):
    if rows is None:
        return None, 0, None
    rows = _i64(rows)
    return rows, rows.shape[0], _p(rows)


def forward_heads(n: int, src, dst, w, x, rows=None):
    """Multi-head Y: w is [e, k] (one weight per edge and head), x is [n, h] with
    h = k * (h/k); head q of Y[i] sums w[e, q] * X[src_e] over head q's columns.
    ``rows`` restricts the output to those rows.  Returns (Y, S) in float64."""
    src, dst, x = _i64(src), _i64(dst), _f32(x)
    w, k = _heads_w(w, src.shape[0])
    h = x.shape[1]
    rows, nr, prow = _rows_arg(rows)
    y = np.empty((nr if rows is not None else n, h), np.float64)
    s = np.empty_like(y)
    rc = _load().oracle_forward_heads(n, src.shape[0], h, k, _p(src), _p(dst), _p(w), _p(x),
                                      nr, prow, _p(y), _p(s))
    if rc == -1:
        raise ValueError("feature width is not a multiple of the head count")
    if rc != 0:
        raise MemoryError("oracle_forward_heads")
    return y, s


def input_grad_heads(n: int, src, dst, w, dy, rows=None):
    """Multi-head dX (the transpose of forward_heads); (dX, S) in float64."""
    src, dst, dy = _i64(src), _i64(dst), _f32(dy)
    w, k = _heads_w(w, src.shape[0])
    h = dy.shape[1]
    rows, nr, prow = _rows_arg(rows)
    dx = np.empty((nr if rows is not None else n, h), np.float64)
    s = np.empty_like(dx)
    rc = _load().oracle_input_grad_heads(n, src.shape[0], h, k, _p(src), _p(dst), _p(w),
                                         _p(dy), nr, prow, _p(dx), _p(s))
    if rc == -1:
        raise ValueError("feature width is not a multiple of the head count")
    if rc != 0:
        raise MemoryError("oracle_input_grad_heads")
    return dx, s


def edge_grad_heads(src, dst, x, dy, k: int, edges=None):
    """Multi-head dw[e, q] = <X[src_e], dY[dst_e]> over head q's columns; [e, k]
    (or [len(edges), k]) float64, with S."""
    src, dst, x, dy = _i64(src), _i64(dst), _f32(x), _f32(dy)
    h = x.shape[1]
    edges, ne, pe = _rows_arg(edges)
    count = ne if edges is not None else src.shape[0]
    dw = np.empty((count, k), np.float64)
    s = np.empty_like(dw)
    rc = _load().oracle_edge_grad_heads(src.shape[0], h, k, _p(src), _p(dst), _p(x), _p(dy),
                                        ne, pe, _p(dw), _p(s))
    if rc == -1:
        raise ValueError("feature width is not a multiple of the head count")
    return dw, s


def edge_softmax_heads(n: int, dst, s):
    """Per-head target softmax of scores s [e, k]: alpha [e, k], row_max and
    row_sum [n, k] (float64)."""
    dst, s = _i64(dst), _f32(s)
    if s.ndim != 2 or s.shape[0] != dst.shape[0]:
        raise ValueError("multi-head scores must be [e, k]")
    s = np.ascontiguousarray(s)
    e, k = s.shape
    alpha = np.empty((e, k), np.float64)
    rmax = np.empty((n, k), np.float64)
    rsum = np.empty((n, k), np.float64)
    _load().oracle_edge_softmax_heads(n, e, k, _p(dst), _p(s), _p(alpha), _p(rmax), _p(rsum))
    return alpha, rmax, rsum


def edge_softmax_backward_heads(n: int, dst, alpha, dalpha):
    """Per-head backward: ds [e, k], row_dot [n, k] and the scale S [e, k] (float64)."""
    dst, alpha, dalpha = _i64(dst), _f32(alpha), _f32(dalpha)
    if alpha.ndim != 2 or alpha.shape != dalpha.shape or alpha.shape[0] != dst.shape[0]:
        raise ValueError("alpha and dalpha must be [e, k]")
    alpha, dalpha = np.ascontiguousarray(alpha), np.ascontiguousarray(dalpha)
    e, k = alpha.shape
    ds = np.empty((e, k), np.float64)
    rdot = np.empty((n, k), np.float64)
    scale = np.empty((e, k), np.float64)
    _load().oracle_edge_softmax_backward_heads(n, e, k, _p(dst), _p(alpha), _p(dalpha), _p(ds),
                                               _p(rdot), _p(scale))
    return ds, rdot, scale
