"""Shared helpers for the GPU parity tests: upload a synthetic workload, run the
library's path through its Python binding (which calls the C ABI), and compare
with the oracle.

Comparison rules:
  * integer outputs (CSR arrays, order maps, degree plans): bit-exact;
  * float outputs: |gpu - oracle| <= tau * S elementwise, where S is the
    oracle's sum of |term| for that element; tau = 1e-5 for fp32 features and
    2e-2 for bf16 feature storage (fp32 accumulation in both cases); where
    S = 0 (no terms) the device value must be exactly zero.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle

TAU = {"f32": 1e-5, "bf16": 2e-2}


def device_features(a_bits, a_f32, feat_dtype, dev):
    if feat_dtype == "bf16":
        return torch.from_numpy(a_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(a_f32).to(dev)


def upload(wl, dev, idx_dtype=torch.int64):
    return {
        "src": torch.from_numpy(wl.src).to(dev).to(idx_dtype),
        "dst": torch.from_numpy(wl.dst).to(dev).to(idx_dtype),
        "w": torch.from_numpy(wl.w).to(dev),
        "x": device_features(wl.x_bits, wl.x, wl.feat_dtype, dev),
        "dy": device_features(wl.dy_bits, wl.dy, wl.feat_dtype, dev),
    }


def run_path(mp, wl, dev, idx_dtype=torch.int64):
    t = upload(wl, dev, idx_dtype)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    y = mp.mp_spmm_fwd(g, t["w"], t["x"])
    dx = mp.mp_spmm_dx(g, t["w"], t["dy"])
    dw = mp.mp_edge_grad_dw(g, t["x"], t["dy"])
    torch.cuda.synchronize()
    return g, t, y, dx, dw


def check_structure(g, wl):
    rowptr, col, order = oracle.lower(wl.n, wl.dst, wl.src)
    rowptr_t, col_t, order_t = oracle.lower(wl.n, wl.src, wl.dst)
    got = {k: g.arrays[k].cpu().numpy().astype(np.int64) for k in g.arrays}
    ref = {"src": wl.src, "dst": wl.dst, "rowptr": rowptr, "col": col, "edge_order": order,
           "rowptr_t": rowptr_t, "col_t": col_t, "transpose_order": order_t}
    plan, cc = oracle.degree_plan(wl.n, rowptr)
    plan_t, cc_t = oracle.degree_plan(wl.n, rowptr_t)
    ref["row_plan"], ref["row_plan_t"] = plan, plan_t
    for k, v in ref.items():
        assert got[k].shape == v.shape, (k, got[k].shape, v.shape)
        if not np.array_equal(got[k], v):
            bad = np.nonzero(got[k] != v)[0]
            raise AssertionError(f"{k} differs at {bad.size} positions, first {bad[:5]}: "
                                 f"gpu {got[k][bad[:5]]} oracle {v[bad[:5]]}")
    assert g.class_count == cc.tolist(), (g.class_count, cc.tolist())
    assert g.class_count_t == cc_t.tolist(), (g.class_count_t, cc_t.tolist())


def check_close(name, got, ref, s, tau):
    got = got.detach().cpu().numpy().astype(np.float64) if isinstance(got, torch.Tensor) else got
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    err = np.abs(got - ref)
    zero = s == 0
    if np.any(got[zero] != 0):
        raise AssertionError(f"{name}: {int(np.sum(got[zero] != 0))} elements with no terms are not 0")
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(zero, 0.0, err / np.where(zero, 1.0, s))
    worst = float(ratio.max()) if ratio.size else 0.0
    if worst > tau:
        i = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        raise AssertionError(f"{name}: max |err|/S = {worst:.3e} > {tau:g} at {i}: "
                             f"gpu {got[i]!r} oracle {ref[i]!r} S {s[i]!r}")
    return worst


def check_floats(wl, y, dx, dw, tau=None):
    tau = TAU[wl.feat_dtype] if tau is None else tau
    ry, sy = oracle.forward(wl.n, wl.src, wl.dst, wl.w, wl.x)
    rdx, sdx = oracle.input_grad(wl.n, wl.src, wl.dst, wl.w, wl.dy)
    rdw, sdw = oracle.edge_grad(wl.src, wl.dst, wl.x, wl.dy)
    return (check_close("Y", y, ry, sy, tau), check_close("dX", dx, rdx, sdx, tau),
            check_close("dw", dw, rdw, sdw, tau))


def oracle_threads() -> int:
    """Threads for oracle work: the host cores this process may use, at most 16."""
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return max(1, min(16, cores))


def ratios(got, ref, s):
    """|got - ref| / S elementwise (0 where S = 0), after checking that every
    element with no terms is exactly 0."""
    err = np.abs(got.astype(np.float64) - ref)
    zero = s == 0
    if np.any(got[zero] != 0):
        raise AssertionError(f"{int(np.sum(got[zero] != 0))} elements with no terms are not 0")
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.where(zero, 0.0, err / np.where(zero, 1.0, s))


def check_all_rows(name, got, n, rows_fn, taus, chunks=None):
    """Compare every row of `got` ([n, H], numpy) with the oracle, whose rows are
    evaluated by rows_fn(rows) -> (ref, S) in strided row sets on several threads
    (the oracle's C calls release the GIL; strided sets spread the long rows of
    skewed graphs).  Raises at the first bound exceeded; returns the worst
    |err|/S."""
    t = oracle_threads()
    c = chunks or 4 * t

    def one(i):
        rows = np.arange(i, n, c, dtype=np.int64)
        ref, s = rows_fn(rows)
        r = ratios(got[rows], ref, s)
        return float(r.max()) if r.size else 0.0, i

    with ThreadPoolExecutor(t) as ex:
        res = list(ex.map(one, range(c)))
    worst, at = max(res)
    for tau in taus:
        if worst > tau:
            raise AssertionError(f"{name}: max |err|/S = {worst:.3e} > {tau:g} (row set {at} of {c})")
    return worst


def check_all_edges(name, got, e, edges_fn, taus, chunks=None):
    """The same for an edge output ([E], numpy): edges_fn(lo, hi) -> (ref, S) for
    the COO range [lo, hi)."""
    t = oracle_threads()
    c = chunks or 4 * t
    bounds = np.linspace(0, e, c + 1).astype(np.int64)

    def one(i):
        lo, hi = int(bounds[i]), int(bounds[i + 1])
        if hi == lo:
            return 0.0, i
        ref, s = edges_fn(lo, hi)
        r = ratios(got[lo:hi], ref, s)
        return float(r.max()), i

    with ThreadPoolExecutor(t) as ex:
        res = list(ex.map(one, range(c)))
    worst, at = max(res)
    for tau in taus:
        if worst > tau:
            raise AssertionError(f"{name}: max |err|/S = {worst:.3e} > {tau:g} "
                                 f"(edges {bounds[at]}..{bounds[at + 1]})")
    return worst
