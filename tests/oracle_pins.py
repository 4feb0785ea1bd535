"""Pins for the oracle: checks against facts that do not come from the oracle.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
the pages, the mathematics, or an independent library routine:

* the printed witness result and the hand-worked witness values
  (tests/golden/witness.json; tinymesh "Weighted aggregation experiment",
  "Exact witness");
* dense brute force: A_w as a dense matrix, Y = A_w X and dX = A_w^T dY as
  numpy matrix products, dw as the dense product dY X^T sampled at each edge;
* scipy.sparse on mid-size graphs;
* numpy's stable argsort / bincount / cumsum for the lowering and the plan;
* closed-form laws: adjoint identity, COO permutation, duplicate merging,
  linearity in w, central differences of <dY, A_w X>, the one-node graph,
  exact zeros on empty rows.

They are plain functions so that tests/test_oracle_mutants.py can run the
same set against deliberately broken copies of the oracle.
"""
from __future__ import annotations

import json
import os

import numpy as np

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _witness():
    with open(os.path.join(GOLDEN, "witness.json")) as f:
        return json.load(f)


def _dense(n, src, dst, w):
    a = np.zeros((n, n), np.float64)
    np.add.at(a, (dst, src), w.astype(np.float64))
    return a


def _dense_abs(n, src, dst, w):
    a = np.zeros((n, n), np.float64)
    np.add.at(a, (dst, src), np.abs(w.astype(np.float64)))
    return a


def _tiny_graphs(count, seed):
    rng = np.random.default_rng(seed)
    for _ in range(count):
        n = int(rng.integers(1, 9))
        e = int(rng.integers(0, 25))
        h = int(rng.integers(1, 5))
        src = rng.integers(0, n, e)
        dst = rng.integers(0, n, e)
        w = rng.uniform(-2, 2, e).astype(np.float32)
        x = rng.standard_normal((n, h)).astype(np.float32)
        dy = rng.standard_normal((n, h)).astype(np.float32)
        yield n, src, dst, w, x, dy


# --------------------------------------------------------------------------- witness

def pin_witness_printed_edge_order():
    g = _witness()
    _, _, order = oracle.lower(g["n"], g["dst"], g["src"])
    assert order.tolist() == g["printed"]["edge_order"], order


def pin_witness_hand_values():
    g = _witness()
    hd = g["hand_derived"]
    n = g["n"]
    src, dst = np.array(g["src"]), np.array(g["dst"])
    w = np.array(g["w"], np.float32)
    x = np.array(g["x"], np.float32)[:, None]
    dy = np.array(g["dy"], np.float32)[:, None]
    y, _ = oracle.forward(n, src, dst, w, x)
    dx, _ = oracle.input_grad(n, src, dst, w, dy)
    dw, _ = oracle.edge_grad(src, dst, x, dy)
    assert y[:, 0].tolist() == hd["Y"], y
    assert dx[:, 0].tolist() == hd["dX"], dx
    assert dw.tolist() == hd["dw"], dw
    rowptr, col, order = oracle.lower(n, dst, src)
    assert rowptr.tolist() == hd["rowptr"] and col.tolist() == hd["col"]
    rowptr_t, col_t, order_t = oracle.lower(n, src, dst)
    assert rowptr_t.tolist() == hd["rowptr_t"] and col_t.tolist() == hd["col_t"]
    assert order_t.tolist() == hd["transpose_order"]


def pin_witness_adjoint():
    g = _witness()
    n = g["n"]
    src, dst = np.array(g["src"]), np.array(g["dst"])
    w = np.array(g["w"], np.float32)
    x = np.array(g["x"], np.float32)[:, None]
    dy = np.array(g["dy"], np.float32)[:, None]
    y, _ = oracle.forward(n, src, dst, w, x)
    dx, _ = oracle.input_grad(n, src, dst, w, dy)
    dw, _ = oracle.edge_grad(src, dst, x, dy)
    a = float((dy.astype(np.float64) * y).sum())
    b = float((x.astype(np.float64) * dx).sum())
    c = float((w.astype(np.float64) * dw).sum())
    assert a == b == c == g["hand_derived"]["adjoint"], (a, b, c)


# --------------------------------------------------------------------------- brute force

def pin_dense_bruteforce():
    """Y = A X, dX = A^T dY, dw_e = (dY X^T)[dst_e, src_e], S from |A| |X|."""
    for n, src, dst, w, x, dy in _tiny_graphs(400, 11):
        a = _dense(n, src, dst, w)
        aa = _dense_abs(n, src, dst, w)
        x64, dy64 = x.astype(np.float64), dy.astype(np.float64)
        y, sy = oracle.forward(n, src, dst, w, x)
        dx, sdx = oracle.input_grad(n, src, dst, w, dy)
        dw, sdw = oracle.edge_grad(src, dst, x, dy)
        np.testing.assert_allclose(y, a @ x64, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dx, a.T @ dy64, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(sy, aa @ np.abs(x64), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(sdx, aa.T @ np.abs(dy64), rtol=1e-12, atol=1e-12)
        g = dy64 @ x64.T
        ga = np.abs(dy64) @ np.abs(x64).T
        np.testing.assert_allclose(dw, g[dst, src] if len(src) else np.zeros(0),
                                   rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(sdw, ga[dst, src] if len(src) else np.zeros(0),
                                   rtol=1e-12, atol=1e-12)


def pin_scipy_midsize():
    import scipy.sparse as sp
    for seed, (n, e, h) in enumerate([(300, 5000, 7), (2000, 20000, 16), (50, 3000, 33)]):
        wl = synth.random_graph(n, e, h, 100 + seed)
        a = sp.coo_matrix((wl.w.astype(np.float64), (wl.dst, wl.src)), shape=(n, n)).tocsr()
        y, _ = oracle.forward(n, wl.src, wl.dst, wl.w, wl.x)
        dx, _ = oracle.input_grad(n, wl.src, wl.dst, wl.w, wl.dy)
        np.testing.assert_allclose(y, a @ wl.x.astype(np.float64), rtol=1e-10, atol=1e-10)
        np.testing.assert_allclose(dx, a.T @ wl.dy.astype(np.float64), rtol=1e-10, atol=1e-10)
        # SDDMM as scipy's elementwise product of the sampled dense product
        dw, _ = oracle.edge_grad(wl.src, wl.dst, wl.x, wl.dy)
        ref = np.einsum("eh,eh->e", wl.x[wl.src].astype(np.float64),
                        wl.dy[wl.dst].astype(np.float64))
        np.testing.assert_allclose(dw, ref, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------- structure

def _check_lowering(n, key, other):
    rowptr, col, order = oracle.lower(n, key, other)
    ref_order = np.argsort(key, kind="stable")
    assert np.array_equal(order, ref_order)
    ref_rowptr = np.concatenate([[0], np.cumsum(np.bincount(key, minlength=n))])
    assert np.array_equal(rowptr, ref_rowptr)
    assert np.array_equal(col, np.asarray(other)[ref_order])


def pin_structure_numpy():
    for n, src, dst, w, x, dy in _tiny_graphs(200, 12):
        _check_lowering(n, dst, src)
        _check_lowering(n, src, dst)
    for wl in (synth.tiny_uniform(), synth.random_graph(5000, 60000, 1, 9)):
        _check_lowering(wl.n, wl.dst, wl.src)
        _check_lowering(wl.n, wl.src, wl.dst)


def pin_structure_invariants():
    wl = synth.random_graph(700, 9000, 1, 21)
    for key, other in ((wl.dst, wl.src), (wl.src, wl.dst)):
        rowptr, col, order = oracle.lower(wl.n, key, other)
        assert np.array_equal(np.sort(order), np.arange(wl.e))        # a permutation
        assert rowptr[0] == 0 and rowptr[-1] == wl.e and np.all(np.diff(rowptr) >= 0)
        k = key[order]
        assert np.all(np.diff(k) >= 0)                                 # rows non-decreasing
        for i in range(wl.n):                                           # stable inside a row
            seg = order[rowptr[i]:rowptr[i + 1]]
            assert np.all(np.diff(seg) > 0)
            assert np.all(key[seg] == i)


def pin_out_of_range_rejected():
    try:
        oracle.lower(3, np.array([0, 3]), np.array([0, 0]))
    except IndexError:
        return
    raise AssertionError("index 3 with n=3 accepted")


# --------------------------------------------------------------------------- laws

def pin_permutation_law():
    wl = synth.random_graph(200, 3000, 5, 31)
    rng = np.random.default_rng(3)
    perm = rng.permutation(wl.e)
    y0, _ = oracle.forward(wl.n, wl.src, wl.dst, wl.w, wl.x)
    y1, _ = oracle.forward(wl.n, wl.src[perm], wl.dst[perm], wl.w[perm], wl.x)
    dx0, _ = oracle.input_grad(wl.n, wl.src, wl.dst, wl.w, wl.dy)
    dx1, _ = oracle.input_grad(wl.n, wl.src[perm], wl.dst[perm], wl.w[perm], wl.dy)
    dw0, _ = oracle.edge_grad(wl.src, wl.dst, wl.x, wl.dy)
    dw1, _ = oracle.edge_grad(wl.src[perm], wl.dst[perm], wl.x, wl.dy)
    np.testing.assert_allclose(y1, y0, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dx1, dx0, rtol=1e-12, atol=1e-12)
    assert np.array_equal(dw1, dw0[perm])
    # the lowering of a permuted COO list: same rows, maps renumbered through perm
    r0, c0, o0 = oracle.lower(wl.n, wl.dst, wl.src)
    r1, c1, o1 = oracle.lower(wl.n, wl.dst[perm], wl.src[perm])
    assert np.array_equal(r0, r1)
    for i in range(wl.n):
        a = sorted(zip(perm[o1[r1[i]:r1[i + 1]]].tolist(), c1[r1[i]:r1[i + 1]].tolist()))
        b = sorted(zip(o0[r0[i]:r0[i + 1]].tolist(), c0[r0[i]:r0[i + 1]].tolist()))
        assert a == b


def pin_duplicate_law():
    """(s, t, w1) and (s, t, w2) act on Y and dX as one edge of weight w1 + w2,
    keep separate positions, and each gets the same dw."""
    src = np.array([0, 1, 1, 2, 1])
    dst = np.array([1, 2, 2, 0, 2])
    w = np.array([0.5, 0.25, -1.5, 2.0, 0.75], np.float32)
    x = np.array([[1.0, -2.0], [3.0, 0.5], [-1.0, 4.0]], np.float32)
    dy = np.array([[2.0, 1.0], [-0.5, 3.0], [1.5, -1.0]], np.float32)
    y, _ = oracle.forward(3, src, dst, w, x)
    msrc, mdst = np.array([0, 1, 2]), np.array([1, 2, 0])
    mw = np.array([0.5, 0.25 - 1.5 + 0.75, 2.0], np.float32)
    ym, _ = oracle.forward(3, msrc, mdst, mw, x)
    np.testing.assert_allclose(y, ym, rtol=1e-12, atol=1e-12)
    dx, _ = oracle.input_grad(3, src, dst, w, dy)
    dxm, _ = oracle.input_grad(3, msrc, mdst, mw, dy)
    np.testing.assert_allclose(dx, dxm, rtol=1e-12, atol=1e-12)
    dw, _ = oracle.edge_grad(src, dst, x, dy)
    assert dw[1] == dw[2] == dw[4]
    rowptr, col, order = oracle.lower(3, dst, src)
    assert order[rowptr[2]:rowptr[3]].tolist() == [1, 2, 4]          # separate positions


def pin_linearity():
    wl = synth.random_graph(100, 1500, 3, 41)
    rng = np.random.default_rng(4)
    w2 = rng.uniform(-1, 1, wl.e).astype(np.float32)
    a, b = 0.5, -2.0                                  # exact scalings in binary
    wsum = (a * wl.w + b * w2).astype(np.float32)
    y1, _ = oracle.forward(wl.n, wl.src, wl.dst, wl.w, wl.x)
    y2, _ = oracle.forward(wl.n, wl.src, wl.dst, w2, wl.x)
    ys, _ = oracle.forward(wl.n, wl.src, wl.dst, wsum, wl.x)
    np.testing.assert_allclose(ys, a * y1 + b * y2, rtol=1e-6, atol=1e-6)
    dx1, _ = oracle.input_grad(wl.n, wl.src, wl.dst, wl.w, wl.dy)
    dx2, _ = oracle.input_grad(wl.n, wl.src, wl.dst, w2, wl.dy)
    dxs, _ = oracle.input_grad(wl.n, wl.src, wl.dst, wsum, wl.dy)
    np.testing.assert_allclose(dxs, a * dx1 + b * dx2, rtol=1e-6, atol=1e-6)


def pin_gradients_central_difference():
    """f(w, X) = <dY, A_w X> is linear in w and in X, so central differences
    recover dw = df/dw and dX = df/dX up to rounding."""
    wl = synth.random_graph(12, 40, 3, 51)
    dy64 = wl.dy.astype(np.float64)

    def f(w, x):
        y, _ = oracle.forward(wl.n, wl.src, wl.dst, w, x)
        return float((dy64 * y).sum())

    dw, _ = oracle.edge_grad(wl.src, wl.dst, wl.x, wl.dy)
    step = np.float32(0.25)
    for j in range(wl.e):
        wp, wm = wl.w.copy(), wl.w.copy()
        wp[j] += step
        wm[j] -= step
        fd = (f(wp, wl.x) - f(wm, wl.x)) / (float(wp[j]) - float(wm[j]))
        assert abs(fd - dw[j]) <= 1e-9 * (1 + abs(dw[j])), (j, fd, dw[j])
    dx, _ = oracle.input_grad(wl.n, wl.src, wl.dst, wl.w, wl.dy)
    for i in range(wl.n):
        for k in range(wl.h):
            xp, xm = wl.x.copy(), wl.x.copy()
            xp[i, k] += step
            xm[i, k] -= step
            fd = (f(wl.w, xp) - f(wl.w, xm)) / (float(xp[i, k]) - float(xm[i, k]))
            assert abs(fd - dx[i, k]) <= 1e-9 * (1 + abs(dx[i, k])), (i, k, fd, dx[i, k])


def pin_one_node():
    e0 = np.zeros(0, np.int64)
    x = np.array([[1.5, -2.0, 0.25]], np.float32)
    y, s = oracle.forward(1, e0, e0, np.zeros(0, np.float32), x)
    dx, _ = oracle.input_grad(1, e0, e0, np.zeros(0, np.float32), x)
    dw, _ = oracle.edge_grad(e0, e0, x, x)
    assert np.all(y == 0) and np.all(s == 0) and np.all(dx == 0) and dw.shape == (0,)
    rowptr, col, order = oracle.lower(1, e0, e0)
    assert rowptr.tolist() == [0, 0] and col.shape == (0,) and order.shape == (0,)
    loops = np.zeros(4, np.int64)
    w = np.array([0.5, -1.0, 2.0, 0.25], np.float32)
    y, _ = oracle.forward(1, loops, loops, w, x)
    np.testing.assert_allclose(y, float(w.astype(np.float64).sum()) * x.astype(np.float64),
                               rtol=1e-12)
    dw, _ = oracle.edge_grad(loops, loops, x, x)
    np.testing.assert_allclose(dw, np.full(4, float((x.astype(np.float64) ** 2).sum())))


def pin_empty_rows_exact_zero():
    wl = synth.random_graph(500, 300, 4, 61)          # most rows empty in both directions
    y, sy = oracle.forward(wl.n, wl.src, wl.dst, wl.w, wl.x)
    dx, sdx = oracle.input_grad(wl.n, wl.src, wl.dst, wl.w, wl.dy)
    no_in = np.bincount(wl.dst, minlength=wl.n) == 0
    no_out = np.bincount(wl.src, minlength=wl.n) == 0
    assert no_in.sum() > 100 and no_out.sum() > 100
    assert np.all(y[no_in] == 0) and np.all(sy[no_in] == 0)
    assert np.all(dx[no_out] == 0) and np.all(sdx[no_out] == 0)
    assert np.all(sy[~no_in] > 0) and np.all(np.abs(y) <= sy)


def pin_sampled_rows_match_full():
    wl = synth.random_graph(400, 6000, 6, 71)
    rows = np.array([0, 399, 17, 250, 3], np.int64)
    y, sy = oracle.forward(wl.n, wl.src, wl.dst, wl.w, wl.x)
    yr, syr = oracle.forward_rows(wl.n, wl.src, wl.dst, wl.w, wl.x, rows)
    assert np.array_equal(yr, y[rows]) and np.array_equal(syr, sy[rows])
    dx, sdx = oracle.input_grad(wl.n, wl.src, wl.dst, wl.w, wl.dy)
    dxr, sdxr = oracle.input_grad_rows(wl.n, wl.src, wl.dst, wl.w, wl.dy, rows)
    assert np.array_equal(dxr, dx[rows]) and np.array_equal(sdxr, sdx[rows])
    dw, sdw = oracle.edge_grad(wl.src, wl.dst, wl.x, wl.dy)
    edges = np.array([5, 0, 5999, 1234], np.int64)
    dwe, sdwe = oracle.edge_grad_edges(wl.src, wl.dst, wl.x, wl.dy, edges)
    assert np.array_equal(dwe, dw[edges]) and np.array_equal(sdwe, sdw[edges])


def pin_degree_plan_numpy():
    """Classes by Python's int.bit_length; plan = numpy stable argsort of -class."""
    for wl in (synth.witness(), synth.tiny_uniform(), synth.random_graph(3000, 2000, 1, 81),
               synth.rmat(10, 16, 82, 1)):
        for key, other in ((wl.dst, wl.src), (wl.src, wl.dst)):
            rowptr, _, _ = oracle.lower(wl.n, key, other)
            perm, counts = oracle.degree_plan(wl.n, rowptr)
            deg = np.diff(rowptr)
            cls = np.array([int(d).bit_length() for d in deg], np.int64)
            assert np.array_equal(counts, np.bincount(cls, minlength=33))
            assert np.array_equal(perm, np.argsort(-cls, kind="stable"))


# --------------------------------------------------------------------------- target softmax

def _segments(dst):
    """Edge ids of each destination, in COO order."""
    order = np.argsort(dst, kind="stable")
    bounds = np.concatenate([[0], np.cumsum(np.bincount(dst))])
    return order, bounds


def pin_softmax_scipy_segments():
    from scipy.special import softmax
    for seed, (n, e) in enumerate([(50, 400), (300, 3000), (7, 60)]):
        rng = np.random.default_rng(200 + seed)
        dst = rng.integers(0, n, e)
        s = (rng.standard_normal(e) * 3).astype(np.float32)
        alpha, rmax, rsum = oracle.edge_softmax(n, dst, s)
        order, bounds = _segments(dst)
        for i in range(n):
            ids = order[bounds[i]:bounds[i + 1]]
            if ids.size == 0:
                assert rmax[i] == -np.inf and rsum[i] == 0
                continue
            np.testing.assert_allclose(alpha[ids], softmax(s[ids].astype(np.float64)),
                                       rtol=1e-12, atol=1e-15)
            assert rmax[i] == s[ids].max()
            np.testing.assert_allclose(np.log(rsum[i]) + rmax[i],
                                       np.log(np.exp(s[ids].astype(np.float64)).sum()),
                                       rtol=1e-12)


def pin_softmax_laws():
    rng = np.random.default_rng(211)
    n, e = 120, 2000
    dst = rng.integers(0, n, e)
    s = rng.standard_normal(e).astype(np.float32)
    alpha, _, _ = oracle.edge_softmax(n, dst, s)
    assert np.all(alpha > 0)
    sums = np.bincount(dst, weights=alpha, minlength=n)
    has = np.bincount(dst, minlength=n) > 0
    np.testing.assert_allclose(sums[has], 1.0, rtol=1e-12)
    # equal scores -> 1/deg
    a_eq, _, _ = oracle.edge_softmax(n, dst, np.full(e, 0.75, np.float32))
    np.testing.assert_allclose(a_eq, 1.0 / np.bincount(dst, minlength=n)[dst], rtol=1e-12)
    # a constant per destination row changes nothing (scores on a 2^-10 grid and
    # shifts on a 2^-4 grid, so every shifted score is exact in fp32)
    sg = (rng.integers(-4096, 4096, e) / 1024.0).astype(np.float32)
    shift = (rng.integers(-64, 64, n) / 16.0).astype(np.float32)
    a_g, _, _ = oracle.edge_softmax(n, dst, sg)
    a_sh, _, _ = oracle.edge_softmax(n, dst, (sg + shift[dst]).astype(np.float32))
    np.testing.assert_allclose(a_sh, a_g, rtol=1e-12)
    # large scores stay finite (the row maximum is subtracted)
    a_big, _, _ = oracle.edge_softmax(n, dst, (s + 1000.0).astype(np.float32))
    assert np.all(np.isfinite(a_big))
    np.testing.assert_allclose(np.bincount(dst, weights=a_big, minlength=n)[has], 1.0, rtol=1e-12)


def pin_softmax_backward_jacobian():
    """ds = J dalpha with the explicit per-row Jacobian J = diag(a) - a a^T."""
    rng = np.random.default_rng(221)
    n, e = 40, 500
    dst = rng.integers(0, n, e)
    alpha = rng.uniform(0.01, 1, e).astype(np.float32)      # any positive values
    dalpha = rng.standard_normal(e).astype(np.float32)
    ds, rdot, scale = oracle.edge_softmax_backward(n, dst, alpha, dalpha)
    order, bounds = _segments(dst)
    a64, d64 = alpha.astype(np.float64), dalpha.astype(np.float64)
    for i in range(n):
        ids = order[bounds[i]:bounds[i + 1]]
        if ids.size == 0:
            assert rdot[i] == 0
            continue
        jac = np.diag(a64[ids]) - np.outer(a64[ids], a64[ids])
        np.testing.assert_allclose(ds[ids], jac @ d64[ids], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(rdot[i], a64[ids] @ d64[ids], rtol=1e-12, atol=1e-14)
    assert np.all(scale >= np.abs(ds) * (1 - 1e-12))


def pin_softmax_backward_central_difference():
    """f(s) = sum_e c_e alpha_e(s): central differences equal the backward with dalpha = c."""
    rng = np.random.default_rng(231)
    n, e = 9, 40
    dst = rng.integers(0, n, e)
    s = rng.standard_normal(e).astype(np.float32)
    c = rng.standard_normal(e)
    alpha, _, _ = oracle.edge_softmax(n, dst, s)
    ds, _, _ = oracle.edge_softmax_backward(n, dst, alpha.astype(np.float32),
                                            c.astype(np.float32))
    for j in range(e):
        sp, sm = s.copy(), s.copy()
        sp[j] += np.float32(1e-2)
        sm[j] -= np.float32(1e-2)
        fp = float(c @ oracle.edge_softmax(n, dst, sp)[0])
        fm = float(c @ oracle.edge_softmax(n, dst, sm)[0])
        fd = (fp - fm) / (float(sp[j]) - float(sm[j]))
        assert abs(fd - ds[j]) <= 2e-4 * (1 + abs(ds[j])), (j, fd, ds[j])


def pin_attention_layer_gradient():
    """Y = A_alpha(s) X with alpha the target softmax of s: d<dY, Y>/ds by central
    differences equals softmax_backward(alpha, edge_grad(X, dY))."""
    wl = synth.random_graph(10, 45, 3, 241)
    s = wl.w
    dy64 = wl.dy.astype(np.float64)

    def f(scores):
        a, _, _ = oracle.edge_softmax(wl.n, wl.dst, scores)
        y, _ = oracle.forward(wl.n, wl.src, wl.dst, a.astype(np.float32), wl.x)
        return float((dy64 * y).sum())

    alpha, _, _ = oracle.edge_softmax(wl.n, wl.dst, s)
    dalpha, _ = oracle.edge_grad(wl.src, wl.dst, wl.x, wl.dy)
    ds, _, _ = oracle.edge_softmax_backward(wl.n, wl.dst, alpha.astype(np.float32),
                                            dalpha.astype(np.float32))
    for j in range(wl.e):
        sp, sm = s.copy(), s.copy()
        sp[j] += np.float32(1e-2)
        sm[j] -= np.float32(1e-2)
        fd = (f(sp) - f(sm)) / (float(sp[j]) - float(sm[j]))
        assert abs(fd - ds[j]) <= 1e-3 * (1 + abs(ds[j])), (j, fd, ds[j])


# --------------------------------------------------------------------------- degree normalisation

def pin_normalize_dense():
    """Dense forms: mean = D_in^-1 A, symmetric = D_in^-1/2 A D_out^-1/2, with
    D from the edge counts (row and column sums of the unweighted A)."""
    for n, src, dst, w, x, dy in _tiny_graphs(300, 251):
        if len(src) == 0:
            continue
        ones = np.zeros((n, n))
        np.add.at(ones, (dst, src), 1.0)
        din, dout = ones.sum(axis=1), ones.sum(axis=0)
        a = _dense(n, src, dst, w)
        wm = oracle.edge_normalize(n, src, dst, oracle.NORM_MEAN, w)
        ws = oracle.edge_normalize(n, src, dst, oracle.NORM_SYM, w)
        am = _dense(n, src, dst, wm)
        asym = _dense(n, src, dst, ws)
        with np.errstate(divide="ignore"):
            rin = np.where(din > 0, 1.0 / din, 0.0)
            rsin = np.where(din > 0, din ** -0.5, 0.0)
            rsout = np.where(dout > 0, dout ** -0.5, 0.0)
        np.testing.assert_allclose(am, rin[:, None] * a, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(asym, rsin[:, None] * a * rsout[None, :], rtol=1e-12,
                                   atol=1e-14)


def pin_normalize_laws():
    wl = synth.random_graph(400, 6000, 1, 261)
    ones = np.ones(wl.e, np.float32)
    mean = oracle.edge_normalize(wl.n, wl.src, wl.dst, oracle.NORM_MEAN, ones)
    sums = np.bincount(wl.dst, weights=mean, minlength=wl.n)
    has = np.bincount(wl.dst, minlength=wl.n) > 0
    np.testing.assert_allclose(sums[has], 1.0, rtol=1e-12)             # mean rows sum to 1
    # symmetric normalisation of an undirected graph (each edge in both directions)
    # is a symmetric matrix whose spectral radius is 1 for a connected graph
    src = np.concatenate([wl.src, wl.dst])
    dst = np.concatenate([wl.dst, wl.src])
    sym = oracle.edge_normalize(wl.n, src, dst, oracle.NORM_SYM, np.ones(src.shape[0], np.float32))
    a = _dense(wl.n, src, dst, sym)
    assert np.allclose(a, a.T, atol=1e-14)
    ev = np.linalg.eigvalsh(a)
    assert abs(max(abs(ev.max()), abs(ev.min())) - 1.0) < 1e-9
    try:
        oracle.edge_normalize(wl.n, wl.src, wl.dst, 7, ones)
    except ValueError:
        return
    raise AssertionError("mode 7 accepted")


def pin_normalized_layer_gradient():
    """f(w) = <dY, A_norm(w) X>: central differences in w equal normalize(edge_grad)."""
    wl = synth.random_graph(11, 50, 3, 271)
    dy64 = wl.dy.astype(np.float64)
    for mode in (oracle.NORM_MEAN, oracle.NORM_SYM):
        def f(w):
            wn = oracle.edge_normalize(wl.n, wl.src, wl.dst, mode, w).astype(np.float32)
            y, _ = oracle.forward(wl.n, wl.src, wl.dst, wn, wl.x)
            return float((dy64 * y).sum())
        dwp, _ = oracle.edge_grad(wl.src, wl.dst, wl.x, wl.dy)
        dw = oracle.edge_normalize(wl.n, wl.src, wl.dst, mode, dwp.astype(np.float32))
        for j in range(wl.e):
            wp, wm = wl.w.copy(), wl.w.copy()
            wp[j] += np.float32(0.25)
            wm[j] -= np.float32(0.25)
            fd = (f(wp) - f(wm)) / (float(wp[j]) - float(wm[j]))
            assert abs(fd - dw[j]) <= 1e-5 * (1 + abs(dw[j])), (mode, j, fd, dw[j])


# --------------------------------------------------------------------------- multi-head weights

def _tiny_head_graphs(count, seed):
    rng = np.random.default_rng(seed)
    for _ in range(count):
        n = int(rng.integers(1, 8))
        e = int(rng.integers(0, 20))
        k = int(rng.integers(1, 5))
        hh = int(rng.integers(1, 4))
        src = rng.integers(0, n, e)
        dst = rng.integers(0, n, e)
        w = rng.uniform(-2, 2, (e, k)).astype(np.float32)
        x = rng.standard_normal((n, k * hh)).astype(np.float32)
        dy = rng.standard_normal((n, k * hh)).astype(np.float32)
        yield n, src, dst, w, x, dy, k, hh


def pin_heads_dense_bruteforce():
    """Head q: Y_q = A_q X_q, dX_q = A_q^T dY_q, dw[e, q] = (dY_q X_q^T)[dst_e, src_e],
    with A_q the dense matrix of the weights w[:, q] and X_q the head's columns."""
    for n, src, dst, w, x, dy, k, hh in _tiny_head_graphs(400, 301):
        y, sy = oracle.forward_heads(n, src, dst, w, x)
        dx, sdx = oracle.input_grad_heads(n, src, dst, w, dy)
        dw, sdw = oracle.edge_grad_heads(src, dst, x, dy, k)
        assert dw.shape == (len(src), k)
        for q in range(k):
            cols = slice(q * hh, (q + 1) * hh)
            a = _dense(n, src, dst, w[:, q])
            aa = _dense_abs(n, src, dst, w[:, q])
            xq, dyq = x[:, cols].astype(np.float64), dy[:, cols].astype(np.float64)
            np.testing.assert_allclose(y[:, cols], a @ xq, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(dx[:, cols], a.T @ dyq, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(sy[:, cols], aa @ np.abs(xq), rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(sdx[:, cols], aa.T @ np.abs(dyq), rtol=1e-12, atol=1e-12)
            g = dyq @ xq.T
            ga = np.abs(dyq) @ np.abs(xq).T
            if len(src):
                np.testing.assert_allclose(dw[:, q], g[dst, src], rtol=1e-12, atol=1e-12)
                np.testing.assert_allclose(sdw[:, q], ga[dst, src], rtol=1e-12, atol=1e-12)


def pin_heads_scipy_midsize():
    import scipy.sparse as sp
    for seed, (n, e, k, hh) in enumerate([(300, 4000, 4, 8), (1000, 9000, 3, 5)]):
        wl = synth.random_graph(n, e, k * hh, 310 + seed)
        w = np.random.default_rng(seed).standard_normal((e, k)).astype(np.float32)
        y, _ = oracle.forward_heads(n, wl.src, wl.dst, w, wl.x)
        dx, _ = oracle.input_grad_heads(n, wl.src, wl.dst, w, wl.dy)
        dw, _ = oracle.edge_grad_heads(wl.src, wl.dst, wl.x, wl.dy, k)
        for q in range(k):
            cols = slice(q * hh, (q + 1) * hh)
            a = sp.coo_matrix((w[:, q].astype(np.float64), (wl.dst, wl.src)), shape=(n, n)).tocsr()
            np.testing.assert_allclose(y[:, cols], a @ wl.x[:, cols].astype(np.float64),
                                       rtol=1e-10, atol=1e-10)
            np.testing.assert_allclose(dx[:, cols], a.T @ wl.dy[:, cols].astype(np.float64),
                                       rtol=1e-10, atol=1e-10)
            ref = np.einsum("eh,eh->e", wl.x[wl.src][:, cols].astype(np.float64),
                            wl.dy[wl.dst][:, cols].astype(np.float64))
            np.testing.assert_allclose(dw[:, q], ref, rtol=1e-12, atol=1e-12)


def pin_heads_laws():
    """Adjoint identity <dY, Y> = <X, dX> = sum w * dw; the per-head edge gradients
    add up to the single-head one; equal weights in every head give the scalar
    aggregation; central differences in w[e, q] (the function is linear in w)."""
    wl = synth.random_graph(40, 300, 12, 321)
    k = 4
    w = np.random.default_rng(5).standard_normal((wl.e, k)).astype(np.float32)
    y, _ = oracle.forward_heads(wl.n, wl.src, wl.dst, w, wl.x)
    dx, _ = oracle.input_grad_heads(wl.n, wl.src, wl.dst, w, wl.dy)
    dw, _ = oracle.edge_grad_heads(wl.src, wl.dst, wl.x, wl.dy, k)
    x64, dy64 = wl.x.astype(np.float64), wl.dy.astype(np.float64)
    a, b, c = (dy64 * y).sum(), (x64 * dx).sum(), (w.astype(np.float64) * dw).sum()
    np.testing.assert_allclose([b, c], [a, a], rtol=1e-11)
    dw1, _ = oracle.edge_grad(wl.src, wl.dst, wl.x, wl.dy)
    np.testing.assert_allclose(dw.sum(axis=1), dw1, rtol=1e-11, atol=1e-11)
    same = np.repeat(wl.w[:, None], k, axis=1)
    ys, _ = oracle.forward_heads(wl.n, wl.src, wl.dst, same, wl.x)
    y1, _ = oracle.forward(wl.n, wl.src, wl.dst, wl.w, wl.x)
    np.testing.assert_allclose(ys, y1, rtol=1e-12, atol=1e-12)
    small = synth.random_graph(6, 20, 6, 322)
    ws = np.random.default_rng(6).standard_normal((small.e, 3)).astype(np.float32)
    dws, _ = oracle.edge_grad_heads(small.src, small.dst, small.x, small.dy, 3)

    def f(wt):
        yy, _ = oracle.forward_heads(small.n, small.src, small.dst, wt, small.x)
        return float((small.dy.astype(np.float64) * yy).sum())
    for j in range(small.e):
        for q in range(3):
            wp, wm = ws.copy(), ws.copy()
            wp[j, q] += np.float32(0.5)
            wm[j, q] -= np.float32(0.5)
            fd = (f(wp) - f(wm)) / (float(wp[j, q]) - float(wm[j, q]))
            assert abs(fd - dws[j, q]) <= 1e-9 * (1 + abs(dws[j, q])), (j, q, fd, dws[j, q])


def pin_heads_samples_and_rejection():
    """Sampled rows / edges equal the full outputs; a width that is not a multiple
    of the head count is rejected."""
    wl = synth.random_graph(500, 6000, 16, 331)
    w = np.random.default_rng(7).standard_normal((wl.e, 2)).astype(np.float32)
    rows = np.array([0, 7, 499, 123, 250])
    y, sy = oracle.forward_heads(wl.n, wl.src, wl.dst, w, wl.x)
    yr, syr = oracle.forward_heads(wl.n, wl.src, wl.dst, w, wl.x, rows=rows)
    assert np.array_equal(yr, y[rows]) and np.array_equal(syr, sy[rows])
    dx, _ = oracle.input_grad_heads(wl.n, wl.src, wl.dst, w, wl.dy)
    dxr, _ = oracle.input_grad_heads(wl.n, wl.src, wl.dst, w, wl.dy, rows=rows)
    assert np.array_equal(dxr, dx[rows])
    dw, _ = oracle.edge_grad_heads(wl.src, wl.dst, wl.x, wl.dy, 2)
    edges = np.array([5, 0, 5999, 42])
    dwe, _ = oracle.edge_grad_heads(wl.src, wl.dst, wl.x, wl.dy, 2, edges=edges)
    assert np.array_equal(dwe, dw[edges])
    for call in (lambda: oracle.forward_heads(wl.n, wl.src, wl.dst,
                                              np.ones((wl.e, 3), np.float32), wl.x),
                 lambda: oracle.edge_grad_heads(wl.src, wl.dst, wl.x, wl.dy, 3)):
        try:
            call()
        except ValueError:
            continue
        raise AssertionError("width 16 accepted with 3 heads")


# --------------------------------------------------------------------------- multi-head softmax

def pin_softmax_heads_scipy_columns():
    """Every head's column is scipy's softmax over each destination segment, with
    its own row maximum and log-sum-exp."""
    from scipy.special import softmax
    for seed, (n, e, k) in enumerate([(40, 500, 3), (9, 70, 4), (200, 2500, 2)]):
        rng = np.random.default_rng(400 + seed)
        dst = rng.integers(0, n, e)
        sc = (rng.standard_normal((e, k)) * 3).astype(np.float32)
        alpha, rmax, rsum = oracle.edge_softmax_heads(n, dst, sc)
        order, bounds = _segments(dst)
        for i in range(n):
            ids = order[bounds[i]:bounds[i + 1]]
            for q in range(k):
                if ids.size == 0:
                    assert rmax[i, q] == -np.inf and rsum[i, q] == 0
                    continue
                col = sc[ids, q].astype(np.float64)
                np.testing.assert_allclose(alpha[ids, q], softmax(col), rtol=1e-12, atol=1e-15)
                assert rmax[i, q] == col.max()
                np.testing.assert_allclose(np.log(rsum[i, q]) + rmax[i, q],
                                           np.log(np.exp(col).sum()), rtol=1e-12)


def pin_softmax_heads_backward_jacobian():
    """Per head and row, ds = (diag(a) - a a^T) dalpha."""
    rng = np.random.default_rng(411)
    n, e, k = 30, 400, 3
    dst = rng.integers(0, n, e)
    alpha = rng.uniform(0.01, 1, (e, k)).astype(np.float32)
    dalpha = rng.standard_normal((e, k)).astype(np.float32)
    ds, rdot, scale = oracle.edge_softmax_backward_heads(n, dst, alpha, dalpha)
    order, bounds = _segments(dst)
    for i in range(n):
        ids = order[bounds[i]:bounds[i + 1]]
        for q in range(k):
            a = alpha[ids, q].astype(np.float64)
            d = dalpha[ids, q].astype(np.float64)
            if ids.size == 0:
                assert rdot[i, q] == 0
                continue
            jac = np.diag(a) - np.outer(a, a)
            np.testing.assert_allclose(ds[ids, q], jac @ d, rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(rdot[i, q], a @ d, rtol=1e-12, atol=1e-14)
    assert np.all(scale >= np.abs(ds) * (1 - 1e-12))


def pin_multihead_attention_gradient():
    """Y = per-head A_alpha(S) X with alpha the per-head target softmax of S:
    d<dY, Y>/dS[e, q] by central differences equals
    softmax_backward_heads(alpha, edge_grad_heads(X, dY))."""
    wl = synth.random_graph(8, 36, 6, 421)
    k = 3
    sc = np.random.default_rng(8).standard_normal((wl.e, k)).astype(np.float32)
    dy64 = wl.dy.astype(np.float64)

    def f(scores):
        a, _, _ = oracle.edge_softmax_heads(wl.n, wl.dst, scores)
        y, _ = oracle.forward_heads(wl.n, wl.src, wl.dst, a.astype(np.float32), wl.x)
        return float((dy64 * y).sum())

    alpha, _, _ = oracle.edge_softmax_heads(wl.n, wl.dst, sc)
    dalpha, _ = oracle.edge_grad_heads(wl.src, wl.dst, wl.x, wl.dy, k)
    ds, _, _ = oracle.edge_softmax_backward_heads(wl.n, wl.dst, alpha.astype(np.float32),
                                                  dalpha.astype(np.float32))
    for j in range(wl.e):
        for q in range(k):
            sp, sm = sc.copy(), sc.copy()
            sp[j, q] += np.float32(1e-2)
            sm[j, q] -= np.float32(1e-2)
            fd = (f(sp) - f(sm)) / (float(sp[j, q]) - float(sm[j, q]))
            assert abs(fd - ds[j, q]) <= 1e-3 * (1 + abs(ds[j, q])), (j, q, fd, ds[j, q])


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
