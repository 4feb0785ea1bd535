"""The full-size power-law workload (N = 2,000,000, E = 100,000,000, H = 128,
bf16 features, fp32 accumulation) through the same entry points and launch
configuration the benchmark times.  The whole lowering is compared with the
oracle bit for bit, and every element of Y, dX and dw with the fp64 oracle
(evaluated in row sets and edge ranges on all host cores) at the bf16-storage
bound 2e-2 and at the fp32 bound 1e-5.  The step's calls (the fused backward,
and both calls on weights and gradients interleaved in one [E][2] array) are
bitwise equal to the separate calls held to the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.harness import TAU, check_all_edges, check_all_rows, check_close, upload

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def run():
    import gnn_sparse_message_amd as mp
    print("full-size power-law workload: generating", flush=True)
    wl = synth.chung_lu()
    t = upload(wl, DEV, torch.int64)
    print("full-size power-law workload: build, forward, gradients", flush=True)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    y = mp.mp_spmm_fwd(g, t["w"], t["x"])
    dx = mp.mp_spmm_dx(g, t["w"], t["dy"])
    dw = mp.mp_edge_grad_dw(g, t["x"], t["dy"])
    # the fused backward, and the benchmark's step calls on the interleaved
    # weights, against the separate calls
    fdx, fdw = mp.mp_spmm_dx_edge_grad(g, t["w"], t["x"], t["dy"])
    wg = torch.empty((wl.e, 2), dtype=torch.float32, device=DEV)
    wg[:, 0] = t["w"]
    py = mp.mp_spmm_fwd_pair(g, wg, t["x"])
    pdx = mp.mp_spmm_dx_edge_grad_pair(g, wg, t["x"], t["dy"])
    torch.cuda.synchronize()
    fused_equal = bool(torch.equal(fdx, dx) and torch.equal(fdw, dw))
    pair_equal = bool(torch.equal(py, y) and torch.equal(pdx, dx) and torch.equal(wg[:, 1], dw)
                      and torch.equal(wg[:, 0], t["w"]))
    out = {"g": {k: v.cpu().numpy() for k, v in g.arrays.items()},
           "cc": g.class_count, "cc_t": g.class_count_t, "fused_equal": fused_equal,
           "pair_equal": pair_equal,
           "y": y.cpu().numpy(), "dx": dx.cpu().numpy(), "dw": dw.cpu().numpy()}
    del t, g, y, dx, dw, fdx, fdw, wg, py, pdx
    torch.cuda.empty_cache()
    return wl, out


def _sample_rows(deg, rng):
    order = np.argsort(-deg, kind="stable")
    rows = [order[:8], rng.choice(deg.shape[0], 48, replace=False),
            np.nonzero(deg == 0)[0][:4], np.array([deg.shape[0] - 1]),
            rng.choice(np.nonzero((deg >= 16) & (deg < 4096))[0], 16, replace=False)]
    return np.unique(np.concatenate(rows)).astype(np.int64)


def test_fullsize_lowering_bit_exact(run):
    wl, out = run
    for key, other, names in ((wl.dst, wl.src, ("rowptr", "col", "edge_order")),
                              (wl.src, wl.dst, ("rowptr_t", "col_t", "transpose_order"))):
        ref = oracle.lower(wl.n, key, other)
        for name, r in zip(names, ref):
            assert np.array_equal(out["g"][name], r), name
    rowptr, _, _ = oracle.lower(wl.n, wl.dst, wl.src)
    plan, cc = oracle.degree_plan(wl.n, rowptr)
    assert np.array_equal(out["g"]["row_plan"], plan)
    assert out["cc"] == cc.tolist()
    rowptr_t, _, _ = oracle.lower(wl.n, wl.src, wl.dst)
    plan_t, cc_t = oracle.degree_plan(wl.n, rowptr_t)
    assert np.array_equal(out["g"]["row_plan_t"], plan_t)
    assert out["cc_t"] == cc_t.tolist()


def test_fullsize_forward_every_row(run):
    wl, out = run
    worst = check_all_rows(
        "Y", out["y"], wl.n,
        lambda rows: oracle.forward_rows(wl.n, wl.src, wl.dst, wl.w, wl.x, rows),
        (TAU["bf16"], TAU["f32"]))   # fp32 accumulation: the fp32 bound holds as well
    print("forward max |err|/S over all", wl.n * wl.h, "elements:", worst)


def test_fullsize_input_grad_every_row(run):
    wl, out = run
    worst = check_all_rows(
        "dX", out["dx"], wl.n,
        lambda rows: oracle.input_grad_rows(wl.n, wl.src, wl.dst, wl.w, wl.dy, rows),
        (TAU["bf16"], TAU["f32"]))
    print("input gradient max |err|/S over all", wl.n * wl.h, "elements:", worst)


def test_fullsize_edge_grad_every_edge(run):
    wl, out = run
    worst = check_all_edges(
        "dw", out["dw"], wl.e,
        lambda lo, hi: oracle.edge_grad(wl.src[lo:hi], wl.dst[lo:hi], wl.x, wl.dy),
        (TAU["bf16"], TAU["f32"]))
    print("edge gradient max |err|/S over all", wl.e, "edges:", worst)


def test_fullsize_fused_backward_equals_separate_calls(run):
    """The fused backward returns the bits of mp_spmm_dx and mp_edge_grad_dw,
    which the tests above hold to the oracle element by element."""
    _, out = run
    assert out["fused_equal"]


def test_fullsize_interleaved_step_equals_separate_calls(run):
    """The benchmark's step calls on the interleaved [E][2] array (forward and
    fused backward) return the bits of mp_spmm_fwd, mp_spmm_dx and
    mp_edge_grad_dw, and leave the weights untouched."""
    _, out = run
    assert out["pair_equal"]


def test_fullsize_outputs_finite_everywhere(run):
    wl, out = run
    assert np.isfinite(out["y"]).all() and np.isfinite(out["dx"]).all()
    assert np.isfinite(out["dw"]).all()
    empty = np.bincount(wl.dst, minlength=wl.n) == 0
    assert np.all(out["y"][empty] == 0)


@pytest.fixture(scope="module")
def run_heads(run):
    """Multi-head weights (K = 4 heads of 32 columns) on the same full-size graph,
    through the forward and the fused backward the benchmark times."""
    import gnn_sparse_message_amd as mp
    wl, _ = run
    k = 4
    w_np = np.random.default_rng(41).uniform(-1, 1, (wl.e, k)).astype(np.float32)
    t = upload(wl, DEV, torch.int64)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    w = torch.from_numpy(w_np).to(DEV)
    y = mp.mp_spmm_fwd_heads(g, w, t["x"])
    dx, dw = mp.mp_spmm_dx_edge_grad_heads(g, w, t["x"], t["dy"])
    torch.cuda.synchronize()
    out = {"y": y.cpu().numpy(), "dx": dx.cpu().numpy(), "dw": dw.cpu().numpy()}
    del t, g, w, y, dx, dw
    torch.cuda.empty_cache()
    return wl, k, w_np, out


def test_fullsize_heads_sampled(run_heads):
    wl, k, w_np, out = run_heads
    rng = np.random.default_rng(5)
    rows = _sample_rows(np.bincount(wl.dst, minlength=wl.n), rng)
    ref, s = oracle.forward_heads(wl.n, wl.src, wl.dst, w_np, wl.x, rows=rows)
    check_close("Y heads rows", out["y"][rows], ref, s, TAU["f32"])
    rows_t = _sample_rows(np.bincount(wl.src, minlength=wl.n), rng)
    ref, s = oracle.input_grad_heads(wl.n, wl.src, wl.dst, w_np, wl.dy, rows=rows_t)
    check_close("dX heads rows", out["dx"][rows_t], ref, s, TAU["f32"])
    hub = int(np.argmax(np.bincount(wl.src, minlength=wl.n)))
    edges = np.unique(np.concatenate([rng.choice(wl.e, 20000, replace=False),
                                      np.nonzero(wl.src == hub)[0][:5000],
                                      np.array([0, wl.e - 1])])).astype(np.int64)
    ref, s = oracle.edge_grad_heads(wl.src, wl.dst, wl.x, wl.dy, k, edges=edges)
    check_close("dw heads edges", out["dw"][edges], ref, s, TAU["f32"])
    assert np.isfinite(out["y"]).all() and np.isfinite(out["dx"]).all()
    assert np.isfinite(out["dw"]).all()
