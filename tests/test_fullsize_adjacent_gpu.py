"""The adjacent operations on the full-size power-law workload (N = 2,000,000,
E = 100,000,000, H = 128 bf16), through the calls and launch configurations the
benchmark times:

* target softmax of the edge weights as scores: every alpha against the
  oracle's softmax of the whole graph, with the bound of the softmax tests;
* its backward with dalpha = the fused backward's dw: every score gradient
  against the oracle;
* symmetric degree normalisation: every edge against the oracle;
* the fetch-normalised forward and fused backward: bitwise equal to normalising
  first and then calling the plain kernels;
* the one-call attention backward: dX bitwise equal to the fused backward's,
  every score gradient bitwise alpha * (dalpha - t[dst]) from that launch's
  dalpha, and the row dots t on sampled rows against the oracle's softmax
  backward over exactly those rows' edges."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.harness import upload

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
DEV = torch.device("cuda:0")
U = 2.0 ** -24


def _lanes(deg):
    return np.where(deg < 64, 1, np.where(deg < 4096, 64, 256))


@pytest.fixture(scope="module")
def run():
    import gnn_sparse_message_amd as mp
    wl = synth.chung_lu()
    t = upload(wl, DEV, torch.int64)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    alpha, stats = mp.mp_edge_softmax(g, t["w"])
    _, dw = mp.mp_spmm_dx_edge_grad(g, t["w"], t["x"], t["dy"])
    ds, rdot = mp.mp_edge_softmax_backward(g, alpha, dw)
    wn = mp.mp_edge_normalize(g, mp.MP_NORM_SYM, t["w"])
    # fetch-normalised calls against normalise-then-call
    y_n = mp.mp_spmm_fwd_norm(g, mp.MP_NORM_SYM, t["w"], t["x"])
    y_ref = mp.mp_spmm_fwd(g, wn, t["x"])
    dx_n, dw_n = mp.mp_spmm_dx_edge_grad_norm(g, mp.MP_NORM_SYM, t["w"], t["x"], t["dy"])
    dx_ref, dwn_ref = mp.mp_spmm_dx_edge_grad(g, wn, t["x"], t["dy"])
    dw_ref = mp.mp_edge_normalize(g, mp.MP_NORM_SYM, dwn_ref)
    fetch_equal = [bool(torch.equal(y_n, y_ref)), bool(torch.equal(dx_n, dx_ref)),
                   bool(torch.equal(dw_n, dw_ref))]
    del y_n, y_ref, dx_n, dw_n, dx_ref, dwn_ref, dw_ref
    # one-call attention backward with alpha = softmax(w)
    y_a = mp.mp_spmm_fwd(g, alpha, t["x"])
    dx_a, ds_a, t_a = mp.mp_attention_backward(g, alpha, t["x"], t["dy"], y_a)
    dx_f, dalpha_f = mp.mp_spmm_dx_edge_grad(g, alpha, t["x"], t["dy"])
    expect = alpha * (dalpha_f - t_a[t["dst"]])
    attention_equal = [bool(torch.equal(dx_a, dx_f)), bool(torch.equal(ds_a, expect))]
    torch.cuda.synchronize()
    out = {"alpha": alpha.cpu().numpy(), "stats": stats.cpu().numpy(), "dw": dw.cpu().numpy(),
           "ds": ds.cpu().numpy(), "rdot": rdot.cpu().numpy(), "wn": wn.cpu().numpy(),
           "t_a": t_a.cpu().numpy(), "fetch_equal": fetch_equal,
           "attention_equal": attention_equal}
    del t, g, alpha, stats, dw, ds, rdot, wn, y_a, dx_a, ds_a, t_a, dx_f, dalpha_f, expect
    torch.cuda.empty_cache()
    return wl, out


def test_fullsize_softmax(run):
    wl, out = run
    ra, rm, rz = oracle.edge_softmax(wl.n, wl.dst, wl.w)
    deg = np.bincount(wl.dst, minlength=wl.n)
    bound = (2.0 * (np.ceil(deg / _lanes(deg)) + 30) * U)[wl.dst]
    rel = np.abs(out["alpha"].astype(np.float64) - ra) / ra
    assert np.all(rel <= bound), f"alpha: worst rel {rel.max():.3e}"
    has = deg > 0
    assert np.array_equal(out["stats"][has, 0].astype(np.float64), rm[has])


def test_fullsize_softmax_backward(run):
    wl, out = run
    rds, _, scale = oracle.edge_softmax_backward(wl.n, wl.dst, out["alpha"], out["dw"])
    deg = np.bincount(wl.dst, minlength=wl.n)
    bound = (2.0 * (np.ceil(deg / _lanes(deg)) + 10) * U)[wl.dst] * scale
    err = np.abs(out["ds"].astype(np.float64) - rds)
    assert np.all(err <= bound), f"ds: worst {(err / np.maximum(scale, 1e-300)).max():.3e}"


def test_fullsize_normalize(run):
    wl, out = run
    ref = oracle.edge_normalize(wl.n, wl.src, wl.dst, oracle.NORM_SYM, wl.w)
    got = out["wn"].astype(np.float64)
    assert np.all(np.abs(got - ref) <= 2.0 ** -22 * np.abs(ref))


def test_fullsize_fetch_normalisation_bitwise(run):
    _, out = run
    assert out["fetch_equal"] == [True, True, True]


def test_fullsize_attention_backward(run):
    wl, out = run
    assert out["attention_equal"] == [True, True]
    # row dots on sampled rows: the oracle's softmax backward over those rows' edges
    rng = np.random.default_rng(7)
    deg = np.bincount(wl.dst, minlength=wl.n)
    rows = np.unique(np.concatenate([np.argsort(-deg, kind="stable")[:4],
                                     rng.choice(np.nonzero(deg > 0)[0], 60, replace=False)]))
    keep = np.isin(wl.dst, rows)
    edges = np.nonzero(keep)[0]
    dalpha, sda = oracle.edge_grad_edges(wl.src, wl.dst, wl.x, wl.dy, edges)
    alpha = out["alpha"][edges]
    _, rt, _ = oracle.edge_softmax_backward(wl.n, wl.dst[edges], alpha, dalpha.astype(np.float32))
    # |t - t_ref| <= tau * T_i, T_i >= sum over the row of alpha * S_dalpha
    t_scale = np.bincount(wl.dst[edges], weights=alpha * sda, minlength=wl.n)
    err = np.abs(out["t_a"][rows].astype(np.float64) - rt[rows])
    assert np.all(err <= 1e-5 * t_scale[rows] + 1e-30), (err / np.maximum(t_scale[rows], 1e-30)).max()
