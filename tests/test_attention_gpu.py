"""Target softmax of edge scores (mp_edge_softmax) and its backward
(mp_edge_softmax_backward) against the oracle, and the whole sparse attention
layer built from them: alpha = softmax(s), Y = A_alpha X, (dX, dalpha) from the
fused backward, ds = softmax_backward(alpha, dalpha).

Tolerances are derived from the device arithmetic.  A row of length d is owned
by 1, 64 or 256 lanes (d < 64, d < 4096, longer); each lane sums
ceil(d / lanes) terms in sequence and the lanes merge in at most 8 butterfly
levels, with one exp and one division per alpha.  The relative error of alpha
is then below (ceil(d / lanes) + 30) u with u = 2^-24; the tests allow twice
that, per edge, from its row length.  The backward is compared element-wise
against S = alpha (|dalpha| + sum over the row of alpha |dalpha|) with
(ceil(d / lanes) + 10) u, doubled."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.harness import TAU, check_close, upload

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
U = 2.0 ** -24


@pytest.fixture(scope="module")
def mp():
    import gnn_sparse_message_amd
    return gnn_sparse_message_amd


def _lanes(deg):
    return np.where(deg < 64, 1, np.where(deg < 4096, 64, 256))


def _alpha_bound(dst, n):
    deg = np.bincount(dst, minlength=n)
    per_row = 2.0 * (np.ceil(deg / _lanes(deg)) + 30) * U
    return per_row[dst]


def _back_bound(dst, n):
    deg = np.bincount(dst, minlength=n)
    per_row = 2.0 * (np.ceil(deg / _lanes(deg)) + 10) * U
    return per_row[dst]


def _softmax(mp, wl, scores):
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    s = torch.from_numpy(scores).to(DEV)
    alpha, stats = mp.mp_edge_softmax(g, s)
    torch.cuda.synchronize()
    return g, t, s, alpha, stats[:, 0], stats[:, 1]


def _check_softmax(wl, scores, alpha, rmax, rsum):
    ra, rm, rz = oracle.edge_softmax(wl.n, wl.dst, scores)
    got = alpha.cpu().numpy().astype(np.float64)
    rel = np.abs(got - ra) / ra
    bound = _alpha_bound(wl.dst, wl.n)
    bad = rel > bound
    assert not bad.any(), (f"alpha: {int(bad.sum())} edges outside the bound, worst rel "
                           f"{rel.max():.3e} (bound there {bound[np.argmax(rel)]:.3e})")
    gm = rmax.cpu().numpy()
    has = np.bincount(wl.dst, minlength=wl.n) > 0
    assert np.array_equal(gm[has].astype(np.float64), rm[has])      # max is exact
    assert np.all(np.isneginf(gm[~has])) and np.all(rsum.cpu().numpy()[~has] == 0)
    gz = rsum.cpu().numpy().astype(np.float64)
    deg = np.bincount(wl.dst, minlength=wl.n)
    zb = 2.0 * (np.ceil(deg / _lanes(deg)) + 30) * U
    assert np.all(np.abs(gz[has] - rz[has]) <= zb[has] * rz[has])
    return float(rel.max()) if rel.size else 0.0


def test_witness(mp):
    wl = synth.witness()
    g, t, s, alpha, rmax, rsum = _softmax(mp, wl, wl.w)
    _check_softmax(wl, wl.w, alpha, rmax, rsum)
    assert alpha[2].item() == 1.0                                  # a row with one edge


@pytest.mark.parametrize("n,e,scale,seed", [(1, 0, 1.0, 1), (1, 1, 1.0, 2), (5, 0, 1.0, 3),
                                            (1, 5000, 1.0, 4), (300, 4000, 3.0, 5),
                                            (7000, 200000, 2.0, 6), (50, 300000, 1.0, 7),
                                            (100000, 50000, 1.0, 8)])
def test_random_graphs(mp, n, e, scale, seed):
    wl = synth.random_graph(n, e, 1, seed)
    scores = (wl.w * scale).astype(np.float32)
    g, t, s, alpha, rmax, rsum = _softmax(mp, wl, scores)
    _check_softmax(wl, scores, alpha, rmax, rsum)


def test_power_law_all_owner_kinds(mp):
    wl = synth.chung_lu(seed=17, n=30000, e=600000, cap=30000.0, h=1, feat_dtype="f32")
    deg = np.bincount(wl.dst, minlength=wl.n)
    assert deg.max() >= 4096 and ((deg >= 64) & (deg < 4096)).any() and (deg == 0).any()
    scores = np.random.default_rng(3).standard_normal(wl.e).astype(np.float32) * 4
    g, t, s, alpha, rmax, rsum = _softmax(mp, wl, scores)
    _check_softmax(wl, scores, alpha, rmax, rsum)


def test_equal_scores_give_one_over_degree(mp):
    wl = synth.random_graph(2000, 100000, 1, 9)
    scores = np.full(wl.e, -2.5, np.float32)
    g, t, s, alpha, rmax, rsum = _softmax(mp, wl, scores)
    deg = np.bincount(wl.dst, minlength=wl.n)
    expect = (np.float32(1.0) / deg[wl.dst].astype(np.float32)).astype(np.float32)
    assert np.array_equal(alpha.cpu().numpy(), expect)              # z = deg exactly


def test_large_scores_are_stable(mp):
    wl = synth.random_graph(500, 20000, 1, 10)
    scores = (wl.w * 10 + 5000.0).astype(np.float32)
    g, t, s, alpha, rmax, rsum = _softmax(mp, wl, scores)
    assert torch.isfinite(alpha).all()
    _check_softmax(wl, scores, alpha, rmax, rsum)


def test_backward_against_oracle(mp):
    wl = synth.chung_lu(seed=19, n=20000, e=400000, cap=20000.0, h=1, feat_dtype="f32")
    rng = np.random.default_rng(4)
    scores = rng.standard_normal(wl.e).astype(np.float32)
    g, t, s, alpha, rmax, rsum = _softmax(mp, wl, scores)
    dalpha_np = rng.standard_normal(wl.e).astype(np.float32)
    dalpha = torch.from_numpy(dalpha_np).to(DEV)
    ds, rdot = mp.mp_edge_softmax_backward(g, alpha, dalpha)
    torch.cuda.synchronize()
    a32 = alpha.cpu().numpy()
    rds, rrdot, scale = oracle.edge_softmax_backward(wl.n, wl.dst, a32, dalpha_np)
    err = np.abs(ds.cpu().numpy().astype(np.float64) - rds)
    bound = _back_bound(wl.dst, wl.n) * scale
    assert np.all(err <= bound), float((err / np.maximum(scale, 1e-300)).max())
    has = np.bincount(wl.dst, minlength=wl.n) > 0
    assert np.all(rdot.cpu().numpy()[~has] == 0)


def test_attention_layer_end_to_end(mp):
    """Each stage against the oracle fed the device's previous stage, and the
    final score gradient against the all-oracle chain."""
    wl = synth.chung_lu(seed=23, n=8000, e=160000, cap=8000.0, h=64, feat_dtype="bf16")
    rng = np.random.default_rng(5)
    scores = rng.standard_normal(wl.e).astype(np.float32)
    g, t, s, alpha, rmax, rsum = _softmax(mp, wl, scores)
    _check_softmax(wl, scores, alpha, rmax, rsum)
    y = mp.mp_spmm_fwd(g, alpha, t["x"])
    dx, dalpha = mp.mp_spmm_dx_edge_grad(g, alpha, t["x"], t["dy"])
    ds, rdot = mp.mp_edge_softmax_backward(g, alpha, dalpha)
    torch.cuda.synchronize()
    a32 = alpha.cpu().numpy()
    ry, sy = oracle.forward(wl.n, wl.src, wl.dst, a32, wl.x)
    check_close("Y", y, ry, sy, TAU["f32"])
    rdx, sdx = oracle.input_grad(wl.n, wl.src, wl.dst, a32, wl.dy)
    check_close("dX", dx, rdx, sdx, TAU["f32"])
    rda, sda = oracle.edge_grad(wl.src, wl.dst, wl.x, wl.dy)
    check_close("dalpha", dalpha, rda, sda, TAU["f32"])
    da32 = dalpha.cpu().numpy()
    rds, _, scale = oracle.edge_softmax_backward(wl.n, wl.dst, a32, da32)
    err = np.abs(ds.cpu().numpy().astype(np.float64) - rds)
    assert np.all(err <= _back_bound(wl.dst, wl.n) * scale)
    # all-oracle chain (fp64 alpha, fp64 dalpha) for the score gradient
    ra, _, _ = oracle.edge_softmax(wl.n, wl.dst, scores)
    full, _, fscale = oracle.edge_softmax_backward(wl.n, wl.dst, ra.astype(np.float32),
                                                   rda.astype(np.float32))
    rel = np.abs(ds.cpu().numpy() - full) / np.maximum(fscale, 1e-30)
    assert rel.max() < 1e-4, rel.max()


def test_rejections(mp):
    wl = synth.random_graph(100, 500, 1, 11)
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    with pytest.raises(TypeError):
        mp.mp_edge_softmax(g, t["w"].double())
    with pytest.raises(ValueError):
        mp.mp_edge_softmax(g, t["w"][:10])
    with pytest.raises(ValueError):                      # alpha aliases the scores
        mp.mp_edge_softmax(g, t["w"], out_alpha=t["w"])
    with pytest.raises(ValueError):                      # host memory
        mp.mp_edge_softmax(g, t["w"].cpu())
    with pytest.raises(ValueError):                      # row statistics are [N, 2]
        mp.mp_edge_softmax(g, t["w"], out_row_stats=torch.empty(wl.n, device=DEV))
    a, _ = mp.mp_edge_softmax(g, t["w"])
    with pytest.raises(ValueError):                      # ds aliases dalpha
        mp.mp_edge_softmax_backward(g, a, t["w"], out_dscores=t["w"])


# ---------------------------------------------------------------- multi-head scores

def _check_softmax_heads(wl, scores, alpha, stats):
    k = scores.shape[1]
    ra, rm, rz = oracle.edge_softmax_heads(wl.n, wl.dst, scores)
    got = alpha.cpu().numpy().astype(np.float64)
    bound = _alpha_bound(wl.dst, wl.n)[:, None]
    rel = np.abs(got - ra) / ra
    assert not (rel > bound).any(), f"alpha: worst rel {rel.max():.3e}"
    st = stats.cpu().numpy()
    has = np.bincount(wl.dst, minlength=wl.n) > 0
    assert np.array_equal(st[has, :, 0].astype(np.float64), rm[has])       # max is exact
    assert np.all(np.isneginf(st[~has, :, 0])) and np.all(st[~has, :, 1] == 0)
    deg = np.bincount(wl.dst, minlength=wl.n)
    zb = (2.0 * (np.ceil(deg / _lanes(deg)) + 30) * U)[:, None]
    assert np.all(np.abs(st[has, :, 1] - rz[has]) <= zb[has] * rz[has])


@pytest.mark.parametrize("k", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("kind", ["random", "power_law"])
def test_softmax_heads_against_oracle(mp, k, kind):
    if kind == "random":
        wl = synth.random_graph(3000, 60000, 1, 600 + k)
    else:
        wl = synth.chung_lu(seed=37, n=20000, e=400000, cap=20000.0, h=1, feat_dtype="f32")
    rng = np.random.default_rng(k)
    scores = (rng.standard_normal((wl.e, k)) * 3).astype(np.float32)
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    s = torch.from_numpy(scores).to(DEV)
    alpha, stats = mp.mp_edge_softmax_heads(g, s)
    dalpha_np = rng.standard_normal((wl.e, k)).astype(np.float32)
    ds, rdot = mp.mp_edge_softmax_backward_heads(g, alpha, torch.from_numpy(dalpha_np).to(DEV))
    torch.cuda.synchronize()
    _check_softmax_heads(wl, scores, alpha, stats)
    a32 = alpha.cpu().numpy()
    rds, rrdot, scale = oracle.edge_softmax_backward_heads(wl.n, wl.dst, a32, dalpha_np)
    err = np.abs(ds.cpu().numpy().astype(np.float64) - rds)
    assert np.all(err <= _back_bound(wl.dst, wl.n)[:, None] * scale)
    if k == 1:                                       # one head is exactly the scalar call
        a1, st1 = mp.mp_edge_softmax(g, s[:, 0].contiguous())
        d1, r1 = mp.mp_edge_softmax_backward(g, alpha[:, 0].contiguous(),
                                             torch.from_numpy(dalpha_np[:, 0].copy()).to(DEV))
        torch.cuda.synchronize()
        assert torch.equal(a1, alpha[:, 0]) and torch.equal(st1, stats[:, 0, :])
        assert torch.equal(d1, ds[:, 0]) and torch.equal(r1, rdot[:, 0])


def test_multihead_attention_layer_end_to_end(mp):
    """alpha = per-head softmax(S); Y = multi-head A_alpha X; (dX, dalpha) from the
    multi-head fused backward; dS from the per-head softmax backward -- each stage
    against the oracle fed the device's previous stage."""
    k = 4
    wl = synth.chung_lu(seed=41, n=8000, e=160000, cap=8000.0, h=64, feat_dtype="bf16")
    rng = np.random.default_rng(9)
    scores = rng.standard_normal((wl.e, k)).astype(np.float32)
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    alpha, stats = mp.mp_edge_softmax_heads(g, torch.from_numpy(scores).to(DEV))
    y = mp.mp_spmm_fwd_heads(g, alpha, t["x"])
    dx, dalpha = mp.mp_spmm_dx_edge_grad_heads(g, alpha, t["x"], t["dy"])
    ds, _ = mp.mp_edge_softmax_backward_heads(g, alpha, dalpha)
    torch.cuda.synchronize()
    _check_softmax_heads(wl, scores, alpha, stats)
    a32 = alpha.cpu().numpy()
    ry, sy = oracle.forward_heads(wl.n, wl.src, wl.dst, a32, wl.x)
    check_close("Y", y, ry, sy, TAU["f32"])
    rdx, sdx = oracle.input_grad_heads(wl.n, wl.src, wl.dst, a32, wl.dy)
    check_close("dX", dx, rdx, sdx, TAU["f32"])
    rda, sda = oracle.edge_grad_heads(wl.src, wl.dst, wl.x, wl.dy, k)
    check_close("dalpha", dalpha, rda, sda, TAU["f32"])
    rds, _, scale = oracle.edge_softmax_backward_heads(wl.n, wl.dst, a32, dalpha.cpu().numpy())
    err = np.abs(ds.cpu().numpy().astype(np.float64) - rds)
    assert np.all(err <= _back_bound(wl.dst, wl.n)[:, None] * scale)


def test_softmax_heads_rejections(mp):
    wl = synth.random_graph(100, 500, 1, 12)
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    s3 = torch.zeros((wl.e, 3), device=DEV)
    with pytest.raises(ValueError):                  # scores must be [E, K]
        mp.mp_edge_softmax_heads(g, torch.zeros(wl.e * 3, device=DEV))
    with pytest.raises(ValueError):                  # statistics are [N, K, 2]
        mp.mp_edge_softmax_heads(g, s3, out_row_stats=torch.empty((wl.n, 3), device=DEV))
    with pytest.raises(ValueError):                  # head counts differ
        mp.mp_edge_softmax_backward_heads(g, s3, torch.zeros((wl.e, 2), device=DEV))
    with pytest.raises(ValueError):                  # dscores aliases dalpha
        mp.mp_edge_softmax_backward_heads(g, s3, s3, out_dscores=s3)
