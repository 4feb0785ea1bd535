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


@pytest.fixture(autouse=True)
def _owner_rule_after_each_test():
    """Tests that set owner overrides leave the rule in place for the next."""
    yield
    import gnn_sparse_message_amd
    gnn_sparse_message_amd.mp_set_owner_overrides(-1, -1, -1)


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


# ---------------------------------------------------------------- fused attention backward
#
# mp_attention_backward against the oracle composition: dX = input_grad(alpha,
# dY), dalpha = edge_grad(X, dY), (ds, t) = softmax_backward(alpha, dalpha).
# The device takes the row term t_i from the kept forward output, <Y_i, dY_i>
# per head; that equals the row sum of alpha * dalpha exactly, and its error
# is bounded by T_i = sum_c |dY_ic| S_Y[i, c] (S_Y the forward's |term| sums)
# times the forward's tau, plus the dot product's own rounding, which the same
# T_i bounds.  So, per edge e into i and head q:
#   |ds - ds_ref| <= tau (alpha_e (S_dalpha_e + T_i) + scale_e),
# scale_e = alpha_e (|dalpha_e| + sum over the row of alpha |dalpha|) covering
# the fp32 rounding of dalpha the oracle is fed, and |t - t_ref| <= tau T_i.

def _attention_case(wl, k, seed):
    rng = np.random.default_rng(seed)
    scores = (rng.standard_normal((wl.e, k)) * 2).astype(np.float32)
    ra, _, _ = oracle.edge_softmax_heads(wl.n, wl.dst, scores)
    a32 = ra.astype(np.float32)
    ry, sy = oracle.forward_heads(wl.n, wl.src, wl.dst, a32, wl.x)
    return a32, ry, sy


def _attention_reference(wl, a32, sy):
    k = a32.shape[1]
    rdx, sdx = oracle.input_grad_heads(wl.n, wl.src, wl.dst, a32, wl.dy)
    rda, sda = oracle.edge_grad_heads(wl.src, wl.dst, wl.x, wl.dy, k)
    rds, rt, scale = oracle.edge_softmax_backward_heads(wl.n, wl.dst, a32, rda.astype(np.float32))
    hw = wl.h // k
    tt = (np.abs(wl.dy.astype(np.float64)) * sy).reshape(wl.n, k, hw).sum(axis=2)
    return rdx, sdx, rda, sda, rds, rt, scale, tt


def _check_attention(wl, a32, sy, dx, ds, rdot, tau=TAU["f32"]):
    rdx, sdx, rda, sda, rds, rt, scale, tt = _attention_reference(wl, a32, sy)
    check_close("dX", dx, rdx, sdx, tau)
    k = a32.shape[1]
    got_ds = ds.cpu().numpy().reshape(wl.e, k).astype(np.float64)
    bound = tau * (a32 * (sda + tt[wl.dst]) + scale)
    err = np.abs(got_ds - rds)
    bad = err > bound
    assert not bad.any(), (f"dscores: {int(bad.sum())} outside the bound, worst "
                           f"{(err / np.maximum(bound, 1e-300)).max():.3g} x bound")
    got_t = rdot.cpu().numpy().reshape(wl.n, k).astype(np.float64)
    terr = np.abs(got_t - rt)
    assert np.all(terr <= tau * tt), f"row_dot: worst {(terr / np.maximum(tt, 1e-300)).max():.3g}"


@pytest.mark.parametrize("case", [
    ("power_law_f32_h64_k1", lambda: synth.chung_lu(seed=51, n=20000, e=400000, cap=20000.0,
                                                    h=64, feat_dtype="f32"), 1),
    ("power_law_bf16_h128_k1", lambda: synth.chung_lu(seed=52, n=8000, e=200000, cap=8000.0,
                                                      h=128, feat_dtype="bf16"), 1),
    ("power_law_bf16_h128_k4", lambda: synth.chung_lu(seed=53, n=8000, e=200000, cap=8000.0,
                                                      h=128, feat_dtype="bf16"), 4),
    ("random_f32_h32_k2", lambda: synth.random_graph(3000, 50000, 32, 54), 2),
    ("ragged_f32_h6_k2", lambda: synth.random_graph(1500, 20000, 6, 55), 2),
    ("ragged_bf16_h15_k3", lambda: synth.random_graph(1500, 20000, 15, 56, feat_dtype="bf16"), 3),
    ("wide_f32_h600_k3", lambda: synth.random_graph(700, 9000, 600, 57), 3),
    ("wide_bf16_h1024_k2", lambda: synth.random_graph(500, 6000, 1024, 58, feat_dtype="bf16"), 2),
    ("one_node_no_edges", lambda: synth.random_graph(1, 0, 8, 59), 2),
    ("no_edges", lambda: synth.random_graph(50, 0, 16, 60), 1),
], ids=lambda c: c[0])
def test_attention_backward_against_oracle(mp, case):
    _, make, k = case
    wl = make()
    a32, ry, sy = _attention_case(wl, k, 7)
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    alpha = torch.from_numpy(a32 if k > 1 else a32[:, 0].copy()).to(DEV)
    y = torch.from_numpy(ry.astype(np.float32)).to(DEV)
    dx, ds, rdot = mp.mp_attention_backward(g, alpha, t["x"], t["dy"], y)
    torch.cuda.synchronize()
    assert ds.shape == alpha.shape and rdot.shape == ((wl.n,) if k == 1 else (wl.n, k))
    _check_attention(wl, a32, sy, dx, ds, rdot)


@pytest.mark.parametrize("k", [1, 4])
def test_attention_backward_equals_unfused_chain(mp, k):
    """Same graph and inputs: dX is bit-identical to the fused input/edge
    gradient call, and each score gradient is exactly alpha * (dalpha - t[dst])
    formed from that call's dalpha and this call's row_dot."""
    wl = synth.chung_lu(seed=61, n=20000, e=400000, cap=20000.0, h=128, feat_dtype="bf16")
    a32, ry, sy = _attention_case(wl, k, 8)
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    alpha = torch.from_numpy(a32).to(DEV)
    y = mp.mp_spmm_fwd_heads(g, alpha, t["x"])                   # the device forward
    dx, ds, rdot = mp.mp_attention_backward(g, alpha, t["x"], t["dy"], y)
    dx2, dalpha = mp.mp_spmm_dx_edge_grad_heads(g, alpha, t["x"], t["dy"])
    dst = t["dst"].long()
    expect = alpha * (dalpha - rdot[dst])
    torch.cuda.synchronize()
    assert torch.equal(dx, dx2)
    assert torch.equal(ds, expect)
    # and the chain through the device forward still meets the oracle bound
    _check_attention(wl, a32, sy, dx, ds, rdot)


def test_attention_layer_fused_end_to_end(mp):
    """scores -> softmax -> forward -> fused backward, all on the device, against
    the all-oracle chain (alpha from the oracle softmax of the same scores)."""
    k = 2
    wl = synth.chung_lu(seed=62, n=8000, e=160000, cap=8000.0, h=64, feat_dtype="bf16")
    rng = np.random.default_rng(10)
    scores = rng.standard_normal((wl.e, k)).astype(np.float32)
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    alpha, _ = mp.mp_edge_softmax_heads(g, torch.from_numpy(scores).to(DEV))
    y = mp.mp_spmm_fwd_heads(g, alpha, t["x"])
    dx, ds, rdot = mp.mp_attention_backward(g, alpha, t["x"], t["dy"], y)
    torch.cuda.synchronize()
    a32 = alpha.cpu().numpy()             # the device's alpha feeds the oracle chain
    _, sy = oracle.forward_heads(wl.n, wl.src, wl.dst, a32, wl.x)
    _check_attention(wl, a32, sy, dx, ds, rdot)
    # against the all-fp64 softmax as well, relative to the score-gradient scale
    ra, _, _ = oracle.edge_softmax_heads(wl.n, wl.dst, scores)
    rda, _ = oracle.edge_grad_heads(wl.src, wl.dst, wl.x, wl.dy, k)
    full, _, fscale = oracle.edge_softmax_backward_heads(wl.n, wl.dst, ra.astype(np.float32),
                                                         rda.astype(np.float32))
    rel = np.abs(ds.cpu().numpy() - full) / np.maximum(fscale, 1e-30)
    assert rel.max() < 1e-4, rel.max()


def test_attention_backward_async_graph(mp):
    """On a graph whose class counts are still on the device the call returns
    the same bits as on the finished graph."""
    wl = synth.chung_lu(seed=63, n=6000, e=90000, cap=6000.0, h=64, feat_dtype="f32")
    a32, ry, sy = _attention_case(wl, 2, 9)
    t = upload(wl, DEV)
    alpha = torch.from_numpy(a32).to(DEV)
    y = torch.from_numpy(ry.astype(np.float32)).to(DEV)
    g1 = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    g2 = mp.mp_graph_build_async(t["src"], t["dst"], wl.n)
    r1 = mp.mp_attention_backward(g1, alpha, t["x"], t["dy"], y)
    r2 = mp.mp_attention_backward(g2, alpha, t["x"], t["dy"], y)
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)
    mp.mp_graph_finish(g2)


def test_attention_backward_rejections(mp):
    wl = synth.random_graph(100, 500, 8, 13)
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    alpha = torch.rand((wl.e, 2), device=DEV)
    y = torch.zeros((wl.n, 8), device=DEV)
    with pytest.raises(TypeError):                   # y must be float32
        mp.mp_attention_backward(g, alpha, t["x"], t["dy"], y.bfloat16())
    with pytest.raises(ValueError):                  # widths differ
        mp.mp_attention_backward(g, alpha, t["x"], t["dy"], y[:, :4].contiguous())
    with pytest.raises(ValueError):                  # 3 heads do not divide 8
        mp.mp_attention_backward(g, torch.rand((wl.e, 3), device=DEV), t["x"], t["dy"], y)
    with pytest.raises(ValueError):                  # dx aliases y
        mp.mp_attention_backward(g, alpha, t["x"], t["dy"], y, out_dx=y)
    with pytest.raises(ValueError):                  # dscores overlaps alpha, shifted
        buf = torch.rand((wl.e + 1, 2), device=DEV)
        mp.mp_attention_backward(g, buf[:-1], t["x"], t["dy"], y, out_dscores=buf[1:])
    ds = torch.empty((wl.e, 2), device=DEV)
    with pytest.raises(ValueError):                  # row_dot inside dscores
        mp.mp_attention_backward(g, alpha, t["x"], t["dy"], y, out_dscores=ds,
                                 out_row_dot=ds.view(-1)[:wl.n * 2].view(wl.n, 2))
    with pytest.raises(TypeError):                   # x and dy dtypes differ
        mp.mp_attention_backward(g, alpha, t["x"].bfloat16(), t["dy"], y)


def test_dot_product_attention_layer_chain(mp):
    """Scores from the SDDMM, softmax over each target's edges, aggregation, and
    the whole backward including the query and key gradients, all through the
    library; every stage against the oracle fed the device's previous stage:
      s = <K[src], Q[dst]>          mp_edge_grad_dw(g, K, Q)
      alpha = softmax_dst(s)        mp_edge_softmax
      Y = A_alpha V                 mp_spmm_fwd
      dV, ds                        mp_attention_backward(g, alpha, V, dY, Y)
      dK[src] += ds_e Q[dst_e]      mp_spmm_dx(g, ds, Q)
      dQ[dst] += ds_e K[src_e]      mp_spmm_fwd(g, ds, K)"""
    wl = synth.chung_lu(seed=64, n=6000, e=120000, cap=6000.0, h=64, feat_dtype="f32")
    other = synth.random_graph(wl.n, 1, wl.h, 65)          # two more feature arrays
    kk, qq = wl.x, (wl.dy / 8.0).astype(np.float32)         # /8 = 1/sqrt(H), exact
    vv, dout = other.x, other.dy
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    K, Q, V, dY = (torch.from_numpy(a).to(DEV) for a in (kk, qq, vv, dout))
    s = mp.mp_edge_grad_dw(g, K, Q)
    alpha, stats = mp.mp_edge_softmax(g, s)
    y = mp.mp_spmm_fwd(g, alpha, V)
    dv, ds, rdot = mp.mp_attention_backward(g, alpha, V, dY, y)
    dk = mp.mp_spmm_dx(g, ds, Q)
    dq = mp.mp_spmm_fwd(g, ds, K)
    torch.cuda.synchronize()
    rs, ss = oracle.edge_grad(wl.src, wl.dst, kk, qq)
    check_close("scores", s, rs, ss, TAU["f32"])
    s32 = s.cpu().numpy()
    _check_softmax(wl, s32, alpha, stats[:, 0], stats[:, 1])
    a32 = alpha.cpu().numpy()
    ry, sy = oracle.forward(wl.n, wl.src, wl.dst, a32, vv)
    check_close("Y", y, ry, sy, TAU["f32"])
    chain = synth.Workload("chain", wl.n, wl.src, wl.dst, a32, vv, dout, "f32", None, None)
    _check_attention(chain, a32[:, None], sy, dv, ds.view(-1, 1), rdot.view(-1, 1))
    ds32 = ds.cpu().numpy()
    rdk, sdk = oracle.input_grad(wl.n, wl.src, wl.dst, ds32, qq)
    check_close("dK", dk, rdk, sdk, TAU["f32"])
    rdq, sdq = oracle.forward(wl.n, wl.src, wl.dst, ds32, kk)
    check_close("dQ", dq, rdq, sdq, TAU["f32"])


@pytest.mark.parametrize("k", [1, 4])
def test_attention_backward_in_place(mp, k):
    """Score gradients written over alpha equal the separate call bit for bit;
    on rows too wide for the fused walk the in-place form is refused."""
    wl = synth.chung_lu(seed=66, n=20000, e=400000, cap=20000.0, h=128, feat_dtype="bf16")
    a32, ry, sy = _attention_case(wl, k, 11)
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    alpha = torch.from_numpy(a32 if k > 1 else a32[:, 0].copy()).to(DEV)
    y = torch.from_numpy(ry.astype(np.float32)).to(DEV)
    dx, ds, rdot = mp.mp_attention_backward(g, alpha, t["x"], t["dy"], y)
    buf = alpha.clone()
    dx2, ds2, rdot2 = mp.mp_attention_backward(g, buf, t["x"], t["dy"], y, out_dscores=buf)
    torch.cuda.synchronize()
    assert ds2.data_ptr() == buf.data_ptr()
    assert torch.equal(dx2, dx) and torch.equal(buf, ds) and torch.equal(rdot2, rdot)
    wide = synth.random_graph(300, 3000, 600, 67)
    tw = upload(wide, DEV)
    gw = mp.mp_graph_build(tw["src"], tw["dst"], wide.n)
    aw = torch.rand((wide.e, 3), device=DEV)
    yw = torch.zeros((wide.n, 600), device=DEV)
    with pytest.raises(ValueError):
        mp.mp_attention_backward(gw, aw, tw["x"], tw["dy"], yw, out_dscores=aw)


def _fwd_softmax_cases():
    yield "witness", synth.witness(), {}
    yield "empty", synth.random_graph(5, 0, 8, 61), {}
    yield "random_f32_h24", synth.random_graph(700, 9000, 24, 62), {}
    yield "random_bf16_h128", synth.random_graph(900, 20000, 128, 63, feat_dtype="bf16"), {}
    yield "random_f32_h7", synth.random_graph(300, 4000, 7, 64), {}              # scalar lanes
    yield "random_f32_h300", synth.random_graph(300, 4000, 300, 65), {}          # column blocks
    yield "power_law", _power_law(66), {}
    yield "power_law_four_wave_hubs", _power_law(67), {"hub_apart": 0, "hub_min_len": 4096}
    yield "rmat16", synth.rmat16(), {}                                          # 16-wave hubs


def _power_law(seed):
    return synth.chung_lu(seed=seed, n=20000, e=400000, cap=20000.0, h=64, feat_dtype="f32")


@pytest.mark.parametrize("idx", range(9))
def test_fwd_softmax_equals_softmax_then_forward(mp, idx):
    """mp_spmm_fwd_softmax (alpha formed at the fetch, never written) against
    mp_edge_softmax followed by mp_spmm_fwd on its alpha: Y and the row
    statistics bit for bit, on synchronously and asynchronously built graphs;
    that alpha against the oracle's softmax and Y against the oracle's
    aggregation with it."""
    name, wl, env = list(_fwd_softmax_cases())[idx]
    mp.mp_set_owner_overrides(**env)   # the module's fixture restores the rule
    print(f"case {name}: N={wl.n} E={wl.e} H={wl.h} {wl.feat_dtype}", flush=True)
    t = upload(wl, DEV)
    scores = torch.from_numpy(wl.w).to(DEV)
    for g in (mp.mp_graph_build(t["src"], t["dst"], wl.n),
              mp.mp_graph_build_async(t["src"], t["dst"], wl.n)):
        y, stats = mp.mp_spmm_fwd_softmax(g, scores, t["x"])
        alpha, ref_stats = mp.mp_edge_softmax(g, scores)
        ref_y = mp.mp_spmm_fwd(g, alpha, t["x"])
        torch.cuda.synchronize()
        assert torch.equal(stats, ref_stats), "row statistics"
        assert torch.equal(y, ref_y), "aggregation"
    if wl.e:
        # the weights used: alpha against the oracle's softmax, then Y against the
        # oracle's aggregation with those float32 weights
        _check_softmax(wl, wl.w, alpha, stats[:, 0], stats[:, 1])
        a32 = alpha.cpu().numpy()
        check_close("Y", y, *oracle.forward(wl.n, wl.src, wl.dst, a32, wl.x), TAU["f32"])


def test_fwd_softmax_rejections(mp):
    wl = synth.random_graph(50, 400, 8, 68)
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    s = torch.from_numpy(wl.w).to(DEV)
    with pytest.raises(TypeError):
        mp.mp_spmm_fwd_softmax(g, s.double(), t["x"])
    with pytest.raises(ValueError):
        mp.mp_spmm_fwd_softmax(g, s[:-1], t["x"])
    y = torch.empty((wl.n, wl.h), device=DEV)
    buf = torch.empty(2 * wl.n + 1, device=DEV)
    with pytest.raises(ValueError, match="align"):      # row statistics off their 8-byte line
        mp.mp_spmm_fwd_softmax(g, s, t["x"], out=y, out_row_stats=buf[1:].view(wl.n, 2))
    with pytest.raises(ValueError, match="overlap"):
        mp.mp_spmm_fwd_softmax(g, s, t["x"], out=y, out_row_stats=y.view(-1)[: 2 * wl.n].view(wl.n, 2))


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4, 6, 7, 8])
def test_attention_backward_scores_equals_alpha_form(mp, idx):
    """mp_attention_backward_scores (alpha formed in the transpose walk from the
    scores and the destinations' statistics) against mp_attention_backward
    given alpha from mp_edge_softmax: dX, the score gradients and the row dots
    bit for bit, on both build forms, and with the score gradients written
    over the scores."""
    name, wl, env = list(_fwd_softmax_cases())[idx]
    mp.mp_set_owner_overrides(**env)   # the module's fixture restores the rule
    print(f"case {name}: N={wl.n} E={wl.e} H={wl.h} {wl.feat_dtype}", flush=True)
    t = upload(wl, DEV)
    scores = torch.from_numpy(wl.w).to(DEV)
    for g in (mp.mp_graph_build(t["src"], t["dst"], wl.n),
              mp.mp_graph_build_async(t["src"], t["dst"], wl.n)):
        y, stats = mp.mp_spmm_fwd_softmax(g, scores, t["x"])
        alpha, _ = mp.mp_edge_softmax(g, scores)
        ref = mp.mp_attention_backward(g, alpha, t["x"], t["dy"], y)
        got = mp.mp_attention_backward_scores(g, scores, stats, t["x"], t["dy"], y)
        s_ip = scores.clone()
        ip = mp.mp_attention_backward_scores(g, s_ip, stats, t["x"], t["dy"], y, out_dscores=s_ip)
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), f"output {k}"
        assert torch.equal(ip[0], ref[0]) and torch.equal(s_ip, ref[1]), "in place"


def test_attention_backward_scores_rejections(mp):
    wl = synth.random_graph(300, 4000, 300, 69)            # wider than one column block
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    s = torch.from_numpy(wl.w).to(DEV)
    y, stats = mp.mp_spmm_fwd_softmax(g, s, t["x"])
    with pytest.raises(ValueError, match="fused walk"):
        mp.mp_attention_backward_scores(g, s, stats, t["x"], t["dy"], y)
    wl = synth.random_graph(50, 400, 8, 70)
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    s = torch.from_numpy(wl.w).to(DEV)
    y, stats = mp.mp_spmm_fwd_softmax(g, s, t["x"])
    buf = torch.empty(2 * wl.n + 1, device=DEV)
    buf[1:].copy_(stats.view(-1))
    with pytest.raises(ValueError, match="align"):
        mp.mp_attention_backward_scores(g, s, buf[1:].view(wl.n, 2), t["x"], t["dy"], y)
    with pytest.raises(ValueError, match="overlap"):
        mp.mp_attention_backward_scores(g, s, stats, t["x"], t["dy"], y,
                                        out_row_dot=stats.view(-1)[: wl.n])
