"""Forward, input gradient and edge gradient on the device against the oracle,
element by element: |gpu - oracle| <= tau * S (tau 1e-5 for fp32 features,
2e-2 for bf16 storage), exact zeros where an element has no terms, exact
equality on the witness."""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.harness import TAU, check_close, check_floats, check_structure, run_path, upload

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def mp():
    import gnn_sparse_message_amd
    return gnn_sparse_message_amd


def test_witness_exact(mp):
    wl = synth.witness()
    g, t, y, dx, dw = run_path(mp, wl, DEV)
    check_structure(g, wl)
    # Hand values (tests/golden/witness.json): small integers, exact in fp32.
    assert y[:, 0].cpu().tolist() == [0.0, 6.0, 0.0]
    assert dx[:, 0].cpu().tolist() == [29.0, -7.0, 0.0]
    assert dw.cpu().tolist() == [14.0, 28.0, 10.0]


def test_tiny_uniform(mp):
    wl = synth.tiny_uniform()
    g, t, y, dx, dw = run_path(mp, wl, DEV)
    check_structure(g, wl)
    check_floats(wl, y, dx, dw)


# Feature widths covering every lane count, the scalar path (H not a multiple of
# the vector width), ragged lanes (H not a power of two) and column blocks
# (H above 64 lanes x vector width).
@pytest.mark.parametrize("feat", ["f32", "bf16"])
@pytest.mark.parametrize("h", [1, 2, 3, 4, 5, 8, 12, 16, 24, 32, 40, 64, 100, 128, 200, 256, 264,
                               512, 520, 1024])
def test_feature_widths(mp, h, feat):
    wl = synth.random_graph(600, 7000, h, 100 + h, feat_dtype=feat)
    g, t, y, dx, dw = run_path(mp, wl, DEV)
    check_floats(wl, y, dx, dw)


def _power_law_small(seed, n=20000, e=400000, h=32, feat="f32"):
    """A small Chung-Lu graph: hub rows, long rows, short rows and empty rows together."""
    wl = synth.chung_lu(seed=seed, n=n, e=e, cap=20000.0, h=h, feat_dtype=feat)
    return wl


@pytest.mark.parametrize("apart", [0, 1])
@pytest.mark.parametrize("feat,h", [("f32", 16), ("f32", 64), ("bf16", 128), ("f32", 256)])
def test_power_law_all_owner_kinds(mp, feat, h, apart):
    """Rows of 4096 edges and more as four-wave workgroups of the main launch
    (the large-graph form) or as 16-wave workgroups of their own launch."""
    wl = _power_law_small(40 + h, h=h, feat=feat)
    deg = np.bincount(wl.dst, minlength=wl.n)
    assert deg.max() >= 4096 and (deg == 0).any()
    with mp.owner_overrides(hub_min_len=4096, hub_apart=apart):
        g, t, y, dx, dw = run_path(mp, wl, DEV)
    check_structure(g, wl)
    check_floats(wl, y, dx, dw)


@pytest.mark.parametrize("hub,wave,apart", [(1, 1, 0), (1, 1, 1),
                                            (1000000000, 1000000000, 0),
                                            (64, 2, 0), (64, 2, 1),
                                            (2, 1000000000, 1)])
def test_owner_thresholds_do_not_change_results(mp, hub, wave, apart):
    """Every row handled by workgroups (four waves in the main launch or 16 in
    their own), by single lane groups, or mixed: same values to tolerance (the
    split only changes the summation order)."""
    wl = _power_law_small(7, n=3000, e=60000, h=40)
    with mp.owner_overrides(hub_min_len=hub, hub_apart=apart, wave_min_len=wave):
        g, t, y, dx, dw = run_path(mp, wl, DEV)
    check_floats(wl, y, dx, dw)


def test_hub_row_only(mp):
    wl = synth.random_graph(3000, 120000, 64, 21)
    wl.dst[:] = 7
    g, t, y, dx, dw = run_path(mp, wl, DEV)
    check_floats(wl, y, dx, dw)


@pytest.mark.parametrize("n,e", [(1, 0), (5, 0), (1, 1), (1, 300), (2, 1), (4097, 1)])
def test_degenerate(mp, n, e):
    wl = synth.random_graph(n, e, 8, 30 + n + e)
    g, t, y, dx, dw = run_path(mp, wl, DEV)
    check_structure(g, wl)
    check_floats(wl, y, dx, dw)
    if e == 0:
        assert torch.count_nonzero(y) == 0 and torch.count_nonzero(dx) == 0 and dw.numel() == 0


def test_one_node_self_loops_closed_form(mp):
    wl = synth.random_graph(1, 50, 16, 33)
    g, t, y, dx, dw = run_path(mp, wl, DEV)
    ref = wl.w.astype(np.float64).sum() * wl.x[0].astype(np.float64)
    np.testing.assert_allclose(y[0].cpu().numpy(), ref, rtol=1e-5, atol=1e-5)


def test_sbm(mp):
    wl = synth.sbm()
    g, t, y, dx, dw = run_path(mp, wl, DEV)
    check_structure(g, wl)
    check_floats(wl, y, dx, dw)


def test_rmat16(mp):
    wl = synth.rmat16()
    g, t, y, dx, dw = run_path(mp, wl, DEV, torch.int32)
    check_structure(g, wl)
    check_floats(wl, y, dx, dw)


def test_minibatches(mp):
    for wl in synth.minibatches(3):
        g, t, y, dx, dw = run_path(mp, wl, DEV)
        check_structure(g, wl)
        check_floats(wl, y, dx, dw)


def test_bf16_accumulates_in_fp32(mp):
    """bf16 storage, fp32 arithmetic: the fp32 bound must hold as well, which it
    would not if products or sums were rounded to bf16."""
    wl = synth.random_graph(2000, 60000, 128, 51, feat_dtype="bf16")
    g, t, y, dx, dw = run_path(mp, wl, DEV)
    check_floats(wl, y, dx, dw, tau=TAU["f32"])


def test_permuted_coo(mp):
    """Permuting the COO list leaves Y and dX unchanged (to tolerance) and permutes dw."""
    wl = synth.random_graph(900, 20000, 32, 61)
    g, t, y, dx, dw = run_path(mp, wl, DEV)
    perm = np.random.default_rng(5).permutation(wl.e)
    wl2 = synth.Workload("perm", wl.n, wl.src[perm], wl.dst[perm], wl.w[perm], wl.x, wl.dy)
    g2, t2, y2, dx2, dw2 = run_path(mp, wl2, DEV)
    check_floats(wl2, y2, dx2, dw2)
    ry, sy = oracle.forward(wl.n, wl.src, wl.dst, wl.w, wl.x)
    check_close("Y(perm) vs oracle(orig)", y2, ry, sy, TAU["f32"])
    assert torch.equal(dw2.cpu(), dw.cpu()[perm])


def test_deterministic(mp):
    wl = _power_law_small(8, n=5000, e=100000, h=64)
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    outs = []
    for _ in range(2):
        outs.append((mp.mp_spmm_fwd(g, t["w"], t["x"]), mp.mp_spmm_dx(g, t["w"], t["dy"]),
                     mp.mp_edge_grad_dw(g, t["x"], t["dy"])))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_outputs_overwritten_not_accumulated(mp):
    wl = synth.random_graph(300, 3000, 16, 71)
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    y = torch.full((wl.n, 16), 1234.5, device=DEV)
    dw = torch.full((wl.e,), -7.0, device=DEV)
    mp.mp_spmm_fwd(g, t["w"], t["x"], out=y)
    mp.mp_edge_grad_dw(g, t["x"], t["dy"], out=dw)
    torch.cuda.synchronize()
    ry, sy = oracle.forward(wl.n, wl.src, wl.dst, wl.w, wl.x)
    check_close("Y", y, ry, sy, TAU["f32"])
    rdw, sdw = oracle.edge_grad(wl.src, wl.dst, wl.x, wl.dy)
    check_close("dw", dw, rdw, sdw, TAU["f32"])


def test_rejections(mp):
    wl = synth.random_graph(100, 500, 8, 81)
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    with pytest.raises(TypeError):                       # float64 features
        mp.mp_spmm_fwd(g, t["w"], t["x"].double())
    with pytest.raises(TypeError):                       # x, dy dtypes differ
        mp.mp_edge_grad_dw(g, t["x"], t["dy"].bfloat16())
    with pytest.raises(ValueError):                      # host memory
        mp.mp_spmm_fwd(g, t["w"].cpu(), t["x"])
    with pytest.raises(ValueError):                      # wrong row count
        mp.mp_spmm_fwd(g, t["w"], t["x"][:50])
    with pytest.raises(ValueError):                      # output aliases the input
        mp.mp_spmm_fwd(g, t["w"], t["x"], out=t["x"])
    with pytest.raises(ValueError):                      # output aliases the graph
        mp.mp_edge_grad_dw(g, t["x"], t["dy"], out=g.col.view(torch.float32))
    with pytest.raises(ValueError):                      # wrong weight count
        mp.mp_spmm_dx(g, t["w"][:10], t["dy"])
    # nothing was launched by the rejected calls: the library still works
    y = mp.mp_spmm_fwd(g, t["w"], t["x"])
    torch.cuda.synchronize()
    ry, sy = oracle.forward(wl.n, wl.src, wl.dst, wl.w, wl.x)
    check_close("Y", y, ry, sy, TAU["f32"])


@pytest.mark.parametrize("feat,h", [("f32", 1), ("f32", 3), ("f32", 16), ("f32", 64), ("f32", 256),
                                    ("f32", 260), ("bf16", 8), ("bf16", 128), ("bf16", 512),
                                    ("bf16", 520)])
def test_fused_backward_matches_separate_calls(mp, feat, h):
    """mp_spmm_dx_edge_grad: dX and dw equal the separate entry points bit for bit
    and the oracle to tolerance, on a graph with all owner kinds."""
    wl = _power_law_small(90 + h, n=4000, e=80000, h=h, feat=feat)
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    dx_sep = mp.mp_spmm_dx(g, t["w"], t["dy"])
    dw_sep = mp.mp_edge_grad_dw(g, t["x"], t["dy"])
    dx, dw = mp.mp_spmm_dx_edge_grad(g, t["w"], t["x"], t["dy"])
    torch.cuda.synchronize()
    assert torch.equal(dx, dx_sep)
    assert torch.equal(dw, dw_sep)
    rdx, sdx = oracle.input_grad(wl.n, wl.src, wl.dst, wl.w, wl.dy)
    rdw, sdw = oracle.edge_grad(wl.src, wl.dst, wl.x, wl.dy)
    check_close("dX", dx, rdx, sdx, TAU[feat])
    check_close("dw", dw, rdw, sdw, TAU[feat])


def test_fused_backward_witness_and_empty(mp):
    wl = synth.witness()
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    dx, dw = mp.mp_spmm_dx_edge_grad(g, t["w"], t["x"], t["dy"])
    assert dx[:, 0].cpu().tolist() == [29.0, -7.0, 0.0]
    assert dw.cpu().tolist() == [14.0, 28.0, 10.0]
    wl = synth.random_graph(7, 0, 16, 3)
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    dx, dw = mp.mp_spmm_dx_edge_grad(g, t["w"], t["x"], t["dy"])
    torch.cuda.synchronize()
    assert torch.count_nonzero(dx) == 0 and dw.numel() == 0


def test_fused_backward_rejections(mp):
    wl = synth.random_graph(100, 500, 8, 82)
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    dx = torch.empty((wl.n, 8), device=DEV)
    with pytest.raises(ValueError):                      # dw aliases dx
        mp.mp_spmm_dx_edge_grad(g, t["w"], t["x"], t["dy"], out_dx=dx,
                                out_dw=dx.view(-1)[:wl.e])
    with pytest.raises(ValueError):                      # dx aliases x
        mp.mp_spmm_dx_edge_grad(g, t["w"], t["x"], t["dy"], out_dx=t["x"])
    with pytest.raises(TypeError):                       # x and dy dtypes differ
        mp.mp_spmm_dx_edge_grad(g, t["w"], t["x"].bfloat16(), t["dy"])
