"""Multi-head edge weights (w is [E, K]; head q owns columns [q*H/K, (q+1)*H/K))
on the device against the oracle's per-head aggregation, element by element
with the same rule as the scalar calls: |gpu - oracle| <= tau * S (tau 1e-5 for
fp32 features, 2e-2 for bf16 storage), exact zeros where an element has no
terms.  The fused backward must equal the two separate calls bitwise, and
K = 1 must equal the scalar calls bitwise."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.harness import TAU, check_close, upload

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def mp():
    import gnn_sparse_message_amd
    return gnn_sparse_message_amd


def _weights(e, k, seed):
    return np.random.default_rng(seed).uniform(-1, 1, (e, k)).astype(np.float32)


def _run(mp, wl, k, seed):
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    w_np = _weights(wl.e, k, seed)
    w = torch.from_numpy(w_np).to(DEV)
    y = mp.mp_spmm_fwd_heads(g, w, t["x"])
    dx = mp.mp_spmm_dx_heads(g, w, t["dy"])
    dw = mp.mp_edge_grad_dw_heads(g, t["x"], t["dy"], k)
    fdx, fdw = mp.mp_spmm_dx_edge_grad_heads(g, w, t["x"], t["dy"])
    torch.cuda.synchronize()
    return g, t, w_np, w, y, dx, dw, fdx, fdw


def _check(wl, k, w_np, y, dx, dw, fdx, fdw):
    tau = TAU[wl.feat_dtype]
    ry, sy = oracle.forward_heads(wl.n, wl.src, wl.dst, w_np, wl.x)
    rdx, sdx = oracle.input_grad_heads(wl.n, wl.src, wl.dst, w_np, wl.dy)
    rdw, sdw = oracle.edge_grad_heads(wl.src, wl.dst, wl.x, wl.dy, k)
    check_close("Y", y, ry, sy, tau)
    check_close("dX", dx, rdx, sdx, tau)
    check_close("dw", dw, rdw, sdw, tau)
    # the fused pass gives the same bits as the two separate calls
    assert torch.equal(fdx, dx), "fused dX differs from mp_spmm_dx_heads"
    assert torch.equal(fdw, dw), "fused dw differs from mp_edge_grad_dw_heads"


# Head widths: vector lanes with a power-of-two lane count per head (8, 16, 32,
# 64 fp32 / bf16), lane counts that are not powers of two (12, 24, 40), the
# scalar path (1, 3, 5: not a multiple of the vector width) and widths that need
# column blocks or the unfused backward (K * H/K above 64 lanes).
@pytest.mark.parametrize("feat", ["f32", "bf16"])
@pytest.mark.parametrize("k,hh", [(2, 1), (3, 3), (2, 5), (4, 8), (2, 12), (4, 16), (3, 24),
                                  (2, 40), (4, 32), (8, 16), (2, 64), (4, 100), (8, 64),
                                  (16, 8), (3, 128)])
def test_head_widths(mp, k, hh, feat):
    wl = synth.random_graph(700, 9000, k * hh, 1000 + 7 * k + hh, feat_dtype=feat)
    g, t, w_np, w, y, dx, dw, fdx, fdw = _run(mp, wl, k, k * 100 + hh)
    _check(wl, k, w_np, y, dx, dw, fdx, fdw)


@pytest.mark.parametrize("feat,k,hh", [("bf16", 4, 32), ("f32", 4, 16), ("bf16", 8, 16),
                                       ("f32", 3, 12)])
def test_power_law_owner_kinds(mp, feat, k, hh):
    """Hub rows (workgroup owners), long rows (wave owners), short and empty rows."""
    wl = synth.chung_lu(seed=31, n=20000, e=400000, cap=20000.0, h=k * hh, feat_dtype=feat)
    deg = np.bincount(wl.dst, minlength=wl.n)
    assert deg.max() >= 4096 and (deg == 0).any()
    g, t, w_np, w, y, dx, dw, fdx, fdw = _run(mp, wl, k, 77)
    _check(wl, k, w_np, y, dx, dw, fdx, fdw)


@pytest.mark.parametrize("feat,h", [("f32", 16), ("bf16", 128), ("f32", 300)])
def test_one_head_equals_scalar_calls(mp, feat, h):
    wl = synth.random_graph(900, 12000, h, 555, feat_dtype=feat)
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    w1 = t["w"].reshape(wl.e, 1)
    pairs = [(mp.mp_spmm_fwd_heads(g, w1, t["x"]), mp.mp_spmm_fwd(g, t["w"], t["x"])),
             (mp.mp_spmm_dx_heads(g, w1, t["dy"]), mp.mp_spmm_dx(g, t["w"], t["dy"])),
             (mp.mp_edge_grad_dw_heads(g, t["x"], t["dy"], 1)[:, 0],
              mp.mp_edge_grad_dw(g, t["x"], t["dy"]))]
    fdx, fdw = mp.mp_spmm_dx_edge_grad_heads(g, w1, t["x"], t["dy"])
    sdx, sdw = mp.mp_spmm_dx_edge_grad(g, t["w"], t["x"], t["dy"])
    pairs += [(fdx, sdx), (fdw[:, 0], sdw)]
    torch.cuda.synchronize()
    for a, b in pairs:
        assert torch.equal(a, b)


def test_equal_head_weights_sum_to_scalar_edge_grad(mp):
    """Per-head dw summed over the heads is the single-head dw (to rounding)."""
    wl = synth.random_graph(500, 8000, 64, 556)
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    dwh = mp.mp_edge_grad_dw_heads(g, t["x"], t["dy"], 4)
    dw = mp.mp_edge_grad_dw(g, t["x"], t["dy"])
    torch.cuda.synchronize()
    rdw, sdw = oracle.edge_grad(wl.src, wl.dst, wl.x, wl.dy)
    check_close("sum over heads", dwh.sum(dim=1), rdw, sdw, 4 * TAU["f32"])
    check_close("scalar", dw, rdw, sdw, TAU["f32"])


@pytest.mark.parametrize("n,e", [(1, 0), (5, 0), (1, 7), (3000, 5)])
def test_degenerate_graphs(mp, n, e):
    wl = synth.random_graph(n, e, 12, 557)
    g, t, w_np, w, y, dx, dw, fdx, fdw = _run(mp, wl, 3, 9)
    _check(wl, 3, w_np, y, dx, dw, fdx, fdw)
    assert dw.shape == (e, 3)


def test_rejections(mp):
    wl = synth.random_graph(100, 500, 12, 558)
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    w5 = torch.zeros((wl.e, 5), device=DEV)
    with pytest.raises(ValueError):                 # 5 heads do not divide 12 columns
        mp.mp_spmm_fwd_heads(g, w5, t["x"])
    with pytest.raises(ValueError):
        mp.mp_edge_grad_dw_heads(g, t["x"], t["dy"], 5)
    with pytest.raises(ValueError):                 # w must be [E, K]
        mp.mp_spmm_dx_heads(g, torch.zeros(wl.e * 3, device=DEV), t["dy"])
    with pytest.raises(TypeError):
        mp.mp_spmm_fwd_heads(g, torch.zeros((wl.e, 3), device=DEV, dtype=torch.float64), t["x"])
    # the C entry points check the head count themselves
    lib = mp._lib
    y = torch.empty((wl.n, 12), device=DEV)
    w3 = torch.zeros((wl.e, 3), device=DEV)
    for heads in (0, -1, 5, 13):
        st = lib.mp_spmm_fwd_heads(ctypes.byref(g._desc), w3.data_ptr(), heads,
                                   t["x"].data_ptr(), mp.MP_F32, 12, y.data_ptr(), None)
        assert st == mp.MP_ERR_SHAPE, (heads, st)
    dw = torch.empty((wl.e, 3), device=DEV)
    st = lib.mp_edge_grad_dw_heads(ctypes.byref(g._desc), t["x"].data_ptr(), t["dy"].data_ptr(),
                                   mp.MP_F32, 12, 5, dw.data_ptr(), None)
    assert st == mp.MP_ERR_SHAPE
    # dw must not overlap the weights in the fused call
    dx = torch.empty((wl.n, 12), device=DEV)
    with pytest.raises(ValueError):
        mp.mp_spmm_dx_edge_grad_heads(g, w3, t["x"], t["dy"], out_dx=dx, out_dw=w3)
