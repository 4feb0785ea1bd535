"""The calls on weights and gradients interleaved in one [E][2] array: the
fused backward (mp_spmm_dx_edge_grad_pair) with dX and dw bit for bit equal to
the two-array call, and the forward (mp_spmm_fwd_pair) bit for bit equal to
mp_spmm_fwd (both held to the oracle by the parity tests), the weight half of
the array left as it was, on an asynchronously built graph as well, and their
rejections; wide rows (column blocks) for the forward."""
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


CASES = [
    ("witness", lambda: synth.witness()),
    ("one_node_no_edges", lambda: synth.random_graph(1, 0, 8, 71)),
    ("self_loops_one_node", lambda: synth.random_graph(1, 40, 4, 72)),
    ("random_f32_h16", lambda: synth.random_graph(700, 9000, 16, 73)),
    ("ragged_f32_h6", lambda: synth.random_graph(900, 12000, 6, 74)),
    ("ragged_bf16_h15", lambda: synth.random_graph(900, 12000, 15, 75, feat_dtype="bf16")),
    ("power_law_bf16_h128", lambda: synth.chung_lu(seed=76, n=20000, e=400000, cap=20000.0,
                                                   h=128, feat_dtype="bf16")),
    ("power_law_f32_h256", lambda: synth.chung_lu(seed=77, n=8000, e=160000, cap=8000.0,
                                                  h=256, feat_dtype="f32")),
]


def _pair(t, wl):
    wg = torch.empty((wl.e, 2), dtype=torch.float32, device=DEV)
    wg[:, 0] = t["w"]
    wg[:, 1] = float("nan")
    return wg


@pytest.mark.parametrize("idx", range(len(CASES)), ids=[c[0] for c in CASES])
def test_pair_equals_two_arrays(mp, idx):
    wl = CASES[idx][1]()
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    wg = _pair(t, wl)
    dx = mp.mp_spmm_dx_edge_grad_pair(g, wg, t["x"], t["dy"])
    rdx, rdw = mp.mp_spmm_dx_edge_grad(g, t["w"], t["x"], t["dy"])
    torch.cuda.synchronize()
    assert torch.equal(dx, rdx)
    assert torch.equal(wg[:, 1], rdw)
    assert torch.equal(wg[:, 0], t["w"])                  # the weights are not written
    y = mp.mp_spmm_fwd_pair(g, wg, t["x"])
    ry = mp.mp_spmm_fwd(g, t["w"], t["x"])
    torch.cuda.synchronize()
    assert torch.equal(y, ry)


@pytest.mark.parametrize("h", [7, 300, 600])
def test_pair_forward_wide_and_scalar_rows(mp, h):
    """Scalar lanes (H = 7) and column blocks (H = 300, 600) read the weights
    at the same stride."""
    wl = synth.random_graph(400, 5000, h, 90 + h)
    t = upload(wl, DEV)
    for g in (mp.mp_graph_build(t["src"], t["dst"], wl.n),
              mp.mp_graph_build_async(t["src"], t["dst"], wl.n)):
        wg = _pair(t, wl)
        y = mp.mp_spmm_fwd_pair(g, wg, t["x"])
        ry = mp.mp_spmm_fwd(g, t["w"], t["x"])
        torch.cuda.synchronize()
        assert torch.equal(y, ry)
    check_close("Y", y, *oracle.forward(wl.n, wl.src, wl.dst, wl.w, wl.x), TAU["f32"])


def test_pair_against_oracle(mp):
    wl = synth.chung_lu(seed=78, n=6000, e=90000, cap=6000.0, h=64, feat_dtype="bf16")
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    wg = _pair(t, wl)
    dx = mp.mp_spmm_dx_edge_grad_pair(g, wg, t["x"], t["dy"])
    torch.cuda.synchronize()
    check_close("dX", dx, *oracle.input_grad(wl.n, wl.src, wl.dst, wl.w, wl.dy), TAU["f32"])
    check_close("dw", wg[:, 1].contiguous(), *oracle.edge_grad(wl.src, wl.dst, wl.x, wl.dy),
                TAU["f32"])


def test_pair_async_graph(mp):
    wl = synth.chung_lu(seed=79, n=6000, e=90000, cap=6000.0, h=64, feat_dtype="f32")
    t = upload(wl, DEV)
    g1 = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    g2 = mp.mp_graph_build_async(t["src"], t["dst"], wl.n)
    a, b = _pair(t, wl), _pair(t, wl)
    dxa = mp.mp_spmm_dx_edge_grad_pair(g1, a, t["x"], t["dy"])
    dxb = mp.mp_spmm_dx_edge_grad_pair(g2, b, t["x"], t["dy"])
    torch.cuda.synchronize()
    assert torch.equal(dxa, dxb) and torch.equal(a, b)
    mp.mp_graph_finish(g2)


def test_pair_rejections(mp):
    wl = synth.random_graph(100, 500, 8, 80)
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    wg = _pair(t, wl)
    with pytest.raises(ValueError):                   # [E] is not [E, 2]
        mp.mp_spmm_dx_edge_grad_pair(g, t["w"], t["x"], t["dy"])
    with pytest.raises(TypeError):
        mp.mp_spmm_dx_edge_grad_pair(g, wg.double(), t["x"], t["dy"])
    with pytest.raises(ValueError):                   # dX inside wg
        big = torch.empty((wl.n * 8 + wl.e * 2,), device=DEV)
        wv = big[:wl.e * 2].view(wl.e, 2)
        mp.mp_spmm_dx_edge_grad_pair(g, wv, t["x"], t["dy"],
                                     out_dx=big[wl.e:wl.e + wl.n * 8].view(wl.n, 8))
    with pytest.raises(ValueError):                   # the forward's output inside wg
        big = torch.empty((wl.n * 8 + wl.e * 2,), device=DEV)
        wv = big[:wl.e * 2].view(wl.e, 2)
        mp.mp_spmm_fwd_pair(g, wv, t["x"], out=big[wl.e:wl.e + wl.n * 8].view(wl.n, 8))
    with pytest.raises(ValueError):
        mp.mp_spmm_fwd_pair(g, t["w"], t["x"])
    wide = synth.random_graph(100, 500, 600, 81)      # beyond one column block
    tw = upload(wide, DEV)
    gw = mp.mp_graph_build(tw["src"], tw["dst"], wide.n)
    with pytest.raises(ValueError):
        mp.mp_spmm_dx_edge_grad_pair(gw, _pair(tw, wide), tw["x"], tw["dy"])
