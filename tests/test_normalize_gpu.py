"""Degree normalisation (mp_edge_normalize) against the oracle, and the
mean / symmetric-normalised layer end to end.  The device forms the factor in
double, rounds it once to fp32 and applies one fp32 multiply, so each output
is within about one fp32 ulp of the fp64 oracle; the tests allow 2^-22
relative."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.harness import TAU, check_close, upload

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
REL = 2.0 ** -22


@pytest.fixture(scope="module")
def mp():
    import gnn_sparse_message_amd
    return gnn_sparse_message_amd


def _graph(mp, wl):
    t = upload(wl, DEV)
    return mp.mp_graph_build(t["src"], t["dst"], wl.n), t


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("n,e,seed", [(1, 0, 1), (1, 9, 2), (3, 3, 3), (500, 8000, 4),
                                      (100000, 300000, 5)])
def test_against_oracle(mp, mode, n, e, seed):
    wl = synth.random_graph(n, e, 1, seed)
    g, t = _graph(mp, wl)
    out = mp.mp_edge_normalize(g, mode, t["w"])
    torch.cuda.synchronize()
    ref = oracle.edge_normalize(wl.n, wl.src, wl.dst, mode, wl.w)
    got = out.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= REL * np.abs(ref)), np.max(np.abs(got - ref) / np.abs(ref))


@pytest.mark.parametrize("mode", [1, 2])
def test_power_law_and_in_place(mp, mode):
    wl = synth.chung_lu(seed=29, n=20000, e=400000, cap=20000.0, h=1, feat_dtype="f32")
    g, t = _graph(mp, wl)
    ref = oracle.edge_normalize(wl.n, wl.src, wl.dst, mode, wl.w)
    buf = t["w"].clone()
    mp.mp_edge_normalize(g, mode, buf, out=buf)                   # in place
    torch.cuda.synchronize()
    got = buf.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= REL * np.abs(ref))


def test_mean_of_ones_sums_to_one(mp):
    wl = synth.random_graph(3000, 50000, 1, 6)
    g, t = _graph(mp, wl)
    out = mp.mp_edge_normalize(g, mp.MP_NORM_MEAN, torch.ones(wl.e, device=DEV))
    sums = np.bincount(wl.dst, weights=out.cpu().numpy().astype(np.float64), minlength=wl.n)
    has = np.bincount(wl.dst, minlength=wl.n) > 0
    np.testing.assert_allclose(sums[has], 1.0, rtol=1e-5)


@pytest.mark.parametrize("mode", [1, 2])
def test_normalized_layer_end_to_end(mp, mode):
    wl = synth.chung_lu(seed=31, n=6000, e=120000, cap=6000.0, h=32, feat_dtype="f32")
    g, t = _graph(mp, wl)
    wn = mp.mp_edge_normalize(g, mode, t["w"])
    y = mp.mp_spmm_fwd(g, wn, t["x"])
    dx, dwn = mp.mp_spmm_dx_edge_grad(g, wn, t["x"], t["dy"])
    dw = mp.mp_edge_normalize(g, mode, dwn)
    torch.cuda.synchronize()
    wn32 = wn.cpu().numpy()
    ry, sy = oracle.forward(wl.n, wl.src, wl.dst, wn32, wl.x)
    check_close("Y", y, ry, sy, TAU["f32"])
    rdx, sdx = oracle.input_grad(wl.n, wl.src, wl.dst, wn32, wl.dy)
    check_close("dX", dx, rdx, sdx, TAU["f32"])
    rdwn, sdwn = oracle.edge_grad(wl.src, wl.dst, wl.x, wl.dy)
    rdw = oracle.edge_normalize(wl.n, wl.src, wl.dst, mode, rdwn.astype(np.float32))
    sdw = oracle.edge_normalize(wl.n, wl.src, wl.dst, mode, sdwn.astype(np.float32))
    check_close("dw", dw, rdw, sdw, TAU["f32"] + 4 * REL)


def test_rejections(mp):
    wl = synth.random_graph(100, 500, 1, 7)
    g, t = _graph(mp, wl)
    with pytest.raises(TypeError):                       # unknown mode
        mp.mp_edge_normalize(g, 5, t["w"])
    with pytest.raises(ValueError):                      # output overlaps the input, shifted
        buf = torch.zeros(wl.e + 1, device=DEV)
        mp.mp_edge_normalize(g, 1, buf[:-1], out=buf[1:])
    with pytest.raises(ValueError):                      # output overlaps the graph
        mp.mp_edge_normalize(g, 1, t["w"], out=g.col.view(torch.float32))
    with pytest.raises(TypeError):
        mp.mp_edge_normalize(g, 1, t["w"].double())


# ---------------------------------------------------------------- normalised at the fetch
#
# mp_spmm_fwd_norm / mp_spmm_dx_norm / mp_spmm_dx_edge_grad_norm form each
# edge's factor exactly as mp_edge_normalize does and use w * factor in the same
# accumulation order, so they equal the two-call chains bit for bit; the chains
# themselves are held to the oracle above and below.

def _fetch_cases():
    yield "witness", synth.witness()
    yield "one_node_no_edges", synth.random_graph(1, 0, 8, 41)
    yield "self_loops_one_node", synth.random_graph(1, 9, 4, 42)
    yield "random_f32_h16", synth.random_graph(700, 9000, 16, 43)
    yield "ragged_f32_h6", synth.random_graph(900, 12000, 6, 44)
    yield "power_law_f32_h32", synth.chung_lu(seed=45, n=20000, e=400000, cap=20000.0, h=32,
                                              feat_dtype="f32")
    yield "power_law_bf16_h128", synth.chung_lu(seed=46, n=8000, e=200000, cap=8000.0, h=128,
                                                feat_dtype="bf16")
    yield "wide_f32_h600", synth.random_graph(400, 5000, 600, 47)


FETCH_CASES = list(_fetch_cases())


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("idx", range(len(FETCH_CASES)), ids=[c[0] for c in FETCH_CASES])
def test_fetch_normalisation_equals_two_calls(mp, mode, idx):
    wl = FETCH_CASES[idx][1]
    g, t = _graph(mp, wl)
    wn = mp.mp_edge_normalize(g, mode, t["w"])
    y_ref = mp.mp_spmm_fwd(g, wn, t["x"])
    dx_ref = mp.mp_spmm_dx(g, wn, t["dy"])
    dw_ref = mp.mp_edge_normalize(g, mode, mp.mp_edge_grad_dw(g, t["x"], t["dy"]))
    y = mp.mp_spmm_fwd_norm(g, mode, t["w"], t["x"])
    dx = mp.mp_spmm_dx_norm(g, mode, t["w"], t["dy"])
    dx2, dw = mp.mp_spmm_dx_edge_grad_norm(g, mode, t["w"], t["x"], t["dy"])
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref), "forward"
    assert torch.equal(dx, dx_ref), "input gradient"
    assert torch.equal(dx2, dx_ref), "fused input gradient"
    assert torch.equal(dw, dw_ref), "fused weight gradient"


@pytest.mark.parametrize("mode", [1, 2])
def test_fetch_normalisation_against_oracle(mp, mode):
    """The whole normalised layer from raw weights against the oracle: weights
    normalised by the oracle (rounded to fp32, within 2^-22 of the device's),
    then the oracle's aggregation, input gradient and edge gradient, the last
    scaled by the oracle's factors."""
    wl = synth.chung_lu(seed=48, n=20000, e=400000, cap=20000.0, h=64, feat_dtype="bf16")
    g, t = _graph(mp, wl)
    y = mp.mp_spmm_fwd_norm(g, mode, t["w"], t["x"])
    dx, dw = mp.mp_spmm_dx_edge_grad_norm(g, mode, t["w"], t["x"], t["dy"])
    torch.cuda.synchronize()
    wn = oracle.edge_normalize(wl.n, wl.src, wl.dst, mode, wl.w).astype(np.float32)
    ry, sy = oracle.forward(wl.n, wl.src, wl.dst, wn, wl.x)
    check_close("Y", y, ry, sy, TAU["f32"])
    rdx, sdx = oracle.input_grad(wl.n, wl.src, wl.dst, wn, wl.dy)
    check_close("dX", dx, rdx, sdx, TAU["f32"])
    factor = oracle.edge_normalize(wl.n, wl.src, wl.dst, mode, np.ones(wl.e, np.float32))
    rdot, sdot = oracle.edge_grad(wl.src, wl.dst, wl.x, wl.dy)
    check_close("dw", dw, rdot * factor, sdot * factor, TAU["f32"] + 4 * REL)


def test_fetch_normalisation_async_graph(mp):
    """A graph whose class counts are still on the device gives the same bits."""
    wl = synth.chung_lu(seed=49, n=6000, e=90000, cap=6000.0, h=64, feat_dtype="f32")
    t = upload(wl, DEV)
    g1 = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    g2 = mp.mp_graph_build_async(t["src"], t["dst"], wl.n)
    for mode in (1, 2):
        a = [mp.mp_spmm_fwd_norm(g1, mode, t["w"], t["x"]),
             *mp.mp_spmm_dx_edge_grad_norm(g1, mode, t["w"], t["x"], t["dy"])]
        b = [mp.mp_spmm_fwd_norm(g2, mode, t["w"], t["x"]),
             *mp.mp_spmm_dx_edge_grad_norm(g2, mode, t["w"], t["x"], t["dy"])]
        torch.cuda.synchronize()
        for u, v in zip(a, b):
            assert torch.equal(u, v)
    mp.mp_graph_finish(g2)


def test_fetch_normalisation_rejections(mp):
    wl = synth.random_graph(100, 500, 8, 50)
    g, t = _graph(mp, wl)
    with pytest.raises(TypeError):                       # unknown mode
        mp.mp_spmm_fwd_norm(g, 0, t["w"], t["x"])
    with pytest.raises(TypeError):
        mp.mp_spmm_dx_norm(g, 3, t["w"], t["dy"])
    with pytest.raises(TypeError):
        mp.mp_spmm_dx_edge_grad_norm(g, 7, t["w"], t["x"], t["dy"])
    with pytest.raises(ValueError):                      # output aliases the features
        mp.mp_spmm_fwd_norm(g, 1, t["w"], t["x"], out=t["x"])
    with pytest.raises(ValueError):                      # dw aliases w
        mp.mp_spmm_dx_edge_grad_norm(g, 2, t["w"], t["x"], t["dy"], out_dw=t["w"])
