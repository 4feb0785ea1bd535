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
