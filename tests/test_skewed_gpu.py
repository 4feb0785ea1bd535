"""A large skewed graph, RMAT scale 20 (N = 1,048,576, E = 16,777,216, H = 128
fp32; the RMAT-16 recipe with 20 levels, edge factor 16), whose longest rows
start far beyond eight wave-slot shares: its rows of 128 edges and more go to
16-wave workgroups in a launch of their own, in both directions.  Every output is compared with the oracle in full; the fused
backward bit for bit with the two separate calls; every compute call on the
asynchronously built graph (owners derived on the device) bit for bit with the
synchronously built one."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.harness import TAU, check_close, check_structure, upload

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
DEV = torch.device("cuda:0")
WAVE_SLOTS = 256 * 4 * 4


def _outputs(mp, g, t):
    y = mp.mp_spmm_fwd(g, t["w"], t["x"])
    dx = mp.mp_spmm_dx(g, t["w"], t["dy"])
    dw = mp.mp_edge_grad_dw(g, t["x"], t["dy"])
    fdx, fdw = mp.mp_spmm_dx_edge_grad(g, t["w"], t["x"], t["dy"])
    return y, dx, dw, fdx, fdw


@pytest.fixture(scope="module")
def run():
    import gnn_sparse_message_amd as mp
    wl = synth.rmat(20, 16, 8, 128, name="rmat20")
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    ga = mp.mp_graph_build_async(t["src"], t["dst"], wl.n)
    sync = _outputs(mp, g, t)
    asyn = _outputs(mp, ga, t)
    torch.cuda.synchronize()
    out = {"async_equal": [bool(torch.equal(a, b)) for a, b in zip(asyn, sync)],
           "fused_equal": [bool(torch.equal(sync[3], sync[1])), bool(torch.equal(sync[4], sync[2]))],
           "y": sync[0].cpu().numpy(), "dx": sync[1].cpu().numpy(), "dw": sync[2].cpu().numpy()}
    check_structure(g, wl)
    del t, g, ga, sync, asyn
    torch.cuda.empty_cache()
    return wl, out


def test_skewed_graph_takes_the_16_wave_launch(run):
    wl, _ = run
    share = wl.e // WAVE_SLOTS
    for key in (wl.dst, wl.src):
        longest = int(np.bincount(key, minlength=wl.n).max())
        top_class_start = 1 << (longest.bit_length() - 1)
        assert top_class_start > 8 * share, (longest, share)


def test_skewed_outputs_against_oracle(run):
    wl, out = run
    tau = TAU["f32"]
    check_close("Y", out["y"], *oracle.forward(wl.n, wl.src, wl.dst, wl.w, wl.x), tau)
    check_close("dX", out["dx"], *oracle.input_grad(wl.n, wl.src, wl.dst, wl.w, wl.dy), tau)
    check_close("dw", out["dw"], *oracle.edge_grad(wl.src, wl.dst, wl.x, wl.dy), tau)


def test_skewed_fused_and_async_bitwise(run):
    _, out = run
    assert out["fused_equal"] == [True, True]
    assert out["async_equal"] == [True] * 5
