"""mp_graph_build_overlap: the lowering with its transpose direction on a second
stream.  The forward aggregation runs on the main stream as soon as the call
returns (while the transpose CSR may still be in flight); the fused backward
and the input gradient run after the transpose-done event.  Every graph array
and every output equals the one-stream build's bit for bit, and the oracle's."""
import numpy as np
import pytest
import torch

import synth
from tests.harness import check_structure, upload

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def mp():
    import gnn_sparse_message_amd
    return gnn_sparse_message_amd


def _workloads():
    yield synth.witness()
    yield synth.random_graph(1, 0, 8, 1)                       # no edges
    yield synth.random_graph(700, 9000, 16, 2)                 # a small list
    yield synth.minibatches(1, h=64)[0]
    # large tiles here, both directions per launch in the one-stream build;
    # rows delimited by the last sort pass
    yield synth.random_graph(20_000, 400_000, 16, 4)
    # large lists (one direction per launch, payloads copied to LDS), a ragged
    # last tile, a skewed power law
    yield synth.random_graph(1 << 20, 4_300_001, 16, 3)
    yield synth.chung_lu(seed=35, n=300_000, e=6_000_000, cap=60_000.0, h=32, feat_dtype="bf16")


@pytest.mark.parametrize("idx", range(7))
def test_overlap_build_equals_one_stream(mp, idx):
    wl = list(_workloads())[idx]
    print(f"case N={wl.n} E={wl.e} H={wl.h}", flush=True)
    t = upload(wl, DEV)
    ref_g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    ref_y = mp.mp_spmm_fwd(ref_g, t["w"], t["x"])
    ref_dx, ref_dw = mp.mp_spmm_dx_edge_grad(ref_g, t["w"], t["x"], t["dy"])
    ref_dx1 = mp.mp_spmm_dx(ref_g, t["w"], t["dy"])
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    g, done = mp.mp_graph_build_overlap(t["src"], t["dst"], wl.n, side)
    assert g.on_device
    y = mp.mp_spmm_fwd(g, t["w"], t["x"])          # forward CSR only: no wait
    dw = mp.mp_edge_grad_dw(g, t["x"], t["dy"])    # COO copies only: no wait
    torch.cuda.current_stream().wait_event(done)
    dx, fdw = mp.mp_spmm_dx_edge_grad(g, t["w"], t["x"], t["dy"])
    dx1 = mp.mp_spmm_dx(g, t["w"], t["dy"])
    torch.cuda.synchronize()
    assert torch.equal(y, ref_y)
    assert torch.equal(dx, ref_dx) and torch.equal(fdw, ref_dw) and torch.equal(dw, ref_dw)
    assert torch.equal(dx1, ref_dx1)
    for name in ref_g.arrays:
        assert torch.equal(g.arrays[name], ref_g.arrays[name]), name
    mp.mp_graph_finish(g)
    assert g.built and not g.on_device
    assert g.class_count == ref_g.class_count and g.class_count_t == ref_g.class_count_t
    check_structure(g, wl)


def test_overlap_build_repeated_on_one_workspace(mp):
    """Back-to-back overlapped builds on one workspace, each step waiting for
    the previous one's transpose: every graph equals its one-stream build."""
    side = torch.cuda.Stream()
    batches = synth.minibatches(3, h=16)
    ws = torch.empty(max(mp.mp_graph_build_overlap_workspace_size(b.n, b.e) for b in batches),
                     dtype=torch.uint8, device=DEV)
    for wl in batches:
        t = upload(wl, DEV)
        g, done = mp.mp_graph_build_overlap(t["src"], t["dst"], wl.n, side, workspace=ws)
        torch.cuda.current_stream().wait_event(done)   # the next build reuses the workspace
        ref = mp.mp_graph_build(t["src"], t["dst"], wl.n)
        torch.cuda.synchronize()
        for name in ref.arrays:
            assert torch.equal(g.arrays[name], ref.arrays[name]), name


def test_overlap_rejections(mp):
    wl = synth.random_graph(100, 1000, 4, 4)
    t = upload(wl, DEV)
    cur = torch.cuda.current_stream()
    with pytest.raises(ValueError):                 # the side stream is the main one
        mp.mp_graph_build_overlap(t["src"], t["dst"], wl.n, cur)
    with pytest.raises(TypeError):
        mp.mp_graph_build_overlap(t["src"], t["dst"], wl.n, None)
    side = torch.cuda.Stream()
    small = torch.empty(mp.mp_graph_build_workspace_size(wl.n, wl.e), dtype=torch.uint8,
                        device=DEV)
    if mp.mp_graph_build_overlap_workspace_size(wl.n, wl.e) > small.numel():
        with pytest.raises(ValueError):             # the one-stream build's workspace
            mp.mp_graph_build_overlap(t["src"], t["dst"], wl.n, side, workspace=small)
    torch.cuda.synchronize()
