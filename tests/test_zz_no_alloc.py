"""mp_graph_build_noalloc, the lowering on the library's static per-GPU
workspace (for callers that cannot allocate): through the C interface, two
builds in a row, the second of a smaller graph over the workspace the first
left behind, each bit for bit equal to mp_graph_build_async with a workspace of
its own (every graph array, the class counts after mp_graph_finish, and a
forward and fused backward computed from the device record before finishing);
no device memory taken by the call; sizes beyond the static workspace
rejected before anything is launched."""
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


def _same_graph(a, b):
    for k in a.arrays:
        assert torch.equal(a.arrays[k], b.arrays[k]), k
    assert a.class_count == b.class_count and a.class_count_t == b.class_count_t


def test_noalloc_two_builds_in_a_row(mp):
    # RMAT-16 (1.05M edges, skewed: 16-wave hub launch), then a smaller graph
    cases = (synth.rmat16(), synth.random_graph(3000, 40000, 16, 5))
    assert cases[1].e < cases[0].e
    for wl in cases:
        print(f"case {wl.name}: N={wl.n} E={wl.e} H={wl.h}", flush=True)
        assert mp.mp_graph_build_workspace_size(wl.n, wl.e) <= mp.STATIC_WORKSPACE_BYTES
        t = upload(wl, DEV)
        g = mp.mp_graph_build_noalloc(t["src"], t["dst"], wl.n)
        ref = mp.mp_graph_build_async(t["src"], t["dst"], wl.n)
        assert g.on_device
        # compute calls read the device record of both graphs
        y, yr = mp.mp_spmm_fwd(g, t["w"], t["x"]), mp.mp_spmm_fwd(ref, t["w"], t["x"])
        dx, dw = mp.mp_spmm_dx_edge_grad(g, t["w"], t["x"], t["dy"])
        dxr, dwr = mp.mp_spmm_dx_edge_grad(ref, t["w"], t["x"], t["dy"])
        mp.mp_graph_finish(g)
        mp.mp_graph_finish(ref)
        torch.cuda.synchronize()
        _same_graph(g, ref)
        assert torch.equal(y, yr) and torch.equal(dx, dxr) and torch.equal(dw, dwr)
        check_structure(g, wl)   # and the lowering against the oracle


def test_noalloc_takes_no_device_memory(mp):
    wl = synth.random_graph(5000, 60000, 8, 6)
    t = upload(wl, DEV)
    g0 = mp.mp_graph_build_noalloc(t["src"], t["dst"], wl.n)   # first use on this device
    mp.mp_graph_finish(g0)
    graphs = [mp.Graph(wl.n, wl.e, DEV) for _ in range(3)]        # outputs, allocated first
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for g in graphs:
        st = mp._lib.mp_graph_build_noalloc(mp._ptr(t["src"]), mp._ptr(t["dst"]), mp.MP_I64,
                                            wl.n, wl.e, mp.ctypes.byref(g._desc),
                                            mp._stream(t["src"]))
        assert st == mp.MP_OK, mp.mp_status_string(st)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0
    for g in graphs:
        mp.mp_graph_finish(g)
        _same_graph(g, g0)


def test_noalloc_rejects_graphs_beyond_the_static_workspace(mp):
    n, e = 1000, 3_000_000
    assert mp.mp_graph_build_workspace_size(n, e) > mp.STATIC_WORKSPACE_BYTES
    src = torch.zeros(e, dtype=torch.int64, device=DEV)
    with pytest.raises(ValueError, match="static workspace"):
        mp.mp_graph_build_noalloc(src, src, n)
    # a graph that fits still builds after the refusal
    wl = synth.random_graph(50, 400, 4, 7)
    t = upload(wl, DEV)
    g = mp.mp_graph_finish(mp.mp_graph_build_noalloc(t["src"], t["dst"], wl.n))
    check_structure(g, wl)


def test_noalloc_index_check_over_the_shared_workspace(mp):
    """The index check of a small list is one range word per intake tile in the
    workspace, reduced by the plan pass. On the static workspace, which keeps
    the last call's contents, a build with an endpoint out of range reports it,
    and the clean build after it reports nothing and equals a build on a
    workspace of its own."""
    wl = synth.random_graph(20_000, 300_000, 1, 8)
    t = upload(wl, DEV)
    bad = t["dst"].clone()
    bad[150_000] = wl.n
    with pytest.raises(IndexError):
        mp.mp_graph_finish(mp.mp_graph_build_noalloc(t["src"], bad, wl.n))
    g = mp.mp_graph_finish(mp.mp_graph_build_noalloc(t["src"], t["dst"], wl.n))
    ref = mp.mp_graph_finish(mp.mp_graph_build_async(t["src"], t["dst"], wl.n))
    _same_graph(g, ref)
    check_structure(g, wl)
