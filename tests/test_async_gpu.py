"""Back-to-back batches: the build without a host synchronisation
(mp_graph_build_async), whose class counts stay on the device, against the
synchronous build and the oracle.

* every graph array of an asynchronous build equals the synchronous one bit for
  bit, and mp_graph_finish fills in the same class counts;
* every compute call on a graph whose counts are still on the device returns
  the same bits as on the finished graph (the kernels derive the same owner
  partition on the device; the larger launch only adds blocks that exit);
* an out-of-range endpoint is reported by mp_graph_finish;
* sampled minibatches pipelined over two streams (build of batch b + 1 on one
  stream while batch b computes on the other) match the oracle;
* the asynchronous path captured in a HIP graph replays correctly several
  times, with eager work and synchronisations between the replays."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.harness import TAU, check_close, check_floats, check_structure, upload

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def mp():
    import gnn_sparse_message_amd
    return gnn_sparse_message_amd


def _all_outputs(mp, g, t, heads_w):
    """Every compute call on g, in one list."""
    out = [mp.mp_spmm_fwd(g, t["w"], t["x"]), mp.mp_spmm_dx(g, t["w"], t["dy"]),
           mp.mp_edge_grad_dw(g, t["x"], t["dy"])]
    out += list(mp.mp_spmm_dx_edge_grad(g, t["w"], t["x"], t["dy"]))
    out += [mp.mp_spmm_fwd_heads(g, heads_w, t["x"]), mp.mp_spmm_dx_heads(g, heads_w, t["dy"])]
    out += list(mp.mp_spmm_dx_edge_grad_heads(g, heads_w, t["x"], t["dy"]))
    alpha, stats = mp.mp_edge_softmax(g, t["w"])
    out += [alpha, stats]
    out += list(mp.mp_edge_softmax_backward(g, alpha, out[2]))
    out += [mp.mp_edge_normalize(g, mp.MP_NORM_SYM, t["w"])]
    return out


def _workloads():
    yield synth.witness()
    yield synth.random_graph(1, 0, 8, 1)
    yield synth.random_graph(700, 9000, 16, 2)
    yield synth.chung_lu(seed=33, n=20000, e=400000, cap=20000.0, h=32, feat_dtype="f32")
    yield synth.chung_lu(seed=34, n=8000, e=160000, cap=8000.0, h=128, feat_dtype="bf16")
    yield synth.minibatches(1, h=64)[0]
    # about 3,000 rows of ~200 edges: four-wave hub owners in the main launch,
    # more of them than its hub blocks, which then stride
    yield synth.random_graph(3000, 600000, 16, 5)
    # RMAT-16: 16-wave hub owners in their own launch, more rows than its blocks
    yield synth.rmat16()


@pytest.mark.parametrize("idx", range(8))
def test_async_build_equals_sync(mp, idx):
    wl = list(_workloads())[idx]
    t = upload(wl, DEV)
    heads = 2 if wl.h % 2 == 0 else 1
    hw = torch.from_numpy(np.random.default_rng(idx).uniform(-1, 1, (wl.e, heads))
                          .astype(np.float32)).to(DEV)
    g_sync = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    g_async = mp.mp_graph_build_async(t["src"], t["dst"], wl.n)
    assert g_async.on_device and not g_sync.on_device
    assert g_async.class_count == [0] * 33
    ref = _all_outputs(mp, g_sync, t, hw)
    got = _all_outputs(mp, g_async, t, hw)     # counts read on the device
    torch.cuda.synchronize()
    for k, (a, b) in enumerate(zip(got, ref)):
        assert torch.equal(a, b), f"output {k} differs on the asynchronously built graph"
    for name in g_sync.arrays:
        assert torch.equal(g_async.arrays[name], g_sync.arrays[name]), name
    mp.mp_graph_finish(g_async)
    assert not g_async.on_device and g_async.built
    assert g_async.class_count == g_sync.class_count
    assert g_async.class_count_t == g_sync.class_count_t
    check_structure(g_async, wl)


def test_finish_reports_bad_index(mp):
    wl = synth.random_graph(100, 1000, 4, 3)
    t = upload(wl, DEV)
    bad = t["dst"].clone()
    bad[517] = 100                                   # == N: out of range
    g = mp.mp_graph_build_async(t["src"], bad, wl.n)
    y = mp.mp_spmm_fwd(g, t["w"], t["x"])            # still in bounds: the endpoint reads as 0
    with pytest.raises(IndexError):
        mp.mp_graph_finish(g)
    assert not g.built
    assert torch.isfinite(y).all()
    with pytest.raises(ValueError):                  # an unbuilt graph is refused
        mp.mp_spmm_fwd(g, t["w"], t["x"])


def test_two_stream_pipeline_minibatches(mp):
    """Build of batch b + 1 (stream B) overlaps the compute of batch b (stream A);
    every batch checked against the oracle."""
    batches = synth.minibatches(6, h=64)
    ups = [upload(wl, DEV) for wl in batches]
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    ws_bytes = max(mp.mp_graph_build_workspace_size(wl.n, wl.e) for wl in batches)
    wss = [torch.empty(ws_bytes, dtype=torch.uint8, device=DEV) for _ in range(2)]
    torch.cuda.synchronize()
    graphs, ready, outs = [None] * len(batches), [None] * len(batches), []

    def build(b):
        with torch.cuda.stream(sb):
            graphs[b] = mp.mp_graph_build_async(ups[b]["src"], ups[b]["dst"], batches[b].n,
                                                workspace=wss[b % 2])
            ready[b] = torch.cuda.Event()
            ready[b].record(sb)

    build(0)
    for b in range(len(batches)):
        if b + 1 < len(batches):
            build(b + 1)     # the workspaces alternate; builds are ordered on stream B
        with torch.cuda.stream(sa):
            sa.wait_event(ready[b])
            t, g = ups[b], graphs[b]
            y = mp.mp_spmm_fwd(g, t["w"], t["x"])
            dx, dw = mp.mp_spmm_dx_edge_grad(g, t["w"], t["x"], t["dy"])
            g.record_stream(sa)
            outs.append((y, dx, dw))
    torch.cuda.synchronize()
    for b, wl in enumerate(batches):
        mp.mp_graph_finish(graphs[b])
        check_structure(graphs[b], wl)
        check_floats(wl, *outs[b])


def test_captured_async_path_replays(mp):
    """build_async + forward + fused backward captured once, replayed three times
    with eager work and a synchronisation between replays; every replay equals
    the eager result."""
    wl = synth.chung_lu(seed=35, n=6000, e=90000, cap=6000.0, h=64, feat_dtype="f32")
    t = upload(wl, DEV)
    g0 = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    ref = [mp.mp_spmm_fwd(g0, t["w"], t["x"])]
    ref += list(mp.mp_spmm_dx_edge_grad(g0, t["w"], t["x"], t["dy"]))
    ws = torch.empty(mp.mp_graph_build_workspace_size(wl.n, wl.e), dtype=torch.uint8, device=DEV)
    y = torch.empty_like(ref[0])
    dx = torch.empty_like(ref[1])
    dw = torch.empty_like(ref[2])
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                    # warm the allocator outside the capture
        g = mp.mp_graph_build_async(t["src"], t["dst"], wl.n, workspace=ws)
        mp.mp_spmm_fwd(g, t["w"], t["x"], out=y)
        mp.mp_spmm_dx_edge_grad(g, t["w"], t["x"], t["dy"], out_dx=dx, out_dw=dw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    cg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(cg, capture_error_mode="relaxed"):
        g = mp.mp_graph_build_async(t["src"], t["dst"], wl.n, workspace=ws)
        mp.mp_spmm_fwd(g, t["w"], t["x"], out=y)
        mp.mp_spmm_dx_edge_grad(g, t["w"], t["x"], t["dy"], out_dx=dx, out_dw=dw)
    for rep in range(3):
        y.fill_(float("nan"))
        dx.fill_(float("nan"))
        dw.fill_(float("nan"))
        cg.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref[0]), f"replay {rep}: Y"
        assert torch.equal(dx, ref[1]), f"replay {rep}: dX"
        assert torch.equal(dw, ref[2]), f"replay {rep}: dw"
        torch.cuda.synchronize()
        _ = (t["x"] * 2).sum().item()              # eager work between replays
    check_close("Y", y, *oracle.forward(wl.n, wl.src, wl.dst, wl.w, wl.x), TAU["f32"])
