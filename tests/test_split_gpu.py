"""The aggregations with their longest rows split across workgroups
(mp_spmm_fwd_split, mp_spmm_dx_split, mp_spmm_dx_edge_grad_split): Y, dX and
dw against the oracle on skewed graphs (RMAT scale 16, graphs with one row of
tens of thousands of edges, rows in several degree classes, every lane layout:
16-byte lanes in fp32 and bf16, scalar lanes, column blocks, the unfused wide
backward), the fused call bitwise equal to the split input gradient and the
edge-gradient kernel, bitwise reproducible, bitwise the plain calls when no row
is long enough, whatever the workspace held before, and the rejections."""
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


@pytest.fixture(autouse=True)
def _owner_rule_after_each_test():
    yield
    import gnn_sparse_message_amd
    gnn_sparse_message_amd.mp_set_owner_overrides(-1, -1, -1)


def _hub_graph(seed, n=4000, e=200_000, h=64, feat="f32", hubs=(50_000, 9_000, 3_000, 1_500)):
    """Uniform edges plus rows of the given lengths in both directions."""
    wl = synth.random_graph(n, e, h, seed, feat_dtype=feat)
    rng = np.random.default_rng(seed)
    at = 0
    for k, ln in enumerate(hubs):
        wl.dst[at:at + ln] = 11 + k
        wl.src[rng.permutation(e)[:ln]] = 23 + k
        at += ln
    return wl


CASES = [
    ("rmat16", lambda: synth.rmat16()),
    ("hubs_f32_h64", lambda: _hub_graph(81)),
    ("hubs_bf16_h128", lambda: _hub_graph(82, h=128, feat="bf16")),
    ("hubs_f32_h7", lambda: _hub_graph(83, h=7)),                 # scalar lanes
    ("hubs_f32_h300", lambda: _hub_graph(84, h=300)),             # column blocks, unfused backward
    ("one_row_all_edges", lambda: _hub_graph(85, n=300, e=60_000, h=32, hubs=(60_000,))),
]


def _run(mp, wl, fill_nan=True):
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    need = mp.mp_spmm_split_workspace_size(g, wl.h)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=DEV)
    if fill_nan:
        ws.view(torch.float32)[: ws.numel() // 4] = float("nan")
    y = mp.mp_spmm_fwd_split(g, t["w"], t["x"], workspace=ws)
    dx = mp.mp_spmm_dx_split(g, t["w"], t["dy"], workspace=ws)
    fdx, fdw = mp.mp_spmm_dx_edge_grad_split(g, t["w"], t["x"], t["dy"], workspace=ws)
    dw = mp.mp_edge_grad_dw(g, t["x"], t["dy"])
    torch.cuda.synchronize()
    return g, t, need, y, dx, fdx, fdw, dw


@pytest.mark.parametrize("idx", range(len(CASES)), ids=[c[0] for c in CASES])
def test_split_against_oracle(mp, idx):
    name, make = CASES[idx]
    wl = make()
    print(f"case {name}: N={wl.n} E={wl.e} H={wl.h} {wl.feat_dtype}", flush=True)
    g, t, need, y, dx, fdx, fdw, dw = _run(mp, wl)
    assert need > 0, "these graphs have rows long enough to split"
    tau = TAU["f32"]                     # fp32 accumulation in either storage
    check_close("Y", y, *oracle.forward(wl.n, wl.src, wl.dst, wl.w, wl.x), tau)
    check_close("dX", dx, *oracle.input_grad(wl.n, wl.src, wl.dst, wl.w, wl.dy), tau)
    assert torch.equal(fdx, dx), "fused dX differs from the split input gradient"
    assert torch.equal(fdw, dw), "fused dw differs from the edge-gradient kernel"
    check_close("dw", fdw, *oracle.edge_grad(wl.src, wl.dst, wl.x, wl.dy), tau)


def test_split_is_reproducible(mp):
    wl = _hub_graph(86, h=128, feat="bf16")
    a = _run(mp, wl)
    b = _run(mp, wl, fill_nan=False)
    for i in (3, 4, 5, 6):
        assert torch.equal(a[i], b[i])


def test_split_with_owner_overrides(mp):
    """Hub rows forced longer or shorter than the split rows: the split rows
    stay split, every other row keeps one owner."""
    wl = _hub_graph(87)
    ry = oracle.forward(wl.n, wl.src, wl.dst, wl.w, wl.x)
    for hub in (1, 64, 1 << 20):
        with mp.owner_overrides(hub_min_len=hub, wave_min_len=2):
            g, t, need, y, dx, fdx, fdw, dw = _run(mp, wl)
        check_close(f"Y hub_min={hub}", y, *ry, TAU["f32"])
        assert torch.equal(fdx, dx) and torch.equal(fdw, dw)


def test_no_split_equals_plain_calls(mp):
    """No row long enough: no workspace, and the bits of the plain calls."""
    wl = synth.random_graph(3000, 50_000, 64, 88)
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    assert mp.mp_spmm_split_workspace_size(g, wl.h) == 0
    y = mp.mp_spmm_fwd_split(g, t["w"], t["x"])
    dx, dw = mp.mp_spmm_dx_edge_grad_split(g, t["w"], t["x"], t["dy"])
    torch.cuda.synchronize()
    assert torch.equal(y, mp.mp_spmm_fwd(g, t["w"], t["x"]))
    rdx, rdw = mp.mp_spmm_dx_edge_grad(g, t["w"], t["x"], t["dy"])
    assert torch.equal(dx, rdx) and torch.equal(dw, rdw)
    assert torch.equal(mp.mp_spmm_dx_split(g, t["w"], t["dy"]), mp.mp_spmm_dx(g, t["w"], t["dy"]))


def test_split_rejections(mp):
    wl = _hub_graph(89)
    t = upload(wl, DEV)
    ga = mp.mp_graph_build_async(t["src"], t["dst"], wl.n)
    with pytest.raises(ValueError):                          # counts still on the device
        mp.mp_spmm_split_workspace_size(ga, wl.h)
    mp.mp_graph_finish(ga)
    need = mp.mp_spmm_split_workspace_size(ga, wl.h)
    assert need > 0
    y = mp.mp_spmm_fwd_split(ga, t["w"], t["x"])             # finished: accepted
    small = torch.empty(need - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        mp.mp_spmm_fwd_split(ga, t["w"], t["x"], workspace=small)
    # the workspace over the output (through the C interface, past the binding)
    st = mp._lib.mp_spmm_fwd_split(mp.ctypes.byref(ga._desc), mp._ptr(t["w"]), mp._ptr(t["x"]),
                                   mp.MP_F32, wl.h, mp._ptr(y), mp._ptr(y), need,
                                   mp._stream(y))
    assert st == mp.MP_ERR_ALIAS
    ws = torch.empty(need + 4096, dtype=torch.uint8, device=DEV)
    st = mp._lib.mp_spmm_fwd_split(mp.ctypes.byref(ga._desc), mp._ptr(t["w"]), mp._ptr(t["x"]),
                                   mp.MP_F32, wl.h, mp._ptr(y), mp._ptr(ws) + 4, need,
                                   mp._stream(y))
    assert st == mp.MP_ERR_ALIGN
    torch.cuda.synchronize()
