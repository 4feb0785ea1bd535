"""The largest edge count the interface allows, E = 2^31 - 1 (N = 2^20, H = 1),
checked through properties that hold at any size, computed independently with
torch on the device:

* lowering: rowptr is the exclusive prefix sum of the in-degrees (bincount),
  edge_order is a permutation of [0, E) (every ordinal counted once), col is
  src gathered through edge_order, and the keys dst[edge_order] are sorted
  with ordinals increasing inside each row (stability);
* aggregation with small-integer inputs, where fp32 sums are exact: with
  w, X, dY in {-2, ..., 2}, Y[i] = sum over the edges into i of w_e X[src_e]
  equals torch's weighted bincount, dX likewise by source, and
  dw_e = X[src_e] dY[dst_e] exactly.

Memory: about 150 GB of HBM at the peak (graph arrays, workspace, checks)."""
import pytest
import torch

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
DEV = torch.device("cuda:0")
E = 2**31 - 1
N = 2**20


@pytest.fixture(scope="module")
def mp():
    import gnn_sparse_message_amd
    return gnn_sparse_message_amd


def _small_ints(shape, gen):
    return (torch.randint(-2, 3, shape, generator=gen, device=DEV, dtype=torch.int32)
            .to(torch.float32))


def test_maximum_edge_count(mp):
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info(DEV)
    if free < 200 * 2**30:
        pytest.skip(f"needs about 200 GB of free device memory, {free / 2**30:.0f} GB free")
    gen = torch.Generator(device=DEV).manual_seed(2024)
    src = torch.randint(0, N, (E,), generator=gen, device=DEV, dtype=torch.int32)
    dst = torch.randint(0, N, (E,), generator=gen, device=DEV, dtype=torch.int32)
    g = mp.mp_graph_build(src, dst, N)
    torch.cuda.synchronize()

    # ---- lowering
    deg = torch.bincount(dst, minlength=N)
    rowptr = g.rowptr.to(torch.int64)
    assert rowptr[0].item() == 0 and rowptr[-1].item() == E
    assert torch.equal(rowptr[1:] - rowptr[:-1], deg)
    del deg, rowptr
    order = g.edge_order
    seen = torch.bincount(order, minlength=E)
    assert seen.numel() == E and bool((seen == 1).all())
    del seen
    assert torch.equal(torch.index_select(src, 0, order), g.col)
    keys = torch.index_select(dst, 0, order)
    step = keys[1:] - keys[:-1]
    assert bool((step >= 0).all())
    same_row = step == 0
    del step, keys
    assert bool(((order[1:] > order[:-1]) | ~same_row).all())
    del same_row
    deg_t = torch.bincount(src, minlength=N)
    assert torch.equal(g.rowptr_t[1:].to(torch.int64) - g.rowptr_t[:-1].to(torch.int64), deg_t)
    del deg_t
    torch.cuda.empty_cache()

    # ---- aggregation, exact in fp32
    w = _small_ints((E,), gen)
    x = _small_ints((N, 1), gen)
    dy = _small_ints((N, 1), gen)
    y = mp.mp_spmm_fwd(g, w, x)
    msg = w * torch.index_select(x[:, 0], 0, src)
    assert torch.equal(y[:, 0], torch.bincount(dst, weights=msg, minlength=N).to(torch.float32))
    del msg, y
    dx, dw = mp.mp_spmm_dx_edge_grad(g, w, x, dy)
    msg = w * torch.index_select(dy[:, 0], 0, dst)
    assert torch.equal(dx[:, 0], torch.bincount(src, weights=msg, minlength=N).to(torch.float32))
    del msg
    ref = torch.index_select(x[:, 0], 0, src) * torch.index_select(dy[:, 0], 0, dst)
    assert torch.equal(dw, ref)


def _classes(deg):
    """Degree class: 0 for no edges, else the number of binary digits."""
    c = torch.zeros_like(deg)
    nz = deg > 0
    c[nz] = torch.floor(torch.log2(deg[nz].to(torch.float64))).to(deg.dtype) + 1
    return c


def test_maximum_node_count(mp):
    """N = 2^31 - 1 nodes (E = 2^20): 31-bit keys, row pointers and degree plans
    over 2^31 rows, and the forward over as many rows (almost all empty)."""
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info(DEV)
    if free < 200 * 2**30:
        pytest.skip(f"needs about 200 GB of free device memory, {free / 2**30:.0f} GB free")
    n, e = 2**31 - 1, 2**20
    gen = torch.Generator(device=DEV).manual_seed(2025)
    src = torch.randint(0, n, (e,), generator=gen, device=DEV, dtype=torch.int64)
    dst = torch.randint(0, n, (e,), generator=gen, device=DEV, dtype=torch.int64)
    dst[:4096] = n - 1                                  # a hub row at the last node
    g = mp.mp_graph_build(src, dst, n)
    torch.cuda.synchronize()
    deg = torch.bincount(dst, minlength=n)
    rowptr = g.rowptr.to(torch.int64)
    assert rowptr[0].item() == 0 and rowptr[-1].item() == e
    assert torch.equal(rowptr[1:] - rowptr[:-1], deg)
    del rowptr
    order = g.edge_order.to(torch.int64)
    keys = dst[order]
    assert bool((keys[1:] >= keys[:-1]).all())
    assert bool(((order[1:] > order[:-1]) | (keys[1:] != keys[:-1])).all())
    assert torch.equal(g.col.to(torch.int64), src[order])
    del order, keys
    # degree plan: a permutation of the rows, classes non-increasing along it,
    # ascending row id inside a class, and the host class counts agree
    plan = g.row_plan.to(torch.int64)
    assert bool((torch.bincount(plan, minlength=n) == 1).all())
    cls = _classes(deg)[plan]
    assert bool((cls[1:] <= cls[:-1]).all())
    assert bool(((plan[1:] > plan[:-1]) | (cls[1:] != cls[:-1])).all())
    counts = torch.bincount(cls, minlength=33).cpu().tolist()
    assert counts == g.class_count
    del plan, cls, deg
    torch.cuda.empty_cache()
    # forward with small integers (exact): Y = weighted bincount by destination
    w = _small_ints((e,), gen)
    x = _small_ints((n, 1), gen)
    y = mp.mp_spmm_fwd(g, w, x)
    ref = torch.bincount(dst, weights=w * x[src, 0], minlength=n)
    assert torch.equal(y[:, 0], ref)
