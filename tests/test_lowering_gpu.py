"""Device lowering (mp_graph_build) against the oracle's stable counting sort:
rowptr, col, edge_order, rowptr_t, col_t, transpose_order, both degree plans
and their class counts must match bit for bit."""
import numpy as np
import pytest
import torch

import synth
from tests.harness import check_structure

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def mp():
    import gnn_sparse_message_amd
    return gnn_sparse_message_amd


def _build(mp, wl, idx_dtype=torch.int64):
    src = torch.from_numpy(wl.src).to(DEV).to(idx_dtype)
    dst = torch.from_numpy(wl.dst).to(DEV).to(idx_dtype)
    g = mp.mp_graph_build(src, dst, wl.n)
    torch.cuda.synchronize()
    return g


def test_witness_printed_edge_order(mp):
    wl = synth.witness()
    g = _build(mp, wl)
    # tinymesh "Weighted aggregation experiment", "Exact witness": edge_order = (2, 0, 1)
    assert g.edge_order.cpu().tolist() == [2, 0, 1]
    check_structure(g, wl)


@pytest.mark.parametrize("idx_dtype", [torch.int32, torch.int64])
def test_tiny_uniform(mp, idx_dtype):
    wl = synth.tiny_uniform()
    check_structure(_build(mp, wl, idx_dtype), wl)


@pytest.mark.parametrize("n,e,seed", [
    (1, 0, 1), (1, 5, 2), (2, 1, 3), (5, 0, 4), (3, 4095, 5), (3, 4096, 6), (3, 4097, 7),
    (257, 1000, 8), (256, 65537, 9), (70000, 9000, 10), (1 << 17, 300000, 11),
    (3_000_000, 200_000, 12),       # 22-bit keys: three digit passes, mostly empty rows
    # small lists sort with 1024-key tiles and both directions per launch:
    # tile edges, the last pass without a scan kernel (<= 64 tiles) and the first
    # with one, and both sides of the switch to one direction per launch
    (50, 1023, 20), (50, 1024, 21), (50, 1025, 22), (5000, 65536, 23), (5000, 65537, 24),
    (1 << 16, (1 << 22), 25), (1 << 16, (1 << 22) + 1, 26),
    (70000, 1024, 27),              # row tiles: 69 plan tiles, past the in-kernel tile sums
    # large lists: the intake counts the first pass's digits of both keys
    (100, 5_000_001, 28),           # 7-bit keys: the counted pass is the only one
    (1 << 16, 6_000_000, 29),       # 16-bit keys: two passes
    (3_000_000, 5_000_000, 30),     # 22-bit keys: three passes, mostly empty rows
    (2, (1 << 22) + 4096 * 3 + 1, 31),   # 1-bit keys, one key past a tile edge
])
def test_random_sizes(mp, n, e, seed):
    wl = synth.random_graph(n, e, 1, seed)
    check_structure(_build(mp, wl), wl)


@pytest.mark.parametrize("idx_dtype", [torch.int32, torch.int64])
def test_large_list_index_dtypes(mp, idx_dtype):
    wl = synth.random_graph(40000, 4_500_000, 1, 32)
    check_structure(_build(mp, wl, idx_dtype), wl)


def test_large_list_bad_index(mp):
    """An endpoint out of range in a list long enough for the counting intake
    is reported, and the build still leaves every array in bounds."""
    wl = synth.random_graph(1000, 5_000_000, 1, 33)
    src = torch.from_numpy(wl.src).to(DEV)
    dst = torch.from_numpy(wl.dst).to(DEV)
    dst[4_999_999] = 1000
    with pytest.raises(IndexError):
        mp.mp_graph_build(src, dst, 1000)
    src[123] = -5
    dst[4_999_999] = 7
    with pytest.raises(IndexError):
        mp.mp_graph_build(src.to(torch.int32), dst.to(torch.int32), 1000)


def test_all_edges_one_row(mp):
    """A single hub row holding every edge, plus empty rows on both sides."""
    rng = np.random.default_rng(13)
    n, e = 5000, 100000
    wl = synth.random_graph(n, e, 1, 13)
    wl.dst[:] = 1234
    wl.src[:] = rng.integers(0, n, e)
    check_structure(_build(mp, wl), wl)


def test_duplicates_and_self_loops(mp):
    wl = synth.random_graph(50, 20000, 1, 14)      # ~8 copies of every pair
    wl.src[::7] = wl.dst[::7]                       # many self-loops
    check_structure(_build(mp, wl), wl)


def test_sbm(mp):
    wl = synth.sbm()
    check_structure(_build(mp, wl), wl)


def test_rmat16(mp):
    wl = synth.rmat16()
    check_structure(_build(mp, wl, torch.int32), wl)


def test_minibatch(mp):
    for wl in synth.minibatches(2):
        check_structure(_build(mp, wl), wl)


def test_rebuild_is_deterministic(mp):
    wl = synth.rmat(12, 16, 15, 1)
    a = _build(mp, wl)
    b = _build(mp, wl)
    for k in a.arrays:
        assert torch.equal(a.arrays[k], b.arrays[k]), k


def test_index_out_of_range(mp):
    src = torch.tensor([0, 1, 5], device=DEV)
    dst = torch.tensor([1, 2, 0], device=DEV)
    with pytest.raises(IndexError):
        mp.mp_graph_build(src, dst, 5)
    with pytest.raises(IndexError):
        mp.mp_graph_build(torch.tensor([0, -1], device=DEV), torch.tensor([0, 0], device=DEV), 3)
    with pytest.raises(IndexError):   # does not fit int32 either
        mp.mp_graph_build(torch.tensor([0, 1 << 40], device=DEV),
                          torch.tensor([0, 0], device=DEV), 3)


def test_rejects_host_and_bad_dtype(mp):
    with pytest.raises(ValueError):
        mp.mp_graph_build(torch.tensor([0, 1]), torch.tensor([1, 0]), 2)       # host memory
    with pytest.raises(TypeError):
        mp.mp_graph_build(torch.tensor([0, 1], device=DEV, dtype=torch.int16),
                          torch.tensor([1, 0], device=DEV, dtype=torch.int16), 2)
    with pytest.raises(ValueError):
        mp.mp_graph_build(torch.tensor([0], device=DEV), torch.tensor([0], device=DEV), 0)
