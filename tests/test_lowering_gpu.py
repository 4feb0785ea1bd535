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


# Lists above 4M edges (one direction per launch, 4096-key tiles, the counted
# first pass): keys of 9 to 26 bits (one to four passes), lists one key either
# side of a multiple of 16,384 keys, and skew onto a few rows.
@pytest.mark.parametrize("n,e,seed,hubs", [
    (300, (1 << 22) + 1, 40, 0),              # 9-bit keys: two passes
    (1 << 20, 16384 * 257 - 1, 41, 0),        # 20-bit keys: three passes, a tile one short
    (1 << 20, 16384 * 257, 42, 0),            # ... the last tile full
    (1 << 20, 16384 * 257 + 1, 43, 0),        # ... one key in the last tile
    (1 << 22, 4_500_000, 44, 0),              # 22-bit keys
    ((1 << 22) + 5, 4_500_000, 45, 0),        # 23-bit keys
    (50_000_000, 4_300_000, 46, 0),           # 26-bit keys: four passes, rows mostly empty
    (5000, 4_500_000, 47, 3),                 # three hub rows hold 3/4 of the edges
    (1 << 21, 4_200_000, 48, 1),              # one row holds 3/4 of the edges, 21-bit keys
    # count scans cut into segments (one per 2048 tiles): two and four segments
    (1 << 21, 20_000_003, 49, 0),             # 4,883 tiles, a ragged last tile
    (1 << 20, 4096 * 8192 + 5, 50, 1),        # 8,193 tiles, one row holding 3/4 of the edges
])
def test_large_list_key_widths(mp, n, e, seed, hubs):
    wl = synth.random_graph(n, e, 1, seed)
    if hubs:
        rng = np.random.default_rng(seed)
        pick = rng.random(e) < 0.75
        wl.dst[pick] = rng.integers(0, hubs, int(pick.sum())) * 7
        wl.src[rng.random(e) < 0.5] = n - 1
    print(f"case N={n} E={e} hubs={hubs}", flush=True)
    check_structure(_build(mp, wl), wl)


# Lists of at least two edges per row, whose last sort pass delimits the rows
# itself: keys already in order (a digit's runs sit in a few tiles, so the
# first run of a digit follows thousands of empty run records), four keys with
# long stretches of empty rows before, between and after them, every edge on
# the first or the last row, keys in part of the range only, and both sides of
# the two-edges-per-row rule.
@pytest.mark.parametrize("n,e,seed,shape", [
    (1 << 21, 20_000_003, 60, "sorted"),
    (1 << 20, 4_500_000, 61, "sorted"),
    (1 << 20, 4_500_000, 62, "few"),
    (1 << 20, 4_500_000, 63, "first"),
    (1 << 20, 4_500_000, 64, "last"),
    (2_500_000, 5_000_002, 65, "random"),    # exactly two edges per row pointer
    (2_500_000, 5_000_001, 66, "random"),    # one short: rows by binary search
    (200, 4_200_000, 67, "sorted"),          # 8-bit keys: the counted pass is the last
    # bipartite: destinations only in the upper half, sources in the lower, so
    # each direction's first or last half of run records is empty
    (1 << 21, 20_000_003, 68, "halves"),
    (1 << 20, 4_500_000, 69, "ends"),        # keys in the first and last eighth only
])
def test_large_list_rows_from_last_pass(mp, n, e, seed, shape):
    wl = synth.random_graph(n, e, 1, seed)
    rng = np.random.default_rng(seed)
    if shape == "sorted":
        wl.dst = np.sort(wl.dst)
        wl.src = np.sort(wl.src)
    elif shape == "few":
        wl.dst = np.array([3, 4097, 500_000, n - 7], dtype=wl.dst.dtype)[rng.integers(0, 4, e)]
    elif shape == "first":
        wl.dst[:] = 0
        wl.src[:] = n - 1
    elif shape == "last":
        wl.dst[:] = n - 1
        wl.src[:] = 0
    elif shape == "halves":
        wl.dst = n // 2 + wl.dst // 2
        wl.src = wl.src // 2
    elif shape == "ends":
        wl.dst = np.where(wl.dst % 2 == 0, wl.dst // 16, n - 1 - wl.dst // 16)
    print(f"case N={n} E={e} shape={shape}", flush=True)
    check_structure(_build(mp, wl), wl)


# 16-bit keys (two 8-bit passes, ballot counts in the intake) and 20-bit keys
# (7-bit passes: the intake reads its endpoints 16 bytes per lane); endpoint
# arrays one element past a 16-byte boundary take the intake's 4- or 8-byte
# loads.
@pytest.mark.parametrize("idx_dtype", [torch.int32, torch.int64])
@pytest.mark.parametrize("n,offset", [(40000, 0), (1 << 20, 0), (1 << 20, 1)])
def test_large_list_index_dtypes(mp, idx_dtype, n, offset):
    wl = synth.random_graph(n, 4_500_000 + 4 * 4096 + 3, 1, 32)
    src = torch.from_numpy(wl.src).to(DEV).to(idx_dtype)[offset:]
    dst = torch.from_numpy(wl.dst).to(DEV).to(idx_dtype)[offset:]
    assert (src.data_ptr() % 16 == 0) == (offset == 0)
    wl.src, wl.dst = wl.src[offset:], wl.dst[offset:]
    g = mp.mp_graph_build(src, dst, n)
    torch.cuda.synchronize()
    check_structure(g, wl)


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


@pytest.mark.parametrize("n,e,bad_at", [(70_000, 168_000, 0), (70_000, 168_000, 167_999),
                                         (156_000, 1_500_000, 700_000)])
def test_index_flag_from_tile_words_with_a_reused_workspace(mp, n, e, bad_at):
    """Small lists report an out-of-range endpoint through one range word per
    intake tile, reduced by the plan pass (no launch clears the flag first).
    On one workspace: a clean build, a build with one bad endpoint (first,
    last or a middle tile; synchronous and asynchronous), then a clean build
    again, which must report nothing and equal the first bit for bit."""
    wl = synth.random_graph(n, e, 1, 70 + bad_at % 7)
    src = torch.from_numpy(wl.src).to(DEV)
    dst = torch.from_numpy(wl.dst).to(DEV)
    ws = torch.empty(mp.mp_graph_build_workspace_size(n, e), dtype=torch.uint8, device=DEV)
    ref = mp.mp_graph_build(src, dst, n, workspace=ws)
    check_structure(ref, wl)
    bad = dst.clone()
    bad[bad_at] = n
    with pytest.raises(IndexError):
        mp.mp_graph_build(src, bad, n, workspace=ws)
    ga = mp.mp_graph_build_async(bad, src, n, workspace=ws)
    with pytest.raises(IndexError):
        mp.mp_graph_finish(ga)
    again = mp.mp_graph_build(src, dst, n, workspace=ws)
    ga = mp.mp_graph_build_async(src, dst, n, workspace=ws)
    mp.mp_graph_finish(ga)
    torch.cuda.synchronize()
    for k in ref.arrays:
        assert torch.equal(again.arrays[k], ref.arrays[k]), k
        assert torch.equal(ga.arrays[k], ref.arrays[k]), k
    assert again.class_count == ref.class_count and again.class_count_t == ref.class_count_t


def test_rejects_host_and_bad_dtype(mp):
    with pytest.raises(ValueError):
        mp.mp_graph_build(torch.tensor([0, 1]), torch.tensor([1, 0]), 2)       # host memory
    with pytest.raises(TypeError):
        mp.mp_graph_build(torch.tensor([0, 1], device=DEV, dtype=torch.int16),
                          torch.tensor([1, 0], device=DEV, dtype=torch.int16), 2)
    with pytest.raises(ValueError):
        mp.mp_graph_build(torch.tensor([0], device=DEV), torch.tensor([0], device=DEV), 0)


@pytest.mark.parametrize("n,e,seed,coo", [
    (3_000_000, 5_000_000, 40, False),   # three passes: the second reads the first's outputs
    (1 << 21, (1 << 22) + 4096 * 5 + 3, 41, False),   # a ragged last tile
    # 8-bit keys: the one pass reads the endpoint copies, which are unaligned
    # too, and delimits the rows itself
    (200, 4_200_000, 42, True),
])
def test_large_list_unaligned_graph_arrays(mp, n, e, seed, coo):
    """Graph arrays need only 4-byte alignment.  With the CSR position maps and
    columns (and, with `coo`, the int32 endpoint copies) 4 bytes past a 16-byte
    boundary the large passes that read them take the register path instead of
    copying 16-byte rows to LDS; the result is the aligned build's, bit for
    bit, and the oracle's."""
    wl = synth.random_graph(n, e, 1, seed)
    src = torch.from_numpy(wl.src).to(DEV)
    dst = torch.from_numpy(wl.dst).to(DEV)
    ref = mp.mp_graph_build(src, dst, n)
    g = mp.Graph(n, e, DEV)
    keep = []
    names = ("col", "edge_order", "col_t", "transpose_order") + (("src", "dst") if coo else ())
    for name in names:
        buf = torch.empty(e + 4, dtype=torch.int32, device=DEV)
        view = buf[1:e + 1]                      # 4 bytes past the allocation's start
        assert view.data_ptr() % 16 == 4
        keep.append(buf)
        g.arrays[name] = view
        setattr(g._desc, name, mp._ptr(view))
    ws = torch.empty(mp.mp_graph_build_workspace_size(n, e), dtype=torch.uint8, device=DEV)
    st = mp._lib.mp_graph_build(mp._ptr(src), mp._ptr(dst), mp.MP_I64, n, e,
                                mp.ctypes.byref(g._desc), mp._ptr(ws), ws.numel(), mp._stream(src))
    assert st == 0
    torch.cuda.synchronize()
    for name in mp.Graph._ARRAYS:
        assert torch.equal(g.arrays[name], ref.arrays[name]), name
    assert g.class_count == ref.class_count and g.class_count_t == ref.class_count_t
    check_structure(g, wl)
