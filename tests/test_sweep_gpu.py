"""A seeded sweep over shapes the hand-picked cases may miss: for each seed a
random graph size (one node to 20,000, no edges to 120,000, skewed or uniform
endpoints), feature dtype and head count (any divisor of the width up to 8);
every feature width of the list (odd widths, one lane, widths around the
16-byte lanes and the column blocks) comes twice.  Every entry point the configuration allows runs
through the C ABI and is compared with the oracle under the same bounds as the
dedicated tests; the fused calls are also compared bit for bit with the
separate ones."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.harness import TAU, check_close, check_structure, upload

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
WIDTHS = [1, 2, 3, 4, 5, 6, 7, 8, 9, 12, 15, 16, 17, 24, 31, 32, 33, 48, 63, 64, 65, 96, 100,
          127, 128, 129, 192, 255, 256, 257, 300, 512, 513, 1024, 1030]
N_CASES = 2 * len(WIDTHS)                  # every width twice


@pytest.fixture(scope="module")
def mp():
    import gnn_sparse_message_amd
    return gnn_sparse_message_amd


def _case(seed):
    rng = np.random.default_rng(10_000 + seed)
    n = int(rng.choice([1, 3, int(rng.integers(4, 300)), int(rng.integers(300, 5000)),
                        int(rng.integers(5000, 20000))], p=[0.1, 0.1, 0.25, 0.3, 0.25]))
    e = int(rng.choice([0, 1, int(rng.integers(2, 2000)), int(rng.integers(2000, 40000)),
                        int(rng.integers(40000, 120000))], p=[0.05, 0.05, 0.3, 0.35, 0.25]))
    h = WIDTHS[seed % len(WIDTHS)]
    dt = "bf16" if rng.random() < 0.5 else "f32"
    wl = synth.random_graph(n, e, h, 20_000 + seed, feat_dtype=dt)
    if e > 0 and rng.random() < 0.5:          # skew: a few rows take most of the edges
        hot = rng.integers(0, n, 3)
        pick = rng.random(e) < 0.6
        wl.dst[pick] = rng.choice(hot, int(pick.sum()))
        if rng.random() < 0.5:
            wl.src[pick] = rng.choice(hot, int(pick.sum()))
    divs = [k for k in range(1, 9) if h % k == 0]
    k = int(rng.choice(divs))
    return wl, k


@pytest.mark.parametrize("seed", range(N_CASES))
def test_sweep(mp, seed):
    wl, k = _case(seed)
    print(f"case {seed}: N={wl.n} E={wl.e} H={wl.h} {wl.feat_dtype} heads={k}", flush=True)
    t = upload(wl, DEV)
    g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
    torch.cuda.synchronize()
    check_structure(g, wl)
    tau = TAU["f32"]                       # exact inputs, fp32 accumulation
    y = mp.mp_spmm_fwd(g, t["w"], t["x"])
    dx = mp.mp_spmm_dx(g, t["w"], t["dy"])
    dw = mp.mp_edge_grad_dw(g, t["x"], t["dy"])
    fdx, fdw = mp.mp_spmm_dx_edge_grad(g, t["w"], t["x"], t["dy"])
    torch.cuda.synchronize()
    assert torch.equal(fdx, dx) and torch.equal(fdw, dw), "fused backward differs"
    check_close("Y", y, *oracle.forward(wl.n, wl.src, wl.dst, wl.w, wl.x), tau)
    check_close("dX", dx, *oracle.input_grad(wl.n, wl.src, wl.dst, wl.w, wl.dy), tau)
    check_close("dw", dw, *oracle.edge_grad(wl.src, wl.dst, wl.x, wl.dy), tau)
    # multi-head weights
    wk = np.random.default_rng(seed).uniform(-1, 1, (wl.e, k)).astype(np.float32)
    twk = torch.from_numpy(wk).to(DEV)
    yk = mp.mp_spmm_fwd_heads(g, twk, t["x"])
    dxk, dwk = mp.mp_spmm_dx_edge_grad_heads(g, twk, t["x"], t["dy"])
    torch.cuda.synchronize()
    check_close("Y heads", yk, *oracle.forward_heads(wl.n, wl.src, wl.dst, wk, wl.x), tau)
    check_close("dX heads", dxk, *oracle.input_grad_heads(wl.n, wl.src, wl.dst, wk, wl.dy), tau)
    check_close("dw heads", dwk, *oracle.edge_grad_heads(wl.src, wl.dst, wl.x, wl.dy, k), tau)
    # degree normalisation at the fetch equals normalising first
    for mode in (mp.MP_NORM_MEAN, mp.MP_NORM_SYM):
        wn = mp.mp_edge_normalize(g, mode, t["w"])
        a = mp.mp_spmm_fwd_norm(g, mode, t["w"], t["x"])
        b_dx, b_dw = mp.mp_spmm_dx_edge_grad_norm(g, mode, t["w"], t["x"], t["dy"])
        ref_dx, ref_dwn = mp.mp_spmm_dx_edge_grad(g, wn, t["x"], t["dy"])
        torch.cuda.synchronize()
        assert torch.equal(a, mp.mp_spmm_fwd(g, wn, t["x"])), f"fetch-normalised forward {mode}"
        assert torch.equal(b_dx, ref_dx), f"fetch-normalised dX {mode}"
        assert torch.equal(b_dw, mp.mp_edge_normalize(g, mode, ref_dwn)), f"raw-weight dw {mode}"
    # attention backward against the two-call chain, bit for bit
    alpha, _ = mp.mp_edge_softmax_heads(g, twk)
    ya = mp.mp_spmm_fwd_heads(g, alpha, t["x"])
    adx, ads, art = mp.mp_attention_backward(g, alpha, t["x"], t["dy"], ya)
    cdx, cda = mp.mp_spmm_dx_edge_grad_heads(g, alpha, t["x"], t["dy"])
    torch.cuda.synchronize()
    assert torch.equal(adx, cdx), "attention dX"
    if wl.e:
        expect = alpha * (cda - art[t["dst"]])
        assert torch.equal(ads, expect), "attention score gradient"
