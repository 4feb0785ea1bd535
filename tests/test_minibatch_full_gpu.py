"""All 64 sampled minibatches of the back-to-back workload (2-hop neighbour
sampling, fanout 15 then 10, 1,024 seeds per batch, H = 256 fp32), one after
another through the calls the benchmark's minibatch schedules run: the
synchronous and the asynchronous build, the forward, the fused backward and
the separate gradient calls.  For every batch the lowering is compared with
the oracle bit for bit and every element of Y, dX and dw with the fp64 oracle
at the fp32 bound; the oracle runs on host threads while the GPU takes the
next batch."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.harness import TAU, check_close, check_structure, oracle_threads, upload

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
DEV = torch.device("cuda:0")
N_BATCHES = 64


def _check_batch(wl, got):
    """Every float output of one batch against the oracle; returns the worst
    |err|/S of Y, dX, dw."""
    ry, sy = oracle.forward(wl.n, wl.src, wl.dst, wl.w, wl.x)
    rdx, sdx = oracle.input_grad(wl.n, wl.src, wl.dst, wl.w, wl.dy)
    rdw, sdw = oracle.edge_grad(wl.src, wl.dst, wl.x, wl.dy)
    return (check_close(f"{wl.name} Y", got["y"], ry, sy, TAU["f32"]),
            check_close(f"{wl.name} dX", got["dx"], rdx, sdx, TAU["f32"]),
            check_close(f"{wl.name} dw", got["dw"], rdw, sdw, TAU["f32"]))


def test_every_minibatch_against_the_oracle():
    import gnn_sparse_message_amd as mp
    base = synth.base_graph(5)
    pending = []
    worst = np.zeros(3)
    threads = oracle_threads()
    with ThreadPoolExecutor(threads) as pool:
        for b in range(N_BATCHES):
            while len(pending) >= 2 * threads:   # bound the host memory held by checks
                worst = np.maximum(worst, pending.pop(0)[1].result())
            wl = synth.minibatches(1, first=b, nbr=base)[0]
            print(f"batch {b}: N={wl.n} E={wl.e} H={wl.h}", flush=True)
            t = upload(wl, DEV)
            g = mp.mp_graph_build(t["src"], t["dst"], wl.n)
            ga = mp.mp_graph_build_async(t["src"], t["dst"], wl.n)
            y = mp.mp_spmm_fwd(g, t["w"], t["x"])
            dx = mp.mp_spmm_dx(g, t["w"], t["dy"])
            dw = mp.mp_edge_grad_dw(g, t["x"], t["dy"])
            ya = mp.mp_spmm_fwd(ga, t["w"], t["x"])
            fdx, fdw = mp.mp_spmm_dx_edge_grad(ga, t["w"], t["x"], t["dy"])
            torch.cuda.synchronize()
            # the asynchronously built graph and the fused backward give the bits
            # of the synchronous graph's separate calls
            assert torch.equal(ya, y), f"batch {b}: forward on the asynchronous build"
            assert torch.equal(fdx, dx) and torch.equal(fdw, dw), f"batch {b}: fused backward"
            mp.mp_graph_finish(ga)
            for k in g.arrays:
                assert torch.equal(ga.arrays[k], g.arrays[k]), f"batch {b}: async {k}"
            check_structure(g, wl)
            got = {"y": y.cpu().numpy(), "dx": dx.cpu().numpy(), "dw": dw.cpu().numpy()}
            pending.append((b, pool.submit(_check_batch, wl, got)))
            del t, g, ga, y, dx, dw, ya, fdx, fdw
        for b, fut in pending:
            worst = np.maximum(worst, fut.result())
    print(f"{N_BATCHES} batches: max |err|/S  Y {worst[0]:.3e}  dX {worst[1]:.3e}  "
          f"dw {worst[2]:.3e}")
