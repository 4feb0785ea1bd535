"""Benchmark: weighted sparse message passing on one MI355X.

One step = one pass of the whole path over one synthetic input: the device
lowering (mp_graph_build), the forward aggregation (mp_spmm_fwd), and both
gradients (mp_spmm_dx_edge_grad: the input gradient and the edge-weight
gradient in one pass over the transpose CSR, bitwise equal to mp_spmm_dx and
mp_edge_grad_dw, which are timed on their own after the steps).  Workload: the
power-law Chung-Lu graph, N = 2,000,000, E = 100,000,000, degree exponent 2.1,
per-direction expected degree capped at 100,000, H = 128 bf16 features with
fp32 accumulation and fp32 outputs; inputs are resident in HBM before timing.

Throughput is effective HBM bandwidth over algorithmic bytes (each edge
touches its operand rows once):
    B_fwd   = E (H s + 12) + 4 (N + 1) + 4 N H        s = bytes per feature
    B_dX    = B_fwd
    B_dw    = E (2 H s + 12)
    B_build = E (2 s_idx + 16) + 8 (N + 1)            s_idx = 8 (int64 input)
value = (B_build + B_fwd + B_dX + B_dw) / step time.  Per-op times come from
HIP events recorded on the stream the kernels run on.

Prints exactly one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0   # MI355X HBM3E peak, 8 TB/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# Sources that define each counted kernel: its recorded counter bytes stand only
# while these files are unchanged.
KERNEL_SOURCES = {
    "spmm_kernel": ["gnn_sparse_message_amd/csrc/spmm.hip", "gnn_sparse_message_amd/csrc/common.h"],
    "sddmm_kernel": ["gnn_sparse_message_amd/csrc/sddmm.hip",
                     "gnn_sparse_message_amd/csrc/common.h"],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(n, e, h, s_feat, s_idx):
    fwd = e * (h * s_feat + 12) + 4 * (n + 1) + 4 * n * h
    return {"build": e * (2 * s_idx + 16) + 8 * (n + 1), "fwd": fwd, "dx": fwd,
            "dw": e * (2 * h * s_feat + 12)}


def _code_only(text):
    """Source text without comments and with runs of white space made one
    blank, so that edits of comments alone leave a kernel's hash unchanged
    (none of the hashed sources has a string literal holding a comment
    marker)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return re.sub(r"\s+", " ", text).strip()


def kernel_source_hash(kernel):
    """Hash of the code (comments left out) of the source files that define
    `kernel` (a key of KERNEL_SOURCES)."""
    hsh = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            hsh.update(_code_only(f.read()).encode())
    return hsh.hexdigest()[:16]


def measured_traffic(kernel_key):
    """HBM bytes per launch ("kernel:use" key) from the committed counter
    summary, or None when that kernel's sources changed since the counters were
    taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    k = rec.get("kernels", {}).get(kernel_key)
    if k is None or k.get("source_hash") != kernel_source_hash(kernel_key.split(":")[0]):
        return None
    return k.get("hbm_bytes_per_launch")


def cpu_baseline(wl, sample_edges):
    """The oracle as it stands (single-threaded C, fp64) on the first
    `sample_edges` COO edges of the same workload, all N nodes, same H."""
    import oracle
    n, h = wl.n, wl.h
    src, dst, w = wl.src[:sample_edges], wl.dst[:sample_edges], wl.w[:sample_edges]
    oracle._load()
    t0 = time.perf_counter()
    oracle.lower(n, dst, src)
    oracle.lower(n, src, dst)
    oracle.forward(n, src, dst, w, wl.x)
    oracle.input_grad(n, src, dst, w, wl.dy)
    oracle.edge_grad(src, dst, wl.x, wl.dy)
    dt = time.perf_counter() - t0
    b = algorithmic_bytes(n, sample_edges, h, 2, 8)
    return {"value": round(sum(b.values()) / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "seconds": round(dt, 2),
            "edges_per_s": round(sample_edges / dt, 1),
            "sample": f"first {sample_edges} of the {wl.e} COO edges, all {n} nodes, H={h}; "
                      "lowering (both directions) + forward + input gradient + edge gradient, "
                      "single-threaded fp64 C oracle"}


def cpu_baseline_adjacent(wl, sample_edges, heads=4):
    """The oracle on the adjacent operations: target softmax and its backward and
    symmetric normalisation on the same sample as cpu_baseline, and the 4-head
    forward / input gradient / edge gradient on its first fifth (those loops cost
    about 10x more per edge).  Per op: seconds and the same algorithmic bytes per
    second as the GPU figures."""
    import numpy as np
    import oracle
    n, h = wl.n, wl.h
    e = sample_edges
    src, dst, w = wl.src[:e], wl.dst[:e], wl.w[:e]
    out = {}

    def timed(name, nbytes, fn):
        t0 = time.perf_counter()
        res = fn()
        dt = time.perf_counter() - t0
        out[name] = {"seconds": round(dt, 3), "GBps": round(nbytes / dt / 1e9, 3)}
        return res

    alpha, _, _ = timed("edge_softmax", 20 * e + 24 * n, lambda: oracle.edge_softmax(n, dst, w))
    timed("edge_softmax_backward", 28 * e + 16 * n,
          lambda: oracle.edge_softmax_backward(n, dst, alpha.astype(np.float32), w))
    timed("edge_normalize_sym", 16 * e + 8 * (n + 1),
          lambda: oracle.edge_normalize(n, src, dst, oracle.NORM_SYM, w))
    eh = max(e // 5, 1)
    wk = np.random.default_rng(7).uniform(-1, 1, (eh, heads)).astype(np.float32)
    b = algorithmic_bytes(n, eh, h, 2, 8)
    timed("fwd_heads", b["fwd"] + 4 * (heads - 1) * eh,
          lambda: oracle.forward_heads(n, src[:eh], dst[:eh], wk, wl.x))
    timed("bwd_heads", b["dx"] + b["dw"] + 8 * (heads - 1) * eh,
          lambda: (oracle.input_grad_heads(n, src[:eh], dst[:eh], wk, wl.dy),
                   oracle.edge_grad_heads(src[:eh], dst[:eh], wl.x, wl.dy, heads)))
    return {"kind": "oracle", "cores": 1, "unit": "GB/s", "ops": out,
            "sample": f"first {e} of the {wl.e} COO edges ({eh} for the {heads}-head ops), "
                      f"all {n} nodes, H={h}; single-threaded fp64 C oracle"}


def other_configs_bench(mp, torch, dev, reps=20):
    """The smaller configurations (tiny uniform, SBM, RMAT-16; fp32 features):
    every entry point timed on its own, median / p10 / p90 of `reps` calls after
    3 warm-ups, with the same algorithmic bytes as the main workload.  These
    graphs fit the caches, so the fractions are reported, not targeted."""
    import numpy as np
    import synth
    out = {}
    for wl in (synth.tiny_uniform(), synth.sbm(), synth.rmat16()):
        src = torch.from_numpy(wl.src).to(dev)
        dst = torch.from_numpy(wl.dst).to(dev)
        w = torch.from_numpy(wl.w).to(dev)
        x = torch.from_numpy(wl.x).to(dev)
        dy = torch.from_numpy(wl.dy).to(dev)
        n, e, h = wl.n, wl.e, wl.h
        y = torch.empty((n, h), device=dev)
        dx = torch.empty_like(y)
        dw = torch.empty(e, device=dev)
        g = mp.mp_graph_build(src, dst, n)
        stream = torch.cuda.current_stream(dev)
        calls = {"build": lambda: mp.mp_graph_build(src, dst, n),
                 "fwd": lambda: mp.mp_spmm_fwd(g, w, x, out=y),
                 "dx": lambda: mp.mp_spmm_dx(g, w, dy, out=dx),
                 "dw": lambda: mp.mp_edge_grad_dw(g, x, dy, out=dw),
                 "bwd": lambda: mp.mp_spmm_dx_edge_grad(g, w, x, dy, out_dx=dx, out_dw=dw)}
        b = algorithmic_bytes(n, e, h, 4, 8)
        b["bwd"] = b["dx"] + b["dw"]
        res = {"num_nodes": n, "num_edges": e, "feature_width": h, "feature_storage": "f32"}
        for name, fn in calls.items():
            for _ in range(3):
                fn()
            ts = []
            for _ in range(reps):
                a0 = torch.cuda.Event(enable_timing=True)
                a1 = torch.cuda.Event(enable_timing=True)
                a0.record(stream)
                fn()
                a1.record(stream)
                torch.cuda.synchronize()
                ts.append(a0.elapsed_time(a1))
            med = float(np.median(ts))
            res[name] = {"ms": round(med, 4), "p10_ms": round(float(np.percentile(ts, 10)), 4),
                         "p90_ms": round(float(np.percentile(ts, 90)), 4),
                         "GBps": round(b[name] / (med * 1e-3) / 1e9, 1),
                         "frac": round(b[name] / (med * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                         "edges_per_s": round(e / (med * 1e-3), 1),
                         "algorithmic_bytes": b[name]}
        out[wl.name] = res
        del g, src, dst, w, x, dy, y, dx, dw
    return out


def minibatch_bench(mp, torch, dev, n_batches=64, h=256):
    """Back-to-back sampled minibatches (2-hop, fanout 15 then 10, 1,024 seeds,
    topology changing every batch), each one step: build + forward + fused
    backward, H = 256 fp32.  Topology and weights come from the seeded sampler;
    X and dY are drawn on the device (torch normal, seed 500 + b).  Three
    schedules over the same staged batches:
      sync      -- mp_graph_build (one host synchronisation per batch), then the
                   compute, all on one stream;
      async     -- mp_graph_build_async, no host synchronisation, one stream;
      pipelined -- mp_graph_build_async of batch b + 1 on a second stream while
                   batch b computes (two workspaces, events between the streams).
    Returns the timings and the aggregate algorithmic rates."""
    import synth
    batches = synth.minibatches(n_batches, h=h, features=False)
    staged = []
    for b, wl in enumerate(batches):
        gen = torch.Generator(device=dev).manual_seed(500 + b)
        staged.append({"n": wl.n, "e": wl.e, "src": torch.from_numpy(wl.src).to(dev),
                       "dst": torch.from_numpy(wl.dst).to(dev),
                       "w": torch.from_numpy(wl.w).to(dev),
                       "x": torch.randn((wl.n, h), generator=gen, device=dev),
                       "dy": torch.randn((wl.n, h), generator=gen, device=dev)})
    n_max = max(t["n"] for t in staged)
    e_max = max(t["e"] for t in staged)
    y = torch.empty((n_max, h), device=dev)
    dx = torch.empty_like(y)
    dw = torch.empty(e_max, device=dev)
    ws_bytes = max(mp.mp_graph_build_workspace_size(t["n"], t["e"]) for t in staged)
    wss = [torch.empty(ws_bytes, dtype=torch.uint8, device=dev) for _ in range(2)]

    def compute(t, g):
        n, e = t["n"], t["e"]
        mp.mp_spmm_fwd(g, t["w"], t["x"], out=y[:n])
        mp.mp_spmm_dx_edge_grad(g, t["w"], t["x"], t["dy"], out_dx=dx[:n], out_dw=dw[:e])

    def run_sync():
        for t in staged:
            compute(t, mp.mp_graph_build(t["src"], t["dst"], t["n"], workspace=wss[0]))

    def run_async():
        for t in staged:
            compute(t, mp.mp_graph_build_async(t["src"], t["dst"], t["n"], workspace=wss[0]))

    sa, sb = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)

    def run_pipelined():
        sa.wait_stream(torch.cuda.current_stream(dev))
        sb.wait_stream(torch.cuda.current_stream(dev))
        graphs, ready = [None] * len(staged), [None] * len(staged)

        def build(b):
            with torch.cuda.stream(sb):
                t = staged[b]
                graphs[b] = mp.mp_graph_build_async(t["src"], t["dst"], t["n"],
                                                    workspace=wss[b % 2])
                ready[b] = torch.cuda.Event()
                ready[b].record(sb)
        build(0)
        for b in range(len(staged)):
            if b + 1 < len(staged):
                build(b + 1)
            with torch.cuda.stream(sa):
                sa.wait_event(ready[b])
                compute(staged[b], graphs[b])
                graphs[b].record_stream(sa)
                graphs[b] = None
        torch.cuda.current_stream(dev).wait_stream(sa)

    out = {}
    for name, fn in (("sync", run_sync), ("async", run_async), ("pipelined", run_pipelined)):
        fn()                                  # warm-up: allocator, code objects
        torch.cuda.synchronize()
        reps = []
        for _ in range(3):
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            reps.append(time.perf_counter() - t0)
        out[name] = statistics.median(reps) * 1e3
    b_total = 0
    for t in staged:
        bb = algorithmic_bytes(t["n"], t["e"], h, 4, 8)
        b_total += bb["build"] + bb["fwd"] + bb["dx"] + bb["dw"]
    e_total = sum(t["e"] for t in staged)
    res = {"batches": len(staged), "feature_width": h, "feature_dtype": "f32",
           "edges_total": e_total, "nodes_max": n_max, "edges_max": e_max,
           "algorithmic_bytes_total": b_total,
           "step": "per batch: build + mp_spmm_fwd + mp_spmm_dx_edge_grad"}
    for name, ms in out.items():
        res[name] = {"ms_total": round(ms, 3), "ms_per_batch": round(ms / len(staged), 4),
                     "GBps": round(b_total / (ms * 1e-3) / 1e9, 1),
                     "edges_per_s": round(e_total / (ms * 1e-3), 1)}
    del staged, y, dx, dw, wss
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-sample-edges", type=int, default=10_000_000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-minibatch", action="store_true",
                    help="skip the back-to-back minibatch schedules")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the timings of the small configurations")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the steps, run one plain 1 GiB -> 1 GiB elementwise copy "
                         "(reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py: this build runs on exactly one GPU (got --gpus {args.gpus}); "
              "multi-GPU sharding is described in the design notes, not implemented.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gnn_sparse_message_amd as mp
    import synth

    t0 = time.perf_counter()
    wl = synth.chung_lu()
    log(f"generated N={wl.n} E={wl.e} H={wl.h} ({wl.feat_dtype}) in {time.perf_counter() - t0:.1f}s")
    dev = torch.device("cuda:0")
    src = torch.from_numpy(wl.src).to(dev)
    dst = torch.from_numpy(wl.dst).to(dev)
    w = torch.from_numpy(wl.w).to(dev)
    x = torch.from_numpy(wl.x_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    dy = torch.from_numpy(wl.dy_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    n, e, h = wl.n, wl.e, wl.h
    y = torch.empty((n, h), dtype=torch.float32, device=dev)
    dx = torch.empty_like(y)
    dw = torch.empty(e, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    ops = ("build", "fwd", "bwd")
    times = {k: [] for k in ops}

    def step(record):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if record else None
        if record:
            ev[0].record(stream)
        g = mp.mp_graph_build(src, dst, n)
        if record:
            ev[1].record(stream)
        mp.mp_spmm_fwd(g, w, x, out=y)
        if record:
            ev[2].record(stream)
        mp.mp_spmm_dx_edge_grad(g, w, x, dy, out_dx=dx, out_dw=dw)
        if record:
            ev[3].record(stream)
        return ev, g

    for i in range(args.warmup):
        step(False)
        log(f"warmup step {i + 1}/{args.warmup}")
    torch.cuda.synchronize()
    events = []
    t_start = time.perf_counter()
    for i in range(args.steps):
        events.append(step(True)[0])
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    for ev in events:
        for k, name in enumerate(ops):
            times[name].append(ev[k].elapsed_time(ev[k + 1]))
    log(f"timed {args.steps} steps in {t_total:.3f}s")

    def time_op(fn, reps=5):
        fn()
        ts = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return statistics.median(ts)

    # The separate gradient entry points, outside the timed steps.
    g = mp.mp_graph_build(src, dst, n)
    dx_alone = torch.empty_like(dx)
    dw_alone = torch.empty_like(dw)
    standalone = {}
    standalone["dx"] = time_op(lambda: mp.mp_spmm_dx(g, w, dy, out=dx_alone))
    standalone["dw"] = time_op(lambda: mp.mp_edge_grad_dw(g, x, dy, out=dw_alone))
    same = bool(torch.equal(dx_alone, dx) and torch.equal(dw_alone, dw))
    # Sparse attention pieces on the same topology (scores = the edge weights).
    alpha = torch.empty_like(w)
    rstats = torch.empty((n, 2), dtype=torch.float32, device=dev)
    dscores = torch.empty_like(w)
    rdot = torch.empty(n, dtype=torch.float32, device=dev)
    wn = torch.empty_like(w)
    standalone["edge_softmax"] = time_op(lambda: mp.mp_edge_softmax(g, w, alpha, rstats))
    standalone["edge_softmax_backward"] = time_op(
        lambda: mp.mp_edge_softmax_backward(g, alpha, dw, dscores, rdot))
    standalone["edge_normalize_sym"] = time_op(
        lambda: mp.mp_edge_normalize(g, mp.MP_NORM_SYM, w, out=wn))
    # The attention forward with alpha formed at the fetch, against the softmax
    # then the aggregation on its alpha (bitwise the same Y).
    y_s = torch.empty_like(y)
    standalone["attention_forward"] = time_op(
        lambda: mp.mp_spmm_fwd_softmax(g, w, x, out=y_s, out_row_stats=rstats))
    attn_fwd_two_calls = time_op(lambda: (mp.mp_edge_softmax(g, w, alpha, rstats),
                                          mp.mp_spmm_fwd(g, alpha, x, out=y)))
    torch.cuda.synchronize()
    attn_fwd_equal = bool(torch.equal(y_s, y))
    # Degree normalisation applied at the weight fetch (GCN's symmetric and
    # SAGE's mean), against normalising the weights first (edge_normalize_sym).
    standalone["fwd_norm_sym"] = time_op(
        lambda: mp.mp_spmm_fwd_norm(g, mp.MP_NORM_SYM, w, x, out=y))
    standalone["fwd_norm_mean"] = time_op(
        lambda: mp.mp_spmm_fwd_norm(g, mp.MP_NORM_MEAN, w, x, out=y))
    dx_n = torch.empty_like(dx)
    dw_n = torch.empty_like(dw)
    standalone["bwd_norm_sym"] = time_op(
        lambda: mp.mp_spmm_dx_edge_grad_norm(g, mp.MP_NORM_SYM, w, x, dy, out_dx=dx_n,
                                             out_dw=dw_n))
    del dx_n, dw_n
    # The fused backward with weights and gradients interleaved ([E, 2]).
    wg = torch.empty((e, 2), dtype=torch.float32, device=dev)
    wg[:, 0] = w
    dx_p = torch.empty_like(dx)
    standalone["bwd_pair"] = time_op(
        lambda: mp.mp_spmm_dx_edge_grad_pair(g, wg, x, dy, out_dx=dx_p))
    same_pair = bool(torch.equal(dx_p, dx) and torch.equal(wg[:, 1], dw))
    del wg, dx_p
    # The whole attention backward in one call (alpha = the edge weights, Y = the
    # forward output of the steps): replaces the fused backward + softmax backward.
    dx_att = torch.empty_like(dx)
    standalone["attention_backward"] = time_op(
        lambda: mp.mp_attention_backward(g, w, x, dy, y, out_dx=dx_att, out_dscores=dscores,
                                         out_row_dot=rdot))
    # ... with the score gradients written over the weights (a copy of them;
    # the work does not depend on the values, so repeated calls time the same)
    a_buf = w.clone()
    standalone["attention_backward_in_place"] = time_op(
        lambda: mp.mp_attention_backward(g, a_buf, x, dy, y, out_dx=dx_att, out_dscores=a_buf,
                                         out_row_dot=rdot))
    # ... with alpha formed in the walk from the scores (the edge weights) and
    # their softmax statistics (rstats, from the attention forward above)
    standalone["attention_backward_scores"] = time_op(
        lambda: mp.mp_attention_backward_scores(g, w, rstats, x, dy, y, out_dx=dx_att,
                                                out_dscores=dscores, out_row_dot=rdot))
    a_buf.copy_(w)
    standalone["attention_backward_scores_in_place"] = time_op(
        lambda: mp.mp_attention_backward_scores(g, a_buf, rstats, x, dy, y, out_dx=dx_att,
                                                out_dscores=a_buf, out_row_dot=rdot))
    del dx_att, a_buf
    log(f"standalone dx {standalone['dx']:.3f} ms, dw {standalone['dw']:.3f} ms, "
        f"equal to the fused results: {same}")
    del alpha, rstats, dscores, rdot, wn
    # Multi-head weights on the same graph: K heads of H/K columns, w [E, K].
    heads = 4
    wk = torch.empty((e, heads), device=dev).uniform_(
        -1.0, 1.0, generator=torch.Generator(device=dev).manual_seed(7))
    dwk = torch.empty((e, heads), dtype=torch.float32, device=dev)
    dxk = torch.empty_like(dx)
    standalone["fwd_heads"] = time_op(lambda: mp.mp_spmm_fwd_heads(g, wk, x, out=y))
    standalone["bwd_heads"] = time_op(
        lambda: mp.mp_spmm_dx_edge_grad_heads(g, wk, x, dy, out_dx=dxk, out_dw=dwk))
    same_heads = bool(torch.equal(mp.mp_spmm_dx_heads(g, wk, dy), dxk)
                      and torch.equal(mp.mp_edge_grad_dw_heads(g, x, dy, heads), dwk))
    # per-head softmax of [E, K] scores (the multi-head weights as scores)
    ak = torch.empty_like(wk)
    sk = torch.empty((n, heads, 2), dtype=torch.float32, device=dev)
    standalone["edge_softmax_heads"] = time_op(lambda: mp.mp_edge_softmax_heads(g, wk, ak, sk))
    dsk = torch.empty_like(wk)
    rdk = torch.empty((n, heads), dtype=torch.float32, device=dev)
    standalone["edge_softmax_backward_heads"] = time_op(
        lambda: mp.mp_edge_softmax_backward_heads(g, ak, dwk, dsk, rdk))
    mp.mp_spmm_fwd_heads(g, wk, x, out=y)
    standalone["attention_backward_heads"] = time_op(
        lambda: mp.mp_attention_backward(g, wk, x, dy, y, out_dx=dxk, out_dscores=dsk,
                                         out_row_dot=rdk))
    del ak, sk, dsk, rdk
    log(f"heads={heads}: fwd {standalone['fwd_heads']:.3f} ms, fused bwd "
        f"{standalone['bwd_heads']:.3f} ms, equal to the separate calls: {same_heads}")
    del wk, dwk, dxk

    if args.copy_calibration:
        a = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        log("copy calibration: 1 GiB read, 1 GiB written")

    bytes_ = algorithmic_bytes(n, e, h, 2, 8)
    bytes_["bwd"] = bytes_["dx"] + bytes_["dw"]
    # target softmax: row pass reads order + score per edge and writes 2 stats per
    # row; the edge pass reads dst + score, writes alpha.  Backward: row pass reads
    # order + alpha + dalpha, the edge pass dst + alpha + dalpha and writes ds.
    # (Definition bytes of the operation, not of this implementation's passes.)
    bytes_["edge_softmax"] = 20 * e + 24 * n
    bytes_["edge_softmax_backward"] = 28 * e + 16 * n
    # symmetric normalisation: in, out, src, dst per edge; both row pointers once.
    bytes_["edge_normalize_sym"] = 16 * e + 8 * (n + 1)
    # attention forward: the aggregation's bytes (the score in the weight's
    # place) plus the softmax's row pass (order + score per edge, two stats per
    # row written, then read once per row)
    bytes_["attention_forward"] = bytes_["fwd"] + 8 * e + 16 * n
    # multi-head: the edge's weight (or dw) term grows from 4 to 4K bytes.
    bytes_["fwd_heads"] = bytes_["fwd"] + 4 * (heads - 1) * e
    bytes_["bwd_heads"] = bytes_["dx"] + bytes_["dw"] + 8 * (heads - 1) * e
    # per-head softmax: the single-head bytes with K values per edge and per row
    bytes_["edge_softmax_heads"] = 4 * e + 16 * e * heads + 24 * n * heads
    bytes_["edge_softmax_backward_heads"] = 8 * e + 20 * e * heads + 16 * n * heads
    # attention backward: the fused backward's bytes (alpha for w, ds for dw) plus
    # the kept forward output Y and dY read once more for the row dots, and the
    # row dots written; with K heads, K values per edge and per row.
    bytes_["attention_backward"] = bytes_["bwd"] + (4 + 2) * n * h + 4 * n
    # normalised at the fetch: the plain call's bytes plus the other CSR's row
    # pointers, where the degrees come from
    bytes_["bwd_pair"] = bytes_["bwd"]
    bytes_["fwd_norm_sym"] = bytes_["fwd"] + 4 * (n + 1)
    bytes_["fwd_norm_mean"] = bytes_["fwd"]
    bytes_["bwd_norm_sym"] = bytes_["bwd"] + 4 * (n + 1)
    bytes_["attention_backward_in_place"] = bytes_["attention_backward"]
    # scores in alpha's place, plus each row's two statistics read once
    bytes_["attention_backward_scores"] = bytes_["attention_backward"] + 8 * n
    bytes_["attention_backward_scores_in_place"] = bytes_["attention_backward_scores"]
    bytes_["attention_backward_heads"] = (bytes_["attention_backward"] + 8 * (heads - 1) * e
                                          + 4 * (heads - 1) * n)
    ms_step = t_total / args.steps * 1e3

    def rate(nbytes, ms):
        gbps = nbytes / (ms * 1e-3) / 1e9
        return {"ms": round(ms, 4), "GBps": round(gbps, 1), "frac": round(gbps / PEAK_HBM_GBPS, 4),
                "edges_per_s": round(e / (ms * 1e-3), 1), "algorithmic_bytes": nbytes}

    def pct(v, q):
        v = sorted(v)
        return v[min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))]

    per_op = {k: rate(bytes_[k], statistics.median(times[k])) for k in ops}
    for k in ops:
        per_op[k]["p10_ms"] = round(pct(times[k], 0.1), 4)
        per_op[k]["p90_ms"] = round(pct(times[k], 0.9), 4)
    per_op_standalone = {k: rate(bytes_[k], v) for k, v in standalone.items()}
    per_op_standalone["equal_to_fused"] = same
    per_op_standalone["heads"] = heads
    per_op_standalone["heads_fused_equal_to_separate"] = same_heads
    per_op_standalone["pair_equal_to_fused"] = same_pair
    # what the fetch-time softmax replaces: the softmax (writing alpha), then the
    # aggregation on alpha; the two give the same Y bit for bit
    per_op_standalone["attention_forward_two_calls_ms"] = round(attn_fwd_two_calls, 4)
    per_op_standalone["attention_forward_equal_to_two_calls"] = attn_fwd_equal
    # what the fetch-time normalisation replaces: a normalisation pass, then the call
    per_op_standalone["fwd_norm_two_calls_ms"] = round(
        standalone["edge_normalize_sym"] + statistics.median(times["fwd"]), 4)
    per_op_standalone["bwd_norm_two_calls_ms"] = round(
        standalone["edge_normalize_sym"] * 2 + statistics.median(times["bwd"]), 4)
    # what the one-call attention backward replaces: fused backward + softmax backward
    per_op_standalone["attention_backward_unfused_ms"] = round(
        statistics.median(times["bwd"]) + standalone["edge_softmax_backward"], 4)
    per_op_standalone["attention_backward_heads_unfused_ms"] = round(
        standalone["bwd_heads"] + standalone["edge_softmax_backward_heads"], 4)
    # Kernels of the compute ops.  The dominant kernel is the one with the most
    # GPU time per step; its achieved bandwidth is the algorithmic bytes of the
    # units one launch processes over its average launch duration (the fused
    # backward processes both the dX and the dw units).  `traffic` is the
    # calibrated HBM counter bytes of one launch.
    kernels = {"spmm_kernel_fused_backward": ("bwd", "spmm_kernel:bwd"),
               "spmm_kernel": ("fwd", "spmm_kernel:fwd")}
    roof = {}
    for kname, (op, tkey) in kernels.items():
        launch_ms = per_op[op]["ms"]
        achieved = bytes_[op] / (launch_ms * 1e-3) / 1e9
        traffic = measured_traffic(tkey)
        roof[kname] = {"bound": "hbm", "kernel": f"{kname} ({op})",
                       "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                       "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic,
                       "traffic_GBps": None if traffic is None
                       else round(traffic / (launch_ms * 1e-3) / 1e9, 1),
                       "algorithmic_bytes_per_launch": bytes_[op], "avg_launch_ms": launch_ms}
    dominant = max(roof, key=lambda k: roof[k]["avg_launch_ms"])
    total_bytes = bytes_["build"] + bytes_["fwd"] + bytes_["dx"] + bytes_["dw"]
    value = total_bytes / (ms_step * 1e-3) / 1e9
    out = {
        "metric": "SpMM fwd/dX + SDDMM dw effective HBM GB/s and edges/s; % of HBM roofline",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "chung_lu_powerlaw", "num_nodes": n, "num_edges": e,
                   "feature_width": h, "degree_exponent": 2.1, "degree_cap": 100000,
                   "feature_storage": "bf16", "index_input": "int64",
                   "step": "mp_graph_build + mp_spmm_fwd + mp_spmm_dx_edge_grad"},
        "edges_per_s": round(e / (ms_step * 1e-3), 1),
        "frac_of_hbm_peak": round(value / PEAK_HBM_GBPS, 4),
        "per_op": per_op,
        "per_op_standalone": per_op_standalone,
        "roofline": roof[dominant],
        "roofline_other_kernels": {k: v for k, v in roof.items() if k != dominant},
    }
    if not args.no_other_configs:
        log("smaller configurations (tiny, SBM, RMAT-16) ...")
        out["other_configs"] = other_configs_bench(mp, torch, dev)
        log("smaller configurations: " + ", ".join(
            f"{k} fwd {v['fwd']['ms']} ms" for k, v in out["other_configs"].items()))
    if not args.no_minibatch:
        del g, dx_alone, dw_alone
        torch.cuda.empty_cache()
        log("minibatch schedules (64 sampled batches) ...")
        out["minibatch"] = minibatch_bench(mp, torch, dev)
        log("minibatch ms per batch: " + ", ".join(
            f"{k} {out['minibatch'][k]['ms_per_batch']}" for k in ("sync", "async", "pipelined")))
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on {args.cpu_sample_edges} edges ...")
        out["cpu_baseline"] = cpu_baseline(wl, min(args.cpu_sample_edges, e))
        log("cpu baseline of the adjacent operations ...")
        out["cpu_baseline_adjacent"] = cpu_baseline_adjacent(wl, min(args.cpu_sample_edges, e))
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
