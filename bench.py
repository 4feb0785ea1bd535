"""Benchmark: weighted sparse message passing on one MI355X.

One step = one pass of the whole path over one synthetic input: the device
lowering (mp_graph_build), the forward aggregation, and both gradients in one
pass over the transpose CSR (the input gradient and the edge-weight gradient,
bitwise equal to mp_spmm_dx and mp_edge_grad_dw, which are timed on their own
after the steps).  The timed step keeps the edge weights and their gradients
interleaved in one [E][2] array, both in COO order (mp_spmm_fwd_pair, then
mp_spmm_dx_edge_grad_pair); the same step on two separate arrays (mp_spmm_fwd,
mp_spmm_dx_edge_grad) is timed after it.  Workload: the power-law Chung-Lu
graph, N = 2,000,000, E = 100,000,000, degree exponent 2.1, per-direction
expected degree capped at 100,000, H = 128 bf16 features with fp32
accumulation and fp32 outputs; inputs are resident in HBM before timing.

Throughput is effective HBM bandwidth over algorithmic bytes (each edge
touches its operand rows once):
    B_fwd   = E (H s + 12) + 4 (N + 1) + 4 N H        s = bytes per feature
    B_dX    = B_fwd
    B_dw    = E (2 H s + 12)
    B_build = E (2 s_idx + 16) + 8 (N + 1)            s_idx = 8 (int64 input)
    B_bwd   = E (H s + 16) + 4 (N + 1) + N H s + 4 N H
B_bwd prices the fused backward launch at what it processes: per edge one
gathered dY row, col_t, transpose_order, w and dw; per row the owner's X row,
the dX row and a row pointer.  value = (B_build + B_fwd + B_bwd) / step time.
B_dX and B_dw price the separate calls.  Per-op times come from HIP events
recorded on the stream the kernels run on.

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
# Sources that define the kernels of each profiled op: its recorded counter
# bytes stand only while these files' code is unchanged.
_SPMM = ["gnn_sparse_message_amd/csrc/spmm.hip", "gnn_sparse_message_amd/csrc/common.h"]
_SOFTMAX = ["gnn_sparse_message_amd/csrc/softmax.hip"] + _SPMM
OP_SOURCES = {
    "build": ["gnn_sparse_message_amd/csrc/lower.hip", "gnn_sparse_message_amd/csrc/common.h"],
    "fwd_pair": _SPMM, "bwd_pair": _SPMM, "fwd": _SPMM, "bwd": _SPMM, "dx": _SPMM,
    "dw": ["gnn_sparse_message_amd/csrc/sddmm.hip", "gnn_sparse_message_amd/csrc/common.h"],
    "edge_softmax": _SOFTMAX, "edge_softmax_backward": _SOFTMAX,
    "edge_normalize_sym": ["gnn_sparse_message_amd/csrc/normalize.hip",
                           "gnn_sparse_message_amd/csrc/common.h"],
    "attention_forward": _SOFTMAX, "fwd_norm_sym": _SPMM, "bwd_norm_sym": _SPMM,
    "fwd_heads": _SPMM, "bwd_heads": _SPMM,
    "attention_backward": ["gnn_sparse_message_amd/csrc/attention.hip"] + _SPMM,
    "attention_backward_in_place": ["gnn_sparse_message_amd/csrc/attention.hip"] + _SPMM,
    "copy_calibration": [],
}
# The ops of the counter runs (bench.py --profile-ops), in launch order; each is
# preceded by one marker kernel (a fill of a small int8 tensor, a kernel nothing
# else here launches), so every dispatch between two markers belongs to one op.
PROFILE_OPS = tuple(OP_SOURCES)
MARKER_KERNEL = "FillFunctor<signed char>"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(n, e, h, s_feat, s_idx):
    """Gather-model bytes of each call: the build, the forward, the separate
    input-gradient and edge-gradient calls, and the fused backward launch (one
    dY row, col_t, transpose_order, w and dw per edge; the owner's X row, its
    dX row and a row pointer per row)."""
    fwd = e * (h * s_feat + 12) + 4 * (n + 1) + 4 * n * h
    return {"build": e * (2 * s_idx + 16) + 8 * (n + 1), "fwd": fwd, "dx": fwd,
            "dw": e * (2 * h * s_feat + 12),
            "bwd": e * (h * s_feat + 16) + 4 * (n + 1) + n * h * s_feat + 4 * n * h}


def _code_only(text):
    """Source text without comments and with runs of white space made one
    blank, so that edits of comments alone leave a kernel's hash unchanged
    (none of the hashed sources has a string literal holding a comment
    marker)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return re.sub(r"\s+", " ", text).strip()


def op_source_hash(op):
    """Hash of the code (comments left out) of the source files that define the
    kernels of `op` (a key of OP_SOURCES)."""
    hsh = hashlib.sha256()
    for rel in OP_SOURCES[op]:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            hsh.update(_code_only(f.read()).encode())
    return hsh.hexdigest()[:16]


def measured_traffic(op):
    """Calibrated HBM bytes of one call of `op` from the committed counter
    summary, or None when the sources of its kernels changed since the counters
    were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    k = rec.get("ops", {}).get(op)
    if k is None or k.get("source_hash") != op_source_hash(op):
        return None
    return k.get("hbm_bytes_per_call")


def cpu_baseline_all_cores(wl):
    """The oracle's definitions on every host core (oracle/baseline_omp.c: an
    OpenMP loop over the rows of the oracle's own CSR for the aggregations,
    over the edges for the edge gradient; the counting sort stays serial), over
    the whole workload: lowering of both directions, forward, input gradient,
    edge gradient, fp64."""
    import platform
    from oracle import baseline
    n, e, h = wl.n, wl.e, wl.h
    nthreads = baseline.threads()
    secs = baseline.run_path(n, wl.src, wl.dst, wl.w, wl.x, wl.dy)
    dt = sum(secs.values())
    b = algorithmic_bytes(n, e, h, 2, 8)
    total = b["build"] + b["fwd"] + b["dx"] + b["dw"]
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(total / dt / 1e9, 3), "unit": "GB/s", "cores": nthreads,
            "kind": "oracle_openmp", "seconds": round(dt, 2),
            "seconds_per_stage": {k: round(v, 2) for k, v in secs.items()},
            "edges_per_s": round(e / dt, 1), "nproc": os.cpu_count(), "cpu_model": model,
            "sample": f"all {e} COO edges, all {n} nodes, H={h}; lowering (both directions, "
                      "serial counting sort) + forward + input gradient (OpenMP over CSR rows) + "
                      "edge gradient (OpenMP over edges), fp64 C"}


def cpu_baseline(wl, sample_edges):
    """The oracle as it stands (single-threaded C, fp64) on the first
    `sample_edges` COO edges of the same workload, all N nodes, same H; one
    progress line per stage."""
    import oracle
    n, h = wl.n, wl.h
    src, dst, w = wl.src[:sample_edges], wl.dst[:sample_edges], wl.w[:sample_edges]
    oracle._load()
    stages = (("lowering", lambda: (oracle.lower(n, dst, src), oracle.lower(n, src, dst))),
              ("forward", lambda: oracle.forward(n, src, dst, w, wl.x)),
              ("input_grad", lambda: oracle.input_grad(n, src, dst, w, wl.dy)),
              ("edge_grad", lambda: oracle.edge_grad(src, dst, wl.x, wl.dy)))
    secs = {}
    for name, fn in stages:
        t0 = time.perf_counter()
        fn()
        secs[name] = time.perf_counter() - t0
        log(f"  oracle {name} over {sample_edges} edges: {secs[name]:.1f}s")
    dt = sum(secs.values())
    b = algorithmic_bytes(n, sample_edges, h, 2, 8)
    total = b["build"] + b["fwd"] + b["dx"] + b["dw"]
    return {"value": round(total / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "seconds": round(dt, 2),
            "seconds_per_stage": {k: round(v, 2) for k, v in secs.items()},
            "edges_per_s": round(sample_edges / dt, 1), "nproc": os.cpu_count(),
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
        # the split calls (longest rows cut across workgroups) where a row is long enough
        need = mp.mp_spmm_split_workspace_size(g, h)
        sws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        calls = {"build": lambda: mp.mp_graph_build(src, dst, n),
                 "fwd": lambda: mp.mp_spmm_fwd(g, w, x, out=y),
                 "dx": lambda: mp.mp_spmm_dx(g, w, dy, out=dx),
                 "dw": lambda: mp.mp_edge_grad_dw(g, x, dy, out=dw),
                 "bwd": lambda: mp.mp_spmm_dx_edge_grad(g, w, x, dy, out_dx=dx, out_dw=dw)}
        if need:
            calls["fwd_split"] = lambda: mp.mp_spmm_fwd_split(g, w, x, out=y, workspace=sws)
            calls["dx_split"] = lambda: mp.mp_spmm_dx_split(g, w, dy, out=dx, workspace=sws)
            calls["bwd_split"] = lambda: mp.mp_spmm_dx_edge_grad_split(g, w, x, dy, out_dx=dx,
                                                                       out_dw=dw, workspace=sws)
        b = algorithmic_bytes(n, e, h, 4, 8)
        b["fwd_split"], b["dx_split"], b["bwd_split"] = b["fwd"], b["dx"], b["bwd"]
        res = {"num_nodes": n, "num_edges": e, "feature_width": h, "feature_storage": "f32",
               "split_workspace_bytes": need}
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
        del g, src, dst, w, x, dy, y, dx, dw, sws
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
      graph     -- the async schedule captured once in a HIP graph and replayed.
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

    # The asynchronous schedule captured once into a HIP graph and replayed: no
    # host launch work per batch (each replay repeats the same 64 builds and
    # compute calls on the staged batches).
    cur = torch.cuda.current_stream(dev)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(cur)
    with torch.cuda.stream(side):                     # allocator warm-up outside the capture
        run_async()
    cur.wait_stream(side)
    torch.cuda.synchronize()
    ref = (y.clone(), dx.clone(), dw.clone())         # the last batch, eager
    cg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(cg, capture_error_mode="relaxed"):
        run_async()

    def run_graph():
        cg.replay()

    out = {}
    for name, fn in (("sync", run_sync), ("async", run_async), ("pipelined", run_pipelined),
                     ("graph", run_graph)):
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
        b_total += bb["build"] + bb["fwd"] + bb["bwd"]
    e_total = sum(t["e"] for t in staged)
    run_graph()
    torch.cuda.synchronize()
    graph_equal = bool(torch.equal(y, ref[0]) and torch.equal(dx, ref[1]) and torch.equal(dw, ref[2]))
    res = {"batches": len(staged), "feature_width": h, "feature_dtype": "f32",
           "graph_replay_equal_to_eager": graph_equal,
           "edges_total": e_total, "nodes_max": n_max, "edges_max": e_max,
           "algorithmic_bytes_total": b_total,
           "step": "per batch: build + mp_spmm_fwd + mp_spmm_dx_edge_grad"}
    for name, ms in out.items():
        res[name] = {"ms_total": round(ms, 3), "ms_per_batch": round(ms / len(staged), 4),
                     "GBps": round(b_total / (ms * 1e-3) / 1e9, 1),
                     "edges_per_s": round(e_total / (ms * 1e-3), 1)}
    del staged, y, dx, dw, wss, cg
    torch.cuda.empty_cache()
    return res


# rocprofv3 commands whose output --summarize-profiles reads (run from the
# repository root on the GPU machine; <repo> is its absolute path, <out> the
# directory that receives the profiler's output).
PROFILE_COMMANDS = {
    "trace": "cd /tmp && TMPDIR=/tmp rocprofv3 --kernel-trace --stats --output-format csv "
             "-d <out>/p_trace -o run -- python3 <repo>/bench.py --steps 5 "
             "--warmup 2 --no-cpu-baseline --no-minibatch --no-other-configs",
    "fetch": "cd /tmp && TMPDIR=/tmp rocprofv3 --pmc FETCH_SIZE --output-format csv "
             "-d <out>/p_fetch -o run -- python3 <repo>/bench.py --profile-ops",
    "write": "cd /tmp && TMPDIR=/tmp rocprofv3 --pmc WRITE_SIZE --output-format csv "
             "-d <out>/p_write -o run -- python3 <repo>/bench.py --profile-ops",
    "l2": "cd /tmp && TMPDIR=/tmp rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum --output-format csv "
          "-d <out>/p_l2 -o run -- python3 <repo>/bench.py --profile-ops",
    "minibatch_trace": "cd /tmp && TMPDIR=/tmp rocprofv3 --kernel-trace --stats --output-format "
                       "csv -d <out>/p_trace_mb -o run -- python3 <repo>/bench.py "
                       "--minibatch-only",
    "summary": "python3 bench.py --summarize-profiles <out>",
}


def run_profile_ops(mp, torch, dev, src, dst, w, x, dy, n, e, h):
    """Each op of PROFILE_OPS once after a warm-up of all of them, each preceded
    by a marker kernel, for the counter runs.  Returns the op names in order."""
    y = torch.empty((n, h), dtype=torch.float32, device=dev)
    dx = torch.empty_like(y)
    dw = torch.empty(e, dtype=torch.float32, device=dev)
    wg = torch.empty((e, 2), dtype=torch.float32, device=dev)
    wg[:, 0] = w
    g = mp.mp_graph_build(src, dst, n)
    alpha = torch.empty_like(w)
    rstats = torch.empty((n, 2), dtype=torch.float32, device=dev)
    dscores = torch.empty_like(w)
    rdot = torch.empty(n, dtype=torch.float32, device=dev)
    wn = torch.empty_like(w)
    a_buf = w.clone()
    heads = 4
    wk = torch.empty((e, heads), device=dev).uniform_(
        -1.0, 1.0, generator=torch.Generator(device=dev).manual_seed(7))
    dwk = torch.empty((e, heads), dtype=torch.float32, device=dev)
    ca = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    cb = torch.empty_like(ca)
    marker = torch.empty(64, dtype=torch.int8, device=dev)
    ops = {
        "build": lambda: mp.mp_graph_build(src, dst, n),
        "fwd_pair": lambda: mp.mp_spmm_fwd_pair(g, wg, x, out=y),
        "bwd_pair": lambda: mp.mp_spmm_dx_edge_grad_pair(g, wg, x, dy, out_dx=dx),
        "fwd": lambda: mp.mp_spmm_fwd(g, w, x, out=y),
        "bwd": lambda: mp.mp_spmm_dx_edge_grad(g, w, x, dy, out_dx=dx, out_dw=dw),
        "dx": lambda: mp.mp_spmm_dx(g, w, dy, out=dx),
        "dw": lambda: mp.mp_edge_grad_dw(g, x, dy, out=dw),
        "edge_softmax": lambda: mp.mp_edge_softmax(g, w, alpha, rstats),
        "edge_softmax_backward": lambda: mp.mp_edge_softmax_backward(g, alpha, dw, dscores, rdot),
        "edge_normalize_sym": lambda: mp.mp_edge_normalize(g, mp.MP_NORM_SYM, w, out=wn),
        "attention_forward": lambda: mp.mp_spmm_fwd_softmax(g, w, x, out=y, out_row_stats=rstats),
        "fwd_norm_sym": lambda: mp.mp_spmm_fwd_norm(g, mp.MP_NORM_SYM, w, x, out=y),
        "bwd_norm_sym": lambda: mp.mp_spmm_dx_edge_grad_norm(g, mp.MP_NORM_SYM, w, x, dy,
                                                             out_dx=dx, out_dw=dw),
        "fwd_heads": lambda: mp.mp_spmm_fwd_heads(g, wk, x, out=y),
        "bwd_heads": lambda: mp.mp_spmm_dx_edge_grad_heads(g, wk, x, dy, out_dx=dx, out_dw=dwk),
        "attention_backward": lambda: mp.mp_attention_backward(
            g, w, x, dy, y, out_dx=dx, out_dscores=dscores, out_row_dot=rdot),
        "attention_backward_in_place": lambda: mp.mp_attention_backward(
            g, a_buf, x, dy, y, out_dx=dx, out_dscores=a_buf, out_row_dot=rdot),
        "copy_calibration": lambda: torch.mul(ca, 1.0, out=cb),
    }
    assert tuple(ops) == PROFILE_OPS
    for fn in ops.values():
        fn()
    torch.cuda.synchronize()
    for name, fn in ops.items():
        marker.fill_(1)
        fn()
        torch.cuda.synchronize()
        log(f"profiled {name}")
    return list(ops)


def _read_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _short_name(name):
    name = name.replace("mp::(anonymous namespace)::", "")
    if name.startswith("void "):
        name = name[5:]
    depth, out = 0, []
    for ch in name:     # drop the argument list, keep template arguments
        if ch == "(" and depth == 0:
            break
        depth += ch == "<"
        depth -= ch == ">"
        out.append(ch)
    return "".join(out)


def _per_op_counters(path, counters):
    """{op: {counter: summed value, "kernels": {short name: dispatches},
    "per_kernel": {short name: {counter: summed value}}}} from a
    counter-collection CSV of a --profile-ops run: the dispatches between one
    marker and the next belong to one op."""
    rows = _read_csv(path)
    by_id = {}
    for r in rows:
        d = by_id.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"]})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    ids = sorted(by_id)
    marks = [i for i in ids if MARKER_KERNEL in by_id[i]["name"]]
    if len(marks) != len(PROFILE_OPS):
        raise SystemExit(f"{path}: {len(marks)} markers, expected {len(PROFILE_OPS)}")
    out = {}
    for k, op in enumerate(PROFILE_OPS):
        lo = marks[k]
        hi = marks[k + 1] if k + 1 < len(marks) else ids[-1] + 1
        rec = {c: 0.0 for c in counters}
        rec["kernels"] = {}
        rec["per_kernel"] = {}
        for i in ids:
            if lo < i < hi:
                nm = _short_name(by_id[i]["name"])
                rec["kernels"][nm] = rec["kernels"].get(nm, 0) + 1
                pk = rec["per_kernel"].setdefault(nm, {c: 0.0 for c in counters})
                for c in counters:
                    rec[c] += by_id[i].get(c, 0.0)
                    pk[c] += by_id[i].get(c, 0.0)
        out[op] = rec
    return out


def summarize_profiles(base):
    """Write profiles/kernel_trace_chung_lu_step.md, profiles/hbm_counters_chung_lu_step.md,
    profiles/l2_hit_rates_chung_lu_step.md and profiles/traffic.json from the
    rocprofv3 output directories p_trace, p_fetch, p_write and p_l2 under `base`
    (the commands of PROFILE_COMMANDS)."""
    prof = os.path.join(ROOT, "profiles")
    cmds = "\n".join(PROFILE_COMMANDS[k] for k in ("fetch", "write"))
    # kernel durations
    stats = _read_csv(os.path.join(base, "p_trace", "run_kernel_stats.csv"))
    lines = ["# Kernel trace: power-law workload (N=2,000,000, E=100,000,000, H=128 bf16), "
             "one step = build + forward + fused backward", "",
             "Command (run from the repository root on the GPU box):", "", "```",
             PROFILE_COMMANDS["trace"], "```", "",
             "Summary from rocprofv3's own `run_kernel_stats.csv` (7 steps on the interleaved "
             "weights, then 7 on two arrays, then each standalone call of the benchmark; "
             "kernels of one template share a line):", "",
             "| kernel | calls | avg us | min us | max us | % of GPU time |",
             "|---|---:|---:|---:|---:|---:|"]
    for r in stats:
        lines.append(f"| `{_short_name(r['Name'])}` | {r['Calls']} | "
                     f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                     f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} |")
    lines += ["", "Generated by `" + PROFILE_COMMANDS["summary"] + "`.", ""]
    with open(os.path.join(prof, "kernel_trace_chung_lu_step.md"), "w") as f:
        f.write("\n".join(lines))
    # HBM bytes per op
    fetch = _per_op_counters(os.path.join(base, "p_fetch", "run_counter_collection.csv"),
                             ["FETCH_SIZE"])
    write = _per_op_counters(os.path.join(base, "p_write", "run_counter_collection.csv"),
                             ["WRITE_SIZE"])
    gib_kib = float(1 << 20)
    cal_f = gib_kib / fetch["copy_calibration"]["FETCH_SIZE"]
    cal_w = gib_kib / write["copy_calibration"]["WRITE_SIZE"]
    rec = {"calibration": {"kernel": "torch elementwise x*1.0, 1 GiB read + 1 GiB written",
                           "FETCH_SIZE_KiB": fetch["copy_calibration"]["FETCH_SIZE"],
                           "WRITE_SIZE_KiB": write["copy_calibration"]["WRITE_SIZE"],
                           "fetch_factor": round(cal_f, 4), "write_factor": round(cal_w, 4)},
           "commands": [PROFILE_COMMANDS[k] for k in ("fetch", "write")], "ops": {}}
    lines = ["# HBM byte counters per call: power-law workload (N=2,000,000, E=100,000,000, "
             "H=128 bf16)", "",
             "Two runs, one counter each (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), of "
             "`bench.py --profile-ops` (every op once, each after a marker kernel):", "", "```",
             cmds, "```", "",
             f"Calibration: a plain elementwise copy of 1 GiB (1 GiB read, 1 GiB written) reads "
             f"FETCH_SIZE = {fetch['copy_calibration']['FETCH_SIZE']:.0f} KiB and WRITE_SIZE = "
             f"{write['copy_calibration']['WRITE_SIZE']:.0f} KiB, so bytes = FETCH_SIZE x 1024 x "
             f"{cal_f:.3f} and WRITE_SIZE x 1024 x {cal_w:.3f}.  FETCH_SIZE counts L2 misses, "
             "whichever of the Infinity Cache and HBM serves them.", "",
             "| op | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | GB read | GB written | "
             "GB total |", "|---|---:|---:|---:|---:|---:|---:|"]
    for op in PROFILE_OPS:
        if op == "copy_calibration":
            continue
        fk, wk = fetch[op]["FETCH_SIZE"], write[op]["WRITE_SIZE"]
        rb, wb = fk * 1024 * cal_f, wk * 1024 * cal_w
        nd = sum(fetch[op]["kernels"].values())
        rec["ops"][op] = {"hbm_bytes_per_call": int(round(rb + wb)), "read_bytes": int(round(rb)),
                          "write_bytes": int(round(wb)), "fetch_KiB": fk, "write_KiB": wk,
                          "dispatches": nd, "kernels": fetch[op]["kernels"],
                          "source_hash": op_source_hash(op)}
        lines.append(f"| {op} | {nd} | {fk:.0f} | {wk:.0f} | {rb / 1e9:.3f} | {wb / 1e9:.3f} | "
                     f"{(rb + wb) / 1e9:.3f} |")
    lines += ["", "Kernels of each op:", ""]
    for op in PROFILE_OPS:
        if op != "copy_calibration":
            ks = ", ".join(f"`{k}` x{v}" for k, v in fetch[op]["kernels"].items())
            lines.append(f"- {op}: {ks}")
    lines += ["", "The build's kernels (one lowering of both directions; a line sums the "
              "dispatches of one template):", "",
              "| kernel | dispatches | GB read | GB written |", "|---|---:|---:|---:|"]
    for nm, nd in fetch["build"]["kernels"].items():
        rb = fetch["build"]["per_kernel"][nm]["FETCH_SIZE"] * 1024 * cal_f
        wb = write["build"]["per_kernel"][nm]["WRITE_SIZE"] * 1024 * cal_w
        lines.append(f"| `{nm}` | {nd} | {rb / 1e9:.3f} | {wb / 1e9:.3f} |")
    lines += ["", "`profiles/traffic.json` holds the same figures with a hash of the code of "
              "each op's source files; bench.py reports an op's traffic only while that hash "
              "matches.", "", "Generated by `" + PROFILE_COMMANDS["summary"] + "`.", ""]
    with open(os.path.join(prof, "hbm_counters_chung_lu_step.md"), "w") as f:
        f.write("\n".join(lines))
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    # L2 hit rates per op
    l2_csv = os.path.join(base, "p_l2", "run_counter_collection.csv")
    if os.path.exists(l2_csv):
        l2 = _per_op_counters(l2_csv, ["TCC_HIT_sum", "TCC_MISS_sum"])
        lines = ["# L2 hits and misses per call: power-law workload (N=2,000,000, "
                 "E=100,000,000, H=128 bf16)", "", "```", PROFILE_COMMANDS["l2"], "```", "",
                 "| op | L2 hits | L2 misses | hit rate |", "|---|---:|---:|---:|"]
        for op in PROFILE_OPS:
            hit, miss = l2[op]["TCC_HIT_sum"], l2[op]["TCC_MISS_sum"]
            rate = hit / (hit + miss) if hit + miss else 0.0
            lines.append(f"| {op} | {hit:.4g} | {miss:.4g} | {rate:.3f} |")
        lines += ["", "Source hashes of the code these figures were taken with: " +
                  ", ".join(f"{op} {op_source_hash(op)}" for op in ("build", "fwd", "dw")),
                  "", "Generated by `" + PROFILE_COMMANDS["summary"] + "`.", ""]
        with open(os.path.join(prof, "l2_hit_rates_chung_lu_step.md"), "w") as f:
            f.write("\n".join(lines))
    mb_csv = os.path.join(base, "p_trace_mb", "run_kernel_stats.csv")
    if os.path.exists(mb_csv):
        summarize_minibatch_trace(mb_csv, os.path.join(prof, "kernel_trace_minibatch.md"))
    print(json.dumps({op: v["hbm_bytes_per_call"] for op, v in rec["ops"].items()}))


# Kernel templates of the lowering (the build) and of the aggregations, by name prefix.
_BUILD_KERNELS = ("zero_words_kernel", "intake_count_kernel", "rs_scan", "rs_upsweep",
                  "rs_downsweep", "rowptr_kernel", "rows_")


def summarize_minibatch_trace(csv_path, out_path):
    """profiles/kernel_trace_minibatch.md from rocprofv3's kernel statistics of
    `bench.py --minibatch-only`: every kernel template, then the GPU time per
    build (each template's calls per build times its average duration; one
    counting intake per build) and per forward and fused backward."""
    stats = _read_csv(csv_path)
    lines = ["# Kernel trace: 64 sampled minibatches (about 156K nodes, 168K edges, H = 256 "
             "fp32 each), build + forward + fused backward per batch", "",
             "Command (run from the repository root on the GPU box):", "", "```",
             PROFILE_COMMANDS["minibatch_trace"], "```", "",
             "Summary from rocprofv3's own `run_kernel_stats.csv` (the four schedules of the "
             "minibatch object, each a warm-up and three timed passes over the 64 batches, and "
             "the captured graph's replays; kernels of one template share a line):", "",
             "| kernel | calls | avg us | min us | max us | % of GPU time |",
             "|---|---:|---:|---:|---:|---:|"]
    builds = 0
    for r in stats:
        nm = _short_name(r["Name"])
        if nm.startswith("intake_count_kernel"):
            builds += int(r["Calls"])
        lines.append(f"| `{nm}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.1f} |")
    if builds:
        per_build, launches = 0.0, 0.0
        fwd = bwd = 0.0
        for r in stats:
            nm = _short_name(r["Name"])
            calls, avg = int(r["Calls"]), float(r["AverageNs"]) / 1e3
            if nm.startswith(_BUILD_KERNELS):
                per_build += calls / builds * avg
                launches += calls / builds
            elif nm.startswith("spmm_kernel<float") and ", 0, " in nm:
                fwd += calls / builds * avg
            elif nm.startswith("spmm_kernel<float") and ", 1, " in nm:
                bwd += calls / builds * avg
        lines += ["", f"Per build ({builds} builds traced): {launches:.1f} launches of the "
                  f"lowering, {per_build:.1f} us of kernel time; forward {fwd:.1f} us and fused "
                  f"backward {bwd:.1f} us per batch (kernel time only, without the gaps between "
                  "launches)."]
    lines += ["", "Generated by `" + PROFILE_COMMANDS["summary"] + "`.", ""]
    with open(out_path, "w") as f:
        f.write("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-sample-edges", type=int, default=10_000_000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-full", action="store_true",
                    help="run the single-core oracle baseline over all E edges (minutes) "
                         "instead of the first --cpu-sample-edges")
    ap.add_argument("--no-minibatch", action="store_true",
                    help="skip the back-to-back minibatch schedules")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the timings of the small configurations")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the steps, run one plain 1 GiB -> 1 GiB elementwise copy "
                         "(reference for the HBM byte counters)")
    ap.add_argument("--profile-ops", action="store_true",
                    help="run every profiled op once, each after a marker kernel (for the "
                         "rocprofv3 counter runs), then exit")
    ap.add_argument("--minibatch-only", action="store_true",
                    help="run only the minibatch schedules and print their object (for the "
                         "minibatch kernel trace)")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write the profiles/ summaries from the rocprofv3 output under DIR "
                         "(p_trace, p_fetch, p_write, p_l2), then exit")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py: this build runs on exactly one GPU (got --gpus {args.gpus}); "
              "multi-GPU sharding is described in the design notes, not implemented.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gnn_sparse_message_amd as mp
    import synth

    if args.minibatch_only:
        print(json.dumps({"minibatch": minibatch_bench(mp, torch, torch.device("cuda:0"))}),
              flush=True)
        return
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
    if args.profile_ops:
        torch.cuda.synchronize()
        print(json.dumps({"profile_ops": run_profile_ops(mp, torch, dev, src, dst, w, x, dy,
                                                         n, e, h)}), flush=True)
        return
    y = torch.empty((n, h), dtype=torch.float32, device=dev)
    dx = torch.empty_like(y)
    dw = torch.empty(e, dtype=torch.float32, device=dev)
    # the parameter and its gradient side by side: wg[:, 0] = w, wg[:, 1] <- dw
    wg = torch.empty((e, 2), dtype=torch.float32, device=dev)
    wg[:, 0] = w
    dx_p = torch.empty_like(dx)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    ops = ("build", "fwd", "bwd")

    def step(record, pair):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if record else None
        if record:
            ev[0].record(stream)
        g = mp.mp_graph_build(src, dst, n)
        if record:
            ev[1].record(stream)
        if pair:
            mp.mp_spmm_fwd_pair(g, wg, x, out=y)
        else:
            mp.mp_spmm_fwd(g, w, x, out=y)
        if record:
            ev[2].record(stream)
        if pair:
            mp.mp_spmm_dx_edge_grad_pair(g, wg, x, dy, out_dx=dx_p)
        else:
            mp.mp_spmm_dx_edge_grad(g, w, x, dy, out_dx=dx, out_dw=dw)
        if record:
            ev[3].record(stream)
        return ev, g

    def run_steps(pair, label):
        for i in range(args.warmup):
            step(False, pair)
            log(f"{label}: warmup step {i + 1}/{args.warmup}")
        torch.cuda.synchronize()
        events = []
        t_start = time.perf_counter()
        for i in range(args.steps):
            events.append(step(True, pair)[0])
        torch.cuda.synchronize()
        t_total = time.perf_counter() - t_start
        times = {k: [] for k in ops}
        for ev in events:
            for k, name in enumerate(ops):
                times[name].append(ev[k].elapsed_time(ev[k + 1]))
        log(f"{label}: timed {args.steps} steps in {t_total:.3f}s")
        return t_total, times

    # The headline steps (interleaved weights and gradients), then the same
    # step on separate weight and gradient arrays.
    t_total, times = run_steps(True, "step")
    t_total_2, times_2 = run_steps(False, "step on two arrays")
    torch.cuda.synchronize()
    same_layouts = bool(torch.equal(dx_p, dx) and torch.equal(wg[:, 1], dw))

    # The same step with the transpose half of the build on a second stream
    # (mp_graph_build_overlap), overlapped with the forward aggregation; the
    # fused backward waits for it.  Same work, another schedule.
    side = torch.cuda.Stream(dev)
    ws_o = torch.empty(mp.mp_graph_build_overlap_workspace_size(n, e), dtype=torch.uint8,
                       device=dev)
    y_o, dx_o = torch.empty_like(y), torch.empty_like(dx)
    wg_o = wg.clone()

    def step_overlap(record):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)] if record else None
        if record:
            ev[0].record(stream)
        g, done = mp.mp_graph_build_overlap(src, dst, n, side, workspace=ws_o)
        mp.mp_spmm_fwd_pair(g, wg_o, x, out=y_o)
        stream.wait_event(done)
        mp.mp_spmm_dx_edge_grad_pair(g, wg_o, x, dy, out_dx=dx_o)
        if record:
            ev[1].record(stream)
        return ev

    for i in range(args.warmup):
        step_overlap(False)
    torch.cuda.synchronize()
    ov_events = []
    t_start = time.perf_counter()
    for i in range(args.steps):
        ov_events.append(step_overlap(True))
    torch.cuda.synchronize()
    t_total_ov = time.perf_counter() - t_start
    ov_ms = [a.elapsed_time(b) for a, b in ov_events]
    log(f"step with the overlapped build: timed {args.steps} steps in {t_total_ov:.3f}s")
    overlap_equal = bool(torch.equal(y_o, y) and torch.equal(dx_o, dx_p)
                         and torch.equal(wg_o[:, 1], wg[:, 1]))

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
    # Gather-model bytes of the adjacent calls: every edge touches its operands
    # once, and a per-edge read of a node-sized array (row statistics, row dots,
    # degrees) counts once per edge, as the feature rows do.
    # target softmax: row pass reads order + score per edge and writes 2 stats per
    # row; the edge pass reads dst + score + the row's two statistics, writes alpha.
    # Backward: row pass reads order + alpha + dalpha, writes a row dot; the edge
    # pass reads dst + alpha + dalpha + the row dot and writes ds.
    # (Definition bytes of the operation, not of this implementation's passes.)
    bytes_["edge_softmax"] = 28 * e + 8 * n
    bytes_["edge_softmax_backward"] = 32 * e + 4 * n
    # symmetric normalisation: in, out, src, dst and two row lengths (two row
    # pointers each) per edge.
    bytes_["edge_normalize_sym"] = 32 * e
    # attention forward: the aggregation's bytes (the score in the weight's
    # place) plus the softmax's row pass (order + score per edge, two stats per
    # row written, then read once per row)
    bytes_["attention_forward"] = bytes_["fwd"] + 8 * e + 16 * n
    # multi-head: the edge's weight (or dw) term grows from 4 to 4K bytes.
    bytes_["fwd_heads"] = bytes_["fwd"] + 4 * (heads - 1) * e
    bytes_["bwd_heads"] = bytes_["bwd"] + 8 * (heads - 1) * e
    # per-head softmax: the single-head bytes with K values per edge and per row
    bytes_["edge_softmax_heads"] = 4 * e + 24 * e * heads + 8 * n * heads
    bytes_["edge_softmax_backward_heads"] = 8 * e + 24 * e * heads + 4 * n * heads
    # attention backward: the fused backward's bytes (alpha for w, ds for dw),
    # the row dot gathered per edge, plus the kept forward output Y and dY read
    # once more for the row dots, and the row dots written; with K heads, K
    # values per edge and per row.
    bytes_["attention_backward"] = bytes_["bwd"] + 4 * e + (4 + 2) * n * h + 4 * n
    # normalised at the fetch: the plain call's bytes plus the gathered
    # endpoint's row length (two row pointers) per edge
    bytes_["fwd_norm_sym"] = bytes_["fwd"] + 8 * e
    bytes_["fwd_norm_mean"] = bytes_["fwd"]
    bytes_["bwd_norm_sym"] = bytes_["bwd"] + 8 * e
    bytes_["attention_backward_in_place"] = bytes_["attention_backward"]
    # scores in alpha's place, plus the destination's two statistics per edge
    bytes_["attention_backward_scores"] = bytes_["attention_backward"] + 8 * e
    bytes_["attention_backward_scores_in_place"] = bytes_["attention_backward_scores"]
    bytes_["attention_backward_heads"] = (bytes_["attention_backward"] + 12 * (heads - 1) * e
                                          + 4 * (heads - 1) * n)
    ms_step = t_total / args.steps * 1e3
    ms_step_2 = t_total_2 / args.steps * 1e3

    def rate(nbytes, ms):
        gbps = nbytes / (ms * 1e-3) / 1e9
        return {"ms": round(ms, 4), "GBps": round(gbps, 1), "frac": round(gbps / PEAK_HBM_GBPS, 4),
                "edges_per_s": round(e / (ms * 1e-3), 1), "algorithmic_bytes": nbytes}

    def pct(v, q):
        v = sorted(v)
        return v[min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))]

    def ops_of(tms):
        res = {k: rate(bytes_[k], statistics.median(tms[k])) for k in ops}
        for k in ops:
            res[k]["p10_ms"] = round(pct(tms[k], 0.1), 4)
            res[k]["p90_ms"] = round(pct(tms[k], 0.9), 4)
        return res

    per_op = ops_of(times)
    per_op_2 = ops_of(times_2)
    build_traffic = measured_traffic("build")
    if build_traffic is not None:
        per_op["build"]["traffic"] = build_traffic
        per_op["build"]["traffic_GBps"] = round(build_traffic / (per_op["build"]["ms"] * 1e-3)
                                                / 1e9, 1)
    per_op_standalone = {k: rate(bytes_[k], v) for k, v in standalone.items()}
    per_op_standalone["equal_to_fused"] = same
    per_op_standalone["heads"] = heads
    per_op_standalone["heads_fused_equal_to_separate"] = same_heads
    # what the fetch-time softmax replaces: the softmax (writing alpha), then the
    # aggregation on alpha; the two give the same Y bit for bit
    per_op_standalone["attention_forward_two_calls_ms"] = round(attn_fwd_two_calls, 4)
    per_op_standalone["attention_forward_equal_to_two_calls"] = attn_fwd_equal
    # what the fetch-time normalisation replaces: a normalisation pass, then the call
    per_op_standalone["fwd_norm_two_calls_ms"] = round(
        standalone["edge_normalize_sym"] + per_op_2["fwd"]["ms"], 4)
    per_op_standalone["bwd_norm_two_calls_ms"] = round(
        standalone["edge_normalize_sym"] * 2 + per_op_2["bwd"]["ms"], 4)
    # what the one-call attention backward replaces: fused backward + softmax backward
    per_op_standalone["attention_backward_unfused_ms"] = round(
        per_op_2["bwd"]["ms"] + standalone["edge_softmax_backward"], 4)
    per_op_standalone["attention_backward_heads_unfused_ms"] = round(
        standalone["bwd_heads"] + standalone["edge_softmax_backward_heads"], 4)
    # Kernels of the step.  The dominant kernel is the one with the most GPU time
    # per step; its achieved bandwidth is the algorithmic bytes of what one launch
    # processes (B_bwd for the fused backward: one gathered dY row per edge feeds
    # both gradients) over its average launch duration.  `traffic` is the
    # calibrated HBM counter bytes of one launch.
    kernels = {"spmm_kernel_fused_backward": ("bwd", "bwd_pair", per_op),
               "spmm_kernel": ("fwd", "fwd_pair", per_op),
               "spmm_kernel_fused_backward_two_arrays": ("bwd", "bwd", per_op_2)}
    roof = {}
    for kname, (op, tkey, src_ops) in kernels.items():
        launch_ms = src_ops[op]["ms"]
        achieved = bytes_[op] / (launch_ms * 1e-3) / 1e9
        traffic = measured_traffic(tkey)
        roof[kname] = {"bound": "hbm", "kernel": f"{kname} ({op})",
                       "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                       "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic,
                       "traffic_GBps": None if traffic is None
                       else round(traffic / (launch_ms * 1e-3) / 1e9, 1),
                       "algorithmic_bytes_per_launch": bytes_[op], "avg_launch_ms": launch_ms}
    dominant = max(("spmm_kernel_fused_backward", "spmm_kernel"),
                   key=lambda k: roof[k]["avg_launch_ms"])
    total_bytes = bytes_["build"] + bytes_["fwd"] + bytes_["bwd"]
    value = total_bytes / (ms_step * 1e-3) / 1e9
    value_2 = total_bytes / (ms_step_2 * 1e-3) / 1e9
    ms_step_ov = t_total_ov / args.steps * 1e3
    value_ov = total_bytes / (ms_step_ov * 1e-3) / 1e9
    out = {
        "metric": "SpMM fwd/dX + SDDMM dw effective HBM GB/s and edges/s; % of HBM roofline",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "chung_lu_powerlaw", "num_nodes": n, "num_edges": e,
                   "feature_width": h, "degree_exponent": 2.1, "degree_cap": 100000,
                   "feature_storage": "bf16", "index_input": "int64",
                   "weights": "w and dw interleaved in one [E][2] array, COO order",
                   "step": "mp_graph_build + mp_spmm_fwd_pair + mp_spmm_dx_edge_grad_pair"},
        "algorithmic_bytes_per_step": total_bytes,
        "edges_per_s": round(e / (ms_step * 1e-3), 1),
        "frac_of_hbm_peak": round(value / PEAK_HBM_GBPS, 4),
        "per_op": per_op,
        "step_two_arrays": {
            "step": "mp_graph_build + mp_spmm_fwd + mp_spmm_dx_edge_grad (w and dw separate)",
            "ms_per_step": round(ms_step_2, 4), "value": round(value_2, 1), "unit": "GB/s",
            "frac_of_hbm_peak": round(value_2 / PEAK_HBM_GBPS, 4), "per_op": per_op_2,
            "outputs_equal_to_interleaved_step": same_layouts},
        "step_overlapped_build": {
            "step": "mp_graph_build_overlap (transpose half on a second stream) + "
                    "mp_spmm_fwd_pair, then mp_spmm_dx_edge_grad_pair after the transpose",
            "ms_per_step": round(ms_step_ov, 4),
            "value": round(value_ov, 1), "unit": "GB/s",
            "frac_of_hbm_peak": round(value_ov / PEAK_HBM_GBPS, 4),
            "event_median_ms_per_step": round(statistics.median(ov_ms), 4),
            "outputs_equal_to_step": overlap_equal},
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
            f"{k} {out['minibatch'][k]['ms_per_batch']}"
            for k in ("sync", "async", "pipelined", "graph")))
    if not args.no_cpu_baseline:
        sample = e if args.cpu_full else min(args.cpu_sample_edges, e)
        log(f"cpu baseline: oracle on {sample} edges, one core ...")
        out["cpu_baseline"] = cpu_baseline(wl, sample)
        log("cpu baseline: the same definitions on every core, all edges ...")
        out["cpu_baseline_all_cores"] = cpu_baseline_all_cores(wl)
        log("cpu baseline of the adjacent operations ...")
        out["cpu_baseline_adjacent"] = cpu_baseline_adjacent(wl, min(args.cpu_sample_edges, e))
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
