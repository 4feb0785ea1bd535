"""Seeded synthetic workloads for weighted sparse message passing.

This module only draws inputs: COO topologies, edge weights and feature /
gradient matrices.  It holds none of the arithmetic of the method itself, so
both the oracle side and the device side of every test can consume the same
arrays.  All draws use numpy ``Generator(PCG64(seed))`` and happen in the
fixed order src, dst, w, X, dY.

Workloads (shapes and distributions after the pages; readings in the design
notes):

* ``witness``       -- the 3-node / 3-edge fixture of tinymesh "Weighted
                       aggregation experiment", section "Exact witness".
* ``tiny_uniform``  -- N=1,000, E=10,000 uniform src/dst (duplicates and
                       self-loops kept), H=16 fp32, w ~ U[-1, 1].
* ``sbm``           -- 8-block stochastic block model on N=16,384 nodes with
                       about 566,564 directed edges (the edge count of the toy
                       SBM in "PyTorch Geometric: one abstraction, the whole GNN
                       literature", "The problem in one sentence"), H=64 fp32.
* ``rmat16``        -- RMAT scale 16, edge factor 16, (a,b,c,d) = (.57,.19,.19,.05),
                       H=128 fp32 (the RMAT scale-16 graph of the same page's
                       footprint question).
* ``chung_lu``      -- power-law Chung-Lu graph, N=2,000,000, E=100,000,000,
                       exponent 2.1, per-direction expected degree capped at
                       100,000, H=128 bf16 features (RNE from fp32 draws).
* ``minibatches``   -- 2-hop sampled subgraphs in the NeighborLoader batch
                       shape of AetherGraph "INTEGRATION.md" ("Batch
                       Attributes", "Rust Sampling Engine"): 1,024 seeds,
                       fanout [15, 10] without replacement from a base graph
                       where every node has 30 distinct uniform out-neighbours,
                       relabelled seeds-first in discovery order, H=256 fp32.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def bf16_round(a: np.ndarray):
    """Round float32 to bfloat16 with round-to-nearest-even.

    Returns (bits uint16, widened float32).  The widened array holds exactly
    the values a device reading the bf16 bits sees, so it is what the oracle
    consumes.  Inputs are finite normal draws, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    bits = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    wide = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return bits, wide


@dataclass
class Workload:
    """One input set.  ``x``/``dy`` are float32 holding the exact device values."""
    name: str
    n: int
    src: np.ndarray          # int64 [E], COO order
    dst: np.ndarray          # int64 [E]
    w: np.ndarray            # float32 [E], COO order
    x: np.ndarray            # float32 [N, H]
    dy: np.ndarray           # float32 [N, H]
    feat_dtype: str = "f32"  # "f32" or "bf16"
    x_bits: Optional[np.ndarray] = None   # uint16 [N, H] when feat_dtype == "bf16"
    dy_bits: Optional[np.ndarray] = None
    meta: dict = field(default_factory=dict)

    @property
    def e(self) -> int:
        return int(self.src.shape[0])

    @property
    def h(self) -> int:
        return int(self.x.shape[1])


def _features(rng, n, h, feat_dtype):
    x = rng.standard_normal((n, h), dtype=np.float32)
    dy = rng.standard_normal((n, h), dtype=np.float32)
    if feat_dtype == "bf16":
        xb, x = bf16_round(x)
        dyb, dy = bf16_round(dy)
        return x, dy, xb, dyb
    return x, dy, None, None


def witness() -> Workload:
    """tinymesh "Weighted aggregation experiment", "Exact witness": edges 0->2, 1->2,
    0->1 with weights (2, -1, 3); node values X = (2, 4, 8); output gradient
    dY = (0, 5, 7); H = 1."""
    return Workload(
        name="witness", n=3,
        src=np.array([0, 1, 0], np.int64), dst=np.array([2, 2, 1], np.int64),
        w=np.array([2, -1, 3], np.float32),
        x=np.array([[2], [4], [8]], np.float32), dy=np.array([[0], [5], [7]], np.float32))


def random_graph(n: int, e: int, h: int, seed: int, feat_dtype: str = "f32",
                 w_low: float = -1.0, w_high: float = 1.0, name: str = "random") -> Workload:
    """Uniform src/dst in [0, n) (duplicates and self-loops kept), w ~ U[w_low, w_high]."""
    rng = _rng(seed)
    src = rng.integers(0, n, e).astype(np.int64)
    dst = rng.integers(0, n, e).astype(np.int64)
    w = rng.uniform(w_low, w_high, e).astype(np.float32)
    x, dy, xb, dyb = _features(rng, n, h, feat_dtype)
    return Workload(name, n, src, dst, w, x, dy, feat_dtype, xb, dyb)


def tiny_uniform(seed: int = 1) -> Workload:
    """N=1,000, E=10,000 uniform edges, w ~ U[-1, 1], X, dY ~ N(0, 1) [N, 16] fp32."""
    return random_graph(1000, 10000, 16, seed, name="tiny_uniform")


def sbm(seed: int = 2, n_blocks: int = 8, block: int = 2048, h: int = 64,
        target_edges: float = 566564.0) -> Workload:
    """Directed 8-block SBM: every ordered pair u != v is an edge independently,
    with p_in inside a block and p_out across blocks.  The nominal 0.0173 / 0.0004
    give about 674K expected edges, not the ~566K the pages quote, so both are
    scaled by the same factor to make the expectation 566,564 (ratio kept).
    Edge (u, v) is stored as src = u, dst = v; the COO order is then shuffled."""
    rng = _rng(seed)
    n = n_blocks * block
    intra_pairs = block * (block - 1)
    inter_pairs = block * block
    base = n_blocks * intra_pairs * 0.0173 + n_blocks * (n_blocks - 1) * inter_pairs * 0.0004
    scale = target_edges / base
    p_in, p_out = 0.0173 * scale, 0.0004 * scale
    srcs, dsts = [], []
    for a in range(n_blocks):
        for b in range(n_blocks):
            if a == b:
                k = rng.binomial(intra_pairs, p_in)
                q = rng.choice(intra_pairs, size=k, replace=False)
                u = q // (block - 1)
                v = q % (block - 1)
                v = v + (v >= u)
            else:
                k = rng.binomial(inter_pairs, p_out)
                q = rng.choice(inter_pairs, size=k, replace=False)
                u = q // block
                v = q % block
            srcs.append(a * block + u)
            dsts.append(b * block + v)
    src = np.concatenate(srcs).astype(np.int64)
    dst = np.concatenate(dsts).astype(np.int64)
    perm = rng.permutation(src.shape[0])
    src, dst = src[perm], dst[perm]
    w = rng.uniform(0.0, 1.0, src.shape[0]).astype(np.float32)
    x, dy, _, _ = _features(rng, n, h, "f32")
    return Workload("sbm", n, src, dst, w, x, dy,
                    meta={"p_in": p_in, "p_out": p_out})


def rmat(scale: int, edge_factor: int, seed: int, h: int,
         probs=(0.57, 0.19, 0.19, 0.05), name: str = "rmat") -> Workload:
    """RMAT: each edge picks one quadrant per level (a=(0,0), b=(0,1), c=(1,0),
    d=(1,1)); the row bit goes to src, the column bit to dst, most significant
    level first.  No noise, no vertex permutation; duplicates and self-loops
    kept; edges in draw order.  w ~ N(0, 1); X, dY ~ N(0, 1) fp32."""
    rng = _rng(seed)
    n = 1 << scale
    e = edge_factor * n
    cdf = np.cumsum(np.asarray(probs, np.float64))
    src = np.zeros(e, np.int64)
    dst = np.zeros(e, np.int64)
    for _ in range(scale):
        q = np.searchsorted(cdf, rng.random(e), side="right")
        q = np.minimum(q, 3)
        src = (src << 1) | (q >> 1)
        dst = (dst << 1) | (q & 1)
    w = rng.standard_normal(e).astype(np.float32)
    x, dy, _, _ = _features(rng, n, h, "f32")
    return Workload(name, n, src, dst, w, x, dy)


def rmat16(seed: int = 3) -> Workload:
    return rmat(16, 16, seed, 128, name="rmat16")


def chung_lu_degrees(n: int, e: int, gamma: float, cap: float) -> np.ndarray:
    """Expected per-direction degrees d_i = min(C (i+1)^(-1/(gamma-1)), cap),
    with C solved by bisection so that sum(d) = e.  Ids are in decreasing-degree
    order."""
    base = np.arange(1, n + 1, dtype=np.float64) ** (-1.0 / (gamma - 1.0))
    lo, hi = 0.0, float(e)
    for _ in range(200):
        c = 0.5 * (lo + hi)
        if np.minimum(c * base, cap).sum() < e:
            lo = c
        else:
            hi = c
    return np.minimum(0.5 * (lo + hi) * base, cap)


class _GuideSampler:
    """Inverse-CDF sampling of a discrete distribution with a guide table
    (equal-probability buckets point at the first candidate index)."""

    def __init__(self, p: np.ndarray):
        cdf = np.cumsum(p / p.sum())
        cdf[-1] = 1.0
        self.cdf = cdf
        self.m = cdf.shape[0]
        self.guide = np.searchsorted(cdf, np.arange(self.m, dtype=np.float64) / self.m,
                                     side="right")

    def draw(self, u: np.ndarray) -> np.ndarray:
        """Smallest index i with cdf[i] > u, for each u in [0, 1)."""
        b = np.minimum((u * self.m).astype(np.int64), self.m - 1)
        idx = self.guide[b]
        act = np.nonzero(self.cdf[idx] <= u)[0]
        while act.size:
            idx[act] += 1
            act = act[self.cdf[idx[act]] <= u[act]]
        return idx


def chung_lu(seed: int = 4, n: int = 2_000_000, e: int = 100_000_000, gamma: float = 2.1,
             cap: float = 100_000.0, h: int = 128, feat_dtype: str = "bf16",
             chunk: int = 10_000_000) -> Workload:
    """Chung-Lu power law: e i.i.d. edges, src and dst drawn independently with
    probability proportional to the expected degree (cap applied per direction).
    Duplicates and self-loops kept; COO order is draw order.  w ~ U[-1, 1];
    X, dY ~ N(0, 1) drawn in fp32 and rounded to bf16 (RNE)."""
    rng = _rng(seed)
    d = chung_lu_degrees(n, e, gamma, cap)
    smp = _GuideSampler(d)
    out = []
    for _ in range(2):                       # src, then dst
        arr = np.empty(e, np.int64)
        for s in range(0, e, chunk):
            m = min(chunk, e - s)
            arr[s:s + m] = smp.draw(rng.random(m))
        out.append(arr)
    src, dst = out
    w = rng.uniform(-1.0, 1.0, e).astype(np.float32)
    x, dy, xb, dyb = _features(rng, n, h, feat_dtype)
    return Workload("chung_lu", n, src, dst, w, x, dy, feat_dtype, xb, dyb,
                    meta={"gamma": gamma, "cap": cap})


def base_graph(seed: int = 5, n: int = 1 << 20, out_degree: int = 30) -> np.ndarray:
    """Every node gets `out_degree` distinct uniform out-neighbours, no self-loop."""
    rng = _rng(seed)
    nbr = rng.integers(0, n - 1, size=(n, out_degree), dtype=np.int64)
    own = np.arange(n, dtype=np.int64)[:, None]
    nbr = nbr + (nbr >= own)
    while True:
        srt = np.sort(nbr, axis=1)
        bad = np.nonzero((srt[:, 1:] == srt[:, :-1]).any(axis=1))[0]
        if bad.size == 0:
            return nbr
        redo = rng.integers(0, n - 1, size=(bad.size, out_degree), dtype=np.int64)
        nbr[bad] = redo + (redo >= bad[:, None])


def _sample_without_replacement(rng, nbr_rows: np.ndarray, k: int) -> np.ndarray:
    """k of each row's entries, uniformly without replacement, in sample order."""
    keys = rng.random(nbr_rows.shape)
    pick = np.argsort(keys, axis=1, kind="stable")[:, :k]
    return np.take_along_axis(nbr_rows, pick, axis=1)


def minibatches(n_batches: int = 64, seed: int = 5, batch_size: int = 1024,
                fanout=(15, 10), h: int = 256, nbr: Optional[np.ndarray] = None,
                first: int = 0, features: bool = True) -> List[Workload]:
    """2-hop sampled subgraphs.  Seeds: disjoint slices of one seeded permutation
    of the base nodes.  Hop 1: each seed samples fanout[0] neighbours; hop 2:
    each newly discovered node samples fanout[1].  Relabel: seeds 0..B-1, then
    new nodes in discovery order; nodes already seen keep their id and are not
    expanded again.  Edges: src = sampled neighbour, dst = the node that sampled
    it, in sampler order.  Batch b draws from seed 500 + b.  Returns batches
    first .. first + n_batches - 1.  The features are drawn after the weights,
    so features=False gives the same topology and weights."""
    if nbr is None:
        nbr = base_graph(seed)
    n_base = nbr.shape[0]
    seeds_all = _rng(seed + 1).permutation(n_base)
    local = np.full(n_base, -1, np.int64)
    out = []
    for b in range(first, first + n_batches):
        rng = _rng(500 + b)
        seeds = seeds_all[b * batch_size:(b + 1) * batch_size]
        local[seeds] = np.arange(seeds.shape[0])
        order = [seeds]
        n_loc = seeds.shape[0]
        frontier = seeds
        srcs, dsts = [], []
        for k in fanout:
            smp = _sample_without_replacement(rng, nbr[frontier], k)      # [F, k] global ids
            flat = smp.reshape(-1)
            dst_g = np.repeat(frontier, k)
            uniq, first_at = np.unique(flat, return_index=True)
            new = uniq[local[uniq] < 0]
            new = new[np.argsort(first_at[local[uniq] < 0], kind="stable")]
            local[new] = n_loc + np.arange(new.shape[0])
            n_loc += new.shape[0]
            order.append(new)
            srcs.append(local[flat])
            dsts.append(local[dst_g])
            frontier = new
        n_id = np.concatenate(order)
        src = np.concatenate(srcs).astype(np.int64)
        dst = np.concatenate(dsts).astype(np.int64)
        local[n_id] = -1
        w = rng.uniform(0.0, 1.0, src.shape[0]).astype(np.float32)
        # features=False leaves X and dY out (None): topology and weights only
        x, dy, _, _ = _features(rng, n_loc, h, "f32") if features else (None, None, None, None)
        out.append(Workload(f"minibatch{b}", n_loc, src, dst, w, x, dy,
                            meta={"n_id": n_id, "batch_size": batch_size}))
    return out
