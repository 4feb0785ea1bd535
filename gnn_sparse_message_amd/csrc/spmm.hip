// spmm.hip -- weighted CSR aggregation out[i, :] = sum_p w[order[p]] * in[col[p], :]
// over p in [rowptr[i], rowptr[i+1]), with w in COO order.
//
// The forward pass Y = A_w X runs it on the destination-owned CSR with
// edge_order, the input gradient dX = A_w^T dY on the source-owned CSR with
// transpose_order (tinymesh "Weighted aggregation experiment", "Decision" and
// the two columns of the diagram under "Edge order is explicit").  Each output
// row has exactly one owner, there are no atomics and no [E, H] message rows.
//
// Mapping on gfx950.  A feature row is split over a "group" of L lanes, each
// lane holding VEC contiguous features (16-byte loads: 4 fp32 or 8 bf16; 8 fp32
// in two loads for rows of 256 fp32 features or more, f32_vec).  Rows
// are visited through the degree plan (rows sorted by length class, longest
// first) and handed to owners of three sizes within one launch, so long rows
// start first and their tail overlaps the short ones:
//   hub  rows -> a whole 256-thread workgroup (4 waves split the edges, then a
//                fixed-order LDS reduction);
//   long rows -> one 64-lane wave (64/L groups split the edges, butterfly
//                reduction across groups);
//   short rows (and empty rows, written as zeros) -> one group of L lanes.
// When a few rows hold much of a graph (owner_rule below) the hub rows instead
// get 1024-thread workgroups, 16 waves each, in a launch just before the main
// one (spmm_hub_kernel).
// For each run of edges the team loads col[p] and order[p] once, coalesced, one
// edge per lane, and gathers w[order[p]]; it broadcasts them with lane permutes
// while every group gathers U feature rows at a time (several 16-byte loads in
// flight per lane).  Accumulation is fp32; bf16 inputs are widened exactly.
// Feature widths above 64*VEC are covered by column blocks in gridDim.y.
//
// The same walk serves the fused backward over the transpose CSR (kDw: the
// edge gradients formed from the gathered dY rows and the owner's X row), the
// attention backward (kScoreGrad: score gradients instead, from the row dots
// <Y, dY>) and the degree normalisation at the fetch (kNorm: each weight
// scaled by its edge's degree factor as it is read).
//
// Multi-head weights (w is [E, K], head q owning columns [q*H/K, (q+1)*H/K) of
// every row; the per-head reading of vector edge weights, which tinymesh
// "Weighted aggregation experiment", "Limits" names as not yet covered): every
// lane's VEC columns lie in one head, so a lane reads the weight of its own
// head, w[order[p] * K + q], beside the feature row; the fused backward reduces
// the edge dot product over the lanes of each head separately.
#include "common.h"

#include <math.h>

#include <atomic>

namespace mp {
namespace {

// ------------------------------------------------------------------ feature loads
template <typename T, int VEC>
struct Feat;

template <>
struct Feat<float, 4> {
    static __device__ __forceinline__ void load(const float *p, float (&v)[4]) {
        const float4 q = *reinterpret_cast<const float4 *>(p);
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    }
};
template <>
struct Feat<float, 8> {
    static __device__ __forceinline__ void load(const float *p, float (&v)[8]) {
        const float4 q0 = *reinterpret_cast<const float4 *>(p);
        const float4 q1 = *reinterpret_cast<const float4 *>(p + 4);
        v[0] = q0.x; v[1] = q0.y; v[2] = q0.z; v[3] = q0.w;
        v[4] = q1.x; v[5] = q1.y; v[6] = q1.z; v[7] = q1.w;
    }
};
template <>
struct Feat<float, 1> {
    static __device__ __forceinline__ void load(const float *p, float (&v)[1]) { v[0] = *p; }
};
template <>
struct Feat<uint16_t, 8> {   // bf16: widen exactly by placing the bits in the high half
    static __device__ __forceinline__ void load(const uint16_t *p, float (&v)[8]) {
        const uint4 q = *reinterpret_cast<const uint4 *>(p);
        const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(u[i] << 16);
            v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    }
};
template <>
struct Feat<uint16_t, 1> {
    static __device__ __forceinline__ void load(const uint16_t *p, float (&v)[1]) {
        v[0] = __uint_as_float((uint32_t)(*p) << 16);
    }
};

// A gathered feature slice as loaded: bf16 stays packed two to a register until
// each value is used (widening is exact, so the values are those of Feat), which
// halves the registers a row in flight holds.
template <typename T, int VEC>
struct Raw;

template <int VEC>
struct Raw<float, VEC> {
    float f[VEC];
    __device__ __forceinline__ void load(const float *p) { Feat<float, VEC>::load(p, f); }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int v = 0; v < VEC; ++v) f[v] = 0.f;
    }
    __device__ __forceinline__ float at(int v) const { return f[v]; }
};
template <>
struct Raw<uint16_t, 8> {
    uint32_t q[4];
    __device__ __forceinline__ void load(const uint16_t *p) {
        const uint4 r = *reinterpret_cast<const uint4 *>(p);
        q[0] = r.x; q[1] = r.y; q[2] = r.z; q[3] = r.w;
    }
    __device__ __forceinline__ void zero() { q[0] = q[1] = q[2] = q[3] = 0u; }
    __device__ __forceinline__ float at(int v) const {
        return (v & 1) ? __uint_as_float(q[v >> 1] & 0xffff0000u) : __uint_as_float(q[v >> 1] << 16);
    }
};
template <>
struct Raw<uint16_t, 1> {
    uint32_t q;
    __device__ __forceinline__ void load(const uint16_t *p) { q = (uint32_t)(*p); }
    __device__ __forceinline__ void zero() { q = 0u; }
    __device__ __forceinline__ float at(int) const { return __uint_as_float(q << 16); }
};

// Output rows are written once and not read again here: non-temporal stores
// keep them from displacing hot feature rows in L2.
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int VEC>
__device__ __forceinline__ void store_row(float *p, const float (&v)[VEC]) {
    if constexpr (VEC % 4 == 0) {
#pragma unroll
        for (int i = 0; i < VEC; i += 4) {
            const f32x4 q = {v[i], v[i + 1], v[i + 2], v[i + 3]};
            __builtin_nontemporal_store(q, reinterpret_cast<f32x4 *>(p + i));
        }
    } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i) __builtin_nontemporal_store(v[i], p + i);
    }
}

// Lane-local part of <xr, xv>: an fma chain from zero in element order, the
// same operations as the COO-order edge-gradient kernel (so both give equal dw).
// No bare product is left, so nothing can be contracted into the lane
// reduction that follows.
template <typename T, int VEC>
__device__ __forceinline__ float edge_dot(const float (&xr)[VEC], const Raw<T, VEC> &xv) {
    float s = 0.f;
#pragma unroll
    for (int v = 0; v < VEC; ++v) s = fmaf(xr[v], xv.at(v), s);
    return s;
}

// Sum of `part` over the `seg` lanes of one head (aligned runs of seg lanes
// inside a group; every lane of the run gets the total).  A power-of-two run is
// reduced by run_sum, any other in lane order; the COO-order multi-head
// edge-gradient kernel reduces its lanes the same way, so both give equal dw.
// `seg` is uniform across the wave.
__device__ __forceinline__ float head_sum(float part, int lane, int sub, int seg) {
    if ((seg & (seg - 1)) == 0) return run_sum(part, seg);
    const int first = lane - sub % seg;
    float t = __shfl(part, first);
    for (int i = 1; i < seg; ++i) t += __shfl(part, first + i);
    return t;
}

// What the kernel writes besides the aggregation.
constexpr int kPlain = 0;        // nothing: forward or input gradient
constexpr int kDw = 1;           // edge-weight gradients (fused backward)
constexpr int kScoreGrad = 2;    // gradients of the scores behind softmax weights
constexpr int kDwPair = 3;       // as kDw, with w and dw interleaved ([E][2]: w, dw)
constexpr int kScoreGradInPlace = 4;   // as kScoreGrad, the score gradients written over
                                       // alpha (dw == w)
constexpr bool score_mode(int m) { return m == kScoreGrad || m == kScoreGradInPlace; }

// Feature rows in flight per group per step.  The single-head aggregation
// keeps six, the fused backward (which also holds the owner row and the dot
// products) and the multi-head kernels four; with the rows held packed (Raw)
// the single-head aggregation then fits seven waves per SIMD.
template <int kMode, bool kHeads, bool kNorm>
constexpr int unroll_for() { return kMode == kPlain && !kHeads ? 6 : 4; }

struct SpmmArgs {
    const int32_t *rowptr;
    const int32_t *col;
    const int32_t *order;
    const int32_t *plan;
    const float *w;
    int64_t w_stride;                 // floats from one edge's weight to the next: 1, or 2
                                      // when weights and gradients are interleaved
    const void *x;                    // gathered rows (X forward, dY input gradient)
    float *y;
    const void *x_own;                // fused backward only: X, read at the owner row
    float *dw;                        // fused backward only: edge gradients (or score
                                      // gradients, see row_dot), COO order
    const float *row_dot;             // score-gradient mode: t[dst, head] = <Y, dY> of the
                                      // row; dw then receives w * (<x_own, x> - t)
    int64_t h;
    int32_t heads;                    // K weights per edge (multi-head kernels only)
    int32_t head_w;                   // H / K columns per head
    int64_t n, e;                     // rows, edges (bounds for the data-dependent indices)
    int32_t n_hub, n_wave, n_group;   // rows of each owner kind, consecutive in the plan
    int32_t blk_hub, blk_wave, blk_group;   // blocks given to each kind (wave and group
                                            // owners stride over their rows)
    int32_t hub_apart;                // hub rows go to spmm_hub_kernel (no hub blocks here)
    int32_t n_full;                   // rows with an edge: plan positions from here on are
                                      // empty rows (class 0 comes last)
    const uint32_t *dev_totals;       // asynchronously built graph: the plan's rows per class
                                      // on the device; the eight fields above are then
                                      // derived in the kernel, by owner_rule
    int32_t wave_min;                 // rows this long or longer (below hub) get a wave
    int32_t force_hub, force_apart;   // owner_rule overrides (> 0 / >= 0), else -1
    NormSpec norm;                    // normalising kernels only: fetch-time weight scaling
    // Split rows (the split calls): plan positions [0, n_split) are cut into
    // chunks of chunk_len edges.  Chunk items come first in the main launch;
    // item i writes its partial row sum to partials[i * h ...]; the combine
    // launch then adds each row's partials in chunk order.  Rows of one degree
    // class get the same number of item slots (enough for its longest row);
    // cls_items / cls_rows are cumulative over the split classes, highest first.
    float *partials;
    int32_t n_split, blk_chunk, chunk_len, n_split_cls;
    int32_t cls_items[MP_NUM_CLASSES], cls_rows[MP_NUM_CLASSES], cls_slots[MP_NUM_CLASSES];
};

constexpr int64_t kMaxKindBlocks = 1 << 22;   // wave and group owners stride beyond this

// Hub rows: workgroups of four waves in the main launch, or of 16 waves in a
// launch of their own (spmm_hub_kernel).
constexpr int kHubWaves = 16;
constexpr int kHubBlock = kHubWaves * kWave;
constexpr int64_t kWaveSlots = 256 * 4 * 4;   // CUs x SIMDs x four waves
// Hub blocks of an asynchronously built graph's launches (counts unknown to the
// host: the grid is a bound, so it is kept small and the blocks stride).
constexpr int64_t kAsyncHubBlocks = 1024, kAsyncHubBlocks16 = 256;
// The same for its wave and lane-group owners: a bound sized for every row of
// the graph would launch hundreds of thousands of blocks that find no work
// (about 0.4 ms on the power-law graph).
constexpr int64_t kAsyncKindBlocks = 16384;
constexpr int kLargeHubLen = 4096;

struct OwnerRule {
    int32_t hub_min;   // rows this long or longer get a workgroup
    int32_t apart;     // ... of 16 waves in their own launch, else of four in the main one
};

// Owner sizes from the edge count, the lane-group width (G edges per wave step)
// and the longest nonempty length class only, all of which the host knows for a
// synchronously built graph and the kernels read for an asynchronously built
// one; the owners, and with them the summation order, are the same either way.
// The chip's wave slots share the edges: a row much longer than one slot's share
// finishes after the rest of the launch.  When the longest class starts beyond
// eight shares (a few hub rows hold a large part of the edges, as in RMAT) even
// four waves leave such a row as the tail, so rows of 128 edges or two steps of
// 16 waves, whichever is longer, get 16 waves each.  Otherwise rows of about one
// share (a power of two, at most 4096 and at least two steps of four waves) get
// the main launch's four-wave workgroups, so no single wave holds more than
// about a share.
__host__ __device__ inline OwnerRule owner_rule(int64_t top_len, int64_t e, int G,
                                                int32_t force_hub, int32_t force_apart) {
    const int64_t share = e / kWaveSlots;
    OwnerRule r;
    r.apart = force_apart >= 0 ? force_apart : (top_len > 8 * share ? 1 : 0);
    int64_t len;
    if (r.apart) {
        len = (int64_t)2 * kHubWaves * G;
        if (len < 128) len = 128;
    } else {
        len = 1;
        while (len * 2 <= share && len < kLargeHubLen) len *= 2;
        const int64_t lo = (int64_t)8 * G > 128 ? (int64_t)8 * G : 128;
        if (len < lo) len = lo;
    }
    r.hub_min = force_hub > 0 ? force_hub : (int32_t)len;
    return r;
}

// Owner partition of a plan: rows of each kind and blocks given to each.
struct Partition {
    int32_t n_hub, n_wave, n_group, blk_hub, blk_wave, blk_group;
};

template <int L>
__host__ __device__ inline Partition partition(int64_t at_hub, int64_t at_wave, int64_t n,
                                               int64_t hub_cap = kMaxKindBlocks,
                                               int64_t kind_cap = kMaxKindBlocks) {
    if (at_wave < at_hub) at_wave = at_hub;
    Partition p;
    p.n_hub = (int32_t)at_hub;
    p.n_wave = (int32_t)(at_wave - at_hub);
    p.n_group = (int32_t)(n - at_wave);
    const int64_t rows_per_blk = kBlock / L;
    const int64_t bw = (p.n_wave + kWavesPerBlock - 1) / kWavesPerBlock;
    const int64_t bg = (p.n_group + rows_per_blk - 1) / rows_per_blk;
    p.blk_hub = (int32_t)(p.n_hub < hub_cap ? p.n_hub : hub_cap);   // hub owners stride too
    p.blk_wave = (int32_t)(bw < kind_cap ? bw : kind_cap);
    p.blk_group = (int32_t)(bg < kind_cap ? bg : kind_cap);
    return p;
}

// Accumulate edges [beg, end) of one row into acc.  The team is TL lanes of one
// wave (TL = 64 for wave and hub owners, TL = L for group owners) and walks the
// row in runs of TL edges: run starts are `first`, `first + stride`, ...  All
// lanes of the team execute every permute with the same trip count, so each
// permute reads from an active lane.
// With kMode >= kDw (the fused backward over the transpose CSR, rows = sources)
// every gathered dY slice also meets the owner row's X slice `xr`: the group
// reduces their dot product over its L lanes (same lane order and butterfly as
// the COO-order edge-gradient kernel) and one lane writes dw[order[p]].  With
// kMode == kScoreGrad the weights are softmax outputs alpha and that lane
// writes the score gradient alpha * (dot - t[dst]) instead (t from row_dot);
// kScoreGradInPlace writes it over alpha itself (each edge is read once, by the
// group that then writes it).
// With kHeads every lane reads the weight of its own head, `head`, per edge.
// With kNorm every weight is scaled as it is fetched by its edge's degree
// factor (own_deg: the owner row's length), and the fused backward's dot by the
// same factor.
template <typename T, int VEC, int L, int TL, int kMode, bool kHeads, bool kNorm>
__device__ __forceinline__ void accumulate(const SpmmArgs &a, int64_t first, int64_t end,
                                           int64_t stride, int lane, int64_t hoff, int head,
                                           bool active, const float (&xr)[VEC],
                                           float (&acc)[VEC], double own_deg, float2 own_st) {
    constexpr int G = TL / L;                 // groups per team
    constexpr int kUnroll = unroll_for<kMode, kHeads, kNorm>();
    const int tl = lane % TL;
    const int tb = lane - tl;                 // first lane of the team
    const int g = tl / L;
    const T *__restrict__ X = static_cast<const T *>(a.x);
    for (int64_t base = first; base < end; base += stride) {
        const int64_t p = base + tl;
        int c = 0;
        uint32_t o = 0;
        float wt = 0.f;
        float sc = 1.f;   // kNorm: the edge's degree factor
        if (p < end) {   // streamed once: non-temporal, so L2 keeps the feature rows
            c = __builtin_nontemporal_load(&a.col[p]);
            o = (uint32_t)__builtin_nontemporal_load(&a.order[p]);
            if ((int64_t)o >= a.e) o = 0u;   // never taken: order is a permutation of [0, e)
            if constexpr (kMode == kDwPair) {
                // an ordinary load: the line stays in L2 for this edge's dw store
                wt = a.w[(int64_t)o * 2];
            } else if constexpr (kMode == kScoreGradInPlace && !kHeads) {
                wt = a.w[o];   // likewise: the score gradient is stored over it
            } else if constexpr (!kHeads) {
                wt = __builtin_nontemporal_load(&a.w[(int64_t)o * a.w_stride]);
            }
            if constexpr (kNorm && score_mode(kMode)) {
                // the score's softmax weight from its destination's statistics (the
                // gathered row here), formed as the softmax apply step does
                const uint32_t cc = (uint64_t)(uint32_t)c < (uint64_t)a.n ? (uint32_t)c : 0u;
                const float2 st = a.norm.stats[cc];
                wt = expf(wt - st.x) / st.y;
            } else if constexpr (kNorm) {
                if (kMode == kPlain && a.norm.mode == kFetchSoftmax) {
                    // the score's softmax weight, formed as the softmax apply step does
                    wt = expf(wt - own_st.x) / own_st.y;
                } else {
                    // mean needs only the destination's degree, the owner's in the
                    // forward; otherwise the gathered endpoint's row length is read
                    const bool mean_own = a.norm.mode == MP_NORM_MEAN && a.norm.own_is_dst;
                    const uint32_t cc =
                        (uint64_t)(uint32_t)c < (uint64_t)a.n ? (uint32_t)c : 0u;
                    const double other = mean_own ? 0.0
                                                  : (double)(a.norm.rowptr_other[cc + 1] -
                                                             a.norm.rowptr_other[cc]);
                    double f;
                    if (a.norm.mode == MP_NORM_MEAN)
                        f = 1.0 / (a.norm.own_is_dst ? own_deg : other);
                    else
                        f = 1.0 / sqrt(own_deg * other);
                    sc = (float)f;
                    wt = wt * sc;
                }
            }
        }
        const int n = end - base < TL ? (int)(end - base) : TL;
        const int trips = (n + G - 1) / G;
        for (int j = 0; j < trips; j += kUnroll) {
            // Column indices first, so the feature-row loads are in flight
            // before the weights (a dependent gather) are waited for.
            int cu[kUnroll], slu[kUnroll];
            bool ok[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int k = g + (j + u) * G;
                ok[u] = (j + u < trips) && k < n;
                slu[u] = tb + (k < n ? k : n - 1);
                cu[u] = __shfl(c, slu[u]);
            }
            uint32_t oh[kUnroll];   // multi-head: the edge's COO ordinal, then its weight
            float wh[kUnroll];
            if constexpr (kHeads) {
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    oh[u] = (uint32_t)__shfl((int)o, slu[u]);
                    wh[u] = ok[u] && active ? a.w[(int64_t)oh[u] * a.heads + head] : 0.f;
                }
            }
            Raw<T, VEC> xv[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                if (ok[u] && active) xv[u].load(X + (int64_t)cu[u] * a.h + hoff);
                else xv[u].zero();
            }
            // Score-gradient mode: the row terms of the gathered rows, loaded with
            // the feature rows so their latency overlaps (a random 4-byte read each).
            float tv[kUnroll];
            if constexpr (score_mode(kMode)) {
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    const int64_t slot = kHeads ? (int64_t)cu[u] * a.heads + head : cu[u];
                    tv[u] = ok[u] && active ? a.row_dot[slot] : 0.f;
                }
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                float wv;
                if constexpr (kHeads) {
                    wv = wh[u];
                } else {
                    const float wu = __shfl(wt, slu[u]);
                    wv = ok[u] ? wu : 0.f;
                }
#pragma unroll
                for (int v = 0; v < VEC; ++v) acc[v] = fmaf(wv, xv[u].at(v), acc[v]);
            }
            if constexpr (kMode != kPlain && !kHeads) {
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    const float part = run_sum(edge_dot<T, VEC>(xr, xv[u]), L);
                    const uint32_t ou = (uint32_t)__shfl((int)o, slu[u]);
                    if constexpr (score_mode(kMode)) {
                        const float wu = __shfl(wt, slu[u]);
                        if (ok[u] && (lane % L) == 0) a.dw[ou] = wu * (part - tv[u]);
                    } else if constexpr (kNorm) {
                        const float su = __shfl(sc, slu[u]);
                        if (ok[u] && (lane % L) == 0) a.dw[ou] = part * su;
                    } else if constexpr (kMode == kDwPair) {
                        if (ok[u] && (lane % L) == 0) a.dw[(int64_t)ou * 2] = part;
                    } else {
                        if (ok[u] && (lane % L) == 0) a.dw[ou] = part;
                    }
                }
            }
            if constexpr (kMode != kPlain && kHeads) {
                const int seg = a.head_w / VEC;    // lanes per head
                const int sub = lane % L;
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    const float part = head_sum(edge_dot<T, VEC>(xr, xv[u]), lane, sub, seg);
                    if (ok[u] && active && sub % seg == 0) {
                        const int64_t slot = (int64_t)oh[u] * a.heads + head;
                        if constexpr (score_mode(kMode))
                            a.dw[slot] = wh[u] * (part - tv[u]);
                        else
                            a.dw[slot] = part;
                    }
                }
            }
        }
    }
}

// The owner row's slice of X (fused backward only).
// Each owner reads its row once, so the load is non-temporal: the row does not
// displace hot gathered rows in L2 (fused backward on the power-law graph 6.580
// against 6.597 ms).  The values are those of Feat.
template <typename T, int VEC, int kMode>
__device__ __forceinline__ void own_row(const SpmmArgs &a, int row, int64_t hoff, bool active,
                                        float (&xr)[VEC]) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) xr[v] = 0.f;
    if constexpr (kMode != kPlain) {
        if (!active) return;
        const T *p = static_cast<const T *>(a.x_own) + (int64_t)row * a.h + hoff;
        if constexpr (sizeof(T) == 2 && VEC == 8) {
            typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
            const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
#pragma unroll
            for (int i = 0; i < 4; ++i) {   // bf16 widened exactly, as Feat does
                xr[2 * i] = __uint_as_float(q[i] << 16);
                xr[2 * i + 1] = __uint_as_float(q[i] & 0xffff0000u);
            }
        } else if constexpr (sizeof(T) == 4 && VEC % 4 == 0) {
#pragma unroll
            for (int i = 0; i < VEC; i += 4) {
                const f32x4 q = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p + i));
                xr[i] = q[0];
                xr[i + 1] = q[1];
                xr[i + 2] = q[2];
                xr[i + 3] = q[3];
            }
        } else {
            Feat<T, VEC>::load(p, xr);
        }
    }
}

// The owner row's softmax statistics (max, sum) when the forward forms softmax
// weights at the fetch; unused otherwise.
template <int kMode, bool kNorm>
__device__ __forceinline__ float2 own_stats(const SpmmArgs &a, int row) {
    if constexpr (kNorm && kMode == kPlain) {
        if (a.norm.mode == kFetchSoftmax) return a.norm.stats[row];
    }
    return make_float2(0.f, 1.f);
}

// Edges [beg, end) of row `row` by the whole workgroup of kWaves waves, the
// waves' partial sums added in wave order and stored to out (the row's slice of
// the output, or a partial row of a split row).  len: the row's full length.
template <typename T, int VEC, int L, int kMode, bool kHeads, bool kNorm, int kWaves>
__device__ __forceinline__ void hub_segment(const SpmmArgs &a, int row, int64_t beg, int64_t end,
                                            int64_t len, float *out,
                                            float (*s_red)[L * VEC]) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int sub = lane % L;
    const int64_t hoff = (int64_t)blockIdx.y * (L * VEC) + (int64_t)sub * VEC;
    const bool active = hoff < a.h;
    const int head = kHeads && active ? (int)(hoff / a.head_w) : 0;
    float acc[VEC], xr[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] = 0.f;
    own_row<T, VEC, kMode>(a, row, hoff, active, xr);
    accumulate<T, VEC, L, kWave, kMode, kHeads, kNorm>(a, beg + (int64_t)wv * kWave, end,
                                                           (int64_t)kWaves * kWave, lane, hoff,
                                                           head, active, xr, acc, (double)len,
                                                           own_stats<kMode, kNorm>(a, row));
#pragma unroll
    for (int off = L; off < kWave; off <<= 1)
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[v] += __shfl_xor(acc[v], off);
    if (lane < L) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) s_red[wv][sub * VEC + v] = acc[v];
    }
    __syncthreads();
    if (wv == 0 && lane < L && active) {
        float r[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            float t = s_red[0][sub * VEC + v];
#pragma unroll
            for (int w2 = 1; w2 < kWaves; ++w2) t += s_red[w2][sub * VEC + v];
            r[v] = t;
        }
        store_row<VEC>(out + hoff, r);
    }
    __syncthreads();   // s_red is written again by the next segment
}

// Hub rows first .. n_hub - 1, every stride-th: each row by the whole workgroup
// of kWaves waves (hub_segment).
template <typename T, int VEC, int L, int kMode, bool kHeads, bool kNorm, int kWaves>
__device__ __forceinline__ void hub_rows(const SpmmArgs &a, int32_t first, int32_t n_hub,
                                         int32_t stride, float (*s_red)[L * VEC]) {
    for (int32_t idx = first; idx < n_hub; idx += stride) {
        const int row = a.plan[idx];
        if ((uint32_t)row >= (uint64_t)a.n) continue;   // the plan is a permutation of [0, n)
        const int64_t beg = a.rowptr[row], end = a.rowptr[row + 1];
        hub_segment<T, VEC, L, kMode, kHeads, kNorm, kWaves>(a, row, beg, end, end - beg,
                                                             a.y + (int64_t)row * a.h, s_red);
    }
}

// Chunk item `item` of the split rows: its class (a short uniform search over
// the split classes), its row and chunk, then the chunk's edges by the whole
// workgroup into its partial row.  Empty slots (rows shorter than their
// class's longest) store nothing.
__device__ __forceinline__ bool chunk_of(const SpmmArgs &a, int32_t item, int &row, int64_t &beg,
                                         int64_t &end, int64_t &len) {
    int c = 0;
    while (c + 1 < a.n_split_cls && item >= a.cls_items[c]) ++c;
    const int32_t item0 = c ? a.cls_items[c - 1] : 0;
    const int32_t pos0 = c ? a.cls_rows[c - 1] : 0;
    const int32_t rel = item - item0;
    const int32_t pos = pos0 + rel / a.cls_slots[c];
    const int64_t k = rel % a.cls_slots[c];
    if (pos >= a.n_split) return false;
    row = a.plan[pos];
    if ((uint32_t)row >= (uint64_t)a.n) return false;
    const int64_t rb = a.rowptr[row], re = a.rowptr[row + 1];
    len = re - rb;
    beg = rb + k * a.chunk_len;
    end = beg + a.chunk_len < re ? beg + a.chunk_len : re;
    return beg < re;
}

template <typename T, int VEC, int L, int kMode, bool kHeads, bool kNorm>
__device__ __forceinline__ void chunk_item(const SpmmArgs &a, int32_t item,
                                           float (*s_red)[L * VEC]) {
    int row;
    int64_t beg, end, len;
    if (!chunk_of(a, item, row, beg, end, len)) return;   // the same for the whole block
    hub_segment<T, VEC, L, kMode, kHeads, kNorm, kWavesPerBlock>(
        a, row, beg, end, len, a.partials + (int64_t)item * a.h, s_red);
}

// Occupancy floors: the single-head fused backward is held to five waves per
// SIMD (8.20 ms against 8.80 ms at four before the rows were held packed; it
// now fits five without spilling), the single-head aggregation to four.  The
// multi-head variants are left to the compiler.
template <int kMode, bool kHeads>
constexpr int min_waves_for() { return kHeads ? 1 : (kMode == kPlain ? 4 : 5); }

template <typename T, int VEC, int L, int kMode, bool kHeads, bool kNorm>
__global__ __launch_bounds__(kBlock)
__attribute__((amdgpu_waves_per_eu(min_waves_for<kMode, kHeads>())))
void spmm_kernel(SpmmArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int sub = lane % L;
    const int64_t hoff = (int64_t)blockIdx.y * (L * VEC) + (int64_t)sub * VEC;
    const bool active = hoff < a.h;
    const int head = kHeads && active ? (int)(hoff / a.head_w) : 0;
    float acc[VEC], xr[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] = 0.f;

    Partition pt{a.n_hub, a.n_wave, a.n_group, a.blk_hub, a.blk_wave, a.blk_group};
    int32_t apart = a.hub_apart;
    int32_t n_full = a.n_full;
    if (a.dev_totals) {   // counts on the device only: the grid is an upper bound
        const ClassLane cr = load_class_lane(a.dev_totals);
        const OwnerRule r = owner_rule(top_class_len(cr), a.e, kWave / L, a.force_hub,
                                       a.force_apart);
        pt = partition<L>(rows_at_least(cr, r.hub_min, a.n), rows_at_least(cr, a.wave_min, a.n),
                          a.n, kAsyncHubBlocks, kAsyncKindBlocks);
        apart = r.apart;
        n_full = (int32_t)rows_at_least(cr, 1, a.n);
    }
    if (apart) pt.blk_hub = 0;
    int64_t b = blockIdx.x;
    __shared__ float s_red[kWavesPerBlock][L * VEC];
    if (b < a.blk_chunk) {
        // ---- chunks of the split rows: partial sums, combined by the next launch
        chunk_item<T, VEC, L, kMode, kHeads, kNorm>(a, (int32_t)b, s_red);
        return;
    }
    b -= a.blk_chunk;
    if (b < pt.blk_hub) {
        // ---- hub rows (after the split ones): the whole workgroup
        hub_rows<T, VEC, L, kMode, kHeads, kNorm, kWavesPerBlock>(a, a.n_split + (int32_t)b,
                                                                  pt.n_hub, pt.blk_hub, s_red);
        return;
    }
    b -= pt.blk_hub;
    if (b < pt.blk_wave) {
        // ---- long rows: one wave each
        for (int64_t idx = b * kWavesPerBlock + wv; idx < pt.n_wave;
             idx += (int64_t)pt.blk_wave * kWavesPerBlock) {
            const int row = a.plan[pt.n_hub + idx];
            if ((uint32_t)row >= (uint64_t)a.n) continue;
            const int64_t beg = a.rowptr[row], end = a.rowptr[row + 1];
#pragma unroll
            for (int v = 0; v < VEC; ++v) acc[v] = 0.f;
            own_row<T, VEC, kMode>(a, row, hoff, active, xr);
            accumulate<T, VEC, L, kWave, kMode, kHeads, kNorm>(a, beg, end, (int64_t)kWave,
                                                                   lane, hoff, head, active, xr,
                                                                   acc, (double)(end - beg),
                                                                   own_stats<kMode, kNorm>(a, row));
#pragma unroll
            for (int off = L; off < kWave; off <<= 1)
#pragma unroll
                for (int v = 0; v < VEC; ++v) acc[v] += __shfl_xor(acc[v], off);
            if (lane < L && active) store_row<VEC>(a.y + (int64_t)row * a.h + hoff, acc);
        }
        return;
    }
    b -= pt.blk_wave;
    if (b >= pt.blk_group) return;   // beyond the work of a device-side partition
    // ---- short or empty rows: one group of L lanes each
    constexpr int64_t kRowsPerBlock = kBlock / L;
    for (int64_t idx = b * kRowsPerBlock + threadIdx.x / L; idx < pt.n_group;
         idx += (int64_t)pt.blk_group * kRowsPerBlock) {
        const int32_t at = pt.n_hub + pt.n_wave + (int32_t)idx;
        const int row = a.plan[at];
        if ((uint32_t)row >= (uint64_t)a.n) continue;
        int64_t beg = 0, end = 0;   // an empty row (at >= n_full) needs no extent read
        if (at < n_full) {
            beg = a.rowptr[row];
            end = a.rowptr[row + 1];
        }
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[v] = 0.f;
        own_row<T, VEC, kMode>(a, row, hoff, active && end > beg, xr);
        accumulate<T, VEC, L, L, kMode, kHeads, kNorm>(a, beg, end, (int64_t)L, lane, hoff,
                                                           head, active, xr, acc,
                                                           (double)(end - beg),
                                                           own_stats<kMode, kNorm>(a, row));
        if (active) store_row<VEC>(a.y + (int64_t)row * a.h + hoff, acc);
    }
}

// Hub rows in a launch of their own, 16 waves per row: a workgroup-owned row is
// bound by the feature rows its waves keep in flight, so four times the waves
// of the main launch take a long row four times as fast when few rows are left
// to overlap it.  Same walk and fixed-order reduction as the hub owners above,
// over 16 waves.

template <typename T, int VEC, int L, int kMode, bool kHeads, bool kNorm>
__global__ __launch_bounds__(kHubBlock) void spmm_hub_kernel(SpmmArgs a) {
    int32_t n_hub = a.n_hub;
    if (a.dev_totals) {
        const ClassLane cr = load_class_lane(a.dev_totals);
        const OwnerRule r = owner_rule(top_class_len(cr), a.e, kWave / L, a.force_hub,
                                       a.force_apart);
        n_hub = r.apart ? (int32_t)rows_at_least(cr, r.hub_min, a.n) : 0;
    }
    __shared__ float s_red[kHubWaves][L * VEC];
    hub_rows<T, VEC, L, kMode, kHeads, kNorm, kHubWaves>(a, (int32_t)blockIdx.x, n_hub,
                                                         (int32_t)gridDim.x, s_red);
}

// Each split row's output: its partial rows added in chunk order (one block per
// split row; plan position = block index).
__global__ __launch_bounds__(kBlock) void split_combine_kernel(SpmmArgs a) {
    const int32_t pos = blockIdx.x;
    int c = 0;
    while (c + 1 < a.n_split_cls && pos >= a.cls_rows[c]) ++c;
    const int32_t item0 = (c ? a.cls_items[c - 1] : 0) +
                          (pos - (c ? a.cls_rows[c - 1] : 0)) * a.cls_slots[c];
    const int row = a.plan[pos];
    if ((uint32_t)row >= (uint64_t)a.n) return;
    const int64_t len = a.rowptr[row + 1] - a.rowptr[row];
    int64_t nk = (len + a.chunk_len - 1) / a.chunk_len;
    if (nk > a.cls_slots[c]) nk = a.cls_slots[c];   // never taken: slots cover the class
    const float *p = a.partials + (int64_t)item0 * a.h;
    for (int64_t col = threadIdx.x; col < a.h; col += blockDim.x) {
        float t = p[col];
        for (int64_t k = 1; k < nk; ++k) t += p[k * a.h + col];
        a.y[(int64_t)row * a.h + col] = t;
    }
}

// ------------------------------------------------------------------ dispatch
// Owner-size overrides set through mp_set_owner_overrides (tests and tuning
// only; none is set unless a caller asks): hub rows from this length, hub rows
// apart (0 or 1), wave rows from this length; -1 leaves the rule's choice.
std::atomic<int32_t> g_force_hub{-1}, g_force_apart{-1}, g_force_wave{-1};

struct Overrides {
    int32_t hub_min, apart, wave_min;
};

Overrides overrides_for(int L) {
    Overrides o;
    const int G = kWave / L;
    o.hub_min = g_force_hub.load(std::memory_order_relaxed);
    o.apart = g_force_apart.load(std::memory_order_relaxed);
    const int32_t wave = g_force_wave.load(std::memory_order_relaxed);
    o.wave_min = wave > 0 ? wave : (G > 1 ? 4 * G : (1 << 30));
    return o;
}

// Rows split across workgroups (the split calls), from the host class counts:
// chunks of at least four shares of the chip's wave slots (512 edges or more),
// rows of two chunks or longer split.  Rows of one class get the slots their
// longest member needs.  items = 0: nothing to split.
struct SplitPlan {
    int32_t n_split = 0, items = 0, chunk_len = 0, n_cls = 0;
    int32_t cls_items[MP_NUM_CLASSES] = {}, cls_rows[MP_NUM_CLASSES] = {},
            cls_slots[MP_NUM_CLASSES] = {};
};

SplitPlan split_plan(const int64_t *cc, int64_t e) {
    SplitPlan p;
    const int64_t share = e / kWaveSlots;
    int64_t chunk = 512;
    while (chunk < 4 * share) chunk *= 2;
    p.chunk_len = (int32_t)chunk;
    int64_t items = 0, rows = 0;
    for (int c = MP_NUM_CLASSES - 1; c >= 1; --c) {
        if (((int64_t)1 << (c - 1)) < 2 * chunk) break;   // lower classes hold shorter rows
        if (cc[c] == 0) continue;
        const int64_t slots = ((((int64_t)1 << c) - 1) + chunk - 1) / chunk;
        items += cc[c] * slots;
        rows += cc[c];
        p.cls_items[p.n_cls] = (int32_t)items;
        p.cls_rows[p.n_cls] = (int32_t)rows;
        p.cls_slots[p.n_cls] = (int32_t)slots;
        ++p.n_cls;
    }
    p.n_split = (int32_t)rows;
    p.items = (int32_t)items;
    return p;
}

// Hub rows first, in their own launch, then every other row.
template <typename T, int VEC, int L, int kMode, bool kHeads, bool kNorm>
void go(const SpmmArgs &a, const dim3 &hub, const dim3 &rest, hipStream_t s) {
    if (hub.x) spmm_hub_kernel<T, VEC, L, kMode, kHeads, kNorm><<<hub, kHubBlock, 0, s>>>(a);
    if (rest.x) spmm_kernel<T, VEC, L, kMode, kHeads, kNorm><<<rest, kBlock, 0, s>>>(a);
}

template <typename T, int VEC, int L>
mp_status launch(const CsrView &csr, const float *w, int64_t heads, const void *x, int64_t h,
                 float *out, const void *x_own, float *dw, const float *row_dot,
                 const NormSpec *norm, bool pair, hipStream_t s, float *split_ws) {
    const bool normed = norm && norm->mode != 0;
    const bool soft = normed && norm->mode == kFetchSoftmax;
    if (normed && (heads != 1 || (row_dot && !soft)))
        return fail(MP_ERR_SHAPE, "fetch-time normalisation takes one head and no row dots");
    if (soft && (!norm->stats || (dw && !row_dot)))
        return fail(MP_ERR_SHAPE, "softmax weights at the fetch need statistics, and with edge "
                                  "outputs the score-gradient form");
    if (pair && (heads != 1 || row_dot || normed))
        return fail(MP_ERR_SHAPE, "the interleaved weight layout takes one head, no row dots and "
                                  "no normalisation");
    const Overrides ov = overrides_for(L);
    const int G = kWave / L;
    SpmmArgs a;
    a.rowptr = csr.rowptr;
    a.col = csr.col;
    a.order = csr.order;
    a.plan = csr.plan;
    a.w = w;
    a.w_stride = pair ? 2 : 1;
    a.x = x;
    a.y = out;
    a.x_own = x_own;
    a.dw = dw;
    a.row_dot = row_dot;
    a.h = h;
    a.heads = (int32_t)heads;
    a.head_w = (int32_t)(h / heads);
    a.n = csr.n;
    a.e = csr.e;
    a.dev_totals = csr.dev_totals;
    a.wave_min = ov.wave_min;
    a.force_hub = ov.hub_min;
    a.force_apart = ov.apart;
    a.norm = normed ? *norm : NormSpec{0, false, nullptr};
    a.partials = nullptr;
    a.n_split = a.blk_chunk = a.chunk_len = a.n_split_cls = 0;
    SplitPlan sp;
    if (split_ws) {
        if (csr.dev_totals || normed || heads != 1 || row_dot || pair)
            return fail(MP_ERR_SHAPE, "split rows need a finished graph, one head and the plain "
                                      "aggregation or fused backward");
        sp = split_plan(csr.class_count, csr.e);
        if (sp.items > 0) {
            a.partials = split_ws;
            a.n_split = sp.n_split;
            a.blk_chunk = sp.items;
            a.chunk_len = sp.chunk_len;
            a.n_split_cls = sp.n_cls;
            for (int c = 0; c < MP_NUM_CLASSES; ++c) {
                a.cls_items[c] = sp.cls_items[c];
                a.cls_rows[c] = sp.cls_rows[c];
                a.cls_slots[c] = sp.cls_slots[c];
            }
        }
    }
    // A launch holds at most 2^32 - 1 work-items; wave and group owners stride.
    Partition pt;
    a.hub_apart = 0;
    int64_t hub_blocks = 0;   // blocks of the 16-wave launch
    if (csr.dev_totals) {
        // Counts live on the device: launch for the largest partition N and E
        // allow (a row of length >= len needs len edges of its own).
        auto most = [&](int64_t len) {
            const int64_t r = csr.e / (len > 0 ? len : 1);
            return r < csr.n ? r : csr.n;
        };
        // The rule is taken in the kernels; bound each launch by the shortest
        // hub length either of its forms may choose.
        const OwnerRule four = owner_rule(0, csr.e, G, ov.hub_min, 0);
        const OwnerRule sixteen = owner_rule(0, csr.e, G, ov.hub_min, 1);
        pt = partition<L>(0, 0, 0);
        const Partition pw = partition<L>(0, most(ov.wave_min), 0, kAsyncHubBlocks,
                                          kAsyncKindBlocks);
        const Partition pg = partition<L>(0, 0, csr.n, kAsyncHubBlocks, kAsyncKindBlocks);
        pt.blk_hub =
            ov.apart == 1 ? 0 : partition<L>(most(four.hub_min), 0, 0, kAsyncHubBlocks).blk_hub;
        pt.blk_wave = pw.blk_wave;
        pt.blk_group = pg.blk_group;
        hub_blocks = ov.apart == 0
                         ? 0
                         : partition<L>(most(sixteen.hub_min), 0, 0, kAsyncHubBlocks16).blk_hub;
    } else if (a.n_split > 0) {
        // Split rows: the longest rows are cut into chunks, so every other hub row
        // takes a four-wave workgroup of the main launch (no 16-wave launch); the
        // split rows lead the hub rows.
        const OwnerRule r = owner_rule(top_class_len_host(csr.class_count), csr.e, G,
                                       ov.hub_min, 0);
        int64_t at_hub = rows_at_least_host(csr.class_count, r.hub_min);
        if (at_hub < a.n_split) at_hub = a.n_split;
        pt = partition<L>(at_hub, rows_at_least_host(csr.class_count, ov.wave_min), csr.n);
        const int64_t rest = pt.n_hub - a.n_split;
        pt.blk_hub = (int32_t)(rest < kMaxKindBlocks ? rest : kMaxKindBlocks);
    } else {
        const OwnerRule r = owner_rule(top_class_len_host(csr.class_count), csr.e, G,
                                       ov.hub_min, ov.apart);
        pt = partition<L>(rows_at_least_host(csr.class_count, r.hub_min),
                          rows_at_least_host(csr.class_count, ov.wave_min), csr.n);
        a.hub_apart = r.apart;
        if (r.apart) {
            hub_blocks = pt.blk_hub;
            pt.blk_hub = 0;   // the main launch skips the hub rows
        }
    }
    a.n_full = csr.dev_totals ? 0 : (int32_t)rows_at_least_host(csr.class_count, 1);
    a.n_hub = pt.n_hub;
    a.n_wave = pt.n_wave;
    a.n_group = pt.n_group;
    a.blk_hub = pt.blk_hub;
    a.blk_wave = pt.blk_wave;
    a.blk_group = pt.blk_group;
    const int64_t hx = hub_blocks;
    const int64_t gx = (int64_t)a.blk_chunk + a.blk_hub + a.blk_wave + a.blk_group;
    const int64_t gy = (h + (int64_t)L * VEC - 1) / ((int64_t)L * VEC);
    if (gx + hx <= 0) return MP_OK;
    if (gx > (int64_t)3 << 22 || hx > (int64_t)3 << 22 || gy > 65535)
        return fail(MP_ERR_SHAPE, "launch grid too large (%lld x %lld)", (long long)gx,
                    (long long)gy);
    const dim3 hub((unsigned)hx, (unsigned)gy), rest((unsigned)gx, (unsigned)gy);
    if (dw) {   // fused backward: one column block holds the whole feature row
        if (gy != 1) return fail(MP_ERR_SHAPE, "fused backward needs H <= %d", L * VEC);
        if (row_dot && dw == w) {   // score gradients written over alpha (or the scores)
            if (heads > 1) go<T, VEC, L, kScoreGradInPlace, true, false>(a, hub, rest, s);
            else if (soft) go<T, VEC, L, kScoreGradInPlace, false, true>(a, hub, rest, s);
            else go<T, VEC, L, kScoreGradInPlace, false, false>(a, hub, rest, s);
        } else if (row_dot) {
            if (heads > 1) go<T, VEC, L, kScoreGrad, true, false>(a, hub, rest, s);
            else if (soft) go<T, VEC, L, kScoreGrad, false, true>(a, hub, rest, s);
            else go<T, VEC, L, kScoreGrad, false, false>(a, hub, rest, s);
        } else if (normed) {
            go<T, VEC, L, kDw, false, true>(a, hub, rest, s);
        } else if (pair) {
            go<T, VEC, L, kDwPair, false, false>(a, hub, rest, s);
        } else {
            if (heads > 1) go<T, VEC, L, kDw, true, false>(a, hub, rest, s);
            else go<T, VEC, L, kDw, false, false>(a, hub, rest, s);
        }
    } else if (normed) {
        go<T, VEC, L, kPlain, false, true>(a, hub, rest, s);
    } else {
        if (heads > 1) go<T, VEC, L, kPlain, true, false>(a, hub, rest, s);
        else go<T, VEC, L, kPlain, false, false>(a, hub, rest, s);
    }
    MP_HIP_CHECK(hipGetLastError(), "spmm launch");
    if (a.n_split > 0) {
        split_combine_kernel<<<(unsigned)a.n_split, kBlock, 0, s>>>(a);
        MP_HIP_CHECK(hipGetLastError(), "split row combine launch");
    }
    return MP_OK;
}

}  // namespace

// Workspace of the split calls: one partial row of h floats per chunk item.
size_t split_workspace_bytes(const int64_t *class_count, int64_t e, int64_t h) {
    return (size_t)split_plan(class_count, e).items * (size_t)h * sizeof(float);
}

namespace {

int lanes_for(int64_t h, int vec) {
    const int64_t need = (h + vec - 1) / vec;
    int L = 1;
    while (L < kWave && L < need) L <<= 1;
    return L;
}

template <typename T, int VEC>
mp_status launch_lanes(const CsrView &csr, const float *w, int64_t heads, const void *x,
                       int64_t h, float *out, const void *x_own, float *dw,
                       const float *row_dot, const NormSpec *nm, bool pair,
                       hipStream_t s, float *sw) {
    switch (lanes_for(h, VEC)) {
        case 1: return launch<T, VEC, 1>(csr, w, heads, x, h, out, x_own, dw, row_dot, nm, pair, s, sw);
        case 2: return launch<T, VEC, 2>(csr, w, heads, x, h, out, x_own, dw, row_dot, nm, pair, s, sw);
        case 4: return launch<T, VEC, 4>(csr, w, heads, x, h, out, x_own, dw, row_dot, nm, pair, s, sw);
        case 8: return launch<T, VEC, 8>(csr, w, heads, x, h, out, x_own, dw, row_dot, nm, pair, s, sw);
        case 16: return launch<T, VEC, 16>(csr, w, heads, x, h, out, x_own, dw, row_dot, nm, pair, s, sw);
        case 32: return launch<T, VEC, 32>(csr, w, heads, x, h, out, x_own, dw, row_dot, nm, pair, s, sw);
        default: return launch<T, VEC, 64>(csr, w, heads, x, h, out, x_own, dw, row_dot, nm, pair, s, sw);
    }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

mp_status spmm_run(const CsrView &csr, const float *w, int64_t heads, const void *x,
                   mp_dtype dt, int64_t h, float *out, hipStream_t s, const NormSpec *norm,
                   bool pair, float *split_ws) {
    return spmm_fused_run(csr, w, heads, x, dt, h, out, nullptr, nullptr, nullptr, s, norm, pair,
                          split_ws);
}

// 16-byte lanes need aligned rows and heads that are whole lanes wide.
bool vector_lanes_ok(int vec, int64_t h, int64_t heads, const void *x, const void *x_own,
                     const void *out) {
    return aligned16(x) && aligned16(out) && (!x_own || aligned16(x_own)) &&
           (h / heads) % vec == 0;
}

bool spmm_fused_supported(mp_dtype dt, int64_t h, int64_t heads, const void *x,
                          const void *x_own, const void *out) {
    const int vec = dt == MP_F32 ? f32_vec(h, heads) : 8;
    return h <= (int64_t)kWave * (vector_lanes_ok(vec, h, heads, x, x_own, out) ? vec : 1);
}

mp_status spmm_fused_run(const CsrView &csr, const float *w, int64_t heads, const void *x,
                         mp_dtype dt, int64_t h, float *out, const void *x_own, float *dw,
                         const float *row_dot, hipStream_t s, const NormSpec *nm,
                         bool pair, float *sw) {
    if (dt == MP_F32) {
        if (f32_vec(h, heads) == 8 && vector_lanes_ok(8, h, heads, x, x_own, out))
            return launch_lanes<float, 8>(csr, w, heads, x, h, out, x_own, dw, row_dot, nm, pair,
                                          s, sw);
        if (vector_lanes_ok(4, h, heads, x, x_own, out))
            return launch_lanes<float, 4>(csr, w, heads, x, h, out, x_own, dw, row_dot, nm, pair,
                                          s, sw);
        return launch_lanes<float, 1>(csr, w, heads, x, h, out, x_own, dw, row_dot, nm, pair, s,
                                      sw);
    }
    if (vector_lanes_ok(8, h, heads, x, x_own, out))
        return launch_lanes<uint16_t, 8>(csr, w, heads, x, h, out, x_own, dw, row_dot, nm, pair,
                                         s, sw);
    return launch_lanes<uint16_t, 1>(csr, w, heads, x, h, out, x_own, dw, row_dot, nm, pair, s,
                                     sw);
}

mp_status set_owner_overrides(int32_t hub_min_len, int32_t hub_apart, int32_t wave_min_len) {
    if (hub_apart > 1)
        return fail(MP_ERR_SHAPE, "hub_apart %d: expected 0, 1 or a negative value", (int)hub_apart);
    g_force_hub.store(hub_min_len > 0 ? hub_min_len : -1, std::memory_order_relaxed);
    g_force_apart.store(hub_apart >= 0 ? hub_apart : -1, std::memory_order_relaxed);
    g_force_wave.store(wave_min_len > 0 ? wave_min_len : -1, std::memory_order_relaxed);
    return MP_OK;
}

}  // namespace mp
