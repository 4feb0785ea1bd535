// softmax.hip -- target normalisation of scalar edge scores for sparse
// attention over the fixed topology (tinymesh "Weighted aggregation
// experiment", "Limits": learned scalar scores normalised over the edges of
// each target, then aggregated by this operation):
//   alpha_e = exp(s_e - m_i) / z_i  for i = dst_e, with the row maximum m_i and
//   z_i = sum over the row of exp(s - m_i);
// and its backward  ds_e = alpha_e (dalpha_e - t_i),  t_i = sum over the row of
// alpha * dalpha.
//
// With K heads the scores are [E, K] (edge-major, COO order) and every head is
// normalised on its own; statistics are then [N, K].
//
// Both run in two steps: per-destination row statistics over the forward CSR
// (rows in degree-plan order; a workgroup owns a hub row, a wave a long row, a
// single lane a short row; each owner combines its lanes in a fixed order, no
// atomics), then one elementwise pass over the edges in COO order, which reads
// s / alpha / dalpha coalesced and the per-row statistics by dst.  Both steps
// are priced by their random reads: the row step gathers one value per edge
// through edge_order, the edge step one per edge by dst.  So the forward keeps
// a row's (max, sum) side by side (one 8-byte read per edge), and the backward
// first writes the products alpha * dalpha into its output (one coalesced
// pass) and gathers those, instead of gathering alpha and dalpha separately.
// The row statistics are outputs of the calls.
#include "common.h"

#include <math.h>

namespace mp {
namespace {

constexpr int kHubLen = 4096;   // rows this long get a workgroup
constexpr int kWaveLen = 64;    // rows this long (below kHubLen) get a wave

// Online (max, sum of exp(x - max)) pair.
struct MaxSum {
    float m, z;
};

__device__ __forceinline__ MaxSum ms_add(MaxSum a, float x) {
    if (x > a.m) {   // also the first element: a.m = -inf, a.z = 0
        a.z = (a.m == -INFINITY ? 0.f : a.z * expf(a.m - x)) + 1.f;
        a.m = x;
    } else {
        a.z += expf(x - a.m);
    }
    return a;
}

__device__ __forceinline__ MaxSum ms_merge(MaxSum a, MaxSum b) {
    const float m = fmaxf(a.m, b.m);
    if (m == -INFINITY) return a;   // both empty
    const float za = a.m == -INFINITY ? 0.f : a.z * expf(a.m - m);
    const float zb = b.m == -INFINITY ? 0.f : b.z * expf(b.m - m);
    return MaxSum{m, za + zb};
}

// Wave-wide combine in a fixed butterfly order; every lane ends with the total.
__device__ __forceinline__ MaxSum ms_wave(MaxSum v) {
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) {
        MaxSum o{__shfl_xor(v.m, off), __shfl_xor(v.z, off)};
        v = ms_merge(v, o);
    }
    return v;
}

__device__ __forceinline__ float sum_wave(float v) {
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

struct RowArgs {
    const int32_t *rowptr;
    const int32_t *order;
    const int32_t *plan;
    const float *a;         // scores (forward) or alpha * dalpha (backward), COO order
    float2 *stats;          // forward: (row max, row sum) per row, [N]
    float *dot;             // backward: row sums of alpha * dalpha, [N]
    int64_t n, e;
    int32_t n_hub, n_wave, n_lane;
    int32_t blk_hub, blk_wave, blk_lane;
    const uint32_t *dev_totals;   // asynchronously built graph: rows per class on the
                                  // device, from which the six fields above are derived
    int32_t heads;                // K values per edge ([E, K]) with the multi-head kernels
    bool vec_ok;                  // `a` allows 8- / 16-byte loads of an edge's heads
};

constexpr int64_t kCap = 1 << 22;   // wave and lane owners stride beyond this many blocks

struct RowSplit {
    int32_t n_hub, n_wave, n_lane, blk_hub, blk_wave, blk_lane;
};

__host__ __device__ inline RowSplit row_split(int64_t at_hub, int64_t at_wave, int64_t n) {
    if (at_wave < at_hub) at_wave = at_hub;
    RowSplit r;
    r.n_hub = (int32_t)at_hub;
    r.n_wave = (int32_t)(at_wave - at_hub);
    r.n_lane = (int32_t)(n - at_wave);
    const int64_t bw = (r.n_wave + kWavesPerBlock - 1) / kWavesPerBlock;
    const int64_t bl = (r.n_lane + kBlock - 1) / kBlock;
    r.blk_hub = r.n_hub;
    r.blk_wave = (int32_t)(bw < kCap ? bw : kCap);
    r.blk_lane = (int32_t)(bl < kCap ? bl : kCap);
    return r;
}

__device__ __forceinline__ uint32_t coo(const RowArgs &r, int64_t p) {
    const uint32_t o = (uint32_t)r.order[p];
    return (int64_t)o < r.e ? o : 0u;   // order is a permutation of [0, e)
}

// An edge's KW adjacent values: one 8- or 16-byte load each when `vec` (the
// row base is aligned to it), else one 4-byte load per value.
template <int KW>
__device__ __forceinline__ void load_heads(const float *p, bool vec, float (&v)[KW]) {
    if constexpr (KW % 4 == 0) {
        if (vec) {
#pragma unroll
            for (int j = 0; j < KW; j += 4) {
                const float4 q = *reinterpret_cast<const float4 *>(p + j);
                v[j] = q.x; v[j + 1] = q.y; v[j + 2] = q.z; v[j + 3] = q.w;
            }
            return;
        }
    } else if constexpr (KW == 2) {
        if (vec) {
            const float2 q = *reinterpret_cast<const float2 *>(p);
            v[0] = q.x;
            v[1] = q.y;
            return;
        }
    }
#pragma unroll
    for (int j = 0; j < KW; ++j) v[j] = p[j];
}

// kBackward = false: online max / sum of exp of the scores.
// kBackward = true : sum of the products alpha * dalpha.
// KT heads per edge are reduced in one walk over the row (KT accumulators per
// lane; an edge's KT values are adjacent, so one gathered line serves them
// all).  KT = 0 takes any head count K from the arguments and walks the row
// once per head.  Statistics are [N, K]; KT = 1 is the single-head case.
template <bool kBackward, int KT>
__global__ __launch_bounds__(kBlock) void row_stats_kernel(RowArgs r) {
    constexpr int KW = KT > 0 ? KT : 1;           // heads reduced per walk
    const int K = KT > 0 ? KT : r.heads;
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    RowSplit sp{r.n_hub, r.n_wave, r.n_lane, r.blk_hub, r.blk_wave, r.blk_lane};
    if (r.dev_totals)   // counts on the device only: the grid is an upper bound
        sp = row_split(rows_at_least_device(r.dev_totals, kHubLen, r.n),
                       rows_at_least_device(r.dev_totals, kWaveLen, r.n), r.n);
    int64_t b = blockIdx.x;
    auto finish = [&](int64_t slot, MaxSum ms, float dot) {   // slot = row * K + head
        if (kBackward) r.dot[slot] = dot;
        else r.stats[slot] = make_float2(ms.m, ms.m == -INFINITY ? 0.f : ms.z);
    };
    // Lane-local pass over positions beg, beg + step, ... < end for heads q0 .. q0 + KW - 1.
    auto walk = [&](int64_t beg, int64_t end, int64_t step, int q0, MaxSum (&ms)[KW],
                    float (&dot)[KW]) {
#pragma unroll
        for (int j = 0; j < KW; ++j) {
            ms[j] = MaxSum{-INFINITY, 0.f};
            dot[j] = 0.f;
        }
        // kU edges at a time: their order entries, then their values, are in
        // flight together before the first is combined (the same sequence of
        // updates as one edge at a time, so the same bits).
        constexpr int kU = KW <= 2 ? 8 : 4;
        for (int64_t p0 = beg; p0 < end; p0 += step * kU) {
            uint32_t o[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int64_t p = p0 + u * step;
                o[u] = p < end ? coo(r, p) : 0u;
            }
            float v[kU][KW];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                if (p0 + u * step < end) {
                    load_heads<KW>(r.a + (int64_t)o[u] * K + q0, r.vec_ok, v[u]);
                } else {
#pragma unroll
                    for (int j = 0; j < KW; ++j) v[u][j] = 0.f;
                }
            }
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                if (p0 + u * step < end) {
#pragma unroll
                    for (int j = 0; j < KW; ++j) {
                        if (kBackward) dot[j] += v[u][j];
                        else ms[j] = ms_add(ms[j], v[u][j]);
                    }
                }
            }
        }
    };
    MaxSum ms[KW];
    float dot[KW];
    if (b < sp.blk_hub) {   // hub row: the whole workgroup, lanes strided over the edges
        __shared__ float s_m[kWavesPerBlock][KW], s_z[kWavesPerBlock][KW];
        const int row = r.plan[b];
        if ((uint32_t)row >= (uint64_t)r.n) return;
        const int64_t beg = r.rowptr[row], end = r.rowptr[row + 1];
        for (int q0 = 0; q0 < K; q0 += KW) {
            walk(beg + threadIdx.x, end, kBlock, q0, ms, dot);
#pragma unroll
            for (int j = 0; j < KW; ++j) {
                if (kBackward) dot[j] = sum_wave(dot[j]);
                else ms[j] = ms_wave(ms[j]);
                if (lane == 0) {
                    s_m[wv][j] = kBackward ? dot[j] : ms[j].m;
                    s_z[wv][j] = ms[j].z;
                }
            }
            __syncthreads();
            if (threadIdx.x == 0) {
#pragma unroll
                for (int j = 0; j < KW; ++j) {
                    MaxSum t{s_m[0][j], s_z[0][j]};
                    float d = s_m[0][j];
                    for (int w = 1; w < kWavesPerBlock; ++w) {
                        if (kBackward) d += s_m[w][j];
                        else t = ms_merge(t, MaxSum{s_m[w][j], s_z[w][j]});
                    }
                    finish((int64_t)row * K + q0 + j, t, d);
                }
            }
            if (KT == 0) __syncthreads();   // s_m / s_z are reused by the next head
        }
        return;
    }
    b -= sp.blk_hub;
    if (b < sp.blk_wave) {   // long rows: one wave each
        for (int64_t idx = b * kWavesPerBlock + wv; idx < sp.n_wave;
             idx += (int64_t)sp.blk_wave * kWavesPerBlock) {
            const int row = r.plan[sp.n_hub + idx];
            if ((uint32_t)row >= (uint64_t)r.n) continue;
            const int64_t beg = r.rowptr[row], end = r.rowptr[row + 1];
            for (int q0 = 0; q0 < K; q0 += KW) {
                walk(beg + lane, end, kWave, q0, ms, dot);
#pragma unroll
                for (int j = 0; j < KW; ++j) {
                    if (kBackward) dot[j] = sum_wave(dot[j]);
                    else ms[j] = ms_wave(ms[j]);
                    if (lane == 0) finish((int64_t)row * K + q0 + j, ms[j], dot[j]);
                }
            }
        }
        return;
    }
    b -= sp.blk_wave;
    if (b >= sp.blk_lane) return;   // beyond the work of a device-side split
    // short and empty rows: one lane each
    for (int64_t idx = b * kBlock + threadIdx.x; idx < sp.n_lane;
         idx += (int64_t)sp.blk_lane * kBlock) {
        const int row = r.plan[sp.n_hub + sp.n_wave + idx];
        if ((uint32_t)row >= (uint64_t)r.n) continue;
        const int64_t beg = r.rowptr[row], end = r.rowptr[row + 1];
        for (int q0 = 0; q0 < K; q0 += KW) {
            walk(beg, end, 1, q0, ms, dot);
#pragma unroll
            for (int j = 0; j < KW; ++j) finish((int64_t)row * K + q0 + j, ms[j], dot[j]);
        }
    }
}

// Row statistics launch for `heads` values per edge.
template <bool kBackward>
void launch_row_stats(RowArgs r, int64_t heads, unsigned grid, hipStream_t st) {
    // vector loads need the array base aligned to an edge's KW values
    const uintptr_t base = reinterpret_cast<uintptr_t>(r.a);
    r.vec_ok = (heads == 2 && base % 8 == 0) || ((heads == 4 || heads == 8) && base % 16 == 0);
    switch (heads) {
        case 1: row_stats_kernel<kBackward, 1><<<grid, kBlock, 0, st>>>(r); break;
        case 2: row_stats_kernel<kBackward, 2><<<grid, kBlock, 0, st>>>(r); break;
        case 4: row_stats_kernel<kBackward, 4><<<grid, kBlock, 0, st>>>(r); break;
        case 8: row_stats_kernel<kBackward, 8><<<grid, kBlock, 0, st>>>(r); break;
        default: row_stats_kernel<kBackward, 0><<<grid, kBlock, 0, st>>>(r); break;
    }
}

// Item i of the [E, K] edge values: edge i / K, head i % K.
template <bool kHeads>
__device__ __forceinline__ int64_t stat_slot(const int32_t *dst, int64_t i, int k) {
    if (!kHeads) return dst[i];
    // 32-bit division while the item index fits (E * K < 2^32, the usual case)
    const int64_t e = i < ((int64_t)1 << 32) ? (int64_t)((uint32_t)i / (uint32_t)k) : i / k;
    return (int64_t)dst[e] * k + (i - e * k);
}

// Items per thread in flight in the edge passes: each item's statistics are a
// gather that depends on its dst, so several chains run side by side.
constexpr int kApplyU = 4;

// alpha_e = exp(s_e - m[dst_e]) / z[dst_e]   (per head with kHeads)
template <bool kHeads>
__global__ __launch_bounds__(kBlock) void softmax_apply_kernel(const int32_t *__restrict__ dst,
                                                               const float *__restrict__ s,
                                                               const float2 *__restrict__ stats,
                                                               float *__restrict__ alpha,
                                                               int64_t items, int k) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i0 = (int64_t)blockIdx.x * kBlock + threadIdx.x; i0 < items;
         i0 += stride * kApplyU) {
        float2 st[kApplyU];
        float sv[kApplyU];
#pragma unroll
        for (int u = 0; u < kApplyU; ++u) {
            const int64_t i = i0 + u * stride;
            st[u] = i < items ? stats[stat_slot<kHeads>(dst, i, k)] : make_float2(0.f, 1.f);
            sv[u] = i < items ? s[i] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kApplyU; ++u) {
            const int64_t i = i0 + u * stride;
            if (i < items) alpha[i] = expf(sv[u] - st[u].x) / st[u].y;
        }
    }
}

// p_e = alpha_e * dalpha_e (into the output array, read back by the row step)
__global__ __launch_bounds__(kBlock) void edge_product_kernel(const float *__restrict__ alpha,
                                                              const float *__restrict__ dalpha,
                                                              float *__restrict__ p, int64_t e) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < e; i += stride)
        p[i] = alpha[i] * dalpha[i];
}

// ds_e = alpha_e (dalpha_e - t[dst_e])   (per head with kHeads)
template <bool kHeads>
__global__ __launch_bounds__(kBlock) void softmax_backward_apply_kernel(
    const int32_t *__restrict__ dst, const float *__restrict__ alpha,
    const float *__restrict__ dalpha, const float *__restrict__ rdot, float *__restrict__ ds,
    int64_t items, int k) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i0 = (int64_t)blockIdx.x * kBlock + threadIdx.x; i0 < items;
         i0 += stride * kApplyU) {
        float t[kApplyU], av[kApplyU], dv[kApplyU];
#pragma unroll
        for (int u = 0; u < kApplyU; ++u) {
            const int64_t i = i0 + u * stride;
            t[u] = i < items ? rdot[stat_slot<kHeads>(dst, i, k)] : 0.f;
            av[u] = i < items ? alpha[i] : 0.f;
            dv[u] = i < items ? dalpha[i] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kApplyU; ++u) {
            const int64_t i = i0 + u * stride;
            if (i < items) ds[i] = av[u] * (dv[u] - t[u]);
        }
    }
}

RowArgs row_args(const mp_graph *g) {
    RowArgs r;
    r.rowptr = g->rowptr;
    r.order = g->edge_order;
    r.plan = g->row_plan;
    r.n = g->num_nodes;
    r.e = g->num_edges;
    RowSplit sp;
    if (g->built == MP_GRAPH_ON_DEVICE) {
        // Launch for the largest split N and E allow; the kernel derives the real one.
        r.dev_totals = g->info + kInfoPlanF;
        auto most = [&](int64_t len) { return r.e / len < r.n ? r.e / len : r.n; };
        sp.blk_hub = row_split(most(kHubLen), most(kHubLen), most(kHubLen)).blk_hub;
        sp.blk_wave = row_split(0, most(kWaveLen), most(kWaveLen)).blk_wave;
        sp.blk_lane = row_split(0, 0, r.n).blk_lane;
        sp.n_hub = sp.n_wave = sp.n_lane = 0;
    } else {
        r.dev_totals = nullptr;
        sp = row_split(rows_at_least_host(g->class_count, kHubLen),
                       rows_at_least_host(g->class_count, kWaveLen), r.n);
    }
    r.n_hub = sp.n_hub;
    r.n_wave = sp.n_wave;
    r.n_lane = sp.n_lane;
    r.blk_hub = sp.blk_hub;
    r.blk_wave = sp.blk_wave;
    r.blk_lane = sp.blk_lane;
    return r;
}

unsigned grid_for(int64_t items) {
    int64_t b = (items + kBlock - 1) / kBlock;
    if (b < 1) b = 1;
    return (unsigned)(b < 65536 ? b : 65536);
}

}  // namespace

mp_status edge_softmax_run(const mp_graph *g, const float *s, int64_t heads, float *alpha,
                           float *row_stats, hipStream_t st) {
    RowArgs r = row_args(g);
    r.a = s;
    r.stats = reinterpret_cast<float2 *>(row_stats);
    r.dot = nullptr;
    r.heads = (int32_t)heads;
    const int64_t gx = (int64_t)r.blk_hub + r.blk_wave + r.blk_lane;
    const int64_t items = g->num_edges * heads;
    const float2 *stats = reinterpret_cast<const float2 *>(row_stats);
    launch_row_stats<false>(r, heads, (unsigned)gx, st);
    if (heads > 1) {
        if (items > 0)
            softmax_apply_kernel<true><<<grid_for(items), kBlock, 0, st>>>(
                g->dst, s, stats, alpha, items, (int)heads);
    } else {
        if (items > 0)
            softmax_apply_kernel<false><<<grid_for(items), kBlock, 0, st>>>(g->dst, s, stats,
                                                                            alpha, items, 1);
    }
    MP_HIP_CHECK(hipGetLastError(), "edge softmax launch");
    return MP_OK;
}

mp_status edge_softmax_stats_run(const mp_graph *g, const float *s, float *row_stats,
                                 hipStream_t st) {
    RowArgs r = row_args(g);
    r.a = s;
    r.stats = reinterpret_cast<float2 *>(row_stats);
    r.dot = nullptr;
    r.heads = 1;
    const int64_t gx = (int64_t)r.blk_hub + r.blk_wave + r.blk_lane;
    launch_row_stats<false>(r, 1, (unsigned)gx, st);
    MP_HIP_CHECK(hipGetLastError(), "edge softmax statistics launch");
    return MP_OK;
}

mp_status edge_softmax_backward_run(const mp_graph *g, const float *alpha, const float *dalpha,
                                    int64_t heads, float *ds, float *rdot, hipStream_t st) {
    RowArgs r = row_args(g);
    r.a = ds;                // holds alpha * dalpha until the last step overwrites it
    r.stats = nullptr;
    r.dot = rdot;
    r.heads = (int32_t)heads;
    const int64_t gx = (int64_t)r.blk_hub + r.blk_wave + r.blk_lane;
    const int64_t items = g->num_edges * heads;
    if (items > 0)
        edge_product_kernel<<<grid_for(items), kBlock, 0, st>>>(alpha, dalpha, ds, items);
    launch_row_stats<true>(r, heads, (unsigned)gx, st);
    if (heads > 1) {
        if (items > 0)
            softmax_backward_apply_kernel<true><<<grid_for(items), kBlock, 0, st>>>(
                g->dst, alpha, dalpha, rdot, ds, items, (int)heads);
    } else {
        if (items > 0)
            softmax_backward_apply_kernel<false><<<grid_for(items), kBlock, 0, st>>>(
                g->dst, alpha, dalpha, rdot, ds, items, 1);
    }
    MP_HIP_CHECK(hipGetLastError(), "edge softmax backward launch");
    return MP_OK;
}

}  // namespace mp
