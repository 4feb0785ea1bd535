// common.h -- internal declarations shared by the library's translation units.
// Not part of the public interface (that is include/mp.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "mp.h"

namespace mp {

constexpr int kWave = 64;             // CDNA wavefront width
constexpr int kBlock = 256;           // threads per workgroup for every kernel here
constexpr int kWavesPerBlock = kBlock / kWave;

// Record a failure detail for mp_last_error_detail() and return `s`.
mp_status fail(mp_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

// Map a HIP error to MP_ERR_HIP with `what` in the detail text.
mp_status hip_fail(hipError_t e, const char *what);

#define MP_HIP_CHECK(expr, what)                       \
    do {                                               \
        hipError_t e__ = (expr);                       \
        if (e__ != hipSuccess) return mp::hip_fail(e__, what); \
    } while (0)

// ---------------------------------------------------------------- lowering
// Layout of mp_graph.info (u32 words): the index-range flag, then the digit
// totals of the two plan passes.  A plan key is 32 - class, so the number of
// rows of class c is info[kInfoPlanF + 32 - c] (forward) / [kInfoPlanT + 32 - c].
constexpr int kInfoFlag = 0;
constexpr int kInfoPlanF = 64;
constexpr int kInfoPlanT = 64 + 256;
static_assert(kInfoPlanT + 256 == MP_GRAPH_INFO_WORDS, "info layout");

// Workspace layout for the lowering (byte offsets from the workspace base), per
// direction (forward, transpose).  When the two directions are sorted one after
// the other their sort buffers coincide.
struct LowerLayout {
    size_t k0[2], k1[2];      // [E] u32: ping-pong keys
    size_t v0[2], o0[2];      // [E] u32: one ordinal and one endpoint buffer
    size_t hist[2];           // [256 * tiles] u32 per-tile digit counts (digit-major)
    size_t seg[2];            // [256 * 8] u32 segment totals of the count scan
    size_t bad;               // [tiles] u32 per-tile range words of a small list's intake
    size_t total;
};
// split_dirs: each direction has its own sort buffers (the two directions of
// mp_graph_build_overlap run at once).
LowerLayout lower_layout(int64_t n, int64_t e, bool split_dirs = false);

// Enqueue the whole lowering.  Unless `async`, then synchronise `stream` and
// copy the class counts and the index flag back to the host.  With a `side`
// stream (async only; the workspace laid out with split_dirs): the intake and
// the forward CSR with its plan go on `stream`, the transpose CSR with its plan
// on `side` after the intake, and `side_done` is recorded on `side` at its end.
mp_status lower_run(const void *src, const void *dst, mp_dtype idx_dtype, int64_t n, int64_t e,
                    mp_graph *g, void *ws, hipStream_t stream, bool async, int *bad_index,
                    hipStream_t side = nullptr, hipEvent_t side_done = nullptr);
// Copy the class counts and the index flag of g->info to the host (synchronous).
mp_status lower_read_info(mp_graph *g, hipStream_t stream, int *bad_index);
// This device's static lowering workspace (MP_STATIC_WORKSPACE_BYTES, shared
// by every mp_graph_build_noalloc on the device): its device address, looked up
// on the first call on each device.
mp_status static_workspace(void **ptr, size_t *bytes);

// Rows whose length is >= len, from class counts: classes are sorted high to
// low in the plan, and a class counts only if all its rows qualify (2^(c-1) >= len).
inline int64_t rows_at_least_host(const int64_t *cc, int64_t len) {
    int64_t r = 0;
    for (int c = MP_NUM_CLASSES - 1; c >= 1; --c)
        if (((int64_t)1 << (c - 1)) >= len) r += cc[c];
    return r;
}
// The same from the device record of a plan (digit totals indexed by 32 - class),
// never more than the n rows there are.
__device__ inline int64_t rows_at_least_device(const uint32_t *totals, int64_t len, int64_t n) {
    int64_t r = 0;
    for (int c = MP_NUM_CLASSES - 1; c >= 1; --c)
        if (((int64_t)1 << (c - 1)) >= len) r += totals[32 - c];
    return r < n ? r : n;
}

// Shortest length of the longest nonempty class (0 when every row is empty).
inline int64_t top_class_len_host(const int64_t *cc) {
    for (int c = MP_NUM_CLASSES - 1; c >= 1; --c)
        if (cc[c] > 0) return (int64_t)1 << (c - 1);
    return 0;
}

// The device record's rows per class spread over one wave: lane c holds class c
// (lanes 0 and 33..63 hold zero), so one load per lane and a few cross-lane steps
// answer both queries above.  Every lane of the wave must call these together.
struct ClassLane {
    uint32_t rows;   // rows of class `lane`
    int lane;
};
__device__ inline ClassLane load_class_lane(const uint32_t *totals) {
    ClassLane r;
    r.lane = (int)(threadIdx.x & 63u);
    r.rows = r.lane >= 1 && r.lane < MP_NUM_CLASSES ? totals[32 - r.lane] : 0u;
    return r;
}
__device__ inline int64_t rows_at_least(const ClassLane &cl, int64_t len, int64_t n) {
    uint32_t v = cl.lane >= 1 && ((int64_t)1 << (cl.lane - 1)) >= len ? cl.rows : 0u;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += (uint32_t)__shfl_xor((int)v, off);
    v = (uint32_t)__builtin_amdgcn_readfirstlane((int)v);   // wave-uniform: scalar registers
    return (int64_t)v < n ? (int64_t)v : n;
}
__device__ inline int64_t top_class_len(const ClassLane &cl) {
    const uint64_t m = __ballot(cl.rows > 0u);
    if (m == 0) return 0;
    const int c = __builtin_amdgcn_readfirstlane(63 - __clzll((long long)m));
    return (int64_t)1 << (c - 1);
}

// ---------------------------------------------------------------- lane reductions
// A DPP move: every lane reads `v` from the lane the control word names inside
// its 16-lane row (no LDS traffic, unlike a lane permute).
template <int kCtrl>
__device__ __forceinline__ float dpp_move(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xF, 0xF, false));
}
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- 7 - i within each 8 lanes
constexpr int kDppMirror = 0x140;      // lane i <- 15 - i within each 16 lanes

// Sum of `v` over each aligned run of `width` lanes (a power of two up to 64,
// uniform across the wave), the total in every lane of the run.  Butterfly
// from the smallest distance up: pairs, quads, eights and sixteens are joined
// with DPP moves, 32s and 64s with lane permutes.  After each step every lane
// of a run of that step's size holds the same bits (fp addition commutes), so
// the mirrors join exactly the runs an xor with 4 and 8 would.  Every kernel
// that must return the same edge dot products (the fused backward and the
// edge-gradient kernel) reduces with this one function.
__device__ __forceinline__ float run_sum(float v, int width) {
    if (width >= 2) v += dpp_move<kDppQuadXor1>(v);
    if (width >= 4) v += dpp_move<kDppQuadXor2>(v);
    if (width >= 8) v += dpp_move<kDppHalfMirror>(v);
    if (width >= 16) v += dpp_move<kDppMirror>(v);
    if (width >= 32) v += __shfl_xor(v, 16);
    if (width >= 64) v += __shfl_xor(v, 32);
    return v;
}

// fp32 feature rows of at least kWideF32Cols columns (and heads whose width is
// a multiple of 8) use 32-byte lane slices, 8 floats in two 16-byte loads, so a
// wave carries two rows of 256 features at once instead of one.  The
// aggregation and the edge-gradient kernels take their lane width from this one
// rule, which keeps their edge dot products equal.
constexpr int64_t kWideF32Cols = 256;
inline int f32_vec(int64_t h, int64_t heads) {
    return h >= kWideF32Cols && (h / heads) % 8 == 0 ? 8 : 4;
}

// ---------------------------------------------------------------- SpMM
// One aggregation over a CSR form (rows = owners).  `x` holds [n, h] features
// of dtype `dt`; `out` receives [n, h] float32.
struct CsrView {
    const int32_t *rowptr;
    const int32_t *col;
    const int32_t *order;
    const int32_t *plan;
    const int64_t *class_count;   // host, MP_NUM_CLASSES entries
    const uint32_t *dev_totals;   // device plan record instead (asynchronously built
                                  // graph), else nullptr
    int64_t n;
    int64_t e;
};
// Degree normalisation applied to every weight as it is fetched (mode 0: none).
// The edge's weight becomes w * (float)c, c formed in double as
// 1 / deg_in(dst) (MP_NORM_MEAN) or 1 / sqrt(deg_out(src) * deg_in(dst))
// (MP_NORM_SYM), exactly as the normalisation pass forms it; degrees are row
// lengths of the two CSR forms.  own_is_dst: the walked CSR's rows are
// destinations (forward); rowptr_other: row pointers of the other form, which
// give the gathered endpoint's degree.
// Weight transform at the fetch: MP_NORM_MEAN / MP_NORM_SYM degree factors, or
// kFetchSoftmax (forward only): the weight read is an edge score s and the
// kernel uses exp(s - m) / z of the owner row's softmax statistics (m, z), as
// the softmax's own apply step forms alpha.
constexpr int32_t kFetchSoftmax = 3;
struct NormSpec {
    int32_t mode;
    bool own_is_dst;
    const int32_t *rowptr_other;
    const float2 *stats;   // kFetchSoftmax: row statistics [N] (max, sum)
};

// `heads` = K: w holds K weights per edge ([E, K], edge-major) and head q owns
// columns [q*h/K, (q+1)*h/K) of every row (h is a multiple of K; K = 1 is the
// scalar case).  pair: one head, the weight of edge e at w[2 e] (weights and
// their gradients interleaved).
// split_ws (the split calls): rows long enough are cut into chunks whose
// partial sums go to this workspace (split_workspace_bytes) and are added in
// chunk order by a second launch.
mp_status spmm_run(const CsrView &csr, const float *w, int64_t heads, const void *x,
                   mp_dtype dt, int64_t h, float *out, hipStream_t stream,
                   const NormSpec *norm = nullptr, bool pair = false, float *split_ws = nullptr);
size_t split_workspace_bytes(const int64_t *class_count, int64_t e, int64_t h);
// The same aggregation over the transpose CSR that also writes, for every edge
// q of owner row j, dw[order[q]] = <x_own[j, :], x[col[q], :]> (fused backward;
// per head, dw[order[q] * K + head], when K > 1).  With row_dot (attention
// backward: w = alpha, row_dot [N, K]) it writes the score gradient
// w * (<x_own[j], x[col[q]]> - row_dot[col[q]]) in that slot instead.  With a
// normalisation (one head only) the dot is scaled by the edge's factor c, the
// gradient of the raw weight.  Only for feature rows that fit one column block
// (spmm_fused_supported).
bool spmm_fused_supported(mp_dtype dt, int64_t h, int64_t heads, const void *x,
                          const void *x_own, const void *out);
// Owner-size overrides (mp_set_owner_overrides): values <= 0 (hub_apart < 0)
// restore the rule's choice.
mp_status set_owner_overrides(int32_t hub_min_len, int32_t hub_apart, int32_t wave_min_len);
// pair: w and dw are one interleaved [E][2] array (w at [e][0], dw stored to
// [e][1]; dw points at [0][1]); one head, no row dots, no normalisation.
mp_status spmm_fused_run(const CsrView &csr, const float *w, int64_t heads, const void *x,
                         mp_dtype dt, int64_t h, float *out, const void *x_own, float *dw,
                         const float *row_dot, hipStream_t stream,
                         const NormSpec *norm = nullptr, bool pair = false,
                         float *split_ws = nullptr);

// ---------------------------------------------------------------- SDDMM
// dw[e * K + q] = <x[src_e], dy[dst_e]> over head q's columns, COO order.
mp_status sddmm_run(const int32_t *src, const int32_t *dst, int64_t e, const void *x,
                    const void *dy, mp_dtype dt, int64_t h, int64_t heads, float *dw,
                    hipStream_t stream);

// ---------------------------------------------------------------- target softmax
// `heads` = K score columns per edge ([E, K]); statistics are [N, K].
mp_status edge_softmax_run(const mp_graph *g, const float *s, int64_t heads, float *alpha,
                           float *row_stats, hipStream_t stream);
// The row statistics (max, sum) of the one-head softmax only (no alpha).
mp_status edge_softmax_stats_run(const mp_graph *g, const float *s, float *row_stats,
                                 hipStream_t st);
mp_status edge_softmax_backward_run(const mp_graph *g, const float *alpha, const float *dalpha,
                                    int64_t heads, float *ds, float *row_dot, hipStream_t stream);

// ---------------------------------------------------------------- attention backward
// t[i * K + q] = <y[i], dy[i]> over head q's columns (y fp32 [N, H], dy of dt).
mp_status attention_row_dot_run(const float *y, const void *dy, mp_dtype dt, int64_t n,
                                int64_t h, int64_t heads, float *t, hipStream_t stream);
// ds[e * K + q] = alpha[e * K + q] (ds[e * K + q] - t[dst_e * K + q]) in place.
mp_status score_grad_apply_run(const int32_t *dst, const float *alpha, const float *t,
                               int64_t e, int64_t heads, float *ds, hipStream_t stream);

// ---------------------------------------------------------------- degree normalisation
mp_status edge_normalize_run(const mp_graph *g, int mode, const float *in, float *out,
                             hipStream_t stream);

}  // namespace mp
