// api.hip -- the extern "C" entry points declared in include/mp.h: argument
// validation on the host, then the launches in lower.hip, spmm.hip, sddmm.hip.
#include <stdarg.h>
#include <stdlib.h>
#include <stdio.h>
#include <string.h>

#include "common.h"

namespace mp {

namespace {
thread_local char g_detail[512] = "";
constexpr int64_t kMaxIndex = (int64_t)1 << 31;           // N, E < 2^31
}  // namespace

mp_status fail(mp_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
    va_end(ap);
    return s;
}

mp_status hip_fail(hipError_t e, const char *what) {
    return fail(MP_ERR_HIP, "%s: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
}

namespace {

size_t dtype_size(mp_dtype t) {
    switch (t) {
        case MP_I32: return 4;
        case MP_I64: return 8;
        case MP_F32: return 4;
        case MP_BF16: return 2;
        default: return 0;
    }
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Device memory of the current device?  (Checked only for non-empty arrays.)
mp_status check_device(const void *p, const char *name) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    hipPointerAttribute_t attr;
    memset(&attr, 0, sizeof(attr));
    e = hipPointerGetAttributes(&attr, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();   // clear the sticky error of the failed query
        return fail(MP_ERR_DEVICE, "%s is not memory known to the HIP runtime", name);
    }
    if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
        return fail(MP_ERR_DEVICE, "%s is not device memory (memory type %d)", name,
                    (int)attr.type);
    if (attr.device != dev)
        return fail(MP_ERR_DEVICE, "%s lives on device %d, current device is %d", name,
                    attr.device, dev);
    return MP_OK;
}

struct Range {
    uintptr_t lo, hi;   // [lo, hi)
    const char *name;
};

Range range(const void *p, int64_t count, size_t elem, const char *name) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, lo + (uintptr_t)count * elem, name};
}

bool overlap(const Range &a, const Range &b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

// A short list of address ranges with a fixed capacity.  A range added beyond
// the capacity is refused and remembered: every check against the list then
// returns MP_ERR_INTERNAL instead of passing on an incomplete list (the largest
// list any entry point builds holds 18 ranges).
#ifndef MP_RANGE_LIST_CAP
#define MP_RANGE_LIST_CAP 24
#endif
struct RangeList {
    static constexpr int kCap = MP_RANGE_LIST_CAP;
    Range r[kCap];
    int k = 0;
    bool refused = false;
    void add(const Range &x) {
        if (k < kCap) r[k++] = x;
        else refused = true;
    }
    // Name of the first range that overlaps `x`, or nullptr.
    const char *overlapping(const Range &x) const {
        for (int i = 0; i < k; ++i)
            if (overlap(x, r[i])) return r[i].name;
        return nullptr;
    }
};

mp_status list_overflow() {
    return fail(MP_ERR_INTERNAL, "internal: more address ranges than the overlap check holds (%d)",
                RangeList::kCap);
}

// MP_OK when `x` overlaps no range of `list`, else MP_ERR_ALIAS naming the
// first one it overlaps (`prefix` opens the detail text).
mp_status apart(const RangeList &list, const Range &x, const char *prefix = "") {
    if (list.refused) return list_overflow();
    if (const char *hit = list.overlapping(x))
        return fail(MP_ERR_ALIAS, "%s%s overlaps %s", prefix, x.name, hit);
    return MP_OK;
}

// Ranges of every array a graph descriptor points to.
RangeList graph_ranges(const mp_graph *g) {
    const int64_t n = g->num_nodes, e = g->num_edges;
    RangeList out;
    out.add(range(g->src, e, 4, "graph src"));
    out.add(range(g->dst, e, 4, "graph dst"));
    out.add(range(g->rowptr, n + 1, 4, "graph rowptr"));
    out.add(range(g->col, e, 4, "graph col"));
    out.add(range(g->edge_order, e, 4, "graph edge_order"));
    out.add(range(g->rowptr_t, n + 1, 4, "graph rowptr_t"));
    out.add(range(g->col_t, e, 4, "graph col_t"));
    out.add(range(g->transpose_order, e, 4, "graph transpose_order"));
    out.add(range(g->row_plan, n, 4, "graph row_plan"));
    out.add(range(g->row_plan_t, n, 4, "graph row_plan_t"));
    out.add(range(g->info, MP_GRAPH_INFO_WORDS, 4, "graph info"));
    return out;
}

mp_status check_graph(const mp_graph *g) {
    if (!g) return fail(MP_ERR_NULL, "graph is NULL");
    if (g->built != MP_GRAPH_BUILT && g->built != MP_GRAPH_ON_DEVICE)
        return fail(MP_ERR_GRAPH, "graph was not produced by a successful mp_graph_build");
    return MP_OK;
}

// The two CSR forms of a built graph; an asynchronously built graph hands the
// kernels its device plan record instead of host counts.
CsrView forward_view(const mp_graph *g) {
    const bool dev = g->built == MP_GRAPH_ON_DEVICE;
    return CsrView{g->rowptr, g->col, g->edge_order, g->row_plan, g->class_count,
                   dev ? g->info + kInfoPlanF : nullptr, g->num_nodes, g->num_edges};
}

CsrView transpose_view(const mp_graph *g) {
    const bool dev = g->built == MP_GRAPH_ON_DEVICE;
    return CsrView{g->rowptr_t, g->col_t, g->transpose_order, g->row_plan_t, g->class_count_t,
                   dev ? g->info + kInfoPlanT : nullptr, g->num_nodes, g->num_edges};
}

mp_status check_sizes(int64_t n, int64_t e) {
    if (n < 1 || n >= kMaxIndex) return fail(MP_ERR_SHAPE, "num_nodes %lld outside [1, 2^31)", (long long)n);
    if (e < 0 || e >= kMaxIndex) return fail(MP_ERR_SHAPE, "num_edges %lld outside [0, 2^31)", (long long)e);
    return MP_OK;
}

mp_status check_h(int64_t n, int64_t h) {
    if (h < 1 || h >= kMaxIndex) return fail(MP_ERR_SHAPE, "feature width %lld outside [1, 2^31)", (long long)h);
    if (n > ((int64_t)1 << 62) / h) return fail(MP_ERR_SHAPE, "N*H overflows");
    return MP_OK;
}

// Head count: 1 <= heads <= h, heads divides h.
mp_status check_heads(int64_t h, int64_t heads) {
    if (heads < 1 || heads > h || h % heads != 0)
        return fail(MP_ERR_SHAPE, "head count %lld does not divide the feature width %lld",
                    (long long)heads, (long long)h);
    return MP_OK;
}

// Shared validation of one aggregation call (forward or input gradient); w
// holds `heads` weights per edge, in w_span floats per edge (0: heads).
mp_status check_spmm(const mp_graph *g, const float *w, int64_t heads, const void *x,
                     mp_dtype dt, int64_t h, float *y, const char *xname, const char *yname,
                     int64_t w_span = 0) {
    mp_status st = check_graph(g);
    if (st != MP_OK) return st;
    const int64_t n = g->num_nodes, e = g->num_edges;
    if (!x) return fail(MP_ERR_NULL, "%s is NULL", xname);
    if (!y) return fail(MP_ERR_NULL, "%s is NULL", yname);
    if (!w && e > 0) return fail(MP_ERR_NULL, "w is NULL with %lld edges", (long long)e);
    if ((st = check_h(n, h)) != MP_OK) return st;
    if ((st = check_heads(h, heads)) != MP_OK) return st;
    if (dt != MP_F32 && dt != MP_BF16)
        return fail(MP_ERR_DTYPE, "%s dtype code %d: expected MP_F32 or MP_BF16", xname, (int)dt);
    const size_t xs = dtype_size(dt);
    if (!aligned(x, xs)) return fail(MP_ERR_ALIGN, "%s not aligned to %zu bytes", xname, xs);
    if (!aligned(y, 4)) return fail(MP_ERR_ALIGN, "%s not aligned to 4 bytes", yname);
    if (w && !aligned(w, 4)) return fail(MP_ERR_ALIGN, "w not aligned to 4 bytes");
    if ((st = check_device(x, xname)) != MP_OK) return st;
    if ((st = check_device(y, yname)) != MP_OK) return st;
    if (e > 0 && (st = check_device(w, "w")) != MP_OK) return st;
    const Range ry = range(y, n * h, 4, yname);
    RangeList others = graph_ranges(g);
    others.add(range(x, n * h, xs, xname));
    others.add(range(w, e * (w_span > 0 ? w_span : heads), 4, "w"));
    return apart(others, ry);
}

mp_status spmm_fwd_impl(const mp_graph *g, const float *w, int64_t heads, const void *x,
                        mp_dtype x_dtype, int64_t h, float *y, void *stream,
                        bool pair = false) {
    // with interleaved weights and gradients the weight array spans 2E floats
    mp_status st = check_spmm(g, w, heads, x, x_dtype, h, y, "x", "y", pair ? 2 : 0);
    if (st != MP_OK) return st;
    return spmm_run(forward_view(g), w, heads, x, x_dtype, h, y,
                    static_cast<hipStream_t>(stream), nullptr, pair);
}

mp_status spmm_dx_impl(const mp_graph *g, const float *w, int64_t heads, const void *dy,
                       mp_dtype dy_dtype, int64_t h, float *dx, void *stream) {
    mp_status st = check_spmm(g, w, heads, dy, dy_dtype, h, dx, "dy", "dx");
    if (st != MP_OK) return st;
    return spmm_run(transpose_view(g), w, heads, dy, dy_dtype, h, dx,
                    static_cast<hipStream_t>(stream));
}

mp_status edge_grad_impl(const mp_graph *g, const void *x, const void *dy, mp_dtype dtype,
                         int64_t h, int64_t heads, float *dw, void *stream) {
    mp_status st = check_graph(g);
    if (st != MP_OK) return st;
    const int64_t n = g->num_nodes, e = g->num_edges;
    if (!x || !dy) return fail(MP_ERR_NULL, "x or dy is NULL");
    if (!dw && e > 0) return fail(MP_ERR_NULL, "dw is NULL with %lld edges", (long long)e);
    if ((st = check_h(n, h)) != MP_OK) return st;
    if ((st = check_heads(h, heads)) != MP_OK) return st;
    if (dtype != MP_F32 && dtype != MP_BF16)
        return fail(MP_ERR_DTYPE, "feature dtype code %d: expected MP_F32 or MP_BF16", (int)dtype);
    const size_t xs = dtype_size(dtype);
    if (!aligned(x, xs) || !aligned(dy, xs))
        return fail(MP_ERR_ALIGN, "x/dy not aligned to %zu bytes", xs);
    if (dw && !aligned(dw, 4)) return fail(MP_ERR_ALIGN, "dw not aligned to 4 bytes");
    if ((st = check_device(x, "x")) != MP_OK) return st;
    if ((st = check_device(dy, "dy")) != MP_OK) return st;
    if (e == 0) return MP_OK;
    if ((st = check_device(dw, "dw")) != MP_OK) return st;
    const Range rdw = range(dw, e * heads, 4, "dw");
    RangeList others = graph_ranges(g);
    others.add(range(x, n * h, xs, "x"));
    others.add(range(dy, n * h, xs, "dy"));
    if ((st = apart(others, rdw)) != MP_OK) return st;
    return sddmm_run(g->src, g->dst, e, x, dy, dtype, h, heads, dw,
                     static_cast<hipStream_t>(stream));
}

// Fetch-time normalisation of a walk over the forward (rows = destinations) or
// the transpose CSR.
NormSpec norm_spec(const mp_graph *g, int32_t mode, bool forward) {
    return NormSpec{mode, forward, forward ? g->rowptr_t : g->rowptr};
}

mp_status check_norm_mode(int32_t mode, const char *what) {
    if (mode != MP_NORM_MEAN && mode != MP_NORM_SYM)
        return fail(MP_ERR_DTYPE, "%s: unknown normalisation mode %d", what, (int)mode);
    return MP_OK;
}

// The split calls' workspace for one CSR form: `need` bytes (0 when no row of
// it is long enough to split), device memory aligned to 256 bytes, overlapping
// none of `others` (the graph arrays and the call's inputs and outputs).
mp_status check_split(const mp_graph *g, const CsrView &v, int64_t h, void *ws, size_t ws_bytes,
                      RangeList others, size_t *need) {
    if (g->built != MP_GRAPH_BUILT)
        return fail(MP_ERR_GRAPH, "the split calls need a finished graph (mp_graph_build, or "
                                  "mp_graph_finish after an asynchronous build)");
    *need = split_workspace_bytes(v.class_count, v.e, h);
    if (*need == 0) return MP_OK;
    if (!ws) return fail(MP_ERR_WORKSPACE, "split workspace is NULL (%zu bytes needed)", *need);
    if (ws_bytes < *need)
        return fail(MP_ERR_WORKSPACE, "split workspace has %zu bytes, %zu needed", ws_bytes, *need);
    if (!aligned(ws, 256)) return fail(MP_ERR_ALIGN, "split workspace not aligned to 256 bytes");
    mp_status st = check_device(ws, "split workspace");
    if (st != MP_OK) return st;
    const uintptr_t lo = reinterpret_cast<uintptr_t>(ws);
    return apart(others, Range{lo, lo + *need, "split workspace"});
}

mp_status dx_edge_grad_impl(const mp_graph *g, const float *w, int64_t heads, const void *x,
                            const void *dy, mp_dtype dtype, int64_t h, float *dx, float *dw,
                            void *stream, int32_t norm_mode = 0, bool split = false,
                            void *split_ws = nullptr, size_t split_bytes = 0) {
    mp_status st = check_spmm(g, w, heads, dy, dtype, h, dx, "dy", "dx");
    if (st != MP_OK) return st;
    const int64_t n = g->num_nodes, e = g->num_edges;
    if (!x) return fail(MP_ERR_NULL, "x is NULL");
    if (!dw && e > 0) return fail(MP_ERR_NULL, "dw is NULL with %lld edges", (long long)e);
    const size_t xs = dtype_size(dtype);
    if (!aligned(x, xs)) return fail(MP_ERR_ALIGN, "x not aligned to %zu bytes", xs);
    if (dw && !aligned(dw, 4)) return fail(MP_ERR_ALIGN, "dw not aligned to 4 bytes");
    if ((st = check_device(x, "x")) != MP_OK) return st;
    if (e > 0 && (st = check_device(dw, "dw")) != MP_OK) return st;
    const Range rdx = range(dx, n * h, 4, "dx"), rdw = range(dw, e * heads, 4, "dw");
    const Range rx = range(x, n * h, xs, "x");
    if (overlap(rdx, rx)) return fail(MP_ERR_ALIAS, "dx overlaps x");
    RangeList others = graph_ranges(g);
    others.add(rx);
    others.add(range(dy, n * h, xs, "dy"));
    others.add(range(w, e * heads, 4, "w"));
    others.add(rdx);
    if ((st = apart(others, rdw)) != MP_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const CsrView v = transpose_view(g);
    const NormSpec nm = norm_spec(g, norm_mode, false);
    const NormSpec *pn = norm_mode ? &nm : nullptr;
    float *sw = nullptr;
    if (split) {
        others.add(rdw);
        size_t need = 0;
        if ((st = check_split(g, v, h, split_ws, split_bytes, others, &need)) != MP_OK) return st;
        if (need) sw = static_cast<float *>(split_ws);
    }
    if (spmm_fused_supported(dtype, h, heads, dy, x, dx))
        return spmm_fused_run(v, w, heads, dy, dtype, h, dx, x, e > 0 ? dw : nullptr,
                              nullptr, s, pn, false, sw);
    // Feature rows wider than one column block: the two kernels back to back
    // (and the edge gradients scaled by their factors in place).
    if ((st = spmm_run(v, w, heads, dy, dtype, h, dx, s, pn, false, sw)) != MP_OK) return st;
    if (e == 0) return MP_OK;
    if ((st = sddmm_run(g->src, g->dst, e, x, dy, dtype, h, heads, dw, s)) != MP_OK) return st;
    return norm_mode ? edge_normalize_run(g, norm_mode, dw, dw, s) : MP_OK;
}

}  // namespace
}  // namespace mp

using namespace mp;

extern "C" {

mp_status mp_graph_build_workspace_size(int64_t num_nodes, int64_t num_edges, size_t *bytes) {
    if (!bytes) return fail(MP_ERR_NULL, "bytes is NULL");
    mp_status st = check_sizes(num_nodes, num_edges);
    if (st != MP_OK) return st;
    *bytes = lower_layout(num_nodes, num_edges).total;
    return MP_OK;
}

mp_status mp_graph_build_overlap_workspace_size(int64_t num_nodes, int64_t num_edges,
                                                size_t *bytes) {
    if (!bytes) return fail(MP_ERR_NULL, "bytes is NULL");
    mp_status st = check_sizes(num_nodes, num_edges);
    if (st != MP_OK) return st;
    *bytes = lower_layout(num_nodes, num_edges, true).total;
    return MP_OK;
}

}  // extern "C"

namespace mp {
namespace {
// static_ws: the workspace is this device's static array (mp_graph_build_noalloc).
// side / side_done: mp_graph_build_overlap (the transpose direction on `side`).
mp_status build_impl(const void *src, const void *dst, mp_dtype idx_dtype, int64_t num_nodes,
                     int64_t num_edges, mp_graph *g, void *workspace, size_t workspace_bytes,
                     void *stream, bool async, bool static_ws = false, void *side = nullptr,
                     void *side_done = nullptr) {
    if (!g) return fail(MP_ERR_NULL, "graph descriptor is NULL");
    g->built = 0;
    mp_status st = check_sizes(num_nodes, num_edges);
    if (st != MP_OK) return st;
    const int64_t n = num_nodes, e = num_edges;
    if (idx_dtype != MP_I32 && idx_dtype != MP_I64)
        return fail(MP_ERR_DTYPE, "index dtype code %d: expected MP_I32 or MP_I64", (int)idx_dtype);
    if (e > 0 && (!src || !dst)) return fail(MP_ERR_NULL, "src or dst is NULL with %lld edges", (long long)e);
    struct {
        const void *p;
        const char *name;
        int64_t count;
    } arrays[] = {
        {g->src, "graph src", e},       {g->dst, "graph dst", e},
        {g->rowptr, "graph rowptr", n + 1}, {g->col, "graph col", e},
        {g->edge_order, "graph edge_order", e}, {g->rowptr_t, "graph rowptr_t", n + 1},
        {g->col_t, "graph col_t", e},   {g->transpose_order, "graph transpose_order", e},
        {g->row_plan, "graph row_plan", n}, {g->row_plan_t, "graph row_plan_t", n},
        {g->info, "graph info", MP_GRAPH_INFO_WORDS},
    };
    for (const auto &a : arrays) {
        if (a.count > 0 && !a.p) return fail(MP_ERR_NULL, "%s is NULL", a.name);
        if (a.p && !aligned(a.p, 4)) return fail(MP_ERR_ALIGN, "%s not aligned to 4 bytes", a.name);
    }
    const size_t need = lower_layout(n, e, side != nullptr).total;
    if (static_ws && need > workspace_bytes)
        return fail(MP_ERR_WORKSPACE,
                    "N = %lld, E = %lld need %zu bytes of workspace; the static workspace of "
                    "mp_graph_build_noalloc holds %zu", (long long)n, (long long)e, need,
                    workspace_bytes);
    if (!workspace) return fail(MP_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (workspace_bytes < need)
        return fail(MP_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
    if (!aligned(workspace, 256)) return fail(MP_ERR_ALIGN, "workspace not aligned to 256 bytes");
    const size_t is = dtype_size(idx_dtype);
    if (e > 0) {
        if (!aligned(src, is) || !aligned(dst, is))
            return fail(MP_ERR_ALIGN, "src/dst not aligned to %zu bytes", is);
        if ((st = check_device(src, "src")) != MP_OK) return st;
        if ((st = check_device(dst, "dst")) != MP_OK) return st;
    }
    for (const auto &a : arrays)
        if (a.count > 0 && (st = check_device(a.p, a.name)) != MP_OK) return st;
    if (!static_ws && (st = check_device(workspace, "workspace")) != MP_OK) return st;

    // Outputs (graph arrays, workspace) must not overlap each other or the inputs.
    g->num_nodes = n;
    g->num_edges = e;
    RangeList r = graph_ranges(g);
    r.add(Range{reinterpret_cast<uintptr_t>(workspace),
                reinterpret_cast<uintptr_t>(workspace) + need, "workspace"});
    const Range in_s = range(src, e, is, "src"), in_d = range(dst, e, is, "dst");
    if (r.refused) return list_overflow();
    for (int i = 0; i < r.k; ++i) {
        if (overlap(r.r[i], in_s) || overlap(r.r[i], in_d))
            return fail(MP_ERR_ALIAS, "%s overlaps the input edge list", r.r[i].name);
        for (int j = i + 1; j < r.k; ++j)
            if (overlap(r.r[i], r.r[j]))
                return fail(MP_ERR_ALIAS, "%s overlaps %s", r.r[i].name, r.r[j].name);
    }

    int bad = 0;
    st = lower_run(src, dst, idx_dtype, n, e, g, workspace, static_cast<hipStream_t>(stream),
                   async, &bad, static_cast<hipStream_t>(side),
                   static_cast<hipEvent_t>(side_done));
    if (st != MP_OK) return st;
    if (bad) return fail(MP_ERR_INDEX, "an edge endpoint lies outside [0, %lld)", (long long)n);
    g->built = async ? MP_GRAPH_ON_DEVICE : MP_GRAPH_BUILT;
    return MP_OK;
}
}  // namespace
}  // namespace mp

extern "C" {

mp_status mp_graph_build(const void *src, const void *dst, mp_dtype idx_dtype, int64_t num_nodes,
                         int64_t num_edges, mp_graph *g, void *workspace, size_t workspace_bytes,
                         void *stream) {
    return build_impl(src, dst, idx_dtype, num_nodes, num_edges, g, workspace, workspace_bytes,
                      stream, false);
}

mp_status mp_graph_build_async(const void *src, const void *dst, mp_dtype idx_dtype,
                               int64_t num_nodes, int64_t num_edges, mp_graph *g,
                               void *workspace, size_t workspace_bytes, void *stream) {
    return build_impl(src, dst, idx_dtype, num_nodes, num_edges, g, workspace, workspace_bytes,
                      stream, true);
}

mp_status mp_graph_build_overlap(const void *src, const void *dst, mp_dtype idx_dtype,
                                 int64_t num_nodes, int64_t num_edges, mp_graph *g,
                                 void *workspace, size_t workspace_bytes, void *stream,
                                 void *side_stream, void *transpose_done) {
    if (!g) return fail(MP_ERR_NULL, "graph descriptor is NULL");
    g->built = 0;
    if (!side_stream) return fail(MP_ERR_NULL, "side_stream is NULL (the null stream would "
                                  "serialise with stream)");
    if (!transpose_done) return fail(MP_ERR_NULL, "transpose_done event is NULL");
    if (side_stream == stream) return fail(MP_ERR_ALIAS, "side_stream is stream");
    return build_impl(src, dst, idx_dtype, num_nodes, num_edges, g, workspace, workspace_bytes,
                      stream, true, false, side_stream, transpose_done);
}

mp_status mp_graph_build_noalloc(const void *src, const void *dst, mp_dtype idx_dtype,
                                 int64_t num_nodes, int64_t num_edges, mp_graph *g,
                                 void *stream) {
    if (!g) return fail(MP_ERR_NULL, "graph descriptor is NULL");
    g->built = 0;
    void *ws = nullptr;
    size_t ws_bytes = 0;
    mp_status st = static_workspace(&ws, &ws_bytes);
    if (st != MP_OK) return st;
    return build_impl(src, dst, idx_dtype, num_nodes, num_edges, g, ws, ws_bytes, stream, true,
                      true);
}

mp_status mp_graph_finish(mp_graph *g, void *stream) {
    if (!g) return fail(MP_ERR_NULL, "graph descriptor is NULL");
    if (g->built == MP_GRAPH_BUILT) return MP_OK;
    if (g->built != MP_GRAPH_ON_DEVICE)
        return fail(MP_ERR_GRAPH, "graph was not produced by a successful build");
    int bad = 0;
    mp_status st = lower_read_info(g, static_cast<hipStream_t>(stream), &bad);
    if (st != MP_OK) return st;
    if (bad) {
        g->built = 0;
        return fail(MP_ERR_INDEX, "an edge endpoint lies outside [0, %lld)",
                    (long long)g->num_nodes);
    }
    g->built = MP_GRAPH_BUILT;
    return MP_OK;
}


mp_status mp_spmm_fwd(const mp_graph *g, const float *w, const void *x, mp_dtype x_dtype,
                      int64_t h, float *y, void *stream) {
    return spmm_fwd_impl(g, w, 1, x, x_dtype, h, y, stream);
}

mp_status mp_spmm_fwd_pair(const mp_graph *g, const float *wg, const void *x, mp_dtype x_dtype,
                           int64_t h, float *y, void *stream) {
    return spmm_fwd_impl(g, wg, 1, x, x_dtype, h, y, stream, true);
}

mp_status mp_spmm_dx(const mp_graph *g, const float *w, const void *dy, mp_dtype dy_dtype,
                     int64_t h, float *dx, void *stream) {
    return spmm_dx_impl(g, w, 1, dy, dy_dtype, h, dx, stream);
}

mp_status mp_edge_grad_dw(const mp_graph *g, const void *x, const void *dy, mp_dtype dtype,
                          int64_t h, float *dw, void *stream) {
    return edge_grad_impl(g, x, dy, dtype, h, 1, dw, stream);
}

mp_status mp_spmm_dx_edge_grad(const mp_graph *g, const float *w, const void *x,
                               const void *dy, mp_dtype dtype, int64_t h, float *dx, float *dw,
                               void *stream) {
    return dx_edge_grad_impl(g, w, 1, x, dy, dtype, h, dx, dw, stream);
}

mp_status mp_spmm_split_workspace_size(const mp_graph *g, int64_t h, size_t *bytes) {
    if (!bytes) return fail(MP_ERR_NULL, "bytes is NULL");
    mp_status st = check_graph(g);
    if (st != MP_OK) return st;
    if (g->built != MP_GRAPH_BUILT)
        return fail(MP_ERR_GRAPH, "the split calls need a finished graph (mp_graph_build, or "
                                  "mp_graph_finish after an asynchronous build)");
    if ((st = check_h(g->num_nodes, h)) != MP_OK) return st;
    const size_t f = split_workspace_bytes(g->class_count, g->num_edges, h);
    const size_t t = split_workspace_bytes(g->class_count_t, g->num_edges, h);
    *bytes = f > t ? f : t;
    return MP_OK;
}

namespace {
// mp_spmm_fwd_split / mp_spmm_dx_split: the aggregation of one CSR form with
// its long rows split.
mp_status spmm_split_impl(const mp_graph *g, const CsrView &v, const float *w, const void *x,
                          mp_dtype dt, int64_t h, float *y, void *ws, size_t ws_bytes,
                          void *stream, const char *xname, const char *yname) {
    mp_status st = check_spmm(g, w, 1, x, dt, h, y, xname, yname);
    if (st != MP_OK) return st;
    const int64_t n = g->num_nodes, e = g->num_edges;
    RangeList others = graph_ranges(g);
    others.add(range(x, n * h, dtype_size(dt), xname));
    others.add(range(w, e, 4, "w"));
    others.add(range(y, n * h, 4, yname));
    size_t need = 0;
    if ((st = check_split(g, v, h, ws, ws_bytes, others, &need)) != MP_OK) return st;
    return spmm_run(v, w, 1, x, dt, h, y, static_cast<hipStream_t>(stream), nullptr, false,
                    need ? static_cast<float *>(ws) : nullptr);
}
}  // namespace

mp_status mp_spmm_fwd_split(const mp_graph *g, const float *w, const void *x, mp_dtype x_dtype,
                            int64_t h, float *y, void *workspace, size_t workspace_bytes,
                            void *stream) {
    if (mp_status st = check_graph(g)) return st;
    return spmm_split_impl(g, forward_view(g), w, x, x_dtype, h, y, workspace, workspace_bytes,
                           stream, "x", "y");
}

mp_status mp_spmm_dx_split(const mp_graph *g, const float *w, const void *dy, mp_dtype dy_dtype,
                           int64_t h, float *dx, void *workspace, size_t workspace_bytes,
                           void *stream) {
    if (mp_status st = check_graph(g)) return st;
    return spmm_split_impl(g, transpose_view(g), w, dy, dy_dtype, h, dx, workspace,
                           workspace_bytes, stream, "dy", "dx");
}

mp_status mp_spmm_dx_edge_grad_split(const mp_graph *g, const float *w, const void *x,
                                     const void *dy, mp_dtype dtype, int64_t h, float *dx,
                                     float *dw, void *workspace, size_t workspace_bytes,
                                     void *stream) {
    return dx_edge_grad_impl(g, w, 1, x, dy, dtype, h, dx, dw, stream, 0, true, workspace,
                             workspace_bytes);
}

mp_status mp_spmm_fwd_heads(const mp_graph *g, const float *w, int64_t heads, const void *x,
                            mp_dtype x_dtype, int64_t h, float *y, void *stream) {
    return spmm_fwd_impl(g, w, heads, x, x_dtype, h, y, stream);
}

mp_status mp_spmm_dx_heads(const mp_graph *g, const float *w, int64_t heads, const void *dy,
                           mp_dtype dy_dtype, int64_t h, float *dx, void *stream) {
    return spmm_dx_impl(g, w, heads, dy, dy_dtype, h, dx, stream);
}

mp_status mp_edge_grad_dw_heads(const mp_graph *g, const void *x, const void *dy,
                                mp_dtype dtype, int64_t h, int64_t heads, float *dw,
                                void *stream) {
    return edge_grad_impl(g, x, dy, dtype, h, heads, dw, stream);
}

mp_status mp_spmm_dx_edge_grad_heads(const mp_graph *g, const float *w, int64_t heads,
                                     const void *x, const void *dy, mp_dtype dtype, int64_t h,
                                     float *dx, float *dw, void *stream) {
    return dx_edge_grad_impl(g, w, heads, x, dy, dtype, h, dx, dw, stream);
}

namespace {
// Shared validation of the softmax calls: `edge_in` / `edge_in2` are [E, K]
// float inputs, `edge_out` an [E, K] float output, `row_out` an
// [N, K, row_width] output.
mp_status check_softmax(const mp_graph *g, int64_t heads, const float *edge_in,
                        const float *edge_in2, float *edge_out, float *row_out, int row_width,
                        const char *what) {
    mp_status st = check_graph(g);
    if (st != MP_OK) return st;
    if (heads < 1 || heads > (1 << 20))
        return fail(MP_ERR_SHAPE, "%s: head count %lld outside [1, 2^20]", what, (long long)heads);
    const int64_t n = g->num_nodes, e = g->num_edges;
    const int64_t ek = e * heads, nk = n * heads * row_width;
    const struct {
        const void *p;
        int64_t count;
        const char *name;
    } arr[] = {{edge_in, ek, "edge input"}, {edge_in2, edge_in2 ? ek : 0, "second edge input"},
               {edge_out, ek, "edge output"}, {row_out, nk, "row output"}};
    for (const auto &a : arr) {
        if (a.count > 0 && !a.p) return fail(MP_ERR_NULL, "%s: %s is NULL", what, a.name);
        if (a.p && !aligned(a.p, row_width == 2 && a.p == row_out ? 8 : 4))
            return fail(MP_ERR_ALIGN, "%s: %s misaligned", what, a.name);
        if (a.count > 0 && (st = check_device(a.p, a.name)) != MP_OK) return st;
    }
    Range outs[2] = {range(edge_out, ek, 4, "edge output"), range(row_out, nk, 4, "row output")};
    RangeList others = graph_ranges(g);
    others.add(range(edge_in, ek, 4, "edge input"));
    others.add(range(edge_in2, edge_in2 ? ek : 0, 4, "second edge input"));
    char prefix[96];
    snprintf(prefix, sizeof(prefix), "%s: ", what);
    for (int i = 0; i < 2; ++i)
        if ((st = apart(others, outs[i], prefix)) != MP_OK) return st;
    if (overlap(outs[0], outs[1]))
        return fail(MP_ERR_ALIAS, "%s: edge output overlaps row output", what);
    return MP_OK;
}

mp_status softmax_impl(const mp_graph *g, const float *scores, int64_t heads, float *alpha,
                       float *row_stats, void *stream, const char *what) {
    mp_status st = check_softmax(g, heads, scores, nullptr, alpha, row_stats, 2, what);
    if (st != MP_OK) return st;
    return edge_softmax_run(g, scores, heads, alpha, row_stats, static_cast<hipStream_t>(stream));
}

mp_status softmax_backward_impl(const mp_graph *g, const float *alpha, const float *dalpha,
                                int64_t heads, float *dscores, float *row_dot, void *stream,
                                const char *what) {
    if (!dalpha && g && g->num_edges > 0) return fail(MP_ERR_NULL, "%s: dalpha is NULL", what);
    mp_status st = check_softmax(g, heads, alpha, dalpha, dscores, row_dot, 1, what);
    if (st != MP_OK) return st;
    return edge_softmax_backward_run(g, alpha, dalpha, heads, dscores, row_dot,
                                     static_cast<hipStream_t>(stream));
}
}  // namespace

mp_status mp_edge_softmax(const mp_graph *g, const float *scores, float *alpha, float *row_stats,
                          void *stream) {
    return softmax_impl(g, scores, 1, alpha, row_stats, stream, "mp_edge_softmax");
}

mp_status mp_edge_softmax_backward(const mp_graph *g, const float *alpha, const float *dalpha,
                                   float *dscores, float *row_dot, void *stream) {
    return softmax_backward_impl(g, alpha, dalpha, 1, dscores, row_dot, stream,
                                 "mp_edge_softmax_backward");
}

mp_status mp_edge_softmax_heads(const mp_graph *g, const float *scores, int64_t heads,
                                float *alpha, float *row_stats, void *stream) {
    return softmax_impl(g, scores, heads, alpha, row_stats, stream, "mp_edge_softmax_heads");
}

mp_status mp_edge_softmax_backward_heads(const mp_graph *g, const float *alpha,
                                         const float *dalpha, int64_t heads, float *dscores,
                                         float *row_dot, void *stream) {
    return softmax_backward_impl(g, alpha, dalpha, heads, dscores, row_dot, stream,
                                 "mp_edge_softmax_backward_heads");
}

mp_status mp_spmm_fwd_norm(const mp_graph *g, int32_t mode, const float *w, const void *x,
                           mp_dtype x_dtype, int64_t h, float *y, void *stream) {
    mp_status st = check_norm_mode(mode, "mp_spmm_fwd_norm");
    if (st != MP_OK) return st;
    if ((st = check_spmm(g, w, 1, x, x_dtype, h, y, "x", "y")) != MP_OK) return st;
    const NormSpec nm = norm_spec(g, mode, true);
    return spmm_run(forward_view(g), w, 1, x, x_dtype, h, y, static_cast<hipStream_t>(stream),
                    &nm);
}

mp_status mp_spmm_fwd_softmax(const mp_graph *g, const float *scores, const void *x,
                              mp_dtype x_dtype, int64_t h, float *y, float *row_stats,
                              void *stream) {
    const char *what = "mp_spmm_fwd_softmax";
    mp_status st = check_spmm(g, scores, 1, x, x_dtype, h, y, "x", "y");
    if (st != MP_OK) return st;
    const int64_t n = g->num_nodes, e = g->num_edges;
    if (!row_stats) return fail(MP_ERR_NULL, "%s: row_stats is NULL", what);
    if (!aligned(row_stats, 8)) return fail(MP_ERR_ALIGN, "%s: row_stats misaligned", what);
    if ((st = check_device(row_stats, "row_stats")) != MP_OK) return st;
    const Range rs = range(row_stats, 2 * n, 4, "row_stats");
    RangeList others = graph_ranges(g);
    others.add(range(x, n * h, dtype_size(x_dtype), "x"));
    others.add(range(scores, e, 4, "scores"));
    others.add(range(y, n * h, 4, "y"));
    if ((st = apart(others, rs, "mp_spmm_fwd_softmax: ")) != MP_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = edge_softmax_stats_run(g, scores, row_stats, s)) != MP_OK) return st;
    NormSpec nm{kFetchSoftmax, true, nullptr, reinterpret_cast<const float2 *>(row_stats)};
    return spmm_run(forward_view(g), scores, 1, x, x_dtype, h, y, s, &nm);
}

mp_status mp_spmm_dx_norm(const mp_graph *g, int32_t mode, const float *w, const void *dy,
                          mp_dtype dy_dtype, int64_t h, float *dx, void *stream) {
    mp_status st = check_norm_mode(mode, "mp_spmm_dx_norm");
    if (st != MP_OK) return st;
    if ((st = check_spmm(g, w, 1, dy, dy_dtype, h, dx, "dy", "dx")) != MP_OK) return st;
    const NormSpec nm = norm_spec(g, mode, false);
    return spmm_run(transpose_view(g), w, 1, dy, dy_dtype, h, dx,
                    static_cast<hipStream_t>(stream), &nm);
}

mp_status mp_spmm_dx_edge_grad_pair(const mp_graph *g, float *wg, const void *x,
                                    const void *dy, mp_dtype dtype, int64_t h, float *dx,
                                    void *stream) {
    mp_status st = check_spmm(g, wg, 1, dy, dtype, h, dx, "dy", "dx", 2);
    if (st != MP_OK) return st;
    const int64_t n = g->num_nodes, e = g->num_edges;
    if (!x) return fail(MP_ERR_NULL, "x is NULL");
    const size_t xs = dtype_size(dtype);
    if (!aligned(x, xs)) return fail(MP_ERR_ALIGN, "x not aligned to %zu bytes", xs);
    if ((st = check_device(x, "x")) != MP_OK) return st;
    const Range rwg = range(wg, 2 * e, 4, "wg");
    RangeList others = graph_ranges(g);
    others.add(range(x, n * h, xs, "x"));
    others.add(range(dy, n * h, xs, "dy"));
    others.add(range(dx, n * h, 4, "dx"));
    if ((st = apart(others, rwg)) != MP_OK) return st;
    if (overlap(range(dx, n * h, 4, "dx"), range(x, n * h, xs, "x")))
        return fail(MP_ERR_ALIAS, "dx overlaps x");
    if (!spmm_fused_supported(dtype, h, 1, dy, x, dx))
        return fail(MP_ERR_SHAPE,
                    "the interleaved layout needs the fused backward (H up to 64 lanes of "
                    "16-byte slices, aligned rows); H = %lld", (long long)h);
    hipStream_t s = static_cast<hipStream_t>(stream);
    return spmm_fused_run(transpose_view(g), wg, 1, dy, dtype, h, dx, x,
                          e > 0 ? wg + 1 : nullptr, nullptr, s, nullptr, e > 0);
}

mp_status mp_spmm_dx_edge_grad_norm(const mp_graph *g, int32_t mode, const float *w,
                                    const void *x, const void *dy, mp_dtype dtype, int64_t h,
                                    float *dx, float *dw, void *stream) {
    mp_status st = check_norm_mode(mode, "mp_spmm_dx_edge_grad_norm");
    if (st != MP_OK) return st;
    return dx_edge_grad_impl(g, w, 1, x, dy, dtype, h, dx, dw, stream, mode);
}

namespace {
// With stats, `alpha` holds the scores and each alpha is formed from its score
// and its destination's softmax statistics [N][2] in the walk (one head).
mp_status attention_backward_impl(const mp_graph *g, const float *alpha, int64_t heads,
                                  const void *x, const void *dy, const float *y, mp_dtype dtype,
                                  int64_t h, float *dx, float *dscores, float *row_dot,
                                  void *stream, const float *stats = nullptr) {
    mp_status st = check_spmm(g, alpha, heads, dy, dtype, h, dx, "dy", "dx");
    if (st != MP_OK) return st;
    const int64_t n = g->num_nodes, e = g->num_edges;
    if (!x) return fail(MP_ERR_NULL, "x is NULL");
    if (!y) return fail(MP_ERR_NULL, "y is NULL");
    if (!row_dot) return fail(MP_ERR_NULL, "row_dot is NULL");
    if (!dscores && e > 0) return fail(MP_ERR_NULL, "dscores is NULL with %lld edges", (long long)e);
    const size_t xs = dtype_size(dtype);
    if (!aligned(x, xs)) return fail(MP_ERR_ALIGN, "x not aligned to %zu bytes", xs);
    if (!aligned(y, 4) || !aligned(row_dot, 4) || (dscores && !aligned(dscores, 4)))
        return fail(MP_ERR_ALIGN, "y, dscores or row_dot not aligned to 4 bytes");
    if ((st = check_device(x, "x")) != MP_OK) return st;
    if ((st = check_device(y, "y")) != MP_OK) return st;
    if ((st = check_device(row_dot, "row_dot")) != MP_OK) return st;
    if (e > 0 && (st = check_device(dscores, "dscores")) != MP_OK) return st;
    const Range rdx = range(dx, n * h, 4, "dx"), rds = range(dscores, e * heads, 4, "dscores");
    const Range rt = range(row_dot, n * heads, 4, "row_dot");
    // dscores may be alpha itself (written over it in the fused walk); any
    // other overlap is rejected.
    const bool in_place = e > 0 && dscores == alpha;
    const bool fused = spmm_fused_supported(dtype, h, heads, dy, x, dx);
    if (in_place && !fused)
        return fail(MP_ERR_ALIAS, "dscores may be alpha only when the feature rows fit the "
                                  "fused walk (H up to 64 lanes of 16-byte slices)");
    if (stats && !fused)
        return fail(MP_ERR_SHAPE, "alpha formed from scores needs feature rows that fit the "
                                  "fused walk (H up to 64 lanes of 16-byte slices)");
    RangeList others = graph_ranges(g);
    if (stats) {
        if (!aligned(stats, 8)) return fail(MP_ERR_ALIGN, "row_stats not aligned to 8 bytes");
        if ((st = check_device(stats, "row_stats")) != MP_OK) return st;
        others.add(range(stats, 2 * n, 4, "row_stats"));
    }
    others.add(range(x, n * h, xs, "x"));
    others.add(range(dy, n * h, xs, "dy"));
    others.add(range(y, n * h, 4, "y"));
    if (!in_place) others.add(range(alpha, e * heads, 4, "alpha"));
    if ((st = apart(others, rdx)) != MP_OK) return st;
    if (in_place && overlap(rdx, rds)) return fail(MP_ERR_ALIAS, "dx overlaps alpha");
    others.add(rdx);
    if ((st = apart(others, rds)) != MP_OK) return st;
    others.add(rds);
    if ((st = apart(others, rt)) != MP_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = attention_row_dot_run(y, dy, dtype, n, h, heads, row_dot, s)) != MP_OK) return st;
    const CsrView v = transpose_view(g);
    if (stats) {
        const NormSpec nm{kFetchSoftmax, false, nullptr, reinterpret_cast<const float2 *>(stats)};
        return spmm_fused_run(v, alpha, 1, dy, dtype, h, dx, x, e > 0 ? dscores : nullptr,
                              row_dot, s, &nm);
    }
    if (fused)
        return spmm_fused_run(v, alpha, heads, dy, dtype, h, dx, x, e > 0 ? dscores : nullptr,
                              row_dot, s);
    // Feature rows wider than one column block: dX, then dalpha into dscores,
    // then the score gradient in place.
    if ((st = spmm_run(v, alpha, heads, dy, dtype, h, dx, s)) != MP_OK) return st;
    if (e == 0) return MP_OK;
    if ((st = sddmm_run(g->src, g->dst, e, x, dy, dtype, h, heads, dscores, s)) != MP_OK)
        return st;
    return score_grad_apply_run(g->dst, alpha, row_dot, e, heads, dscores, s);
}
}  // namespace

mp_status mp_attention_backward_scores(const mp_graph *g, const float *scores,
                                       const float *row_stats, const void *x, const void *dy,
                                       const float *y, mp_dtype dtype, int64_t h, float *dx,
                                       float *dscores, float *row_dot, void *stream) {
    if (!row_stats) return fail(MP_ERR_NULL, "row_stats is NULL");
    return attention_backward_impl(g, scores, 1, x, dy, y, dtype, h, dx, dscores, row_dot,
                                   stream, row_stats);
}

mp_status mp_attention_backward(const mp_graph *g, const float *alpha, int64_t heads,
                                const void *x, const void *dy, const float *y, mp_dtype dtype,
                                int64_t h, float *dx, float *dscores, float *row_dot,
                                void *stream) {
    return attention_backward_impl(g, alpha, heads, x, dy, y, dtype, h, dx, dscores, row_dot,
                                   stream);
}

mp_status mp_edge_normalize(const mp_graph *g, int32_t mode, const float *in, float *out,
                            void *stream) {
    mp_status st = check_graph(g);
    if (st != MP_OK) return st;
    if (mode != MP_NORM_MEAN && mode != MP_NORM_SYM)
        return fail(MP_ERR_DTYPE, "mp_edge_normalize: unknown mode %d", (int)mode);
    const int64_t e = g->num_edges;
    if (e == 0) return MP_OK;
    if (!in || !out) return fail(MP_ERR_NULL, "mp_edge_normalize: in or out is NULL");
    if (!aligned(in, 4) || !aligned(out, 4))
        return fail(MP_ERR_ALIGN, "mp_edge_normalize: in/out not aligned to 4 bytes");
    if ((st = check_device(in, "in")) != MP_OK) return st;
    if ((st = check_device(out, "out")) != MP_OK) return st;
    const Range ro = range(out, e, 4, "out"), ri = range(in, e, 4, "in");
    if (ro.lo != ri.lo && overlap(ro, ri))
        return fail(MP_ERR_ALIAS, "mp_edge_normalize: out partially overlaps in");
    if ((st = apart(graph_ranges(g), ro, "mp_edge_normalize: ")) != MP_OK) return st;
    return edge_normalize_run(g, mode, in, out, static_cast<hipStream_t>(stream));
}

const char *mp_status_string(mp_status s) {
    switch (s) {
        case MP_OK: return "MP_OK";
        case MP_ERR_NULL: return "MP_ERR_NULL: a required pointer is NULL";
        case MP_ERR_SHAPE: return "MP_ERR_SHAPE: a size is out of range";
        case MP_ERR_DTYPE: return "MP_ERR_DTYPE: unsupported dtype";
        case MP_ERR_DEVICE: return "MP_ERR_DEVICE: pointer is not device memory of the current GPU";
        case MP_ERR_INDEX: return "MP_ERR_INDEX: edge endpoint outside [0, N)";
        case MP_ERR_ALIAS: return "MP_ERR_ALIAS: output overlaps an input or the graph";
        case MP_ERR_ALIGN: return "MP_ERR_ALIGN: pointer misaligned for its element type";
        case MP_ERR_WORKSPACE: return "MP_ERR_WORKSPACE: workspace missing or too small";
        case MP_ERR_GRAPH: return "MP_ERR_GRAPH: graph not built";
        case MP_ERR_HIP: return "MP_ERR_HIP: HIP runtime error";
        case MP_ERR_INTERNAL: return "MP_ERR_INTERNAL: internal limit of the library reached";
        default: return "unknown mp_status";
    }
}

const char *mp_last_error_detail(void) { return g_detail; }

mp_status mp_set_owner_overrides(int32_t hub_min_len, int32_t hub_apart, int32_t wave_min_len) {
    return set_owner_overrides(hub_min_len, hub_apart, wave_min_len);
}

int32_t mp_version(void) { return 100; }   // 0.1.0

}  // extern "C"
