// Drives every validating entry point of libmp's C interface through the
// host-only build of its argument checks (api.hip with tests/asan/stubs.hip):
// plain valid calls, calls whose output overlaps an input, and, in a build
// whose overlap lists hold fewer ranges than the calls need ("small"), the
// MP_ERR_INTERNAL refusal that replaces writing past the list.  Pointers are
// fake, disjoint device addresses; nothing is dereferenced.
//   driver normal   -- every valid call returns MP_OK and reaches its launcher
//   driver small    -- every call that checks overlaps returns MP_ERR_INTERNAL
// Prints one line per failed expectation; exit status = their number.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mp.h"

extern "C" int g_launches;

static int failures = 0;
static bool small_lists = false;

// Slot k of the fake address space: 64 GiB apart, so no two arrays overlap.
static void *slot(int k) { return reinterpret_cast<void *>((uintptr_t)(k + 1) << 36); }

static void expect(const char *what, mp_status got, mp_status want, int launches_before) {
    const bool launched = g_launches > launches_before;
    const bool ok = got == want && (want != MP_OK || launched);
    if (!ok) {
        printf("FAIL %s: status %d (%s), wanted %d; detail: %s\n", what, (int)got,
               mp_status_string(got), (int)want, mp_last_error_detail());
        ++failures;
    }
}

// A valid call: MP_OK and a launch, or MP_ERR_INTERNAL in the small-list build.
#define VALID(call)                                                                   \
    do {                                                                              \
        const int b__ = g_launches;                                                   \
        expect(#call, (call), small_lists ? MP_ERR_INTERNAL : MP_OK, b__);            \
    } while (0)
// An output overlapping an input: MP_ERR_ALIAS (or MP_ERR_INTERNAL, small lists).
#define ALIAS(call)                                                                   \
    do {                                                                              \
        const int b__ = g_launches;                                                   \
        expect(#call, (call), small_lists ? MP_ERR_INTERNAL : MP_ERR_ALIAS, b__);     \
    } while (0)

int main(int argc, char **argv) {
    small_lists = argc > 1 && strcmp(argv[1], "small") == 0;
    const int64_t n = 1000, e = 5000, h = 64, k = 4;
    int s = 0;
    mp_graph g;
    memset(&g, 0, sizeof(g));
    g.num_nodes = n;
    g.num_edges = e;
    int32_t **arrays[] = {&g.src, &g.dst, &g.rowptr, &g.col, &g.edge_order, &g.rowptr_t,
                          &g.col_t, &g.transpose_order, &g.row_plan, &g.row_plan_t};
    for (int32_t **a : arrays) *a = static_cast<int32_t *>(slot(s++));
    g.info = static_cast<uint32_t *>(slot(s++));
    const void *src = slot(s++), *dst = slot(s++);
    void *ws = slot(s++);
    size_t ws_bytes = 0;
    if (mp_graph_build_workspace_size(n, e, &ws_bytes) != MP_OK) {
        printf("FAIL workspace size\n");
        return 1;
    }
    float *w = static_cast<float *>(slot(s++)), *w2 = static_cast<float *>(slot(s++));
    const void *x = slot(s++), *dy = slot(s++);
    float *y = static_cast<float *>(slot(s++)), *dx = static_cast<float *>(slot(s++));
    float *dw = static_cast<float *>(slot(s++)), *rs = static_cast<float *>(slot(s++));
    float *rd = static_cast<float *>(slot(s++)), *alpha = static_cast<float *>(slot(s++));

    VALID(mp_graph_build(src, dst, MP_I64, n, e, &g, ws, ws_bytes, nullptr));
    VALID(mp_graph_build_async(src, dst, MP_I64, n, e, &g, ws, ws_bytes, nullptr));
    VALID(mp_graph_build_noalloc(src, dst, MP_I64, n, e, &g, nullptr));
    {   // too large for the static workspace: refused before any range list
        const int b = g_launches;
        mp_graph big = g;
        big.num_edges = 5000000;
        expect("mp_graph_build_noalloc (too large)",
               mp_graph_build_noalloc(src, dst, MP_I64, n, 5000000, &big, nullptr),
               MP_ERR_WORKSPACE, b);
    }
    {   // the two-stream build: its own workspace size, two streams, an event
        size_t ows = 0;
        if (mp_graph_build_overlap_workspace_size(n, e, &ows) != MP_OK || ows < ws_bytes) {
            printf("FAIL overlap workspace size\n");
            ++failures;
        }
        void *s0 = reinterpret_cast<void *>(0x100), *s1 = reinterpret_cast<void *>(0x200);
        void *ev = reinterpret_cast<void *>(0x300);
        VALID(mp_graph_build_overlap(src, dst, MP_I64, n, e, &g, ws, ows, s0, s1, ev));
        ALIAS(mp_graph_build_overlap(src, dst, MP_I64, n, e, &g, g.col_t, ows, s0, s1, ev));
        int b = g_launches;
        expect("mp_graph_build_overlap (no side stream)",
               mp_graph_build_overlap(src, dst, MP_I64, n, e, &g, ws, ows, s0, nullptr, ev),
               MP_ERR_NULL, b);
        expect("mp_graph_build_overlap (no event)",
               mp_graph_build_overlap(src, dst, MP_I64, n, e, &g, ws, ows, s0, s1, nullptr),
               MP_ERR_NULL, b);
        expect("mp_graph_build_overlap (one stream)",
               mp_graph_build_overlap(src, dst, MP_I64, n, e, &g, ws, ows, s0, s0, ev),
               MP_ERR_ALIAS, b);
        expect("mp_graph_build_overlap (workspace of the one-stream build)",
               mp_graph_build_overlap(src, dst, MP_I64, n, e, &g, ws, ws_bytes, s0, s1, ev),
               ows > ws_bytes ? MP_ERR_WORKSPACE : (small_lists ? MP_ERR_INTERNAL : MP_OK), b);
    }
    // the workspace over a graph array
    ALIAS(mp_graph_build(src, dst, MP_I64, n, e, &g, g.col, ws_bytes, nullptr));
    g.built = MP_GRAPH_BUILT;

    VALID(mp_spmm_fwd(&g, w, x, MP_BF16, h, y, nullptr));
    ALIAS(mp_spmm_fwd(&g, w, x, MP_BF16, h, (float *)g.col, nullptr));
    VALID(mp_spmm_dx(&g, w, dy, MP_BF16, h, dx, nullptr));
    ALIAS(mp_spmm_dx(&g, w, dy, MP_F32, h, (float *)dy, nullptr));
    VALID(mp_edge_grad_dw(&g, x, dy, MP_BF16, h, dw, nullptr));
    ALIAS(mp_edge_grad_dw(&g, x, dy, MP_BF16, h, (float *)x, nullptr));
    VALID(mp_spmm_dx_edge_grad(&g, w, x, dy, MP_BF16, h, dx, dw, nullptr));
    ALIAS(mp_spmm_dx_edge_grad(&g, w, x, dy, MP_BF16, h, dx, w, nullptr));
    VALID(mp_spmm_dx_edge_grad_pair(&g, w, x, dy, MP_BF16, h, dx, nullptr));
    ALIAS(mp_spmm_dx_edge_grad_pair(&g, (float *)g.col_t, x, dy, MP_BF16, h, dx, nullptr));
    VALID(mp_spmm_fwd_pair(&g, w, x, MP_BF16, h, y, nullptr));
    ALIAS(mp_spmm_fwd_pair(&g, w, x, MP_BF16, h, (float *)g.rowptr, nullptr));
    {   // split calls: a workspace of the size the (stub) plan asks for
        size_t need = 0;
        if (mp_spmm_split_workspace_size(&g, h, &need) != MP_OK) {
            printf("FAIL split workspace size\n");
            ++failures;
        }
        void *sw = slot(s++);
        VALID(mp_spmm_fwd_split(&g, w, x, MP_BF16, h, y, sw, need, nullptr));
        VALID(mp_spmm_dx_split(&g, w, dy, MP_BF16, h, dx, sw, need, nullptr));
        VALID(mp_spmm_dx_edge_grad_split(&g, w, x, dy, MP_BF16, h, dx, dw, sw, need, nullptr));
        ALIAS(mp_spmm_fwd_split(&g, w, x, MP_BF16, h, y, y, need, nullptr));
        ALIAS(mp_spmm_dx_edge_grad_split(&g, w, x, dy, MP_BF16, h, dx, dw, dw, need, nullptr));
    }
    VALID(mp_spmm_fwd_heads(&g, w, k, x, MP_BF16, h, y, nullptr));
    VALID(mp_spmm_dx_heads(&g, w, k, dy, MP_BF16, h, dx, nullptr));
    VALID(mp_edge_grad_dw_heads(&g, x, dy, MP_BF16, h, k, dw, nullptr));
    VALID(mp_spmm_dx_edge_grad_heads(&g, w, k, x, dy, MP_BF16, h, dx, dw, nullptr));
    ALIAS(mp_spmm_dx_edge_grad_heads(&g, w, k, x, dy, MP_BF16, h, dx, (float *)g.info, nullptr));
    VALID(mp_edge_softmax(&g, w, alpha, rs, nullptr));
    ALIAS(mp_edge_softmax(&g, w, alpha, (float *)g.dst, nullptr));
    VALID(mp_spmm_fwd_softmax(&g, w, x, MP_BF16, h, y, rs, nullptr));
    ALIAS(mp_spmm_fwd_softmax(&g, w, x, MP_BF16, h, y, w, nullptr));
    VALID(mp_edge_softmax_backward(&g, alpha, w2, dw, rd, nullptr));
    ALIAS(mp_edge_softmax_backward(&g, alpha, w2, dw, (float *)g.src, nullptr));
    VALID(mp_edge_softmax_heads(&g, w, k, alpha, rs, nullptr));
    VALID(mp_edge_softmax_backward_heads(&g, alpha, w2, k, dw, rd, nullptr));
    VALID(mp_attention_backward(&g, alpha, 1, x, dy, y, MP_BF16, h, dx, dw, rd, nullptr));
    VALID(mp_attention_backward(&g, alpha, 1, x, dy, y, MP_BF16, h, dx, alpha, rd, nullptr));
    ALIAS(mp_attention_backward(&g, alpha, 1, x, dy, y, MP_BF16, h, dx, dw, (float *)y, nullptr));
    VALID(mp_attention_backward_scores(&g, w, rs, x, dy, y, MP_BF16, h, dx, dw, rd, nullptr));
    ALIAS(mp_attention_backward_scores(&g, w, rs, x, dy, y, MP_BF16, h, dx, dw, rs, nullptr));
    VALID(mp_edge_normalize(&g, MP_NORM_SYM, w, w2, nullptr));
    ALIAS(mp_edge_normalize(&g, MP_NORM_SYM, w, (float *)g.col, nullptr));
    VALID(mp_spmm_fwd_norm(&g, MP_NORM_SYM, w, x, MP_BF16, h, y, nullptr));
    VALID(mp_spmm_dx_norm(&g, MP_NORM_MEAN, w, dy, MP_BF16, h, dx, nullptr));
    VALID(mp_spmm_dx_edge_grad_norm(&g, MP_NORM_SYM, w, x, dy, MP_BF16, h, dx, dw, nullptr));
    ALIAS(mp_spmm_dx_edge_grad_norm(&g, MP_NORM_SYM, w, x, dy, MP_BF16, h, dx, (float *)x,
                                    nullptr));
    printf("%s lists: %d failures, %d launches\n", small_lists ? "small" : "full", failures,
           g_launches);
    return failures;
}
