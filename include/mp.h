/*
 * mp.h -- C ABI of the weighted sparse message-passing library (libmp.so) for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (tinymesh, "Weighted aggregation experiment"):
 *   given COO edges e = 0..E-1 with (src_e, dst_e) in [0, N)^2, one scalar
 *   weight w_e per edge in COO order, node features X[N, H] and an upstream
 *   gradient dY[N, H], with A_w[dst_e, src_e] += w_e (duplicates add):
 *     forward          Y  = A_w   X     destination-owned CSR    ("Decision")
 *     input gradient   dX = A_w^T dY    source-owned (transpose) CSR
 *     edge gradient    dw_e = <X[src_e, :], dY[dst_e, :]>, one owner per edge
 *   No call materialises per-edge [E, H] message rows; the forward and input
 *   gradient use no atomics; w and dw stay in the caller's COO order
 *   ("Edge order is explicit").
 *
 * Conventions shared by every entry point
 *   - Memory: every array argument is device memory on the current HIP device,
 *     allocated and owned by the caller.  The library never allocates device
 *     memory, never frees caller memory, never keeps a pointer past a call
 *     except those stored in an mp_graph, and never writes an input.
 *   - Layout: X, dY, Y, dX are contiguous row-major [N, H]; w and dw are
 *     contiguous [E] in COO order; graph arrays are contiguous int32.
 *   - Sizes: 1 <= N < 2^31, 0 <= E < 2^31, 1 <= H < 2^31, N*H < 2^62.
 *   - Outputs are overwritten completely (never accumulated into); a row with
 *     no edges is written as exact zeros.
 *   - Streams: `stream` is a hipStream_t (0 = the null stream).  All device
 *     work is enqueued on it.  Only mp_graph_build and mp_graph_finish
 *     synchronise that stream (once, at their end); every compute call returns
 *     without waiting.
 *   - Errors: arguments are validated on the host before anything is
 *     enqueued; a rejected call launches nothing and writes nothing.  No C++
 *     exception crosses this interface.  mp_last_error_detail() returns a
 *     thread-local text describing the last non-OK status on this thread.
 *   - Determinism: for a fixed graph, H, feature dtype and device, results
 *     are bitwise reproducible (fixed reduction order, no atomics).  The one
 *     thing outside the arguments that changes the bits is
 *     mp_set_owner_overrides (tests and tuning only; unset by default), which
 *     moves rows between owners and so changes their summation order.
 */
#ifndef MP_H
#define MP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
typedef int32_t mp_status;
#define MP_OK             0
#define MP_ERR_NULL      (-1)   /* a required pointer is NULL                         */
#define MP_ERR_SHAPE     (-2)   /* a size is out of range                             */
#define MP_ERR_DTYPE     (-3)   /* unsupported dtype code for this argument           */
#define MP_ERR_DEVICE    (-4)   /* a pointer is not device memory of the current GPU  */
#define MP_ERR_INDEX     (-5)   /* an edge endpoint lies outside [0, N)               */
#define MP_ERR_ALIAS     (-6)   /* an output overlaps an input or the graph           */
#define MP_ERR_ALIGN     (-7)   /* a pointer is not aligned to its element size       */
#define MP_ERR_WORKSPACE (-8)   /* workspace missing or smaller than required         */
#define MP_ERR_GRAPH     (-9)   /* mp_graph not produced by a successful build        */
#define MP_ERR_HIP      (-10)   /* the HIP runtime reported an error (see detail)     */
#define MP_ERR_INTERNAL (-11)   /* an internal limit of the library was reached (a bug) */

/* Element type codes. */
typedef int32_t mp_dtype;
#define MP_I32  1
#define MP_I64  2
#define MP_F32  3
#define MP_BF16 4

/* Number of degree classes: class 0 holds rows with no edges, class c >= 1
 * holds rows whose length has c binary digits (lengths 2^(c-1) .. 2^c - 1). */
#define MP_NUM_CLASSES 33

/* Words of the device-side build record a graph carries (mp_graph.info). */
#define MP_GRAPH_INFO_WORDS 576

/*
 * mp_graph -- the lowered topology, a plain descriptor in host memory.
 *
 * The caller allocates the descriptor and every device array it points to
 * (sizes below), fills in the pointers, and passes it to mp_graph_build,
 * which writes every array and the host-side fields.  Afterwards the arrays
 * are read-only; the graph stays valid as long as the caller keeps them.
 *
 *   src, dst           [E]    edge identity in COO order (int32 copies of the
 *                             caller's endpoints)
 *   rowptr             [N+1]  forward CSR (rows = destinations)
 *   col                [E]    col[p] = src[edge_order[p]]
 *   edge_order         [E]    CSR position -> COO ordinal, ascending ordinal
 *                             inside a row ("Edge order is explicit")
 *   rowptr_t           [N+1]  transpose CSR (rows = sources)
 *   col_t              [E]    col_t[q] = dst[transpose_order[q]]
 *   transpose_order    [E]    transpose position -> COO ordinal
 *   row_plan, row_plan_t [N]  rows of each CSR listed by degree class, highest
 *                             class first, ascending row id within a class
 *   info   [MP_GRAPH_INFO_WORDS] uint32, device: the build's own record (the
 *                             index check and the rows per class of both
 *                             plans), read by the compute calls when the host
 *                             copies below are not filled in yet
 *   class_count, class_count_t  host copies of the number of rows per class
 *
 * Together the two CSR forms hold 2E + 2(N+1) integers and the edge identity
 * 4E integers, as tallied in "Edge order is explicit"; the two plans add 2N.
 */
typedef struct mp_graph {
    int64_t num_nodes;
    int64_t num_edges;
    int32_t *src;
    int32_t *dst;
    int32_t *rowptr;
    int32_t *col;
    int32_t *edge_order;
    int32_t *rowptr_t;
    int32_t *col_t;
    int32_t *transpose_order;
    int32_t *row_plan;
    int32_t *row_plan_t;
    uint32_t *info;
    int64_t class_count[MP_NUM_CLASSES];
    int64_t class_count_t[MP_NUM_CLASSES];
    uint64_t built;     /* MP_GRAPH_BUILT, MP_GRAPH_ON_DEVICE or 0 */
} mp_graph;

/* States of mp_graph.built. */
#define MP_GRAPH_BUILT     0x6d705f6772617068ull  /* lowered; host counts valid      */
#define MP_GRAPH_ON_DEVICE 0x6d705f6465766963ull  /* lowered on the stream; counts
                                                    on the device only (async build) */

/*
 * Device workspace (bytes) that mp_graph_build needs for N nodes and E edges.
 * Returns MP_ERR_SHAPE for sizes out of range, MP_ERR_NULL if `bytes` is NULL.
 */
mp_status mp_graph_build_workspace_size(int64_t num_nodes, int64_t num_edges, size_t *bytes);

/*
 * Lower a COO edge list into the two CSR forms, their order maps and the
 * degree plans (tinymesh "Weighted aggregation experiment", "Edge order is
 * explicit": a stable sort by destination gives edge_order, by source gives
 * transpose_order; the witness of "Exact witness" lowers to edge_order =
 * (2, 0, 1)).
 *
 *   src, dst    device arrays [E] of `idx_dtype` (MP_I32 or MP_I64), COO order;
 *               e.g. the two rows of a PyTorch edge_index.
 *   num_nodes   N (explicit; trailing isolated nodes are allowed).
 *   num_edges   E (0 allowed).
 *   g           descriptor with every device array pointer set (see mp_graph).
 *   workspace   device scratch of at least mp_graph_build_workspace_size bytes,
 *               256-byte aligned; contents on entry are ignored.
 *   stream      hipStream_t.
 *
 * Enqueues the lowering on `stream`, then synchronises it once to read the
 * class counts and the index check back.  An endpoint outside [0, N) returns
 * MP_ERR_INDEX and leaves g->built = 0 (the arrays then hold unspecified
 * values).  On success g->built is set.
 */
mp_status mp_graph_build(const void *src, const void *dst, mp_dtype idx_dtype,
                         int64_t num_nodes, int64_t num_edges, mp_graph *g,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * The same lowering without the final synchronisation, for back-to-back
 * batches with a changing topology (tinymesh "Weighted aggregation
 * experiment", "Limits", names batching and topology changes as open): the
 * host can enqueue the build of the next batch on one stream while the
 * current batch computes on another, and the whole sequence can be captured
 * in a HIP graph (nothing here waits on the host or sets memory with memset).
 *
 * Arguments and host-side validation are those of mp_graph_build.  On return
 * the work is only enqueued: g->built = MP_GRAPH_ON_DEVICE, the host class
 * counts are zero, and every compute call on `g` reads the counts from g->info
 * on the device instead (its launch then covers the largest plan N and E
 * allow; blocks without work exit).  Work on other streams must wait for
 * `stream` (an event) before using the graph.  The workspace is in use until
 * the build has run: concurrent builds need separate workspaces.
 *
 * The index check is not reported here.  An endpoint outside [0, N) is stored
 * as 0, so later kernels stay in bounds, but the graph then describes a
 * different edge list; mp_graph_finish reports it.
 */
mp_status mp_graph_build_async(const void *src, const void *dst, mp_dtype idx_dtype,
                               int64_t num_nodes, int64_t num_edges, mp_graph *g,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * The asynchronous lowering with its two directions on two streams, so that
 * the forward CSR can be used while the transpose CSR is still being built:
 * a training step's forward aggregation then overlaps the transpose half of
 * the build (the forward needs only rowptr, col, edge_order and row_plan;
 * "Edge order is explicit" keeps the two lowerings independent).
 *
 *   stream          the intake, then the forward CSR (rowptr, col, edge_order)
 *                   and its degree plan (row_plan).
 *   side_stream     the transpose CSR (rowptr_t, col_t, transpose_order) and its
 *                   plan (row_plan_t), after the intake; not NULL, not `stream`.
 *   transpose_done  a hipEvent_t created by the caller; recorded on side_stream
 *                   once the transpose CSR and its plan are written.
 *   workspace       at least mp_graph_build_overlap_workspace_size(N, E) bytes
 *                   (each direction has its own sort buffers), 256-byte aligned.
 *
 * The other arguments, the validation and the results (bit for bit those of
 * mp_graph_build) are those of mp_graph_build_async; g is left as it leaves it
 * (g->built = MP_GRAPH_ON_DEVICE).  Work on `stream` may use the forward CSR at
 * once (mp_spmm_fwd and its forms, and mp_edge_grad_dw, which reads only the
 * COO copies the intake writes); work that reads the transpose CSR
 * (mp_spmm_dx and its forms, the fused backward calls, the attention backward
 * calls) and mp_graph_finish must first wait for transpose_done
 * (hipStreamWaitEvent).  The workspace is in use until both streams have run
 * the build.  Returns MP_ERR_NULL for a NULL side_stream or transpose_done,
 * MP_ERR_ALIAS when side_stream is stream.
 */
mp_status mp_graph_build_overlap_workspace_size(int64_t num_nodes, int64_t num_edges,
                                                size_t *bytes);
mp_status mp_graph_build_overlap(const void *src, const void *dst, mp_dtype idx_dtype,
                                 int64_t num_nodes, int64_t num_edges, mp_graph *g,
                                 void *workspace, size_t workspace_bytes, void *stream,
                                 void *side_stream, void *transpose_done);

/*
 * mp_graph_build_async without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The lowering's scratch is a static array
 * of MP_STATIC_WORKSPACE_BYTES in the library's device code, one per GPU the
 * library runs on, held until the process ends; this call allocates nothing
 * and calls no allocating routine.  The caller still allocates the graph
 * arrays (see mp_graph) and the inputs.
 *   Sizes: N and E whose mp_graph_build_workspace_size is at most
 *   MP_STATIC_WORKSPACE_BYTES (about 1.9 million edges when N <= E); larger
 *   ones return MP_ERR_WORKSPACE and launch nothing.
 *   Sharing: every call on one GPU uses that GPU's one array, and the work it
 *   enqueues is in flight until the stream reaches it.  Calls whose work
 *   overlaps on one GPU (enqueued on different streams without ordering, or
 *   from several threads) race on the array and corrupt each other's graphs;
 *   calls on one stream, or ordered by events, are safe.  The array's contents
 *   on entry are ignored (everything the lowering reads is written first).
 * Arguments, validation, results (bit for bit those of mp_graph_build) and
 * completion (mp_graph_finish, or compute calls reading the device record)
 * are those of mp_graph_build_async.
 */
#define MP_STATIC_WORKSPACE_BYTES 67108864u   /* 64 MiB */
mp_status mp_graph_build_noalloc(const void *src, const void *dst, mp_dtype idx_dtype,
                                 int64_t num_nodes, int64_t num_edges, mp_graph *g,
                                 void *stream);

/*
 * Complete an asynchronous build: synchronise `stream`, copy the class counts
 * from g->info into the descriptor and check the endpoints.  Returns MP_OK and
 * sets g->built = MP_GRAPH_BUILT, or MP_ERR_INDEX (and g->built = 0) when an
 * endpoint lay outside [0, N).  A graph that is already MP_GRAPH_BUILT is left
 * as it is (MP_OK); an unbuilt one gives MP_ERR_GRAPH.
 */
mp_status mp_graph_finish(mp_graph *g, void *stream);

/*
 * Forward aggregation Y = A_w X ("Decision"; the left column of the diagram
 * under "Edge order is explicit").
 *   w      [E] float32, COO order (may be NULL when E = 0).
 *   x      [N, H] of `x_dtype` (MP_F32 or MP_BF16); products and sums in fp32.
 *   y      [N, H] float32 output; must not overlap w, x or the graph arrays.
 * Enqueued on `stream`; does not synchronise.
 */
mp_status mp_spmm_fwd(const mp_graph *g, const float *w, const void *x, mp_dtype x_dtype,
                      int64_t h, float *y, void *stream);

/*
 * Input gradient dX = A_w^T dY over the transpose CSR ("Decision"; the right
 * column of the diagram under "Edge order is explicit").
 *   w      [E] float32, COO order (may be NULL when E = 0).
 *   dy     [N, H] of `dy_dtype` (MP_F32 or MP_BF16).
 *   dx     [N, H] float32 output; must not overlap w, dy or the graph arrays.
 */
mp_status mp_spmm_dx(const mp_graph *g, const float *w, const void *dy, mp_dtype dy_dtype,
                     int64_t h, float *dx, void *stream);

/*
 * Edge-weight gradient dw_e = <X[src_e, :], dY[dst_e, :]> for every edge, in
 * COO order, one owner per edge ("Decision"; the bottom of the diagram under
 * "Edge order is explicit").
 *   x, dy  [N, H] of `dtype` (MP_F32 or MP_BF16), same dtype for both.
 *   dw     [E] float32 output (may be NULL when E = 0); must not overlap x, dy
 *          or the graph arrays.
 */
mp_status mp_edge_grad_dw(const mp_graph *g, const void *x, const void *dy, mp_dtype dtype,
                          int64_t h, float *dw, void *stream);

/*
 * Both first-order gradients in one pass ("Decision": dX = A_w^T dY and
 * dw_e = <X[src_e, :], dY[dst_e, :]>).  The transpose CSR groups edges by
 * source, so the owner of row j holds X[j, :] while it gathers dY[dst, :] for
 * each of its edges; that one gathered row feeds both the dX accumulation and
 * the edge's dot product.  Results are exactly those of mp_spmm_dx followed by
 * mp_edge_grad_dw (bitwise, for H <= 64 x the 16-byte vector width, i.e. 256
 * fp32 or 512 bf16 features with 16-byte aligned arrays; wider or unaligned
 * rows run the two separate kernels).
 *   w      [E] float32, COO order (may be NULL when E = 0).
 *   x, dy  [N, H] of `dtype` (MP_F32 or MP_BF16).
 *   dx     [N, H] float32 output;  dw  [E] float32 output, COO order.
 *   Outputs must not overlap each other, the inputs or the graph arrays.
 */
mp_status mp_spmm_dx_edge_grad(const mp_graph *g, const float *w, const void *x, const void *dy,
                               mp_dtype dtype, int64_t h, float *dx, float *dw, void *stream);

/*
 * The same fused backward with the weights and their gradients interleaved in
 * one array, still in COO order ("Edge order is explicit"): wg[e * 2] holds
 * w_e (read) and wg[e * 2 + 1] receives dw_e (written; nothing else of wg is).
 * Each edge's weight and gradient then share a cache line, so the scattered
 * gradient store finds the line its weight load just brought into L2 instead
 * of writing a partial line of its own (on the power-law graph 6.65 against
 * 7.70 ms for the two-array call).  dX and dw are bitwise those of
 * mp_spmm_dx_edge_grad.  For callers that can keep a parameter and its
 * gradient side by side (e.g. torch views wg[:, 0] and wg[:, 1]).
 *   wg     [E][2] float32 (may be NULL when E = 0).
 *   x, dy  [N, H] of `dtype`;  dx  [N, H] float32 output.
 * Only for rows the fused kernel covers (H up to 64 lanes of 16-byte slices,
 * 16-byte aligned rows); other shapes return MP_ERR_SHAPE.  wg must not
 * overlap dx, x, dy or the graph arrays.
 */
mp_status mp_spmm_dx_edge_grad_pair(const mp_graph *g, float *wg, const void *x,
                                    const void *dy, mp_dtype dtype, int64_t h, float *dx,
                                    void *stream);

/*
 * The forward aggregation Y = A_w X of mp_spmm_fwd with the weights read from
 * the interleaved array of mp_spmm_dx_edge_grad_pair: wg[e * 2] holds w_e
 * (COO order, "Edge order is explicit"); nothing else of wg is read.  Y is
 * bitwise that of mp_spmm_fwd on the weights w_e.  With it, a training step
 * keeps one [E][2] array for a parameter and its gradient: this forward, then
 * mp_spmm_dx_edge_grad_pair, which writes dw_e into wg[e * 2 + 1].
 *   wg     [E][2] float32 (may be NULL when E = 0).
 *   x      [N, H] of `x_dtype` (MP_F32 or MP_BF16).   y  [N, H] float32 output.
 * Errors as mp_spmm_fwd; y must not overlap wg, x or the graph arrays.
 */
mp_status mp_spmm_fwd_pair(const mp_graph *g, const float *wg, const void *x, mp_dtype x_dtype,
                           int64_t h, float *y, void *stream);

/*
 * The aggregations with their longest rows split across workgroups, for graphs
 * where a few rows hold much of the edges (tinymesh "Weighted aggregation
 * experiment", "Limits": degree skew still weighs on both CSR directions).
 * A row of at least two chunks (a chunk is at least four of the chip's
 * E / 4096 edge shares, and at least 512 edges) is cut into chunks; each chunk's
 * partial row sum is written to the caller's workspace, and a second launch adds
 * each row's partials in chunk order into the output.  Every other row is
 * summed as in the plain calls, but with no row left to a 16-wave workgroup.
 * Results are deterministic (fixed chunks, fixed order, no atomics) and within
 * the plain calls' tolerance of the exact sums, but not bitwise equal to them
 * when a row is split; the split fused backward gives dX bitwise equal to
 * mp_spmm_dx_split and dw bitwise equal to mp_edge_grad_dw.  When no row is
 * long enough, each call is exactly its plain counterpart and needs no
 * workspace.
 *
 * mp_spmm_split_workspace_size: bytes of workspace (one float partial row of
 *   H per chunk item, for whichever CSR form needs more) that the split calls
 *   take for this graph and feature width; 0 when no row is split.  The graph
 *   must be finished (MP_GRAPH_BUILT: mp_graph_build, or mp_graph_finish after
 *   an asynchronous build), else MP_ERR_GRAPH.
 * The calls take the arguments of mp_spmm_fwd, mp_spmm_dx and
 *   mp_spmm_dx_edge_grad plus the workspace: device memory, 256-byte aligned,
 *   at least mp_spmm_split_workspace_size bytes (else MP_ERR_WORKSPACE /
 *   MP_ERR_ALIGN), overlapping no input, output or graph array (MP_ERR_ALIAS);
 *   it may be NULL when the size is 0.  Its contents on entry are ignored; calls
 *   that share one workspace must not overlap in time.  One weight per edge;
 *   finished graphs only.
 */
mp_status mp_spmm_split_workspace_size(const mp_graph *g, int64_t h, size_t *bytes);
mp_status mp_spmm_fwd_split(const mp_graph *g, const float *w, const void *x, mp_dtype x_dtype,
                            int64_t h, float *y, void *workspace, size_t workspace_bytes,
                            void *stream);
mp_status mp_spmm_dx_split(const mp_graph *g, const float *w, const void *dy, mp_dtype dy_dtype,
                           int64_t h, float *dx, void *workspace, size_t workspace_bytes,
                           void *stream);
mp_status mp_spmm_dx_edge_grad_split(const mp_graph *g, const float *w, const void *x,
                                     const void *dy, mp_dtype dtype, int64_t h, float *dx,
                                     float *dw, void *workspace, size_t workspace_bytes,
                                     void *stream);

/*
 * Multi-head edge weights.  tinymesh "Weighted aggregation experiment",
 * "Limits" lists vector edge weights among what the scalar experiment leaves
 * open; these calls take the per-head reading of it.  Each edge carries
 * `heads` = K weights, w[e * K + q] ([E, K] row-major, COO order), the feature
 * width H is a multiple of K, and head q owns columns [q*H/K, (q+1)*H/K) of
 * every feature row.  Head q of the output aggregates head q of the inputs
 * with weight w[e, q]:
 *   Y[i, c]  = sum over edges e into i   of w[e, q(c)] * X[src_e, c],
 *   dX[j, c] = sum over edges e out of j of w[e, q(c)] * dY[dst_e, c],
 *   dw[e, q] = sum over c in head q of X[src_e, c] * dY[dst_e, c],
 * q(c) = c / (H/K).  K = 1 is exactly the scalar call of the same name.  No
 * [E, H] intermediate is formed; the owners, layouts, tolerances and error
 * codes are those of the scalar calls, plus MP_ERR_SHAPE when K < 1 or K does
 * not divide H.  dw is [E, K] float32 in COO order.  The fused call gives dX
 * and dw bitwise equal to mp_spmm_dx_heads and mp_edge_grad_dw_heads under the
 * same condition as mp_spmm_dx_edge_grad (H within one column block, 16-byte
 * aligned rows whose heads are whole 16-byte lanes wide).
 */
mp_status mp_spmm_fwd_heads(const mp_graph *g, const float *w, int64_t heads, const void *x,
                            mp_dtype x_dtype, int64_t h, float *y, void *stream);
mp_status mp_spmm_dx_heads(const mp_graph *g, const float *w, int64_t heads, const void *dy,
                           mp_dtype dy_dtype, int64_t h, float *dx, void *stream);
mp_status mp_edge_grad_dw_heads(const mp_graph *g, const void *x, const void *dy,
                                mp_dtype dtype, int64_t h, int64_t heads, float *dw,
                                void *stream);
mp_status mp_spmm_dx_edge_grad_heads(const mp_graph *g, const float *w, int64_t heads,
                                     const void *x, const void *dy, mp_dtype dtype, int64_t h,
                                     float *dx, float *dw, void *stream);

/*
 * Target normalisation of scalar edge scores, the step a sparse attention layer
 * puts between learned scores and this aggregation ("Limits": scores
 * normalised over the edges of each target).  For every edge e with i = dst_e:
 *   alpha_e = exp(s_e - m_i) / z_i,
 *   m_i = max over the edges into i of s,
 *   z_i = sum over the edges into i of exp(s - m_i);
 * duplicate edges are separate terms; a row with no edges gets m = -inf and
 * z = 0.  Scores must be finite.  Row statistics are computed per destination
 * over the forward CSR (one owner per row, no atomics), alpha in COO order;
 * fp32 throughout.
 *   scores     [E] float32, COO order.    alpha  [E] float32 output, COO order.
 *   row_stats  [N][2] float32 output: (m_i, z_i) side by side, so the edge pass
 *              fetches both statistics of a row in one access.
 * Then Y = A_alpha X is mp_spmm_fwd(g, alpha, X, ...).
 */
mp_status mp_edge_softmax(const mp_graph *g, const float *scores, float *alpha, float *row_stats,
                          void *stream);

/*
 * The attention layer's forward, Y = A_alpha X with alpha = softmax(scores)
 * over each target ("Limits"), without writing alpha: the row statistics
 * pass of mp_edge_softmax, then the aggregation forms each edge's weight as
 * it fetches the score, exp(s_e - m_i) / z_i with the owner row's statistics,
 * in the same fp32 operations as mp_edge_softmax forms alpha.  Y and
 * row_stats are bit for bit those of mp_edge_softmax followed by mp_spmm_fwd
 * on its alpha.  For inference, or with a backward that recomputes alpha; the
 * one-call attention backward takes alpha itself.
 *   scores     [E] float32, COO order (one head).
 *   x          [N, H] of x_dtype (MP_F32 or MP_BF16).   h = H.
 *   y          [N, H] float32 output.
 *   row_stats  [N][2] float32 output, 8-byte aligned: (m_i, z_i) as in
 *              mp_edge_softmax.
 * Errors as mp_spmm_fwd, plus MP_ERR_NULL / MP_ERR_ALIGN / MP_ERR_DEVICE for
 * row_stats and MP_ERR_ALIAS when it overlaps an input, y or the graph arrays.
 */
mp_status mp_spmm_fwd_softmax(const mp_graph *g, const float *scores, const void *x,
                              mp_dtype x_dtype, int64_t h, float *y, float *row_stats,
                              void *stream);

/*
 * Backward of mp_edge_softmax: given alpha and the upstream gradient dalpha
 * (for the attention layer, dalpha = mp_edge_grad_dw(g, X, dY) or the dw of
 * mp_spmm_dx_edge_grad), writes
 *   dscores_e = alpha_e * (dalpha_e - row_dot[dst_e]),
 *   row_dot[i] = sum over the edges into i of alpha * dalpha.
 * dscores first holds the products alpha * dalpha (one coalesced pass), so the
 * per-row sums gather one value per edge instead of two.
 *   alpha, dalpha  [E] float32, COO order.   dscores  [E] float32 output.
 *   row_dot  [N] float32 output.
 */
mp_status mp_edge_softmax_backward(const mp_graph *g, const float *alpha, const float *dalpha,
                                   float *dscores, float *row_dot, void *stream);

/*
 * Multi-head scores, for a multi-head attention layer over the multi-head
 * aggregation above: each edge carries `heads` = K scores, scores[e * K + q]
 * ([E, K] row-major, COO order), and every head is normalised on its own, as
 * mp_edge_softmax does for one ("Limits": scores normalised over each target;
 * the per-head reading of vector edge values).  alpha and dscores are [E, K];
 * row_stats is [N][K][2] (maximum, sum) and row_dot [N, K].  K = 1 is exactly
 * the single-head call.  MP_ERR_SHAPE for K outside [1, 2^20].
 */
mp_status mp_edge_softmax_heads(const mp_graph *g, const float *scores, int64_t heads,
                                float *alpha, float *row_stats, void *stream);
mp_status mp_edge_softmax_backward_heads(const mp_graph *g, const float *alpha,
                                         const float *dalpha, int64_t heads, float *dscores,
                                         float *row_dot, void *stream);

/*
 * Whole backward of the attention layer Y = A_alpha X with alpha =
 * softmax(scores) over each target ("Limits"; per head when heads > 1), in one
 * walk of the transpose CSR instead of an input gradient, an edge gradient and
 * a softmax backward one after another.  It rests on the identity
 *   sum over the edges e into i of alpha_e <X[src_e], dY[i]> = <Y[i], dY[i]>
 * (over head q's columns with K heads), so the row term of the softmax
 * backward is a row-wise dot product of the kept forward output with dY, and
 * each edge's score gradient is written where its dalpha is formed:
 *   row_dot[i * K + q]   = <Y[i], dY[i]> over head q's columns,
 *   dX                   = A_alpha^T dY            (as mp_spmm_dx_heads),
 *   dscores[e * K + q]   = alpha[e * K + q] (<X[src_e], dY[dst_e]>_q - row_dot[dst_e * K + q]).
 * Equal, up to rounding order, to mp_spmm_dx_edge_grad_heads followed by
 * mp_edge_softmax_backward_heads; row_dot is the same quantity computed the
 * other way.
 *   alpha    [E, K] float32, COO order: the softmax weights the forward used.
 *   x, dy    [N, H] of `dtype` (MP_F32 or MP_BF16).   h = H, a multiple of K.
 *   y        [N, H] float32: the forward output A_alpha X for these alpha and x.
 *   dx       [N, H] float32 output.   dscores  [E, K] float32 output, COO order.
 *   row_dot  [N, K] float32 output.
 * dscores may be alpha itself: the score gradients are then written over the
 * weights (each edge's alpha is read once, by the lanes that then write its
 * score gradient), and the store finds the line its alpha load brought into
 * L2 (on the power-law graph 7.24 against 8.26 ms).  Otherwise no output may
 * overlap an input, another output or the graph arrays (MP_ERR_ALIAS).
 * Feature rows wider than one column block take the unfused path (dX, the
 * edge gradients into dscores, then the score gradient in place), with the
 * same results up to rounding order; there dscores may not be alpha.
 */
mp_status mp_attention_backward(const mp_graph *g, const float *alpha, int64_t heads,
                                const void *x, const void *dy, const float *y, mp_dtype dtype,
                                int64_t h, float *dx, float *dscores, float *row_dot,
                                void *stream);

/*
 * mp_attention_backward for one head with alpha never stored: given the scores
 * and the row statistics of mp_spmm_fwd_softmax (or mp_edge_softmax), the
 * transpose walk forms each edge's alpha_e = exp(s_e - m_dst) / z_dst from its
 * score and its destination's statistics, in the fp32 operations the softmax
 * forms alpha, then proceeds as mp_attention_backward.  Its outputs are bit
 * for bit those of mp_attention_backward given that alpha.
 *   scores     [E] float32, COO order.   row_stats  [N][2] float32, 8-byte aligned.
 *   x, dy, y, h, dtype, dx, dscores, row_dot as mp_attention_backward (K = 1).
 * dscores may be scores itself (written over them).  Feature rows must fit the
 * fused walk (H up to 64 lanes of 16-byte slices), else MP_ERR_SHAPE; other
 * errors as mp_attention_backward, and MP_ERR_NULL / MP_ERR_ALIGN /
 * MP_ERR_DEVICE / MP_ERR_ALIAS for row_stats.
 */
mp_status mp_attention_backward_scores(const mp_graph *g, const float *scores,
                                       const float *row_stats, const void *x, const void *dy,
                                       const float *y, mp_dtype dtype, int64_t h, float *dx,
                                       float *dscores, float *row_dot, void *stream);

/* Normalisation modes for mp_edge_normalize. */
#define MP_NORM_MEAN 1
#define MP_NORM_SYM  2

/*
 * Degree normalisation of per-edge values, in COO order, for mean and
 * symmetric-normalised aggregation ("PyTorch Geometric: one abstraction, the
 * whole GNN literature", Step 3: GCN's normalised adjacency and SAGE's mean,
 * each followed by one SpMM).  Degrees are edge counts taken from the two CSR
 * row pointers (duplicates and self-loops counted):
 *   MP_NORM_MEAN:  out_e = in_e / deg_in(dst_e)
 *   MP_NORM_SYM:   out_e = in_e / sqrt(deg_out(src_e) * deg_in(dst_e))
 * Forward: mp_spmm_fwd(g, normalize(w), X).  Backward: dX through the same
 * normalised weights, and the weight gradient is normalize(dw') where dw' is
 * the edge gradient (the factor is constant in w).  fp32 in and out; the
 * factor is formed in double and rounded once.  `out` may equal `in` (the map
 * is elementwise) but must not overlap it otherwise, nor the graph arrays.
 *   in, out  [E] float32, COO order.   mode  MP_NORM_MEAN or MP_NORM_SYM.
 */
mp_status mp_edge_normalize(const mp_graph *g, int32_t mode, const float *in, float *out,
                            void *stream);

/*
 * The same normalisation applied to each weight as the aggregation fetches it
 * (Step 3's normalised adjacency without a separate pass over the weights):
 * every edge's weight is used as w_e * (float)c_e, with c_e formed in double
 * exactly as mp_edge_normalize forms it, so each call returns bit for bit what
 * mp_edge_normalize followed by the plain call returns.
 *   mp_spmm_fwd_norm           Y  = A_{norm(w)} X        (as mp_spmm_fwd)
 *   mp_spmm_dx_norm            dX = A_{norm(w)}^T dY     (as mp_spmm_dx)
 *   mp_spmm_dx_edge_grad_norm  dX as above and dw_e = c_e <X[src_e], dY[dst_e]>,
 *                              the gradient with respect to the raw weights
 *                              (as mp_spmm_dx_edge_grad, then mp_edge_normalize
 *                              of its dw).
 * In the forward walk deg_in(dst) is the owner row's length, so MP_NORM_MEAN
 * reads nothing extra there; the other cases read the gathered endpoint's row
 * length, one 8-byte random read per edge.  One weight per edge (no heads).
 * Arguments and errors as the plain calls, plus MP_ERR_DTYPE for an unknown
 * mode.
 */
mp_status mp_spmm_fwd_norm(const mp_graph *g, int32_t mode, const float *w, const void *x,
                           mp_dtype x_dtype, int64_t h, float *y, void *stream);
mp_status mp_spmm_dx_norm(const mp_graph *g, int32_t mode, const float *w, const void *dy,
                          mp_dtype dy_dtype, int64_t h, float *dx, void *stream);
mp_status mp_spmm_dx_edge_grad_norm(const mp_graph *g, int32_t mode, const float *w,
                                    const void *x, const void *dy, mp_dtype dtype, int64_t h,
                                    float *dx, float *dw, void *stream);

/*
 * Owner sizes of the aggregation kernels, for tests and tuning only.  Every
 * aggregation (forward, input gradient, fused backward, and their multi-head,
 * normalised and attention forms) hands each row to an owner -- a lane group,
 * one wave, or a workgroup -- by a rule taken from E, the feature width and
 * the degree classes of the graph.  These values replace the rule's results
 * for every later call in the process:
 *   hub_min_len   rows at least this long get a workgroup (<= 0: the rule's)
 *   hub_apart     1: those workgroups have 16 waves and run in a launch of
 *                 their own; 0: four waves, inside the main launch
 *                 (< 0: the rule's; > 1 is MP_ERR_SHAPE)
 *   wave_min_len  rows at least this long (and below hub_min_len) get one
 *                 wave (<= 0: four lane-group steps, the default)
 * Results stay within the same tolerance of the exact sums, but rows summed
 * by other owners round differently, so bits are reproducible only for the
 * same overrides.  mp_set_owner_overrides(-1, -1, -1) restores the rule.  The
 * setting is process-wide; set it while no compute call is being enqueued.
 */
mp_status mp_set_owner_overrides(int32_t hub_min_len, int32_t hub_apart, int32_t wave_min_len);

/* Static text for a status code. */
const char *mp_status_string(mp_status status);

/* Thread-local detail for the last non-OK status returned on this thread. */
const char *mp_last_error_detail(void);

/* Library version, as major * 10000 + minor * 100 + patch. */
int32_t mp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MP_H */
