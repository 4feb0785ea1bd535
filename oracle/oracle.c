/*
 * oracle.c -- plain, slow, obviously correct CPU model of weighted sparse
 * message passing over a fixed COO topology.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or constant with
 * the HIP library: it is written from the pages' definitions alone.
 *
 * Sources (cited by page title and section):
 *   [W] tinymesh, "Weighted aggregation experiment":
 *       "Decision"             -- forward Y = A_w X over destination-owned CSR,
 *                                  input gradient dX = A_w^T dY, edge gradient
 *                                  dw_e = <X[source_e], dY[target_e]>;
 *       "Edge order is explicit" -- the two order maps send a CSR position to
 *                                  the original COO ordinal, weights and dw stay
 *                                  in COO order, duplicates keep their own
 *                                  positions;
 *       "Exact witness"        -- edge_order = (2, 0, 1) on the 3-edge fixture.
 *   [P] "PyTorch Geometric: one abstraction, the whole GNN literature",
 *       Step 2 (the COO edge loop: gather the source row, scale it, add it into
 *       the destination row) -- this file runs that loop without materialising
 *       the per-edge message rows.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - A_w[dst, src] += w_e, so CSR rows are destinations (fixed by the witness:
 *     Y = (0, 6, 0)).
 *   - Inside a CSR row, positions follow ascending COO ordinal (a stable sort
 *     keyed on the row index alone).
 *   - N is given explicitly; N >= 1, E >= 0; self-loops and duplicates allowed.
 *   - Outputs are overwritten; a row with no edges is exactly zero.
 *
 * Arithmetic: indices are int64; feature and weight inputs arrive as float
 * (the exact values the device receives, bf16 already widened exactly by the
 * caller) and every product and sum is taken in double.  Beside each float
 * output the oracle returns S = sum of |term| over the same terms, the scale
 * that the parity tolerance is relative to.
 *
 * Pins: tests/test_oracle.py checks every function here against the printed
 * witness, dense brute force, scipy.sparse, numpy's stable argsort, closed-form
 * laws (adjoint identity, permutation, duplicates, linearity) and hand values;
 * tests/test_oracle_mutants.py shows that planted mistakes fail those pins.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

/* ------------------------------------------------------------------------- */
/* Lowering: COO -> CSR keyed on `key`, with the position -> ordinal map.      */
/* [W] "Edge order is explicit": edge_order[p] is the COO ordinal stored at CSR */
/* position p; duplicates keep separate positions.  Stable counting sort:      */
/* count each row, prefix-sum the counts into row pointers, then walk the      */
/* edges in ascending ordinal and drop each one into the next free slot of its */
/* row.  col[p] = other[order[p]].                                             */
/* Returns 0, or -1 if a key lies outside [0, n).                              */
/* ------------------------------------------------------------------------- */
int oracle_lower(int64_t n, int64_t e, const int64_t *key, const int64_t *other,
                 int64_t *rowptr, int64_t *col, int64_t *order)
{
    int64_t i, j;
    int64_t *cursor;

    for (j = 0; j < e; j++)
        if (key[j] < 0 || key[j] >= n)
            return -1;

    for (i = 0; i <= n; i++)
        rowptr[i] = 0;
    for (j = 0; j < e; j++)
        rowptr[key[j] + 1] += 1;            /* row lengths, shifted by one */
    for (i = 0; i < n; i++)
        rowptr[i + 1] += rowptr[i];          /* inclusive sum = row starts  */

    cursor = (int64_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof(int64_t));
    if (!cursor)
        return -2;
    for (i = 0; i < n; i++)
        cursor[i] = rowptr[i];
    for (j = 0; j < e; j++) {               /* ascending COO ordinal       */
        int64_t p = cursor[key[j]];
        cursor[key[j]] = p + 1;
        order[p] = j;
        col[p] = other[j];
    }
    free(cursor);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Forward aggregation, [W] "Decision" and the left column of the diagram in   */
/* "Edge order is explicit":  Y = A_w X  with  A_w[dst_e, src_e] += w_e, i.e.  */
/*   Y[i, :] = sum over edges e with dst_e = i of  w_e * X[src_e, :].          */
/* Written as the plain edge loop of [P] Step 2, accumulating straight into Y. */
/* ------------------------------------------------------------------------- */
void oracle_forward(int64_t n, int64_t e, int64_t h,
                    const int64_t *src, const int64_t *dst, const float *w,
                    const float *x, double *y, double *s)
{
    int64_t j, k;
    for (j = 0; j < n * h; j++) {
        y[j] = 0.0;
        s[j] = 0.0;
    }
    for (j = 0; j < e; j++) {
        for (k = 0; k < h; k++) {
            double t = (double)w[j] * (double)x[src[j] * h + k];
            y[dst[j] * h + k] += t;
            s[dst[j] * h + k] += fabs(t);
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Input gradient, [W] "Decision" and the right column of the diagram:         */
/*   dX = A_w^T dY,  i.e.  dX[j, :] = sum over edges e with src_e = j of       */
/*                                    w_e * dY[dst_e, :].                      */
/* ------------------------------------------------------------------------- */
void oracle_input_grad(int64_t n, int64_t e, int64_t h,
                       const int64_t *src, const int64_t *dst, const float *w,
                       const float *dy, double *dx, double *s)
{
    int64_t j, k;
    for (j = 0; j < n * h; j++) {
        dx[j] = 0.0;
        s[j] = 0.0;
    }
    for (j = 0; j < e; j++) {
        for (k = 0; k < h; k++) {
            double t = (double)w[j] * (double)dy[dst[j] * h + k];
            dx[src[j] * h + k] += t;
            s[src[j] * h + k] += fabs(t);
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Edge-weight gradient, [W] "Decision" and the bottom of the diagram:         */
/*   dw_e = sum over h of X[src_e, h] * dY[dst_e, h]     (COO order).          */
/* ------------------------------------------------------------------------- */
void oracle_edge_grad(int64_t e, int64_t h,
                      const int64_t *src, const int64_t *dst,
                      const float *x, const float *dy, double *dw, double *s)
{
    int64_t j, k;
    for (j = 0; j < e; j++) {
        double acc = 0.0, sa = 0.0;
        for (k = 0; k < h; k++) {
            double t = (double)x[src[j] * h + k] * (double)dy[dst[j] * h + k];
            acc += t;
            sa += fabs(t);
        }
        dw[j] = acc;
        s[j] = sa;
    }
}

/* ------------------------------------------------------------------------- */
/* Row-sampled forms of the two aggregations, for graphs too large to hold     */
/* the full fp64 output: the same definitions evaluated only for the rows      */
/* listed in `rows` (distinct, in [0, n)).  One pass over all edges in COO     */
/* order; an edge contributes iff its owning row is listed.                    */
/* ------------------------------------------------------------------------- */
static int64_t *slot_table(int64_t n, int64_t nr, const int64_t *rows)
{
    int64_t i;
    int64_t *slot = (int64_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof(int64_t));
    if (!slot)
        return NULL;
    for (i = 0; i < n; i++)
        slot[i] = -1;
    for (i = 0; i < nr; i++)
        slot[rows[i]] = i;
    return slot;
}

int oracle_forward_rows(int64_t n, int64_t e, int64_t h,
                        const int64_t *src, const int64_t *dst, const float *w,
                        const float *x, int64_t nr, const int64_t *rows,
                        double *y, double *s)
{
    int64_t j, k;
    int64_t *slot = slot_table(n, nr, rows);
    if (!slot)
        return -2;
    for (j = 0; j < nr * h; j++) {
        y[j] = 0.0;
        s[j] = 0.0;
    }
    for (j = 0; j < e; j++) {
        int64_t r = slot[dst[j]];
        if (r < 0)
            continue;
        for (k = 0; k < h; k++) {
            double t = (double)w[j] * (double)x[src[j] * h + k];
            y[r * h + k] += t;
            s[r * h + k] += fabs(t);
        }
    }
    free(slot);
    return 0;
}

int oracle_input_grad_rows(int64_t n, int64_t e, int64_t h,
                           const int64_t *src, const int64_t *dst, const float *w,
                           const float *dy, int64_t nr, const int64_t *rows,
                           double *dx, double *s)
{
    int64_t j, k;
    int64_t *slot = slot_table(n, nr, rows);
    if (!slot)
        return -2;
    for (j = 0; j < nr * h; j++) {
        dx[j] = 0.0;
        s[j] = 0.0;
    }
    for (j = 0; j < e; j++) {
        int64_t r = slot[src[j]];
        if (r < 0)
            continue;
        for (k = 0; k < h; k++) {
            double t = (double)w[j] * (double)dy[dst[j] * h + k];
            dx[r * h + k] += t;
            s[r * h + k] += fabs(t);
        }
    }
    free(slot);
    return 0;
}

/* Edge gradient for a list of COO ordinals only. */
void oracle_edge_grad_edges(int64_t h, int64_t ne, const int64_t *edges,
                            const int64_t *src, const int64_t *dst,
                            const float *x, const float *dy, double *dw, double *s)
{
    int64_t i, k;
    for (i = 0; i < ne; i++) {
        int64_t j = edges[i];
        double acc = 0.0, sa = 0.0;
        for (k = 0; k < h; k++) {
            double t = (double)x[src[j] * h + k] * (double)dy[dst[j] * h + k];
            acc += t;
            sa += fabs(t);
        }
        dw[i] = acc;
        s[i] = sa;
    }
}

/* ------------------------------------------------------------------------- */
/* Degree plan.  [W] "Limits" notes that degree skew still affects both CSR     */
/* directions; the library answers it by visiting rows grouped by degree class. */
/* The class of a row of length d is 0 for d = 0, else the number of binary    */
/* digits of d (1 for d = 1, 2 for 2..3, 3 for 4..7, ...).  The plan lists the */
/* rows by class, highest first, ascending row id within a class, and counts   */
/* the rows of each class (33 classes, 0..32).                                 */
/* ------------------------------------------------------------------------- */
void oracle_degree_plan(int64_t n, const int64_t *rowptr, int64_t *perm,
                        int64_t *class_count)
{
    int64_t i, c, p = 0;
    for (c = 0; c <= 32; c++)
        class_count[c] = 0;
    for (i = 0; i < n; i++) {
        int64_t d = rowptr[i + 1] - rowptr[i];
        int64_t k = 0;
        while (d > 0) {
            k += 1;
            d /= 2;
        }
        class_count[k] += 1;
    }
    for (c = 32; c >= 0; c--) {              /* highest class first          */
        if (class_count[c] == 0)
            continue;
        for (i = 0; i < n; i++) {            /* ascending row id inside      */
            int64_t d = rowptr[i + 1] - rowptr[i];
            int64_t k = 0;
            while (d > 0) {
                k += 1;
                d /= 2;
            }
            if (k == c)
                perm[p++] = i;
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Target normalisation of scalar edge scores ([W] "Limits": a sparse          */
/* attention step puts learned scalar scores through a normalisation over the  */
/* edges of each target before this aggregation).  Plain definition, a softmax */
/* over the incoming edges of each destination:                                 */
/*   alpha_e = exp(s_e - m_i) / z_i,  m_i = max over e' into i of s_e',        */
/*   z_i = sum over e' into i of exp(s_e' - m_i),   i = dst_e.                 */
/* Duplicates are separate terms.  Row statistics m_i, z_i are returned too    */
/* (m_i = -inf and z_i = 0 for a row with no edges).                           */
/* ------------------------------------------------------------------------- */
void oracle_edge_softmax(int64_t n, int64_t e, const int64_t *dst, const float *s,
                         double *alpha, double *row_max, double *row_sum)
{
    int64_t i, j;
    for (i = 0; i < n; i++) {
        row_max[i] = -INFINITY;
        row_sum[i] = 0.0;
    }
    for (j = 0; j < e; j++)
        if ((double)s[j] > row_max[dst[j]])
            row_max[dst[j]] = (double)s[j];
    for (j = 0; j < e; j++)
        row_sum[dst[j]] += exp((double)s[j] - row_max[dst[j]]);
    for (j = 0; j < e; j++)
        alpha[j] = exp((double)s[j] - row_max[dst[j]]) / row_sum[dst[j]];
}

/* ------------------------------------------------------------------------- */
/* Backward of the target softmax: with upstream gradient dalpha_e,            */
/*   ds_e = alpha_e * (dalpha_e - t_i),  t_i = sum over e' into i of           */
/*                                             alpha_e' * dalpha_e'.           */
/* (the Jacobian of a softmax applied row by row).  S_e = alpha_e * (|dalpha_e| */
/* + sum over e' into i of alpha_e' |dalpha_e'|) is the scale of each term.    */
/* ------------------------------------------------------------------------- */
void oracle_edge_softmax_backward(int64_t n, int64_t e, const int64_t *dst,
                                  const float *alpha, const float *dalpha,
                                  double *ds, double *row_dot, double *s_scale)
{
    int64_t i, j;
    double *row_abs = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    for (i = 0; i < n; i++) {
        row_dot[i] = 0.0;
        row_abs[i] = 0.0;
    }
    for (j = 0; j < e; j++) {
        row_dot[dst[j]] += (double)alpha[j] * (double)dalpha[j];
        row_abs[dst[j]] += fabs((double)alpha[j] * (double)dalpha[j]);
    }
    for (j = 0; j < e; j++) {
        ds[j] = (double)alpha[j] * ((double)dalpha[j] - row_dot[dst[j]]);
        s_scale[j] = fabs((double)alpha[j]) * (fabs((double)dalpha[j]) + row_abs[dst[j]]);
    }
    free(row_abs);
}

/* ------------------------------------------------------------------------- */
/* Degree normalisation of edge values, for mean and symmetric-normalised     */
/* aggregation ([P] Step 3: GCN builds a normalised adjacency before its       */
/* single SpMM, SAGE aggregates a mean; [P] "Done when": sum and mean are the  */
/* reductions that keep gradients).  Degrees are edge counts (duplicates and   */
/* self-loops counted): deg_in(i) = edges ending at i, deg_out(j) = edges      */
/* leaving j.                                                                   */
/*   mode 1 (mean):      out_e = in_e / deg_in(dst_e)                           */
/*   mode 2 (symmetric): out_e = in_e / sqrt(deg_out(src_e) * deg_in(dst_e))    */
/* The same scaling maps a weight gradient dL/dw' back to dL/dw (w' = c w).   */
/* Returns -1 for an unknown mode.                                              */
/* ------------------------------------------------------------------------- */
int oracle_edge_normalize(int64_t n, int64_t e, const int64_t *src, const int64_t *dst,
                          int mode, const float *in, double *out)
{
    int64_t i, j;
    double *din = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    double *dout = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    if (mode != 1 && mode != 2) {
        free(din);
        free(dout);
        return -1;
    }
    for (i = 0; i < n; i++) {
        din[i] = 0.0;
        dout[i] = 0.0;
    }
    for (j = 0; j < e; j++) {
        din[dst[j]] += 1.0;
        dout[src[j]] += 1.0;
    }
    for (j = 0; j < e; j++) {
        if (mode == 1)
            out[j] = (double)in[j] / din[dst[j]];
        else
            out[j] = (double)in[j] / sqrt(dout[src[j]] * din[dst[j]]);
    }
    free(din);
    free(dout);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Multi-head edge weights.  [W] "Limits" lists vector edge weights among the  */
/* cases its scalar experiment does not cover; the plainest reading, used      */
/* here, is the per-head form of the same aggregation: the feature width h is  */
/* split into k heads of h/k contiguous columns, edge e carries one weight per */
/* head, w[e*k + q] (edge-major, COO order), and head q of every output row    */
/* aggregates only head q of the input rows:                                    */
/*   Y[i, c]  = sum over e with dst_e = i of  w[e, q(c)] * X[src_e, c]          */
/*   dX[j, c] = sum over e with src_e = j of  w[e, q(c)] * dY[dst_e, c]         */
/*   dw[e, q] = sum over c in head q of  X[src_e, c] * dY[dst_e, c]             */
/* with q(c) = c / (h/k).  k = 1 is the scalar case above.  h must be a        */
/* multiple of k.  `rows` (nr entries, distinct, in [0, n)) or `edges` (ne COO  */
/* ordinals) restrict the outputs to a sample; NULL means every row / edge.    */
/* Returns 0, -1 if h is not a multiple of k, -2 on allocation failure.        */
/* ------------------------------------------------------------------------- */
static int heads_aggregate(int64_t n, int64_t e, int64_t h, int64_t k,
                           const int64_t *owner, const int64_t *other, const float *w,
                           const float *in, int64_t nr, const int64_t *rows,
                           double *out, double *s)
{
    int64_t j, c, r, hh, nout;
    int64_t *slot = NULL;
    if (k < 1 || h % k != 0)
        return -1;
    hh = h / k;
    nout = rows ? nr : n;
    if (rows) {
        slot = slot_table(n, nr, rows);
        if (!slot)
            return -2;
    }
    for (j = 0; j < nout * h; j++) {
        out[j] = 0.0;
        s[j] = 0.0;
    }
    for (j = 0; j < e; j++) {
        r = rows ? slot[owner[j]] : owner[j];
        if (r < 0)
            continue;
        for (c = 0; c < h; c++) {
            double t = (double)w[j * k + c / hh] * (double)in[other[j] * h + c];
            out[r * h + c] += t;
            s[r * h + c] += fabs(t);
        }
    }
    free(slot);
    return 0;
}

int oracle_forward_heads(int64_t n, int64_t e, int64_t h, int64_t k,
                         const int64_t *src, const int64_t *dst, const float *w,
                         const float *x, int64_t nr, const int64_t *rows,
                         double *y, double *s)
{
    /* rows are destinations; the gathered row is the source's */
    return heads_aggregate(n, e, h, k, dst, src, w, x, nr, rows, y, s);
}

int oracle_input_grad_heads(int64_t n, int64_t e, int64_t h, int64_t k,
                            const int64_t *src, const int64_t *dst, const float *w,
                            const float *dy, int64_t nr, const int64_t *rows,
                            double *dx, double *s)
{
    /* rows are sources; the gathered row is the destination's */
    return heads_aggregate(n, e, h, k, src, dst, w, dy, nr, rows, dx, s);
}

int oracle_edge_grad_heads(int64_t e, int64_t h, int64_t k,
                           const int64_t *src, const int64_t *dst,
                           const float *x, const float *dy, int64_t ne, const int64_t *edges,
                           double *dw, double *s)
{
    int64_t i, q, c, hh, count;
    if (k < 1 || h % k != 0)
        return -1;
    hh = h / k;
    count = edges ? ne : e;
    for (i = 0; i < count; i++) {
        int64_t j = edges ? edges[i] : i;
        for (q = 0; q < k; q++) {
            double acc = 0.0, sa = 0.0;
            for (c = q * hh; c < (q + 1) * hh; c++) {
                double t = (double)x[src[j] * h + c] * (double)dy[dst[j] * h + c];
                acc += t;
                sa += fabs(t);
            }
            dw[i * k + q] = acc;
            s[i * k + q] = sa;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Multi-head scores: edge e carries one score per head, s[e*k + q] ([e, k],   */
/* COO order), and each head is normalised on its own over the edges of each   */
/* target -- the target softmax above applied to every head's column, the     */
/* scores of a multi-head attention layer feeding the multi-head aggregation. */
/* Row statistics are [n, k] (row_max[i*k + q], row_sum[i*k + q]).             */
/* ------------------------------------------------------------------------- */
void oracle_edge_softmax_heads(int64_t n, int64_t e, int64_t k, const int64_t *dst,
                               const float *s, double *alpha, double *row_max,
                               double *row_sum)
{
    int64_t i, j, q;
    for (i = 0; i < n * k; i++) {
        row_max[i] = -INFINITY;
        row_sum[i] = 0.0;
    }
    for (j = 0; j < e; j++)
        for (q = 0; q < k; q++)
            if ((double)s[j * k + q] > row_max[dst[j] * k + q])
                row_max[dst[j] * k + q] = (double)s[j * k + q];
    for (j = 0; j < e; j++)
        for (q = 0; q < k; q++)
            row_sum[dst[j] * k + q] += exp((double)s[j * k + q] - row_max[dst[j] * k + q]);
    for (j = 0; j < e; j++)
        for (q = 0; q < k; q++)
            alpha[j * k + q] = exp((double)s[j * k + q] - row_max[dst[j] * k + q])
                               / row_sum[dst[j] * k + q];
}

/* Backward per head: ds[e,q] = alpha[e,q] (dalpha[e,q] - t[dst_e,q]),         */
/* t[i,q] = sum over e into i of alpha[e,q] dalpha[e,q]; S as for one head.    */
void oracle_edge_softmax_backward_heads(int64_t n, int64_t e, int64_t k, const int64_t *dst,
                                        const float *alpha, const float *dalpha,
                                        double *ds, double *row_dot, double *s_scale)
{
    int64_t i, j, q;
    double *row_abs = (double *)malloc((size_t)(n * k > 0 ? n * k : 1) * sizeof(double));
    for (i = 0; i < n * k; i++) {
        row_dot[i] = 0.0;
        row_abs[i] = 0.0;
    }
    for (j = 0; j < e; j++)
        for (q = 0; q < k; q++) {
            double t = (double)alpha[j * k + q] * (double)dalpha[j * k + q];
            row_dot[dst[j] * k + q] += t;
            row_abs[dst[j] * k + q] += fabs(t);
        }
    for (j = 0; j < e; j++)
        for (q = 0; q < k; q++) {
            int64_t r = dst[j] * k + q;
            ds[j * k + q] = (double)alpha[j * k + q] * ((double)dalpha[j * k + q] - row_dot[r]);
            s_scale[j * k + q] = fabs((double)alpha[j * k + q])
                                 * (fabs((double)dalpha[j * k + q]) + row_abs[r]);
        }
    free(row_abs);
}
