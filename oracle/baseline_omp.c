/*
 * baseline_omp.c -- the CPU baseline of the benchmark on all host cores.
 *
 * BENCHMARK INFRASTRUCTURE ONLY, and not part of the checker: no test compares
 * against it and nothing in the library links, loads or calls it.  The
 * benchmark's cpu_baseline leg times it beside the single-threaded oracle
 * (oracle.c) to say what the same fp64 arithmetic costs on every host core.
 *
 * It computes what oracle.c computes, from the same definitions (tinymesh
 * "Weighted aggregation experiment": "Decision" and "Edge order is explicit"):
 *   - the stable counting-sort lowering, serial, exactly as oracle.c does it;
 *   - Y[i, :] = sum over the edges e into i of w_e X[src_e, :], and
 *     dX[j, :] = sum over the edges e out of j of w_e dY[dst_e, :], each as one
 *     OpenMP loop over the rows of that CSR form (each row owned by one thread,
 *     its edges taken in CSR order, i.e. ascending COO ordinal);
 *   - dw_e = <X[src_e, :], dY[dst_e, :]> as one OpenMP loop over the edges;
 * all in fp64, with the same |term| sums S beside every output as oracle.c.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include <omp.h>

int baseline_threads(void) { return omp_get_max_threads(); }

/* Stable counting sort keyed on `key` (serial): rowptr[n+1], col[e], order[e]. */
int baseline_lower(int64_t n, int64_t e, const int64_t *key, const int64_t *other,
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
        rowptr[key[j] + 1] += 1;
    for (i = 0; i < n; i++)
        rowptr[i + 1] += rowptr[i];
    cursor = (int64_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof(int64_t));
    if (!cursor)
        return -2;
    for (i = 0; i < n; i++)
        cursor[i] = rowptr[i];
    for (j = 0; j < e; j++) {
        int64_t p = cursor[key[j]];
        cursor[key[j]] = p + 1;
        order[p] = j;
        col[p] = other[j];
    }
    free(cursor);
    return 0;
}

/* out[i, :] = sum over p in row i of w[order[p]] * in[col[p], :], one row per
 * thread at a time (dynamic schedule: row lengths are skewed). */
void baseline_aggregate(int64_t n, int64_t h, const int64_t *rowptr, const int64_t *col,
                        const int64_t *order, const float *w, const float *in, double *out,
                        double *s)
{
    int64_t i;
#pragma omp parallel for schedule(dynamic, 256)
    for (i = 0; i < n; i++) {
        int64_t p, k;
        double *yo = out + i * h, *so = s + i * h;
        for (k = 0; k < h; k++) {
            yo[k] = 0.0;
            so[k] = 0.0;
        }
        for (p = rowptr[i]; p < rowptr[i + 1]; p++) {
            const double wp = (double)w[order[p]];
            const float *xr = in + col[p] * h;
            for (k = 0; k < h; k++) {
                double t = wp * (double)xr[k];
                yo[k] += t;
                so[k] += fabs(t);
            }
        }
    }
}

/* dw_e = <x[src_e], dy[dst_e]> for every edge, COO order. */
void baseline_edge_grad(int64_t e, int64_t h, const int64_t *src, const int64_t *dst,
                        const float *x, const float *dy, double *dw, double *s)
{
    int64_t j;
#pragma omp parallel for schedule(static)
    for (j = 0; j < e; j++) {
        int64_t k;
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
