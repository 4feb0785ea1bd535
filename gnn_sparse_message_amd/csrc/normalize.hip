// normalize.hip -- degree normalisation of per-edge values in COO order, for
// mean and symmetric-normalised aggregation ("PyTorch Geometric: one
// abstraction, the whole GNN literature", Step 3: GCN aggregates with a
// normalised adjacency, SAGE with a mean; sum and mean are the reductions
// that keep gradients, "Done when").  With deg_in(i) = rowptr[i+1] - rowptr[i]
// and deg_out(j) = rowptr_t[j+1] - rowptr_t[j] (edge counts):
//   MP_NORM_MEAN: out_e = in_e / deg_in(dst_e)
//   MP_NORM_SYM:  out_e = in_e / sqrt(deg_out(src_e) * deg_in(dst_e))
// The scale factor is formed in double (the degree product is exact there),
// rounded once to fp32, and applied with one fp32 multiply.
#include "common.h"

#include <math.h>

namespace mp {
namespace {

template <int kMode>
__global__ __launch_bounds__(kBlock) void normalize_kernel(const int32_t *__restrict__ src,
                                                           const int32_t *__restrict__ dst,
                                                           const int32_t *__restrict__ rowptr,
                                                           const int32_t *__restrict__ rowptr_t,
                                                           const float *__restrict__ in,
                                                           float *__restrict__ out, int64_t e) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < e; i += stride) {
        const int d = dst[i];
        const double din = (double)(rowptr[d + 1] - rowptr[d]);
        double c;
        if (kMode == MP_NORM_MEAN) {
            c = 1.0 / din;
        } else {
            const int s = src[i];
            const double dout = (double)(rowptr_t[s + 1] - rowptr_t[s]);
            c = 1.0 / sqrt(dout * din);
        }
        out[i] = in[i] * (float)c;
    }
}

}  // namespace

mp_status edge_normalize_run(const mp_graph *g, int mode, const float *in, float *out,
                             hipStream_t s) {
    const int64_t e = g->num_edges;
    if (e == 0) return MP_OK;
    int64_t blocks = (e + kBlock - 1) / kBlock;
    if (blocks > 65536) blocks = 65536;
    if (mode == MP_NORM_MEAN)
        normalize_kernel<MP_NORM_MEAN><<<(unsigned)blocks, kBlock, 0, s>>>(
            g->src, g->dst, g->rowptr, g->rowptr_t, in, out, e);
    else
        normalize_kernel<MP_NORM_SYM><<<(unsigned)blocks, kBlock, 0, s>>>(
            g->src, g->dst, g->rowptr, g->rowptr_t, in, out, e);
    MP_HIP_CHECK(hipGetLastError(), "edge normalisation launch");
    return MP_OK;
}

}  // namespace mp
