// attention.hip -- the row term of the score gradient of a sparse attention
// layer (tinymesh "Weighted aggregation experiment", "Limits": scalar scores
// normalised over each target's edges by a softmax, then aggregated with
// Y = A_alpha X).
//
// The softmax backward needs, per target i and head q, the row sum
//   t[i, q] = sum over edges e into i of alpha_e dalpha_e,
// with dalpha_e = <X[src_e], dY[i]> over head q's columns.  Pulling dY[i] out
// of the sum gives t[i, q] = <Y[i], dY[i]> over those columns, since
// Y[i] = sum over those edges of alpha_e X[src_e].  So once the forward output
// Y is kept, t is a dense row-wise dot product: one coalesced pass over Y and
// dY, no gather, and the fused backward can write ds_e = alpha_e (dalpha_e -
// t[dst_e]) in the same walk that produces dalpha_e.
#include "common.h"

namespace mp {
namespace {

template <typename T, int VEC>
struct Vec;

template <>
struct Vec<float, 4> {
    static __device__ __forceinline__ void load(const float *p, float (&v)[4]) {
        const float4 q = *reinterpret_cast<const float4 *>(p);
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    }
};
template <>
struct Vec<float, 1> {
    static __device__ __forceinline__ void load(const float *p, float (&v)[1]) { v[0] = *p; }
};
template <>
struct Vec<uint16_t, 4> {   // bf16: the bits in the high half of a float are exact
    static __device__ __forceinline__ void load(const uint16_t *p, float (&v)[4]) {
        const uint2 q = *reinterpret_cast<const uint2 *>(p);
        v[0] = __uint_as_float(q.x << 16);
        v[1] = __uint_as_float(q.x & 0xffff0000u);
        v[2] = __uint_as_float(q.y << 16);
        v[3] = __uint_as_float(q.y & 0xffff0000u);
    }
};
template <>
struct Vec<uint16_t, 1> {
    static __device__ __forceinline__ void load(const uint16_t *p, float (&v)[1]) {
        v[0] = __uint_as_float((uint32_t)(*p) << 16);
    }
};

// Items are (row, head) pairs in row-major order, so item it = i * K + q covers
// the contiguous columns [it * hw, (it + 1) * hw) of Y and dY.  A group of S
// lanes (a power of two, S <= 64) owns one item: lane `sub` takes columns
// sub * VEC, (sub + S) * VEC, ... in order, then the group sums its lanes in a
// butterfly.  The loop over item blocks is wave-uniform, so every lane reaches
// each shuffle.
template <typename T, int VEC>
__global__ __launch_bounds__(kBlock) void row_dot_kernel(const float *__restrict__ y,
                                                         const T *__restrict__ dy,
                                                         float *__restrict__ t, int64_t items,
                                                         int64_t hw, int s_lanes) {
    const int lane = threadIdx.x & (kWave - 1);
    const int sub = lane & (s_lanes - 1);
    const int per_wave = kWave / s_lanes;
    const int64_t wave = ((int64_t)blockIdx.x * kBlock + threadIdx.x) / kWave;
    const int64_t waves = (int64_t)gridDim.x * (kBlock / kWave);
    for (int64_t base = wave * per_wave; base < items; base += waves * per_wave) {
        const int64_t it = base + lane / s_lanes;
        float acc = 0.f;
        if (it < items) {
            const float *yr = y + it * hw;
            const T *dr = dy + it * hw;
            for (int64_t c = (int64_t)sub * VEC; c < hw; c += (int64_t)s_lanes * VEC) {
                float a[VEC], b[VEC];
                Vec<float, VEC>::load(yr + c, a);
                Vec<T, VEC>::load(dr + c, b);
#pragma unroll
                for (int v = 0; v < VEC; ++v) acc = fmaf(a[v], b[v], acc);
            }
        }
        for (int off = s_lanes / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
        if (it < items && sub == 0) t[it] = acc;
    }
}

// ds_e = alpha_e (ds_e - t[dst_e]) in place, per head: the edge gradients
// dalpha already sit in ds (the unfused path).
__global__ __launch_bounds__(kBlock) void score_grad_apply_kernel(
    const int32_t *__restrict__ dst, const float *__restrict__ alpha,
    const float *__restrict__ t, float *ds, int64_t items, int k) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < items; i += stride) {
        const int64_t e = i / k;
        const float d = ds[i];
        ds[i] = alpha[i] * (d - t[(int64_t)dst[e] * k + (i - e * k)]);
    }
}

unsigned blocks_for(int64_t threads) {
    int64_t b = (threads + kBlock - 1) / kBlock;
    if (b < 1) b = 1;
    return (unsigned)(b < 65536 ? b : 65536);
}

template <typename T, int VEC>
void launch_row_dot(const float *y, const void *dy, float *t, int64_t items, int64_t hw,
                    hipStream_t st) {
    int64_t lanes = (hw + VEC - 1) / VEC;
    int s = 1;
    while (s < lanes && s < kWave) s <<= 1;
    const int64_t waves = (items + (kWave / s) - 1) / (kWave / s);
    row_dot_kernel<T, VEC><<<blocks_for(waves * kWave), kBlock, 0, st>>>(
        y, static_cast<const T *>(dy), t, items, hw, s);
}

}  // namespace

mp_status attention_row_dot_run(const float *y, const void *dy, mp_dtype dt, int64_t n,
                                int64_t h, int64_t heads, float *t, hipStream_t st) {
    const int64_t hw = h / heads, items = n * heads;
    const uintptr_t py = reinterpret_cast<uintptr_t>(y), pd = reinterpret_cast<uintptr_t>(dy);
    if (dt == MP_F32) {
        if (hw % 4 == 0 && py % 16 == 0 && pd % 16 == 0)
            launch_row_dot<float, 4>(y, dy, t, items, hw, st);
        else
            launch_row_dot<float, 1>(y, dy, t, items, hw, st);
    } else {
        if (hw % 4 == 0 && py % 16 == 0 && pd % 8 == 0)
            launch_row_dot<uint16_t, 4>(y, dy, t, items, hw, st);
        else
            launch_row_dot<uint16_t, 1>(y, dy, t, items, hw, st);
    }
    MP_HIP_CHECK(hipGetLastError(), "attention row-dot launch");
    return MP_OK;
}

mp_status score_grad_apply_run(const int32_t *dst, const float *alpha, const float *t,
                               int64_t e, int64_t heads, float *ds, hipStream_t st) {
    const int64_t items = e * heads;
    if (items == 0) return MP_OK;
    score_grad_apply_kernel<<<blocks_for(items), kBlock, 0, st>>>(dst, alpha, t, ds, items,
                                                                  (int)heads);
    MP_HIP_CHECK(hipGetLastError(), "score-gradient launch");
    return MP_OK;
}

}  // namespace mp
