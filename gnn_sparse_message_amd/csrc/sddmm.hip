// sddmm.hip -- edge-weight gradient dw_e = <X[src_e, :], dY[dst_e, :]> for every
// edge, written in COO order with one owner per edge (tinymesh "Weighted
// aggregation experiment", "Decision" and the bottom of the diagram under
// "Edge order is explicit"; the SDDMM of "PyTorch Geometric: one abstraction,
// the whole GNN literature", Step 4, evaluated at the edges only).
//
// Mapping on gfx950.  Each wave takes 64 consecutive edges: one coalesced load
// of src/dst per lane, then groups of L lanes (VEC features per lane: 16-byte
// loads, or two for rows of 256 fp32 features or more, by the same rule as the
// aggregation, f32_vec) take the edges G = 64/L at a time, U edges per group in flight.  Each
// group reduces its dot product across its L lanes (run_sum: DPP moves inside a
// 16-lane row, lane permutes beyond), the
// results are collected so that lane k holds edge k, and the wave writes its
// 64 values with one coalesced store.  fp32 accumulation; bf16 widened exactly.
//
// Multi-head weights (K per edge, head q owning columns [q*H/K, (q+1)*H/K)):
// the work items are the E*K (edge, head) pairs in dw's own [E, K] order, each
// a dot product over one head's columns, so the store stays coalesced.  A
// head's lanes are reduced with run_sum when their count is a power of two (or
// the whole wave), else in lane order -- the same order as the fused backward,
// so both give equal dw.
#include "common.h"

namespace mp {
namespace {

constexpr int kUnroll = 4;

template <typename T, int VEC>
struct Feat2;

template <>
struct Feat2<float, 4> {
    static __device__ __forceinline__ float dot(const float *a, const float *b) {
        const float4 p = *reinterpret_cast<const float4 *>(a);
        const float4 q = *reinterpret_cast<const float4 *>(b);
        float s = fmaf(p.x, q.x, 0.f);
        s = fmaf(p.y, q.y, s);
        s = fmaf(p.z, q.z, s);
        return fmaf(p.w, q.w, s);
    }
};
template <>
struct Feat2<float, 8> {
    static __device__ __forceinline__ float dot(const float *a, const float *b) {
        const float4 p0 = *reinterpret_cast<const float4 *>(a);
        const float4 q0 = *reinterpret_cast<const float4 *>(b);
        const float4 p1 = *reinterpret_cast<const float4 *>(a + 4);
        const float4 q1 = *reinterpret_cast<const float4 *>(b + 4);
        float s = fmaf(p0.x, q0.x, 0.f);
        s = fmaf(p0.y, q0.y, s);
        s = fmaf(p0.z, q0.z, s);
        s = fmaf(p0.w, q0.w, s);
        s = fmaf(p1.x, q1.x, s);
        s = fmaf(p1.y, q1.y, s);
        s = fmaf(p1.z, q1.z, s);
        return fmaf(p1.w, q1.w, s);
    }
};
template <>
struct Feat2<float, 1> {
    static __device__ __forceinline__ float dot(const float *a, const float *b) {
        return fmaf(*a, *b, 0.f);
    }
};
template <>
struct Feat2<uint16_t, 8> {
    static __device__ __forceinline__ float dot(const uint16_t *a, const uint16_t *b) {
        const uint4 p = *reinterpret_cast<const uint4 *>(a);
        const uint4 q = *reinterpret_cast<const uint4 *>(b);
        const uint32_t u[4] = {p.x, p.y, p.z, p.w};
        const uint32_t v[4] = {q.x, q.y, q.z, q.w};
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s = fmaf(__uint_as_float(u[i] << 16), __uint_as_float(v[i] << 16), s);
            s = fmaf(__uint_as_float(u[i] & 0xffff0000u), __uint_as_float(v[i] & 0xffff0000u), s);
        }
        return s;
    }
};
template <>
struct Feat2<uint16_t, 1> {
    static __device__ __forceinline__ float dot(const uint16_t *a, const uint16_t *b) {
        return fmaf(__uint_as_float((uint32_t)(*a) << 16), __uint_as_float((uint32_t)(*b) << 16), 0.f);
    }
};

// Items are edges (kHeads = false; hw = h) or (edge, head) pairs, item i being
// edge i / heads and head i % heads, over hw = h / heads columns.
template <typename T, int VEC, int L, bool kHeads>
__global__ __launch_bounds__(kBlock) void sddmm_kernel(const int32_t *__restrict__ src,
                                                       const int32_t *__restrict__ dst,
                                                       const T *__restrict__ X,
                                                       const T *__restrict__ dY,
                                                       float *__restrict__ dw, int64_t e,
                                                       int64_t h, int32_t heads, int32_t hw) {
    constexpr int G = kWave / L;                       // items per wave step
    const int lane = threadIdx.x & (kWave - 1);
    const int g = lane / L;
    const int sub = lane % L;
    const int64_t nf = (hw + (int64_t)L * VEC - 1) / ((int64_t)L * VEC);  // feature chunks
    const int seg = hw / VEC;                          // lanes holding one head (multi-head)
    const bool tree = (seg & (seg - 1)) == 0 || seg >= kWave;
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t base = ((int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave) * kWave;
         base < e; base += nwaves * kWave) {
        const int64_t me = base + lane;
        int s = 0, d = 0, q = 0;
        if (me < e) {   // streamed once: non-temporal, so L2 keeps the feature rows
            if constexpr (kHeads) {
                const int64_t ed = me / heads;
                q = (int)(me - ed * heads);
                s = src[ed];
                d = dst[ed];
            } else {
                s = __builtin_nontemporal_load(&src[me]);
                d = __builtin_nontemporal_load(&dst[me]);
            }
        }
        const int n = e - base < kWave ? (int)(e - base) : kWave;
        const int trips = (n + G - 1) / G;
        float mine = 0.f;
        for (int j = 0; j < trips; j += kUnroll) {
            float part[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int k = g + (j + u) * G;
                const bool ok = (j + u < trips) && k < n;
                const int sl = k < n ? k : n - 1;
                const int su = __shfl(s, sl);
                const int du = __shfl(d, sl);
                const int64_t col0 = kHeads ? (int64_t)__shfl(q, sl) * hw : 0;
                // Lane-local dot: an fma chain from zero per chunk (no bare product
                // that could be contracted into the lane reduction below).
                float acc = 0.f;
                if (ok) {
                    for (int64_t f = 0; f < nf; ++f) {
                        const int64_t hoff = (f * L + sub) * VEC;
                        if (hoff < hw) {
                            const float d = Feat2<T, VEC>::dot(X + (int64_t)su * h + col0 + hoff,
                                                               dY + (int64_t)du * h + col0 + hoff);
                            acc = f == 0 ? d : acc + d;
                        }
                    }
                }
                part[u] = acc;
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                if (!kHeads || tree) {
                    part[u] = run_sum(part[u], L);
                } else {   // a head of seg < 64 lanes, seg not a power of two: lane order
                    float t = __shfl(part[u], g * L);
                    for (int i = 1; i < seg; ++i) t += __shfl(part[u], g * L + i);
                    part[u] = t;
                }
                // Edge k = g' + (j+u)*G sits in every lane of group g'; lane k collects it.
                const float got = __shfl(part[u], (lane % G) * L);
                if (lane / G == j + u) mine = got;
            }
        }
        if (me < e) __builtin_nontemporal_store(mine, &dw[me]);
    }
}

template <typename T, int VEC, int L>
mp_status launch(const int32_t *src, const int32_t *dst, int64_t e, const void *x,
                 const void *dy, int64_t h, int64_t heads, float *dw, hipStream_t s) {
    const int64_t items = e * heads;
    const int64_t per_block = (int64_t)kWavesPerBlock * kWave;
    int64_t blocks = (items + per_block - 1) / per_block;
    const int64_t cap = 1 << 22;
    if (blocks > cap) blocks = cap;
    if (blocks <= 0) return MP_OK;
    const T *xt = static_cast<const T *>(x), *dyt = static_cast<const T *>(dy);
    const int32_t hw = (int32_t)(h / heads);
    if (heads > 1)
        sddmm_kernel<T, VEC, L, true><<<(unsigned)blocks, kBlock, 0, s>>>(
            src, dst, xt, dyt, dw, items, h, (int32_t)heads, hw);
    else
        sddmm_kernel<T, VEC, L, false><<<(unsigned)blocks, kBlock, 0, s>>>(
            src, dst, xt, dyt, dw, items, h, 1, hw);
    MP_HIP_CHECK(hipGetLastError(), "sddmm launch");
    return MP_OK;
}

int lanes_for(int64_t h, int vec) {
    const int64_t need = (h + vec - 1) / vec;
    int L = 1;
    while (L < kWave && L < need) L <<= 1;
    return L;
}

// Lanes per item come from the columns one item covers (a head's, or the row's).
template <typename T, int VEC>
mp_status launch_lanes(const int32_t *src, const int32_t *dst, int64_t e, const void *x,
                       const void *dy, int64_t h, int64_t heads, float *dw, hipStream_t s) {
    switch (lanes_for(h / heads, VEC)) {
        case 1: return launch<T, VEC, 1>(src, dst, e, x, dy, h, heads, dw, s);
        case 2: return launch<T, VEC, 2>(src, dst, e, x, dy, h, heads, dw, s);
        case 4: return launch<T, VEC, 4>(src, dst, e, x, dy, h, heads, dw, s);
        case 8: return launch<T, VEC, 8>(src, dst, e, x, dy, h, heads, dw, s);
        case 16: return launch<T, VEC, 16>(src, dst, e, x, dy, h, heads, dw, s);
        case 32: return launch<T, VEC, 32>(src, dst, e, x, dy, h, heads, dw, s);
        default: return launch<T, VEC, 64>(src, dst, e, x, dy, h, heads, dw, s);
    }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

mp_status sddmm_run(const int32_t *src, const int32_t *dst, int64_t e, const void *x,
                    const void *dy, mp_dtype dt, int64_t h, int64_t heads, float *dw,
                    hipStream_t s) {
    const bool vec_ok = aligned16(x) && aligned16(dy);
    const int64_t hw = h / heads;
    if (dt == MP_F32) {
        if (vec_ok && hw % 4 == 0 && f32_vec(h, heads) == 8)
            return launch_lanes<float, 8>(src, dst, e, x, dy, h, heads, dw, s);
        if (vec_ok && hw % 4 == 0)
            return launch_lanes<float, 4>(src, dst, e, x, dy, h, heads, dw, s);
        return launch_lanes<float, 1>(src, dst, e, x, dy, h, heads, dw, s);
    }
    if (vec_ok && hw % 8 == 0)
        return launch_lanes<uint16_t, 8>(src, dst, e, x, dy, h, heads, dw, s);
    return launch_lanes<uint16_t, 1>(src, dst, e, x, dy, h, heads, dw, s);
}

}  // namespace mp
