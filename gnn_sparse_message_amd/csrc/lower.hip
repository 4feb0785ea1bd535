// lower.hip -- device lowering of a COO edge list into the forward CSR
// (rows = destinations) and the transpose CSR (rows = sources), with the
// position -> COO-ordinal maps, plus the degree-class row plans.
//
// What is computed follows tinymesh "Weighted aggregation experiment",
// "Edge order is explicit": both maps send a CSR position to the original COO
// ordinal, duplicates keep their own positions, and the sort is stable, so
// positions inside a row follow ascending ordinal (the witness of "Exact
// witness" lowers to edge_order = (2, 0, 1)).
//
// How it is computed (gfx950): a least-significant-digit radix sort of
// (key, ordinal) pairs with 8-bit digits.  Each pass is three kernels:
//   upsweep   -- every block counts the digits of its contiguous run of tiles;
//   scan      -- one block per digit turns the per-block counts into offsets;
//   downsweep -- every block re-reads its tiles, ranks each key among equal
//                digits with 64-lane ballots (stable: rank order = input order),
//                regroups the tile by digit in LDS and writes it out in runs.
// Block-local ranks, never atomics, decide where equal keys land, so the
// result is the unique stable order.  Rows are then delimited by a binary
// search per row over the sorted keys, and col[p] = other[order[p]].
#include "common.h"

namespace mp {
namespace {

constexpr int kItems = 16;                        // keys per thread per tile
constexpr int kTile = kBlock * kItems;            // 4096 keys per tile
constexpr int kWaveChunk = kWave * kItems;        // 1024 keys per wave per tile
constexpr int kBins = 256;                        // 8-bit digits
constexpr int kDigitBits = 8;
constexpr int kMaxBlocks = 1024;                  // sort blocks per pass (bounds the count table)
constexpr int kSmallFlag = 0;                     // small[0]: index-range flag
constexpr int kSmallPlanF = 64;                   // small[64..320): digit totals of the forward plan
constexpr int kSmallPlanT = 64 + kBins;           // small[320..576): digit totals of the transpose plan
constexpr int kSmallWords = 64 + 2 * kBins;
constexpr int kPlanBits = 6;                      // plan keys 32 - class lie in [0, 32]

static_assert(kBlock == kBins, "scan and downsweep map one thread to one digit");

// ------------------------------------------------------------------ key sources
struct KeysFromArray {
    const uint32_t *k;
    __device__ __forceinline__ uint32_t operator()(int64_t i) const { return k[i]; }
};

// Plan key of row i: 32 - class(length), so the highest class sorts first.
struct KeysFromDegree {
    const int32_t *rowptr;
    __device__ __forceinline__ uint32_t operator()(int64_t i) const {
        uint32_t d = (uint32_t)(rowptr[i + 1] - rowptr[i]);
        uint32_t c = d == 0 ? 0u : 32u - (uint32_t)__clz(d);
        return 32u - c;
    }
};

// ------------------------------------------------------------------ wave / block helpers
// Mask of the valid lanes of this wave whose digit equals ours.
__device__ __forceinline__ uint64_t match_digit(uint32_t d, bool valid, int bits) {
    uint64_t m = __builtin_amdgcn_ballot_w64(valid);
    for (int b = 0; b < bits; ++b) {
        const bool bit = (d >> b) & 1u;
        const uint64_t bb = __builtin_amdgcn_ballot_w64(bit);
        m &= bit ? bb : ~bb;
    }
    return m;
}

// Exclusive prefix sum over the 256 threads of a block; *total receives the sum.
// Contains barriers: every thread of the block must call it.
__device__ uint32_t block_exclusive_scan(uint32_t x, uint32_t *total) {
    __shared__ uint32_t s_wsum[kWavesPerBlock];
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    uint32_t inc = x;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t y = __shfl_up(inc, off);
        if (lane >= off) inc += y;
    }
    if (lane == kWave - 1) s_wsum[wv] = inc;
    __syncthreads();
    uint32_t wbase = 0, tot = 0;
#pragma unroll
    for (int k = 0; k < kWavesPerBlock; ++k) {
        const uint32_t s = s_wsum[k];
        wbase += (k < wv) ? s : 0u;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return wbase + inc - x;
}

// ------------------------------------------------------------------ intake
// Copy the caller's endpoints to int32, checking 0 <= v < n.  Out-of-range
// values are stored as 0 (so later kernels stay in bounds) and raise the flag.
template <typename IdxT>
__global__ __launch_bounds__(kBlock) void intake_kernel(const IdxT *__restrict__ src,
                                                        const IdxT *__restrict__ dst, int64_t e,
                                                        int64_t n, int32_t *__restrict__ src32,
                                                        int32_t *__restrict__ dst32,
                                                        uint32_t *__restrict__ flag) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < e; i += stride) {
        const int64_t s = (int64_t)src[i];
        const int64_t d = (int64_t)dst[i];
        const bool ok_s = s >= 0 && s < n;
        const bool ok_d = d >= 0 && d < n;
        src32[i] = ok_s ? (int32_t)s : 0;
        dst32[i] = ok_d ? (int32_t)d : 0;
        if (!(ok_s && ok_d)) *flag = 1u;   // plain store: every writer stores the same value
    }
}

__global__ void zero_words_kernel(uint32_t *p, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

// ------------------------------------------------------------------ radix pass kernels
template <class KeySrc>
__global__ __launch_bounds__(kBlock) void rs_upsweep(KeySrc keys, int64_t count, int shift,
                                                     int bits, int64_t tiles_per_block,
                                                     int64_t ntiles, int nblocks,
                                                     uint32_t *__restrict__ hist) {
    __shared__ uint32_t s_cnt[kWavesPerBlock][kBins];
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    for (int i = threadIdx.x; i < kWavesPerBlock * kBins; i += kBlock) (&s_cnt[0][0])[i] = 0u;
    __syncthreads();
    const uint32_t mask = (1u << bits) - 1u;
    const int64_t t0 = (int64_t)blockIdx.x * tiles_per_block;
    const int64_t t1 = t0 + tiles_per_block < ntiles ? t0 + tiles_per_block : ntiles;
    for (int64_t t = t0; t < t1; ++t) {
        const int64_t base = t * kTile + (int64_t)wv * kWaveChunk + lane;
        uint32_t k[kItems];
#pragma unroll
        for (int r = 0; r < kItems; ++r) {
            const int64_t i = base + (int64_t)r * kWave;
            k[r] = i < count ? keys(i) : 0u;
        }
#pragma unroll
        for (int r = 0; r < kItems; ++r) {
            const bool valid = base + (int64_t)r * kWave < count;
            const uint32_t d = (k[r] >> shift) & mask;
            const uint64_t m = match_digit(d, valid, bits);
            // One leader per distinct digit updates this wave's private counter.
            if (valid && __builtin_ctzll(m) == lane) s_cnt[wv][d] += (uint32_t)__popcll(m);
        }
    }
    __syncthreads();
    const int d = threadIdx.x;
    uint32_t c = 0;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) c += s_cnt[w][d];
    hist[(int64_t)d * nblocks + blockIdx.x] = c;
}

// One block per digit: exclusive scan of that digit's per-block counts (in place),
// and the digit's total.
__global__ __launch_bounds__(kBlock) void rs_scan(uint32_t *__restrict__ hist, int nblocks,
                                                  uint32_t *__restrict__ dtot) {
    constexpr int kPer = kMaxBlocks / kBlock;
    uint32_t *row = hist + (int64_t)blockIdx.x * nblocks;
    const int beg = threadIdx.x * kPer;
    uint32_t v[kPer];
    uint32_t sum = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        v[j] = beg + j < nblocks ? row[beg + j] : 0u;
        sum += v[j];
    }
    uint32_t total;
    uint32_t run = block_exclusive_scan(sum, &total);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        if (beg + j < nblocks) row[beg + j] = run;
        run += v[j];
    }
    if (threadIdx.x == 0) dtot[blockIdx.x] = total;
}

template <class KeySrc, bool kIotaVals, bool kWriteKeys>
__global__ __launch_bounds__(kBlock) void rs_downsweep(
    KeySrc keys, const uint32_t *__restrict__ vals_in, int64_t count, int shift, int bits,
    int64_t tiles_per_block, int64_t ntiles, int nblocks, const uint32_t *__restrict__ hist,
    const uint32_t *__restrict__ dtot, uint32_t *__restrict__ keys_out,
    uint32_t *__restrict__ vals_out) {
    __shared__ uint32_t s_key[kTile];
    __shared__ uint32_t s_val[kTile];
    __shared__ uint32_t s_cnt[kWavesPerBlock][kBins];
    __shared__ uint32_t s_tstart[kBins];
    __shared__ uint32_t s_gbase[kBins];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wv = tid / kWave;
    const uint32_t mask = (1u << bits) - 1u;
    const uint64_t lanes_below = (1ull << lane) - 1ull;

    {   // where this block's run of each digit starts in the output
        uint32_t tot;
        const uint32_t dbase = block_exclusive_scan(dtot[tid], &tot);
        s_gbase[tid] = dbase + hist[(int64_t)tid * nblocks + blockIdx.x];
    }
    const int64_t t0 = (int64_t)blockIdx.x * tiles_per_block;
    const int64_t t1 = t0 + tiles_per_block < ntiles ? t0 + tiles_per_block : ntiles;
    for (int64_t t = t0; t < t1; ++t) {
        for (int i = tid; i < kWavesPerBlock * kBins; i += kBlock) (&s_cnt[0][0])[i] = 0u;
        __syncthreads();
        const int64_t base = t * kTile + (int64_t)wv * kWaveChunk + lane;
        uint32_t k[kItems], v[kItems], rk[kItems];
#pragma unroll
        for (int r = 0; r < kItems; ++r) {
            const int64_t i = base + (int64_t)r * kWave;
            const bool valid = i < count;
            k[r] = valid ? keys(i) : 0u;
            if (kIotaVals) v[r] = (uint32_t)i;
            else v[r] = valid ? vals_in[i] : 0u;
        }
        // Rank inside the wave: earlier rounds (running count) + lower lanes now.
#pragma unroll
        for (int r = 0; r < kItems; ++r) {
            const bool valid = base + (int64_t)r * kWave < count;
            const uint32_t d = (k[r] >> shift) & mask;
            const uint64_t m = match_digit(d, valid, bits);
            const uint32_t before = s_cnt[wv][d];
            rk[r] = before + (uint32_t)__popcll(m & lanes_below);
            if (valid && __builtin_ctzll(m) == lane) s_cnt[wv][d] = before + (uint32_t)__popcll(m);
        }
        __syncthreads();
        // Thread `tid` owns digit `tid`: per-wave offsets and the tile's digit starts.
        const uint32_t c0 = s_cnt[0][tid], c1 = s_cnt[1][tid], c2 = s_cnt[2][tid],
                       c3 = s_cnt[3][tid];
        const uint32_t ttot = c0 + c1 + c2 + c3;
        uint32_t all;
        const uint32_t tstart = block_exclusive_scan(ttot, &all);   // barriers inside
        s_cnt[0][tid] = tstart;
        s_cnt[1][tid] = tstart + c0;
        s_cnt[2][tid] = tstart + c0 + c1;
        s_cnt[3][tid] = tstart + c0 + c1 + c2;
        s_tstart[tid] = tstart;
        __syncthreads();
#pragma unroll
        for (int r = 0; r < kItems; ++r) {
            if (base + (int64_t)r * kWave < count) {
                const uint32_t d = (k[r] >> shift) & mask;
                const uint32_t pos = s_cnt[wv][d] + rk[r];
                s_key[pos] = k[r];
                s_val[pos] = v[r];
            }
        }
        __syncthreads();
        const int64_t left = count - t * kTile;
        const int tile_n = left < kTile ? (int)left : kTile;
        for (int i = tid; i < tile_n; i += kBlock) {
            const uint32_t kk = s_key[i];
            const uint32_t d = (kk >> shift) & mask;
            const uint32_t g = s_gbase[d] + ((uint32_t)i - s_tstart[d]);
            if ((int64_t)g < count) {   // always true for a consistent count table
                if (kWriteKeys) keys_out[g] = kk;
                vals_out[g] = s_val[i];
            }
        }
        __syncthreads();
        s_gbase[tid] += ttot;
    }
}

// ------------------------------------------------------------------ rows and columns
// rowptr[i] = number of sorted keys below i (binary search), for i in [0, n].
__global__ __launch_bounds__(kBlock) void rowptr_kernel(const uint32_t *__restrict__ sorted,
                                                        int64_t e, int64_t n,
                                                        int32_t *__restrict__ rowptr) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i <= n; i += stride) {
        int64_t lo = 0, hi = e;
        while (lo < hi) {
            const int64_t mid = (lo + hi) >> 1;
            if ((int64_t)sorted[mid] < i) lo = mid + 1;
            else hi = mid;
        }
        rowptr[i] = (int32_t)lo;
    }
}

__global__ __launch_bounds__(kBlock) void gather_kernel(const int32_t *__restrict__ order,
                                                        const int32_t *__restrict__ other,
                                                        int64_t e, int32_t *__restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < e; i += stride) {
        const uint32_t o = (uint32_t)order[i];
        out[i] = (int64_t)o < e ? other[o] : 0;   // order is a permutation of [0, e)
    }
}

// ------------------------------------------------------------------ host side
struct Part {
    int64_t ntiles;
    int64_t tpb;
    int nblocks;
};

Part partition(int64_t count) {
    Part p;
    p.ntiles = count > 0 ? (count + kTile - 1) / kTile : 1;
    int64_t nb = p.ntiles < kMaxBlocks ? p.ntiles : kMaxBlocks;
    p.tpb = (p.ntiles + nb - 1) / nb;
    p.nblocks = (int)((p.ntiles + p.tpb - 1) / p.tpb);
    return p;
}

unsigned grid_for(int64_t items, int64_t cap = 65536) {
    int64_t b = (items + kBlock - 1) / kBlock;
    if (b < 1) b = 1;
    return (unsigned)(b < cap ? b : cap);
}

int key_bits(int64_t n) {
    int bits = 0;
    while (bits < 31 && ((int64_t)1 << bits) < n) ++bits;
    return bits > 0 ? bits : 1;   // one pass even for n = 1 (a stable copy)
}

template <class KeySrc>
mp_status radix_pass(KeySrc keys, const uint32_t *vals_in, bool iota_vals, bool write_keys,
                     int64_t count, int shift, int bits, uint32_t *hist, uint32_t *dtot,
                     uint32_t *keys_out, uint32_t *vals_out, hipStream_t s) {
    const Part p = partition(count);
    rs_upsweep<KeySrc><<<p.nblocks, kBlock, 0, s>>>(keys, count, shift, bits, p.tpb, p.ntiles,
                                                    p.nblocks, hist);
    rs_scan<<<kBins, kBlock, 0, s>>>(hist, p.nblocks, dtot);
    if (iota_vals && write_keys)
        rs_downsweep<KeySrc, true, true><<<p.nblocks, kBlock, 0, s>>>(
            keys, vals_in, count, shift, bits, p.tpb, p.ntiles, p.nblocks, hist, dtot, keys_out,
            vals_out);
    else if (iota_vals)
        rs_downsweep<KeySrc, true, false><<<p.nblocks, kBlock, 0, s>>>(
            keys, vals_in, count, shift, bits, p.tpb, p.ntiles, p.nblocks, hist, dtot, keys_out,
            vals_out);
    else if (write_keys)
        rs_downsweep<KeySrc, false, true><<<p.nblocks, kBlock, 0, s>>>(
            keys, vals_in, count, shift, bits, p.tpb, p.ntiles, p.nblocks, hist, dtot, keys_out,
            vals_out);
    else
        rs_downsweep<KeySrc, false, false><<<p.nblocks, kBlock, 0, s>>>(
            keys, vals_in, count, shift, bits, p.tpb, p.ntiles, p.nblocks, hist, dtot, keys_out,
            vals_out);
    MP_HIP_CHECK(hipGetLastError(), "radix pass launch");
    return MP_OK;
}

// Stable sort of the ordinals 0..e-1 by key[0..e); final ordinals land in
// `order`, final keys in *sorted (one of k0 / k1).
mp_status sort_edges(const int32_t *key, int64_t e, int64_t n, uint32_t *k0, uint32_t *k1,
                     uint32_t *v0, uint32_t *hist, uint32_t *dtot, int32_t *order,
                     const uint32_t **sorted, hipStream_t s) {
    const int bits = key_bits(n);
    const int passes = (bits + kDigitBits - 1) / kDigitBits;
    const uint32_t *kin = reinterpret_cast<const uint32_t *>(key);
    const uint32_t *vin = nullptr;
    uint32_t *kbuf[2] = {k0, k1};
    for (int pass = 0; pass < passes; ++pass) {
        const int shift = pass * kDigitBits;
        const int pb = bits - shift < kDigitBits ? bits - shift : kDigitBits;
        // Values alternate between `order` and v0 so that the last pass lands in `order`.
        uint32_t *vout = ((passes - 1 - pass) % 2 == 0) ? reinterpret_cast<uint32_t *>(order) : v0;
        uint32_t *kout = kbuf[pass % 2];
        mp_status st = radix_pass(KeysFromArray{kin}, vin, pass == 0, true, e, shift, pb, hist,
                                  dtot, kout, vout, s);
        if (st != MP_OK) return st;
        kin = kout;
        vin = vout;
    }
    *sorted = kin;
    return MP_OK;
}

mp_status lower_direction(const int32_t *key, const int32_t *other, int64_t e, int64_t n,
                          uint32_t *k0, uint32_t *k1, uint32_t *v0, uint32_t *hist,
                          uint32_t *dtot, int32_t *rowptr, int32_t *col, int32_t *order,
                          hipStream_t s) {
    const uint32_t *sorted = k0;
    if (e > 0) {
        mp_status st = sort_edges(key, e, n, k0, k1, v0, hist, dtot, order, &sorted, s);
        if (st != MP_OK) return st;
    }
    rowptr_kernel<<<grid_for(n + 1), kBlock, 0, s>>>(sorted, e, n, rowptr);
    if (e > 0) gather_kernel<<<grid_for(e), kBlock, 0, s>>>(order, other, e, col);
    MP_HIP_CHECK(hipGetLastError(), "row/column launch");
    return MP_OK;
}

mp_status plan_direction(const int32_t *rowptr, int64_t n, uint32_t *hist, uint32_t *totals,
                         int32_t *plan, hipStream_t s) {
    return radix_pass(KeysFromDegree{rowptr}, nullptr, true, false, n, 0, kPlanBits, hist,
                      totals, nullptr, reinterpret_cast<uint32_t *>(plan), s);
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

LowerLayout lower_layout(int64_t n, int64_t e) {
    (void)n;
    LowerLayout L;
    size_t off = 0;
    const size_t ebytes = align_up((size_t)(e > 0 ? e : 1) * sizeof(uint32_t));
    L.k0 = off; off += ebytes;
    L.k1 = off; off += ebytes;
    L.v0 = off; off += ebytes;
    L.hist = off; off += align_up((size_t)kBins * kMaxBlocks * sizeof(uint32_t));
    L.dtot = off; off += align_up(kBins * sizeof(uint32_t));
    L.small = off; off += align_up(kSmallWords * sizeof(uint32_t));
    L.total = off;
    return L;
}

mp_status lower_run(const void *src, const void *dst, mp_dtype idx_dtype, int64_t n, int64_t e,
                    mp_graph *g, void *ws, hipStream_t s, int *bad_index) {
    const LowerLayout L = lower_layout(n, e);
    char *base = static_cast<char *>(ws);
    uint32_t *k0 = reinterpret_cast<uint32_t *>(base + L.k0);
    uint32_t *k1 = reinterpret_cast<uint32_t *>(base + L.k1);
    uint32_t *v0 = reinterpret_cast<uint32_t *>(base + L.v0);
    uint32_t *hist = reinterpret_cast<uint32_t *>(base + L.hist);
    uint32_t *dtot = reinterpret_cast<uint32_t *>(base + L.dtot);
    uint32_t *small = reinterpret_cast<uint32_t *>(base + L.small);

    zero_words_kernel<<<1, kBlock, 0, s>>>(small, kSmallWords);
    if (e > 0) {
        if (idx_dtype == MP_I64)
            intake_kernel<int64_t><<<grid_for(e), kBlock, 0, s>>>(
                static_cast<const int64_t *>(src), static_cast<const int64_t *>(dst), e, n, g->src,
                g->dst, small + kSmallFlag);
        else
            intake_kernel<int32_t><<<grid_for(e), kBlock, 0, s>>>(
                static_cast<const int32_t *>(src), static_cast<const int32_t *>(dst), e, n, g->src,
                g->dst, small + kSmallFlag);
    }
    MP_HIP_CHECK(hipGetLastError(), "intake launch");

    mp_status st = lower_direction(g->dst, g->src, e, n, k0, k1, v0, hist, dtot, g->rowptr,
                                   g->col, g->edge_order, s);
    if (st != MP_OK) return st;
    st = lower_direction(g->src, g->dst, e, n, k0, k1, v0, hist, dtot, g->rowptr_t, g->col_t,
                         g->transpose_order, s);
    if (st != MP_OK) return st;
    st = plan_direction(g->rowptr, n, hist, small + kSmallPlanF, g->row_plan, s);
    if (st != MP_OK) return st;
    st = plan_direction(g->rowptr_t, n, hist, small + kSmallPlanT, g->row_plan_t, s);
    if (st != MP_OK) return st;

    uint32_t host[kSmallWords];
    MP_HIP_CHECK(hipMemcpyAsync(host, small, sizeof(host), hipMemcpyDeviceToHost, s),
                 "copy of build results to host");
    MP_HIP_CHECK(hipStreamSynchronize(s), "build synchronisation");
    *bad_index = host[kSmallFlag] != 0u;
    for (int c = 0; c < MP_NUM_CLASSES; ++c) {
        g->class_count[c] = host[kSmallPlanF + (32 - c)];
        g->class_count_t[c] = host[kSmallPlanT + (32 - c)];
    }
    return MP_OK;
}

}  // namespace mp
