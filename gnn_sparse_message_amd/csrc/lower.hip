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
// result is the unique stable order.  The opposite endpoint travels with each
// key, so the last pass writes col[p] = other[order[p]] directly.  Rows are
// then delimited by a binary search per row over the sorted keys.
#include "common.h"

namespace mp {
namespace {

constexpr int kItems = 16;                        // keys per thread per tile
constexpr int kTile = kBlock * kItems;            // 4096 keys per tile
constexpr int kWaveChunk = kWave * kItems;        // 1024 keys per wave per tile
constexpr int kBins = 256;                        // 8-bit digits
constexpr int kDigitBits = 8;                     // at most 8 bits per pass
constexpr int kPlanBits = 6;                      // plan keys 32 - class lie in [0, 32]

static_assert(kBlock == kBins, "scan and downsweep map one thread to one digit");
static_assert(kInfoPlanT - kInfoPlanF == kBins, "one plan record holds every digit total");

// ------------------------------------------------------------------ key sources
// A key source is read at 32-bit offsets from the start of a tile (`at`).
struct KeysFromArray {
    const uint32_t *k;
    __device__ __forceinline__ KeysFromArray at(int64_t base) const { return {k + base}; }
    __device__ __forceinline__ uint32_t operator()(int i) const { return k[i]; }
};

// Plan key of row i: 32 - class(length), so the highest class sorts first.
struct KeysFromDegree {
    const int32_t *rowptr;
    __device__ __forceinline__ KeysFromDegree at(int64_t base) const { return {rowptr + base}; }
    __device__ __forceinline__ uint32_t operator()(int i) const {
        uint32_t d = (uint32_t)(rowptr[i + 1] - rowptr[i]);
        uint32_t c = d == 0 ? 0u : 32u - (uint32_t)__clz(d);
        return 32u - c;
    }
};

// ------------------------------------------------------------------ wave / block helpers
// Mask of the valid lanes of this wave whose digit equals ours.  One ballot per
// digit bit (digits are masked, so bits above the pass width are zero in every
// lane and leave the mask unchanged); each half of the mask keeps the lanes
// whose bit agrees with ours, m &= ~(ballot ^ f) with f = 0 or ~0 from our bit,
// as one three-input bit operation (truth table 0x90: a & (b == c)).
__device__ __forceinline__ uint64_t match_digit(uint32_t d, bool valid) {
    const uint64_t v = __builtin_amdgcn_ballot_w64(valid);
    uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
#pragma unroll
    for (int b = 0; b < kDigitBits; ++b) {
        const uint32_t f = (uint32_t)__builtin_amdgcn_sbfe((int)d, b, 1);
        const uint64_t bb = __builtin_amdgcn_ballot_w64(f != 0u);
        lo = __builtin_amdgcn_bitop3_b32(lo, (uint32_t)bb, f, 0x90);
        hi = __builtin_amdgcn_bitop3_b32(hi, (uint32_t)(bb >> 32), f, 0x90);
    }
    return ((uint64_t)hi << 32) | lo;
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
// Every block sorts exactly one 4096-key tile.  Blocks are handed out round-robin
// over the 8 XCDs, so the logical tile of a block is chosen to make consecutive
// tiles run on the same XCD: their output runs for a digit are adjacent in
// memory and merge in that XCD's L2 instead of being written as partial lines
// from several L2s.
__device__ __forceinline__ int64_t xcd_local_tile() {
    const int64_t g = gridDim.x, b = blockIdx.x;
    const int64_t q = g >> 3, r = g & 7, x = b & 7;
    return x * q + (x < r ? x : r) + (b >> 3);
}

template <class KeySrc>
__global__ __launch_bounds__(kBlock) void rs_upsweep(KeySrc keys, int64_t count, int shift,
                                                     int bits, int64_t ntiles,
                                                     uint32_t *__restrict__ hist) {
    __shared__ uint32_t s_cnt[kWavesPerBlock][kBins];
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    for (int i = threadIdx.x; i < kWavesPerBlock * kBins; i += kBlock) (&s_cnt[0][0])[i] = 0u;
    __syncthreads();
    const uint32_t mask = (1u << bits) - 1u;
    const int64_t t = xcd_local_tile();
    const int64_t left = count - t * kTile;
    const int lim = left < kTile ? (int)left : kTile;        // keys in this tile
    const KeySrc tk = keys.at(t * kTile);
    const int li0 = wv * kWaveChunk + lane;                   // tile-local index, round 0
    uint32_t k[kItems];
#pragma unroll
    for (int r = 0; r < kItems; ++r) {
        const int li = li0 + r * kWave;
        k[r] = li < lim ? tk(li) : 0u;
    }
#pragma unroll
    for (int r = 0; r < kItems; ++r) {
        const bool valid = li0 + r * kWave < lim;
        const uint32_t d = (k[r] >> shift) & mask;
        const uint64_t m = match_digit(d, valid);
        // One leader per distinct digit updates this wave's private counter.
        if (valid && __builtin_ctzll(m) == lane) s_cnt[wv][d] += (uint32_t)__popcll(m);
    }
    __syncthreads();
    const int d = threadIdx.x;
    uint32_t c = 0;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) c += s_cnt[w][d];
    hist[(int64_t)d * ntiles + t] = c;
}

// One block per digit: exclusive scan, in tile order, of that digit's per-tile
// counts (in place), and the digit's total.
__global__ __launch_bounds__(kBlock) void rs_scan(uint32_t *__restrict__ hist, int64_t ntiles,
                                                  uint32_t *__restrict__ dtot) {
    constexpr int kPer = 16;
    uint32_t *row = hist + (int64_t)blockIdx.x * ntiles;
    uint32_t carry = 0;
    for (int64_t chunk = 0; chunk < ntiles; chunk += (int64_t)kBlock * kPer) {
        const int64_t beg = chunk + (int64_t)threadIdx.x * kPer;
        uint32_t v[kPer];
        uint32_t sum = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            v[j] = beg + j < ntiles ? row[beg + j] : 0u;
            sum += v[j];
        }
        uint32_t total;
        uint32_t run = carry + block_exclusive_scan(sum, &total);
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            if (beg + j < ntiles) row[beg + j] = run;
            run += v[j];
        }
        carry += total;
    }
    if (threadIdx.x == 0) dtot[blockIdx.x] = carry;
}

// Payload arrays carried by a pass.  vals are COO ordinals (generated on the
// first pass), other is the opposite endpoint (so the final pass writes the
// column array directly, with no gather).
struct Payload {
    const uint32_t *vals_in;
    const uint32_t *other_in;
    uint32_t *keys_out;
    uint32_t *vals_out;
    uint32_t *other_out;
};

template <class KeySrc, bool kIotaVals, bool kOther, bool kWriteKeys>
__global__ __launch_bounds__(kBlock) void rs_downsweep(KeySrc keys, Payload pl, int64_t count,
                                                       int shift, int bits, int64_t ntiles,
                                                       const uint32_t *__restrict__ hist,
                                                       const uint32_t *__restrict__ dtot) {
    __shared__ uint32_t s_buf[kTile];          // one payload at a time, in tile-sorted order
    __shared__ uint8_t s_dig[kTile];           // digit of each tile-sorted position
    __shared__ uint32_t s_cnt[kWavesPerBlock][kBins];
    __shared__ uint32_t s_tstart[kBins];
    __shared__ uint32_t s_gbase[kBins];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wv = tid / kWave;
    const uint32_t mask = (1u << bits) - 1u;
    const uint64_t lanes_below = (1ull << lane) - 1ull;
    const int64_t t = xcd_local_tile();
    const int64_t tbase = t * kTile;
    const int64_t left = count - tbase;
    const int lim = left < kTile ? (int)left : kTile;        // keys in this tile
    const KeySrc tk = keys.at(tbase);
    const int li0 = wv * kWaveChunk + lane;                   // tile-local index, round 0

    for (int i = tid; i < kWavesPerBlock * kBins; i += kBlock) (&s_cnt[0][0])[i] = 0u;
    uint32_t k[kItems];
#pragma unroll
    for (int r = 0; r < kItems; ++r) {
        const int li = li0 + r * kWave;
        k[r] = li < lim ? tk(li) : 0u;
    }
    __syncthreads();
    // Rank inside the wave: earlier rounds (running count) + lower lanes now.
    uint32_t pos[kItems];
#pragma unroll
    for (int r = 0; r < kItems; ++r) {
        const bool valid = li0 + r * kWave < lim;
        const uint32_t d = (k[r] >> shift) & mask;
        const uint64_t m = match_digit(d, valid);
        const uint32_t before = s_cnt[wv][d];
        pos[r] = before + (uint32_t)__popcll(m & lanes_below);
        if (valid && __builtin_ctzll(m) == lane) s_cnt[wv][d] = before + (uint32_t)__popcll(m);
    }
    __syncthreads();
    // Thread `tid` owns digit `tid`: per-wave starts, the tile's digit starts and
    // the global start of this tile's run of the digit.
    const uint32_t c0 = s_cnt[0][tid], c1 = s_cnt[1][tid], c2 = s_cnt[2][tid], c3 = s_cnt[3][tid];
    uint32_t all;
    const uint32_t tstart = block_exclusive_scan(c0 + c1 + c2 + c3, &all);   // barriers inside
    const uint32_t dbase = block_exclusive_scan(dtot[tid], &all);
    s_cnt[0][tid] = tstart;
    s_cnt[1][tid] = tstart + c0;
    s_cnt[2][tid] = tstart + c0 + c1;
    s_cnt[3][tid] = tstart + c0 + c1 + c2;
    s_tstart[tid] = tstart;
    s_gbase[tid] = dbase + hist[(int64_t)tid * ntiles + t];
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kItems; ++r) {
        const uint32_t d = (k[r] >> shift) & mask;
        pos[r] += s_cnt[wv][d];          // tile-local sorted position
        if (li0 + r * kWave < lim) s_dig[pos[r]] = (uint8_t)d;
    }
    __syncthreads();
    uint32_t gp[kItems];                  // output position of tile-sorted slot tid + j * kBlock
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
        const int i = tid + j * kBlock;
        gp[j] = 0xffffffffu;
        if (i < lim) {
            const uint32_t d = s_dig[i];
            gp[j] = s_gbase[d] + ((uint32_t)i - s_tstart[d]);
        }
    }
    // Regroup each payload through LDS, then write it out in digit runs.  The
    // ordinal and endpoint payloads are read only now, which keeps few
    // registers live across the ranking (more resident blocks per CU).
    auto emit = [&](const uint32_t(&src)[kItems], uint32_t *__restrict__ out) {
#pragma unroll
        for (int r = 0; r < kItems; ++r)
            if (li0 + r * kWave < lim) s_buf[pos[r]] = src[r];
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kItems; ++j)
            if ((int64_t)gp[j] < count) out[gp[j]] = s_buf[tid + j * kBlock];
        __syncthreads();
    };
    if (kWriteKeys) emit(k, pl.keys_out);
    {
        uint32_t v[kItems];
        const uint32_t *vin = kIotaVals ? nullptr : pl.vals_in + tbase;
#pragma unroll
        for (int r = 0; r < kItems; ++r) {
            const int li = li0 + r * kWave;
            if (kIotaVals) v[r] = (uint32_t)tbase + (uint32_t)li;
            else v[r] = li < lim ? vin[li] : 0u;
        }
        emit(v, pl.vals_out);
    }
    if (kOther) {
        uint32_t o[kItems];
        const uint32_t *oin = pl.other_in + tbase;
#pragma unroll
        for (int r = 0; r < kItems; ++r) {
            const int li = li0 + r * kWave;
            o[r] = li < lim ? oin[li] : 0u;
        }
        emit(o, pl.other_out);
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

// ------------------------------------------------------------------ host side
int64_t tiles_for(int64_t count) { return count > 0 ? (count + kTile - 1) / kTile : 1; }

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

template <class KeySrc, bool kIota, bool kOther, bool kWriteKeys>
mp_status radix_pass(KeySrc keys, const Payload &pl, int64_t count, int shift, int bits,
                     uint32_t *hist, uint32_t *dtot, hipStream_t s) {
    const int64_t ntiles = tiles_for(count);
    rs_upsweep<KeySrc><<<(unsigned)ntiles, kBlock, 0, s>>>(keys, count, shift, bits, ntiles, hist);
    rs_scan<<<kBins, kBlock, 0, s>>>(hist, ntiles, dtot);
    rs_downsweep<KeySrc, kIota, kOther, kWriteKeys><<<(unsigned)ntiles, kBlock, 0, s>>>(
        keys, pl, count, shift, bits, ntiles, hist, dtot);
    MP_HIP_CHECK(hipGetLastError(), "radix pass launch");
    return MP_OK;
}

// Stable sort of the edges by key[0..e): the final pass writes the sorted keys
// to one of k0 / k1 (*sorted), the ordinals to `order` and other[order[p]] to `col`.
mp_status sort_edges(const int32_t *key, const int32_t *other, int64_t e, int64_t n,
                     uint32_t *k0, uint32_t *k1, uint32_t *v0, uint32_t *o0, uint32_t *hist,
                     uint32_t *dtot, int32_t *order, int32_t *col, const uint32_t **sorted,
                     hipStream_t s) {
    const int bits = key_bits(n);
    const int passes = (bits + kDigitBits - 1) / kDigitBits;
    const uint32_t *kin = reinterpret_cast<const uint32_t *>(key);
    Payload pl;
    pl.vals_in = nullptr;
    pl.other_in = reinterpret_cast<const uint32_t *>(other);
    uint32_t *kbuf[2] = {k0, k1};
    for (int pass = 0; pass < passes; ++pass) {
        // Split the key bits evenly over the passes (21 bits -> 7 + 7 + 7): fewer
        // bins per pass than 8 + 8 + 5 gives longer output runs per tile.
        const int per = (bits + passes - 1) / passes;
        const int shift = pass * per;
        const int pb = bits - shift < per ? bits - shift : per;
        // Payloads alternate between the outputs and v0 / o0 so that the last
        // pass lands in `order` and `col`.
        const bool to_out = (passes - 1 - pass) % 2 == 0;
        pl.keys_out = kbuf[pass % 2];
        pl.vals_out = to_out ? reinterpret_cast<uint32_t *>(order) : v0;
        pl.other_out = to_out ? reinterpret_cast<uint32_t *>(col) : o0;
        mp_status st = pass == 0
            ? radix_pass<KeysFromArray, true, true, true>(KeysFromArray{kin}, pl, e, shift, pb,
                                                           hist, dtot, s)
            : radix_pass<KeysFromArray, false, true, true>(KeysFromArray{kin}, pl, e, shift, pb,
                                                            hist, dtot, s);
        if (st != MP_OK) return st;
        kin = pl.keys_out;
        pl.vals_in = pl.vals_out;
        pl.other_in = pl.other_out;
    }
    *sorted = kin;
    return MP_OK;
}

mp_status lower_direction(const int32_t *key, const int32_t *other, int64_t e, int64_t n,
                          uint32_t *k0, uint32_t *k1, uint32_t *v0, uint32_t *o0, uint32_t *hist,
                          uint32_t *dtot, int32_t *rowptr, int32_t *col, int32_t *order,
                          hipStream_t s) {
    const uint32_t *sorted = k0;
    if (e > 0) {
        mp_status st = sort_edges(key, other, e, n, k0, k1, v0, o0, hist, dtot, order, col,
                                  &sorted, s);
        if (st != MP_OK) return st;
    }
    rowptr_kernel<<<grid_for(n + 1), kBlock, 0, s>>>(sorted, e, n, rowptr);
    MP_HIP_CHECK(hipGetLastError(), "row pointer launch");
    return MP_OK;
}

mp_status plan_direction(const int32_t *rowptr, int64_t n, uint32_t *hist, uint32_t *totals,
                         int32_t *plan, hipStream_t s) {
    Payload pl;
    pl.vals_in = nullptr;
    pl.other_in = nullptr;
    pl.keys_out = nullptr;
    pl.vals_out = reinterpret_cast<uint32_t *>(plan);
    pl.other_out = nullptr;
    return radix_pass<KeysFromDegree, true, false, false>(KeysFromDegree{rowptr}, pl, n, 0,
                                                          kPlanBits, hist, totals, s);
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

LowerLayout lower_layout(int64_t n, int64_t e) {
    LowerLayout L;
    size_t off = 0;
    const size_t ebytes = align_up((size_t)(e > 0 ? e : 1) * sizeof(uint32_t));
    const int64_t most = e > n ? e : n;
    L.k0 = off; off += ebytes;
    L.k1 = off; off += ebytes;
    L.v0 = off; off += ebytes;
    L.o0 = off; off += ebytes;
    L.hist = off; off += align_up((size_t)kBins * tiles_for(most) * sizeof(uint32_t));
    L.dtot = off; off += align_up(kBins * sizeof(uint32_t));
    L.total = off;
    return L;
}

mp_status lower_read_info(mp_graph *g, hipStream_t s, int *bad_index) {
    uint32_t host[MP_GRAPH_INFO_WORDS];
    MP_HIP_CHECK(hipMemcpyAsync(host, g->info, sizeof(host), hipMemcpyDeviceToHost, s),
                 "copy of build results to host");
    MP_HIP_CHECK(hipStreamSynchronize(s), "build synchronisation");
    *bad_index = host[kInfoFlag] != 0u;
    for (int c = 0; c < MP_NUM_CLASSES; ++c) {
        g->class_count[c] = host[kInfoPlanF + (32 - c)];
        g->class_count_t[c] = host[kInfoPlanT + (32 - c)];
    }
    return MP_OK;
}

mp_status lower_run(const void *src, const void *dst, mp_dtype idx_dtype, int64_t n, int64_t e,
                    mp_graph *g, void *ws, hipStream_t s, bool async, int *bad_index) {
    const LowerLayout L = lower_layout(n, e);
    char *base = static_cast<char *>(ws);
    uint32_t *k0 = reinterpret_cast<uint32_t *>(base + L.k0);
    uint32_t *k1 = reinterpret_cast<uint32_t *>(base + L.k1);
    uint32_t *v0 = reinterpret_cast<uint32_t *>(base + L.v0);
    uint32_t *o0 = reinterpret_cast<uint32_t *>(base + L.o0);
    uint32_t *hist = reinterpret_cast<uint32_t *>(base + L.hist);
    uint32_t *dtot = reinterpret_cast<uint32_t *>(base + L.dtot);
    uint32_t *info = g->info;

    // A fill kernel, not a memset: the sequence stays valid under graph capture.
    zero_words_kernel<<<1, kBlock, 0, s>>>(info, MP_GRAPH_INFO_WORDS);
    if (e > 0) {
        if (idx_dtype == MP_I64)
            intake_kernel<int64_t><<<grid_for(e), kBlock, 0, s>>>(
                static_cast<const int64_t *>(src), static_cast<const int64_t *>(dst), e, n, g->src,
                g->dst, info + kInfoFlag);
        else
            intake_kernel<int32_t><<<grid_for(e), kBlock, 0, s>>>(
                static_cast<const int32_t *>(src), static_cast<const int32_t *>(dst), e, n, g->src,
                g->dst, info + kInfoFlag);
    }
    MP_HIP_CHECK(hipGetLastError(), "intake launch");

    mp_status st = lower_direction(g->dst, g->src, e, n, k0, k1, v0, o0, hist, dtot, g->rowptr,
                                   g->col, g->edge_order, s);
    if (st != MP_OK) return st;
    st = lower_direction(g->src, g->dst, e, n, k0, k1, v0, o0, hist, dtot, g->rowptr_t, g->col_t,
                         g->transpose_order, s);
    if (st != MP_OK) return st;
    st = plan_direction(g->rowptr, n, hist, info + kInfoPlanF, g->row_plan, s);
    if (st != MP_OK) return st;
    st = plan_direction(g->rowptr_t, n, hist, info + kInfoPlanT, g->row_plan_t, s);
    if (st != MP_OK) return st;

    *bad_index = 0;
    if (async) {
        for (int c = 0; c < MP_NUM_CLASSES; ++c) g->class_count[c] = g->class_count_t[c] = 0;
        return MP_OK;
    }
    return lower_read_info(g, s, bad_index);
}

}  // namespace mp
