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
// (key, ordinal) pairs with digits of at most 8 bits.  Each pass is three kernels:
//   upsweep   -- every block counts the digits of its 4096-key tile;
//   scan      -- one block per digit turns the per-tile counts into offsets;
//   downsweep -- every block re-reads its tile, ranks each key among equal
//                digits with 64-lane ballots (stable: rank order = input order),
//                regroups the tile by digit in LDS and writes it out in runs.
// The intake already counts the first pass's digits of both keys, so the
// first pass of each direction starts at its scan.  Small edge
// lists (a sampled minibatch) are launch-bound rather than bandwidth-bound, so
// there both directions share every launch and, when a pass has few tiles,
// each downsweep block sums the per-tile counts it needs itself (no scan
// kernel).
// Block-local ranks, never atomics, decide where equal keys land, so the
// result is the unique stable order.  The opposite endpoint travels with each
// key, so the last pass writes col[p] = other[order[p]] directly.  Rows are
// then delimited by a binary search per row over the sorted keys.
#include "common.h"

namespace mp {
namespace {

constexpr int kItems = 16;                        // keys per thread per tile (large lists)
constexpr int kItemsSmall = 4;                    // the same for small lists: 1024-key tiles,
                                                  // four times the blocks per pass
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

// Plan key of a row of length d: 32 - class(d), so the highest class sorts
// first (class 0 for d = 0, else the number of binary digits of d).
__device__ __forceinline__ uint32_t plan_key(uint32_t d) {
    const uint32_t c = d == 0 ? 0u : 32u - (uint32_t)__clz(d);
    return 32u - c;
}

// Plan key of row i from the row pointers.
struct KeysFromDegree {
    const int32_t *rowptr;
    __device__ __forceinline__ KeysFromDegree at(int64_t base) const { return {rowptr + base}; }
    __device__ __forceinline__ uint32_t operator()(int i) const {
        return plan_key((uint32_t)(rowptr[i + 1] - rowptr[i]));
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

// Block -> (direction, tile).  A launch for one direction renumbers its tiles
// per XCD; a launch for both gives blocks [0, ntiles) to direction 0 and the
// rest to direction 1.
template <bool kDual>
__device__ __forceinline__ int64_t block_tile(int64_t ntiles, int &dir) {
    if constexpr (kDual) {
        const int64_t b = blockIdx.x;
        dir = b >= ntiles ? 1 : 0;
        return dir ? b - ntiles : b;
    } else {
        dir = 0;
        return xcd_local_tile();
    }
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

// One direction's share of a pass.
template <class KeySrc>
struct PassDir {
    KeySrc keys;
    Payload pl;
    uint32_t *hist;   // [kBins * ntiles] per-tile digit counts, digit-major
    uint32_t *dtot;   // [kBins] digit totals (from the scan, or from tile 0 of an
                      // inline-scan downsweep when not nullptr)
};

// Digit counts of one tile: k[r] is the key at tile-local index li0 + r * 64,
// valid below lim.  Writes hist[d * ntiles + t] for every digit d.  Contains
// barriers: every thread of the block calls it.
template <int IT>
__device__ __forceinline__ void tile_digit_counts(const uint32_t (&k)[IT], int li0, int lim,
                                                  int shift, uint32_t mask,
                                                  uint32_t *__restrict__ hist, int64_t ntiles,
                                                  int64_t t) {
    __shared__ uint32_t s_cnt[kWavesPerBlock][kBins];
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    for (int i = threadIdx.x; i < kWavesPerBlock * kBins; i += kBlock) (&s_cnt[0][0])[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < IT; ++r) {
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

template <class KeySrc, bool kDual, int IT>
__global__ __launch_bounds__(kBlock) void rs_upsweep(PassDir<KeySrc> a0, PassDir<KeySrc> a1,
                                                     int64_t count, int shift, int bits,
                                                     int64_t ntiles) {
    int dir;
    const int64_t t = block_tile<kDual>(ntiles, dir);
    const PassDir<KeySrc> &a = dir ? a1 : a0;
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const uint32_t mask = (1u << bits) - 1u;
    const int64_t left = count - t * (kBlock * IT);
    const int lim = left < (kBlock * IT) ? (int)left : (kBlock * IT);        // keys in this tile
    const KeySrc tk = a.keys.at(t * (kBlock * IT));
    const int li0 = wv * (kWave * IT) + lane;                   // tile-local index, round 0
    uint32_t k[IT];
#pragma unroll
    for (int r = 0; r < IT; ++r) {
        const int li = li0 + r * kWave;
        k[r] = li < lim ? tk(li) : 0u;
    }
    tile_digit_counts(k, li0, lim, shift, mask, a.hist, ntiles, t);
}

// Intake: block t copies tile t of the caller's endpoints to int32, checking
// 0 <= v < n (an out-of-range value is stored as 0, so later kernels stay in
// bounds, and raises the flag), and writes the first pass's digit counts of
// both keys, dst for the forward sort and src for the transpose sort, so the
// first pass of each direction needs no upsweep of its own.  Tiles as in the
// radix passes (IT keys per thread, digit-major counts).
template <typename IdxT, int IT>
__global__ __launch_bounds__(kBlock) void intake_count_kernel(
    const IdxT *__restrict__ src, const IdxT *__restrict__ dst, int64_t e, int64_t n,
    int32_t *__restrict__ src32, int32_t *__restrict__ dst32, uint32_t *__restrict__ flag,
    int bits, uint32_t *__restrict__ hist_f, uint32_t *__restrict__ hist_t, int64_t ntiles) {
    const int64_t t = xcd_local_tile();
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int64_t tbase = t * (kBlock * IT);
    const int64_t left = e - tbase;
    const int lim = left < (kBlock * IT) ? (int)left : (kBlock * IT);
    const int li0 = wv * (kWave * IT) + lane;
    uint32_t kd[IT], ks[IT];
    bool bad = false;
#pragma unroll
    for (int r = 0; r < IT; ++r) {
        const int li = li0 + r * kWave;
        kd[r] = ks[r] = 0u;
        if (li < lim) {
            const int64_t sv = (int64_t)src[tbase + li];
            const int64_t dv = (int64_t)dst[tbase + li];
            const bool ok_s = sv >= 0 && sv < n;
            const bool ok_d = dv >= 0 && dv < n;
            ks[r] = ok_s ? (uint32_t)sv : 0u;
            kd[r] = ok_d ? (uint32_t)dv : 0u;
            src32[tbase + li] = (int32_t)ks[r];
            dst32[tbase + li] = (int32_t)kd[r];
            bad |= !(ok_s && ok_d);
        }
    }
    if (bad) *flag = 1u;   // plain store: every writer stores the same value
    const uint32_t mask = (1u << bits) - 1u;
    tile_digit_counts(kd, li0, lim, 0, mask, hist_f, ntiles, t);
    __syncthreads();       // the counts' LDS is reused by the second key
    tile_digit_counts(ks, li0, lim, 0, mask, hist_t, ntiles, t);
}

// One block per digit (and direction): exclusive scan, in tile order, of that
// digit's per-tile counts (in place), and the digit's total.
template <bool kDual>
__global__ __launch_bounds__(kBlock) void rs_scan(uint32_t *__restrict__ hist0,
                                                  uint32_t *__restrict__ dtot0,
                                                  uint32_t *__restrict__ hist1,
                                                  uint32_t *__restrict__ dtot1, int64_t ntiles) {
    constexpr int kPer = 16;
    const int dir = kDual && blockIdx.x >= kBins ? 1 : 0;
    const int digit = blockIdx.x - dir * kBins;
    uint32_t *row = (dir ? hist1 : hist0) + (int64_t)digit * ntiles;
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
    if (threadIdx.x == 0) (dir ? dtot1 : dtot0)[digit] = carry;
}

// kInlineScan: hist holds raw per-tile counts (no scan kernel ran); each thread
// sums its digit's counts over all tiles and over the tiles before this one.
template <class KeySrc, bool kIotaVals, bool kOther, bool kWriteKeys, bool kDual,
          bool kInlineScan, int IT>
__global__ __launch_bounds__(kBlock) void rs_downsweep(PassDir<KeySrc> a0, PassDir<KeySrc> a1,
                                                       int64_t count, int shift, int bits,
                                                       int64_t ntiles) {
    __shared__ uint32_t s_buf[(kBlock * IT)];          // one payload at a time, in tile-sorted order
    __shared__ uint8_t s_dig[(kBlock * IT)];           // digit of each tile-sorted position
    __shared__ uint32_t s_cnt[kWavesPerBlock][kBins];
    __shared__ uint32_t s_tstart[kBins];
    __shared__ uint32_t s_gbase[kBins];
    int dir;
    const int64_t t = block_tile<kDual>(ntiles, dir);
    const PassDir<KeySrc> &a = dir ? a1 : a0;
    const Payload &pl = a.pl;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wv = tid / kWave;
    const uint32_t mask = (1u << bits) - 1u;
    const uint64_t lanes_below = (1ull << lane) - 1ull;
    const int64_t tbase = t * (kBlock * IT);
    const int64_t left = count - tbase;
    const int lim = left < (kBlock * IT) ? (int)left : (kBlock * IT);        // keys in this tile
    const KeySrc tk = a.keys.at(tbase);
    const int li0 = wv * (kWave * IT) + lane;                   // tile-local index, round 0

    for (int i = tid; i < kWavesPerBlock * kBins; i += kBlock) (&s_cnt[0][0])[i] = 0u;
    uint32_t k[IT];
#pragma unroll
    for (int r = 0; r < IT; ++r) {
        const int li = li0 + r * kWave;
        k[r] = li < lim ? tk(li) : 0u;
    }
    __syncthreads();
    // Rank inside the wave: earlier rounds (running count) + lower lanes now.
    uint32_t pos[IT];
#pragma unroll
    for (int r = 0; r < IT; ++r) {
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
    uint32_t dsum, before_tile;
    if constexpr (kInlineScan) {
        // 16 independent loads in flight per step (ntiles is small here).
        const uint32_t *row = a.hist + (int64_t)tid * ntiles;
        dsum = 0u;
        before_tile = 0u;
        for (int64_t u0 = 0; u0 < ntiles; u0 += 16) {
            uint32_t c[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) c[j] = u0 + j < ntiles ? row[u0 + j] : 0u;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                dsum += c[j];
                before_tile += u0 + j < t ? c[j] : 0u;
            }
        }
        if (t == 0 && a.dtot) a.dtot[tid] = dsum;
    } else {
        dsum = a.dtot[tid];
        before_tile = a.hist[(int64_t)tid * ntiles + t];
    }
    const uint32_t dbase = block_exclusive_scan(dsum, &all);
    s_cnt[0][tid] = tstart;
    s_cnt[1][tid] = tstart + c0;
    s_cnt[2][tid] = tstart + c0 + c1;
    s_cnt[3][tid] = tstart + c0 + c1 + c2;
    s_tstart[tid] = tstart;
    s_gbase[tid] = dbase + before_tile;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < IT; ++r) {
        const uint32_t d = (k[r] >> shift) & mask;
        pos[r] += s_cnt[wv][d];          // tile-local sorted position
        if (li0 + r * kWave < lim) s_dig[pos[r]] = (uint8_t)d;
    }
    __syncthreads();
    uint32_t gp[IT];                  // output position of tile-sorted slot tid + j * kBlock
#pragma unroll
    for (int j = 0; j < IT; ++j) {
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
    auto emit = [&](const uint32_t(&src)[IT], uint32_t *__restrict__ out) {
#pragma unroll
        for (int r = 0; r < IT; ++r)
            if (li0 + r * kWave < lim) s_buf[pos[r]] = src[r];
        __syncthreads();
#pragma unroll
        for (int j = 0; j < IT; ++j)
            if ((int64_t)gp[j] < count) out[gp[j]] = s_buf[tid + j * kBlock];
        __syncthreads();
    };
    if (kWriteKeys) emit(k, pl.keys_out);
    {
        uint32_t v[IT];
        const uint32_t *vin = kIotaVals ? nullptr : pl.vals_in + tbase;
#pragma unroll
        for (int r = 0; r < IT; ++r) {
            const int li = li0 + r * kWave;
            if (kIotaVals) v[r] = (uint32_t)tbase + (uint32_t)li;
            else v[r] = li < lim ? vin[li] : 0u;
        }
        emit(v, pl.vals_out);
    }
    if (kOther) {
        uint32_t o[IT];
        const uint32_t *oin = pl.other_in + tbase;
#pragma unroll
        for (int r = 0; r < IT; ++r) {
            const int li = li0 + r * kWave;
            o[r] = li < lim ? oin[li] : 0u;
        }
        emit(o, pl.other_out);
    }
}

// ------------------------------------------------------------------ rows
// One direction's row pointers: rowptr[i] = number of sorted keys below i.
struct RowsDir {
    const uint32_t *sorted;   // the direction's keys in sorted order [e]
    int32_t *rowptr;          // [n + 1]
};

// One thread per row pointer (binary search over the sorted keys); with kDual
// the first half of the grid serves r0, the second half r1.
template <bool kDual>
__global__ __launch_bounds__(kBlock) void rowptr_kernel(RowsDir r0, RowsDir r1, int64_t e,
                                                        int64_t n, int64_t blocks_per_dir) {
    int64_t b = blockIdx.x;
    const int dir = kDual && b >= blocks_per_dir ? 1 : 0;
    b -= dir * blocks_per_dir;
    const RowsDir &r = dir ? r1 : r0;
    const int64_t stride = blocks_per_dir * kBlock;
    for (int64_t i = b * kBlock + threadIdx.x; i <= n; i += stride) {
        int64_t lo = 0, hi = e;
        while (lo < hi) {
            const int64_t mid = (lo + hi) >> 1;
            if ((int64_t)r.sorted[mid] < i) lo = mid + 1;
            else hi = mid;
        }
        r.rowptr[i] = (int32_t)lo;
    }
}

// ------------------------------------------------------------------ host side
int64_t tiles_for(int64_t count, int it) {
    const int64_t tile = (int64_t)kBlock * it;
    return count > 0 ? (count + tile - 1) / tile : 1;
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

// Width of the first pass's digit, as sort_edges splits the key bits.
int first_pass_bits(int64_t n) {
    const int bits = key_bits(n);
    const int passes = (bits + kDigitBits - 1) / kDigitBits;
    const int per = (bits + passes - 1) / passes;
    return per < bits ? per : bits;
}

// Counting intake over tiles of 256 * IT edges.
template <int IT>
void intake_count(const void *src, const void *dst, mp_dtype idx_dtype, int64_t e, int64_t n,
                  mp_graph *g, int first_bits, uint32_t *hist_f, uint32_t *hist_t,
                  hipStream_t s) {
    const int64_t nt = tiles_for(e, IT);
    if (idx_dtype == MP_I64)
        intake_count_kernel<int64_t, IT><<<(unsigned)nt, kBlock, 0, s>>>(
            static_cast<const int64_t *>(src), static_cast<const int64_t *>(dst), e, n, g->src,
            g->dst, g->info + kInfoFlag, first_bits, hist_f, hist_t, nt);
    else
        intake_count_kernel<int32_t, IT><<<(unsigned)nt, kBlock, 0, s>>>(
            static_cast<const int32_t *>(src), static_cast<const int32_t *>(dst), e, n, g->src,
            g->dst, g->info + kInfoFlag, first_bits, hist_f, hist_t, nt);
}


// Edge lists up to this size run both directions in every launch (their
// workspace then holds a second set of sort buffers).
constexpr int64_t kDualMaxEdges = (int64_t)1 << 22;
// Passes over at most this many tiles sum the per-tile counts inside the
// downsweep instead of launching the scan.
constexpr int64_t kInlineScanMaxTiles = 64;

bool dual_mode(int64_t e) { return e <= kDualMaxEdges; }

// One radix pass for one direction (d1 unused) or both (kDual), with tiles of
// 256 * IT keys.
// counted: the per-tile digit counts are already in hist (the counting intake).
template <class KeySrc, bool kIota, bool kOther, bool kWriteKeys, bool kDual, int IT>
mp_status radix_pass(const PassDir<KeySrc> &d0, const PassDir<KeySrc> &d1, int64_t count,
                     int shift, int bits, hipStream_t s, bool counted = false) {
    const int64_t ntiles = tiles_for(count, IT);
    const unsigned grid = (unsigned)((kDual ? 2 : 1) * ntiles);
    if (!counted)
        rs_upsweep<KeySrc, kDual, IT><<<grid, kBlock, 0, s>>>(d0, d1, count, shift, bits,
                                                              ntiles);
    if (ntiles <= kInlineScanMaxTiles) {
        rs_downsweep<KeySrc, kIota, kOther, kWriteKeys, kDual, true, IT>
            <<<grid, kBlock, 0, s>>>(d0, d1, count, shift, bits, ntiles);
    } else {
        rs_scan<kDual><<<(kDual ? 2 : 1) * kBins, kBlock, 0, s>>>(d0.hist, d0.dtot, d1.hist,
                                                                   d1.dtot, ntiles);
        rs_downsweep<KeySrc, kIota, kOther, kWriteKeys, kDual, false, IT>
            <<<grid, kBlock, 0, s>>>(d0, d1, count, shift, bits, ntiles);
    }
    MP_HIP_CHECK(hipGetLastError(), "radix pass launch");
    return MP_OK;
}

// Sort buffers of one direction.
struct SortBufs {
    uint32_t *k0, *k1, *v0, *o0, *hist, *dtot;
};

// One direction of the edge sort: keys, the opposite endpoint, and where the
// final pass puts the ordinals (order) and endpoints (col).
struct EdgeDir {
    const int32_t *key;
    const int32_t *other;
    int32_t *order;
    int32_t *col;
    SortBufs b;
};

// Stable sort of the edges by key for each direction given: the final pass
// writes the ordinals to `order` and other[order[p]] to `col`; sorted[i]
// receives the buffer holding direction i's sorted keys.  kDual: both
// directions in every launch; else dirs[0] only.
// first_counted: the first pass's per-tile counts are already in the hist
// buffers (the counting intake).
template <bool kDual>
mp_status sort_edges(const EdgeDir *dirs, int64_t e, int64_t n, const uint32_t **sorted,
                     hipStream_t s, bool first_counted = false) {
    constexpr int kDirs = kDual ? 2 : 1;
    const int bits = key_bits(n);
    const int passes = (bits + kDigitBits - 1) / kDigitBits;
    PassDir<KeysFromArray> pd[2];
    const uint32_t *kin[2];
    for (int i = 0; i < kDirs; ++i) {
        kin[i] = reinterpret_cast<const uint32_t *>(dirs[i].key);
        pd[i].pl.vals_in = nullptr;
        pd[i].pl.other_in = reinterpret_cast<const uint32_t *>(dirs[i].other);
        pd[i].hist = dirs[i].b.hist;
        pd[i].dtot = dirs[i].b.dtot;
    }
    if (!kDual) pd[1] = pd[0];
    for (int pass = 0; pass < passes; ++pass) {
        // Split the key bits evenly over the passes (21 bits -> 7 + 7 + 7): fewer
        // bins per pass than 8 + 8 + 5 gives longer output runs per tile.
        const int per = (bits + passes - 1) / passes;
        const int shift = pass * per;
        const int pb = bits - shift < per ? bits - shift : per;
        // Payloads alternate between the outputs and v0 / o0 so that the last
        // pass lands in `order` and `col`.
        const bool to_out = (passes - 1 - pass) % 2 == 0;
        for (int i = 0; i < kDirs; ++i) {
            const SortBufs &b = dirs[i].b;
            pd[i].keys = KeysFromArray{kin[i]};
            pd[i].pl.keys_out = pass % 2 == 0 ? b.k0 : b.k1;
            pd[i].pl.vals_out = to_out ? reinterpret_cast<uint32_t *>(dirs[i].order) : b.v0;
            pd[i].pl.other_out = to_out ? reinterpret_cast<uint32_t *>(dirs[i].col) : b.o0;
        }
        if (!kDual) pd[1] = pd[0];
        // Small lists (both directions per launch) use small tiles.
        constexpr int IT = kDual ? kItemsSmall : kItems;
        mp_status st = pass == 0
            ? radix_pass<KeysFromArray, true, true, true, kDual, IT>(pd[0], pd[1], e, shift, pb, s,
                                                                    first_counted)
            : radix_pass<KeysFromArray, false, true, true, kDual, IT>(pd[0], pd[1], e, shift, pb,
                                                                     s);
        if (st != MP_OK) return st;
        for (int i = 0; i < kDirs; ++i) {
            kin[i] = pd[i].pl.keys_out;
            pd[i].pl.vals_in = pd[i].pl.vals_out;
            pd[i].pl.other_in = pd[i].pl.other_out;
        }
    }
    for (int i = 0; i < kDirs; ++i) sorted[i] = kin[i];
    return MP_OK;
}

// Row pointers of one direction (r1 unused) or both (kDual).
template <bool kDual>
mp_status row_pointers(const RowsDir &r0, const RowsDir &r1, int64_t e, int64_t n,
                       hipStream_t s) {
    const int64_t per_dir = grid_for(n + 1);
    rowptr_kernel<kDual><<<(unsigned)((kDual ? 2 : 1) * per_dir), kBlock, 0, s>>>(
        r0, r1, e, n, per_dir);
    MP_HIP_CHECK(hipGetLastError(), "row pointer launch");
    return MP_OK;
}

// Degree plans of both directions from their row pointers: one radix pass on
// the plan key, both directions in each launch (its scan only when there are
// many row tiles).  The digit totals, i.e. the rows per class, land in
// totals0 / totals1.
template <int IT>
mp_status plans(int64_t n, mp_graph *g, uint32_t *hist0, uint32_t *hist1, uint32_t *totals0,
                uint32_t *totals1, hipStream_t s) {
    PassDir<KeysFromDegree> p0, p1;
    p0.keys = KeysFromDegree{g->rowptr};
    p1.keys = KeysFromDegree{g->rowptr_t};
    p0.pl = Payload{nullptr, nullptr, nullptr, reinterpret_cast<uint32_t *>(g->row_plan), nullptr};
    p1.pl = Payload{nullptr, nullptr, nullptr, reinterpret_cast<uint32_t *>(g->row_plan_t),
                    nullptr};
    p0.hist = hist0;
    p1.hist = hist1;
    p0.dtot = totals0;
    p1.dtot = totals1;
    return radix_pass<KeysFromDegree, true, false, false, true, IT>(p0, p1, n, 0, kPlanBits, s);
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

LowerLayout lower_layout(int64_t n, int64_t e) {
    LowerLayout L;
    size_t off = 0;
    const size_t ebytes = align_up((size_t)(e > 0 ? e : 1) * sizeof(uint32_t));
    const int64_t most = e > n ? e : n;
    const int it = dual_mode(e) ? kItemsSmall : kItems;
    const size_t hbytes = align_up((size_t)kBins * tiles_for(most, it) * sizeof(uint32_t));
    for (int i = 0; i < 2; ++i) {
        if (i == 1 && !dual_mode(e)) {   // one direction at a time: one set of sort buffers
            L.k0[1] = L.k0[0];
            L.k1[1] = L.k1[0];
            L.v0[1] = L.v0[0];
            L.o0[1] = L.o0[0];
        } else {
            L.k0[i] = off; off += ebytes;
            L.k1[i] = off; off += ebytes;
            L.v0[i] = off; off += ebytes;
            L.o0[i] = off; off += ebytes;
        }
        L.hist[i] = off; off += hbytes;
        L.dtot[i] = off; off += align_up(kBins * sizeof(uint32_t));
    }
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
    auto at = [&](size_t off) { return reinterpret_cast<uint32_t *>(base + off); };
    SortBufs b[2];
    for (int i = 0; i < 2; ++i)
        b[i] = SortBufs{at(L.k0[i]), at(L.k1[i]), at(L.v0[i]), at(L.o0[i]), at(L.hist[i]),
                        at(L.dtot[i])};
    uint32_t *info = g->info;

    // A fill kernel, not a memset: the sequence stays valid under graph capture.
    zero_words_kernel<<<1, kBlock, 0, s>>>(info, MP_GRAPH_INFO_WORDS);
    // The intake also counts the first pass's digits of both keys, in the tiles
    // of that pass (1024 keys when both directions share the launches).
    const bool counted = e > 0;
    if (counted) {
        const int fb = first_pass_bits(n);
        if (dual_mode(e))
            intake_count<kItemsSmall>(src, dst, idx_dtype, e, n, g, fb, b[0].hist, b[1].hist, s);
        else
            intake_count<kItems>(src, dst, idx_dtype, e, n, g, fb, b[0].hist, b[1].hist, s);
    }
    MP_HIP_CHECK(hipGetLastError(), "intake launch");

    // Forward CSR: keyed by destination; transpose CSR: keyed by source.
    const EdgeDir dirs[2] = {{g->dst, g->src, g->edge_order, g->col, b[0]},
                             {g->src, g->dst, g->transpose_order, g->col_t, b[1]}};
    // Sorted keys of each direction (not read when e = 0).  One direction at a
    // time shares the sort buffers, so its row pointers are taken before the
    // other direction's sort overwrites them.
    const uint32_t *sorted[2] = {b[0].k0, b[1].k0};
    mp_status st = MP_OK;
    if (dual_mode(e)) {
        if (e > 0) st = sort_edges<true>(dirs, e, n, sorted, s, counted);
        if (st == MP_OK)
            st = row_pointers<true>(RowsDir{sorted[0], g->rowptr},
                                    RowsDir{sorted[1], g->rowptr_t}, e, n, s);
    } else {
        for (int i = 0; i < 2 && st == MP_OK; ++i) {
            st = sort_edges<false>(&dirs[i], e, n, &sorted[i], s, counted);
            const RowsDir r{sorted[i], i == 0 ? g->rowptr : g->rowptr_t};
            if (st == MP_OK) st = row_pointers<false>(r, r, e, n, s);
        }
    }
    if (st == MP_OK)
        st = dual_mode(e)
            ? plans<kItemsSmall>(n, g, b[0].hist, b[1].hist, info + kInfoPlanF,
                                 info + kInfoPlanT, s)
            : plans<kItems>(n, g, b[0].hist, b[1].hist, info + kInfoPlanF, info + kInfoPlanT, s);
    if (st != MP_OK) return st;

    *bad_index = 0;
    if (async) {
        for (int c = 0; c < MP_NUM_CLASSES; ++c) g->class_count[c] = g->class_count_t[c] = 0;
        return MP_OK;
    }
    return lower_read_info(g, s, bad_index);
}

}  // namespace mp
