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
// delimited by the last pass itself when a list has at least two edges per
// row (each key's first position, see row_heads), else by a binary search per
// row over the sorted keys.
#include "common.h"

#include <mutex>
#include <type_traits>

// The lowering's workspace for mp_graph_build_noalloc, whose callers cannot
// allocate device memory: one array per GPU, held until the process ends.
// Host code never passes its name to a kernel (on the host the name is only a
// stand-in); it takes the device address from static_workspace() below.
static __device__ __align__(256) unsigned char scratch[MP_STATIC_WORKSPACE_BYTES];

namespace mp {
namespace {

constexpr int kItems = 16;                        // keys per thread per tile (large lists)
constexpr int kItemsSmall = 4;                    // the same for small lists: 1024-key tiles,
                                                  // four times the blocks per pass
constexpr int kBins = 256;                        // 8-bit digits
constexpr int kDigitBits = 8;                     // at most 8 bits per pass
constexpr int kPlanBits = 6;                      // plan keys 32 - class lie in [0, 32]
constexpr int kScanSegs = 8;                      // most blocks per digit in the count scan
// Rows of 64 lanes x 16 bytes per wave that copy the segment totals of all
// kBins digits (kBins * kScanSegs words) with the four waves of a block.
constexpr int kSegRowsPerWave = kBins * kScanSegs / (kWave * 4 * kWavesPerBlock);
constexpr int64_t kScanSegTiles = 2048;           // tiles per extra segment

// Segments of a digit's count row: one per 2048 tiles, at most kScanSegs (a
// short row is scanned by one block, as more blocks would only add launch
// work).
__host__ __device__ inline int scan_segs(int64_t ntiles) {
    const int64_t k = ntiles / kScanSegTiles;
    return k < 1 ? 1 : (k > kScanSegs ? kScanSegs : (int)k);
}

// Tiles per segment (the last segment may be shorter).
__host__ __device__ inline int64_t scan_seg_len(int64_t ntiles) {
    const int k = scan_segs(ntiles);
    return (ntiles + k - 1) / k;
}

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

// Exclusive scan over R * kBlock entries held round-wise (entry tid + j * kBlock
// is v[j], so that loads and stores of the entries are coalesced): ex[j] =
// op over the entries before it (kFromLeft) or after it, `none` if there are
// none.  Returns op over all entries.  op is associative and commutative with
// identity `none`.  Contains barriers: every thread of the block calls it.
template <bool kFromLeft, int R, class Op>
__device__ __forceinline__ uint32_t rounds_exclusive(const uint32_t (&v)[R], uint32_t (&ex)[R],
                                                     uint32_t none, Op op) {
    __shared__ uint32_t s_t[R][kWavesPerBlock];
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
#pragma unroll
    for (int j = 0; j < R; ++j) {
        uint32_t inc = v[j];
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            if constexpr (kFromLeft) {
                const uint32_t y = __shfl_up(inc, off);
                if (lane >= off) inc = op(inc, y);
            } else {
                const uint32_t y = __shfl_down(inc, off);
                if (lane + off < kWave) inc = op(inc, y);
            }
        }
        if (lane == (kFromLeft ? kWave - 1 : 0)) s_t[j][wv] = inc;
        // this wave's lanes before (after) this one in the round
        uint32_t w;
        if constexpr (kFromLeft) {
            w = __shfl_up(inc, 1);
            if (lane == 0) w = none;
        } else {
            w = __shfl_down(inc, 1);
            if (lane == kWave - 1) w = none;
        }
        ex[j] = w;
    }
    __syncthreads();
    uint32_t run = none;   // the whole rounds already passed
#pragma unroll
    for (int jj = 0; jj < R; ++jj) {
        const int j = kFromLeft ? jj : R - 1 - jj;
        uint32_t waves = none, all = none;
#pragma unroll
        for (int w = 0; w < kWavesPerBlock; ++w) {
            const uint32_t t = s_t[j][w];
            if (kFromLeft ? w < wv : w > wv) waves = op(waves, t);
            all = op(all, t);
        }
        ex[j] = op(run, op(waves, ex[j]));
        run = op(run, all);
    }
    __syncthreads();
    return run;
}

struct OpSum {
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; }
};
struct OpMax {
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a > b ? a : b; }
};
struct OpMin {
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a < b ? a : b; }
};

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

// What the last pass of an edge sort writes instead of the sorted keys when it
// also delimits the rows (see row_heads): the first position of every key
// that is not the first of its tile's run, and one record per (digit, tile)
// run, digit-major like hist.
struct RowsOut {
    int32_t *rowptr;   // [n + 1]
    uint2 *runs;       // (first key, last key + 1) of the run; (0, 0) if empty
                       // (hist receives the run's output position)
};

// One direction's share of a pass.
template <class KeySrc>
struct PassDir {
    KeySrc keys;
    Payload pl;
    uint32_t *hist;   // [kBins * ntiles] per-tile digit counts, digit-major
    uint32_t *seg;    // [kBins * kScanSegs] per-segment digit totals from the scan
    uint32_t *dtot;   // [kBins] digit totals, written by tile 0 of the downsweep when
                      // not nullptr
    RowsOut rows;     // only for the row-delimiting last pass
    // When flag is not nullptr (the plan pass of a small list), tile 0 of the
    // downsweep also writes *flag = 1 if any of the intake's per-tile range
    // words bad[0 .. nbad) is set, else 0, so the flag needs no clearing
    // launch before the intake.
    const uint32_t *bad = nullptr;
    int64_t nbad = 0;
    uint32_t *flag = nullptr;
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

// Digits of at most this many bits may be counted with tile_lane_counts.
constexpr int kLaneDigitBits = 7;
constexpr int kLaneBins = 1 << kLaneDigitBits;

// The same counts for digits below kLaneBins, with byte counters per lane
// slot instead of matching: word (j, lane) of the block's table holds, one
// byte per digit, how many keys of lane `lane` of any wave have digit 4j,
// 4j+1, 4j+2 or 4j+3, so each key is one LDS add (atomic: the four waves share
// the words) and a wave's adds never meet in a bank.  A byte counts at most
// 4 * IT keys (below 256).  The reduction splits each word into two 16-bit
// fields (digits 4j and 4j+2, 4j+1 and 4j+3) and adds them over the 64 lanes,
// 8 words per thread and then across the 8 threads of a row.  One table of
// 8 KB, not one per wave, so that more blocks fit on a CU.  Digits from
// kLaneBins to kBins - 1 are written as 0.  kVec4: k holds the keys of
// 16-byte loads, tile-local index li0 + (r / 4) * 256 + r % 4 for k[r] (else
// li0 + r * 64).  Contains barriers: every thread of the block calls it.
template <int IT, bool kVec4 = false>
__device__ __forceinline__ void tile_lane_counts(const uint32_t (&k)[IT], int li0, int lim,
                                                 int shift, uint32_t mask,
                                                 uint32_t *__restrict__ hist, int64_t ntiles,
                                                 int64_t t) {
    static_assert(kWavesPerBlock * IT < 256, "a byte holds one lane slot's keys of a digit");
    constexpr int kRows = kLaneBins / 4;                      // words per lane slot
    constexpr int kWords = kRows * kWave;
    static_assert(kWords / 4 <= 2 * kBlock, "two 16-byte stores per thread clear the table");
    __shared__ uint4 s_lc4[kWords / 4];
    uint32_t *s_lc = reinterpret_cast<uint32_t *>(s_lc4);
    const int lane = threadIdx.x & (kWave - 1);
    for (int i = threadIdx.x; i < kWords / 4; i += kBlock) s_lc4[i] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    uint32_t *mine = s_lc + lane;
#pragma unroll
    for (int r = 0; r < IT; ++r) {
        const uint32_t d = (k[r] >> shift) & mask;          // keys past the tile add 0
        const int li = kVec4 ? li0 + (r >> 2) * (kWave * 4) + (r & 3) : li0 + r * kWave;
        const uint32_t one = li < lim ? 1u : 0u;
        __hip_atomic_fetch_add(mine + (d >> 2) * kWave, one << ((d & 3u) * 8u), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    __syncthreads();
    // Thread (j, part) adds the words of lane slots [8 part, 8 part + 8) of row j.
    const int j = threadIdx.x >> 3, part = threadIdx.x & 7;
    uint32_t lo = 0u, hi = 0u;                                // digits (4j, 4j+2), (4j+1, 4j+3)
    {
        const uint4 *q = reinterpret_cast<const uint4 *>(s_lc + j * kWave + part * 8);
        const uint4 x = q[0], y = q[1];
        const uint32_t w[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            lo += w[i] & 0x00ff00ffu;
            hi += (w[i] >> 8) & 0x00ff00ffu;
        }
    }
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) {
        lo += __shfl_xor(lo, off);
        hi += __shfl_xor(hi, off);
    }
    const uint32_t f = (part & 1) ? hi : lo;
    const uint32_t c = (part & 2) ? f >> 16 : f & 0xffffu;
    const int d = part < 4 ? 4 * j + part : kLaneBins + 4 * j + (part - 4);
    hist[(int64_t)d * ntiles + t] = part < 4 ? c : 0u;
}

// Digit counts of a tile by whichever method the template selects.
template <bool kLane, int IT>
__device__ __forceinline__ void count_tile(const uint32_t (&k)[IT], int li0, int lim, int shift,
                                           uint32_t mask, uint32_t *__restrict__ hist,
                                           int64_t ntiles, int64_t t) {
    if constexpr (kLane) tile_lane_counts(k, li0, lim, shift, mask, hist, ntiles, t);
    else tile_digit_counts(k, li0, lim, shift, mask, hist, ntiles, t);
}

// kLane: the pass's digits have at most kLaneDigitBits bits.
// kVec4 (keys from a 16-byte aligned array, lane counts): each lane loads four
// consecutive keys at a time.
template <class KeySrc, bool kDual, bool kLane, int IT, bool kVec4 = false>
__global__ __launch_bounds__(kBlock) void rs_upsweep(PassDir<KeySrc> a0, PassDir<KeySrc> a1,
                                                     int64_t count, int shift, int bits,
                                                     int64_t ntiles) {
    static_assert(!kVec4 || (kLane && IT % 4 == 0), "16-byte loads feed the lane counters");
    int dir;
    const int64_t t = block_tile<kDual>(ntiles, dir);
    const PassDir<KeySrc> &a = dir ? a1 : a0;
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const uint32_t mask = (1u << bits) - 1u;
    const int64_t left = count - t * (kBlock * IT);
    const int lim = left < (kBlock * IT) ? (int)left : (kBlock * IT);        // keys in this tile
    const KeySrc tk = a.keys.at(t * (kBlock * IT));
    uint32_t k[IT];
    if constexpr (kVec4) {
        const int l4 = wv * (kWave * IT) + lane * 4;            // tile-local index of k[0]
#pragma unroll
        for (int q = 0; q < IT / 4; ++q) {
            const int li = l4 + q * (kWave * 4);
            if (li + 3 < lim) {
                const uint4 v = *reinterpret_cast<const uint4 *>(tk.k + li);
                k[4 * q] = v.x;
                k[4 * q + 1] = v.y;
                k[4 * q + 2] = v.z;
                k[4 * q + 3] = v.w;
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) k[4 * q + c] = li + c < lim ? tk.k[li + c] : 0u;
            }
        }
        tile_lane_counts<IT, true>(k, l4, lim, shift, mask, a.hist, ntiles, t);
        return;
    }
    const int li0 = wv * (kWave * IT) + lane;                   // tile-local index, round 0
#pragma unroll
    for (int r = 0; r < IT; ++r) {
        const int li = li0 + r * kWave;
        k[r] = li < lim ? tk(li) : 0u;
    }
    count_tile<kLane>(k, li0, lim, shift, mask, a.hist, ntiles, t);
}

// Intake: block t copies tile t of the caller's endpoints to int32, checking
// 0 <= v < n (an out-of-range value is stored as 0, so later kernels stay in
// bounds, and raises the flag), and writes the first pass's digit counts of
// both keys, dst for the forward sort and src for the transpose sort, so the
// first pass of each direction needs no upsweep of its own.  Tiles as in the
// radix passes (IT keys per thread, digit-major counts).  With bad_tiles (small
// lists) the block writes bad_tiles[t] = 1 or 0 instead of raising *flag, so
// no launch has to clear the flag first (the plan pass reduces the words).
template <typename IdxT, bool kLane, int IT>
__global__ __launch_bounds__(kBlock) void intake_count_kernel(
    const IdxT *__restrict__ src, const IdxT *__restrict__ dst, int64_t e, int64_t n,
    int32_t *__restrict__ src32, int32_t *__restrict__ dst32, uint32_t *__restrict__ flag,
    uint32_t *__restrict__ bad_tiles, int bits, uint32_t *__restrict__ hist_f,
    uint32_t *__restrict__ hist_t, int64_t ntiles) {
    const int64_t t = xcd_local_tile();
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int64_t tbase = t * (kBlock * IT);
    const int64_t left = e - tbase;
    const int lim = left < (kBlock * IT) ? (int)left : (kBlock * IT);
    const int li0 = wv * (kWave * IT) + lane;
    uint32_t kd[IT], ks[IT];
    bool bad = false;
    // Every load is issued before the first store, so that a wave has all of
    // its tile's loads in flight at once.
    int64_t svs[IT], dvs[IT];
#pragma unroll
    for (int r = 0; r < IT; ++r) {
        const int li = li0 + r * kWave;
        svs[r] = li < lim ? (int64_t)src[tbase + li] : 0;
        dvs[r] = li < lim ? (int64_t)dst[tbase + li] : 0;
    }
#pragma unroll
    for (int r = 0; r < IT; ++r) {
        const int li = li0 + r * kWave;
        kd[r] = ks[r] = 0u;
        if (li < lim) {
            const int64_t sv = svs[r];
            const int64_t dv = dvs[r];
            const bool ok_s = sv >= 0 && sv < n;
            const bool ok_d = dv >= 0 && dv < n;
            ks[r] = ok_s ? (uint32_t)sv : 0u;
            kd[r] = ok_d ? (uint32_t)dv : 0u;
            src32[tbase + li] = (int32_t)ks[r];
            dst32[tbase + li] = (int32_t)kd[r];
            bad |= !(ok_s && ok_d);
        }
    }
    if (bad_tiles) {       // the same for the whole block
        const int any = __syncthreads_or((int)bad);
        if (threadIdx.x == 0) bad_tiles[t] = any ? 1u : 0u;
    } else if (bad) {
        *flag = 1u;        // plain store: every writer stores the same value
    }
    const uint32_t mask = (1u << bits) - 1u;
    count_tile<kLane>(kd, li0, lim, 0, mask, hist_f, ntiles, t);
    __syncthreads();       // the counts' LDS is reused by the second key
    count_tile<kLane>(ks, li0, lim, 0, mask, hist_t, ntiles, t);
}

// One block per (direction, digit, segment): exclusive scan, in tile order, of
// that digit's per-tile counts over the segment's tiles (in place), and the
// segment's total.  The downsweep adds the totals of the earlier segments.
// Only the pass's own digits are scanned: the rows of the others hold zeros,
// which are their own exclusive scan.
// kPer counts per thread per step: segments of up to a few hundred tiles take
// one or four, so a short row does not pay for sixteen rounds of scan.
template <bool kDual, int kPer>
__global__ __launch_bounds__(kBlock) void rs_scan(uint32_t *__restrict__ hist0,
                                                  uint32_t *__restrict__ seg0,
                                                  uint32_t *__restrict__ hist1,
                                                  uint32_t *__restrict__ seg1, int64_t ntiles,
                                                  int digits) {
    const int segs = scan_segs(ntiles);
    const int per_dir = digits * segs;
    const int dir = kDual && (int)blockIdx.x >= per_dir ? 1 : 0;
    const int rem = (int)blockIdx.x - dir * per_dir;
    const int digit = rem / segs, sg = rem % segs;
    const int64_t len = scan_seg_len(ntiles);
    const int64_t lo = sg * len;
    const int64_t hi = lo + len < ntiles ? lo + len : ntiles;
    uint32_t *row = (dir ? hist1 : hist0) + (int64_t)digit * ntiles;
    uint32_t carry = 0;
    for (int64_t chunk = lo; chunk < hi; chunk += (int64_t)kBlock * kPer) {
        uint32_t v[kPer], ex[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int64_t i = chunk + threadIdx.x + (int64_t)j * kBlock;
            v[j] = i < hi ? row[i] : 0u;
        }
        const uint32_t total = rounds_exclusive<true>(v, ex, 0u, OpSum{});
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int64_t i = chunk + threadIdx.x + (int64_t)j * kBlock;
            if (i < hi) row[i] = carry + ex[j];
        }
        carry += total;
    }
    if (threadIdx.x == 0) (dir ? seg1 : seg0)[digit * kScanSegs + sg] = carry;
}

// Rows from the last pass of an edge sort, in place of writing the sorted keys
// for a search.  The tile's keys are regrouped into buf in tile-sorted order; a
// tile's run of one digit is written to consecutive output positions, so
// inside a run (buf[i - 1] of the same digit) the key before slot i is
// buf[i - 1].  Where it differs, slot i holds the first edge of its key:
// rowptr[key] = its position.  The first slot of a run has its predecessor in
// another tile; the run's record (first key, last key + 1; its output
// position in hist) lets rows_fixup_kernel settle it.  Keys that occur
// nowhere keep the marker rows_init_kernel wrote (rows_apply_kernel fills
// them).  Contains barriers: every thread of the block calls it.
template <int IT>
__device__ __forceinline__ void row_heads(const uint32_t (&k)[IT], const uint32_t (&pos)[IT],
                                          const uint32_t (&gp)[IT], int li0, int lim,
                                          uint32_t *buf, int shift, uint32_t mask,
                                          const uint32_t *tstart, const uint32_t *gbase,
                                          int digits, const RowsOut &ro,
                                          uint32_t *__restrict__ hist, int64_t ntiles,
                                          int64_t t) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int r = 0; r < IT; ++r)
        if (li0 + r * kWave < lim) buf[pos[r]] = k[r];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < IT; ++j) {
        const int i = tid + j * kBlock;
        if (i > 0 && i < lim) {
            const uint32_t key = buf[i], prev = buf[i - 1];
            if (key != prev && (((key ^ prev) >> shift) & mask) == 0u)
                ro.rowptr[key] = (int32_t)gp[j];
        }
    }
    if (tid < digits) {
        const uint32_t b = tstart[tid];
        const uint32_t end = tid + 1 < kBins ? tstart[tid + 1] : (uint32_t)lim;
        const int64_t q = (int64_t)tid * ntiles + t;
        ro.runs[q] = end > b ? make_uint2(buf[b], buf[end - 1] + 1u) : make_uint2(0u, 0u);
        hist[q] = gbase[tid];   // only this block reads its column of hist
    }
}

// kInlineScan: hist holds raw per-tile counts (no scan kernel ran); each thread
// sums its digit's counts over all tiles and over the tiles before this one.
// kDma (large tiles carrying the endpoint, payload inputs 16-byte aligned):
// the ordinal and endpoint tiles, and the tile's digit offsets, are copied to
// LDS by direct global->LDS loads issued with the key loads, so a block waits
// for memory once (before its ranking) and holds no registers for them; each
// payload tile is then regrouped in place.
// kRows (the last pass of an edge sort, one direction, after the scan): the
// rows are delimited by row_heads instead of writing the keys.
template <class KeySrc, bool kIotaVals, bool kOther, bool kWriteKeys, bool kDual,
          bool kInlineScan, int IT, bool kDma = false, bool kRows = false>
__global__ __launch_bounds__(kBlock) void rs_downsweep(PassDir<KeySrc> a0, PassDir<KeySrc> a1,
                                                       int64_t count, int shift, int bits,
                                                       int64_t ntiles) {
    static_assert(!kDma || (kOther && IT % 4 == 0 && !kInlineScan),
                  "the copied tiles are whole 16-byte rows; the offsets come from the scan");
    static_assert(!kRows || (!kWriteKeys && !kDual && !kInlineScan),
                  "row heads replace the key output of a one-direction pass after the scan");
    static_assert(kBins == kWavesPerBlock * kWave, "one digit offset per thread");
    constexpr int kTile = kBlock * IT;
    // kDma: [0, kTile) the ordinal tile, then the regroup buffer of the keys;
    // [kTile, 2 kTile) the endpoint tile.  Otherwise one regroup buffer.
    uint32_t *pay;
    if constexpr (kDma) {
        __shared__ __attribute__((aligned(16))) uint32_t s_pay[2 * kTile];
        pay = s_pay;
    } else {
        __shared__ uint32_t s_buf[kTile];              // one payload at a time, in tile-sorted order
        pay = s_buf;
    }
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

    // Each wave clears and then ranks with its own row of counters, so no block
    // barrier is needed before the ranking (a wave's LDS accesses stay in
    // order).
#pragma unroll
    for (int m = 0; m < kBins / kWave; ++m) s_cnt[wv][lane + m * kWave] = 0u;
    uint32_t k[IT];
#pragma unroll
    for (int r = 0; r < IT; ++r) {
        const int li = li0 + r * kWave;
        k[r] = li < lim ? tk(li) : 0u;
    }
    // The ordinal and endpoint payloads.  Small tiles (few keys per thread, few
    // registers) load them with the keys, so a block waits for memory once;
    // large tiles copy them to LDS with the keys (kDma), or else load each
    // just before writing it out (see below).
    constexpr bool kEarly = IT <= kItemsSmall;
    uint32_t v[IT], o[IT];
    auto load_payloads = [&]() {
        const uint32_t *vin = kIotaVals ? nullptr : pl.vals_in + tbase;
        const uint32_t *oin = kOther ? pl.other_in + tbase : nullptr;
#pragma unroll
        for (int r = 0; r < IT; ++r) {
            const int li = li0 + r * kWave;
            if constexpr (kIotaVals) v[r] = (uint32_t)tbase + (uint32_t)li;
            else v[r] = li < lim ? vin[li] : 0u;
            if constexpr (kOther) o[r] = li < lim ? oin[li] : 0u;
        }
    };
    if constexpr (kEarly) load_payloads();
    // kDma: each wave copies its own quarter of a payload tile, which is exactly
    // the slots its threads read back (tile-local indices wv * 1024 + [0, 1024)):
    // rows of 64 lanes x 16 bytes for a whole tile, 64 x 4 bytes (indices past
    // the list read the tile's first word, never used) for the last one.
    auto dma = [&](const uint32_t *src, uint32_t *dst) {
        if constexpr (kDma) {
            typedef __attribute__((address_space(3))) void *lds_ptr;
            const int w0 = wv * (kWave * IT);
            if (lim == kTile) {
#pragma unroll
                for (int i = 0; i < IT / 4; ++i) {
                    const int w = w0 + i * (kWave * 4);
                    __builtin_amdgcn_global_load_lds(src + tbase + w + lane * 4, (lds_ptr)(dst + w),
                                                     16, 0, 0);
                }
            } else {
#pragma unroll
                for (int i = 0; i < IT; ++i) {
                    const int w = w0 + i * kWave;
                    const int li = w + lane;
                    __builtin_amdgcn_global_load_lds(src + tbase + (li < lim ? li : 0),
                                                     (lds_ptr)(dst + w), 4, 0, 0);
                }
            }
        }
    };
    if constexpr (kDma) {
        if constexpr (!kIotaVals) dma(pl.vals_in, pay);
        dma(pl.other_in, pay + kTile);
    }
    // kDma (the scan kernel ran): this tile's exclusive count of every digit
    // within its segment (one word per lane, wave w taking digits 64w ...) and
    // the segment totals (16-byte rows, wave w taking those of the same 64
    // digits), copied to LDS with the payloads; each thread later reads only
    // its own digit's, copied by its own wave.
    __shared__ uint32_t s_hv[kDma ? kBins : 1];
    __shared__ __attribute__((aligned(16))) uint32_t s_sv[kDma ? kBins * kScanSegs : 1];
    // (Every pointer is an argument, as in dma: built with the pass record's
    // pointers taken inside the lambda, the host pass dropped this kernel's
    // launch stub and the library failed to load.)
    auto dma_offsets = [&](const uint32_t *hist, const uint32_t *seg, uint32_t *hv, uint32_t *sv) {
        if constexpr (kDma) {
            typedef __attribute__((address_space(3))) void *lds_ptr;
            const int d = wv * kWave + lane;
            __builtin_amdgcn_global_load_lds(hist + (int64_t)d * ntiles + t,
                                             (lds_ptr)(hv + wv * kWave), 4, 0, 0);
            // 16-byte rows of 64 lanes: kSegRowsPerWave per wave
#pragma unroll
            for (int i = 0; i < kSegRowsPerWave; ++i) {
                const int w = (wv * kSegRowsPerWave + i) * (kWave * 4);
                __builtin_amdgcn_global_load_lds(seg + w + lane * 4, (lds_ptr)(sv + w), 16, 0,
                                                 0);
            }
        }
    };
    if constexpr (kDma) dma_offsets(a.hist, a.seg, s_hv, s_sv);
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
        // The scan left the exclusive count within this tile's segment; add the
        // totals of the segments before it (digits beyond the pass have none).
        // kDma: both are in LDS already.
        const int segs = scan_segs(ntiles);
        const int64_t sg = t / scan_seg_len(ntiles);
        // kDma: this thread's digit offsets were copied by its own wave; wait for
        // that wave's copies (the compiler has in practice waited already).
        if constexpr (kDma) __builtin_amdgcn_s_waitcnt(0);
        if constexpr (kDma) before_tile = s_hv[tid];
        else before_tile = a.hist[(int64_t)tid * ntiles + t];
        dsum = 0u;
        if (tid < (1 << bits)) {
            uint32_t c[kScanSegs];
#pragma unroll
            for (int j = 0; j < kScanSegs; ++j) {
                if constexpr (kDma) c[j] = j < segs ? s_sv[tid * kScanSegs + j] : 0u;
                else c[j] = j < segs ? a.seg[tid * kScanSegs + j] : 0u;
            }
#pragma unroll
            for (int j = 0; j < kScanSegs; ++j) {
                dsum += c[j];
                before_tile += j < sg ? c[j] : 0u;
            }
        }
        if (t == 0 && a.dtot) a.dtot[tid] = dsum;
    }
    if (t == 0 && a.flag) {   // the same for the whole block
        uint32_t bad = 0u;
        for (int64_t i = tid; i < a.nbad; i += kBlock) bad |= a.bad[i];
        bad = (uint32_t)__syncthreads_or((int)bad);
        if (tid == 0) *a.flag = bad ? 1u : 0u;
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
    // Regroup each payload through LDS, then write it out in digit runs.
    auto emit_to = [&](const uint32_t(&src)[IT], uint32_t *buf, uint32_t *__restrict__ out) {
#pragma unroll
        for (int r = 0; r < IT; ++r)
            if (li0 + r * kWave < lim) buf[pos[r]] = src[r];
        __syncthreads();
#pragma unroll
        for (int j = 0; j < IT; ++j)
            if ((int64_t)gp[j] < count) out[gp[j]] = buf[tid + j * kBlock];
        __syncthreads();
    };
    auto emit = [&](const uint32_t(&src)[IT], uint32_t *__restrict__ out) {
        emit_to(src, pay, out);
    };
    if constexpr (kDma) {
        // The copies were issued before the ranking; wait for this wave's (no
        // store is outstanding yet), then regroup each tile in place: every
        // thread reads its own slots, and writes them by rank after a barrier.
        __builtin_amdgcn_s_waitcnt(0);
        auto emit_lds = [&](uint32_t *buf, uint32_t *__restrict__ out) {
            uint32_t x[IT];
#pragma unroll
            for (int r = 0; r < IT; ++r) x[r] = buf[li0 + r * kWave];
            __syncthreads();
            emit_to(x, buf, out);
        };
        if constexpr (kIotaVals) {
#pragma unroll
            for (int r = 0; r < IT; ++r) v[r] = (uint32_t)tbase + (uint32_t)(li0 + r * kWave);
            emit_to(v, pay, pl.vals_out);
        } else {
            emit_lds(pay, pl.vals_out);
        }
        emit_lds(pay + kTile, pl.other_out);
        if (kWriteKeys) emit_to(k, pay, pl.keys_out);
        if constexpr (kRows)
            row_heads(k, pos, gp, li0, lim, pay, shift, mask, s_tstart, s_gbase, 1 << bits,
                      a.rows, a.hist, ntiles, t);
        return;
    }
    if (kWriteKeys) emit(k, pl.keys_out);
    if constexpr (kEarly) {
        emit(v, pl.vals_out);
        if constexpr (kOther) emit(o, pl.other_out);
    } else {
        // One payload at a time keeps few registers live across the ranking
        // (more resident blocks per CU for the large tiles).
        {
            const uint32_t *vin = kIotaVals ? nullptr : pl.vals_in + tbase;
#pragma unroll
            for (int r = 0; r < IT; ++r) {
                const int li = li0 + r * kWave;
                if constexpr (kIotaVals) v[r] = (uint32_t)tbase + (uint32_t)li;
                else v[r] = li < lim ? vin[li] : 0u;
            }
            emit(v, pl.vals_out);
        }
        if constexpr (kOther) {
            const uint32_t *oin = pl.other_in + tbase;
#pragma unroll
            for (int r = 0; r < IT; ++r) {
                const int li = li0 + r * kWave;
                o[r] = li < lim ? oin[li] : 0u;
            }
            emit(o, pl.other_out);
        }
    }
    if constexpr (kRows)
        row_heads(k, pos, gp, li0, lim, pay, shift, mask, s_tstart, s_gbase, 1 << bits, a.rows,
                  a.hist, ntiles, t);
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

// Rows delimited by the last sort pass (row_heads), then completed here:
//   rows_init   -- before that pass: every row pointer holds the marker
//                  0xffffffff, rowptr[n] = e;
//   rows_chunk_max, rows_fixup -- the first slot of each nonempty run starts
//                  its key when the edge before it (the last of the nearest
//                  earlier nonempty run, in digit-major order) has a smaller
//                  key;
//   rows_chunk_min, rows_apply -- a key that occurs nowhere starts where the
//                  next key that occurs does: every marker takes the smallest
//                  row pointer after it (the row pointers of occurring keys
//                  increase with the key, and rowptr[n] = e ends the list).
// Each row pointer is written by exactly one of them; none uses atomics.
constexpr int kRowsPer = 16;                        // entries per thread
constexpr int kRowsChunk = kBlock * kRowsPer;       // entries per block
constexpr uint32_t kNoRow = 0xffffffffu;

// op (OpMax or OpMin) over the block.  Contains barriers.
template <class Op>
__device__ uint32_t block_reduce(uint32_t x, Op op) {
    __shared__ uint32_t s_red[kWavesPerBlock];
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) x = op(x, __shfl_xor(x, off));
    if (lane == 0) s_red[wv] = x;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) x = op(x, s_red[w]);
    __syncthreads();
    return x;
}

__global__ __launch_bounds__(kBlock) void rows_init_kernel(int32_t *__restrict__ rowptr,
                                                           int64_t n, int64_t e) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i <= n; i += stride)
        rowptr[i] = i == n ? (int32_t)e : (int32_t)kNoRow;
}

// cmax[c]: the largest run end (last key + 1) of record chunk c, 0 if all its
// runs are empty.
__global__ __launch_bounds__(kBlock) void rows_chunk_max_kernel(const uint2 *__restrict__ runs,
                                                                int64_t count,
                                                                uint32_t *__restrict__ cmax) {
    const int64_t c0 = (int64_t)blockIdx.x * kRowsChunk;
    uint32_t m = 0u;
#pragma unroll
    for (int j = 0; j < kRowsPer; ++j) {
        const int64_t q = c0 + threadIdx.x + (int64_t)j * kBlock;
        const uint32_t v = q < count ? runs[q].y : 0u;
        m = v > m ? v : m;
    }
    m = block_reduce(m, OpMax{});
    if (threadIdx.x == 0) cmax[blockIdx.x] = m;
}

// One block per kRowsChunk run records (count = digits * ntiles).
__global__ __launch_bounds__(kBlock) void rows_fixup_kernel(const uint2 *__restrict__ runs,
                                                            const uint32_t *__restrict__ pstart,
                                                            const uint32_t *__restrict__ cmax,
                                                            int64_t count,
                                                            int32_t *__restrict__ rowptr) {
    const int64_t c0 = (int64_t)blockIdx.x * kRowsChunk;
    const int tid = threadIdx.x;
    uint32_t l[kRowsPer], f[kRowsPer], ps[kRowsPer];
#pragma unroll
    for (int j = 0; j < kRowsPer; ++j) {
        const int64_t q = c0 + tid + (int64_t)j * kBlock;
        const bool in = q < count;
        const uint2 r = in ? runs[q] : make_uint2(0u, 0u);
        f[j] = r.x;
        l[j] = r.y;
        ps[j] = in ? pstart[q] : 0u;
    }
    // The last key (+ 1) before this chunk: the nearest earlier chunk maximum
    // that is not 0 (they grow along the records), found kRowsChunk chunks at
    // a time.  The trip count is the same for the whole block.
    uint32_t carry = 0u;
    for (int64_t wend = blockIdx.x; carry == 0u && wend > 0;) {
        const int64_t wbeg = wend > kRowsChunk ? wend - kRowsChunk : 0;
        uint32_t m = 0u;
#pragma unroll
        for (int j = 0; j < kRowsPer; ++j) {
            const int64_t c = wbeg + tid + (int64_t)j * kBlock;
            const uint32_t v = c < wend ? cmax[c] : 0u;
            m = v > m ? v : m;
        }
        carry = block_reduce(m, OpMax{});
        wend = wbeg;
    }
    uint32_t ex[kRowsPer];
    rounds_exclusive<true>(l, ex, 0u, OpMax{});
#pragma unroll
    for (int j = 0; j < kRowsPer; ++j) {
        // a nonempty run starts its key when the edge before it has a smaller one
        const uint32_t before = ex[j] > carry ? ex[j] : carry;   // last key + 1; 0: none
        if (l[j] > 0u && before <= f[j]) rowptr[f[j]] = (int32_t)ps[j];
    }
}

// cmin[c]: the smallest row pointer of chunk c (kNoRow if it holds only markers).
__global__ __launch_bounds__(kBlock) void rows_chunk_min_kernel(const int32_t *__restrict__ rowptr,
                                                                int64_t n1,
                                                                uint32_t *__restrict__ cmin) {
    const int64_t c0 = (int64_t)blockIdx.x * kRowsChunk;
    uint32_t m = kNoRow;
#pragma unroll
    for (int j = 0; j < kRowsPer; ++j) {
        const int64_t i = c0 + threadIdx.x + (int64_t)j * kBlock;
        const uint32_t v = i < n1 ? (uint32_t)rowptr[i] : kNoRow;
        m = v < m ? v : m;
    }
    m = block_reduce(m, OpMin{});
    if (threadIdx.x == 0) cmin[blockIdx.x] = m;
}

// Every marker of chunk blockIdx.x takes the smallest row pointer after it.
__global__ __launch_bounds__(kBlock) void rows_apply_kernel(int32_t *__restrict__ rowptr,
                                                            int64_t n1,
                                                            const uint32_t *__restrict__ cmin,
                                                            int64_t nchunks) {
    const int64_t c0 = (int64_t)blockIdx.x * kRowsChunk;
    const int tid = threadIdx.x;
    uint32_t v[kRowsPer];
#pragma unroll
    for (int j = 0; j < kRowsPer; ++j) {
        const int64_t i = c0 + tid + (int64_t)j * kBlock;
        v[j] = i < n1 ? (uint32_t)rowptr[i] : kNoRow;
    }
    // The smallest row pointer after this chunk: the first chunk minimum that
    // is not a marker (they grow with the chunk).  Uniform trip count.
    uint32_t carry = kNoRow;
    for (int64_t w = (int64_t)blockIdx.x + 1; carry == kNoRow && w < nchunks; w += kRowsChunk) {
        uint32_t m = kNoRow;
#pragma unroll
        for (int j = 0; j < kRowsPer; ++j) {
            const int64_t q = w + tid + (int64_t)j * kBlock;
            const uint32_t x = q < nchunks ? cmin[q] : kNoRow;
            m = x < m ? x : m;
        }
        carry = block_reduce(m, OpMin{});
    }
    uint32_t ex[kRowsPer];
    rounds_exclusive<false>(v, ex, kNoRow, OpMin{});
#pragma unroll
    for (int j = 0; j < kRowsPer; ++j) {
        const int64_t i = c0 + tid + (int64_t)j * kBlock;
        const uint32_t after = ex[j] < carry ? ex[j] : carry;
        if (i < n1 && v[j] == kNoRow) rowptr[i] = (int32_t)after;
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

// Large tiles count digits of at most kLaneDigitBits bits with lane-private
// counters; small tiles (4 keys per lane) and wider digits match with ballots.
template <int IT>
constexpr bool lane_counts(int bits) {
    return IT == kItems && bits <= kLaneDigitBits;
}

template <bool kLane, int IT>
void intake_launch(const void *src, const void *dst, mp_dtype idx_dtype, int64_t e, int64_t n,
                   mp_graph *g, int first_bits, uint32_t *hist_f, uint32_t *hist_t, int64_t nt,
                   uint32_t *bad_tiles, hipStream_t s) {
    if (idx_dtype == MP_I64)
        intake_count_kernel<int64_t, kLane, IT><<<(unsigned)nt, kBlock, 0, s>>>(
            static_cast<const int64_t *>(src), static_cast<const int64_t *>(dst), e, n, g->src,
            g->dst, g->info + kInfoFlag, bad_tiles, first_bits, hist_f, hist_t, nt);
    else
        intake_count_kernel<int32_t, kLane, IT><<<(unsigned)nt, kBlock, 0, s>>>(
            static_cast<const int32_t *>(src), static_cast<const int32_t *>(dst), e, n, g->src,
            g->dst, g->info + kInfoFlag, bad_tiles, first_bits, hist_f, hist_t, nt);
}

// Counting intake over tiles of 256 * IT edges.
// bad_tiles: per-tile range words instead of the flag (see intake_count_kernel).
template <int IT>
void intake_count(const void *src, const void *dst, mp_dtype idx_dtype, int64_t e, int64_t n,
                  mp_graph *g, int first_bits, uint32_t *hist_f, uint32_t *hist_t,
                  uint32_t *bad_tiles, hipStream_t s) {
    const int64_t nt = tiles_for(e, IT);
    if (lane_counts<IT>(first_bits))
        intake_launch<true, IT>(src, dst, idx_dtype, e, n, g, first_bits, hist_f, hist_t, nt,
                                bad_tiles, s);
    else
        intake_launch<false, IT>(src, dst, idx_dtype, e, n, g, first_bits, hist_f, hist_t, nt,
                                 bad_tiles, s);
}


// Edge lists up to this size run both directions in every launch (their
// workspace then holds a second set of sort buffers).
constexpr int64_t kDualMaxEdges = (int64_t)1 << 22;
// Passes over at most this many tiles sum the per-tile counts inside the
// downsweep instead of launching the scan.
constexpr int64_t kInlineScanMaxTiles = 64;

bool dual_mode(int64_t e) { return e <= kDualMaxEdges; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// The count scan of a pass over ntiles tiles (the digits' rows of both
// directions with kDual), with as many counts per thread per step as the
// segment length calls for.
template <bool kDual, class KeySrc>
void scan_launch(const PassDir<KeySrc> &d0, const PassDir<KeySrc> &d1, int64_t ntiles,
                 int digits, hipStream_t s) {
    const unsigned grid = (unsigned)((kDual ? 2 : 1) * digits * scan_segs(ntiles));
    const int64_t len = scan_seg_len(ntiles);
    if (len <= kBlock)
        rs_scan<kDual, 1><<<grid, kBlock, 0, s>>>(d0.hist, d0.seg, d1.hist, d1.seg, ntiles, digits);
    else if (len <= 4 * kBlock)
        rs_scan<kDual, 4><<<grid, kBlock, 0, s>>>(d0.hist, d0.seg, d1.hist, d1.seg, ntiles, digits);
    else
        rs_scan<kDual, 16><<<grid, kBlock, 0, s>>>(d0.hist, d0.seg, d1.hist, d1.seg, ntiles,
                                                   digits);
}

// One radix pass for one direction (d1 unused) or both (kDual), with tiles of
// 256 * IT keys.
// counted: the per-tile digit counts are already in hist (the counting intake).
// kRows: the last pass of a one-direction edge sort over more than
// kInlineScanMaxTiles tiles, delimiting the rows (d0.rows) instead of writing
// the keys.
template <class KeySrc, bool kIota, bool kOther, bool kWriteKeys, bool kDual, int IT,
          bool kRows = false>
mp_status radix_pass(const PassDir<KeySrc> &d0, const PassDir<KeySrc> &d1, int64_t count,
                     int shift, int bits, hipStream_t s, bool counted = false) {
    const int64_t ntiles = tiles_for(count, IT);
    if (kRows && ntiles <= kInlineScanMaxTiles)
        return fail(MP_ERR_INTERNAL, "row heads need the scan kernel");
    const unsigned grid = (unsigned)((kDual ? 2 : 1) * ntiles);
    if (!counted) {
        bool vec = false;   // keys read 16 bytes at a time (lane counts, aligned keys)
        if constexpr (std::is_same<KeySrc, KeysFromArray>::value && IT % 4 == 0)
            vec = lane_counts<IT>(bits) && aligned16(d0.keys.k) && aligned16(d1.keys.k);
        if (vec) {
            if constexpr (std::is_same<KeySrc, KeysFromArray>::value && IT % 4 == 0)
                rs_upsweep<KeySrc, kDual, true, IT, true><<<grid, kBlock, 0, s>>>(
                    d0, d1, count, shift, bits, ntiles);
        } else if (lane_counts<IT>(bits))
            rs_upsweep<KeySrc, kDual, true, IT><<<grid, kBlock, 0, s>>>(d0, d1, count, shift, bits,
                                                                        ntiles);
        else
            rs_upsweep<KeySrc, kDual, false, IT><<<grid, kBlock, 0, s>>>(d0, d1, count, shift,
                                                                         bits, ntiles);
    }
    if constexpr (kRows) {
        const int digits = 1 << bits;
        scan_launch<false>(d0, d0, ntiles, digits, s);
        const bool dma = IT == kItems && (kIota || aligned16(d0.pl.vals_in)) &&
                         aligned16(d0.pl.other_in);
        if (dma)
            rs_downsweep<KeySrc, kIota, true, false, false, false, IT, true, true>
                <<<grid, kBlock, 0, s>>>(d0, d1, count, shift, bits, ntiles);
        else
            rs_downsweep<KeySrc, kIota, true, false, false, false, IT, false, true>
                <<<grid, kBlock, 0, s>>>(d0, d1, count, shift, bits, ntiles);
    } else if (ntiles <= kInlineScanMaxTiles) {
        rs_downsweep<KeySrc, kIota, kOther, kWriteKeys, kDual, true, IT>
            <<<grid, kBlock, 0, s>>>(d0, d1, count, shift, bits, ntiles);
    } else {
        const int digits = 1 << bits;
        scan_launch<kDual>(d0, d1, ntiles, digits, s);
        // Large single-direction edge passes copy their payload tiles to LDS
        // directly when the inputs allow 16-byte rows.
        const bool dma = kOther && !kDual && IT == kItems &&
                         (kIota || aligned16(d0.pl.vals_in)) && aligned16(d0.pl.other_in);
        if (dma)
            rs_downsweep<KeySrc, kIota, kOther, kWriteKeys, kDual, false, IT, kOther && !kDual>
                <<<grid, kBlock, 0, s>>>(d0, d1, count, shift, bits, ntiles);
        else
            rs_downsweep<KeySrc, kIota, kOther, kWriteKeys, kDual, false, IT>
                <<<grid, kBlock, 0, s>>>(d0, d1, count, shift, bits, ntiles);
    }
    MP_HIP_CHECK(hipGetLastError(), "radix pass launch");
    return MP_OK;
}

// Whether the last pass of a one-direction sort delimits the rows itself
// (row_heads and the rows_* kernels) rather than writing the sorted keys for
// a binary search per row.  It saves a key write and a search read per edge
// and costs about 16 bytes per row pointer (markers, chunk minima, fill), so it
// is taken for at least two edges per row; it needs the scan kernel (more than
// kInlineScanMaxTiles tiles) and room for the run records and the chunk
// maxima and minima in the pass's free key buffer ([e] words).
bool rows_by_sort(int64_t e, int64_t n, int last_bits) {
    const int64_t ntiles = tiles_for(e, kItems);
    const int64_t runs = ((int64_t)1 << last_bits) * ntiles;
    const int64_t rchunks = (runs + kRowsChunk - 1) / kRowsChunk;
    const int64_t nchunks = (n + 1 + kRowsChunk - 1) / kRowsChunk;
    return ntiles > kInlineScanMaxTiles && 2 * (n + 1) <= e && 2 * runs + rchunks + nchunks <= e;
}

// Sort buffers of one direction.
struct SortBufs {
    uint32_t *k0, *k1, *v0, *o0, *hist, *seg;
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
// rowptr (one direction only): where the rows may be delimited by the last
// pass (rows_by_sort); *rows_done tells whether they were, else the caller
// takes them from the sorted keys.
template <bool kDual>
mp_status sort_edges(const EdgeDir *dirs, int64_t e, int64_t n, const uint32_t **sorted,
                     hipStream_t s, bool first_counted = false, int32_t *rowptr = nullptr,
                     bool *rows_done = nullptr) {
    constexpr int kDirs = kDual ? 2 : 1;
    const int bits = key_bits(n);
    const int passes = (bits + kDigitBits - 1) / kDigitBits;
    const int per_bits = (bits + passes - 1) / passes;
    const int last_bits = bits - (passes - 1) * per_bits;
    const bool by_sort = !kDual && rowptr && rows_by_sort(e, n, last_bits);
    if (rows_done) *rows_done = by_sort;
    if (by_sort) {
        rows_init_kernel<<<grid_for(n + 1), kBlock, 0, s>>>(rowptr, n, e);
        MP_HIP_CHECK(hipGetLastError(), "row pointer marker launch");
    }
    PassDir<KeysFromArray> pd[2];
    const uint32_t *kin[2];
    for (int i = 0; i < kDirs; ++i) {
        kin[i] = reinterpret_cast<const uint32_t *>(dirs[i].key);
        pd[i].pl.vals_in = nullptr;
        pd[i].pl.other_in = reinterpret_cast<const uint32_t *>(dirs[i].other);
        pd[i].hist = dirs[i].b.hist;
        pd[i].seg = dirs[i].b.seg;
        pd[i].dtot = nullptr;
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
        mp_status st;
        if (by_sort && pass == passes - 1) {
            // The free key buffer holds the run records, then the chunk maxima
            // of their ends and the chunk minima of the row pointers.
            const int64_t runs = ((int64_t)1 << pb) * tiles_for(e, IT);
            uint32_t *rec = pd[0].pl.keys_out;
            uint2 *run_recs = reinterpret_cast<uint2 *>(rec);
            pd[0].rows = RowsOut{rowptr, run_recs};
            pd[1] = pd[0];
            st = pass == 0
                ? radix_pass<KeysFromArray, true, true, false, false, IT, true>(
                      pd[0], pd[1], e, shift, pb, s, first_counted)
                : radix_pass<KeysFromArray, false, true, false, false, IT, true>(
                      pd[0], pd[1], e, shift, pb, s);
            if (st != MP_OK) return st;
            const int64_t rchunks = (runs + kRowsChunk - 1) / kRowsChunk;
            const int64_t nchunks = (n + 1 + kRowsChunk - 1) / kRowsChunk;
            uint32_t *cmax = rec + 2 * runs;
            uint32_t *cmin = cmax + rchunks;
            rows_chunk_max_kernel<<<(unsigned)rchunks, kBlock, 0, s>>>(run_recs, runs, cmax);
            rows_fixup_kernel<<<(unsigned)rchunks, kBlock, 0, s>>>(run_recs, pd[0].hist, cmax,
                                                                    runs, rowptr);
            rows_chunk_min_kernel<<<(unsigned)nchunks, kBlock, 0, s>>>(rowptr, n + 1, cmin);
            rows_apply_kernel<<<(unsigned)nchunks, kBlock, 0, s>>>(rowptr, n + 1, cmin, nchunks);
            MP_HIP_CHECK(hipGetLastError(), "row pointer launches");
            sorted[0] = nullptr;
            return MP_OK;
        }
        st = pass == 0
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
// bad / nbad (small lists): the intake's per-tile range words, reduced into the
// graph's index flag by the plan's downsweep.
template <int IT>
mp_status plans(int64_t n, mp_graph *g, const SortBufs &b0, const SortBufs &b1,
                uint32_t *totals0, uint32_t *totals1, hipStream_t s,
                const uint32_t *bad = nullptr, int64_t nbad = 0) {
    PassDir<KeysFromDegree> p0, p1;
    p0.keys = KeysFromDegree{g->rowptr};
    p1.keys = KeysFromDegree{g->rowptr_t};
    p0.pl = Payload{nullptr, nullptr, nullptr, reinterpret_cast<uint32_t *>(g->row_plan), nullptr};
    p1.pl = Payload{nullptr, nullptr, nullptr, reinterpret_cast<uint32_t *>(g->row_plan_t),
                    nullptr};
    p0.hist = b0.hist;
    p1.hist = b1.hist;
    p0.seg = b0.seg;
    p1.seg = b1.seg;
    p0.dtot = totals0;
    p1.dtot = totals1;
    if (bad) {
        p0.bad = bad;
        p0.nbad = nbad;
        p0.flag = g->info + kInfoFlag;
    }
    return radix_pass<KeysFromDegree, true, false, false, true, IT>(p0, p1, n, 0, kPlanBits, s);
}

// The degree plan of one direction (the plan pass on its own launches).
mp_status plan_one(int64_t n, const int32_t *rowptr, int32_t *row_plan, const SortBufs &b,
                   uint32_t *totals, hipStream_t s) {
    PassDir<KeysFromDegree> p;
    p.keys = KeysFromDegree{rowptr};
    p.pl = Payload{nullptr, nullptr, nullptr, reinterpret_cast<uint32_t *>(row_plan), nullptr};
    p.hist = b.hist;
    p.seg = b.seg;
    p.dtot = totals;
    return radix_pass<KeysFromDegree, true, false, false, false, kItems>(p, p, n, 0, kPlanBits, s);
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

LowerLayout lower_layout(int64_t n, int64_t e, bool split_dirs) {
    LowerLayout L;
    size_t off = 0;
    const size_t ebytes = align_up((size_t)(e > 0 ? e : 1) * sizeof(uint32_t));
    const int64_t most = e > n ? e : n;
    const int it = dual_mode(e) ? kItemsSmall : kItems;
    const size_t hbytes = align_up((size_t)kBins * tiles_for(most, it) * sizeof(uint32_t));
    for (int i = 0; i < 2; ++i) {
        if (i == 1 && !dual_mode(e) && !split_dirs) {   // one direction at a time: one set
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
        L.seg[i] = off; off += align_up((size_t)kBins * kScanSegs * sizeof(uint32_t));
    }
    // Per-tile range words of a small list's intake (one word per 1024-edge tile).
    L.bad = off; off += dual_mode(e) ? align_up((size_t)tiles_for(e, kItemsSmall) * 4) : 0;
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
                    mp_graph *g, void *ws, hipStream_t s, bool async, int *bad_index,
                    hipStream_t side, hipEvent_t side_done) {
    const bool split = side != nullptr;
    if (split && (!async || !side_done))
        return fail(MP_ERR_INTERNAL, "a side-stream lowering is asynchronous and records an event");
    const LowerLayout L = lower_layout(n, e, split);
    char *base = static_cast<char *>(ws);
    auto at = [&](size_t off) { return reinterpret_cast<uint32_t *>(base + off); };
    SortBufs b[2];
    for (int i = 0; i < 2; ++i)
        b[i] = SortBufs{at(L.k0[i]), at(L.k1[i]), at(L.v0[i]), at(L.o0[i]), at(L.hist[i]),
                        at(L.seg[i])};
    uint32_t *info = g->info;

    // Small lists (both directions per launch): the intake writes a range word
    // per tile and the plan pass, the build's last launch, reduces them into
    // the index flag, so the record needs no clearing launch.  Otherwise a fill
    // kernel clears it (not a memset: the sequence stays valid under graph
    // capture).
    const bool small = dual_mode(e) && !split;
    uint32_t *bad_tiles = small ? at(L.bad) : nullptr;
    if (!small) zero_words_kernel<<<1, kBlock, 0, s>>>(info, MP_GRAPH_INFO_WORDS);
    // The intake also counts the first pass's digits of both keys, in the tiles
    // of that pass (1024 keys when both directions share the launches).
    const bool counted = e > 0;
    if (counted) {
        const int fb = first_pass_bits(n);
        if (small)
            intake_count<kItemsSmall>(src, dst, idx_dtype, e, n, g, fb, b[0].hist, b[1].hist,
                                      bad_tiles, s);
        else
            intake_count<kItems>(src, dst, idx_dtype, e, n, g, fb, b[0].hist, b[1].hist,
                                 nullptr, s);
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
    if (split) {
        // Each direction on its own stream, with its own sort buffers and large
        // tiles (the intake counted the first passes in them); the transpose
        // waits only for the intake.
        hipEvent_t fork = nullptr;
        MP_HIP_CHECK(hipEventCreateWithFlags(&fork, hipEventDisableTiming), "fork event");
        hipError_t he = hipEventRecord(fork, s);
        if (he == hipSuccess) he = hipStreamWaitEvent(side, fork, 0);
        (void)hipEventDestroy(fork);   // released once the wait no longer needs it
        MP_HIP_CHECK(he, "fork of the transpose lowering");
        for (int i = 0; i < 2 && st == MP_OK; ++i) {
            hipStream_t q = i == 0 ? s : side;
            int32_t *rowptr = i == 0 ? g->rowptr : g->rowptr_t;
            bool rows_done = false;
            if (e > 0)
                st = sort_edges<false>(&dirs[i], e, n, &sorted[i], q, counted, rowptr, &rows_done);
            const RowsDir r{sorted[i], rowptr};
            if (st == MP_OK && !rows_done) st = row_pointers<false>(r, r, e, n, q);
            if (st == MP_OK)
                st = plan_one(n, i == 0 ? g->rowptr : g->rowptr_t,
                              i == 0 ? g->row_plan : g->row_plan_t, b[i],
                              info + (i == 0 ? kInfoPlanF : kInfoPlanT), q);
        }
        if (st != MP_OK) return st;
        MP_HIP_CHECK(hipEventRecord(side_done, side), "transpose lowering event");
        *bad_index = 0;
        for (int c = 0; c < MP_NUM_CLASSES; ++c) g->class_count[c] = g->class_count_t[c] = 0;
        return MP_OK;
    }
    if (dual_mode(e)) {
        if (e > 0) st = sort_edges<true>(dirs, e, n, sorted, s, counted);
        if (st == MP_OK)
            st = row_pointers<true>(RowsDir{sorted[0], g->rowptr},
                                    RowsDir{sorted[1], g->rowptr_t}, e, n, s);
    } else {
        for (int i = 0; i < 2 && st == MP_OK; ++i) {
            int32_t *rowptr = i == 0 ? g->rowptr : g->rowptr_t;
            bool rows_done = false;
            st = sort_edges<false>(&dirs[i], e, n, &sorted[i], s, counted, rowptr, &rows_done);
            const RowsDir r{sorted[i], rowptr};
            if (st == MP_OK && !rows_done) st = row_pointers<false>(r, r, e, n, s);
        }
    }
    // The plans; a small list's plan downsweep also settles the index flag.
    const int64_t nbad = counted ? tiles_for(e, kItemsSmall) : 0;
    if (st == MP_OK)
        st = dual_mode(e)
            ? plans<kItemsSmall>(n, g, b[0], b[1], info + kInfoPlanF, info + kInfoPlanT, s,
                                 bad_tiles, nbad)
            : plans<kItems>(n, g, b[0], b[1], info + kInfoPlanF, info + kInfoPlanT, s);
    if (st != MP_OK) return st;

    *bad_index = 0;
    if (async) {
        for (int c = 0; c < MP_NUM_CLASSES; ++c) g->class_count[c] = g->class_count_t[c] = 0;
        return MP_OK;
    }
    return lower_read_info(g, s, bad_index);
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch[kMaxDevices] = {};   // device address of `scratch` on each GPU
}  // namespace

mp_status static_workspace(void **ptr, size_t *bytes) {
    int dev = -1;
    MP_HIP_CHECK(hipGetDevice(&dev), "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(MP_ERR_DEVICE, "device %d beyond the %d the static workspace serves", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch[dev]) {   // first use on this device, with it current
        void *p = nullptr;
        MP_HIP_CHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)),
                     "address of the static workspace");
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    *bytes = sizeof(scratch);
    return MP_OK;
}

}  // namespace mp
