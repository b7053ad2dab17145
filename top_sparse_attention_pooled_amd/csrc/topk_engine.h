// topk_engine.h -- exact block-wide top-B selection of blocks by score.
//
// Ranking: score descending, ties to the lower block index, -0 == +0.  Each
// candidate is a pair (k, u): k = order-preserving 32-bit key of its finite
// score (never 0; 0 marks "no candidate") and u = ~block (so a larger u is a
// lower block).  The kept set is the B largest pairs (k, u) in lexicographic
// order, which is unique because blocks are distinct.
//
// Phase A selects on k alone: a radix select whose digit window follows the
// live key range -- each round bins the keys inside [lo, hi] by
// (k - lo) >> shift, with shift chosen so the range spans 1024..2048 bins, and
// the bin holding the B-th key becomes the next range.  Offsetting by lo
// spreads the clustered keys of a top-k over the whole histogram (a fixed
// digit would put them into a few bins and serialise the LDS atomics).  It
// stops as soon as the threshold bin is taken whole.  Only if the B-th key
// value is shared by several blocks (ties) does phase B run the same select
// on u among the tied blocks.  At most 3 rounds per phase.
//
// The element source is a functor for_each(f) that calls f(k, u) for every
// element the calling thread owns; register-cached and streamed sources use
// the same code.
#pragma once

#include "qsa_internal.h"
#include "wave_ops.h"

namespace qsa {

constexpr int kBinBits = 11;
constexpr int kBins = 1 << kBinBits;

template <int NT>
struct TopkSmem {
    uint32_t hist[kBins];
    uint32_t red[NT / 64];
    uint32_t red2[NT / 64];
    uint32_t b_lo, b_hi, b_above, b_cnt;
};

// The kept set: valid (k != 0) and (k > T, or k == T and (!tie or u >= U)).
struct Thresh {
    uint32_t T;
    uint32_t U;
    bool tie;
    __device__ __forceinline__ bool keep(uint32_t k, uint32_t u) const {
        return k != 0 && (k > T || (k == T && (!tie || u >= U)));
    }
};

// Cross-wave combination of one value per wavefront, red[0 .. NW) (read
// after a barrier): lane l loads red[l] once and the wavefront combines the
// values with DPP.  (A loop over the array in every thread pays one LDS
// round trip per step: the loads reuse registers and wait one by one.)
template <int NW>
__device__ __forceinline__ uint32_t waves_sum(const uint32_t *red) {
    const int lane = threadIdx.x & (kWave - 1);
    return wave_sum_u32(lane < NW ? red[lane] : 0u);
}

// before = sum over wavefronts w < wave, total = sum over all (wave uniform).
template <int NW>
__device__ __forceinline__ void waves_prefix(const uint32_t *red, int wave, uint32_t &before,
                                             uint32_t &total) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t incl = wave_incl_scan_u32(lane < NW ? red[lane] : 0u);
    total = lane_value(incl, kWave - 1);
    before = wave > 0 ? lane_value(incl, wave - 1) : 0u;
}

template <int NT>
__device__ __forceinline__ uint32_t block_sum_u32(uint32_t v, TopkSmem<NT> &sm) {
    const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
    v = wave_sum_u32(v);
    if (lane == 0) sm.red[wave] = v;
    __syncthreads();
    const uint32_t t = waves_sum<NT / 64>(sm.red);
    __syncthreads();
    return t;
}

// Block-wide (min, max) of per-thread values.
template <int NT>
__device__ __forceinline__ void block_minmax_u32(uint32_t &mn, uint32_t &mx, TopkSmem<NT> &sm) {
    const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
    mn = wave_min_u32(mn);
    mx = wave_max_u32(mx);
    if (lane == 0) {
        sm.red[wave] = mn;
        sm.red2[wave] = mx;
    }
    __syncthreads();
    constexpr int NW = NT / 64;
    mn = wave_min_u32(lane < NW ? sm.red[lane] : ~0u);
    mx = wave_max_u32(lane < NW ? sm.red2[lane] : 0u);
    __syncthreads();
}

__device__ __forceinline__ int range_shift(uint32_t lo, uint32_t hi) {
    const uint32_t span = hi - lo;
    const int bits = span ? 32 - __builtin_clz(span) : 0;
    return bits > kBinBits ? bits - kBinBits : 0;
}

// Find the bin holding the krem-th largest value: sets b_lo/b_hi (the bin's
// value range), b_above (values in higher bins) and b_cnt.
template <int NT>
__device__ __forceinline__ void pick_bin(TopkSmem<NT> &sm, uint32_t lo, uint32_t hi, int shift,
                                         uint32_t krem) {
    constexpr int PER = kBins / NT;  // consecutive bins per thread
    const int t = threadIdx.x;
    uint32_t local = 0;
    uint32_t h[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        h[q] = sm.hist[t * PER + q];
        local += h[q];
    }
    // suffix sums: values in bins above this thread's bins
    const int lane = t & (kWave - 1), wave = wave_id();
    const uint32_t prefix = wave_incl_scan_u32(local);     // lanes <= this one
    const uint32_t total = lane_value(prefix, kWave - 1);  // whole wave
    if (lane == 0) sm.red[wave] = total;
    __syncthreads();
    uint32_t before, all;
    waves_prefix<NT / 64>(sm.red, wave, before, all);
    uint32_t above = all - before - prefix;  // higher lanes and higher wavefronts
#pragma unroll
    for (int q = PER - 1; q >= 0; --q) {
        if (above < krem && above + h[q] >= krem) {
            const uint32_t blo = lo + ((uint32_t)(t * PER + q) << shift);
            uint32_t bhi = blo + ((1u << shift) - 1u);
            if (bhi > hi || bhi < blo) bhi = hi;
            sm.b_lo = blo;
            sm.b_hi = bhi;
            sm.b_above = above;
            sm.b_cnt = h[q];
        }
        above += h[q];
    }
    __syncthreads();
}

// Radix select of the krem-th largest of the values v = VAL(k, u) over the
// elements with PRED(k, u), starting from their range [lo, hi].  Returns the
// threshold value; n_above gets the count strictly above it; done tells
// whether count(v >= threshold) == krem (no tie left at the threshold).
template <int NT, typename ForEach, typename Pred, typename Val>
__device__ __forceinline__ uint32_t select_u32(const ForEach &for_each, Pred pred, Val val, uint32_t krem, uint32_t lo,
                               uint32_t hi, TopkSmem<NT> &sm, uint32_t &n_above, bool &done) {
    n_above = 0;
    for (int round = 0; round < 4; ++round) {
        const int shift = range_shift(lo, hi);
        for (int j = threadIdx.x; j < kBins; j += NT) sm.hist[j] = 0;
        __syncthreads();
        for_each([&](uint32_t k, uint32_t u) {
            if (!pred(k, u)) return;
            const uint32_t v = val(k, u);
            if (v >= lo && v <= hi) atomicAdd(&sm.hist[(v - lo) >> shift], 1u);
        });
        __syncthreads();
        pick_bin<NT>(sm, lo, hi, shift, krem);
        const uint32_t above = sm.b_above, cnt = sm.b_cnt;
        lo = sm.b_lo;
        hi = sm.b_hi;
        __syncthreads();
        n_above += above;
        krem -= above;
        if (cnt == krem) {
            done = true;
            return lo;
        }
        if (lo == hi) break;  // a single value shared by more than krem elements
    }
    done = false;
    return lo;
}

// The krem-th largest value among the keys k in [lo, hi] (k = 0 never
// counts when lo > 0): the same binning, continued until the bin is a single
// value (at most 3 rounds of 11 bits).  The caller guarantees that [lo, hi]
// holds at least krem keys.
template <int NT, typename ForEach>
__device__ __forceinline__ uint32_t kth_largest_u32(const ForEach &for_each, uint32_t krem,
                                                    uint32_t lo, uint32_t hi, TopkSmem<NT> &sm) {
    while (lo != hi) {
        const int shift = range_shift(lo, hi);
        for (int j = threadIdx.x; j < kBins; j += NT) sm.hist[j] = 0;
        __syncthreads();
        for_each([&](uint32_t k, uint32_t) {
            if (k >= lo && k <= hi) atomicAdd(&sm.hist[(k - lo) >> shift], 1u);
        });
        __syncthreads();
        pick_bin<NT>(sm, lo, hi, shift, krem);
        krem -= sm.b_above;
        lo = sm.b_lo;
        hi = sm.b_hi;
        __syncthreads();
    }
    return lo;
}

// The exact kept set of the top B (or every valid element if there are at
// most B).
template <int NT, typename ForEach>
__device__ __forceinline__ Thresh topk_threshold(const ForEach &for_each, uint32_t B, TopkSmem<NT> &sm) {
    Thresh th{0u, 0u, false};
    uint32_t cnt = 0, mn = ~0u, mx = 0u;
    for_each([&](uint32_t k, uint32_t) {
        if (!k) return;
        ++cnt;
        mn = min(mn, k);
        mx = max(mx, k);
    });
    const uint32_t n_valid = block_sum_u32<NT>(cnt, sm);
    if (n_valid <= B) return th;  // T = 0: every valid element
    block_minmax_u32<NT>(mn, mx, sm);
    uint32_t n_above;
    bool done;
    th.T = select_u32<NT>(
        for_each, [](uint32_t k, uint32_t) { return k != 0; },
        [](uint32_t k, uint32_t) { return k; }, B, mn, mx, sm, n_above, done);
    if (done) return th;
    // ties at score key T: keep the lowest blocks (largest u) among them
    const uint32_t T = th.T;
    uint32_t umn = ~0u, umx = 0u;
    for_each([&](uint32_t k, uint32_t u) {
        if (k != T) return;
        umn = min(umn, u);
        umx = max(umx, u);
    });
    block_minmax_u32<NT>(umn, umx, sm);
    th.U = select_u32<NT>(
        for_each, [T](uint32_t k, uint32_t) { return k == T; },
        [](uint32_t, uint32_t u) { return u; }, B - n_above, umn, umx, sm, n_above, done);
    th.tie = true;
    return th;
}

// Ascending emission of the kept blocks from an LDS bitmap over
// [0, n_words*32): each thread owns a run of words, counts, scans, emits.
// Writes *n_sel = kept blocks * r + tail (first, so its store is not queued
// behind the list), sel_blocks[0..B) (-1 padded) and sel_cells[0..ld_cells)
// (each kept block's r cells, then the tail cells, -1 padded).  Ends without
// a barrier: the caller must not reuse sm or the bitmap afterwards.
template <int NT>
__device__ void emit_from_bitmap(const uint32_t *bm, int n_words, int B, int r, int64_t nc,
                                 int tail, int32_t *sel_blocks, int32_t *sel_cells, int ld_cells,
                                 int32_t *n_sel, TopkSmem<NT> &sm) {
    const int per = (n_words + NT - 1) / NT;
    const int w0 = threadIdx.x * per;
    uint32_t local = 0;
    for (int w = w0; w < w0 + per && w < n_words; ++w) local += __popc(bm[w]);
    const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
    const uint32_t incl = wave_incl_scan_u32(local);
    if (lane == kWave - 1) sm.red[wave] = incl;
    __syncthreads();
    uint32_t before, total;
    waves_prefix<NT / 64>(sm.red, wave, before, total);
    uint32_t pos = before + incl - local;
    const int n_keep = (int)(total < (uint32_t)B ? total : (uint32_t)B);
    if (threadIdx.x == 0) *n_sel = n_keep * r + tail;
    for (int w = w0; w < w0 + per && w < n_words; ++w) {
        uint32_t bits = bm[w];
        while (bits) {
            const int bit = __builtin_ctz(bits);
            bits &= bits - 1;
            const int32_t b = w * 32 + bit;
            if ((int)pos < B) {
                sel_blocks[pos] = b;
                for (int c = 0; c < r; ++c) sel_cells[pos * r + c] = b * r + c;
            }
            ++pos;
        }
    }
    for (int j = n_keep + threadIdx.x; j < B; j += NT) sel_blocks[j] = -1;
    const int n_full = n_keep * r;
    for (int j = n_full + threadIdx.x; j < ld_cells; j += NT)
        sel_cells[j] = (j < n_full + tail) ? (int32_t)(nc * r + (j - n_full)) : -1;
}

// Register-resident element source for topk_threshold.  (A functor object,
// not a capturing lambda: with the array a member, full unrolling keeps every
// element in a register.)
template <int C, int NT>
struct RegKeys32 {  // score keys of blocks s*NT + tid, 0 = none
    uint32_t k[C];
    int tid;
    template <typename F>
    __device__ __forceinline__ void operator()(F &&fn) const {
#pragma unroll
        for (int s = 0; s < C; ++s) fn(k[s], ~(uint32_t)(s * NT + tid));
    }
};

// 64-bit sortable key of a candidate: (score key, ~block); 0 = none.
__device__ __forceinline__ uint64_t block_key(float s, int64_t b) {
    return ((uint64_t)score_key(s) << 32) | (uint64_t)(~(uint32_t)b);
}

__device__ __forceinline__ int32_t key_block(uint64_t key) { return (int32_t)(~(uint32_t)key); }

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
    const uint32_t lo = xor_lane_rt((uint32_t)v, m);
    const uint32_t hi = xor_lane_rt((uint32_t)(v >> 32), m);
    return ((uint64_t)hi << 32) | lo;
}

}  // namespace qsa
