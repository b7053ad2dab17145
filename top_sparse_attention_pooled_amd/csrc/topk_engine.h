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

// A histogram of kBins bins, bin q at word q + q / 32: one wavefront reads
// it with lane l holding bins [32 l, 32 l + 32), and those reads hit
// different banks.
constexpr int kHistWords = kBins + kBins / 32;
__device__ __forceinline__ int hist_slot(uint32_t q) { return (int)(q + (q >> 5)); }

template <int NT>
struct TopkSmem {
    uint32_t hist[2][kHistWords];  // the radix rounds alternate between two
    uint32_t red[NT / 64];
    uint32_t red2[NT / 64];
    uint32_t red3[NT / 64];
    uint32_t b_lo, b_hi, b_above, b_cnt;
};

// The kept set: valid (k != 0) and (k > T, or k == T and (!tie or u >= U)).
// As one unsigned comparison of the 64-bit key k:u with the bound
// T:(tie ? U : 0), raised to 1:0 so that k = 0 stays out (T is a valid key,
// so T >= 1, whenever it is not 0 with no tie).  (The short-circuit form
// compiles to three nested branches per key, several hundred cycles each
// time a workgroup tests its keys.)
struct Thresh {
    uint32_t T;
    uint32_t U;
    bool tie;
    __device__ __forceinline__ uint64_t bound() const {
        const uint64_t b = ((uint64_t)T << 32) | (tie ? U : 0u);
        return b > (1ull << 32) ? b : (1ull << 32);
    }
    __device__ __forceinline__ bool keep(uint32_t k, uint32_t u) const {
        return (((uint64_t)k << 32) | u) >= bound();
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

__device__ __forceinline__ int range_shift(uint32_t lo, uint32_t hi) {
    const uint32_t span = hi - lo;
    const int bits = span ? 32 - __builtin_clz(span) : 0;
    return bits > kBinBits ? bits - kBinBits : 0;
}

// One radix round's choice, made by a single wavefront (every lane gets the
// result): the bin of hist (kBins bins of width 2^shift over [lo, hi]) that
// holds the krem-th largest value; its range [blo, bhi], the values in
// higher bins (babove) and in it (bcnt).  Lane l sums bins [32 l, 32 l +
// 32); a scan over the lanes finds the lane L whose bins hold the crossing,
// then lane q < 32 reads bin 32 L + q and a second scan finds the bin (few
// registers: the fused decode kernel keeps two workgroups per CU).
__device__ __forceinline__ void wave_pick_bin(const uint32_t *hist, uint32_t lo, uint32_t hi,
                                              int shift, uint32_t krem, uint32_t &blo,
                                              uint32_t &bhi, uint32_t &babove, uint32_t &bcnt) {
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t local = 0;
#pragma unroll
    for (int q = 0; q < 32; ++q) local += hist[lane * 33 + q];
    const uint32_t incl = wave_incl_scan_u32(local);
    const uint32_t above = lane_value(incl, kWave - 1) - incl;  // values in higher lanes' bins
    const int L = __builtin_ctzll(__ballot(above < krem && above + local >= krem));
    const uint32_t above_l = lane_value(above, L);
    const uint32_t h = lane < 32 ? hist[L * 33 + lane] : 0u;
    const uint32_t incl2 = wave_incl_scan_u32(h);
    const uint32_t ab = above_l + (lane_value(incl2, 31) - incl2);  // values in higher bins
    const int q = __builtin_ctzll(__ballot(lane < 32 && ab < krem && ab + h >= krem));
    const uint32_t bin = (uint32_t)(L * 32 + q);
    babove = lane_value(ab, q);
    bcnt = lane_value(h, q);
    blo = lo + (bin << shift);
    bhi = blo + ((1u << shift) - 1u);
    if (bhi > hi || bhi < blo) bhi = hi;
}

// Radix select of the krem-th largest of the values v = VAL(k, u) over the
// elements with PRED(k, u), in [lo, hi].  Histogram hist[buf] is clear on
// entry; each round fills it, wavefront 0 picks the bin while the others
// clear the other one for the next round (two barriers per round; every
// thread has read the round's result when it returns, no barrier after).
// Returns the threshold value; n_above gets the count strictly above it;
// done tells whether count(v >= threshold) == krem (no tie left at the
// threshold).  On return hist[buf] is clear again.
template <int NT, typename ForEach, typename Pred, typename Val>
__device__ __forceinline__ uint32_t select_u32(const ForEach &for_each, Pred pred, Val val,
                                               uint32_t krem, uint32_t lo, uint32_t hi,
                                               TopkSmem<NT> &sm, int &buf, uint32_t &n_above,
                                               bool &done) {
    const int wave = wave_id();
    n_above = 0;
    done = false;
    // not unrolled: a workgroup runs this once, and each copy of a round
    // would be instructions fetched cold
#pragma unroll 1
    for (int round = 0; round < 4; ++round) {
        const int shift = range_shift(lo, hi);
        uint32_t *hist = sm.hist[buf];
        // (one branch per element, around the atomic: v in [lo, hi] as one
        // unsigned compare, the predicate combined without short circuit)
        for_each([&](uint32_t k, uint32_t u) {
            const uint32_t v = val(k, u);
            if (pred(k, u) & (v - lo <= hi - lo))
                atomicAdd(&hist[hist_slot((v - lo) >> shift)], 1u);
        });
        __syncthreads();
        if (wave == 0) {
            uint32_t blo, bhi, babove, bcnt;
            wave_pick_bin(hist, lo, hi, shift, krem, blo, bhi, babove, bcnt);
            if ((threadIdx.x & (kWave - 1)) == 0) {
                sm.b_lo = blo;
                sm.b_hi = bhi;
                sm.b_above = babove;
                sm.b_cnt = bcnt;
            }
        } else {
            uint32_t *other = sm.hist[buf ^ 1];
            for (int j = (int)threadIdx.x - kWave; j < kHistWords; j += NT - kWave) other[j] = 0u;
        }
        __syncthreads();
        QSA_STAMP_LDS(8 + (round < 3 ? round : 3));
        const uint32_t above = sm.b_above, cnt = sm.b_cnt;
        lo = sm.b_lo;
        hi = sm.b_hi;
        n_above += above;
        krem -= above;
        buf ^= 1;
        if (cnt == krem) {
            done = true;
            break;
        }
        if (__builtin_expect(lo == hi, 0)) break;  // one value shared by more than krem elements
    }
    return lo;
}

// The exact kept set of the top B (or every valid element if there are at
// most B).  Count and range of the valid keys in one reduction (both
// histograms cleared meanwhile), then radix rounds over the score keys and,
// for a tie at the threshold, over the block order.  When it returns, every
// thread is past its reads of sm.red: the caller may reuse that.
template <int NT, typename ForEach>
__device__ __forceinline__ Thresh topk_threshold(const ForEach &for_each, uint32_t B, TopkSmem<NT> &sm) {
    constexpr int NW = NT / 64;
    static_assert(NW >= 2, "a wavefront picks while the others clear");
    const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
    Thresh th{0u, 0u, false};
    uint32_t cnt = 0, mn = ~0u, mx = 0u;
    for_each([&](uint32_t k, uint32_t) {  // (selects, no branches)
        cnt += k != 0 ? 1u : 0u;
        mn = min(mn, k != 0 ? k : ~0u);
        mx = max(mx, k);
    });
    QSA_STAMP_LDS(1);
    cnt = wave_sum_u32(cnt);
    mn = wave_min_u32(mn);
    mx = wave_max_u32(mx);
    if (lane == 0) {
        sm.red[wave] = cnt;
        sm.red2[wave] = mn;
        sm.red3[wave] = mx;
    }
    for (int j = threadIdx.x; j < 2 * kHistWords; j += NT) (&sm.hist[0][0])[j] = 0u;
    __syncthreads();
    const uint32_t n_valid = wave_sum_u32(lane < NW ? sm.red[lane] : 0u);
    const uint32_t lo = wave_min_u32(lane < NW ? sm.red2[lane] : ~0u);
    const uint32_t hi = wave_max_u32(lane < NW ? sm.red3[lane] : 0u);
    QSA_STAMP_LDS(7);
    if (__builtin_expect(n_valid <= B, 0)) {  // T = 0: every valid element
        __syncthreads();
        return th;
    }
    int buf = 0;
    uint32_t n_above;
    bool done;
    th.T = select_u32<NT>(
        for_each, [](uint32_t k, uint32_t) { return k != 0; },
        [](uint32_t k, uint32_t) { return k; }, B, lo, hi, sm, buf, n_above, done);
    if (__builtin_expect(done, 1)) return th;
    // ties at score key T: keep the lowest blocks (largest u) among them
    const uint32_t T = th.T;
    uint32_t umn = ~0u, umx = 0u;
    for_each([&](uint32_t k, uint32_t u) {
        const bool at_t = k == T;
        umn = min(umn, at_t ? u : ~0u);
        umx = max(umx, at_t ? u : 0u);
    });
    umn = wave_min_u32(umn);
    umx = wave_max_u32(umx);
    if (lane == 0) {
        sm.red2[wave] = umn;
        sm.red3[wave] = umx;
    }
    __syncthreads();
    const uint32_t ulo = wave_min_u32(lane < NW ? sm.red2[lane] : ~0u);
    const uint32_t uhi = wave_max_u32(lane < NW ? sm.red3[lane] : 0u);
    th.U = select_u32<NT>(
        for_each, [T](uint32_t k, uint32_t) { return k == T; },
        [](uint32_t, uint32_t u) { return u; }, B - n_above, ulo, uhi, sm, buf, n_above, done);
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
