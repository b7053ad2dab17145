// prefill.hip -- the prefill indexer: block scores of many queries on the
// matrix cores with an exact block top-k per query (llama.cpp issue #28734,
// fix summary, "lever3": whole blocks compete, ties to the lower block), in
// the canonical order T over bf16-rounded operands.
//
// The bf16 contraction runs on MFMA, whose fp32 sums differ from T only in
// the order of the additions: each order is within (d - 1) * 2^-24 * sum
// |q_t k_t| of the true sum, and sum |q_t k_t| <= |q_i| * |k| with |k| <=
// sqrt(d) * max(1, |gamma|) for an RMS-normed key, so |s_mfma - s_T| <=
// Delta_i = 2^-15 * |q_i| * sqrt(d) * max(1, |gamma|) * (1 + 2^-8), rounded
// up.  The MFMA scores are never stored:
//   1. k_rope_queries_delta: roped bf16 queries and Delta_i;
//   2. k_prefill_scores<kSubMax>: per query, the largest MFMA score of each
//      16-block subgroup of its causal blocks;
//   3. k_prefill_tau: tau_i = a value that at least B of those maxima reach:
//      the lower edge of the bin that holds the B-th largest after two radix
//      rounds over the maxima's keys, at most 2^10 units in the last place
//      (about 2^-13 of the score) below the B-th largest itself, which a
//      third round would pin.  One round is too coarse: its range spans the
//      negative and the positive keys, and its bin lets far more blocks
//      through to the rescoring.  B distinct blocks then have MFMA score >=
//      tau_i, so the exact B-th largest score S_B is >= tau_i - Delta, and
//      every block of the exact top-B has MFMA score >= S_B - Delta >= tau_i
//      - 2 Delta.  The filter threshold is tau_i - 2 Delta rounded down
//      (-inf, every causal block, when there are fewer than B subgroups);
//   4. k_prefill_scores<kMask>: per (query, 64-block group), a bit mask of
//      the blocks whose MFMA score reaches the threshold;
//   5. k_select_prefill: the masked blocks rescored in order T; their exact
//      top-B is the exact top-B of all blocks, which lies among them.  If
//      more blocks pass than the LDS list holds, or Delta is outside the
//      range where no partial sum can overflow or underflow, every causal
//      block is rescored instead.
#include <type_traits>

#include "mfma_tile.h"
#include "topk_engine.h"
#include "wave_ops.h"

namespace qsa {

namespace {

constexpr int kSelPNT = 256;      // selection workgroup (two share a CU)
constexpr int kBandCap = 4096;    // masked blocks rescored from the LDS list (8 x B)
constexpr int kTauNT = 256;       // threshold workgroup
constexpr int kPrefMaxBlocks = kFusedMaxBlocks;
constexpr float kDeltaMin = 0x1p-100f, kDeltaMax = 0x1p100f;

__device__ __forceinline__ float key_value(uint32_t k) {
    const uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}

__device__ __forceinline__ float bf16_value(uint16_t h) {
    return __uint_as_float((uint32_t)h << 16);
}

// One wavefront per query: the roped query rounded to bf16 (zeros if the
// query is invalid) and Delta_i = 2^-15 * |q_i| * sqrt(d) * max(1, |gamma|)
// * (1 + 2^-8), each factor rounded up.
__global__ __launch_bounds__(256) void k_rope_queries_delta(ScoreArgs a, const float *gamma,
                                                            PrefillWs w) {
    const int lane = threadIdx.x & (kWave - 1);
    const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= a.n_q) return;
    int s;
    int64_t p;
    bool valid;
    query_blocks(a.q_seq, a.q_pos, i, a.g.n_seq, a.g.cap_cells, a.g.n_cells, a.r, s, p, valid);
    uint16_t lo16 = 0, hi16 = 0;
    if (valid) {
        float lo, hi;
        rope_query_pair(a.q_idx + (int64_t)i * kDIdx, lane, p, a.rope, lo, hi);
        lo16 = bf16_rne(lo);
        hi16 = bf16_rne(hi);
    }
    w.qr[(int64_t)i * kDIdx + lane] = lo16;
    w.qr[(int64_t)i * kDIdx + lane + 64] = hi16;
    const float ql = bf16_value(lo16), qh = bf16_value(hi16);
    float ss = ql * ql + qh * qh;
    ss += xor_lane_f<1>(ss);
    ss += xor_lane_f<2>(ss);
    ss += xor_lane_f<4>(ss);
    ss += xor_lane_f<8>(ss);
    ss += xor_lane_f<16>(ss);
    ss += xor_lane_f<32>(ss);
    float gm = 1.0f;
    if (gamma) gm = fmaxf(gm, fmaxf(fabsf(gamma[lane]), fabsf(gamma[lane + 64])));
    gm = wave_max_f32(gm);
    if (lane == 0) {
        // fp32 sum of 128 squares: relative error below 2^-17; inflate
        const double qn = sqrt((double)ss * (1.0 + 0x1p-14));
        w.delta[i] = valid ? (float)(0x1p-15 * qn * sqrt((double)kDIdx) * (double)gm *
                                     (1.0 + 0x1p-8) * (1.0 + 0x1p-10))
                           : 0.0f;
    }
}

// What a k_prefill_scores pass leaves per query row and group of 64 blocks.
constexpr int kSubMax = 0;  // the largest MFMA score of each 16-block subgroup
constexpr int kMask = 1;    // the bit mask of blocks whose score reaches the threshold

// Max of v[0..3] (the four 16-block subgroups of a group, cb) over the 16
// lanes of a DPP row: exchange-halving steps, so lane col ends with the
// maximum of subgroup 2*bit3(col) + bit2(col).
__device__ __forceinline__ float row16_max4(float (&v)[4], int col) {
    const bool hi8 = col & 8, hi4 = col & 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const float keep = hi8 ? v[h + 2] : v[h];
        const float send = hi8 ? v[h] : v[h + 2];
        v[h] = fmaxf(keep, xor_lane_f<8>(send));
    }
    const float keep = hi4 ? v[1] : v[0];
    const float send = hi4 ? v[0] : v[1];
    float m = fmaxf(keep, xor_lane_f<4>(send));
    m = fmaxf(m, xor_lane_f<2>(m));
    m = fmaxf(m, xor_lane_f<1>(m));
    return m;
}

// 1-D grid over (slab sb of `slab` group tiles, query tile qt of 64
// queries); a group tile is 4 groups of 64 blocks, one per wavefront.  The
// hardware deals workgroup ids to the 8 XCDs round-robin, so ids are laid out
// to put the query tiles of one slab on one XCD, where its keys are read
// from HBM once and then hit that XCD's L2.  A workgroup loads its queries
// once and sweeps its slab.  Per query row and group it writes, for every
// group any row of its sequence needs (blocks past a row's causal limit never
// count):
//   kSubMax: w.smax[q][4*grp + c], the largest score of subgroup c (-inf if
//            none of its blocks is causal);
//   kMask:   w.mask[q][grp], bit j set when block 64*grp + j is causal and
//            its score is >= w.thr[q].
// When all valid queries of the tile belong to one sequence (the usual
// ubatch) the next group's keys are in flight while the current group is on
// the matrix cores; otherwise each group is swept once per distinct sequence.
template <int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_prefill_scores(ScoreArgs a, PrefillWs w, int n_gt,
                                                       int n_qt, int slab) {
    const int id = blockIdx.x;
    const int n_slab = (n_gt + slab - 1) / slab;
    const int sb = (id / (8 * n_qt)) * 8 + (id & 7);
    const int qt = (id / 8) % n_qt;
    if (sb >= n_slab) return;
    const int gt0 = sb * slab, gt1 = min(n_gt, gt0 + slab);
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & (kWave - 1);
    const int q0 = qt * 64;
    const int64_t cap_blocks = a.g.cap_cells / a.r;
    auto grp_of = [&](int gt) { return (int64_t)(gt * 4 + wave); };
    // lane r: the query of row r (sequence, -1 if invalid or past n_q)
    int my_seq = -1, my_nc = 0;
    {
        const int qi = q0 + lane;
        if (qi < a.n_q) {
            int64_t p;
            bool valid;
            const int64_t nc = query_blocks(a.q_seq, a.q_pos, qi, a.g.n_seq, a.g.cap_cells,
                                            a.g.n_cells, a.r, my_seq, p, valid);
            if (!valid) my_seq = -1;
            my_nc = (int)(nc < a.nb_max ? nc : a.nb_max);
        }
    }
    const uint64_t valid_rows = __ballot(my_seq >= 0);
    if (!valid_rows) return;  // (the same for every wavefront of the workgroup)
    // the 64 rows' causal limits and thresholds, for the result layout: lane
    // l holds rows rb*16 + 4*(l/16) + jj of column l % 16
    __shared__ int s_nc[64];
    __shared__ float s_thr[64];
    // the 64 roped queries (A operands), rows padded to 272 bytes so the 16
    // rows one MFMA operand read touches fall in different banks
    constexpr int kQPitch = kDIdx + 8;
    __shared__ __align__(16) uint16_t s_q[64][kQPitch];
    if (wave == 0) {
        s_nc[lane] = my_nc;
        if constexpr (MODE == kMask) s_thr[lane] = q0 + lane < a.n_q ? w.thr[q0 + lane] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int x = u * 256 + (int)threadIdx.x;  // 16-byte piece: row x / 16, part x % 16
        const int rr = x >> 4, part = x & 15;
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (q0 + rr < a.n_q)
            v = *reinterpret_cast<const u32x4_t *>(w.qr + (int64_t)(q0 + rr) * kDIdx + part * 8);
        *reinterpret_cast<u32x4_t *>(&s_q[rr][part * 8]) = v;
    }
    __syncthreads();
    const int col = lane & 15, quad = lane >> 4;
    const int64_t n_sub = 4 * (int64_t)w.n_grp;
    // One 16-row band rb of the 64 x 64 tile on the matrix cores, then its
    // epilogue (the band's accumulators are all that is live).
    // FULL: every block of the group is causal for every stored row, so no
    // per-element limit test
    auto tile_as = [&](auto full, const bf16x8_t (&B)[4][4], int64_t grp, uint64_t rows) {
        constexpr bool FULL = decltype(full)::value;
        const int64_t gb0 = grp * 64;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            bf16x8_t A[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                A[ks] = __builtin_bit_cast(
                    bf16x8_t, *reinterpret_cast<const u32x4_t *>(&s_q[rb * 16 + col][ks * 32 + quad * 8]));
            f32x4_t acc[4];
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[ks], B[cb][ks], c, 0, 0, 0);
                acc[cb] = c;
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int r = rb * 16 + quad * 4 + jj;
                const int lim = FULL ? 0 : s_nc[r];
                if constexpr (MODE == kSubMax) {
                    float v[4];
#pragma unroll
                    for (int cb = 0; cb < 4; ++cb)
                        v[cb] = (FULL || gb0 + cb * 16 + col < lim) ? acc[cb][jj] : -INFINITY;
                    const float m = row16_max4(v, col);
                    // lanes 0, 4, 8, 12 of the row hold subgroups 0, 1, 2, 3
                    if ((col & 3) == 0 && ((rows >> r) & 1))
                        w.smax[(int64_t)(q0 + r) * n_sub + 4 * grp + (col >> 2)] = m;
                } else {
                    const float t = s_thr[r];
                    uint64_t mk = 0;
#pragma unroll
                    for (int cb = 0; cb < 4; ++cb) {
                        const bool pass = (FULL || gb0 + cb * 16 + col < lim) && acc[cb][jj] >= t;
                        const uint64_t bal = __ballot(pass);
                        mk |= ((bal >> (16 * quad)) & 0xffffull) << (16 * cb);
                    }
                    if (col == 0 && ((rows >> r) & 1))
                        w.mask[(int64_t)(q0 + r) * w.n_grp + grp] = mk;
                }
            }
        }
    };
    auto tile = [&](const bf16x8_t (&B)[4][4], int64_t grp, uint64_t rows) {
        // smallest causal limit of the stored rows (lane r holds row r's)
        const uint32_t ncmin = wave_min_u32(((rows >> lane) & 1) ? (uint32_t)my_nc : ~0u);
        if ((uint64_t)grp * 64 + 64 <= ncmin)
            tile_as(std::true_type{}, B, grp, rows);
        else
            tile_as(std::false_type{}, B, grp, rows);
    };

    const int sq0 = __shfl(my_seq, __builtin_ctzll(valid_rows));
    if (__ballot(my_seq >= 0 && my_seq != sq0) == 0) {
        const int ncmax = (int)wave_max_u32(my_seq >= 0 ? (uint32_t)my_nc : 0u);
        const uint16_t *keys = a.pooled_bf16 + (int64_t)sq0 * cap_blocks * kDIdx;
        auto live_of = [&](int gt) {
            return grp_of(gt) < w.n_grp && grp_of(gt) * 64 < ncmax;
        };
        // one key buffer: the other wavefront on the SIMD covers the wait
        for (int gt = gt0; gt < gt1; ++gt) {
            if (!live_of(gt)) continue;
            bf16x8_t B[4][4];
            load_key_tile(keys, grp_of(gt) * 64, cap_blocks, true, B);
            tile(B, grp_of(gt), valid_rows);
        }
        return;
    }
    for (int gt = gt0; gt < gt1; ++gt) {
        if (grp_of(gt) >= w.n_grp) continue;
        const int64_t gb0 = grp_of(gt) * 64;
        uint64_t done = ~valid_rows;
        while (done != ~0ull) {
            const int sq = __shfl(my_seq, __builtin_ctzll(~done));
            const uint64_t rows = __ballot(my_seq == sq);
            const int ncmax = (int)wave_max_u32((my_seq == sq) ? (uint32_t)my_nc : 0u);
            done |= rows;
            if (gb0 >= ncmax) continue;
            bf16x8_t B[4][4];
            load_key_tile(a.pooled_bf16 + (int64_t)sq * cap_blocks * kDIdx, gb0, cap_blocks, true, B);
            tile(B, grp_of(gt), rows);
        }
    }
}

// Exact score of block b under order T: bf16 key row against the query held
// in LDS as fp32 (both bf16 values, so every product is exact).  Dims t and
// t + 64 meet at T's first level and t, t + 32 at the second, so the row is
// taken in two halves (dims 0-31 with 64-95, then 32-63 with 96-127) and the
// second half folded in as it arrives.
__device__ __forceinline__ float exact_score(const uint16_t *krow, const float *q) {
    float v[32];
    const u32x4_t *kp = reinterpret_cast<const u32x4_t *>(krow);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {  // dims 32h + 8c .. +7 and 64 + 32h + 8c .. +7
            const u32x4_t lo = kp[4 * half + c], hi = kp[8 + 4 * half + c];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 32 * half + 8 * c + 2 * e;
                const float k0 = __uint_as_float(lo[e] << 16);
                const float k1 = __uint_as_float(lo[e] & 0xffff0000u);
                const float h0 = __uint_as_float(hi[e] << 16);
                const float h1 = __uint_as_float(hi[e] & 0xffff0000u);
                const float p0 = q[t] * k0, p1 = q[t + 1] * k1;
                const float r0 = q[t + 64] * h0, r1 = q[t + 65] * h1;
                const float v0 = p0 + r0, v1 = p1 + r1;  // level h = 64
                if (half == 0) {
                    v[t] = v0;
                    v[t + 1] = v1;
                } else {
                    v[t - 32] = v[t - 32] + v0;  // level h = 32
                    v[t - 31] = v[t - 31] + v1;
                }
            }
        }
    }
#pragma unroll
    for (int h = 16; h >= 1; h >>= 1)
#pragma unroll
        for (int t = 0; t < h; ++t) v[t] = v[t] + v[t + h];
    return v[0];
}

struct PrefSelSmem {
    TopkSmem<kSelPNT> tk;
    float q[kDIdx];
    uint32_t bitmap[kPrefMaxBlocks / 32];
    uint64_t band[kBandCap];  // masked blocks, then their exact keys
};

__device__ __forceinline__ uint32_t approx_key(float v) {
    return finite_f32(v) ? score_key(v) : 0u;
}

// Exact keys of the masked blocks (slot c holds entry c * kSelPNT + tid).
struct BandKeys {
    uint64_t k[kBandCap / kSelPNT];
    template <typename F>
    __device__ __forceinline__ void operator()(F &&fn) const {
#pragma unroll
        for (int c = 0; c < kBandCap / kSelPNT; ++c) fn((uint32_t)(k[c] >> 32), (uint32_t)k[c]);
    }
};

// Every causal block rescored exactly, on each pass.
struct ExactStream {
    int64_t limit;
    const uint16_t *keys;
    const float *q;
    template <typename F>
    __device__ __forceinline__ void operator()(F &&fn) const {
        for (int64_t b = threadIdx.x; b < limit; b += kSelPNT) {
            const float sc = exact_score(keys + b * kDIdx, q);
            fn(finite_f32(sc) ? score_key(sc) : 0u, ~(uint32_t)b);
        }
    }
};

__device__ __forceinline__ void mark(uint32_t *bm, uint32_t b) {
    atomicOr(&bm[b >> 5], 1u << (b & 31));
}

__device__ __forceinline__ bool delta_in_range(float delta) {
    return delta >= kDeltaMin && delta <= kDeltaMax;  // false for NaN
}

// grid (n_q), kTauNT threads: w.thr[i] = tau_i - 2 Delta_i rounded down,
// tau_i the B-th largest subgroup maximum of query i; -inf when fewer than B
// subgroups hold a causal block or Delta_i is out of range (every causal
// block then passes the filter).
constexpr int kTauPer = kPrefMaxBlocks / 16 / kTauNT;  // subgroup maxima per thread
__global__ __launch_bounds__(kTauNT) void k_prefill_tau(ScoreArgs a, PrefillWs w, int top_k) {
    __shared__ TopkSmem<kTauNT> sm;
    const int i = blockIdx.x, tid = threadIdx.x;
    int s;
    int64_t p;
    bool valid;
    const int64_t nc = query_blocks(a.q_seq, a.q_pos, i, a.g.n_seq, a.g.cap_cells, a.g.n_cells,
                                    a.r, s, p, valid);
    const int64_t limit = nc < a.nb_max ? nc : a.nb_max;
    const int n_sub = (int)((limit + 15) / 16);
    const int B = top_k / a.r;
    const float delta = w.delta[i];
    const float *row = w.smax + (int64_t)i * 4 * w.n_grp;
    RegKeys32<kTauPer, kTauNT> keys;
    keys.tid = tid;
    uint32_t cnt = 0, mn = ~0u, mx = 0u;
#pragma unroll
    for (int c = 0; c < kTauPer; ++c) {
        const int x = c * kTauNT + tid;
        const uint32_t k = x < n_sub ? approx_key(row[x]) : 0u;
        keys.k[c] = k;
        if (k) {
            ++cnt;
            mn = min(mn, k);
            mx = max(mx, k);
        }
    }
    const uint32_t n_valid = block_sum_u32<kTauNT>(cnt, sm);
    float thr = -INFINITY;
    if (n_valid >= (uint32_t)B && delta_in_range(delta)) {
        block_minmax_u32<kTauNT>(mn, mx, sm);
        // two rounds: the bin holding the B-th largest key, then the sub-bin
        // within it; every key at or above the sub-bin's lower edge is >= it,
        // and there are at least B of them
        uint32_t lo = mn, hi = mx, krem = (uint32_t)B;
        for (int round = 0; round < 2 && lo != hi; ++round) {
            const int shift = range_shift(lo, hi);
            for (int j = tid; j < kBins; j += kTauNT) sm.hist[j] = 0;
            __syncthreads();
            keys([&](uint32_t k, uint32_t) {
                if (k >= lo && k <= hi) atomicAdd(&sm.hist[(k - lo) >> shift], 1u);
            });
            __syncthreads();
            pick_bin<kTauNT>(sm, lo, hi, shift, krem);
            krem -= sm.b_above;
            lo = sm.b_lo;
            hi = sm.b_hi;
            __syncthreads();
        }
        const float tau = key_value(lo);
        const double t = (double)tau - 2.0 * (double)delta;
        thr = (float)t;
        if ((double)thr > t) thr = nextafterf(thr, -INFINITY);
    }
    if (tid == 0) w.thr[i] = thr;
}

// grid (n_q), kSelPNT threads: the exact top-B of query i among its masked
// blocks, rescored in order T.
constexpr int kMaskPer = kPrefMaxBlocks / 64 / kSelPNT;  // group masks per thread
__global__ __launch_bounds__(kSelPNT) void k_select_prefill(ScoreArgs a, PrefillWs w, int top_k,
                                                            int32_t *sel_blocks,
                                                            int32_t *sel_cells, int32_t *n_sel) {
    __shared__ PrefSelSmem sm;
    const int i = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = wave_id();
    int s;
    int64_t p;
    bool valid;
    const int64_t nc = query_blocks(a.q_seq, a.q_pos, i, a.g.n_seq, a.g.cap_cells, a.g.n_cells,
                                    a.r, s, p, valid);
    const int64_t limit = nc < a.nb_max ? nc : a.nb_max;
    const int B = top_k / a.r;
    const int64_t cap_blocks = a.g.cap_cells / a.r;
    const uint16_t *keys = a.pooled_bf16 + (valid ? (int64_t)s * cap_blocks * kDIdx : 0);
    if (tid < kDIdx) sm.q[tid] = bf16_value(w.qr[(int64_t)i * kDIdx + tid]);
    const int n_words = (int)((limit + 31) / 32);
    for (int x = tid; x < n_words; x += kSelPNT) sm.bitmap[x] = 0;
    bool exact_all = limit > 0 && !delta_in_range(w.delta[i]);

    if (limit > 0 && !exact_all) {
        // the masked blocks, listed by a prefix count over the masks
        const int n_g = (int)((limit + 63) / 64);
        uint64_t mk[kMaskPer];
        uint32_t cnt = 0;
#pragma unroll
        for (int c = 0; c < kMaskPer; ++c) {
            const int g = tid * kMaskPer + c;
            mk[c] = g < n_g ? w.mask[(int64_t)i * w.n_grp + g] : 0ull;
            cnt += (uint32_t)__popcll(mk[c]);
        }
        const uint32_t incl = wave_incl_scan_u32(cnt);
        if (lane == kWave - 1) sm.tk.red[wave] = incl;
        __syncthreads();
        uint32_t before, total;
        waves_prefix<kSelPNT / kWave>(sm.tk.red, wave, before, total);
        if (total > (uint32_t)kBandCap) {
            exact_all = true;
        } else {
            uint32_t at = before + incl - cnt;
#pragma unroll
            for (int c = 0; c < kMaskPer; ++c) {
                uint64_t bits = mk[c];
                const int64_t g0 = (int64_t)(tid * kMaskPer + c) * 64;
                while (bits) {
                    sm.band[at++] = (uint64_t)(g0 + __builtin_ctzll(bits));
                    bits &= bits - 1;
                }
            }
            __syncthreads();
            for (int x = tid; x < (int)total; x += kSelPNT) {
                const int64_t b = (int64_t)sm.band[x];
                sm.band[x] = block_key(exact_score(keys + b * kDIdx, sm.q), b);
            }
            __syncthreads();
            BandKeys bk;
#pragma unroll
            for (int c = 0; c < kBandCap / kSelPNT; ++c) {
                const int x = c * kSelPNT + tid;
                bk.k[c] = x < (int)total ? sm.band[x] : 0ull;
            }
            const Thresh th = topk_threshold<kSelPNT>(bk, (uint32_t)B, sm.tk);
            bk([&](uint32_t k, uint32_t u) {
                if (th.keep(k, u)) mark(sm.bitmap, ~u);
            });
        }
    }
    if (exact_all) {
        ExactStream src;
        src.limit = limit;
        src.keys = keys;
        src.q = sm.q;
        const Thresh th = topk_threshold<kSelPNT>(src, (uint32_t)B, sm.tk);
        src([&](uint32_t k, uint32_t u) {
            if (th.keep(k, u)) mark(sm.bitmap, ~u);
        });
    }
    __syncthreads();
    const int tail = valid ? (int)(p + 1 - nc * a.r) : 0;
    const int ld_cells = top_k + a.r - 1;
    emit_from_bitmap<kSelPNT>(sm.bitmap, n_words, B, a.r, nc, tail,
                              sel_blocks + (int64_t)i * B, sel_cells + (int64_t)i * ld_cells,
                              ld_cells, n_sel + i, sm.tk);
}

}  // namespace

// Workspace layout (each part 256-byte aligned); with base == nullptr only
// the total is computed.
static size_t prefill_layout(char *base, int n_q, int nb_max, PrefillWs *w) {
    PrefillWs d{};
    d.n_grp = (nb_max + 255) / 256 * 4;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += (bytes + 255) / 256 * 256;
        return base ? base + at : nullptr;
    };
    d.smax = reinterpret_cast<float *>(take((size_t)n_q * d.n_grp * 4 * 4));
    d.thr = reinterpret_cast<float *>(take((size_t)n_q * 4));
    d.mask = reinterpret_cast<uint64_t *>(take((size_t)n_q * d.n_grp * 8));
    d.qr = reinterpret_cast<uint16_t *>(take((size_t)n_q * kDIdx * 2));
    d.delta = reinterpret_cast<float *>(take((size_t)n_q * 4));
    if (w) *w = d;
    return off;
}

size_t prefill_ws_bytes(int n_q, int nb_max) {
    return n_q > 0 ? prefill_layout(nullptr, n_q, nb_max, nullptr) : 0;
}

hipError_t launch_score_select_prefill(const ScoreArgs &a, const float *gamma, void *ws,
                                       int top_k, int32_t *sel_blocks, int32_t *sel_cells,
                                       int32_t *n_sel, hipStream_t st) {
    if (a.n_q <= 0) return hipSuccess;
    PrefillWs w;
    prefill_layout(static_cast<char *>(ws), a.n_q, a.nb_max, &w);
    hipLaunchKernelGGL(k_rope_queries_delta, dim3((a.n_q + 3) / 4), dim3(256), 0, st, a, gamma,
                       w);
    const int qt = (a.n_q + 63) / 64;
    // slabs of group tiles: about 512 workgroups (two per CU); the grid is
    // padded to whole rounds of the 8 XCDs (k_prefill_scores maps ids)
    const int n_gt = w.n_grp / 4;
    const int n_slab = max(1, min(n_gt, 512 / qt));
    const int slab = max(1, (n_gt + n_slab - 1) / n_slab);
    const int grid = ((n_gt + slab - 1) / slab + 7) / 8 * 8 * qt;
    if (n_gt > 0)
        hipLaunchKernelGGL(k_prefill_scores<kSubMax>, dim3(grid), dim3(256), 0, st, a, w, n_gt,
                           qt, slab);
    hipLaunchKernelGGL(k_prefill_tau, dim3(a.n_q), dim3(kTauNT), 0, st, a, w, top_k);
    if (n_gt > 0)
        hipLaunchKernelGGL(k_prefill_scores<kMask>, dim3(grid), dim3(256), 0, st, a, w, n_gt, qt,
                           slab);
    hipLaunchKernelGGL(k_select_prefill, dim3(a.n_q), dim3(kSelPNT), 0, st, a, w, top_k,
                       sel_blocks, sel_cells, n_sel);
    return hipGetLastError();
}

}  // namespace qsa
