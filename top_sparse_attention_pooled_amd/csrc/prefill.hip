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
//   5. k_select_prefill: the exact top-B of all blocks lies among the masked
//      ones.  Ranked by MFMA score, those more than 2 Delta above the B-th
//      largest are in it and those more than 2 Delta below are not; the few
//      between are rescored in order T and decide the rest.  If more blocks
//      pass than the LDS list holds, or Delta is outside the range where no
//      partial sum can overflow or underflow, every causal block is
//      rescored instead.
#include <type_traits>

#include "mfma_tile.h"
#include "topk_engine.h"
#include "wave_ops.h"

namespace qsa {

namespace {

constexpr int kSelPNT = 256;      // selection workgroup (two share a CU)
constexpr int kTauNT = 256;       // threshold workgroup
constexpr int kBandCap = 4096;    // masked blocks rescored from the LDS list (8 x B)
constexpr int kPrefMaxBlocks = kFusedMaxBlocks;
constexpr float kDeltaMin = 0x1p-100f, kDeltaMax = 0x1p100f;

__device__ __forceinline__ float key_value(uint32_t k) {
    const uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}

__device__ __forceinline__ float bf16_value(uint16_t h) {
    return __uint_as_float((uint32_t)h << 16);
}

// One launch, two roles.  Workgroups 0 .. ceil(n_q/4)-1: one wavefront per
// query, the roped query rounded to bf16 (zeros if the query is invalid) and
// Delta_i = 2^-15 * |q_i| * sqrt(d) * max(1, |gamma|) * (1 + 2^-8), each
// factor rounded up.  The rest: one wavefront per entry of the dirty list,
// its pooled key recomputed (the pooled-key update of the ubatch, which the
// scoring passes read; it shares the launch instead of taking one of its own).
__global__ __launch_bounds__(256) void k_rope_queries_delta(ScoreArgs a, const float *gamma,
                                                            PrefillWs w, UpdateArgs upd) {
    const int lane = threadIdx.x & (kWave - 1);
    const int n_rope_wg = (a.n_q + 3) / 4;
    if ((int)blockIdx.x >= n_rope_wg) {  // ---- update role ----
        const int e = ((int)blockIdx.x - n_rope_wg) * 4 + (int)(threadIdx.x >> 6);
        if (e >= upd.n_dirty) return;
        const int s = upd.dirty[2 * e], b = upd.dirty[2 * e + 1];
        if (s < 0 || s >= upd.g.n_seq || b < 0) return;
        const int64_t cap_blocks = upd.g.cap_cells / upd.r;
        if (b >= cap_blocks) return;
        int64_t n = upd.g.n_cells[s];
        if (n > upd.g.cap_cells) n = upd.g.cap_cells;
        if ((int64_t)b * upd.r >= n) return;
        float lo, hi;
        pooled_key_lane(upd.kidx, upd.g, s, b, n, upd.r, upd.eps, upd.gamma, upd.rope, lane, lo,
                        hi);
        store_pooled_lane(upd.pooled, upd.pooled_bf16, cap_blocks, s, b, lane, lo, hi);
        return;
    }
    const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= a.n_q) return;
    int s;
    int64_t p;
    bool valid;
    const int64_t nc =
        query_blocks(a.q_seq, a.q_pos, i, a.g.n_seq, a.g.cap_cells, a.g.n_cells, a.r, s, p, valid);
    if (lane == 0) w.qmeta[i] = make_int2(valid ? s : -1, (int)(nc < a.nb_max ? nc : a.nb_max));
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

// Maximum of two and of three floats.  The scores are MFMA results or lane
// exchanges of them, never NaN, so the NaN-propagating maximum (one
// v_maximum3_f32 for three operands) gives the same value as fmaxf without
// the quieting instructions fmaxf adds around a value it cannot prove
// canonical.  Builtins, not inline asm: the compiler then keeps the wait
// states an MFMA result needs before a vector instruction may read it.
__device__ __forceinline__ float max2f(float a, float b) {
    return __builtin_elementwise_maximum(a, b);
}
__device__ __forceinline__ float max3f(float a, float b, float c) {
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// The contraction: a panel of up to 512 queries against key groups of 64
// blocks, in work units of (group, half panel of 256 queries) with one
// wavefront per unit.  A workgroup = 8 wavefronts (one per CU) keeps one
// half panel's roped bf16 queries in LDS (68 KiB) and takes units of one set
// of 8 groups at a time, a group per wavefront; the two halves of a set go
// to workgroups on the same XCD (workgroups are dealt to the 8 XCDs round
// robin), so a group's second key load comes from that XCD's L2.  The
// wavefront loads its group's 16 KiB of keys straight into registers, then
// runs the half panel's queries through the matrix cores 16 at a time with
// the keys as the A operand and the queries, read from LDS, as the B
// operand.  The result tile is blocks x queries: lane (R, col) = (lane / 16,
// lane % 16) holds blocks 16*c + 4*R + jj (c, jj < 4) of query col, so the
// 16 blocks of a subgroup c lie in one register of the four lanes of a
// column, and a subgroup's maximum or a group's mask is an in-lane step and
// two permlane-swap steps across the rows.  Per query row and group of 64
// blocks a pass writes, for every group any row of its sequence needs
// (blocks past a row's causal limit never count):
//   kSubMax: w.smax[q][4*grp + c], the largest score of subgroup c (-inf if
//            none of its blocks is causal);
//   kMask:   w.mask[q][grp], bit j set when block 64*grp + j is causal and
//            its score is >= w.thr[q].
// The panel's rows usually belong to one sequence; otherwise the units are
// swept once per distinct sequence, storing only that sequence's rows.
constexpr int kPanelNT = 512;
constexpr int kPanelQ = 512;          // queries per panel
constexpr int kHalfQ = kPanelQ / 2;   // queries a workgroup holds
constexpr int kHalfTiles = kHalfQ / 64;
constexpr int kSetGroups = kPanelNT / kWave;  // groups per set: one per wavefront
constexpr int kXcds = 8;
constexpr int kQPitch = kDIdx + 8;  // LDS query row, padded: 16 rows of one read hit distinct banks

// Workgroups per panel for n_grp groups: both halves of every set, a
// multiple of 2 * kXcds so that a workgroup keeps its half in every round,
// at most the chip's CUs over the panels (but at least one round).
__host__ __device__ inline int panel_wgs(int n_grp, int n_panel) {
    const int n_sets = (n_grp + kSetGroups - 1) / kSetGroups;
    const int need = (2 * n_sets + 2 * kXcds - 1) / (2 * kXcds) * (2 * kXcds);
    const int room = max(2 * kXcds, 256 / max(n_panel, 1) / (2 * kXcds) * (2 * kXcds));
    return max(2 * kXcds, min(need, room));
}

// Workgroup slot v of a panel -> (half, set): v = 16*m + 8*h + x takes half
// h of set 8*m + x, and v + 8 the other half of the same set on the same XCD.
__device__ __forceinline__ void slot_unit(int v, int &half, int &set) {
    const int x = v % kXcds, k = v / kXcds;
    half = k & 1;
    set = (k >> 1) * kXcds + x;
}

// One group's 16 queries: 16 MFMA with the keys K as A and the queries of
// LDS rows rl (this lane's column) as B.
__device__ __forceinline__ void group_x_queries(const bf16x8_t (&K)[4][4],
                                                const uint16_t *qrow, int quad,
                                                f32x4_t (&acc)[4]) {
    bf16x8_t Q[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        Q[ks] = __builtin_bit_cast(bf16x8_t,
                                   *reinterpret_cast<const u32x4_t *>(qrow + ks * 32 + quad * 8));
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        f32x4_t z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(K[c][ks], Q[ks], z, 0, 0, 0);
        acc[c] = z;
    }
}

// Subgroup maxima of the tile (avail = causal blocks of the lane's query in
// the group, 64 when all are): lane (R, col) returns subgroup R of query col.
template <bool FULL>
__device__ __forceinline__ float tile_submax(const f32x4_t (&acc)[4], int avail, int quad) {
    float x[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        float v[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            v[jj] = (FULL || 16 * c + 4 * quad + jj < avail) ? acc[c][jj] : -INFINITY;
        x[c] = max2f(max3f(v[0], v[1], v[2]), v[3]);
    }
    // rows R, R+2 of subgroups (0, 2) and (1, 3), then rows R, R+1
    const auto p02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[0]),
                                                      __float_as_uint(x[2]), false, false);
    const auto p13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[1]),
                                                      __float_as_uint(x[3]), false, false);
    const float y02 = max2f(__uint_as_float(p02[0]), __uint_as_float(p02[1]));
    const float y13 = max2f(__uint_as_float(p13[0]), __uint_as_float(p13[1]));
    const auto pr = __builtin_amdgcn_permlane16_swap(__float_as_uint(y02), __float_as_uint(y13),
                                                     false, false);
    return max2f(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
}

// Mask word of the tile: rows 0-1 return the low word (blocks 0-31) of
// query col, rows 2-3 the high word.
template <bool FULL>
__device__ __forceinline__ uint32_t tile_mask(const f32x4_t (&acc)[4], float t, int avail,
                                              int quad) {
    uint32_t nib[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        uint32_t b = 0;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) b |= (acc[c][jj] >= t ? 1u : 0u) << jj;
        nib[c] = b;
    }
    const uint32_t lo = (nib[0] | nib[1] << 16) << (4 * quad);
    const uint32_t hi = (nib[2] | nib[3] << 16) << (4 * quad);
    // rows R, R+2 of the low and the high word, then rows R, R+1
    const auto p = __builtin_amdgcn_permlane32_swap(lo, hi, false, false);
    const uint32_t z = p[0] | p[1];
    const auto pz = __builtin_amdgcn_permlane16_swap(z, z, false, false);
    uint32_t m = pz[0] | pz[1];
    if (!FULL) {
        const int ab = avail - (quad >= 2 ? 32 : 0);  // causal blocks in this word
        if (ab < 32) m &= ab <= 0 ? 0u : (1u << ab) - 1u;
    }
    return m;
}

template <int MODE>
__global__ __launch_bounds__(kPanelNT) void k_prefill_scores(ScoreArgs a, PrefillWs w,
                                                             int wg_per_panel) {
    constexpr int kSt = MODE == kSubMax ? 0 : 4;  // stamp slots of this pass
    QSA_STAMP(kSt);
    __shared__ __align__(16) uint16_t s_q[kHalfQ][kQPitch];
    __shared__ int s_seq[kHalfQ];
    __shared__ int s_nc[kHalfQ];
    __shared__ float s_thr[kHalfQ];
    __shared__ uint64_t s_trows[kHalfTiles];  // per query tile: its rows of the swept sequence
    __shared__ int s_tmin[kHalfTiles], s_tmax[kHalfTiles];  // and their causal limits
    __shared__ int s_next;
    const int panel = blockIdx.x / wg_per_panel, wc = blockIdx.x % wg_per_panel;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & (kWave - 1);
    const int col = lane & 15, quad = lane >> 4;
    int half, set0;
    slot_unit(wc, half, set0);
    const int qh0 = panel * kPanelQ + half * kHalfQ;  // first query of the half
    const int n_rows = max(0, min(kHalfQ, a.n_q - qh0));
    const int n_qt = (n_rows + 63) / 64;
    const int64_t cap_blocks = a.g.cap_cells / a.r;
    const int64_t n_sub = 4 * (int64_t)w.n_grp;

    // every operand requested before the first wait: the rows' sequence and
    // causal limit (and threshold), the half's queries, then the first
    // unit's keys, for the sequence of the half's first row (the first sweep
    // is almost always over it; a wrong guess is reloaded).  Query pieces are
    // 16 bytes, row x / 16, part x % 16; rows past the last query repeat it:
    // a column of the B operand only reaches its own column of results, and
    // those are never stored.
    const int s0 = n_rows > 0 ? a.q_seq[qh0] : -1;
    int2 meta = make_int2(-1, 0);
    float thr_row = 0.f;
    if (tid < kHalfQ && tid < n_rows) {
        meta = w.qmeta[qh0 + tid];
        if constexpr (MODE == kMask) thr_row = w.thr[qh0 + tid];
    }
    constexpr int kPer = kHalfQ * 16 / kPanelNT;
    u32x4_t v[kPer];
    if (n_rows > 0) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int x = tid + i * kPanelNT, rr = min(x >> 4, n_rows - 1), part = x & 15;
            v[i] = *reinterpret_cast<const u32x4_t *>(w.qr + (int64_t)(qh0 + rr) * kDIdx +
                                                      part * 8);
        }
    }
    bf16x8_t K[4][4];
    int k_seq = -1, k_grp = set0 * kSetGroups + wave;
    if (s0 >= 0 && s0 < a.g.n_seq && k_grp < w.n_grp) {
        k_seq = s0;
        load_key_tile(a.pooled_bf16 + (int64_t)s0 * cap_blocks * kDIdx, (int64_t)k_grp * 64,
                      cap_blocks, true, K);
    }
    // row tid of the half (wavefronts 0-3): sequence, causal limit, threshold
    const int my_seq = meta.x, my_nc = meta.y;
    if (tid < kHalfQ) {
        s_seq[tid] = my_seq;
        s_nc[tid] = my_nc;
        if constexpr (MODE == kMask) s_thr[tid] = thr_row;
    }
    if (n_rows > 0) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int x = tid + i * kPanelNT, rr = x >> 4, part = x & 15;
            *reinterpret_cast<u32x4_t *>(&s_q[rr][part * 8]) = v[i];
        }
    }

    int sq = -1;  // the sequence being swept; rows of others are not stored
    bool first = true;
    for (;;) {
        // next sequence: the smallest valid one above sq among the half's rows
        if (tid == 0) s_next = 0x7fffffff;
        __syncthreads();
        {
            const int cand = my_seq > sq ? my_seq : 0x7fffffff;
            const int m = (int)wave_min_u32((uint32_t)cand);
            if (lane == 0 && m != 0x7fffffff) atomicMin(&s_next, m);
        }
        __syncthreads();
        const int nsq = s_next;
        if (nsq == 0x7fffffff) break;
        sq = nsq;
        if (wave < kHalfTiles) {  // wavefront t describes query tile t for this sweep
            const bool mine = my_seq == sq;
            const uint64_t rows = __ballot(mine);
            const uint32_t mx = wave_max_u32(mine ? (uint32_t)my_nc : 0u);
            const uint32_t mn = wave_min_u32(mine ? (uint32_t)my_nc : 0x7fffffffu);
            if (lane == 0) {
                s_trows[wave] = rows;
                s_tmax[wave] = (int)mx;
                s_tmin[wave] = (int)mn;
            }
        }
        __syncthreads();
        if (first) {
            QSA_STAMP(kSt + 1);
            first = false;
        }
        int ncmax = 0;
#pragma unroll
        for (int t = 0; t < kHalfTiles; ++t) ncmax = max(ncmax, s_tmax[t]);
        const int n_g = min((ncmax + 63) / 64, w.n_grp);
        const uint16_t *keys = a.pooled_bf16 + (int64_t)sq * cap_blocks * kDIdx;
        for (int v = wc; ; v += wg_per_panel) {
            int h, set;
            slot_unit(v, h, set);
            if (set * kSetGroups >= n_g) break;  // sets grow with v
            const int grp = set * kSetGroups + wave;
            if (grp >= n_g) continue;
            const int gb0 = grp * 64;
            if (k_seq != sq || k_grp != grp) {
                load_key_tile(keys, gb0, cap_blocks, true, K);
                k_seq = sq;
                k_grp = grp;
            }
            for (int qt = 0; qt < n_qt; ++qt) {
                const uint64_t rows = s_trows[qt];
                if (!rows || gb0 >= s_tmax[qt]) continue;
                const int64_t q0 = qh0 + qt * 64;
                if (rows == ~0ull && gb0 + 64 <= s_tmin[qt]) {
                    // every row of the tile is the sweep's and sees every block:
                    // straight-line code, every lane stores
#pragma unroll
                    for (int st = 0; st < 4; ++st) {
                        f32x4_t acc[4];
                        group_x_queries(K, &s_q[qt * 64 + st * 16 + col][0], quad, acc);
                        const int64_t qg = q0 + st * 16 + col;
                        if constexpr (MODE == kSubMax) {
                            w.smax[qg * n_sub + 4 * grp + quad] = tile_submax<true>(acc, 64, quad);
                        } else {
                            const uint32_t m = tile_mask<true>(acc, s_thr[qt * 64 + st * 16 + col],
                                                               64, quad);
                            // rows 0 and 1 (2 and 3) hold the same word
                            reinterpret_cast<uint32_t *>(w.mask)[(qg * w.n_grp + grp) * 2 +
                                                                 (quad >> 1)] = m;
                        }
                    }
                } else {
                    for (int st = 0; st < 4; ++st) {
                        const int rl = qt * 64 + st * 16 + col;  // this lane's query row
                        f32x4_t acc[4];
                        group_x_queries(K, &s_q[rl][0], quad, acc);
                        const bool store = (rows >> (st * 16 + col)) & 1;
                        const int64_t qg = q0 + st * 16 + col;
                        const int avail = s_nc[rl] - gb0;
                        if constexpr (MODE == kSubMax) {
                            const float m = tile_submax<false>(acc, avail, quad);
                            if (store) w.smax[qg * n_sub + 4 * grp + quad] = m;
                        } else {
                            const uint32_t m = tile_mask<false>(acc, s_thr[rl], avail, quad);
                            if (store && (quad & 1) == 0)
                                reinterpret_cast<uint32_t *>(w.mask)[(qg * w.n_grp + grp) * 2 +
                                                                     (quad >> 1)] = m;
                        }
                    }
                }
            }
            if (v == wc) QSA_STAMP(kSt + 2);
        }
    }
    QSA_STAMP(kSt + 3);
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

constexpr int kUCap = kWave;  // rescored band blocks one wavefront ranks
// Band histogram: 2^10 bins, lane l of one wavefront holding bins [16 l, 16
// l + 16); bin b at word b + b / 16, so that the lanes' reads hit different
// banks.
constexpr int kSelBinBits = 10;
constexpr int kSelBins = 1 << kSelBinBits;
constexpr int kSelBinsPerLane = kSelBins / kWave;
constexpr int kSelHistWords = kSelBins + kSelBins / kSelBinsPerLane;
__device__ __forceinline__ int hist_word(uint32_t b) { return (int)(b + (b >> 4)); }
__device__ __forceinline__ int sel_shift(uint32_t lo, uint32_t hi) {
    const uint32_t span = hi - lo;
    const int bits = span ? 32 - __builtin_clz(span) : 0;
    return bits > kSelBinBits ? bits - kSelBinBits : 0;
}

struct PrefSelSmem {
    TopkSmem<kSelPNT> tk;
    float q[kDIdx];
    // every-block path: the kept blocks' bitmap; band path: the histogram
    uint32_t bitmap[kPrefMaxBlocks / 32];
    uint64_t band[kBandCap];  // masked blocks, then their keys
    uint16_t xlist[kBandCap];  // band entries to rescore
    uint32_t n_unscored, kmin, kmax, n_in, n_u;
    float in_edge, out_edge;  // the bin of the B-th largest band score
};
static_assert(kSelHistWords <= kPrefMaxBlocks / 32, "histogram shares the bitmap");
static_assert(kSelBinsPerLane == 16, "bin padding assumes 16 bins per lane");

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
// tau_i the lower edge of the bin holding the B-th largest subgroup maximum
// of query i after two radix rounds (2^11 bins over [lo, hi] at the smallest
// power-of-two width, then within the chosen bin); -inf when fewer than B
// subgroups hold a causal block or Delta_i is out of range (every causal
// block then passes the filter).  PER (a power of two) maxima per thread
// cover up to kTauNT * PER subgroups.  Four workgroup barriers: after the
// count and range, after each round's histogram, after the first pick.
constexpr int kTauMaxPer = kPrefMaxBlocks / 16 / kTauNT;
template <int PER>
__global__ __launch_bounds__(kTauNT) void k_prefill_tau(ScoreArgs a, PrefillWs w, int top_k) {
    QSA_STAMP(8);
    constexpr int kW = kTauNT / kWave;
    __shared__ uint32_t s_hist[2][kHistWords];
    __shared__ uint32_t s_cnt[kW], s_mn[kW], s_mx[kW];
    __shared__ uint32_t s_pick[3];
    const int i = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = wave_id();
    const float *row = w.smax + (int64_t)i * 4 * w.n_grp;
    // every load issued before the first is used: indexes clamped to the
    // row (n_sub <= 4 n_grp), entries past n_sub dropped afterwards
    const int last = 4 * w.n_grp - 1;
    float v[PER];
#pragma unroll
    for (int c = 0; c < PER; ++c) v[c] = last >= 0 ? row[min(c * kTauNT + tid, last)] : 0.0f;
    const int n_sub = (w.qmeta[i].y + 15) / 16;
    const int B = top_k / a.r;
    const float delta = w.delta[i];
    for (int j = tid; j < 2 * kHistWords; j += kTauNT) (&s_hist[0][0])[j] = 0u;
    uint32_t key[PER];
    uint32_t cnt = 0, mn = ~0u, mx = 0u;
#pragma unroll
    for (int c = 0; c < PER; ++c) {
        const int x = c * kTauNT + tid;
        const uint32_t k = x < n_sub ? approx_key(v[c]) : 0u;
        key[c] = k;
        cnt += k != 0 ? 1u : 0u;  // (selects: a branch per key costs far more)
        mn = min(mn, k != 0 ? k : ~0u);
        mx = max(mx, k);
    }
    cnt = wave_sum_u32(cnt);
    mn = wave_min_u32(mn);
    mx = wave_max_u32(mx);
    if (lane == 0) {
        s_cnt[wave] = cnt;
        s_mn[wave] = mn;
        s_mx[wave] = mx;
    }
    __syncthreads();
    uint32_t n_valid = 0, lo = ~0u, hi = 0u;
#pragma unroll
    for (int u = 0; u < kW; ++u) {
        n_valid += s_cnt[u];
        lo = min(lo, s_mn[u]);
        hi = max(hi, s_mx[u]);
    }
    float thr = -INFINITY;
    if (n_valid >= (uint32_t)B && delta_in_range(delta)) {  // (block-uniform)
        uint32_t krem = (uint32_t)B;
        if (lo != hi) {
            int shift = range_shift(lo, hi);
#pragma unroll
            for (int c = 0; c < PER; ++c)
                if (key[c]) atomicAdd(&s_hist[0][hist_slot((key[c] - lo) >> shift)], 1u);
            __syncthreads();
            if (wave == 0) {
                uint32_t blo, bhi, babove, bcnt;
                wave_pick_bin(s_hist[0], lo, hi, shift, krem, blo, bhi, babove, bcnt);
                if (lane == 0) {
                    s_pick[0] = blo;
                    s_pick[1] = bhi;
                    s_pick[2] = babove;
                }
            }
            __syncthreads();
            lo = s_pick[0];
            hi = s_pick[1];
            krem -= s_pick[2];
            if (lo != hi) {
                shift = range_shift(lo, hi);
#pragma unroll
                for (int c = 0; c < PER; ++c)
                    if (key[c] - lo <= hi - lo)  // key in [lo, hi]
                        atomicAdd(&s_hist[1][hist_slot((key[c] - lo) >> shift)], 1u);
                __syncthreads();
                if (wave != 0) return;  // (no barrier follows)
                uint32_t bhi, babove, bcnt;
                wave_pick_bin(s_hist[1], lo, hi, shift, krem, lo, bhi, babove, bcnt);
            }
        }
        const float tau = key_value(lo);
        const double t = (double)tau - 2.0 * (double)delta;
        thr = (float)t;
        if ((double)thr > t) thr = nextafterf(thr, -INFINITY);
    }
    if (tid == 0) w.thr[i] = thr;
    QSA_STAMP(9);
}

// The kept entries of the band (ascending block order, exact keys) as the
// outputs emit_from_bitmap writes: blocks ascending, their cells, then the
// tail cells, -1 past them.  Thread tid takes a contiguous slice of the band.
__device__ void emit_from_band(const uint64_t *band, int total, Thresh th, int B, int r,
                               int64_t nc, int tail, int32_t *sel_blocks, int32_t *sel_cells,
                               int ld_cells, int32_t *n_sel, TopkSmem<kSelPNT> &sm) {
    const int per = (total + kSelPNT - 1) / kSelPNT;
    const int x0 = threadIdx.x * per, x1 = min(total, x0 + per);
    uint32_t local = 0;
    for (int x = x0; x < x1; ++x) {
        const uint64_t k = band[x];
        local += th.keep((uint32_t)(k >> 32), (uint32_t)k) ? 1u : 0u;
    }
    const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
    const uint32_t incl = wave_incl_scan_u32(local);
    if (lane == kWave - 1) sm.red[wave] = incl;
    __syncthreads();
    uint32_t before, kept;
    waves_prefix<kSelPNT / kWave>(sm.red, wave, before, kept);
    uint32_t pos = before + incl - local;
    const int n_keep = (int)(kept < (uint32_t)B ? kept : (uint32_t)B);
    if (threadIdx.x == 0) *n_sel = n_keep * r + tail;
    for (int x = x0; x < x1; ++x) {
        const uint64_t k = band[x];
        if (!th.keep((uint32_t)(k >> 32), (uint32_t)k)) continue;
        if ((int)pos < B) {
            const int32_t b = key_block(k);
            sel_blocks[pos] = b;
            for (int c = 0; c < r; ++c) sel_cells[pos * r + c] = b * r + c;
        }
        ++pos;
    }
    for (int j = n_keep + threadIdx.x; j < B; j += kSelPNT) sel_blocks[j] = -1;
    const int n_full = n_keep * r;
    for (int j = n_full + threadIdx.x; j < ld_cells; j += kSelPNT)
        sel_cells[j] = (j < n_full + tail) ? (int32_t)(nc * r + (j - n_full)) : -1;
}

// grid (n_q), kSelPNT threads: the exact top-B of query i among its masked
// blocks.  A masked block alone in its 16-block subgroup is the subgroup's
// maximum, so its MFMA score m_j is the stored maximum; a block sharing its
// subgroup with another masked one is rescored in order T (m_j = s_j).
// Either way |m_j - s_j| <= Delta.  With M the B-th largest m over the
// band: a block with m_j > M + 2 Delta is in the top-B (only blocks with m
// > M, fewer than B, can reach its score; blocks outside the band score
// below thr + Delta <= M + Delta), one with m_j < M - 2 Delta is not (B
// blocks score above it).  One histogram round brackets M; the blocks
// within 2 Delta of the bracket are rescored in order T, and the best of
// them by (s, lower block) fill the top-B up.
constexpr int kMaskPer = kPrefMaxBlocks / 64 / kSelPNT;  // group masks per thread, at most
__global__ __launch_bounds__(kSelPNT) void k_select_prefill(ScoreArgs a, PrefillWs w, int top_k,
                                                            int32_t *sel_blocks,
                                                            int32_t *sel_cells, int32_t *n_sel) {
    __shared__ PrefSelSmem sm;
    QSA_STAMP(10);
    const int i = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = wave_id();
    // thread tid takes groups [tid * per, tid * per + per), per from nb_max
    // (not from the query's own limit), so that the mask words and subgroup
    // maxima are requested before anything else returns; indexes clamped
    const int per = ((a.nb_max + 63) / 64 + kSelPNT - 1) / kSelPNT;
    const int g0 = tid * per, last = w.n_grp - 1;
    uint64_t mk[kMaskPer];
    f32x4_t mx[kMaskPer];
#pragma unroll
    for (int c = 0; c < kMaskPer; ++c) {
        if (c < per) {
            const int64_t g = (int64_t)i * w.n_grp + min(g0 + c, last);
            mk[c] = w.mask[g];
            mx[c] = *reinterpret_cast<const f32x4_t *>(w.smax + g * 4);
        } else {
            mk[c] = 0ull;
            mx[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
    const uint16_t qv = w.qr[(int64_t)i * kDIdx + (tid & (kDIdx - 1))];
    // the query's validity and sequence as the first launch resolved them
    // (no dependent load of the sequence's cell count here)
    const int2 meta = w.qmeta[i];
    const int64_t p = a.q_pos[i];
    const bool valid = meta.x >= 0;
    const int s = valid ? meta.x : 0;
    const int64_t nc = valid ? (p + 1) / a.r : 0;  // the complete visible blocks
    const int64_t limit = meta.y;                   // nc capped at nb_max
    const int B = top_k / a.r;
    const int64_t cap_blocks = a.g.cap_cells / a.r;
    const uint16_t *keys = a.pooled_bf16 + (valid ? (int64_t)s * cap_blocks * kDIdx : 0);
    const int n_words = (int)((limit + 31) / 32);
    const float delta = w.delta[i];
    bool exact_all = limit > 0 && !delta_in_range(delta);
    const int tail = valid ? (int)(p + 1 - nc * a.r) : 0;
    const int ld_cells = top_k + a.r - 1;
    int32_t *out_blocks = sel_blocks + (int64_t)i * B;
    int32_t *out_cells = sel_cells + (int64_t)i * ld_cells;

    if (!exact_all) {  // (limit 0: an empty band, the tail alone)
        const int n_g = (int)((limit + 63) / 64);
        for (int j = tid; j < kSelHistWords; j += kSelPNT) sm.bitmap[j] = 0u;
        if (tid == 0) {
            sm.n_unscored = 0u;
            sm.kmin = ~0u;
            sm.kmax = 0u;
            sm.n_in = 0u;
            sm.n_u = 0u;
            sm.in_edge = INFINITY;    // no block certainly in
            sm.out_edge = -INFINITY;  // none certainly out
        }
        uint32_t cnt = 0;
#pragma unroll
        for (int c = 0; c < kMaskPer; ++c) {
            if (g0 + c >= n_g) mk[c] = 0ull;
            cnt += (uint32_t)__popcll(mk[c]);
        }
        const uint32_t incl = wave_incl_scan_u32(cnt);
        if (lane == kWave - 1) sm.tk.red[wave] = incl;
        if (tid < kDIdx) sm.q[tid] = bf16_value(qv);
        __syncthreads();
        uint32_t before, total;
        waves_prefix<kSelPNT / kWave>(sm.tk.red, wave, before, total);
        if (total > (uint32_t)kBandCap) {
            exact_all = true;
        } else {
            // the masked blocks in ascending order, listed by the prefix
            // count; entry: (MFMA score bits << 32) | block, NaN where the
            // block shares its subgroup with another masked one
            // (the walk has no branch or atomic per bit: a block that needs
            // rescoring is marked by a NaN score and found by the pass below)
            uint32_t at = before + incl - cnt;
            uint32_t kmn = ~0u, kmx = 0u;
#pragma unroll
            for (int c = 0; c < kMaskPer; ++c) {
                const uint64_t M = mk[c];
                const f32x4_t v = mx[c];
                const int64_t gb = (int64_t)(g0 + c) * 64;
                uint64_t bits = M;
                while (bits) {
                    const int bit = __builtin_ctzll(bits);
                    bits &= bits - 1;
                    const int sub = bit >> 4;
                    const bool alone = __popc((uint32_t)(M >> (16 * sub)) & 0xffffu) == 1;
                    const float vs =
                        (sub & 2) ? ((sub & 1) ? v[3] : v[2]) : ((sub & 1) ? v[1] : v[0]);
                    const float m = alone ? vs : __builtin_nanf("");
                    const uint32_t k = approx_key(vs);
                    kmn = min(kmn, alone ? k : ~0u);
                    kmx = max(kmx, alone ? k : 0u);
                    sm.band[at++] = ((uint64_t)__float_as_uint(m) << 32) | (uint64_t)(gb + bit);
                }
            }
            __syncthreads();
            QSA_STAMP(11);
            // the listed blocks without an MFMA score (NaN), gathered into an
            // index list (one short pass), then rescored in order T at once
            for (int x = tid; x < (int)total; x += kSelPNT) {
                const float m = __uint_as_float((uint32_t)(sm.band[x] >> 32));
                if (m != m) sm.xlist[atomicAdd(&sm.n_unscored, 1u)] = (uint16_t)x;
            }
            __syncthreads();
            const int n_unscored = (int)sm.n_unscored;
            for (int j = tid; j < n_unscored; j += kSelPNT) {
                const int x = sm.xlist[j];
                const uint32_t b = (uint32_t)sm.band[x];
                const float sc = exact_score(keys + (int64_t)b * kDIdx, sm.q);
                const uint32_t k = approx_key(sc);
                kmn = min(kmn, k);
                kmx = max(kmx, k);
                sm.band[x] = ((uint64_t)__float_as_uint(sc) << 32) | b;
            }
            kmn = wave_min_u32(kmn);
            kmx = wave_max_u32(kmx);
            if (lane == 0) {
                atomicMin(&sm.kmin, kmn);
                atomicMax(&sm.kmax, kmx);
            }
            __syncthreads();
            const uint32_t klo = sm.kmin, khi = sm.kmax;
            const bool all_in = total <= (uint32_t)B;  // every masked block is kept
            if (!all_in) {  // (block-uniform) the bin holding the B-th largest m
                const int shift = sel_shift(klo, khi);
                for (int x = tid; x < (int)total; x += kSelPNT) {
                    const float m = __uint_as_float((uint32_t)(sm.band[x] >> 32));
                    atomicAdd(&sm.bitmap[hist_word((approx_key(m) - klo) >> shift)], 1u);
                }
                __syncthreads();
                if (wave == 0) {
                    uint32_t h[kSelBinsPerLane], local = 0;
#pragma unroll
                    for (int q = 0; q < kSelBinsPerLane; ++q) {
                        h[q] = sm.bitmap[lane * (kSelBinsPerLane + 1) + q];
                        local += h[q];
                    }
                    const uint32_t sc = wave_incl_scan_u32(local);
                    uint32_t above = lane_value(sc, kWave - 1) - sc;
                    uint32_t bin = 0;
                    bool found = false;
#pragma unroll
                    for (int q = kSelBinsPerLane - 1; q >= 0; --q) {
                        if (above < (uint32_t)B && above + h[q] >= (uint32_t)B) {
                            found = true;
                            bin = (uint32_t)(lane * kSelBinsPerLane + q);
                        }
                        above += h[q];
                    }
                    const uint64_t hit = __ballot(found);
                    bin = lane_value(bin, __builtin_ctzll(hit));
                    if (lane == 0) {
                        const uint64_t e = (uint64_t)klo + ((uint64_t)(bin + 1) << shift) - 1;
                        sm.in_edge = key_value(e < (uint64_t)khi ? (uint32_t)e : khi);
                        sm.out_edge = key_value(klo + (bin << shift));
                    }
                }
                __syncthreads();
            }
            QSA_STAMP(12);
            // final keys: blocks certainly in above every order-T key, blocks
            // certainly out 0; the rest listed, then rescored in order T
            const double d2 = 2.0 * (double)delta;
            const double in_above = (double)sm.in_edge + d2, out_below = (double)sm.out_edge - d2;
            uint32_t my_in = 0;
            for (int x = tid; x < (int)total; x += kSelPNT) {
                const uint64_t e = sm.band[x];
                const double m = (double)__uint_as_float((uint32_t)(e >> 32));
                const uint32_t b = (uint32_t)e;
                if (all_in || m > in_above) {
                    sm.band[x] = (0xffffffffull << 32) | (uint64_t)(~b);
                    ++my_in;
                } else if (m < out_below) {
                    sm.band[x] = 0ull;
                } else {
                    sm.xlist[atomicAdd(&sm.n_u, 1u)] = (uint16_t)x;
                }
            }
            my_in = wave_sum_u32(my_in);
            if (lane == 0 && my_in) atomicAdd(&sm.n_in, my_in);
            __syncthreads();
            const uint32_t n_u = sm.n_u, n_in = sm.n_in;
            Thresh th{0u, 0u, false};  // every nonzero key kept
            if (n_u > (uint32_t)kUCap) {
                for (int j = tid; j < (int)n_u; j += kSelPNT) {
                    const int x = sm.xlist[j];
                    const uint32_t b = (uint32_t)sm.band[x];
                    sm.band[x] = block_key(exact_score(keys + (int64_t)b * kDIdx, sm.q), b);
                }
                __syncthreads();
                BandKeys bk;
#pragma unroll
                for (int c = 0; c < kBandCap / kSelPNT; ++c) {
                    const int x = c * kSelPNT + tid;
                    bk.k[c] = x < (int)total ? sm.band[x] : 0ull;
                }
                th = topk_threshold<kSelPNT>(bk, (uint32_t)B, sm.tk);
            } else if (n_u > 0) {
                if (wave == 0) {  // one block per lane; the best B - n_in stay
                    const uint32_t need = (uint32_t)B > n_in ? (uint32_t)B - n_in : 0u;
                    const bool mine_live = lane < (int)n_u;
                    const int x = mine_live ? sm.xlist[lane] : 0;
                    uint64_t mine = 0ull;
                    if (mine_live) {
                        const uint32_t b = (uint32_t)sm.band[x];
                        mine = block_key(exact_score(keys + (int64_t)b * kDIdx, sm.q), b);
                    }
                    uint32_t rank = 0;
                    for (int j = 0; j < (int)n_u; ++j) {
                        const uint64_t o = ((uint64_t)lane_value((uint32_t)(mine >> 32), j) << 32) |
                                           lane_value((uint32_t)mine, j);
                        rank += o > mine ? 1u : 0u;
                    }
                    if (mine_live) sm.band[x] = rank < need ? mine : 0ull;
                }
                __syncthreads();
            }
            QSA_STAMP(13);
            emit_from_band(sm.band, (int)total, th, B, a.r, nc, tail, out_blocks, out_cells,
                           ld_cells, n_sel + i, sm.tk);
        }
    }
    if (exact_all) {
        if (tid < kDIdx) sm.q[tid] = bf16_value(w.qr[(int64_t)i * kDIdx + tid]);
        for (int x = tid; x < n_words; x += kSelPNT) sm.bitmap[x] = 0;
        __syncthreads();
        ExactStream src;
        src.limit = limit;
        src.keys = keys;
        src.q = sm.q;
        const Thresh th = topk_threshold<kSelPNT>(src, (uint32_t)B, sm.tk);
        src([&](uint32_t k, uint32_t u) {
            if (th.keep(k, u)) mark(sm.bitmap, ~u);
        });
        __syncthreads();
        emit_from_bitmap<kSelPNT>(sm.bitmap, n_words, B, a.r, nc, tail, out_blocks, out_cells,
                                  ld_cells, n_sel + i, sm.tk);
    }
    QSA_STAMP(14);
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
    d.qmeta = reinterpret_cast<int2 *>(take((size_t)n_q * 8));
    if (w) *w = d;
    return off;
}

QSA_STAMP_READER(prefill)

size_t prefill_ws_bytes(int n_q, int nb_max) {
    return n_q > 0 ? prefill_layout(nullptr, n_q, nb_max, nullptr) : 0;
}

hipError_t launch_score_select_prefill(const ScoreArgs &a, const float *gamma, void *ws,
                                       int top_k, int32_t *sel_blocks, int32_t *sel_cells,
                                       int32_t *n_sel, const UpdateArgs &upd, hipStream_t st) {
    if (a.n_q <= 0) return launch_update_pooled(upd, st);
    PrefillWs w;
    prefill_layout(static_cast<char *>(ws), a.n_q, a.nb_max, &w);
    const int n_upd_wg = upd.n_dirty > 0 ? (upd.n_dirty + 3) / 4 : 0;
    hipLaunchKernelGGL(k_rope_queries_delta, dim3((a.n_q + 3) / 4 + n_upd_wg), dim3(256), 0, st,
                       a, gamma, w, upd);
    // per panel of 512 queries, workgroups for both halves of its sets of
    // groups, XCD-paired (one per CU, at most the chip's 256 CUs in all)
    const int n_panel = (a.n_q + kPanelQ - 1) / kPanelQ;
    const int wg_per_panel = panel_wgs(w.n_grp, n_panel);
    const int grid = n_panel * wg_per_panel;
    if (w.n_grp > 0)
        hipLaunchKernelGGL(k_prefill_scores<kSubMax>, dim3(grid), dim3(kPanelNT), 0, st, a, w,
                           wg_per_panel);
    {
        const int64_t n_sub = (a.nb_max + 15) / 16;  // subgroups of the longest query, at most
        if (n_sub <= 4 * kTauNT)
            hipLaunchKernelGGL(k_prefill_tau<4>, dim3(a.n_q), dim3(kTauNT), 0, st, a, w, top_k);
        else if (n_sub <= 8 * kTauNT)
            hipLaunchKernelGGL(k_prefill_tau<8>, dim3(a.n_q), dim3(kTauNT), 0, st, a, w, top_k);
        else if (n_sub <= 16 * kTauNT)
            hipLaunchKernelGGL(k_prefill_tau<16>, dim3(a.n_q), dim3(kTauNT), 0, st, a, w, top_k);
        else
            hipLaunchKernelGGL(k_prefill_tau<kTauMaxPer>, dim3(a.n_q), dim3(kTauNT), 0, st, a, w,
                               top_k);
    }
    if (w.n_grp > 0)
        hipLaunchKernelGGL(k_prefill_scores<kMask>, dim3(grid), dim3(kPanelNT), 0, st, a, w,
                           wg_per_panel);
    hipLaunchKernelGGL(k_select_prefill, dim3(a.n_q), dim3(kSelPNT), 0, st, a, w, top_k,
                       sel_blocks, sel_cells, n_sel);
    return hipGetLastError();
}

}  // namespace qsa
