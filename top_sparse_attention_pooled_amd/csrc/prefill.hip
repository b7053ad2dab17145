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
// up.  Selection then needs exact scores only near the cut:
//   1. k_rope_queries_delta: roped bf16 queries and Delta_i;
//   2. k_prefill_scores: the MFMA score matrix, written densely;
//   3. k_select_prefill, per query: a_B = the B-th largest MFMA score
//      (radix select on the row).  Since at least B blocks have MFMA score
//      >= a_B, the exact B-th largest S_B is >= a_B - Delta; and S_B <= a_B
//      + Delta.  So a block with MFMA score > a_B + 2 Delta scores exactly
//      above S_B (kept), one below a_B - 2 Delta exactly below S_B (dropped),
//      and only the band in between is rescored in order T; the exact top
//      (B - kept) of the band completes the set.  If the band overflows its
//      LDS list, or Delta is outside the range where no partial sum can
//      overflow or underflow, every causal block is rescored instead.
#include "mfma_tile.h"
#include "topk_engine.h"
#include "wave_ops.h"

namespace qsa {

namespace {

constexpr int kSelPNT = 512;      // selection workgroup (256 registers per lane)
constexpr int kApproxVec = 26;    // score vectors of 4 blocks held in registers per thread
constexpr int kBandCap = 4096;    // band blocks rescored from the LDS list
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

// 1-D grid over (slab sb of `slab` group tiles, query tile qt of 64
// queries); a group tile is 4 groups of 64 blocks, one per wavefront.  The
// hardware deals workgroup ids to the 8 XCDs round-robin, so ids are laid out
// to put the query tiles of one slab on one XCD, where its keys are read
// from HBM once and then hit that XCD's L2.  A workgroup loads its queries
// once and sweeps its slab, writing w.approx[q][b] for every causal block of
// its rows (other entries are left as they are: the selection never reads
// them).  When all valid queries of the tile belong to one sequence (the
// usual ubatch) the next group's keys are in flight while the current group
// is on the matrix cores; otherwise each group is swept once per distinct
// sequence.
__global__ __launch_bounds__(256) void k_prefill_scores(ScoreArgs a, PrefillWs w, int n_gt,
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
    if (!valid_rows) return;
    bf16x8_t A[4][4];
    load_query_tile(w.qr, q0, a.n_q, A);
    // result lane l holds rows rb*16 + 4*(l/16) + jj of column l % 16
    const int rsub = (lane >> 4) * 4;
    float *const out = w.approx + (int64_t)q0 * w.ld + (lane & 15);
    f32x4_t acc[4][4];
    auto store_rows = [&](int64_t gb0, uint64_t rows) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int r = rb * 16 + rsub + jj;
                if (!((rows >> r) & 1)) continue;
                float *const p = out + (int64_t)r * w.ld + gb0;
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) p[cb * 16] = acc[rb][cb][jj];
            }
    };

    const int sq0 = __shfl(my_seq, __builtin_ctzll(valid_rows));
    if (__ballot(my_seq >= 0 && my_seq != sq0) == 0) {
        const int ncmax = (int)wave_max_u32(my_seq >= 0 ? (uint32_t)my_nc : 0u);
        const uint16_t *keys = a.pooled_bf16 + (int64_t)sq0 * cap_blocks * kDIdx;
        auto live_of = [&](int gt) {
            return grp_of(gt) < w.n_grp && grp_of(gt) * 64 < ncmax;
        };
        auto sweep = [&](int gt, const bf16x8_t (&B)[4][4]) {
            if (!live_of(gt)) return;
            mfma_tile(A, B, acc);
            store_rows(grp_of(gt) * 64, valid_rows);
        };
        // two key buffers: the next group's keys are in flight while the
        // current group is on the matrix cores
        bf16x8_t B0[4][4], B1[4][4];
        load_key_tile(keys, grp_of(gt0) * 64, cap_blocks, live_of(gt0), B0);
        for (int gt = gt0; gt < gt1; gt += 2) {
            if (gt + 1 < gt1)
                load_key_tile(keys, grp_of(gt + 1) * 64, cap_blocks, live_of(gt + 1), B1);
            sweep(gt, B0);
            if (gt + 1 >= gt1) break;
            if (gt + 2 < gt1)
                load_key_tile(keys, grp_of(gt + 2) * 64, cap_blocks, live_of(gt + 2), B0);
            sweep(gt + 1, B1);
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
            wave_tile_mfma(A, a.pooled_bf16 + (int64_t)sq * cap_blocks * kDIdx, gb0, cap_blocks,
                           true, acc);
            store_rows(gb0, rows);
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
    uint64_t band[kBandCap];  // band blocks, then their exact keys
    uint32_t n_band;
};

__device__ __forceinline__ uint32_t approx_key(float v, int64_t b, int64_t limit) {
    return (b < limit && finite_f32(v)) ? score_key(v) : 0u;
}

// Keys of the MFMA scores of one query's causal blocks, as (k, ~block):
// blocks 4x .. 4x+3 for x = c * kSelPNT + tid, in registers for c <
// kApproxVec and re-read from the row beyond.
struct ApproxKeys {
    uint32_t k[kApproxVec][4];
    const float *row;
    int64_t limit;
    int n_vec;
    template <typename F>
    __device__ __forceinline__ void operator()(F &&fn) const {
        const int tid = threadIdx.x;
#pragma unroll
        for (int c = 0; c < kApproxVec; ++c) {
            const uint32_t b0 = (uint32_t)(c * kSelPNT + tid) * 4u;
#pragma unroll
            for (int e = 0; e < 4; ++e) fn(k[c][e], ~(b0 + e));
        }
        for (int x = kApproxVec * kSelPNT + tid; x < n_vec; x += kSelPNT) {
            const f32x4_t v = *reinterpret_cast<const f32x4_t *>(row + 4 * (int64_t)x);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t b = 4 * (int64_t)x + e;
                fn(approx_key(v[e], b, limit), ~(uint32_t)b);
            }
        }
    }
};

// Exact keys of the band list (slot c holds entry c * kSelPNT + tid).
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

// grid (n_q), kSelPNT threads: the exact top-B of query i from its row of
// MFMA scores plus exact rescoring of the band around the cut.
__global__ __launch_bounds__(kSelPNT) void k_select_prefill(ScoreArgs a, PrefillWs w, int top_k,
                                                            int32_t *sel_blocks,
                                                            int32_t *sel_cells, int32_t *n_sel) {
    __shared__ PrefSelSmem sm;
    const int i = blockIdx.x, tid = threadIdx.x;
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
    if (tid == 0) sm.n_band = 0;
    const int n_words = (int)((limit + 31) / 32);
    for (int x = tid; x < n_words; x += kSelPNT) sm.bitmap[x] = 0;
    const float delta = w.delta[i];
    const bool safe = delta >= kDeltaMin && delta <= kDeltaMax;  // false for NaN
    bool exact_all = limit > 0 && !safe;

    if (limit > 0 && safe) {
        ApproxKeys ak;
        ak.row = w.approx + (int64_t)i * w.ld;
        ak.limit = limit;
        ak.n_vec = (int)((limit + 3) / 4);
#pragma unroll
        for (int c = 0; c < kApproxVec; ++c) {
            const int x = c * kSelPNT + tid;
            f32x4_t v = {0.f, 0.f, 0.f, 0.f};
            if (x < ak.n_vec) v = *reinterpret_cast<const f32x4_t *>(ak.row + 4 * (int64_t)x);
#pragma unroll
            for (int e = 0; e < 4; ++e) ak.k[c][e] = approx_key(v[e], 4 * (int64_t)x + e, limit);
        }
        // with Delta in range no sum overflows, so every causal block has a
        // finite score under both orders
        uint32_t cnt = 0, mn = ~0u, mx = 0u;
        ak([&](uint32_t k, uint32_t) {
            if (!k) return;
            ++cnt;
            mn = min(mn, k);
            mx = max(mx, k);
        });
        // low 18 bits: valid keys (<= 2^17); above: threads holding one
        const uint32_t packed = block_sum_u32<kSelPNT>(cnt + (cnt ? 1u << 18 : 0u), sm.tk);
        const uint32_t n_valid = packed & ((1u << 18) - 1u), n_holders = packed >> 18;
        if (n_valid <= (uint32_t)B) {
            ak([&](uint32_t k, uint32_t u) {
                if (k) mark(sm.bitmap, ~u);
            });
        } else {
            // Every holder has a key >= its own largest, so at least
            // n_holders keys are >= the smallest of those maxima: if that is
            // B or more, the B-th largest lies above it, and the first
            // radix round bins only the top of the distribution (not the
            // bulk, whose keys would crowd a few bins).
            uint32_t lo = cnt ? mx : ~0u, hi = mx;
            block_minmax_u32<kSelPNT>(lo, hi, sm.tk);
            if (n_holders < (uint32_t)B) {
                uint32_t unused = 0u;
                block_minmax_u32<kSelPNT>(mn, unused, sm.tk);
                lo = mn;
            }
            const float a_B = key_value(kth_largest_u32<kSelPNT>(ak, (uint32_t)B, lo, hi, sm.tk));
            const double tlo = (double)a_B - 2.0 * (double)delta;
            const double thi = (double)a_B + 2.0 * (double)delta;
            float flo = (float)tlo, fhi = (float)thi;
            if ((double)flo > tlo) flo = nextafterf(flo, -INFINITY);
            if ((double)fhi < thi) fhi = nextafterf(fhi, INFINITY);
            const uint32_t k_lo = score_key(flo), k_hi = score_key(fhi);
            uint32_t n_keep = 0;
            ak([&](uint32_t k, uint32_t u) {
                if (k > k_hi) {
                    mark(sm.bitmap, ~u);
                    ++n_keep;
                } else if (k >= k_lo) {
                    const uint32_t at = atomicAdd(&sm.n_band, 1u);
                    if (at < (uint32_t)kBandCap) sm.band[at] = (uint64_t)(~u);
                }
            });
            n_keep = block_sum_u32<kSelPNT>(n_keep, sm.tk);  // ends with a barrier
            const uint32_t n_band = sm.n_band;
            if (n_band > (uint32_t)kBandCap) {
                exact_all = true;
                for (int x = tid; x < n_words; x += kSelPNT) sm.bitmap[x] = 0;
                __syncthreads();
            } else {
                for (int x = tid; x < (int)n_band; x += kSelPNT) {
                    const int64_t b = (int64_t)sm.band[x];
                    sm.band[x] = block_key(exact_score(keys + b * kDIdx, sm.q), b);
                }
                __syncthreads();
                BandKeys bk;
#pragma unroll
                for (int c = 0; c < kBandCap / kSelPNT; ++c) {
                    const int x = c * kSelPNT + tid;
                    bk.k[c] = x < (int)n_band ? sm.band[x] : 0ull;
                }
                const Thresh th = topk_threshold<kSelPNT>(bk, (uint32_t)B - n_keep, sm.tk);
                bk([&](uint32_t k, uint32_t u) {
                    if (th.keep(k, u)) mark(sm.bitmap, ~u);
                });
            }
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
    d.ld = (int64_t)d.n_grp * 64;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += (bytes + 255) / 256 * 256;
        return base ? base + at : nullptr;
    };
    d.approx = reinterpret_cast<float *>(take((size_t)n_q * d.ld * 4));
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
        hipLaunchKernelGGL(k_prefill_scores, dim3(grid), dim3(256), 0, st, a, w, n_gt, qt, slab);
    hipLaunchKernelGGL(k_select_prefill, dim3(a.n_q), dim3(kSelPNT), 0, st, a, w, top_k,
                       sel_blocks, sel_cells, n_sel);
    return hipGetLastError();
}

}  // namespace qsa
