// prefill.hip -- the prefill indexer: block scores of many queries on the
// matrix cores with an exact block top-k per query (llama.cpp issue #28734,
// fix summary, "lever3": whole blocks compete, ties to the lower block), in
// the canonical order T over bf16-rounded operands.
//
// The bf16 contraction runs on MFMA, whose fp32 sums differ from T only in
// order: |s_mfma - s_T| <= Delta_i = 2^-15 * |q_i| * K_max bounds it (twice
// (d - 1) * 2^-24 * sum |q_t k_t|, with room for the 6 key bits used as a
// tie-break below).  The full score matrix (512 x ~50k floats at depth) is
// never written:
//   1. k_rope_queries_delta: roped bf16 queries and Delta_i;
//   2. k_prefill_tiles<kSample>: MFMA over every 8th 64-block group, scores
//      to a small matrix;
//   3. k_sample_threshold: per query the B-th largest sampled score s_B;
//      since at least B blocks score >= s_B - Delta exactly, every block of
//      the exact top-B has an MFMA score >= theta_lo = s_B - 2 Delta;
//   4. k_prefill_tiles<kFilter>: MFMA over all groups; each score is
//      compared with theta_lo and a 64-bit mask per (query, group) marks the
//      candidates (one compare per score; the masks are assembled from the
//      compare results on the scalar unit);
//   5. k_select_prefill: per query the candidates are rescored exactly in
//      order T and the exact top-B taken, then emitted like every selection.
#include "mfma_tile.h"
#include "topk_engine.h"
#include "wave_ops.h"

namespace qsa {

namespace {

constexpr int kSampleStride = 8;  // every 8th 64-block group is sampled
constexpr int kSampNT = 1024;     // sample-threshold workgroup
constexpr int kSelPNT = 512;      // selection workgroup (256 registers per lane)
constexpr int kPrefCandCap = 8192;   // candidates per query before the slow path
constexpr int kPrefMaxBlocks = kFusedMaxBlocks;

enum { kSample = 0, kFilter = 1 };

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

// 1-D grid over (group tile gt of 4 groups, query tile qt of 64 queries):
// the hardware deals workgroup ids to the 8 XCDs round-robin, so ids are
// laid out to put the query tiles of one group tile on one XCD, where its
// keys are read from HBM once and then hit that XCD's L2.  Wavefront w takes
// 64-block group (4*gt + w) * stride (sample: stride 8) for 64 queries.
// kSample: the scores (-inf where not causal) go to w.sample[q][(4gt+w)*64 +
// col].  kFilter: bit col of w.mask[q][group] is set if the block is causal
// and its MFMA score >= w.theta[q].  Queries of one tile may belong to
// different sequences: the tile is swept once per distinct sequence.
template <int MODE>
__global__ __launch_bounds__(256) void k_prefill_tiles(ScoreArgs a, PrefillWs w, int n_gt,
                                                      int n_qt) {
    const int id = blockIdx.x;
    const int gt = (id / (8 * n_qt)) * 8 + (id & 7);
    const int qt = (id / 8) % n_qt;
    if (gt >= n_gt) return;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & (kWave - 1);
    const int q0 = qt * 64;
    const int slot = gt * 4 + wave;  // sample column group, or group
    const int64_t grp = MODE == kSample ? (int64_t)slot * kSampleStride : slot;
    const int64_t gb0 = grp * 64;
    const int64_t cap_blocks = a.g.cap_cells / a.r;
    const bool group_ok = MODE == kSample ? slot < w.n_sgrp : grp < w.n_grp;
    if (!group_ok) return;
    // lane r: the query of row r (sequence, causal blocks, threshold)
    int my_seq = -2, my_nc = 0;
    float my_th = 0.0f;
    {
        const int qi = q0 + lane;
        if (qi < a.n_q) {
            int64_t p;
            bool valid;
            const int64_t nc = query_blocks(a.q_seq, a.q_pos, qi, a.g.n_seq, a.g.cap_cells,
                                            a.g.n_cells, a.r, my_seq, p, valid);
            if (!valid) my_seq = -1;
            my_nc = (int)(nc < a.nb_max ? nc : a.nb_max);
            if (MODE == kFilter) my_th = w.theta[qi];
        }
    }

    bf16x8_t A[4][4];
    load_query_tile(w.qr, q0, a.n_q, A);
    // per-lane row constants: row rb*16 + 4*(lane/16) + jj
    int nc_r[4][4];
    float th_r[4][4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int r = rb * 16 + (lane >> 4) * 4 + jj;
            nc_r[rb][jj] = __shfl(my_nc, r);
            th_r[rb][jj] = __shfl(my_th, r);
        }
    const int mrow = lane & 15;

    uint64_t done = __ballot(my_seq == -2);  // rows past n_q: nothing to write
    while (done != ~0ull) {
        const int r0 = __builtin_ctzll(~done);
        const int sq = __shfl(my_seq, r0);
        const uint64_t rows = __ballot(my_seq == sq);
        const int ncmax = (int)wave_max_u32((my_seq == sq) ? (uint32_t)my_nc : 0u);
        done |= rows;
        const bool live = sq >= 0 && gb0 < ncmax;
        f32x4_t acc[4][4];
        if (live) {
            const uint16_t *keys = a.pooled_bf16 + (int64_t)sq * cap_blocks * kDIdx;
            wave_tile_mfma(A, keys, gb0, cap_blocks, true, acc);
        }
        if (MODE == kSample) {
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int r = rb * 16 + (lane >> 4) * 4 + jj;
                        if (!((rows >> r) & 1)) continue;
                        const int64_t b = gb0 + cb * 16 + mrow;
                        const float v = (live && b < nc_r[rb][jj]) ? acc[rb][cb][jj] : -INFINITY;
                        w.sample[(int64_t)(q0 + r) * w.ld_s + slot * 64 + cb * 16 + mrow] = v;
                    }
        } else {
            // lane r collects the mask of row r
            uint32_t m_lo = 0, m_hi = 0;
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    uint64_t mc[4];
#pragma unroll
                    for (int cb = 0; cb < 4; ++cb) {
                        const int64_t b = gb0 + cb * 16 + mrow;
                        const bool pass = live && b < nc_r[rb][jj] &&
                                          acc[rb][cb][jj] >= th_r[rb][jj];
                        mc[cb] = __ballot(pass);
                    }
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const uint32_t lo = (uint32_t)((mc[0] >> (16 * k)) & 0xffffu) |
                                            (uint32_t)(((mc[1] >> (16 * k)) & 0xffffu) << 16);
                        const uint32_t hi = (uint32_t)((mc[2] >> (16 * k)) & 0xffffu) |
                                            (uint32_t)(((mc[3] >> (16 * k)) & 0xffffu) << 16);
                        const int r = rb * 16 + k * 4 + jj;
                        if (lane == r) {
                            m_lo = lo;
                            m_hi = hi;
                        }
                    }
                }
            if ((rows >> lane) & 1)
                w.mask[(int64_t)(q0 + lane) * w.n_grp + grp] =
                    ((uint64_t)m_hi << 32) | (uint64_t)m_lo;
        }
    }
}

// grid (n_q), 1024 threads: theta_lo = s_B - 2 Delta rounded down, s_B the
// B-th largest sampled MFMA score (-inf if the sample holds at most B).
__global__ __launch_bounds__(kSampNT) void k_sample_threshold(ScoreArgs a, PrefillWs w, int B) {
    __shared__ TopkSmem<kSampNT> sm;
    const int i = blockIdx.x, tid = threadIdx.x;
    constexpr int C = kPrefMaxBlocks / kSampleStride / kSampNT;  // 16
    RegKeys32<C, kSampNT> keys;
    keys.tid = tid;
    const float *row = w.sample + (int64_t)i * w.ld_s;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int x = c * kSampNT + tid;
        const float v = x < w.ld_s ? row[x] : -INFINITY;
        keys.k[c] = finite_f32(v) ? score_key(v) : 0u;
    }
    const Thresh th = topk_threshold<kSampNT>(keys, (uint32_t)B, sm);
    if (tid == 0) {
        float lo = -INFINITY;
        if (th.T != 0) {
            const double t = (double)key_value(th.T) - 2.0 * (double)w.delta[i];
            lo = (float)t;
            if ((double)lo > t) lo = nextafterf(lo, -INFINITY);
        }
        w.theta[i] = lo;
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
    uint64_t list[kPrefCandCap];  // candidate blocks, then their exact keys
};

// Candidate keys, exact, in registers (slot c holds list entry c*NT + tid);
// or, if the candidates overflowed the list, every causal block rescored on
// each pass.
struct PrefSource {
    uint64_t k[kPrefCandCap / kSelPNT];
    bool stream;
    int64_t limit;
    const uint16_t *keys;
    const float *q;
    template <typename F>
    __device__ __forceinline__ void operator()(F &&fn) const {
        if (!stream) {
#pragma unroll
            for (int c = 0; c < kPrefCandCap / kSelPNT; ++c)
                fn((uint32_t)(k[c] >> 32), (uint32_t)k[c]);
            return;
        }
        for (int64_t b = threadIdx.x; b < limit; b += kSelPNT) {
            const float sc = exact_score(keys + b * kDIdx, q);
            fn(finite_f32(sc) ? score_key(sc) : 0u, ~(uint32_t)b);
        }
    }
};

// grid (n_q), 1024 threads.
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
    const int n_words = (int)((limit + 31) / 32);
    for (int x = tid; x < n_words; x += kSelPNT) sm.bitmap[x] = 0;

    // candidate masks of this query's groups: count, scan, list
    constexpr int kMW = kPrefMaxBlocks / 64 / kSelPNT;  // mask words per thread
    const int n_g = (int)((limit + 63) / 64);
    uint64_t m[kMW];
    uint32_t local = 0;
#pragma unroll
    for (int c = 0; c < kMW; ++c) {
        const int g = tid * kMW + c;  // consecutive groups per thread
        m[c] = g < n_g ? w.mask[(int64_t)i * w.n_grp + g] : 0ull;
        local += __popcll(m[c]);
    }
    const int lane = tid & (kWave - 1), wave = tid >> 6;
    const uint32_t incl = wave_incl_scan_u32(local);
    if (lane == kWave - 1) sm.tk.red[wave] = incl;
    __syncthreads();
    uint32_t pos = incl - local, total = 0;
#pragma unroll
    for (int x = 0; x < kSelPNT / kWave; ++x) {
        if (x < wave) pos += sm.tk.red[x];
        total += sm.tk.red[x];
    }
    const bool stream = total > (uint32_t)kPrefCandCap;
    if (!stream) {
#pragma unroll
        for (int c = 0; c < kMW; ++c) {
            uint64_t bits = m[c];
            const int g = tid * kMW + c;
            while (bits) {
                const int bit = __builtin_ctzll(bits);
                bits &= bits - 1;
                sm.list[pos++] = (uint64_t)(g * 64 + bit);
            }
        }
    }
    __syncthreads();
    // exact keys in place, two candidates per thread at a time (their key
    // rows in flight together)
    if (!stream) {
        for (int x = tid; x < (int)total; x += 2 * kSelPNT) {
            const int x2 = x + kSelPNT;
            const int64_t b = (int64_t)sm.list[x];
            const int64_t b2 = x2 < (int)total ? (int64_t)sm.list[x2] : b;
            const float sc = exact_score(keys + b * kDIdx, sm.q);
            const float sc2 = exact_score(keys + b2 * kDIdx, sm.q);
            sm.list[x] = finite_f32(sc) ? block_key(sc, b) : 0ull;
            if (x2 < (int)total) sm.list[x2] = finite_f32(sc2) ? block_key(sc2, b2) : 0ull;
        }
    }
    __syncthreads();
    PrefSource src;
    src.stream = stream;
    src.limit = limit;
    src.keys = keys;
    src.q = sm.q;
#pragma unroll
    for (int c = 0; c < kPrefCandCap / kSelPNT; ++c) {
        const int x = c * kSelPNT + tid;
        src.k[c] = (!stream && x < (int)total) ? sm.list[x] : 0ull;
    }
    const Thresh th = topk_threshold<kSelPNT>(src, (uint32_t)B, sm.tk);
    src([&](uint32_t k, uint32_t u) {
        if (th.keep(k, u)) {
            const uint32_t bb = ~u;
            atomicOr(&sm.bitmap[bb >> 5], 1u << (bb & 31));
        }
    });
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
    d.n_sgrp = (d.n_grp + kSampleStride - 1) / kSampleStride;
    d.n_sgrp = (d.n_sgrp + 3) / 4 * 4;
    d.ld_s = (int64_t)d.n_sgrp * 64;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += (bytes + 255) / 256 * 256;
        return base ? base + at : nullptr;
    };
    d.mask = reinterpret_cast<uint64_t *>(take((size_t)n_q * d.n_grp * 8));
    d.sample = reinterpret_cast<float *>(take((size_t)n_q * d.ld_s * 4));
    d.qr = reinterpret_cast<uint16_t *>(take((size_t)n_q * kDIdx * 2));
    d.delta = reinterpret_cast<float *>(take((size_t)n_q * 4));
    d.theta = reinterpret_cast<float *>(take((size_t)n_q * 4));
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
    // group tiles padded to whole rounds of the 8 XCDs (k_prefill_tiles maps ids)
    auto tiles = [&](int n_gt) { return (n_gt + 7) / 8 * 8 * qt; };
    hipLaunchKernelGGL(k_prefill_tiles<kSample>, dim3(tiles(w.n_sgrp / 4)), dim3(256), 0, st, a,
                       w, w.n_sgrp / 4, qt);
    hipLaunchKernelGGL(k_sample_threshold, dim3(a.n_q), dim3(kSampNT), 0, st, a, w,
                       top_k / a.r);
    hipLaunchKernelGGL(k_prefill_tiles<kFilter>, dim3(tiles(w.n_grp / 4)), dim3(256), 0, st, a, w,
                       w.n_grp / 4, qt);
    hipLaunchKernelGGL(k_select_prefill, dim3(a.n_q), dim3(kSelPNT), 0, st, a, w, top_k,
                       sel_blocks, sel_cells, n_sel);
    return hipGetLastError();
}

}  // namespace qsa
