// score.hip -- indexer scoring of every causal block against each query
// (llama.cpp issue #28734, fix summary, "lever3": fully-future blocks get -inf
// and the incomplete tail block is not scored; the README of
// llama.cpp-multigpu, section 5, keeps that causal bias on the device).
//
// Decode (fp32).  The pooled keys are stored as 64-block tiles with the 64
// blocks of each 4-dim quad side by side, so lane l of a wavefront owns block
// 64*tile + l and reads its 128 dims with 32 fully coalesced 1 KiB loads; the
// whole 128-term dot product then runs in-lane in the fixed order T with no
// cross-lane traffic.  The kernel is a pure HBM stream: 512 bytes of key per
// block, 4 bytes of score out.
//
// Prefill (bf16).  The same contraction for many queries is a dense
// [queries x 128] x [128 x blocks] product, done on the matrix cores with
// v_mfma_f32_16x16x32_bf16 from bf16 copies of the roped queries and keys.
#include "cand_select.h"
#include "mfma_tile.h"

namespace qsa {

namespace {

// ---------------------------------------------------------------------------
// fp32 decode scoring
// ---------------------------------------------------------------------------

// Score of this lane's block b = b0 + lane (wave-uniform tile start b0) for
// one query, in order T; -inf if b >= nc.  qr4 must hold the roped query.
__device__ __forceinline__ float tile_score(const float4 (&k)[kQuads], const float4 *qr4,
                                            int64_t b, int64_t nc) {
    float sc = -INFINITY;
    if (b < nc) {
        // T: level 64 pairs quad q with q+16, level 32 q with q+8, ... level 4
        // quad 0 with quad 1, then components (0,2), (1,3), then the pair.
        float4 acc[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const float4 qa = qr4[q], qb = qr4[q + 16];
            const float4 ka = k[q], kb = k[q + 16];
            float4 pa, pb;
            pa.x = qa.x * ka.x; pa.y = qa.y * ka.y; pa.z = qa.z * ka.z; pa.w = qa.w * ka.w;
            pb.x = qb.x * kb.x; pb.y = qb.y * kb.y; pb.z = qb.z * kb.z; pb.w = qb.w * kb.w;
            acc[q].x = pa.x + pb.x; acc[q].y = pa.y + pb.y;
            acc[q].z = pa.z + pb.z; acc[q].w = pa.w + pb.w;
        }
#pragma unroll
        for (int h = 8; h >= 1; h >>= 1) {
#pragma unroll
            for (int q = 0; q < h; ++q) {
                acc[q].x = acc[q].x + acc[q + h].x;
                acc[q].y = acc[q].y + acc[q + h].y;
                acc[q].z = acc[q].z + acc[q + h].z;
                acc[q].w = acc[q].w + acc[q + h].w;
            }
        }
        const float x0 = acc[0].x + acc[0].z;
        const float x1 = acc[0].y + acc[0].w;
        sc = x0 + x1;
    }
    return sc;
}

// Load the 64-block tile starting at b0 (if any block of it is scored) and
// rope the query into qr4 (wave 0), then synchronise the workgroup.
__device__ __forceinline__ void load_tile_and_query(const ScoreArgs &a, int i, int s, int64_t p,
                                                    int64_t nc, int64_t wg_b0, int64_t b0,
                                                    float4 (&k)[kQuads], float4 *qr4) {
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t cap_blocks = a.g.cap_cells / a.r;
    // issue the key loads first; the query rotation below overlaps them
    if (b0 < nc) {
        const float4 *src = reinterpret_cast<const float4 *>(
                                a.pooled + ((int64_t)s * (cap_blocks / kTile) + b0 / kTile) *
                                               kTileFloats) +
                            lane;
#pragma unroll
        for (int q = 0; q < kQuads; ++q) k[q] = src[q * kTile];
    }
    if (wg_b0 < nc && wave == 0) {
        float lo, hi;
        rope_query_pair(a.q_idx + (int64_t)i * kDIdx, lane, p, a.rope, lo, hi);
        float *qr = reinterpret_cast<float *>(qr4);
        qr[lane] = lo;
        qr[lane + 64] = hi;
    }
    __syncthreads();
}

// grid (ceil(nb_max/256), n_q); 4 wavefronts, one 64-block tile each.
__global__ __launch_bounds__(256) void k_score_f32(ScoreArgs a) {
    __shared__ float4 qr4[kQuads];
    const int i = blockIdx.y;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & (kWave - 1);
    int s;
    int64_t p;
    bool valid;
    const int64_t nc = query_blocks(a.q_seq, a.q_pos, i, a.g.n_seq, a.g.cap_cells,
                                    a.g.n_cells, a.r, s, p, valid);
    const int64_t wg_b0 = (int64_t)blockIdx.x * 256;
    const int64_t b0 = wg_b0 + wave * kTile;
    const int64_t b = b0 + lane;
    float4 k[kQuads];
    load_tile_and_query(a, i, s, p, nc, wg_b0, b0, k, qr4);
    const float sc = tile_score(k, qr4, b, nc);
    if (b < a.nb_max) a.scores[(int64_t)i * a.ld + b] = sc;
}

// ---------------------------------------------------------------------------
// decode indexer step: update + scoring + candidates, then exact selection
// ---------------------------------------------------------------------------

// A 16-byte load of data read exactly once (the pooled-key stream): marked
// non-temporal so it does not displace what the L2 holds for the next
// kernels -- the candidates, and the selection kernel's instructions, which
// would otherwise come back from memory one cache line at a time.
__device__ __forceinline__ float4 load_stream(const float4 *p) {
    typedef float v4f __attribute__((ext_vector_type(4)));
    const v4f v = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}

constexpr int kSelNT = 1024;  // selection workgroup

// Descending bitonic sort of one 64-bit key per lane across a wavefront.
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t key) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int kk = 2; kk <= kWave; kk <<= 1) {
#pragma unroll
        for (int j = kk >> 1; j > 0; j >>= 1) {
            const uint64_t o = shfl_xor64(key, j);  // j is a constant once unrolled
            const bool take_max = ((lane & j) == 0) == ((lane & kk) == 0);
            key = take_max ? (o > key ? o : key) : (o < key ? o : key);
        }
    }
    return key;
}

// One compare-exchange of a bitonic network (stage KK, partner lane ^ J).
template <int KK, int J>
__device__ __forceinline__ void bitonic_step(uint64_t &k, int lane) {
    const uint64_t o = xor_lane64<J>(k);
    const bool take_max = ((lane & J) == 0) == ((lane & KK) == 0);
    k = take_max ? (o > k ? o : k) : (o < k ? o : k);
}

// Lanes [0, n) (n = 4, 6, 8 or 16, wave-uniform) hold keys (score key <<
// 32 | ~block); on return they hold the same keys by descending ~block,
// that is ascending block, with zero keys last.  A bitonic network over
// groups of 4, 8 or 16 lanes (n = 6: 8, lanes 6 and 7 emptied first) on the
// swapped halves; lanes from n on end up with other keys of their own
// groups.
__device__ __forceinline__ uint64_t group_sort_by_block(uint64_t key, int n) {
    const int lane = threadIdx.x & (kWave - 1);
    if (n == 6 && (lane & 7) >= 6) key = 0ull;
    uint64_t k = (key << 32) | (key >> 32);
    bitonic_step<2, 1>(k, lane);
    bitonic_step<4, 2>(k, lane);
    bitonic_step<4, 1>(k, lane);
    if (n >= 6) {
        bitonic_step<8, 4>(k, lane);
        bitonic_step<8, 2>(k, lane);
        bitonic_step<8, 1>(k, lane);
    }
    if (n >= 16) {
        bitonic_step<16, 8>(k, lane);
        bitonic_step<16, 4>(k, lane);
        bitonic_step<16, 2>(k, lane);
        bitonic_step<16, 1>(k, lane);
    }
    return (k << 32) | (k >> 32);
}

// Scoring workgroups: one per query and 64-block group, the groups padded
// to a multiple of 8 (one round per XCD).
__host__ __device__ inline int score_wgs(int n_grp, int n_q) { return (n_grp + 7) / 8 * 8 * n_q; }

// 1-D grid: score_wgs(4*n_wg, n_q) scoring workgroups (one per query and
// 64-block group, and the padding), then ceil(n_dirty/4) update workgroups
// (one wavefront per dirty entry).
//
// Scoring: lane l of wavefront w owns block 64*g + l and the quads (4 dims)
// q = w, w + 4, ..., w + 28 of it, so each load is 1 KiB contiguous and a
// lane makes 8 of them (many workgroups, few loads each: the shape that
// streams fastest from HBM).  Order T in this split: levels 64, 32 and 16
// pair quads q, q + 16, q + 8 and q + 4, all within the wavefront; the
// wavefront's quad-w partial then meets the others in LDS for level 8 (quad
// w with w + 2), level 4 (0 with 1) and the two levels inside the quad.
__global__ __launch_bounds__(256) void k_score_cand(DecodeIdxArgs f) {
    QSA_STAMP(0);
    __shared__ float4 qr4[kQuads];
    __shared__ float4 patch[kQuads];
    __shared__ float4 part[4][kTile];  // quad-w partial of each block
    __shared__ int s_hit[256];
    __shared__ int s_n_hit;
    const ScoreArgs &a = f.s;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & (kWave - 1);
    const int64_t cap_blocks = a.g.cap_cells / a.r;
    const int n_grp = f.n_wg * 4;
    const int n_score_wg = score_wgs(n_grp, a.n_q);

    if ((int)blockIdx.x >= n_score_wg) {  // ---- update role ----
        const int e = ((int)blockIdx.x - n_score_wg) * 4 + wave;
        if (e >= f.n_dirty) return;
        const int s = f.dirty[2 * e], b = f.dirty[2 * e + 1];
        if (s < 0 || s >= a.g.n_seq || b < 0 || b >= cap_blocks) return;
        int64_t n = a.g.n_cells[s];
        if (n > a.g.cap_cells) n = a.g.cap_cells;
        if ((int64_t)b * a.r >= n) return;
        float lo, hi;
        pooled_key_lane(f.kidx, a.g, s, b, n, a.r, f.eps, f.gamma, a.rope, lane, lo, hi);
        store_pooled_lane(f.pooled_w, f.pooled_bf16, cap_blocks, s, b, lane, lo, hi);
        return;
    }

    // ---- scoring role: query i, blocks [64*gg, 64*gg + 64) ----
    // Loads are issued before anything waits: the query (no dependence),
    // the key tile (needs only the sequence), then the dirty list; the
    // causal count comes from scalar loads, which wait on their own counter.
    // Ids are dealt to the 8 XCDs round robin (id mod 8): the k-th id of XCD x
    // takes group position 8*(k / n_q) + x for query k % n_q, so the queries'
    // workgroups of one key group run back to back on one XCD, and several
    // tokens of one sequence read that tile from HBM once (their L2 serves the
    // rest).  Positions count groups in reverse: the tail group, which usually
    // holds the dirty block and recomputes it, is dispatched first.
    const int xcd = (int)(blockIdx.x & 7), kth = (int)(blockIdx.x >> 3);
    const int i = kth % a.n_q, gpos = 8 * (kth / a.n_q) + xcd;
    if (gpos >= n_grp) return;  // padding of the last round of 8 groups
    const int gg = n_grp - 1 - gpos;
    const int64_t b0 = (int64_t)gg * kTile;
    const int64_t b = b0 + lane;
    const float qxl = a.q_idx[(int64_t)i * kDIdx + lane];
    const float qxh = a.q_idx[(int64_t)i * kDIdx + lane + 64];
    const double omega = a.rope.omega[lane];
    const int s_in = a.q_seq[i];
    // (issued unconditionally, from tile 0 if the tile does not exist, so the
    // wait counts below stay exact)
    const bool tile_ok = s_in >= 0 && s_in < a.g.n_seq && b0 < cap_blocks;
    const float4 *src = reinterpret_cast<const float4 *>(
                            a.pooled + (tile_ok ? ((int64_t)s_in * (cap_blocks / kTile) + gg) *
                                                      kTileFloats
                                                : 0)) + lane;
    float4 k[8];  // quads wave + 4m of block b
#pragma unroll
    for (int m = 0; m < 8; ++m) k[m] = load_stream(src + (wave + 4 * m) * kTile);
    // (unconditional, clamped loads: a load under a lane condition would be
    // waited for, with the keys, right after it)
    const int32_t *dl = f.n_dirty > 0 ? f.dirty : a.q_seq;
    const int nd2 = f.n_dirty > 0 ? 2 * f.n_dirty : 1;
    int my_ds = dl[min(2 * tid, nd2 - 1)], my_db = dl[min(2 * tid + 1, nd2 - 1)];
    if (tid >= f.n_dirty) my_ds = -1;
    int s;
    int64_t p;
    bool valid;
    const int64_t nc = query_blocks(a.q_seq, a.q_pos, i, a.g.n_seq, a.g.cap_cells,
                                    a.g.n_cells, a.r, s, p, valid);
    const int64_t limit = nc < a.nb_max ? nc : a.nb_max;
    const bool live = b0 < nc;  // implies a valid sequence and b0 < cap_blocks
    if (tid == 0) s_n_hit = 0;
    if (live && wave == 0) {
        float lo, hi;
        rope_pair_omega(qxl, qxh, omega, p, lo, hi);
        float *qr = reinterpret_cast<float *>(qr4);
        qr[lane] = lo;
        qr[lane + 64] = hi;
    }
    __syncthreads();
    // dirty entries among this group's scored blocks (lists longer than 256
    // are covered by the loop below reading the rest directly)
    if (my_ds == s && my_db >= b0 && my_db < b0 + kTile && my_db < nc)
        s_hit[atomicAdd(&s_n_hit, 1)] = my_db;
    __syncthreads();
    const int n_hit = s_n_hit;

    // a dirty block scored here may not be written yet: recompute it in place
    if (live && (n_hit > 0 || f.n_dirty > 256)) {
        int64_t n = a.g.n_cells[s];
        if (n > a.g.cap_cells) n = a.g.cap_cells;
        const int n_iter = f.n_dirty > 256 ? n_hit + (f.n_dirty - 256) : n_hit;
        for (int e = 0; e < n_iter; ++e) {  // workgroup-uniform loop
            int64_t db;
            if (e < n_hit) {
                db = s_hit[e];
            } else {
                const int de = 256 + (e - n_hit);
                if (f.dirty[2 * de] != s) continue;
                db = f.dirty[2 * de + 1];
                if (db < b0 || db >= b0 + kTile || db >= nc) continue;
            }
            if (wave == 0) {
                float lo, hi;
                pooled_key_lane(f.kidx, a.g, s, db, n, a.r, f.eps, f.gamma, a.rope,
                                lane, lo, hi);
                float *pf = reinterpret_cast<float *>(patch);
                pf[lane] = lo;
                pf[lane + 64] = hi;
            }
            __syncthreads();
            if (b == db) {
#pragma unroll
                for (int m = 0; m < 8; ++m) k[m] = patch[wave + 4 * m];
            }
            __syncthreads();
        }
    }

    // levels 64, 32, 16 within the wavefront
    if (live) {
        float4 v[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const float4 qq = qr4[wave + 4 * m];
            v[m].x = qq.x * k[m].x;
            v[m].y = qq.y * k[m].y;
            v[m].z = qq.z * k[m].z;
            v[m].w = qq.w * k[m].w;
        }
        // slot m is quad wave + 4m: level 64 pairs m with m + 4, 32 m with
        // m + 2, 16 m with m + 1
#pragma unroll
        for (int h = 4; h >= 1; h >>= 1)
#pragma unroll
            for (int m = 0; m < h; ++m) {
                v[m].x = v[m].x + v[m + h].x;
                v[m].y = v[m].y + v[m + h].y;
                v[m].z = v[m].z + v[m + h].z;
                v[m].w = v[m].w + v[m + h].w;
            }
        part[wave][lane] = v[0];
    }
    __syncthreads();
    QSA_STAMP(2);  // (slot 1 is the selection engine's)
    if (wave != 0) return;
    float sc = -INFINITY;
    if (live && b < nc) {
        const float4 p0 = part[0][lane], p1 = part[1][lane];
        const float4 p2 = part[2][lane], p3 = part[3][lane];
        float4 u0, u1;  // level 8: quad 0 with 2, quad 1 with 3
        u0.x = p0.x + p2.x; u0.y = p0.y + p2.y; u0.z = p0.z + p2.z; u0.w = p0.w + p2.w;
        u1.x = p1.x + p3.x; u1.y = p1.y + p3.y; u1.z = p1.z + p3.z; u1.w = p1.w + p3.w;
        float4 t;  // level 4
        t.x = u0.x + u1.x; t.y = u0.y + u1.y; t.z = u0.z + u1.z; t.w = u0.w + u1.w;
        const float x0 = t.x + t.z, x1 = t.y + t.w;  // level 2
        sc = x0 + x1;                                 // level 1
    }
    float *srow = a.scores + (int64_t)i * a.ld;
    if (b < a.nb_max) srow[b] = sc;
    uint64_t key = (b < limit && finite_f32(sc)) ? block_key(sc, b) : 0ull;
    key = wave_sort_desc(key);
    const int64_t grp = (int64_t)i * n_grp + gg;
    if (lane == f.n_cand) f.drop[grp] = key;
    // the kept keys in ascending block order (zeros last), so that the
    // candidates of all groups, read in order, ascend by block
    key = group_sort_by_block(key, f.n_cand);
    if (lane < f.n_cand) f.cand[grp * f.n_cand + lane] = key;
    QSA_STAMP(3);
}

// grid (n_q), 1024 threads: the exact selection from the candidates, then
// the ascending emission of blocks and cells.
template <int MAXB>
__global__ __launch_bounds__(kSelNT) void k_select_cand(DecodeIdxArgs f) {
    __shared__ CandSelSmem<kSelNT, MAXB> sm;
    const ScoreArgs &a = f.s;
    const int i = blockIdx.x;
    // the query's sequence and position, then the candidates, then the
    // sequence's cell count (the selection does not wait for it)
    QueryFields qf{0, 0, 0, a.g.n_seq, a.g.cap_cells, a.r, a.nb_max};
    const int s_first = a.q_seq[i];
    const int64_t p_first = a.q_pos[i];
    CandKeys<kSelNT, MAXB, kCandWide> ck;
    uint64_t drop[MAXB / kGroup / kSelNT];
    load_candidates(f, i, ck, drop);
    qf.s = s_first;
    qf.p = p_first;
    qf.ncell = a.g.n_cells[min(max(s_first, 0), a.g.n_seq - 1)];
    const int B = f.top_k / a.r;
    Thresh th;
    const bool fast = select_candidates<kSelNT, MAXB, kCandWide, true>(f, i, qf, B, sm, ck, drop, th);
    bool valid;
    const int64_t nc = qf.blocks(valid);
    const int64_t limit = nc < a.nb_max ? nc : a.nb_max;
    const int64_t p = qf.p;
    const int n_words = (int)((limit + 31) / 32);
    const int tail = valid ? (int)(p + 1 - nc * a.r) : 0;
    const int ld_cells = f.top_k + a.r - 1;
    int32_t *sel_blocks = f.sel_blocks + (int64_t)i * B;
    int32_t *sel_cells = f.sel_cells + (int64_t)i * ld_cells;
    if (!fast) {  // a group was re-admitted or the row streamed: the bitmap holds the set
        emit_from_bitmap<kSelNT>(sm.bitmap, n_words, B, a.r, nc, tail, sel_blocks, sel_cells,
                                 ld_cells, f.n_sel + i, sm.tk);
        return;
    }
    // The kept set is the base candidates th keeps, and they ascend by block
    // in the order (wavefront, slot, lane): a kept one's rank is the kept
    // count of the earlier wavefronts, then of its wavefront's earlier slots,
    // then of its slot's lower lanes (ballots) -- no bitmap to mark or scan.
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
    uint64_t bal[decltype(ck)::kBase];  // each slot's ballot, kept for the ranks below
    uint32_t in_wave = 0;
#pragma unroll
    for (int x = 0; x < decltype(ck)::kBase; ++x) {
        bal[x] = x < ck.nb ? __ballot(th.keep((uint32_t)(ck.k[x] >> 32), (uint32_t)ck.k[x]))
                           : 0ull;
        in_wave += __popcll(bal[x]);
    }
    if (lane == 0) sm.tk.red[wave] = in_wave;
    __syncthreads();
    uint32_t before, total;
    waves_prefix<kSelNT / kWave>(sm.tk.red, wave, before, total);
    const int n_keep = (int)(total < (uint32_t)B ? total : (uint32_t)B);
    const uint64_t below = (1ull << lane) - 1ull;
    uint32_t k0 = before;  // rank of this wavefront's next kept slot
#pragma unroll
    for (int x = 0; x < decltype(ck)::kBase; ++x) {
        const bool kp = (bal[x] >> lane) & 1ull;
        const int k = (int)(k0 + __popcll(bal[x] & below));
        if (kp && k < n_keep) {
            const int32_t b = key_block(ck.k[x]);
            sel_blocks[k] = b;
            for (int c = 0; c < a.r; ++c) sel_cells[k * a.r + c] = b * a.r + c;
        }
        k0 += __popcll(bal[x]);
    }
    if (threadIdx.x == 0) f.n_sel[i] = n_keep * a.r + tail;
    for (int j = n_keep + (int)threadIdx.x; j < B; j += kSelNT) sel_blocks[j] = -1;
    const int n_full = n_keep * a.r;
    for (int j = n_full + (int)threadIdx.x; j < ld_cells; j += kSelNT)
        sel_cells[j] = (j < n_full + tail) ? (int32_t)(nc * a.r + (j - n_full)) : -1;
}

// ---------------------------------------------------------------------------
// bf16 prefill scoring on the matrix cores
// ---------------------------------------------------------------------------

// One wavefront per query: roped query rounded to bf16 (zeros if invalid).
__global__ __launch_bounds__(256) void k_rope_queries_bf16(ScoreArgs a, uint16_t *qr_bf16) {
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
    qr_bf16[(int64_t)i * kDIdx + lane] = lo16;
    qr_bf16[(int64_t)i * kDIdx + lane + 64] = hi16;
}

// grid (ceil(nb_max/256), ceil(n_q/64)); workgroup tile 64 queries x 256
// blocks, each wavefront 64 queries x 64 blocks as 4x4 16x16 MFMA tiles.
// Queries of one tile may belong to different sequences: the tile is swept
// once per distinct sequence, storing only that sequence's rows.
__global__ __launch_bounds__(256) void k_score_bf16(ScoreArgs a, const uint16_t *qr_bf16) {
    __shared__ int s_seq[64];
    __shared__ int64_t s_nc[64];
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & (kWave - 1);
    const int q0 = blockIdx.y * 64;
    const int64_t bw0 = (int64_t)blockIdx.x * 256 + wave * 64;
    const int64_t cap_blocks = a.g.cap_cells / a.r;
    if (threadIdx.x < 64) {
        const int qi = q0 + threadIdx.x;
        int s = -1;
        int64_t nc = 0;
        if (qi < a.n_q) {
            int64_t p;
            bool valid;
            nc = query_blocks(a.q_seq, a.q_pos, qi, a.g.n_seq, a.g.cap_cells, a.g.n_cells, a.r,
                              s, p, valid);
            if (!valid) s = -1;
        }
        s_seq[threadIdx.x] = qi < a.n_q ? s : -2;
        s_nc[threadIdx.x] = nc;
    }
    __syncthreads();

    const int mrow = lane & 15;        // A row / B column within a 16-tile
    const int kseg = (lane >> 4) * 8;  // 8 consecutive k per lane
    bf16x8_t A[4][4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
        const int qi = q0 + rb * 16 + mrow;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (qi < a.n_q)
                A[rb][ks] = load_bf16x8(qr_bf16 + (int64_t)qi * kDIdx + ks * 32 + kseg);
            else
                A[rb][ks] = bf16x8_t{};
        }
    }

    // rows with an invalid query: -inf over this wavefront's columns
    for (int r = 0; r < 64; ++r) {
        if (s_seq[r] != -1) continue;
        const int64_t b = bw0 + lane;
        if (b < a.nb_max) a.scores[(int64_t)(q0 + r) * a.ld + b] = -INFINITY;
    }

    uint64_t done = 0;  // rows handled (wave-uniform)
    for (int r = 0; r < 64; ++r)
        if (s_seq[r] < 0) done |= 1ull << r;
    while (done != ~0ull) {
        const int r0 = __builtin_ctzll(~done);
        const int sq = s_seq[r0];
        uint64_t rows = 0;
        int64_t ncmax = 0;
        for (int r = r0; r < 64; ++r)
            if (s_seq[r] == sq) {
                rows |= 1ull << r;
                ncmax = s_nc[r] > ncmax ? s_nc[r] : ncmax;
            }
        done |= rows;
        const uint16_t *keys = a.pooled_bf16 + (int64_t)sq * cap_blocks * kDIdx;
#pragma unroll 1
        for (int cb = 0; cb < 4; ++cb) {
            const int64_t bc0 = bw0 + cb * 16;
            if (bc0 >= a.nb_max) break;
            const int64_t nb = bc0 + mrow;  // this lane's B column (block)
            const bool live = bc0 < ncmax;  // any row sees any block here
            bf16x8_t B[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                if (live && nb < cap_blocks)
                    B[ks] = load_bf16x8(keys + nb * kDIdx + ks * 32 + kseg);
                else
                    B[ks] = bf16x8_t{};
            }
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
                if (live) {
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[rb][ks], B[ks], acc, 0, 0,
                                                                      0);
                }
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int r = rb * 16 + (lane >> 4) * 4 + jj;
                    if (!((rows >> r) & 1)) continue;
                    if (nb >= a.nb_max) continue;
                    const float v = nb < s_nc[r] ? acc[jj] : -INFINITY;
                    a.scores[(int64_t)(q0 + r) * a.ld + nb] = v;
                }
            }
        }
    }
}

}  // namespace

QSA_STAMP_READER(score)

size_t fused_select_ws_bytes(int n_q, int nb_max) { return cand_ws_bytes(n_q, nb_max); }

hipError_t launch_decode_candidates(DecodeIdxArgs f, void *ws, hipStream_t st) {
    bind_candidates(f, ws);
    const int grid = score_wgs(f.n_wg * 4, f.s.n_q) + (f.n_dirty + 3) / 4;
    if (grid > 0) hipLaunchKernelGGL(k_score_cand, dim3(grid), dim3(256), 0, st, f);
    return hipGetLastError();
}

hipError_t launch_decode_select(DecodeIdxArgs f, void *ws, hipStream_t st) {
    bind_candidates(f, ws);
    if (f.s.n_q <= 0) return hipSuccess;
    // the smaller instance (half the bitmap and register slots) up to 65536 blocks
    if (f.s.nb_max <= kSelAttnMaxBlocks)
        hipLaunchKernelGGL(k_select_cand<kSelAttnMaxBlocks>, dim3(f.s.n_q), dim3(kSelNT), 0, st, f);
    else
        hipLaunchKernelGGL(k_select_cand<kFusedMaxBlocks>, dim3(f.s.n_q), dim3(kSelNT), 0, st, f);
    return hipGetLastError();
}

hipError_t launch_score_f32(const ScoreArgs &a, hipStream_t st) {
    if (a.n_q <= 0 || a.nb_max <= 0) return hipSuccess;
    dim3 grid((a.nb_max + 255) / 256, a.n_q);
    hipLaunchKernelGGL(k_score_f32, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

// ws must hold n_q * 128 bf16 values (the roped queries).
hipError_t launch_score_bf16_ws(const ScoreArgs &a, uint16_t *qr_bf16, hipStream_t st) {
    if (a.n_q <= 0 || a.nb_max <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_rope_queries_bf16, dim3((a.n_q + 3) / 4), dim3(256), 0, st, a,
                       qr_bf16);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid((a.nb_max + 255) / 256, (a.n_q + 63) / 64);
    hipLaunchKernelGGL(k_score_bf16, grid, dim3(256), 0, st, a,
                       static_cast<const uint16_t *>(qr_bf16));
    return hipGetLastError();
}

}  // namespace qsa
