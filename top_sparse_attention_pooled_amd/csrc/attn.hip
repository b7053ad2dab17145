// attn.hip -- attention over the selected cells only (llama.cpp issue #28734,
// fix summary, "lever1": the top-k set, not the whole cache, is what attention
// visits), with q8_0 rows dequantised inside the gather (discussion #30071:
// the compact-gather path that keeps a quantised cache on the sparse path,
// where converting the whole cache first would cost O(n_kv)).
//
// Work unit: one workgroup = one (query, run of cells, pair of query heads
// that share a KV head).  Its 256 threads are 8 groups of 32; lane j of a
// group owns dims 8j .. 8j+7 of both heads.  A decode workgroup takes one
// 32-cell chunk (a 2051-cell set and 16 query heads make 65 x 8 = 520
// workgroups, two wavefronts per SIMD) and issues every index, K and V load
// before it uses any; the workgroups of one chunk run on one XCD, so its K/V
// rows cross HBM once.  Per chunk: the groups score their cells (dot products
// reduced over 32 lanes with a transposing butterfly), the chunk's softmax
// statistics come from one half-wavefront per head, and the groups
// accumulate P*V; across chunks the running (max, sum, output) are rescaled
// once per chunk.  Decode splits a query's cells over many workgroups and
// merges their partial states in a second kernel; prefill gives each
// workgroup all cells of its query.
//
// q8_0 rows: 8 blocks of (binary16 scale, 32 int8) = 272 bytes.  A lane's
// 8 int8 start at byte 34*(j/4) + 2 + 8*(j%4), which is 2 mod 4 for even
// blocks: they are read as aligned dwords and realigned with a funnel shift.
#include "cand_select.h"
#include "kv_rows.h"
#include "qsa_internal.h"
#include "wave_ops.h"

namespace qsa {

namespace {

constexpr int kChunk = 32;   // cells per chunk; a decode workgroup takes one chunk
constexpr int kGroups = 8;   // 32-lane groups per workgroup
constexpr int kCPG = kChunk / kGroups;  // cells per group per chunk

// Sum v[0..G) over the 32 lanes of a group.  On return lane j holds the full
// sum for head head_of_lane<G>(j) in v[0]: each halving step exchanges half
// of the remaining values, so 8 heads cost 4+2+1+1+1 shuffles, not 8*5.
template <int G, int O>
__device__ __forceinline__ void group_reduce_step(float (&v)[G], int &n) {
    if (n > 1) {
        const int half = n >> 1;
        const bool upper = (threadIdx.x & O) != 0;
#pragma unroll
        for (int h = 0; h < G / 2; ++h) {
            if (h < half) {
                const float keep = upper ? v[h + half] : v[h];
                const float send = upper ? v[h] : v[h + half];
                v[h] = keep + xor_lane_f<O>(send);
            }
        }
        n = half;
    } else {
        v[0] = v[0] + xor_lane_f<O>(v[0]);
    }
}

template <int G>
__device__ __forceinline__ void group_reduce(float (&v)[G]) {
    int n = G;
    group_reduce_step<G, 16>(v, n);
    group_reduce_step<G, 8>(v, n);
    group_reduce_step<G, 4>(v, n);
    group_reduce_step<G, 2>(v, n);
    group_reduce_step<G, 1>(v, n);
}

// Max / sum over the 32 lanes of a half-wavefront.
__device__ __forceinline__ float half_max(float v) {
    v = fmaxf(v, xor_lane_f<16>(v));
    v = fmaxf(v, xor_lane_f<8>(v));
    v = fmaxf(v, xor_lane_f<4>(v));
    v = fmaxf(v, xor_lane_f<2>(v));
    v = fmaxf(v, xor_lane_f<1>(v));
    return v;
}
__device__ __forceinline__ float half_sum(float v) {
    v += xor_lane_f<16>(v);
    v += xor_lane_f<8>(v);
    v += xor_lane_f<4>(v);
    v += xor_lane_f<2>(v);
    v += xor_lane_f<1>(v);
    return v;
}

template <int G>
__device__ __forceinline__ int head_of_lane(int j) {
    // the halving steps fix head bits from the top: lane bit 4 picks the upper
    // half of the heads first, then bit 3, ...
    int h = 0, n = G;
    for (int o = 16; o >= 1 && n > 1; o >>= 1) {
        n >>= 1;
        if (j & o) h += n;
    }
    return h;
}

template <int G>
__device__ __forceinline__ bool lane_reports(int j) {
    // lanes that agree on the head bits hold equal copies; the lowest reports
    int bits = 0, n = G;
    for (int o = 16; o >= 1 && n > 1; o >>= 1) {
        n >>= 1;
        bits |= o;
    }
    return (j & ~bits & 31) == 0;
}

template <int G>
struct AttnSmem {
    float p[G][kChunk];
    float red[kGroups][G * kHeadDim];
    float stat[G][2];  // chunk max, chunk sum
};

// Workgroup -> unit (query i, run of chunks, group hg of G heads), head group
// fastest; the G heads share one KV head.  The hardware deals workgroup ids
// to the 8 XCDs round-robin (id mod 8), and each XCD has its own L2, so the
// 1-D grid gives XCD x the contiguous unit range [x*per, (x+1)*per): the head
// groups of one (query, run), which read the same K/V rows, then share an L2
// and the rows come from HBM once.  Returns false for the padding ids.
__device__ __forceinline__ bool unit_of(int n_q, int n_runs, int n_hg, int &i, int &run,
                                        int &hg) {
    const int total = n_q * n_runs * n_hg;
    const int per = (total + 7) >> 3;  // units per XCD; the grid is 8*per
    const int unit = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    if (unit >= total) return false;
    hg = unit % n_hg;
    run = (unit / n_hg) % n_runs;
    i = unit / (n_hg * n_runs);
    return true;
}

// Lane j's slice (dims 8j .. 8j+7) of query i's heads h0 .. h0+G-1.
template <int G>
__device__ __forceinline__ void load_q(const AttnArgs &a, int i, int h0, int j,
                                       float (&qv)[G][8]) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float4 *qp = reinterpret_cast<const float4 *>(
            a.q + ((int64_t)i * a.n_head + h0 + h) * kHeadDim + 8 * j);
        const float4 u = qp[0], v = qp[1];
        qv[h][0] = u.x; qv[h][1] = u.y; qv[h][2] = u.z; qv[h][3] = u.w;
        qv[h][4] = v.x; qv[h][5] = v.y; qv[h][6] = v.z; qv[h][7] = v.w;
    }
}

// Attention of query i (sequence s), heads h0.. (KV head g), over positions
// [c_begin, c_end) of its cell list, one 32-cell chunk at a time, by the 256
// threads of one part (threadIdx.x / 256) of the workgroup; every part
// of the workgroup calls it with the same c_begin, c_end (it has workgroup
// barriers).  cell[] holds this thread's cells of the first chunk (positions
// c_begin + grp*4 + u); later chunks read theirs from `cells` (global).
// active: write results (false for an idle part).  direct: write the
// normalised output; else the partial state (o[G][256], m[G], l[G]) to part.
template <int G, int KVT>
__device__ __forceinline__ void attend_chunks(const AttnArgs &a, int i, int s, int g, int h0,
                                              int c_begin, int c_end, int (&cell)[kCPG],
                                              const int32_t *cells, const float (&qv)[G][8],
                                              AttnSmem<G> &sm, float *part, bool direct,
                                              bool active) {
    const int tid = threadIdx.x & 255, grp = tid >> 5, j = tid & 31, wave = tid >> 6,
              lane = tid & 63;
    float m_run[G], l_run[G], o[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m_run[h] = -INFINITY;
        l_run[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
    }

    if (c_begin < c_end) {
        for (int c0 = c_begin; c0 < c_end; c0 += kChunk) {
            QSA_STAMP_LDS(12);
            const int c1 = min(c_end, c0 + kChunk);
            if (c0 != c_begin) {
#pragma unroll
                for (int u = 0; u < kCPG; ++u) {
                    const int cc = c0 + grp * kCPG + u;
                    cell[u] = cc < a.ld_cells ? cells[cc] : -1;
                }
            }
            // K/V rows and the present-cell count.  Every load is issued (a
            // cell outside 0 .. cap_cells-1 reads cell 0 and is not used):
            // a load under a lane condition is waited for right after it,
            // which would serialise the cells' round trips.
            RawRow<KVT> rk[kCPG], rv[kCPG];
#pragma unroll
            for (int u = 0; u < kCPG; ++u) {
                const bool in_cap = cell[u] >= 0 && cell[u] < a.g.cap_cells;
                const int64_t row = cell_row(a.g, s, in_cap ? cell[u] : 0) * a.n_head_kv + g;
                rk[u] = load_raw<KVT>(a.k, row, j);
                rv[u] = load_raw<KVT>(a.v, row, j);
            }
            int64_t n_present = a.g.n_cells[s];
            n_present = n_present < a.g.cap_cells ? n_present : a.g.cap_cells;
            // scores of this group's cells
#pragma unroll
            for (int u = 0; u < kCPG; ++u) {
                const int cc = c0 + grp * kCPG + u;
                const bool ok = cc < c1 && cell[u] >= 0 && cell[u] < n_present;
                float kf[8];
                if (ok) {
                    dequant<KVT>(rk[u], j, kf);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) kf[e] = 0.f;
                }
                float sv[G];
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    float acc = qv[h][0] * kf[0];
#pragma unroll
                    for (int e = 1; e < 8; ++e) acc = fmaf(qv[h][e], kf[e], acc);
                    sv[h] = acc;
                }
                group_reduce<G>(sv);
                if (cc < c1 && lane_reports<G>(j))
                    sm.p[head_of_lane<G>(j)][cc - c0] = ok ? sv[0] * a.scale : -INFINITY;
            }
            __syncthreads();
            QSA_STAMP_LDS(13);
            // chunk statistics: 32 lanes per head, two heads per wavefront
#pragma unroll
            for (int h = 0; h < G; ++h) {
                if (((h >> 1) & 3) != wave || ((h & 1) != (lane >> 5))) continue;
                const int c = lane & 31;
                const bool in = c0 + c < c1;
                const float x = in ? sm.p[h][c] : -INFINITY;
                const float mx = half_max(x);
                const float m_new = fmaxf(m_run[h], mx);  // m_run equal in every thread
                const float pe = (in && x != -INFINITY) ? __expf(x - m_new) : 0.f;
                const float sum = half_sum(pe);
                sm.p[h][c] = pe;
                if (c == 0) {
                    sm.stat[h][0] = m_new;
                    sm.stat[h][1] = sum;
                }
            }
            __syncthreads();
            // rescale the running state, then accumulate P*V
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float m_new = sm.stat[h][0];
                const float corr = m_run[h] == -INFINITY ? 0.f : __expf(m_run[h] - m_new);
                l_run[h] = l_run[h] * corr + sm.stat[h][1];
                m_run[h] = m_new;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[h][e] *= corr;
            }
#pragma unroll
            for (int u = 0; u < kCPG; ++u) {
                const int cc = c0 + grp * kCPG + u;
                const bool ok = cc < c1 && cell[u] >= 0 && cell[u] < n_present;
                if (!ok) continue;
                float vf[8];
                dequant<KVT>(rv[u], j, vf);
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const float pw = sm.p[h][cc - c0];
#pragma unroll
                    for (int e = 0; e < 8; ++e) o[h][e] = fmaf(pw, vf[e], o[h][e]);
                }
            }
            __syncthreads();
            QSA_STAMP_LDS(14);
        }
    }

    // merge the 8 groups (same running max in every group), fixed order
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) sm.red[grp][h * kHeadDim + 8 * j + e] = o[h][e];
    __syncthreads();
    if (!active) return;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const int t = h * kHeadDim + tid;  // 256 threads = 256 dims
        float acc = sm.red[0][t];
#pragma unroll
        for (int q = 1; q < kGroups; ++q) acc += sm.red[q][t];
        if (direct) {
            const float l = l_run[h];
            a.out[((int64_t)i * a.n_head + h0 + h) * kHeadDim + tid] = l > 0.f ? acc / l : 0.f;
        } else {
            part[t] = acc;
            if (tid == 0) {
                part[G * kHeadDim + h] = m_run[h];
                part[G * kHeadDim + G + h] = l_run[h];
            }
        }
    }
}

// Partial state of (query i, head group hg, run) in the decode workspace.
template <int G>
__device__ __forceinline__ float *partial_of(const AttnArgs &a, int i, int hg, int run,
                                             int n_runs) {
    return a.ws + (((int64_t)i * (a.n_head / G) + hg) * n_runs + run) * (G * kHeadDim + 2 * G);
}

// Attention over a given cell list: one workgroup per unit (see unit_of);
// a decode run is one chunk, a prefill run all of the query's chunks.
template <int G, int KVT>
__global__ __launch_bounds__(256) void k_attn(AttnArgs a, int chunks_per_run, int n_runs,
                                              int direct) {
    __shared__ AttnSmem<G> sm;
    QSA_STAMP_HOLD(t_start);
    QSA_STAMP_LDS_BEGIN();
    const int n_hg = a.n_head / G;
    int i, run, hg;
    if (!unit_of(a.n_q, n_runs, n_hg, i, run, hg)) return;
    const int hpk = a.n_head / a.n_head_kv;  // query heads per KV head
    const int g = (hg * G) / hpk;            // the KV head
    const int h0 = hg * G;
    const int grp = threadIdx.x >> 5, j = threadIdx.x & 31;
    const int c_begin = run * chunks_per_run * kChunk;
    const int32_t *cells = a.sel_cells + (int64_t)i * a.ld_cells;

    // first round trip: nothing here depends on another load
    const int s = a.q_seq[i];
    const int n_raw = a.n_sel[i];
    int cell[kCPG];
#pragma unroll
    for (int u = 0; u < kCPG; ++u) {
        const int cc = c_begin + grp * kCPG + u;
        cell[u] = cc < a.ld_cells ? cells[cc] : -1;
    }
    float qv[G][8];
    load_q<G>(a, i, h0, j, qv);
    const bool qvalid = s >= 0 && s < a.g.n_seq;
    const int n = qvalid ? (n_raw < 0 ? 0 : (n_raw > a.ld_cells ? a.ld_cells : n_raw)) : 0;
    const int c_end = min(n, c_begin + chunks_per_run * kChunk);
    attend_chunks<G, KVT>(a, i, s, g, h0, c_begin, c_end, cell, cells, qv, sm,
                          direct ? nullptr : partial_of<G>(a, i, hg, run, n_runs), direct != 0,
                          true);
    QSA_STAMP_HOLD(t_end);
    QSA_STAMP_LDS_FLUSH();
    QSA_STAMP_SAVE(0, t_start);
    QSA_STAMP_SAVE(4, t_end);
}

constexpr int kSelAttnNT = 512;
constexpr int kParts = kSelAttnNT / 256;  // 256-thread attention parts per workgroup
constexpr int kSelAttnOnChip = 512;       // fused workgroups resident at once (2 per CU)

// Decode selection fused with attention.  Workgroup = (query i, run of 32
// cells, set of 2 head groups); part q (256 threads) attends for head group
// 2*set + q, so both parts share one KV head whenever the query heads per KV
// head are a multiple of 4 (16 heads over 2 KV heads: 4 sets per run, 260
// workgroups for a 2051-cell set, about one per CU).  First the whole
// workgroup derives query i's exact kept set from the candidates (the kept
// set is unique, so all workgroups derive the same), then finds the cells at
// positions [32*run, 32*run + 32) of the ascending cell list -- kept blocks
// by rank, then the tail cells -- and the parts attend over them.  Without
// a re-admitted group the ranks come from ballots over the candidates, which
// ascend by block, and each run's set-0 workgroup writes its own share of
// the selection outputs; after a re-admission the kept blocks are marked in
// a bitmap, ranked by a prefix count over it, and the workgroup of (run 0,
// set 0) writes all the outputs.  The outputs are written after the
// attention.  Cells, outputs and partial states equal those of the selection
// kernel followed by k_attn.
template <int G, int KVT>
__global__ __launch_bounds__(kSelAttnNT) void k_sel_attn(DecodeIdxArgs f, AttnArgs a,
                                                         int n_runs) {
    __shared__ CandSelSmem<kSelAttnNT, kSelAttnMaxBlocks> ss;
    __shared__ AttnSmem<G> sm[kParts];
    __shared__ int s_cells[kChunk];
    __shared__ int s_blk[kChunk + 1];  // kept blocks of ranks k_lo .. k_hi
    const int n_hg = a.n_head / G;
    const int n_set = (n_hg + kParts - 1) / kParts;
    // workgroup -> (query, run, set), set fastest
    const int set = blockIdx.x % n_set;
    const int run = (blockIdx.x / n_set) % n_runs;
    const int i = blockIdx.x / (n_set * n_runs);
    const int tid = threadIdx.x, part = tid >> 8, lt = tid & 255;
    const int grp = lt >> 5, j = lt & 31;
    const int lane = tid & (kWave - 1), wave = wave_id();
    const int hg_raw = set * kParts + part;
    const bool active = hg_raw < n_hg;
    const int hg = active ? hg_raw : n_hg - 1;  // an idle part mirrors a real one
    const int hpk = a.n_head / a.n_head_kv;
    const int g = (hg * G) / hpk;
    const int h0 = hg * G;
    QSA_STAMP_HOLD(t_start);
    QSA_STAMP_LDS_BEGIN();
    // requests in order: the query's sequence and position, the candidates,
    // the query rows, then the sequence's cell count -- which the selection
    // does not wait for (only the re-admission path and the tail need it)
    const ScoreArgs &sa = f.s;
    QueryFields qf{0, 0, 0, sa.g.n_seq, sa.g.cap_cells, sa.r, sa.nb_max};
    const int s_first = sa.q_seq[i];
    const int64_t p_first = sa.q_pos[i];
    CandKeys<kSelAttnNT, kSelAttnMaxBlocks, kCand> ck;
    uint64_t drop[kSelAttnMaxBlocks / kGroup / kSelAttnNT];
    load_candidates(f, i, ck, drop);
    float qv[G][8];
    load_q<G>(a, i, h0, j, qv);
    qf.s = s_first;
    qf.p = p_first;
    qf.ncell = sa.g.n_cells[min(max(s_first, 0), sa.g.n_seq - 1)];
    const int r = sa.r;
    const int B = f.top_k / r;
    Thresh th;
    const bool fast = select_candidates<kSelAttnNT, kSelAttnMaxBlocks, kCand, true>(f, i, qf, B, ss,
                                                                            ck, drop, th);
    QSA_STAMP_HOLD(t_thresh);
    bool valid;
    const int64_t nc = qf.blocks(valid);
    const int64_t limit = nc < sa.nb_max ? nc : sa.nb_max;
    const int s = qf.s;
    const int tail = valid ? (int)(qf.p + 1 - nc * r) : 0;

    // List positions [c_begin, c_begin + 32): the kept blocks of ascending
    // rank [k_lo, k_hi] (block k covers positions k*r .. k*r + r-1), then
    // the tail cells, then -1.
    const int c_begin = run * kChunk;
    const int k_lo = c_begin / r, k_hi = (c_begin + kChunk - 1) / r;
    const int ld_cells = f.top_k + r - 1;
    int32_t *sel_blocks = f.sel_blocks + (int64_t)i * B;
    // Each path leaves the kept blocks of ranks k_lo .. k_hi in s_blk; one
    // wavefront then expands them (and the tail) into the run's cells.  (The
    // expansion is one short loop-free step rather than a copy per kept key:
    // this code runs once per workgroup, so its size is fetch time.)
    int n_keep_all;
    if (__builtin_expect(fast, 1)) {
        // the kept set is the base candidates th keeps; they ascend by block
        // in the order (wavefront, slot, lane), so a kept one's rank is the
        // kept count of the earlier wavefronts, then of the wavefront's
        // earlier slots, then of its slot's lower lanes (ballots)
        // (each slot's ballot is kept for the ranks below)
        uint64_t bal[decltype(ck)::kBase];
        uint32_t in_wave = 0;
#pragma unroll
        for (int x = 0; x < decltype(ck)::kBase; ++x) {
            bal[x] = x < ck.nb ? __ballot(th.keep((uint32_t)(ck.k[x] >> 32), (uint32_t)ck.k[x]))
                               : 0ull;
            in_wave += __popcll(bal[x]);
        }
        if (lane == 0) ss.tk.red[wave] = in_wave;
        __syncthreads();
        uint32_t before, total;
        {
            constexpr int NW = kSelAttnNT / kWave;
            const uint32_t incl = wave_incl_scan_u32(lane < NW ? ss.tk.red[lane] : 0u);
            total = lane_value(incl, kWave - 1);
            before = wave > 0 ? lane_value(incl, wave - 1) : 0u;
        }
        const int n_keep = (int)(total < (uint32_t)B ? total : (uint32_t)B);
        const uint64_t below = (1ull << lane) - 1ull;
        uint32_t k0 = before;  // rank of this wavefront's next kept slot
#pragma unroll
        for (int x = 0; x < decltype(ck)::kBase; ++x) {
            const bool kp = (bal[x] >> lane) & 1ull;
            const int k = (int)(k0 + __popcll(bal[x] & below));
            if (kp && k >= k_lo && k <= k_hi && k < n_keep) s_blk[k - k_lo] = key_block(ck.k[x]);
            k0 += __popcll(bal[x]);
        }
        n_keep_all = n_keep;
    } else {
        // ranks of this thread's bitmap words
        const int n_words = (int)((limit + 31) / 32);
        const int per = (n_words + kSelAttnNT - 1) / kSelAttnNT;
        const int w0 = tid * per;
        uint32_t local = 0;
        for (int w = w0; w < w0 + per && w < n_words; ++w) local += __popc(ss.bitmap[w]);
        const uint32_t incl = wave_incl_scan_u32(local);
        if (lane == kWave - 1) ss.tk.red[wave] = incl;
        __syncthreads();
        uint32_t before, total;
        waves_prefix<kSelAttnNT / kWave>(ss.tk.red, wave, before, total);
        const uint32_t rank = before + incl - local;
        const int n_keep = (int)(total < (uint32_t)B ? total : (uint32_t)B);
        if (local && (int)rank <= k_hi && (int)(rank + local) > k_lo) {
            uint32_t k = rank;
            for (int w = w0; w < w0 + per && w < n_words; ++w) {
                uint32_t bits = ss.bitmap[w];
                while (bits) {
                    const int bit = __builtin_ctz(bits);
                    bits &= bits - 1;
                    if ((int)k >= k_lo && (int)k <= k_hi && (int)k < n_keep)
                        s_blk[k - k_lo] = w * 32 + bit;
                    ++k;
                }
            }
        }
        n_keep_all = n_keep;
    }
    __syncthreads();
    if (tid < kChunk) {
        // position c_begin + tid: cell pos % r of the kept block of rank
        // pos / r, else a tail cell, else -1
        const int pos = c_begin + tid;
        const int n_blk_cells = n_keep_all * r;
        int cell;
        if (pos < n_blk_cells) {
            const int k = pos / r;
            cell = s_blk[k - k_lo] * r + (pos - k * r);
        } else {
            cell = pos < n_blk_cells + tail ? (int)(nc * r + (pos - n_blk_cells)) : -1;
        }
        s_cells[tid] = cell;
    }
    __syncthreads();
    const int n_sel = n_keep_all * r + tail;
    QSA_STAMP_HOLD(t_placed);
    int cell[kCPG];
#pragma unroll
    for (int u = 0; u < kCPG; ++u) cell[u] = s_cells[grp * kCPG + u];
    const int c_end = min(n_sel, c_begin + kChunk);
    attend_chunks<G, KVT>(a, i, s, g, h0, c_begin, c_end, cell, nullptr, qv, sm[part],
                          partial_of<G>(a, i, hg, run, n_runs), false, active);

    // The selection outputs, after the attention: a barrier waits for every
    // store issued before it, so stores issued earlier would delay the
    // gather.  attend_chunks leaves s_cells, s_blk and ss untouched.
    if (__builtin_expect(fast, 1)) {
        // this run's share (set 0): its blocks, -1 past the kept blocks (the
        // runs' block ranks cover [0, B)), its list positions; the count
        // from run 0
        if (set == 0) {
            const int k = k_lo + tid;
            if (k <= k_hi && k < B) sel_blocks[k] = k < n_keep_all ? s_blk[tid] : -1;
            if (tid < kChunk && c_begin + tid < ld_cells)
                f.sel_cells[(int64_t)i * ld_cells + c_begin + tid] = s_cells[tid];
            if (run == 0 && tid == 0) f.n_sel[i] = n_sel;
        }
    } else if (run == 0 && set == 0) {
        const int n_words = (int)((limit + 31) / 32);
        emit_from_bitmap<kSelAttnNT>(ss.bitmap, n_words, B, r, nc, tail, sel_blocks,
                                     f.sel_cells + (int64_t)i * ld_cells, ld_cells, f.n_sel + i,
                                     ss.tk);
    }
    QSA_STAMP_LDS_FLUSH();
    QSA_STAMP_SAVE(0, t_start);
    QSA_STAMP_SAVE(2, t_thresh);
    QSA_STAMP_SAVE(3, t_placed);
    QSA_STAMP(4);
}

constexpr int kCombNT = 256;
constexpr int kCombWaves = kCombNT / kWave;
constexpr int kCombSlices = kHeadDim / kWave;  // workgroups per head: 64 output dims each
constexpr int kCombPre = 17;                    // runs per wavefront loaded up front
// longest cell list: top_k/r <= 4096 blocks of r <= 16 cells plus r-1 tail
// cells, 65,551 positions in runs of 32
constexpr int kCombMaxRuns = (4096 * 16 + 15 + kChunk - 1) / kChunk;
static_assert(kCombWaves == 4, "the merge adds its wavefronts' values two by two");

// grid (n_head * 4, n_q).  Workgroup (head h, 64-dim slice) merges the runs'
// partial states of that head for its 64 output dims: wavefront w sums runs
// w, w+4, ... with lane = output dim.  Its first kCombPre runs are loaded
// together with the (m, l) pairs, before the weights are known (every run's
// partial is written, zeros for a run that saw no cell), so a decode set of up
// to 4*kCombPre = 68 runs (2,176 cells) costs one memory round trip.  The
// wavefronts' sums are added in a fixed order.
template <int G>
__global__ __launch_bounds__(kCombNT) void k_attn_combine(AttnArgs a, int n_runs) {
    __shared__ float s_w[kCombMaxRuns];  // m of run r, then its weight exp(m_r - M)
    __shared__ float s_l[kCombMaxRuns];
    __shared__ float s_red[kCombWaves];
    __shared__ float s_acc[kCombWaves][kWave];
    QSA_STAMP(5);
    const int h = blockIdx.x / kCombSlices, slice = blockIdx.x % kCombSlices;
    const int i = blockIdx.y, tid = threadIdx.x, wave = tid >> 6, lane = tid & (kWave - 1);
    const int hg = h / G, hh = h % G;
    const int stride = G * kHeadDim + 2 * G;
    const float *base = a.ws + ((int64_t)i * (a.n_head / G) + hg) * n_runs * stride;
    const int col = hh * kHeadDim + slice * kWave + lane;
    // every load is issued (clamped to the last run; a run past n_runs gets
    // weight 0): a load under a lane condition is waited for right after it
    float pre[kCombPre];
#pragma unroll
    for (int u = 0; u < kCombPre; ++u)
        pre[u] = base[(int64_t)min(wave + kCombWaves * u, n_runs - 1) * stride + col];
    // (m, l) of runs tid, tid + 256, ...; a run that saw no cell has l = 0
    float mloc = -INFINITY;
    for (int r = tid; r < n_runs; r += kCombNT) {
        const float m = base[(int64_t)r * stride + G * kHeadDim + hh];
        const float l = base[(int64_t)r * stride + G * kHeadDim + G + hh];
        const bool seen = l > 0.f;
        s_w[r] = seen ? m : -INFINITY;
        s_l[r] = seen ? l : 0.f;
        mloc = fmaxf(mloc, seen ? m : -INFINITY);
    }
    mloc = wave_max_f32(mloc);
    if (lane == 0) s_red[wave] = mloc;
    __syncthreads();
    const float M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    // weights exp(m_r - M) of this thread's own runs (no barrier needed)
    float lw = 0.f;
    for (int r = tid; r < n_runs; r += kCombNT) {
        const float m = s_w[r];
        const float w = m != -INFINITY ? __expf(m - M) : 0.f;
        s_w[r] = w;
        lw += s_l[r] * w;
    }
    lw = wave_sum_f32(lw);
    __syncthreads();  // every M read before s_red is reused; every weight written
    if (lane == 0) s_red[wave] = lw;
    __syncthreads();
    const float L = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);

    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < kCombPre; ++u) {
        const int r = wave + kCombWaves * u;
        acc = fmaf(pre[u], r < n_runs ? s_w[r] : 0.f, acc);
    }
    constexpr int U = 8;
    for (int r0 = wave + kCombWaves * kCombPre; r0 < n_runs; r0 += kCombWaves * U) {
        float v[U], w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = r0 + kCombWaves * u;
            w[u] = r < n_runs ? s_w[r] : 0.f;
            v[u] = base[(int64_t)min(r, n_runs - 1) * stride + col];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc = fmaf(v[u], w[u], acc);
    }
    s_acc[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
        const float t = (s_acc[0][lane] + s_acc[1][lane]) + (s_acc[2][lane] + s_acc[3][lane]);
        a.out[((int64_t)i * a.n_head + h) * kHeadDim + slice * kWave + lane] = L > 0.f ? t / L : 0.f;
    }
    QSA_STAMP(6);
}

template <int G, int KVT>
hipError_t launch_g(const AttnArgs &a, int chunks_per_run, int n_runs, bool direct,
                    hipStream_t st) {
    // 8 equal unit ranges, one per XCD (k_attn maps ids to units)
    const int units = a.n_q * (a.n_head / G) * n_runs;
    const int grid = (units + 7) / 8 * 8;
    hipLaunchKernelGGL((k_attn<G, KVT>), dim3(grid), dim3(256), 0, st, a, chunks_per_run, n_runs,
                       direct ? 1 : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || direct) return e;
    hipLaunchKernelGGL((k_attn_combine<G>), dim3(a.n_head * kCombSlices, a.n_q), dim3(kCombNT),
                       0, st, a, n_runs);
    return hipGetLastError();
}

// Heads per workgroup: 2 (enough workgroups to give every SIMD two
// wavefronts on a single decode query, and a quarter of the registers of
// 8); 4 (wide) when a call's queries fill the chip -- fewer, longer
// workgroups, each K/V row loaded once for twice the heads; 8 heads cost
// too many registers.  It must divide the query heads per KV head.
template <int KVT>
hipError_t launch_kvt(const AttnArgs &a, int chunks_per_run, int n_runs, bool direct,
                      bool wide, hipStream_t st) {
    const int hpk = a.n_head / a.n_head_kv;
    if (wide && hpk % 4 == 0) return launch_g<4, KVT>(a, chunks_per_run, n_runs, direct, st);
    if (hpk % 2 == 0) return launch_g<2, KVT>(a, chunks_per_run, n_runs, direct, st);
    return launch_g<1, KVT>(a, chunks_per_run, n_runs, direct, st);
}

hipError_t launch(const AttnArgs &a, int chunks_per_run, int n_runs, bool direct, bool wide,
                  hipStream_t st) {
    if (a.n_q <= 0) return hipSuccess;
    if (a.kv_type == QSA_KV_F32)
        return launch_kvt<QSA_KV_F32>(a, chunks_per_run, n_runs, direct, wide, st);
    if (a.kv_type == QSA_KV_F16)
        return launch_kvt<QSA_KV_F16>(a, chunks_per_run, n_runs, direct, wide, st);
    return launch_kvt<QSA_KV_Q8_0>(a, chunks_per_run, n_runs, direct, wide, st);
}

int decode_runs(int ld_cells) { return (ld_cells + kChunk - 1) / kChunk; }

// Chunks per run of the decode attention: one while a call fits the fused
// grid (65 runs of a 2,051-cell list spread one query over the chip), two
// past it (half the workgroups and partial states; measured on five
// 250k-cell sessions, 4 heads x 2 chunks beat 2 x 1, 2 x 2, 4 x 1, 4 x 3,
// 4 x 4 and 8 x 1).
constexpr int kMultiChunks = 2;

template <int G, int KVT>
hipError_t launch_sel_g(const DecodeIdxArgs &f, const AttnArgs &a, hipStream_t st) {
    const int n_runs = decode_runs(a.ld_cells);
    const int n_set = (a.n_head / G + kParts - 1) / kParts;
    const int grid = a.n_q * n_runs * n_set;
    hipLaunchKernelGGL((k_sel_attn<G, KVT>), dim3(grid), dim3(kSelAttnNT), 0, st, f, a, n_runs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_attn_combine<G>), dim3(a.n_head * kCombSlices, a.n_q), dim3(kCombNT),
                       0, st, a, n_runs);
    return hipGetLastError();
}

template <int KVT>
hipError_t launch_sel_kvt(const DecodeIdxArgs &f, const AttnArgs &a, hipStream_t st) {
    const int hpk = a.n_head / a.n_head_kv;
    if (hpk % 2 == 0) return launch_sel_g<2, KVT>(f, a, st);
    return launch_sel_g<1, KVT>(f, a, st);
}

}  // namespace

QSA_STAMP_READER(attn)

size_t attn_decode_ws_bytes(int n_q, int n_head, int ld_cells) {
    // per (query, run, head group): G*256 + 2G floats; over the head groups
    // this is n_head*(256 + 2) floats per run
    return (size_t)n_q * decode_runs(ld_cells) * n_head * (kHeadDim + 2) * sizeof(float);
}

// Whether the fused selection + attention grid of this call fits the chip
// in one round (it then runs; otherwise selection and attention split).
static_assert(kSelAttnOnChip == 512 && kParts == 2 && kChunk == 32,
              "fused_decode_fits assumes these");
static bool fused_fits(const AttnArgs &a) {
    return fused_decode_fits(a.n_q, a.ld_cells, a.n_head, a.n_head_kv);
}

// The attention units are those of the fused kernel whenever that could
// run (so the two paths give identical outputs); past it the units widen.
hipError_t launch_attn_decode(const AttnArgs &a, hipStream_t st) {
    if (!fused_fits(a)) {
        const int span = kMultiChunks * kChunk;
        return launch(a, kMultiChunks, (a.ld_cells + span - 1) / span, false, true, st);
    }
    return launch(a, 1, decode_runs(a.ld_cells), false, false, st);
}

hipError_t launch_select_attn_decode(DecodeIdxArgs f, void *ws_idx, const AttnArgs &a,
                                     hipStream_t st) {
    if (a.n_q <= 0) return hipSuccess;
    // Every fused workgroup derives the selection itself: free while the
    // grid fits the chip in one round, wasteful beyond (several queries).
    // Then select once per query and attend over the lists instead; the
    // selection and the attention arithmetic are the same, so are the results.
    if (!fused_fits(a)) {
        hipError_t e = launch_decode_select(f, ws_idx, st);
        if (e != hipSuccess) return e;
        return launch_attn_decode(a, st);
    }
    bind_candidates(f, ws_idx);
    if (a.kv_type == QSA_KV_F32) return launch_sel_kvt<QSA_KV_F32>(f, a, st);
    if (a.kv_type == QSA_KV_F16) return launch_sel_kvt<QSA_KV_F16>(f, a, st);
    return launch_sel_kvt<QSA_KV_Q8_0>(f, a, st);
}


}  // namespace qsa
