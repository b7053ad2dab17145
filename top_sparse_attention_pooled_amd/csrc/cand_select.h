// cand_select.h -- exact block top-k of one decode query from the scoring
// kernel's candidates (llama.cpp issue #28734, fix summary, "lever3": whole
// blocks compete, ranked by score with ties to the lower block).
//
// The scoring kernel leaves, for every group of 64 blocks (one wavefront's
// tile), the group's 4 largest 64-bit keys (score key << 32 | ~block), in
// ascending block order, and the largest key it dropped.  The selection
// takes the top-B threshold over the candidates; a group whose dropped key
// would itself be kept under that threshold may hold more winners, so all 64
// of its keys are re-admitted (or, past 32 such groups, the whole score row
// is streamed) and the threshold is taken again.  A dropped key of any other
// group lies below the first threshold, which can only rise as keys are
// added, so the final kept set is the exact top-B of all scores.  Without a
// re-admission the kept set lies among the candidates, and since they ascend
// by block, a kept candidate's place in the ascending output is the number
// of kept candidates before it.
//
// The same routine runs in a 1024-thread selection workgroup and inside each
// 512-thread fused attention workgroup; the kept set is unique, so every caller
// derives the same one.
#pragma once

#include "topk_engine.h"

namespace qsa {

constexpr int kGroup = kTile;   // blocks per candidate group (one wavefront)
// Keys kept per group at the least, and the candidates a selection
// workgroup holds in registers.  The fused decode kernel (512 threads,
// every attention workgroup selecting): 4 per group up to nb_max 65536, 8
// up to 32768, 16 up to 16384 blocks -- more slots would cost it the
// registers that let two of its workgroups share a CU.  The per-query
// selection (1024 threads, used when a call's queries overflow the fused
// grid): 6 per group up to nb_max 65536 (per 65536), 8 up to 49152, 16 up
// to 24576.
constexpr int kCand = 4;
constexpr int kCandSlots = 4096;
constexpr int kCandWide = 6;
constexpr int kCandSlotsWide = 6144;
constexpr int kMaxExpand = 32;  // groups re-admitted whole before streaming

// Workspace of the decode indexer: cand [n_q][groups][n_cand], then drop
// [n_q][groups], groups = 4 per 256 blocks of nb_max.
__host__ __device__ inline int cand_groups(int nb_max) { return (nb_max + 255) / 256 * 4; }

// Keys kept per group: as many (16, 8, then the least) as the on-chip
// candidate slots allow.  A group with more winners than it kept must be
// re-admitted whole, which costs the selection a second pass: with B = 512
// of ~62,000 blocks (250k cells) a group of 64 holds 0.53 winners on
// average; with 4 kept keys about one selection in five meets a group of 5
// or more, with 6 about one in a thousand one of 7 or more (a step of five
// sessions would otherwise re-admit in most steps).  Winners spread over
// fewer groups in a shorter context (512 of ~12,400 blocks at 50k cells is
// 2.6 per group on average).
__host__ __device__ inline int cand_per_group(int nb_max, bool wide) {
    const int g = cand_groups(nb_max);
    const int slots = wide ? kCandSlotsWide : kCandSlots;
    return g * 16 <= slots ? 16 : (g * 8 <= slots ? 8 : (wide ? kCandWide : kCand));
}

// Sized for the larger (wide) count, so one workspace serves every call.
inline size_t cand_ws_bytes(int n_q, int nb_max) {
    return (size_t)n_q * cand_groups(nb_max) * (cand_per_group(nb_max, true) + 1) *
           sizeof(uint64_t);
}

inline void bind_candidates(DecodeIdxArgs &f, void *ws) {
    f.n_wg = (f.s.nb_max + 255) / 256;
    f.n_cand = cand_per_group(f.s.nb_max, f.wide_cand != 0);
    f.cand = static_cast<uint64_t *>(ws);
    f.drop = f.cand + (size_t)f.s.n_q * cand_groups(f.s.nb_max) * f.n_cand;
}

// The candidate keys of one query in registers, for up to MAXB blocks: base
// slot s of lane l of wavefront w holds candidate cand_index(nb, s) =
// (w*nb + s)*64 + l -- each wavefront a run of consecutive candidates, slot
// by slot, so every load is 512 contiguous bytes and the candidates ascend
// by block in the order (wavefront, slot, lane).  Expansion slot e holds key
// e*NT + tid of the re-admitted groups' keys (group over[x] at x = (e*NT +
// tid) / 64).  nb / ne: slots in use (workgroup-uniform), so unused slots
// cost one scalar branch.
__device__ __forceinline__ int cand_index(int nb, int s) {
    return ((int)(threadIdx.x >> 6) * nb + s) * kWave + (int)(threadIdx.x & (kWave - 1));
}

template <int NT, int MAXB, int KC>
struct CandKeys {
    static constexpr int kBase = MAXB / kGroup * KC / NT;
    static constexpr int kExp = kMaxExpand * kGroup / NT;
    uint64_t k[kBase + kExp];
    int nb, ne;
    template <typename F>
    __device__ __forceinline__ void operator()(F &&fn) const {
        // (a guarded body, not an early exit: an exit would turn the loop
        // into a runtime-count loop that indexes k[] dynamically)
#pragma unroll
        for (int s = 0; s < kBase; ++s)
            if (s < nb) fn((uint32_t)(k[s] >> 32), (uint32_t)k[s]);
#pragma unroll
        for (int s = 0; s < kExp; ++s)
            if (s < ne) fn((uint32_t)(k[kBase + s] >> 32), (uint32_t)k[kBase + s]);
    }
};

template <int NT, int MAXB>
struct CandSelSmem {
    TopkSmem<NT> tk;
    uint32_t bitmap[MAXB / 32];
    int n_over;
    int over[kMaxExpand];
};

// Query i's candidate keys into ck and each group's largest dropped key into
// drop: every load issued at once, none depending on another load, so a
// kernel issues them first.
template <int NT, int MAXB, int KC>
__device__ __forceinline__ void load_candidates(const DecodeIdxArgs &f, int i,
                                                CandKeys<NT, MAXB, KC> &ck,
                                                uint64_t (&drop)[MAXB / kGroup / NT]) {
    using Keys = CandKeys<NT, MAXB, KC>;
    const int n_grp = cand_groups(f.s.nb_max);
    const int64_t qbase = (int64_t)i * n_grp;
    const int kc = f.n_cand;
    const int n_cand = n_grp * kc;
    ck.nb = (n_cand + NT - 1) / NT;
    ck.ne = 0;
#pragma unroll
    for (int s = 0; s < Keys::kBase; ++s) {
        const int fi = cand_index(ck.nb, s);
        ck.k[s] = (s < ck.nb && fi < n_cand) ? f.cand[qbase * kc + fi] : 0ull;
    }
#pragma unroll
    for (int s = 0; s < Keys::kExp; ++s) ck.k[Keys::kBase + s] = 0ull;
#pragma unroll
    for (int q = 0; q < MAXB / kGroup / NT; ++q) {
        const int g = (int)threadIdx.x + NT * q;
        drop[q] = g < n_grp ? f.drop[qbase + g] : 0ull;
    }
}

// The exact top-B blocks among query i's scored blocks [0, limit), limit =
// qf.limit(): the threshold th over the candidates ck (loaded by
// load_candidates, with drop) (both returned).  Returns true when no group
// was re-admitted and the score row was not streamed: the kept set is then
// exactly the base slots of ck that th keeps, and the query's cell count
// has not been needed.  The kept blocks are also marked in sm.bitmap (words
// [0, ceil(limit/32)) all written), except in that case when
// SKIP_FAST_MARK.  Needs nb_max <= MAXB.  Workgroup-uniform; ends with a
// barrier.
template <int NT, int MAXB, int KC, bool SKIP_FAST_MARK = false>
__device__ __forceinline__ bool select_candidates(const DecodeIdxArgs &f, int i,
                                                  const QueryFields &qf, int B,
                                                  CandSelSmem<NT, MAXB> &sm,
                                                  CandKeys<NT, MAXB, KC> &ck,
                                                  const uint64_t (&drop)[MAXB / kGroup / NT],
                                                  Thresh &th) {
    const int tid = threadIdx.x;
    const float *srow = f.s.scores + (int64_t)i * f.s.ld;
    using Keys = CandKeys<NT, MAXB, KC>;
    constexpr int kDrop = MAXB / kGroup / NT;
    static_assert(kDrop >= 1, "drop slots");
    if (tid == 0) sm.n_over = 0;
    th = topk_threshold<NT>(ck, (uint32_t)B, sm.tk);

#pragma unroll
    for (int q = 0; q < kDrop; ++q) {
        const uint64_t d = drop[q];
        if (__builtin_expect(th.keep((uint32_t)(d >> 32), (uint32_t)d), 0)) {  // (d = 0: never)
            const int at = atomicAdd(&sm.n_over, 1);
            if (at < kMaxExpand) sm.over[at] = tid + NT * q;
        }
    }
    __syncthreads();
    const int n_over = sm.n_over;
    const bool fast = n_over == 0;
    // (the common case: its code is laid out first, the rest out of line)
    if (SKIP_FAST_MARK && __builtin_expect(fast, 1)) return true;

    const int64_t limit = qf.limit();
    const int n_words = (int)((limit + 31) / 32);
    for (int w = tid; w < n_words; w += NT) sm.bitmap[w] = 0;
    if (fast) __syncthreads();  // (otherwise a threshold pass orders the clearing and marking)
    auto from_memory = [&](auto &&fn) {
        constexpr int U = 16;
        for (int64_t base = 0; base < limit; base += (int64_t)NT * U) {
            float v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t bb = base + (int64_t)u * NT + tid;
                v[u] = bb < limit ? srow[bb] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t bb = base + (int64_t)u * NT + tid;
                if (bb < limit) fn(finite_f32(v[u]) ? score_key(v[u]) : 0u, ~(uint32_t)bb);
            }
        }
    };
    const bool stream = n_over > kMaxExpand;
    if (stream) {
        th = topk_threshold<NT>(from_memory, (uint32_t)B, sm.tk);
    } else if (n_over > 0) {
        // replace the kept keys of the re-admitted groups by all of theirs
        const int kc = f.n_cand;
#pragma unroll
        for (int s = 0; s < Keys::kBase; ++s) {
            const int g = cand_index(ck.nb, s) / kc;
            for (int e = 0; e < n_over; ++e)
                if (sm.over[e] == g) ck.k[s] = 0ull;
        }
        ck.ne = (n_over * kGroup + NT - 1) / NT;
        // every score requested before the first is used (indexes clamped)
        float sc[Keys::kExp];
        int64_t bbs[Keys::kExp];
#pragma unroll
        for (int s = 0; s < Keys::kExp; ++s) {
            const int idx = s * NT + tid;
            const int x = idx / kGroup;
            const int64_t bb = x < n_over ? (int64_t)sm.over[x] * kGroup + idx % kGroup : -1;
            bbs[s] = bb;
            sc[s] = srow[bb >= 0 && bb < limit ? bb : 0];
        }
#pragma unroll
        for (int s = 0; s < Keys::kExp; ++s) {
            const int64_t bb = bbs[s];
            ck.k[Keys::kBase + s] =
                (bb >= 0 && bb < limit && finite_f32(sc[s])) ? block_key(sc[s], bb) : 0ull;
        }
        th = topk_threshold<NT>(ck, (uint32_t)B, sm.tk);
    }

    auto mark = [&](uint32_t k, uint32_t u) {
        if (th.keep(k, u)) {
            const uint32_t bb = ~u;
            atomicOr(&sm.bitmap[bb >> 5], 1u << (bb & 31));
        }
    };
    if (stream)
        from_memory(mark);
    else
        ck(mark);
    __syncthreads();
    return fast;
}

}  // namespace qsa
