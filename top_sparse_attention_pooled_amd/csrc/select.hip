// select.hip -- block-granular top-k, expanded to cells (llama.cpp issue
// #28734, fix summary, "lever3": select whole blocks first, expand only the
// selected ones; goodbadwolf's comment on the same issue gives the set's
// capacity n_kv_max = top_k + r - 1, the budget plus the tail).
//
// One 1024-thread workgroup per query.  Candidate block b (finite score,
// b < number of complete blocks) has the unique key
//     (order-preserving bits of its score) << 32 | ~b,
// so the kept set is exactly the blocks with the top_k/r largest keys: the
// ranking's ties go to the lower block index.  Up to 24,576 blocks the keys
// live in registers (24 per thread, loaded once with every load in flight);
// beyond that they are re-streamed from memory each round.  The threshold
// comes from topk_engine.h; the kept blocks are marked in an LDS bitmap and
// emitted in ascending order, each expanded to its r cells, followed by the
// tail cells of the incomplete block.
#include "topk_engine.h"

namespace qsa {

namespace {

constexpr int kNT = 1024;
constexpr int kC = 24;                        // register-cached keys per thread
constexpr int kMaxBitmapBlocks = 1 << 19;      // 64 KiB bitmap
constexpr int kMaxKeep = 4096;

struct SelSmem {
    TopkSmem<kNT> tk;
    union {
        uint32_t bitmap[kMaxBitmapBlocks / 32];
        int32_t list[kMaxKeep];
    };
    uint32_t count;
};

// Keys of one query's score row re-read from memory, 16 loads in flight.
struct RowStream {
    const float *row;
    int64_t limit;
    template <typename F>
    __device__ __forceinline__ void operator()(F &&fn) const {
        constexpr int U = 16;
        const int tid = threadIdx.x;
        for (int64_t base = 0; base < limit; base += (int64_t)kNT * U) {
            float v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t b = base + (int64_t)u * kNT + tid;
                v[u] = b < limit ? row[b] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t b = base + (int64_t)u * kNT + tid;
                if (b < limit) fn(finite_f32(v[u]) ? score_key(v[u]) : 0u, ~(uint32_t)b);
            }
        }
    }
};

struct SelSource {
    RegKeys32<kC, kNT> regs;
    RowStream mem;
    bool in_regs;
    template <typename F>
    __device__ __forceinline__ void operator()(F &&fn) const {
        if (in_regs)
            regs(fn);
        else
            mem(fn);
    }
};

__global__ __launch_bounds__(kNT) void k_select(SelectArgs a) {
    __shared__ SelSmem sm;
    const int i = blockIdx.x;
    const int tid = threadIdx.x;
    int s;
    int64_t p;
    bool valid;
    const int64_t nc = query_blocks(a.q_seq, a.q_pos, i, a.g.n_seq, a.g.cap_cells, a.g.n_cells,
                                    a.r, s, p, valid);
    const int64_t limit = nc < a.nb_max ? nc : a.nb_max;
    const int B = a.top_k / a.r;
    const float *row = a.scores + (int64_t)i * a.ld;

    // score keys cached in registers (block = s2*kNT + tid), or, past
    // 24576 blocks, the score row re-read from memory on every pass (one
    // source type, so the engine is instantiated once)
    SelSource src;
    src.regs.tid = tid;
    src.mem = RowStream{row, limit};
    src.in_regs = limit <= (int64_t)kNT * kC;
    if (src.in_regs) {
        // (limit == 0 reads nothing: the score row may then be absent, NULL)
#pragma unroll
        for (int s2 = 0; s2 < kC; ++s2) src.regs.k[s2] = 0u;
        if (limit > 0) {  // workgroup-uniform
#pragma unroll
            for (int s2 = 0; s2 < kC; ++s2) {
                const int64_t b = (int64_t)s2 * kNT + tid;
                const float sc = row[b < limit ? b : 0];  // unconditional: no wait per load
                src.regs.k[s2] = (b < limit && finite_f32(sc)) ? score_key(sc) : 0u;
            }
        }
    }
    const Thresh th = topk_threshold<kNT>(src, (uint32_t)B, sm.tk);
    const RowStream &from_memory = src.mem;

    const int tail = valid ? (int)(p + 1 - nc * a.r) : 0;
    const int ld_cells = a.top_k + a.r - 1;
    int32_t *ob = a.sel_blocks + (int64_t)i * B;
    int32_t *oc = a.sel_cells + (int64_t)i * ld_cells;
    if (limit <= kMaxBitmapBlocks) {
        const int n_words = (int)((limit + 31) / 32);
        for (int w = tid; w < n_words; w += kNT) sm.bitmap[w] = 0;
        __syncthreads();
        auto mark = [&](uint32_t k, uint32_t u) {
            if (th.keep(k, u)) {
                const uint32_t b = ~u;
                atomicOr(&sm.bitmap[b >> 5], 1u << (b & 31));
            }
        };
        src(mark);
        __syncthreads();
        emit_from_bitmap<kNT>(sm.bitmap, n_words, B, a.r, nc, tail, ob, oc, ld_cells,
                              a.n_sel + i, sm.tk);
    } else {
        // very long contexts: collect the <= B kept blocks, bitonic-sort them
        if (tid == 0) sm.count = 0;
        __syncthreads();
        from_memory([&](uint32_t k, uint32_t u) {
            if (th.keep(k, u)) {
                const uint32_t at = atomicAdd(&sm.count, 1u);
                if (at < (uint32_t)kMaxKeep) sm.list[at] = (int32_t)(~u);
            }
        });
        __syncthreads();
        const int n_keep = (int)(sm.count < (uint32_t)B ? sm.count : (uint32_t)B);
        if (tid == 0) a.n_sel[i] = n_keep * a.r + tail;
        int P = 1;
        while (P < n_keep) P <<= 1;
        for (int j = n_keep + tid; j < P; j += kNT) sm.list[j] = 0x7fffffff;
        __syncthreads();
        for (int kk = 2; kk <= P; kk <<= 1)
            for (int j = kk >> 1; j > 0; j >>= 1) {
                for (int t = tid; t < P; t += kNT) {
                    const int u = t ^ j;
                    if (u > t) {
                        const int x = sm.list[t], y = sm.list[u];
                        if ((x > y) == ((t & kk) == 0)) {
                            sm.list[t] = y;
                            sm.list[u] = x;
                        }
                    }
                }
                __syncthreads();
            }
        for (int j = tid; j < B; j += kNT) ob[j] = j < n_keep ? sm.list[j] : -1;
        const int n_full = n_keep * a.r;
        for (int j = tid; j < ld_cells; j += kNT) {
            int32_t c = -1;
            if (j < n_full)
                c = sm.list[j / a.r] * a.r + j % a.r;
            else if (j < n_full + tail)
                c = (int32_t)(nc * a.r + (j - n_full));
            oc[j] = c;
        }
    }
}

}  // namespace

hipError_t launch_select(const SelectArgs &a, hipStream_t st) {
    if (a.n_q <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_select, dim3(a.n_q), dim3(kNT), 0, st, a);
    return hipGetLastError();
}

}  // namespace qsa
