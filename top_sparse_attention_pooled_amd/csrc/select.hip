// select.hip -- block-granular top-k, expanded to cells (llama.cpp issue
// #28734, fix summary, "lever3": select whole blocks first, expand only the
// selected ones; goodbadwolf's comment on the same issue gives the set's
// capacity n_kv_max = top_k + r - 1, the budget plus the tail).
//
// One 1024-thread workgroup per query.  Every candidate block b (finite score,
// b < number of complete blocks) gets the 64-bit key
//     K(b) = (order-preserving bits of its score) << 32 | ~b,
// so a larger key means a higher score and, on equal scores, a lower block
// index: the ranking is a strict total order and the kept set is exactly the
// blocks with the top_k/r largest keys.  An LDS radix select finds the
// threshold key 11 bits at a time (usually two or three passes over the
// scores suffice: it stops once the threshold digit's bucket is taken whole),
// one more pass collects the kept blocks, and a bitonic sort in LDS puts them
// in ascending order before the expansion to cells.
#include "qsa_internal.h"

namespace qsa {

namespace {

constexpr int kThreads = 1024;
constexpr int kBins = 2048;
constexpr int kMaxKeep = 4096;  // top_k / r supported

__device__ __forceinline__ uint64_t block_key(float s, int64_t b) {
    return ((uint64_t)score_key(s) << 32) | (uint64_t)(~(uint32_t)b);
}

// Inclusive scan (sum) across the workgroup of one value per thread, in
// thread order; returns the inclusive prefix, writes the total.
__device__ __forceinline__ uint32_t block_scan_incl(uint32_t v, uint32_t *s_wave,
                                                    uint32_t &total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t t = __shfl_up(v, o, kWave);
        if (lane >= o) v += t;
    }
    if (lane == kWave - 1) s_wave[wave] = v;
    __syncthreads();
    if (wave == 0) {
        uint32_t w = lane < kThreads / kWave ? s_wave[lane] : 0u;
#pragma unroll
        for (int o = 1; o < kThreads / kWave; o <<= 1) {
            const uint32_t t = __shfl_up(w, o, kWave);
            if (lane >= o) w += t;
        }
        if (lane < kThreads / kWave) s_wave[lane] = w;
    }
    __syncthreads();
    const uint32_t before = wave > 0 ? s_wave[wave - 1] : 0u;
    total = s_wave[kThreads / kWave - 1];
    __syncthreads();
    return v + before;
}

__global__ __launch_bounds__(kThreads) void k_select(SelectArgs a) {
    __shared__ uint32_t hist[kBins];
    __shared__ uint32_t s_wave[kThreads / kWave];
    __shared__ int32_t keep[kMaxKeep];
    __shared__ uint32_t s_digit, s_krem, s_eq, s_count;

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

    // --- radix select of the B-th largest key -------------------------------
    // Digits from the top: score bits [31:21], [20:10], [9:0], then index bits
    // [31:21], [20:10], [9:0] of the 64-bit key.
    const int widths[6] = {11, 11, 10, 11, 11, 10};
    uint64_t prefix = 0;   // fixed high bits of the threshold
    int fixed = 0;         // how many high bits are fixed
    uint32_t krem = (uint32_t)B;
    bool take_all = false;
    for (int pass = 0; pass < 6; ++pass) {
        const int w = widths[pass];
        const int shift = 64 - fixed - w;
        for (int j = tid; j < kBins; j += kThreads) hist[j] = 0;
        __syncthreads();
        for (int64_t b = tid; b < limit; b += kThreads) {
            const float sc = row[b];
            if (!finite_f32(sc)) continue;
            const uint64_t K = block_key(sc, b);
            if (fixed > 0 && (K >> (64 - fixed)) != (prefix >> (64 - fixed))) continue;
            atomicAdd(&hist[(uint32_t)(K >> shift) & ((1u << w) - 1u)], 1u);
        }
        __syncthreads();
        // suffix counts: bins above each thread's pair (2*tid, 2*tid+1)
        const uint32_t h0 = hist[2 * tid], h1 = hist[2 * tid + 1];
        uint32_t total;
        // scan in reversed thread order so each thread gets the bins above it
        const uint32_t h_rev0 = hist[2 * (kThreads - 1 - tid)];
        const uint32_t h_rev1 = hist[2 * (kThreads - 1 - tid) + 1];
        const uint32_t incl_rev = block_scan_incl(h_rev0 + h_rev1, s_wave, total);
        // incl_rev at reversed thread u = sum of pairs kThreads-1-u .. kThreads-1
        hist[2 * (kThreads - 1 - tid)] = incl_rev;  // reuse: inclusive suffix of pair
        __syncthreads();
        const uint32_t suffix_incl = hist[2 * tid];  // pairs tid .. end
        const uint32_t above = suffix_incl - h0 - h1;  // pairs tid+1 .. end
        __syncthreads();
        if (pass == 0 && total <= krem) {
            take_all = true;  // every finite candidate is kept
            break;
        }
        // bin 2*tid+1 then bin 2*tid
        if (above < krem && above + h1 >= krem) {
            s_digit = 2 * tid + 1;
            s_krem = krem - above;
            s_eq = h1;
        } else if (above + h1 < krem && above + h1 + h0 >= krem) {
            s_digit = 2 * tid;
            s_krem = krem - above - h1;
            s_eq = h0;
        }
        __syncthreads();
        if (w < 11 && s_digit >= (1u << w)) {
            // cannot happen: bins >= 2^w stay empty
        }
        prefix |= (uint64_t)s_digit << shift;
        fixed += w;
        krem = s_krem;
        const uint32_t eq = s_eq;
        __syncthreads();
        if (eq == krem) break;  // the threshold bucket is taken whole
    }

    // --- collect the kept blocks ---------------------------------------------
    if (tid == 0) s_count = 0;
    __syncthreads();
    for (int64_t b = tid; b < limit; b += kThreads) {
        const float sc = row[b];
        if (!finite_f32(sc)) continue;
        const uint64_t K = block_key(sc, b);
        const bool sel = take_all || (K >> (64 - fixed)) >= (prefix >> (64 - fixed));
        if (sel) {
            const uint32_t at = atomicAdd(&s_count, 1u);
            if (at < (uint32_t)kMaxKeep) keep[at] = (int32_t)b;
        }
    }
    __syncthreads();
    int n_keep = (int)s_count;
    if (n_keep > B) n_keep = B;  // defensive: the key order is strict

    // --- ascending order: bitonic sort of keep[0 .. P) in LDS ---------------
    int P = 1;
    while (P < n_keep) P <<= 1;
    for (int j = n_keep + tid; j < P; j += kThreads) keep[j] = 0x7fffffff;
    __syncthreads();
    for (int k = 2; k <= P; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int t = tid; t < P; t += kThreads) {
                const int u = t ^ j;
                if (u > t) {
                    const int x = keep[t], y = keep[u];
                    const bool up = (t & k) == 0;
                    if ((x > y) == up) {
                        keep[t] = y;
                        keep[u] = x;
                    }
                }
            }
            __syncthreads();
        }
    }

    // --- outputs -----------------------------------------------------------
    const int tail = valid ? (int)(p + 1 - nc * a.r) : 0;
    const int ld_cells = a.top_k + a.r - 1;
    int32_t *ob = a.sel_blocks + (int64_t)i * B;
    int32_t *oc = a.sel_cells + (int64_t)i * ld_cells;
    for (int j = tid; j < B; j += kThreads) ob[j] = j < n_keep ? keep[j] : -1;
    const int n_full = n_keep * a.r;
    for (int j = tid; j < ld_cells; j += kThreads) {
        int32_t c = -1;
        if (j < n_full)
            c = keep[j / a.r] * a.r + j % a.r;
        else if (j < n_full + tail)
            c = (int32_t)(nc * a.r + (j - n_full));
        oc[j] = c;
    }
    if (tid == 0) a.n_sel[i] = n_full + tail;
}

}  // namespace

hipError_t launch_select(const SelectArgs &a, hipStream_t st) {
    if (a.n_q <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_select, dim3(a.n_q), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace qsa
