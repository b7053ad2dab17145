// pooled.hip -- the persistent pooled block-key cache (llama.cpp issue #28734,
// fix summary, "lever2": pooled + normed + roped block keys kept in their own
// buffer, only dirtied blocks recomputed, the dirty ones found by comparing
// each block's member cells with those it was built from -- which also
// catches defrag, rollback and sequence edits without invalidation hooks;
// "lever2b": block membership resolved on the device).  A block's members are
// the rows of positions b*r .. b*r+r-1 of its sequence (through the caller's
// cell table when there is one).
//
// One wavefront per dirty block (pooled_key_lane in qsa_internal.h): lane t
// owns the split-half RoPE pair (t, t+64), so the mean-pool, the RMS norm and
// the rotation all stay in registers.
#include "qsa_internal.h"

namespace qsa {

namespace {

__global__ __launch_bounds__(256) void k_update_pooled(UpdateArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= a.n_dirty) return;
    const int s = a.dirty[2 * i];
    const int b = a.dirty[2 * i + 1];
    if (s < 0 || s >= a.g.n_seq || b < 0) return;
    const int64_t cap_blocks = a.g.cap_cells / a.r;
    if (b >= cap_blocks) return;
    int64_t n = a.g.n_cells[s];
    if (n > a.g.cap_cells) n = a.g.cap_cells;
    if ((int64_t)b * a.r >= n) return;
    float lo, hi;
    pooled_key_lane(a.kidx, a.g, s, b, n, a.r, a.eps, a.gamma, a.rope, lane, lo, hi);
    store_pooled_lane(a.pooled, a.pooled_bf16, cap_blocks, s, b, lane, lo, hi);
}

__global__ __launch_bounds__(256) void k_dirty_reset(DirtyArgs a) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t < 2 * (int64_t)a.max_dirty) a.dirty[t] = -1;
    if (t == 0) *a.n_found = 0u;
}

// One thread per (sequence, block) of the capacity: compare the block's
// present member count and member rows with its snapshot; a changed
// non-empty block is listed and its snapshot updated (a block the list has no
// room for keeps its snapshot, so the next call finds it again); an emptied
// block is recorded, not listed.
__global__ __launch_bounds__(256) void k_detect_dirty(DirtyArgs a) {
    const int64_t cap_blocks = a.g.cap_cells / a.r;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= (int64_t)a.g.n_seq * cap_blocks) return;
    const int s = (int)(t / cap_blocks);
    const int64_t b = t - (int64_t)s * cap_blocks;
    int64_t n = a.g.n_cells[s];
    n = n < 0 ? 0 : (n > a.g.cap_cells ? a.g.cap_cells : n);
    const int64_t first = b * a.r;
    const int m = n > first ? (int)(n - first < a.r ? n - first : a.r) : 0;
    int32_t *sn = a.snap + t * (a.r + 1);
    bool same = sn[0] == m;
    for (int j = 0; j < m; ++j) same = same && sn[1 + j] == (int32_t)cell_row(a.g, s, first + j);
    if (same) return;
    if (m == 0) {
        sn[0] = 0;
        return;
    }
    const uint32_t at = atomicAdd(a.n_found, 1u);
    if (at >= (uint32_t)a.max_dirty) return;
    a.dirty[2 * at] = s;
    a.dirty[2 * at + 1] = (int32_t)b;
    sn[0] = m;
    for (int j = 0; j < m; ++j) sn[1 + j] = (int32_t)cell_row(a.g, s, first + j);
}

}  // namespace

hipError_t launch_detect_dirty(const DirtyArgs &a, hipStream_t st) {
    const int64_t reset = 2 * (int64_t)a.max_dirty > 1 ? 2 * (int64_t)a.max_dirty : 1;
    hipLaunchKernelGGL(k_dirty_reset, dim3((unsigned)((reset + 255) / 256)), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)a.g.n_seq * (a.g.cap_cells / a.r);
    if (n > 0)
        hipLaunchKernelGGL(k_detect_dirty, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_update_pooled(const UpdateArgs &a, hipStream_t st) {
    if (a.n_dirty <= 0) return hipSuccess;
    const int grid = (a.n_dirty + 3) / 4;
    hipLaunchKernelGGL(k_update_pooled, dim3(grid), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace qsa
