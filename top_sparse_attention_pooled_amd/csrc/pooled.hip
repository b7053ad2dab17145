// pooled.hip -- the persistent pooled block-key cache (llama.cpp issue #28734,
// fix summary, "lever2": pooled + normed + roped block keys kept in their own
// buffer, only dirtied blocks recomputed; "lever2b": block membership resolved
// on the device, here simply cells b*r .. b*r+r-1 of the block's sequence).
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
    pooled_key_lane(a.kidx, a.g.cap_cells, s, b, n, a.r, a.eps, a.gamma, a.rope, lane, lo, hi);
    store_pooled_lane(a.pooled, a.pooled_bf16, cap_blocks, s, b, lane, lo, hi);
}

}  // namespace

hipError_t launch_update_pooled(const UpdateArgs &a, hipStream_t st) {
    if (a.n_dirty <= 0) return hipSuccess;
    const int grid = (a.n_dirty + 3) / 4;
    hipLaunchKernelGGL(k_update_pooled, dim3(grid), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace qsa
