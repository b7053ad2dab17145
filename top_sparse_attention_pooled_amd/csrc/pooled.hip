// pooled.hip -- the persistent pooled block-key cache (llama.cpp issue #28734,
// fix summary, "lever2": pooled + normed + roped block keys kept in their own
// buffer, only dirtied blocks recomputed; "lever2b": block membership resolved
// on the device, here simply cells b*r .. b*r+r-1 of the block's sequence).
//
// One wavefront per dirty block.  Lane t owns the split-half RoPE pair
// (t, t+64), so the mean-pool, the RMS norm and the rotation all stay in
// registers; the mean of squares is the fixed order T: the first level
// (t, t+64) is in-lane, the rest an xor butterfly whose lane-0 value is
// exactly the stride-halving tree (xor h pairs lane t < h with t + h).
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
    const int64_t first = (int64_t)b * a.r;
    if (first >= n) return;
    const int m = (int)((n - first) < a.r ? (n - first) : a.r);

    // mean over the present cells: left-to-right sum, one divide
    const float *x = a.kidx + ((int64_t)s * a.g.cap_cells + first) * kDIdx;
    float lo = x[lane];
    float hi = x[lane + 64];
    for (int j = 1; j < m; ++j) {
        lo = lo + x[j * kDIdx + lane];
        hi = hi + x[j * kDIdx + lane + 64];
    }
    const float fm = (float)m;
    lo = lo / fm;
    hi = hi / fm;

    // mean of squares in order T, then 1/sqrt(ms + eps), correctly rounded
    const float plo = lo * lo;
    const float phi2 = hi * hi;
    float v = plo + phi2;
#pragma unroll
    for (int h = 32; h >= 1; h >>= 1) v = v + __shfl_xor(v, h, kWave);
    v = __shfl(v, 0, kWave);
    const float ms = v / (float)kDIdx;
    const float inv = 1.0f / sqrtf(ms + a.eps);
    lo = lo * inv;
    hi = hi * inv;
    if (a.gamma) {
        lo = lo * a.gamma[lane];
        hi = hi * a.gamma[lane + 64];
    }

    // RoPE at the block position b*r
    float c, sn;
    rope_cs(a.rope, lane, first, c, sn);
    const float lc = lo * c, hs = hi * sn;
    const float hc = hi * c, ls = lo * sn;
    const float out_lo = lc - hs;
    const float out_hi = hc + ls;

    float *tile = a.pooled + ((int64_t)s * (cap_blocks / kTile) + b / kTile) * kTileFloats;
    const int col = (b % kTile) * 4;
    tile[(lane >> 2) * (kTile * 4) + col + (lane & 3)] = out_lo;
    tile[((lane + 64) >> 2) * (kTile * 4) + col + (lane & 3)] = out_hi;
    if (a.pooled_bf16) {
        uint16_t *row = a.pooled_bf16 + ((int64_t)s * cap_blocks + b) * kDIdx;
        row[lane] = bf16_rne(out_lo);
        row[lane + 64] = bf16_rne(out_hi);
    }
}

}  // namespace

hipError_t launch_update_pooled(const UpdateArgs &a, hipStream_t st) {
    if (a.n_dirty <= 0) return hipSuccess;
    const int grid = (a.n_dirty + 3) / 4;
    hipLaunchKernelGGL(k_update_pooled, dim3(grid), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace qsa
