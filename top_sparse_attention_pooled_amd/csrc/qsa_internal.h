// qsa_internal.h -- device helpers and launch interfaces shared by the
// libqsa translation units.  Compiled for gfx950 only (64-lane wavefronts).
//
// Every translation unit is built with -ffp-contract=off: the pooled-key and
// decode-score arithmetic must round each multiply and add separately so it
// reproduces the fixed order T bit for bit.  Kernels that may fuse (attention)
// call fmaf explicitly.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qsa.h"

namespace qsa {

constexpr int kWave = 64;
constexpr int kDIdx = 128;   // indexer dim this build implements
constexpr int kHeadDim = 256;
constexpr int kTile = 64;    // blocks per pooled-key tile
constexpr int kQuads = kDIdx / 4;
constexpr int kTileFloats = kTile * kDIdx;
constexpr int kQ8Bytes = 34;
constexpr int kQ8Row = kHeadDim / 32 * kQ8Bytes;  // 272 bytes

// ---------------------------------------------------------------------------
// Scalar helpers
// ---------------------------------------------------------------------------

// RoPE inverse frequencies omega_t = theta^(-2t/d), t < d/2, in fp64.  The
// table is formed on the host (rope_table() in api.hip) and passed by value
// in the kernel arguments; see there for how it is evaluated.
struct RopeTable {
    double omega[kDIdx / 2];
};

// cos and sin of pos * omega_t: the angle and both functions in fp64, each
// rounded once to fp32.
__device__ __forceinline__ void rope_cs(const RopeTable &rt, int t, int64_t pos, float &c,
                                        float &s) {
    const double phi = (double)pos * rt.omega[t];
    double sd, cd;
    sincos(phi, &sd, &cd);
    c = (float)cd;
    s = (float)sd;
}

// Order-preserving 32-bit key of a finite fp32 score (-0 maps like +0):
// a larger key is a larger score.
__device__ __forceinline__ uint32_t score_key(float s) {
    uint32_t u = __float_as_uint(s);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ bool finite_f32(float s) {
    return (__float_as_uint(s) & 0x7f800000u) != 0x7f800000u;
}

// fp32 -> bf16 bits, round to nearest even.
__device__ __forceinline__ uint16_t bf16_rne(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(((uint32_t)h) << 16);
}

// Validity of query i; returns the number of complete visible blocks
// (0 for an invalid query) and the sequence / position.
__device__ __forceinline__ int64_t query_blocks(const int32_t *q_seq, const int32_t *q_pos,
                                                int i, int n_seq, int64_t cap_cells,
                                                const int32_t *n_cells, int r, int &s,
                                                int64_t &p, bool &valid) {
    s = q_seq[i];
    p = q_pos[i];
    valid = false;
    if (s < 0 || s >= n_seq || p < 0) return 0;
    int64_t n = n_cells[s];
    if (n > cap_cells) n = cap_cells;
    if (p >= n) return 0;
    valid = true;
    return (p + 1) / r;
}

// ---------------------------------------------------------------------------
// Launch interfaces (host side, one per kernel family)
// ---------------------------------------------------------------------------

struct SeqGeom {
    int32_t n_seq;
    int64_t cap_cells;
    const int32_t *n_cells;
};

struct UpdateArgs {
    SeqGeom g;
    const float *kidx;
    const int32_t *dirty;
    int32_t n_dirty;
    float *pooled;
    uint16_t *pooled_bf16;
    int32_t r;
    float eps;
    const float *gamma;
    RopeTable rope;
};

struct ScoreArgs {
    SeqGeom g;
    const float *q_idx;
    const int32_t *q_seq;
    const int32_t *q_pos;
    int32_t n_q;
    const float *pooled;
    const uint16_t *pooled_bf16;
    int32_t nb_max;
    float *scores;
    int64_t ld;
    int32_t r;
    RopeTable rope;
};

// Fused decode scoring + selection (score.hip).  Per query, each workgroup of
// 256 blocks leaves its 16 best keys, the largest key it dropped (0 = none)
// and its count of finite candidates in the workspace; the last workgroup
// to arrive selects.
struct FusedSelectArgs {
    ScoreArgs s;
    int32_t top_k;
    int32_t *sel_blocks;
    int32_t *sel_cells;
    int32_t *n_sel;
    uint32_t *arrive;  // [n_q] arrival counters, zero between launches
    uint64_t *cand;    // [n_q][n_wg][16]
    uint64_t *drop;    // [n_q][n_wg]
    uint32_t *fin;     // [n_q][n_wg]
    int32_t n_wg;
};

struct SelectArgs {
    SeqGeom g;
    const float *scores;
    int64_t ld;
    const int32_t *q_seq;
    const int32_t *q_pos;
    int32_t n_q;
    int32_t nb_max;
    int32_t r;
    int32_t top_k;
    int32_t *sel_blocks;
    int32_t *sel_cells;
    int32_t *n_sel;
};

struct AttnArgs {
    SeqGeom g;
    const float *q;
    const int32_t *q_seq;
    int32_t n_q;
    int32_t n_head;
    int32_t n_head_kv;
    int32_t kv_type;
    const void *k;
    const void *v;
    const int32_t *sel_cells;
    const int32_t *n_sel;
    int32_t ld_cells;
    float scale;
    float *out;
    float *ws;
    size_t ws_bytes;
};

hipError_t launch_update_pooled(const UpdateArgs &a, hipStream_t st);
hipError_t launch_score_f32(const ScoreArgs &a, hipStream_t st);
hipError_t launch_score_bf16_ws(const ScoreArgs &a, uint16_t *qr_bf16, hipStream_t st);
hipError_t launch_select(const SelectArgs &a, hipStream_t st);
constexpr int kFusedMaxBlocks = 1 << 17;  // fused score+select handles nb_max up to this
size_t fused_select_ws_bytes(int n_q, int nb_max);
hipError_t launch_score_select_f32(const ScoreArgs &s, int32_t top_k, int32_t *sel_blocks,
                                   int32_t *sel_cells, int32_t *n_sel, void *ws,
                                   hipStream_t st);
size_t attn_decode_ws_bytes(int n_q, int n_head, int ld_cells);
hipError_t launch_attn_decode(const AttnArgs &a, hipStream_t st);
size_t attn_prefill_ws_bytes(int n_q, int n_head, int ld_cells);
hipError_t launch_attn_prefill(const AttnArgs &a, hipStream_t st);

}  // namespace qsa
