// qsa_internal.h -- device helpers and launch interfaces shared by the
// libqsa translation units.  Compiled for gfx950 only (64-lane wavefronts).
//
// Every translation unit is built with -ffp-contract=off: the pooled-key and
// decode-score arithmetic must round each multiply and add separately so it
// reproduces the fixed order T bit for bit.  Kernels that may fuse (attention)
// call fmaf explicitly.
#pragma once

#include <type_traits>

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qsa.h"
#include "wave_ops.h"

namespace qsa {

constexpr int kWave = 64;

// Index of the calling wavefront in its workgroup, as a scalar (uniform).
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}
constexpr int kDIdx = 128;   // indexer dim the library implements
constexpr int kHeadDim = 256;
constexpr int kTile = 64;    // blocks per pooled-key tile
constexpr int kQuads = kDIdx / 4;
constexpr int kTileFloats = kTile * kDIdx;
constexpr int kQ8Bytes = 34;
constexpr int kQ8Row = kHeadDim / 32 * kQ8Bytes;  // 272 bytes

// ---------------------------------------------------------------------------
// Phase stamps: a measurement build option (QSA_STAMPS, off by default).
// Thread 0 of a workgroup records the 100 MHz real-time clock at numbered
// points of a kernel; the last slot holds the XCD the workgroup ran on.  Each
// translation unit keeps its own table, read and cleared through
// qsa_stamps_<unit> (exported by stamp builds only).  Without the option the
// macros expand to nothing.
// ---------------------------------------------------------------------------
#ifdef QSA_STAMPS
constexpr int kStampWgs = 4096;
constexpr int kStampSlots = 16;
static __device__ uint64_t g_stamps[kStampWgs][kStampSlots];
__device__ __forceinline__ void stamp_at(int slot) {
    const uint32_t wg = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    if (threadIdx.x == 0 && wg < (uint32_t)kStampWgs) {
        g_stamps[wg][slot] = __builtin_amdgcn_s_memrealtime();
        if (slot == 0) {
            uint32_t xcc;
            asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
            g_stamps[wg][kStampSlots - 1] = xcc;
        }
    }
}
#define QSA_STAMP(slot) ::qsa::stamp_at(slot)
// Held stamps: the clock read into a register now and stored by
// QSA_STAMP_SAVE at the kernel's end, so that no stamp store is outstanding
// at the kernel's barriers (a barrier waits for the workgroup's stores).
__device__ __forceinline__ void stamp_save(int slot, uint64_t t) {
    const uint32_t wg = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    if (threadIdx.x == 0 && wg < (uint32_t)kStampWgs) {
        g_stamps[wg][slot] = t;
        if (slot == 0) {
            uint32_t xcc;
            asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
            g_stamps[wg][kStampSlots - 1] = xcc;
        }
    }
}
// LDS stamps: for points inside device functions; QSA_STAMP_LDS_FLUSH at the
// kernel's end stores every slot written since QSA_STAMP_LDS_BEGIN.
__device__ __forceinline__ uint64_t *stamp_lds_buf() {
    __shared__ uint64_t buf[kStampSlots];
    return buf;
}
__device__ __forceinline__ void stamp_lds_begin() {
    if (threadIdx.x == 0)
        for (int k = 0; k < kStampSlots; ++k) stamp_lds_buf()[k] = 0;
}
__device__ __forceinline__ void stamp_lds(int slot) {
    if (threadIdx.x == 0) stamp_lds_buf()[slot] = __builtin_amdgcn_s_memrealtime();
}
__device__ __forceinline__ void stamp_lds_flush() {
    const uint32_t wg = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    if (threadIdx.x == 0 && wg < (uint32_t)kStampWgs)
        for (int k = 0; k < kStampSlots - 1; ++k)
            if (stamp_lds_buf()[k]) g_stamps[wg][k] = stamp_lds_buf()[k];
}
#define QSA_STAMP_LDS_BEGIN() ::qsa::stamp_lds_begin()
#define QSA_STAMP_LDS(slot) ::qsa::stamp_lds(slot)
#define QSA_STAMP_LDS_FLUSH() ::qsa::stamp_lds_flush()
#define QSA_STAMP_HOLD(name) const uint64_t name = __builtin_amdgcn_s_memrealtime()
#define QSA_STAMP_SAVE(slot, name) ::qsa::stamp_save(slot, name)
#define QSA_STAMP_READER(unit)                                                            \
    extern "C" int qsa_stamps_##unit(void *dst, int clear) {                              \
        hipError_t e = hipSuccess;                                                        \
        if (dst)                                                                          \
            e = hipMemcpyFromSymbol(dst, HIP_SYMBOL(::qsa::g_stamps),                     \
                                    sizeof(::qsa::g_stamps));                             \
        if (e == hipSuccess && clear) {                                                   \
            static uint64_t zero[::qsa::kStampWgs][::qsa::kStampSlots];                   \
            e = hipMemcpyToSymbol(HIP_SYMBOL(::qsa::g_stamps), zero, sizeof(zero));       \
        }                                                                                 \
        return (int)e;                                                                    \
    }
#else
#define QSA_STAMP(slot) ((void)0)
#define QSA_STAMP_HOLD(name) ((void)0)
#define QSA_STAMP_LDS_BEGIN() ((void)0)
#define QSA_STAMP_LDS(slot) ((void)0)
#define QSA_STAMP_LDS_FLUSH() ((void)0)
#define QSA_STAMP_SAVE(slot, name) ((void)0)
#define QSA_STAMP_READER(unit)
#endif

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
__device__ __forceinline__ void rope_cs_omega(double omega, int64_t pos, float &c, float &s) {
    const double phi = (double)pos * omega;
    double sd, cd;
    sincos(phi, &sd, &cd);
    c = (float)cd;
    s = (float)sd;
}
__device__ __forceinline__ void rope_cs(const RopeTable &rt, int t, int64_t pos, float &c,
                                        float &s) {
    rope_cs_omega(rt.omega[t], pos, c, s);
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

// query_blocks in two steps, for kernels that request the query's fields
// before their other loads and resolve them later: QueryFields::load reads
// the sequence and position, then the sequence's cell count at a clamped
// index (no check between the loads); blocks() gives what query_blocks
// returns, limit() that capped at nb_max.
struct QueryFields {
    int s;
    int64_t p;
    int32_t ncell;
    int n_seq;
    int64_t cap_cells;
    int r;
    int64_t nb_max;
    __device__ __forceinline__ void load(const int32_t *q_seq, const int32_t *q_pos,
                                         const int32_t *n_cells, int i) {
        s = q_seq[i];
        p = q_pos[i];
        ncell = n_cells[min(max(s, 0), n_seq - 1)];
    }
    __device__ __forceinline__ int64_t blocks(bool &valid) const {
        valid = false;
        if (s < 0 || s >= n_seq || p < 0) return 0;
        int64_t n = ncell;
        if (n > cap_cells) n = cap_cells;
        if (p >= n) return 0;
        valid = true;
        return (p + 1) / r;
    }
    __device__ __forceinline__ int64_t limit() const {
        bool v;
        const int64_t nc = blocks(v);
        return nc < nb_max ? nc : nb_max;
    }
};

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

// Roped query element pair (t, t+64) of a query at position p, fp32.
// Roped pair (t, t+64) from the two values and omega_t.
__device__ __forceinline__ void rope_pair_omega(float xl, float xh, double omega, int64_t p,
                                                float &lo, float &hi) {
    float c, s;
    rope_cs_omega(omega, p, c, s);
    const float lc = xl * c, hs = xh * s;
    const float hc = xh * c, ls = xl * s;
    lo = lc - hs;
    hi = hc + ls;
}
__device__ __forceinline__ void rope_query_pair(const float *q, int t, int64_t p,
                                                const RopeTable &rt, float &lo, float &hi) {
    rope_pair_omega(q[t], q[t + 64], rt.omega[t], p, lo, hi);
}

// Pooled key of block b of sequence s, whose first m = min(r, n - b*r) cells
// are present (n > b*r): mean of the m per-cell keys (left-to-right fp32 sum,
// one divide), RMS-normed (mean of squares in order T, 1/sqrt(ms + eps)
// correctly rounded, optional weight gamma), roped at position b*r.  All 64
// lanes of a wavefront call it together; lane t gets dims t and t + 64 (its
// split-half RoPE pair).  The first level of T pairs dims (t, t+64) in-lane;
// the rest is an xor butterfly whose lane-0 value is exactly the
// stride-halving tree (xor h pairs lane t < h with t + h).
struct SeqGeom {
    int32_t n_seq;
    int64_t cap_cells;
    const int32_t *n_cells;
    const int32_t *rows;  // optional cell table [n_seq][cap_cells]
    int64_t n_rows;
};

// Row of position p of sequence s in the per-cell arrays (kidx, K, V): the
// cell table's entry at = s*cap_cells + p (out-of-range entries read row 0),
// else at itself.
__device__ __forceinline__ int64_t cell_row_at(const SeqGeom &g, int64_t at) {
    if (!g.rows) return at;
    const int32_t r = g.rows[at];
    return (r >= 0 && r < g.n_rows) ? r : 0;
}
__device__ __forceinline__ int64_t cell_row(const SeqGeom &g, int s, int64_t p) {
    return cell_row_at(g, (int64_t)s * g.cap_cells + p);
}

// Per-cell indexer keys: float32, or bfloat16 bits widened exactly to fp32.
struct KidxRef {
    const void *p;
    int32_t bf16;
};

template <bool BF16>
__device__ __forceinline__ float kidx_value(const void *p, int64_t i) {
    if constexpr (BF16)
        return __uint_as_float((uint32_t)static_cast<const uint16_t *>(p)[i] << 16);
    else
        return static_cast<const float *>(p)[i];
}

__device__ __forceinline__ void pooled_key_lane(KidxRef kidx, const SeqGeom &g, int s,
                                                int64_t b, int64_t n, int r, float eps,
                                                const float *gamma, const RopeTable &rt,
                                                int lane, float &out_lo, float &out_hi) {
    const int64_t first = b * r;
    const int m = (int)((n - first) < r ? (n - first) : r);
    float lo, hi;
    auto cell_sum = [&](auto bf16) {
        constexpr bool BF = decltype(bf16)::value;
        const int64_t x0 = cell_row(g, s, first) * kDIdx;
        lo = kidx_value<BF>(kidx.p, x0 + lane);
        hi = kidx_value<BF>(kidx.p, x0 + lane + 64);
        for (int j = 1; j < m; ++j) {
            const int64_t x = cell_row(g, s, first + j) * kDIdx;
            lo = lo + kidx_value<BF>(kidx.p, x + lane);
            hi = hi + kidx_value<BF>(kidx.p, x + lane + 64);
        }
    };
    if (kidx.bf16)
        cell_sum(std::true_type{});
    else
        cell_sum(std::false_type{});
    const float fm = (float)m;
    lo = lo / fm;
    hi = hi / fm;
    const float plo = lo * lo;
    const float phi2 = hi * hi;
    float v = plo + phi2;
    v = v + xor_lane_f<32>(v);
    v = v + xor_lane_f<16>(v);
    v = v + xor_lane_f<8>(v);
    v = v + xor_lane_f<4>(v);
    v = v + xor_lane_f<2>(v);
    v = v + xor_lane_f<1>(v);
    v = __uint_as_float(lane_value(__float_as_uint(v), 0));
    const float ms = v / (float)kDIdx;
    const float inv = 1.0f / sqrtf(ms + eps);
    lo = lo * inv;
    hi = hi * inv;
    if (gamma) {
        lo = lo * gamma[lane];
        hi = hi * gamma[lane + 64];
    }
    float c, sn;
    rope_cs(rt, lane, first, c, sn);
    const float lc = lo * c, hs = hi * sn;
    const float hc = hi * c, ls = lo * sn;
    out_lo = lc - hs;
    out_hi = hc + ls;
}

// Store a pooled key (lane t: dims t, t+64) into the tiled fp32 cache and, if
// given, the row-major bf16 copy.
__device__ __forceinline__ void store_pooled_lane(float *pooled, uint16_t *pooled_bf16,
                                                  int64_t cap_blocks, int s, int64_t b, int lane,
                                                  float out_lo, float out_hi) {
    float *tile = pooled + ((int64_t)s * (cap_blocks / kTile) + b / kTile) * kTileFloats;
    const int col = (int)(b % kTile) * 4;
    tile[(lane >> 2) * (kTile * 4) + col + (lane & 3)] = out_lo;
    tile[((lane + 64) >> 2) * (kTile * 4) + col + (lane & 3)] = out_hi;
    if (pooled_bf16) {
        uint16_t *row = pooled_bf16 + ((int64_t)s * cap_blocks + b) * kDIdx;
        row[lane] = bf16_rne(out_lo);
        row[lane + 64] = bf16_rne(out_hi);
    }
}

// ---------------------------------------------------------------------------
// Launch interfaces (host side, one per kernel family)
// ---------------------------------------------------------------------------

struct UpdateArgs {
    SeqGeom g;
    KidxRef kidx;
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

// Decode indexer step (score.hip): pooled-key update of the dirty blocks,
// block scores, and the exact top-k, in two launches.  The first scores every
// block and leaves, per group of 64 blocks, its 4 best keys and the largest
// key it dropped; it also writes the dirty blocks (extra workgroups) while
// any scoring workgroup that holds a dirty block recomputes it in registers,
// so no ordering between the two is needed.  The second selects from those
// candidates (a selection kernel, or each attention workgroup).
struct DecodeIdxArgs {
    ScoreArgs s;
    float *pooled_w;        // same buffer as s.pooled, written by the update part
    uint16_t *pooled_bf16;  // optional bf16 copy, written by the update part
    KidxRef kidx;
    const int32_t *dirty;
    int32_t n_dirty;
    float eps;
    const float *gamma;
    int32_t top_k;
    int32_t *sel_blocks;
    int32_t *sel_cells;
    int32_t *n_sel;
    uint64_t *cand;  // [n_q][4*n_wg][n_cand]: largest keys of each 64-block group
    uint64_t *drop;  // [n_q][4*n_wg]: largest key each group dropped
    int32_t n_wg;
    int32_t n_cand;  // keys kept per group (see cand_per_group)
    int32_t wide_cand;  // the call's queries overflow the fused grid: more keys per group
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

// Structural dirty detection (pooled.hip).
struct DirtyArgs {
    SeqGeom g;
    int32_t r;
    int32_t *snap;      // [n_seq][cap_blocks][r + 1]: member count, then member rows
    int32_t *dirty;     // [max_dirty][2] (seq, block), (-1, -1) padded
    int32_t max_dirty;
    uint32_t *n_found;  // changed blocks found (may exceed max_dirty)
};
hipError_t launch_detect_dirty(const DirtyArgs &a, hipStream_t st);
hipError_t launch_score_f32(const ScoreArgs &a, hipStream_t st);
hipError_t launch_score_bf16_ws(const ScoreArgs &a, uint16_t *qr_bf16, hipStream_t st);
hipError_t launch_select(const SelectArgs &a, hipStream_t st);
constexpr int kFusedMaxBlocks = 1 << 17;  // fused score+select handles nb_max up to this
// decode selection fused into attention (256-thread workgroups holding the
// candidates in registers) handles nb_max up to this: 262144-cell contexts
constexpr int kSelAttnMaxBlocks = 1 << 16;

// Whether the fused decode selection + attention grid of a call -- one
// 512-thread workgroup per (query, run of 32 list cells, pair of 2-head
// groups) -- fits the chip in one round (512 workgroups, two per CU).  It
// then runs; otherwise the selection runs once per query and the attention
// over the lists.  The indexer calls use the same rule to choose how many
// candidates a group keeps.
__host__ __device__ inline bool fused_decode_fits(int n_q, int ld_cells, int n_head,
                                                  int n_head_kv) {
    const int hpk = n_head / n_head_kv;
    const int n_set = (n_head / (hpk % 2 == 0 ? 2 : 1) + 1) / 2;
    const int n_runs = (ld_cells + 31) / 32;
    return (int64_t)n_q * n_runs * n_set <= 512;
}
size_t fused_select_ws_bytes(int n_q, int nb_max);
// part 1: update + scores + candidates; part 2: selection from candidates
hipError_t launch_decode_candidates(DecodeIdxArgs f, void *ws, hipStream_t st);
hipError_t launch_decode_select(DecodeIdxArgs f, void *ws, hipStream_t st);
// Prefill indexer (prefill.hip): MFMA scores, then per query the exact top-B
// with exact rescoring of the blocks near the cut.
struct PrefillWs {
    float *smax;      // [n_q][4*n_grp] largest MFMA score of each causal 16-block subgroup
    float *thr;       // [n_q] filter threshold: tau - 2*Delta rounded down (-inf: all causal)
    uint64_t *mask;   // [n_q][n_grp] blocks of each 64-block group with MFMA score >= thr
    uint16_t *qr;     // [n_q][128] roped queries, bf16
    float *delta;     // [n_q] bound on |MFMA score - T score|
    int2 *qmeta;      // [n_q] (sequence, -1 if the query is invalid; causal blocks, at most nb_max)
    int32_t n_grp;
};
size_t prefill_ws_bytes(int n_q, int nb_max);
hipError_t launch_score_select_prefill(const ScoreArgs &a, const float *gamma, void *ws,
                                       int top_k, int32_t *sel_blocks, int32_t *sel_cells,
                                       int32_t *n_sel, const UpdateArgs &upd, hipStream_t st);
size_t attn_decode_ws_bytes(int n_q, int n_head, int ld_cells);
hipError_t launch_attn_decode(const AttnArgs &a, hipStream_t st);
size_t attn_prefill_ws_bytes(int n_q, int n_head, int ld_cells);
hipError_t launch_attn_prefill(const AttnArgs &a, hipStream_t st);

// Decode tokens in groups over the union of their cell lists
// (attn_prefill.hip).  Workspace: the union rows and token bits per group,
// the union sizes, then the per-run partial states of every (token, head).
constexpr int kUPartStride = kHeadDim + 2;  // o[256], m, l
struct UnionArgs {
    int32_t t_group;   // tokens per group
    int32_t n_groups;
    int32_t cap;       // union entries per group: t_group * ld_cells
    int32_t n_runs;    // attention runs per (group, KV head): ceil(cap / run length)
    int32_t *urow;     // [n_groups][cap] K/V cell rows (s * cap_cells + cell), ascending
    uint8_t *umask;    // [n_groups][cap] bit t: token t of the group holds the row
    int32_t *n_union;  // [n_groups]
    float *part;       // [n_groups][n_head_kv][n_runs][t_group * hpk][kUPartStride]
};
size_t union_layout(char *base, int n_q, int t_group, int n_head, int n_head_kv, int ld_cells,
                    UnionArgs *u);
size_t union_ws_bytes(int n_q, int t_group, int n_head, int n_head_kv, int ld_cells);
hipError_t launch_attn_decode_union(const AttnArgs &a, int t_group, hipStream_t st);
constexpr int kUnionMaxTokens = 8;
constexpr int kUnionMaxEntries = 16448;  // 8 tokens of top_k + r - 1 = 2056 cells

// Memory-traffic probes (probe.hip, attn_prefill.hip): loads only, each
// wavefront's XOR folded into sink[wavefront % n_sink] -- a plain
// read-modify-write when the sink has a word per wavefront (the sole writer),
// else an atomic (many wavefronts on a few words serialise at L2, which a
// probe must not time).  Called by one lane per wavefront.
__device__ __forceinline__ void fold_sink(uint32_t *sink, int n_sink, uint32_t v) {
    const uint32_t wpg = blockDim.x / kWave;
    const uint32_t n_waves = gridDim.x * gridDim.y * gridDim.z * wpg;
    const uint32_t id = blockIdx.x * wpg + threadIdx.x / kWave;  // (1-D grids)
    if ((uint32_t)n_sink >= n_waves)
        sink[id] ^= v;
    else
        atomicXor(&sink[id % (uint32_t)n_sink], v);
}
hipError_t launch_probe_read(const void *src, size_t n_bytes, bool nontemporal, uint32_t *sink,
                             int n_sink, hipStream_t st);
hipError_t launch_probe_gather_prefill(const AttnArgs &a, uint32_t *sink, int n_sink,
                                       hipStream_t st);
// decode selection (from the candidates in ws_idx) fused with attention; the
// attention workspace is the one launch_attn_decode uses
hipError_t launch_select_attn_decode(DecodeIdxArgs f, void *ws_idx, const AttnArgs &a,
                                     hipStream_t st);

}  // namespace qsa
