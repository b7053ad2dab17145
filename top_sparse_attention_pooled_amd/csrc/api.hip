// api.hip -- the extern "C" boundary of libqsa (declared in include/qsa.h):
// host-side validation, workspace sizing and dispatch to the kernels.  No
// call allocates, frees or synchronises; errors are returned before anything
// is enqueued, with a message kept per thread.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "qsa_internal.h"
#include "../../include/qsa_probe.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return QSA_OK;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_dims(const qsa_dims *d) {
    if (!d) return fail(QSA_EINVAL, "dims is NULL");
    if (d->head_dim != qsa::kHeadDim)
        return fail(QSA_ENOTSUP, "head_dim %d not supported (256 only)", d->head_dim);
    if (d->d_idx != qsa::kDIdx)
        return fail(QSA_ENOTSUP, "d_idx %d not supported (128 only)", d->d_idx);
    if (d->n_head <= 0 || d->n_head_kv <= 0 || d->n_head % d->n_head_kv)
        return fail(QSA_EINVAL, "n_head %d must be a positive multiple of n_head_kv %d",
                    d->n_head, d->n_head_kv);
    const int G = d->n_head / d->n_head_kv;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(QSA_ENOTSUP, "n_head/n_head_kv = %d not in {1,2,4,8}", G);
    if (d->r < 1 || d->r > 16) return fail(QSA_ENOTSUP, "r = %d outside 1..16", d->r);
    if (d->top_k < d->r || d->top_k % d->r)
        return fail(QSA_EINVAL, "top_k %d must be a positive multiple of r %d", d->top_k, d->r);
    if (d->top_k / d->r > 4096)
        return fail(QSA_ENOTSUP, "top_k/r = %d above 4096", d->top_k / d->r);
    if (d->kv_type != QSA_KV_F32 && d->kv_type != QSA_KV_Q8_0 && d->kv_type != QSA_KV_F16)
        return fail(QSA_EINVAL, "kv_type %d unknown", d->kv_type);
    if (d->kidx_type != QSA_KIDX_F32 && d->kidx_type != QSA_KIDX_BF16)
        return fail(QSA_EINVAL, "kidx_type %d unknown", d->kidx_type);
    if (!(d->rope_theta > 1.0f)) return fail(QSA_EINVAL, "rope_theta must be > 1");
    if (!(d->rms_eps >= 0.0f)) return fail(QSA_EINVAL, "rms_eps must be >= 0");
    if (d->idx_norm_w_dev && !aligned(d->idx_norm_w_dev, 4))
        return fail(QSA_EINVAL, "idx_norm_w_dev misaligned");
    return QSA_OK;
}

int check_seqs(const qsa_dims *d, const qsa_seqs *s) {
    if (!s) return fail(QSA_EINVAL, "seqs is NULL");
    if (s->n_seq <= 0) return fail(QSA_EINVAL, "n_seq must be positive");
    if (s->cap_cells <= 0 || s->cap_cells % ((int64_t)qsa::kTile * d->r))
        return fail(QSA_EINVAL, "cap_cells %lld must be a positive multiple of 64*r",
                    (long long)s->cap_cells);
    if (s->cap_cells > ((int64_t)1 << 31) - 1)
        return fail(QSA_ENOTSUP, "cap_cells above 2^31-1");
    if (!s->n_cells_dev || !aligned(s->n_cells_dev, 4))
        return fail(QSA_EINVAL, "n_cells_dev NULL or misaligned");
    if (s->cell_rows_dev) {
        if (!aligned(s->cell_rows_dev, 4)) return fail(QSA_EINVAL, "cell_rows_dev misaligned");
        if (s->n_rows <= 0 || s->n_rows > ((int64_t)1 << 31) - 1)
            return fail(QSA_EINVAL, "n_rows %lld outside 1 .. 2^31-1 with a cell table",
                        (long long)s->n_rows);
    }
    return QSA_OK;
}

qsa::SeqGeom geom(const qsa_seqs *s) {
    return {s->n_seq, s->cap_cells, s->n_cells_dev, s->cell_rows_dev,
            s->cell_rows_dev ? s->n_rows : 0};
}

// Rows of the per-cell arrays (kidx, K, V).
int64_t cell_rows(const qsa_seqs *s) {
    return s->cell_rows_dev ? s->n_rows : (int64_t)s->n_seq * s->cap_cells;
}

size_t kidx_align(const qsa_dims *d) { return d->kidx_type == QSA_KIDX_BF16 ? 2 : 4; }
qsa::KidxRef kidx_ref(const qsa_dims *d, const void *kidx) {
    return {kidx, d->kidx_type == QSA_KIDX_BF16 ? 1 : 0};
}

// RoPE inverse frequencies omega_t = theta^(-2t/d) for d = 128, in fp64.
// With d/2 = 2^6, theta^(-2t/d) = theta^(-t/64) is the product over the set
// bits k of t of theta^(-1/2^(6-k)), and theta^(1/2^j) is j nested square
// roots of theta.  Only correctly rounded IEEE operations are used (sqrt,
// divide, multiply, in ascending k), so every conforming machine gets the
// same bits; the kernels then form the angles pos * omega_t themselves.
qsa::RopeTable rope_table(float theta_f) {
    qsa::RopeTable t;
    double root[7];
    root[0] = (double)theta_f;
    for (int j = 1; j <= 6; ++j) root[j] = sqrt(root[j - 1]);
    for (int i = 0; i < qsa::kDIdx / 2; ++i) {
        double w = 1.0;
        for (int k = 0; k < 6; ++k)
            if ((i >> k) & 1) w = w * (1.0 / root[6 - k]);
        t.omega[i] = w;
    }
    return t;
}

int check_queries(const int32_t *q_seq, const int32_t *q_pos, int32_t n_q, bool need_pos) {
    if (n_q < 0) return fail(QSA_EINVAL, "n_q negative");
    if (n_q > 65535) return fail(QSA_ENOTSUP, "n_q above 65535");
    if (n_q == 0) return QSA_OK;
    if (!q_seq || !aligned(q_seq, 4)) return fail(QSA_EINVAL, "q_seq_dev NULL or misaligned");
    if (need_pos && (!q_pos || !aligned(q_pos, 4)))
        return fail(QSA_EINVAL, "q_pos_dev NULL or misaligned");
    return QSA_OK;
}

int launched(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(QSA_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

// Scratch of qsa_sparse_attn_decode_noalloc (the attention's partial states),
// a file-scope device array: every GPU the library runs on holds its own copy
// until the process ends.  Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the symbol): the device
// address of each GPU's copy comes from hipGetSymbolAddress, taken once per
// device with that device current, and is kept here.
constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The current device's scratch address, or an error code.
int scratch_of_current_device(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(QSA_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(QSA_ENOTSUP, "device %d beyond the %d the scratch table holds", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(QSA_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return QSA_OK;
}

}  // namespace

extern "C" {

int qsa_version(void) { return QSA_ABI_VERSION; }

const char *qsa_last_error(void) { return g_err; }

int qsa_workspace_size(const qsa_dims *dims, int32_t op, int32_t n_q, int32_t nb_max,
                       size_t *bytes) {
    (void)nb_max;
    int rc = check_dims(dims);
    if (rc) return rc;
    if (!bytes) return fail(QSA_EINVAL, "bytes is NULL");
    if (n_q < 0) return fail(QSA_EINVAL, "n_q negative");
    const int ld_cells = dims->top_k + dims->r - 1;
    switch (op) {
        case QSA_OP_SELECT: *bytes = 0; break;
        case QSA_OP_ATTN_DECODE:
            *bytes = qsa::attn_decode_ws_bytes(n_q, dims->n_head, ld_cells);
            break;
        case QSA_OP_ATTN_PREFILL:
            *bytes = qsa::attn_prefill_ws_bytes(n_q, dims->n_head, ld_cells);
            break;
        case QSA_OP_SCORE_BF16: *bytes = (size_t)n_q * qsa::kDIdx * sizeof(uint16_t); break;
        case QSA_OP_SCORE_SELECT:
            if (nb_max < 0) return fail(QSA_EINVAL, "nb_max negative");
            *bytes = qsa::fused_select_ws_bytes(n_q, nb_max);
            break;
        case QSA_OP_SCORE_SELECT_PREFILL:
            if (nb_max < 0) return fail(QSA_EINVAL, "nb_max negative");
            *bytes = qsa::prefill_ws_bytes(n_q, nb_max);
            break;
        case QSA_OP_ATTN_DECODE_UNION:  // nb_max carries t_group
            if (nb_max < 1 || nb_max > qsa::kUnionMaxTokens)
                return fail(QSA_EINVAL, "t_group %d outside 1..%d", nb_max, qsa::kUnionMaxTokens);
            *bytes = qsa::union_ws_bytes(n_q, nb_max, dims->n_head, dims->n_head_kv, ld_cells);
            break;
        default: return fail(QSA_EINVAL, "unknown op %d", op);
    }
    return ok();
}

int qsa_update_pooled_keys(const qsa_dims *dims, const qsa_seqs *seqs, const void *kidx_dev,
                           const int32_t *dirty_dev, int32_t n_dirty, float *pooled_dev,
                           uint16_t *pooled_bf16_dev, void *stream) {
    int rc = check_dims(dims);
    if (!rc) rc = check_seqs(dims, seqs);
    if (rc) return rc;
    if (n_dirty < 0) return fail(QSA_EINVAL, "n_dirty negative");
    if (n_dirty == 0) return ok();
    if (!kidx_dev || !aligned(kidx_dev, kidx_align(dims)))
        return fail(QSA_EINVAL, "kidx_dev NULL or misaligned");
    if (!dirty_dev || !aligned(dirty_dev, 4)) return fail(QSA_EINVAL, "dirty_dev NULL or misaligned");
    if (!pooled_dev || !aligned(pooled_dev, 16))
        return fail(QSA_EINVAL, "pooled_dev NULL or not 16-byte aligned");
    if (pooled_bf16_dev && !aligned(pooled_bf16_dev, 16))
        return fail(QSA_EINVAL, "pooled_bf16_dev not 16-byte aligned");
    qsa::UpdateArgs a{geom(seqs), kidx_ref(dims, kidx_dev), dirty_dev, n_dirty,
                      pooled_dev, pooled_bf16_dev, dims->r, dims->rms_eps,
                      dims->idx_norm_w_dev, rope_table(dims->rope_theta)};
    return launched(qsa::launch_update_pooled(a, (hipStream_t)stream), "update_pooled_keys");
}

int qsa_detect_dirty_blocks(const qsa_dims *dims, const qsa_seqs *seqs, int32_t *snapshot_dev,
                            int32_t *dirty_dev, int32_t max_dirty, uint32_t *n_found_dev,
                            void *stream) {
    int rc = check_dims(dims);
    if (!rc) rc = check_seqs(dims, seqs);
    if (rc) return rc;
    if (max_dirty < 0) return fail(QSA_EINVAL, "max_dirty negative");
    if (!snapshot_dev || !aligned(snapshot_dev, 4))
        return fail(QSA_EINVAL, "snapshot_dev NULL or misaligned");
    if ((max_dirty > 0 && (!dirty_dev || !aligned(dirty_dev, 4))) || !n_found_dev ||
        !aligned(n_found_dev, 4))
        return fail(QSA_EINVAL, "dirty_dev/n_found_dev NULL or misaligned");
    qsa::DirtyArgs a{geom(seqs), dims->r, snapshot_dev, dirty_dev, max_dirty, n_found_dev};
    return launched(qsa::launch_detect_dirty(a, (hipStream_t)stream), "detect_dirty_blocks");
}

int qsa_score_blocks(const qsa_dims *dims, const qsa_seqs *seqs, const float *q_idx_dev,
                     const int32_t *q_seq_dev, const int32_t *q_pos_dev, int32_t n_q,
                     const float *pooled_dev, const uint16_t *pooled_bf16_dev, int32_t nb_max,
                     float *scores_dev, int64_t ld_scores, int32_t mode, void *ws_dev,
                     size_t ws_bytes, void *stream) {
    int rc = check_dims(dims);
    if (!rc) rc = check_seqs(dims, seqs);
    if (!rc) rc = check_queries(q_seq_dev, q_pos_dev, n_q, true);
    if (rc) return rc;
    const int64_t cap_blocks = seqs->cap_cells / dims->r;
    if (nb_max < 0 || nb_max > cap_blocks)
        return fail(QSA_EINVAL, "nb_max %d outside 0..cap_cells/r", nb_max);
    if (ld_scores < nb_max) return fail(QSA_EINVAL, "ld_scores below nb_max");
    if (n_q == 0 || nb_max == 0) return ok();
    if (!q_idx_dev || !aligned(q_idx_dev, 4)) return fail(QSA_EINVAL, "q_idx_dev NULL or misaligned");
    if (!scores_dev || !aligned(scores_dev, 4))
        return fail(QSA_EINVAL, "scores_dev NULL or misaligned");
    qsa::ScoreArgs a{geom(seqs),     q_idx_dev,  q_seq_dev, q_pos_dev, n_q,     pooled_dev,
                     pooled_bf16_dev, nb_max,     scores_dev, ld_scores, dims->r,
                     rope_table(dims->rope_theta)};
    if (mode == QSA_SCORE_F32) {
        if (!pooled_dev || !aligned(pooled_dev, 16))
            return fail(QSA_EINVAL, "pooled_dev NULL or not 16-byte aligned");
        return launched(qsa::launch_score_f32(a, (hipStream_t)stream), "score_blocks");
    }
    if (mode == QSA_SCORE_BF16) {
        if (!pooled_bf16_dev || !aligned(pooled_bf16_dev, 16))
            return fail(QSA_EINVAL, "pooled_bf16_dev NULL or not 16-byte aligned");
        const size_t need = (size_t)n_q * qsa::kDIdx * sizeof(uint16_t);
        if (!ws_dev || ws_bytes < need || !aligned(ws_dev, 16))
            return fail(QSA_EWS, "score workspace needs %zu bytes, 16-byte aligned", need);
        return launched(qsa::launch_score_bf16_ws(a, (uint16_t *)ws_dev, (hipStream_t)stream),
                        "score_blocks(bf16)");
    }
    return fail(QSA_EINVAL, "unknown score mode %d", mode);
}

int qsa_select_topk_blocks(const qsa_dims *dims, const qsa_seqs *seqs, const float *scores_dev,
                           int64_t ld_scores, const int32_t *q_seq_dev, const int32_t *q_pos_dev,
                           int32_t n_q, int32_t nb_max, int32_t *sel_blocks_dev,
                           int32_t *sel_cells_dev, int32_t *n_sel_dev, void *ws_dev,
                           size_t ws_bytes, void *stream) {
    (void)ws_dev;
    (void)ws_bytes;
    int rc = check_dims(dims);
    if (!rc) rc = check_seqs(dims, seqs);
    if (!rc) rc = check_queries(q_seq_dev, q_pos_dev, n_q, true);
    if (rc) return rc;
    const int64_t cap_blocks = seqs->cap_cells / dims->r;
    if (nb_max < 0 || nb_max > cap_blocks)
        return fail(QSA_EINVAL, "nb_max %d outside 0..cap_cells/r", nb_max);
    if (ld_scores < nb_max) return fail(QSA_EINVAL, "ld_scores below nb_max");
    if (n_q == 0) return ok();
    if (nb_max > 0 && (!scores_dev || !aligned(scores_dev, 4)))
        return fail(QSA_EINVAL, "scores_dev NULL or misaligned");
    if (!sel_blocks_dev || !sel_cells_dev || !n_sel_dev || !aligned(sel_blocks_dev, 4) ||
        !aligned(sel_cells_dev, 4) || !aligned(n_sel_dev, 4))
        return fail(QSA_EINVAL, "selection outputs NULL or misaligned");
    qsa::SelectArgs a{geom(seqs), scores_dev, ld_scores, q_seq_dev, q_pos_dev, n_q, nb_max,
                      dims->r, dims->top_k, sel_blocks_dev, sel_cells_dev, n_sel_dev};
    return launched(qsa::launch_select(a, (hipStream_t)stream), "select_topk_blocks");
}

// Shared validation of the decode indexer calls; fills *f.
static int decode_idx_args(const qsa_dims *dims, const qsa_seqs *seqs, const void *kidx_dev,
                           const int32_t *dirty_dev, int32_t n_dirty, float *pooled_dev,
                           uint16_t *pooled_bf16_dev, const float *q_idx_dev,
                           const int32_t *q_seq_dev, const int32_t *q_pos_dev, int32_t n_q,
                           int32_t nb_max, float *scores_dev, int64_t ld_scores,
                           int32_t *sel_blocks_dev, int32_t *sel_cells_dev, int32_t *n_sel_dev,
                           void *ws_dev, size_t ws_bytes, bool need_scoring, bool need_select,
                           qsa::DecodeIdxArgs *f) {
    int rc = check_dims(dims);
    if (!rc) rc = check_seqs(dims, seqs);
    if (!rc) rc = check_queries(q_seq_dev, q_pos_dev, n_q, true);
    if (rc) return rc;
    const int64_t cap_blocks = seqs->cap_cells / dims->r;
    if (nb_max < 0 || nb_max > cap_blocks)
        return fail(QSA_EINVAL, "nb_max %d outside 0..cap_cells/r", nb_max);
    if (nb_max > qsa::kFusedMaxBlocks)
        return fail(QSA_ENOTSUP, "nb_max %d above %d: use the separate calls", nb_max,
                    qsa::kFusedMaxBlocks);
    if (ld_scores < nb_max) return fail(QSA_EINVAL, "ld_scores below nb_max");
    if (n_q > 0 && (!scores_dev || !aligned(scores_dev, 4)))
        return fail(QSA_EINVAL, "scores_dev NULL or misaligned");
    if (need_scoring) {
        if (n_dirty < 0) return fail(QSA_EINVAL, "n_dirty negative");
        if (n_dirty > 0 &&
            (!kidx_dev || !dirty_dev || !aligned(kidx_dev, kidx_align(dims)) ||
             !aligned(dirty_dev, 4)))
            return fail(QSA_EINVAL, "kidx_dev/dirty_dev NULL or misaligned");
        if (pooled_bf16_dev && !aligned(pooled_bf16_dev, 16))
            return fail(QSA_EINVAL, "pooled_bf16_dev not 16-byte aligned");
        if (!pooled_dev || !aligned(pooled_dev, 16))
            return fail(QSA_EINVAL, "pooled_dev NULL or not 16-byte aligned");
        if (n_q > 0 && (!q_idx_dev || !aligned(q_idx_dev, 4)))
            return fail(QSA_EINVAL, "q_idx_dev NULL or misaligned");
    }
    if (need_select && n_q > 0 &&
        (!sel_blocks_dev || !sel_cells_dev || !n_sel_dev || !aligned(sel_blocks_dev, 4) ||
         !aligned(sel_cells_dev, 4) || !aligned(n_sel_dev, 4)))
        return fail(QSA_EINVAL, "selection outputs NULL or misaligned");
    const size_t need = qsa::fused_select_ws_bytes(n_q, nb_max);
    if (need && (!ws_dev || ws_bytes < need || !aligned(ws_dev, 16)))
        return fail(QSA_EWS, "decode indexer workspace needs %zu bytes, 16-byte aligned", need);
    *f = qsa::DecodeIdxArgs{};
    f->s = qsa::ScoreArgs{geom(seqs),      q_idx_dev, q_seq_dev,  q_pos_dev, n_q,     pooled_dev,
                          pooled_bf16_dev, nb_max,    scores_dev, ld_scores, dims->r,
                          rope_table(dims->rope_theta)};
    f->pooled_w = pooled_dev;
    f->pooled_bf16 = pooled_bf16_dev;
    f->kidx = kidx_ref(dims, kidx_dev);
    f->dirty = dirty_dev;
    f->n_dirty = need_scoring ? n_dirty : 0;
    f->eps = dims->rms_eps;
    f->gamma = dims->idx_norm_w_dev;
    f->top_k = dims->top_k;
    f->sel_blocks = sel_blocks_dev;
    f->sel_cells = sel_cells_dev;
    f->n_sel = n_sel_dev;
    // the scoring call and the selection call of one step bind the same count
    f->wide_cand = qsa::fused_decode_fits(n_q, dims->top_k + dims->r - 1, dims->n_head,
                                          dims->n_head_kv)
                       ? 0
                       : 1;
    return QSA_OK;
}

int qsa_score_select_prefill(const qsa_dims *dims, const qsa_seqs *seqs, const void *kidx_dev,
                             const int32_t *dirty_dev, int32_t n_dirty, float *pooled_dev,
                             uint16_t *pooled_bf16_dev, const float *q_idx_dev,
                             const int32_t *q_seq_dev, const int32_t *q_pos_dev, int32_t n_q,
                             int32_t nb_max, int32_t *sel_blocks_dev, int32_t *sel_cells_dev,
                             int32_t *n_sel_dev, void *ws_dev, size_t ws_bytes, void *stream) {
    int rc = check_dims(dims);
    if (!rc) rc = check_seqs(dims, seqs);
    if (!rc) rc = check_queries(q_seq_dev, q_pos_dev, n_q, true);
    if (rc) return rc;
    const int64_t cap_blocks = seqs->cap_cells / dims->r;
    if (nb_max < 0 || nb_max > cap_blocks)
        return fail(QSA_EINVAL, "nb_max %d outside 0..cap_cells/r", nb_max);
    if (nb_max > qsa::kFusedMaxBlocks)
        return fail(QSA_ENOTSUP, "nb_max %d above %d", nb_max, qsa::kFusedMaxBlocks);
    if (n_dirty < 0) return fail(QSA_EINVAL, "n_dirty negative");
    if (n_dirty > 0 && (!kidx_dev || !dirty_dev || !aligned(kidx_dev, kidx_align(dims)) ||
                        !aligned(dirty_dev, 4)))
        return fail(QSA_EINVAL, "kidx_dev/dirty_dev NULL or misaligned");
    if (!pooled_dev || !aligned(pooled_dev, 16))
        return fail(QSA_EINVAL, "pooled_dev NULL or not 16-byte aligned");
    if (!pooled_bf16_dev || !aligned(pooled_bf16_dev, 16))
        return fail(QSA_EINVAL, "pooled_bf16_dev NULL or not 16-byte aligned");
    if (n_q > 0 && (!q_idx_dev || !aligned(q_idx_dev, 4)))
        return fail(QSA_EINVAL, "q_idx_dev NULL or misaligned");
    if (n_q > 0 && (!sel_blocks_dev || !sel_cells_dev || !n_sel_dev || !aligned(sel_blocks_dev, 4) ||
                    !aligned(sel_cells_dev, 4) || !aligned(n_sel_dev, 4)))
        return fail(QSA_EINVAL, "selection outputs NULL or misaligned");
    const size_t need = qsa::prefill_ws_bytes(n_q, nb_max);
    if (need && (!ws_dev || ws_bytes < need || !aligned(ws_dev, 16)))
        return fail(QSA_EWS, "prefill indexer workspace needs %zu bytes, 16-byte aligned", need);
    const qsa::RopeTable rope = rope_table(dims->rope_theta);
    // the update shares the first launch of the indexer (alone when n_q is 0;
    // nb_max 0: every query keeps its tail only)
    const qsa::UpdateArgs u{geom(seqs), kidx_ref(dims, kidx_dev), dirty_dev,
                            n_dirty > 0 ? n_dirty : 0, pooled_dev, pooled_bf16_dev, dims->r,
                            dims->rms_eps, dims->idx_norm_w_dev, rope};
    const qsa::ScoreArgs a{geom(seqs),      q_idx_dev, q_seq_dev, q_pos_dev, n_q, pooled_dev,
                           pooled_bf16_dev, nb_max,    nullptr,   0,         dims->r, rope};
    const hipError_t e = qsa::launch_score_select_prefill(
        a, dims->idx_norm_w_dev, ws_dev, dims->top_k, sel_blocks_dev, sel_cells_dev, n_sel_dev, u,
        (hipStream_t)stream);
    return launched(e, "score_select_prefill");
}

int qsa_decode_score_candidates(const qsa_dims *dims, const qsa_seqs *seqs,
                                const void *kidx_dev, const int32_t *dirty_dev, int32_t n_dirty,
                                float *pooled_dev, uint16_t *pooled_bf16_dev,
                                const float *q_idx_dev, const int32_t *q_seq_dev,
                                const int32_t *q_pos_dev, int32_t n_q, int32_t nb_max,
                                float *scores_dev, int64_t ld_scores, void *ws_dev,
                                size_t ws_bytes, void *stream) {
    qsa::DecodeIdxArgs f;
    const int rc = decode_idx_args(dims, seqs, kidx_dev, dirty_dev, n_dirty, pooled_dev,
                                   pooled_bf16_dev, q_idx_dev, q_seq_dev, q_pos_dev, n_q, nb_max,
                                   scores_dev, ld_scores, nullptr, nullptr, nullptr, ws_dev,
                                   ws_bytes, true, false, &f);
    if (rc) return rc;
    return launched(qsa::launch_decode_candidates(f, ws_dev, (hipStream_t)stream),
                    "decode_score_candidates");
}

int qsa_decode_select_candidates(const qsa_dims *dims, const qsa_seqs *seqs,
                                 const int32_t *q_seq_dev, const int32_t *q_pos_dev, int32_t n_q,
                                 int32_t nb_max, const float *scores_dev, int64_t ld_scores,
                                 int32_t *sel_blocks_dev, int32_t *sel_cells_dev,
                                 int32_t *n_sel_dev, const void *ws_dev, size_t ws_bytes,
                                 void *stream) {
    qsa::DecodeIdxArgs f;
    const int rc = decode_idx_args(dims, seqs, nullptr, nullptr, 0, nullptr, nullptr, nullptr,
                                   q_seq_dev, q_pos_dev, n_q, nb_max, (float *)scores_dev,
                                   ld_scores, sel_blocks_dev, sel_cells_dev, n_sel_dev,
                                   (void *)ws_dev, ws_bytes, false, true, &f);
    if (rc) return rc;
    return launched(qsa::launch_decode_select(f, (void *)ws_dev, (hipStream_t)stream),
                    "decode_select_candidates");
}

int qsa_score_select_decode(const qsa_dims *dims, const qsa_seqs *seqs, const void *kidx_dev,
                            const int32_t *dirty_dev, int32_t n_dirty, float *pooled_dev,
                            uint16_t *pooled_bf16_dev, const float *q_idx_dev,
                            const int32_t *q_seq_dev, const int32_t *q_pos_dev, int32_t n_q,
                            int32_t nb_max, float *scores_dev, int64_t ld_scores,
                            int32_t *sel_blocks_dev, int32_t *sel_cells_dev, int32_t *n_sel_dev,
                            void *ws_dev, size_t ws_bytes, void *stream) {
    if (dims && seqs && dims->r >= 1 && nb_max > qsa::kFusedMaxBlocks &&
        nb_max <= seqs->cap_cells / dims->r) {
        // beyond the selection kernel's LDS bitmap: the three general calls
        int rc = qsa_update_pooled_keys(dims, seqs, kidx_dev, dirty_dev, n_dirty, pooled_dev,
                                        pooled_bf16_dev, stream);
        if (!rc)
            rc = qsa_score_blocks(dims, seqs, q_idx_dev, q_seq_dev, q_pos_dev, n_q, pooled_dev,
                                  pooled_bf16_dev, nb_max, scores_dev, ld_scores, QSA_SCORE_F32,
                                  nullptr, 0, stream);
        if (!rc)
            rc = qsa_select_topk_blocks(dims, seqs, scores_dev, ld_scores, q_seq_dev, q_pos_dev,
                                        n_q, nb_max, sel_blocks_dev, sel_cells_dev, n_sel_dev,
                                        nullptr, 0, stream);
        return rc;
    }
    qsa::DecodeIdxArgs f;
    const int rc = decode_idx_args(dims, seqs, kidx_dev, dirty_dev, n_dirty, pooled_dev,
                                   pooled_bf16_dev, q_idx_dev, q_seq_dev, q_pos_dev, n_q, nb_max,
                                   scores_dev, ld_scores, sel_blocks_dev, sel_cells_dev,
                                   n_sel_dev, ws_dev, ws_bytes, true, true, &f);
    if (rc) return rc;
    hipError_t e = qsa::launch_decode_candidates(f, ws_dev, (hipStream_t)stream);
    if (e == hipSuccess) e = qsa::launch_decode_select(f, ws_dev, (hipStream_t)stream);
    return launched(e, "score_select_decode");
}

// Validates the attention arguments and fills *a (sel_cells/n_sel may be
// outputs of the same launch when check_sel is false).
static int attn_args(const qsa_dims *dims, const qsa_seqs *seqs, const float *q_dev,
                     const int32_t *q_seq_dev, int32_t n_q, const void *k_cache_dev,
                     const void *v_cache_dev, const int32_t *sel_cells_dev,
                     const int32_t *n_sel_dev, float *out_dev, void *ws_dev, size_t ws_bytes,
                     bool prefill, qsa::AttnArgs *a, bool gather_only = false,
                     int64_t ws_need = -1) {
    int rc = check_dims(dims);
    if (!rc) rc = check_seqs(dims, seqs);
    if (!rc) rc = check_queries(q_seq_dev, nullptr, n_q, false);
    if (rc) return rc;
    if (n_q == 0) return QSA_OK;
    if (!gather_only && (!q_dev || !aligned(q_dev, 16)))
        return fail(QSA_EINVAL, "q_dev NULL or not 16-byte aligned");
    if (!gather_only && (!out_dev || !aligned(out_dev, 4)))
        return fail(QSA_EINVAL, "out_dev NULL or misaligned");
    if (!k_cache_dev || !v_cache_dev || !aligned(k_cache_dev, 16) || !aligned(v_cache_dev, 16))
        return fail(QSA_EINVAL, "K/V cache NULL or not 16-byte aligned");
    if (!sel_cells_dev || !n_sel_dev || !aligned(sel_cells_dev, 4) || !aligned(n_sel_dev, 4))
        return fail(QSA_EINVAL, "selection NULL or misaligned");
    if (cell_rows(seqs) * dims->n_head_kv >= ((int64_t)1 << 31))
        return fail(QSA_EINVAL, "K/V cache of 2^31 rows or more");
    const int ld_cells = dims->top_k + dims->r - 1;
    const size_t need = ws_need >= 0 ? (size_t)ws_need
                        : gather_only ? 0
                        : prefill     ? qsa::attn_prefill_ws_bytes(n_q, dims->n_head, ld_cells)
                                      : qsa::attn_decode_ws_bytes(n_q, dims->n_head, ld_cells);
    if (need && (!ws_dev || ws_bytes < need || !aligned(ws_dev, 16)))
        return fail(QSA_EWS, "attention workspace needs %zu bytes, 16-byte aligned", need);
    const float scale =
        dims->kq_scale > 0.0f ? dims->kq_scale : 1.0f / sqrtf((float)dims->head_dim);
    *a = qsa::AttnArgs{geom(seqs), q_dev,         q_seq_dev,     n_q,           dims->n_head,
                       dims->n_head_kv, dims->kv_type, k_cache_dev, v_cache_dev, sel_cells_dev,
                       n_sel_dev,      ld_cells,      scale,         out_dev,       (float *)ws_dev,
                       ws_bytes};
    return QSA_OK;
}

static int attn_common(const qsa_dims *dims, const qsa_seqs *seqs, const float *q_dev,
                       const int32_t *q_seq_dev, int32_t n_q, const void *k_cache_dev,
                       const void *v_cache_dev, const int32_t *sel_cells_dev,
                       const int32_t *n_sel_dev, float *out_dev, void *ws_dev, size_t ws_bytes,
                       void *stream, bool prefill) {
    qsa::AttnArgs a;
    const int rc = attn_args(dims, seqs, q_dev, q_seq_dev, n_q, k_cache_dev, v_cache_dev,
                             sel_cells_dev, n_sel_dev, out_dev, ws_dev, ws_bytes, prefill, &a);
    if (rc) return rc;
    if (n_q == 0) return ok();
    hipError_t e = prefill ? qsa::launch_attn_prefill(a, (hipStream_t)stream)
                           : qsa::launch_attn_decode(a, (hipStream_t)stream);
    return launched(e, prefill ? "sparse_attn_prefill" : "sparse_attn_decode");
}

int qsa_sparse_attn_decode(const qsa_dims *dims, const qsa_seqs *seqs, const float *q_dev,
                           const int32_t *q_seq_dev, int32_t n_q, const void *k_cache_dev,
                           const void *v_cache_dev, const int32_t *sel_cells_dev,
                           const int32_t *n_sel_dev, float *out_dev, void *ws_dev,
                           size_t ws_bytes, void *stream) {
    return attn_common(dims, seqs, q_dev, q_seq_dev, n_q, k_cache_dev, v_cache_dev,
                       sel_cells_dev, n_sel_dev, out_dev, ws_dev, ws_bytes, stream, false);
}

int qsa_sparse_attn_decode_union(const qsa_dims *dims, const qsa_seqs *seqs, const float *q_dev,
                                 const int32_t *q_seq_dev, int32_t n_q, int32_t t_group,
                                 const void *k_cache_dev, const void *v_cache_dev,
                                 const int32_t *sel_cells_dev, const int32_t *n_sel_dev,
                                 float *out_dev, void *ws_dev, size_t ws_bytes, void *stream) {
    int rc = check_dims(dims);
    if (!rc) rc = check_seqs(dims, seqs);
    if (rc) return rc;
    if (t_group < 1 || t_group > qsa::kUnionMaxTokens)
        return fail(QSA_EINVAL, "t_group %d outside 1..%d", t_group, qsa::kUnionMaxTokens);
    if (dims->kv_type != QSA_KV_Q8_0)
        return fail(QSA_ENOTSUP, "the union path reads q8_0 caches");
    const int hpk = dims->n_head / dims->n_head_kv;
    if (hpk < 4 || 16 % hpk)
        return fail(QSA_ENOTSUP, "query heads per KV head %d: the union path takes 4, 8 or 16", hpk);
    const int ld_cells = dims->top_k + dims->r - 1;
    if ((int64_t)t_group * ld_cells > qsa::kUnionMaxEntries)
        return fail(QSA_ENOTSUP, "t_group * (top_k + r - 1) = %lld above %d",
                    (long long)t_group * ld_cells, qsa::kUnionMaxEntries);
    if (seqs->cell_rows_dev) return fail(QSA_ENOTSUP, "the union path takes no cell table");
    if (seqs->cap_cells >= ((int64_t)1 << 28))
        return fail(QSA_ENOTSUP, "cap_cells of 2^28 or more");
    const size_t need =
        qsa::union_ws_bytes(n_q, t_group, dims->n_head, dims->n_head_kv, ld_cells);
    qsa::AttnArgs a;
    rc = attn_args(dims, seqs, q_dev, q_seq_dev, n_q, k_cache_dev, v_cache_dev, sel_cells_dev,
                   n_sel_dev, out_dev, ws_dev, ws_bytes, false, &a, false, (int64_t)need);
    if (rc) return rc;
    if (n_q == 0) return ok();
    return launched(qsa::launch_attn_decode_union(a, t_group, (hipStream_t)stream),
                    "sparse_attn_decode_union");
}

int qsa_sparse_attn_decode_noalloc(const qsa_dims *dims, const qsa_seqs *seqs,
                                   const float *q_dev, const int32_t *q_seq_dev, int32_t n_q,
                                   const void *k_cache_dev, const void *v_cache_dev,
                                   const int32_t *sel_cells_dev, const int32_t *n_sel_dev,
                                   float *out_dev, void *stream) {
    int rc = check_dims(dims);
    if (rc) return rc;
    if (n_q < 0) return fail(QSA_EINVAL, "n_q negative");
    const size_t need =
        qsa::attn_decode_ws_bytes(n_q, dims->n_head, dims->top_k + dims->r - 1);
    if (need > kNoAllocScratchBytes)
        return fail(QSA_EWS,
                    "decode attention of %d queries needs %zu bytes of partial states; the "
                    "library's scratch holds %zu",
                    n_q, need, kNoAllocScratchBytes);
    if (n_q == 0) return ok();
    void *ws = nullptr;
    rc = scratch_of_current_device(&ws);
    if (rc) return rc;
    return attn_common(dims, seqs, q_dev, q_seq_dev, n_q, k_cache_dev, v_cache_dev,
                       sel_cells_dev, n_sel_dev, out_dev, ws, kNoAllocScratchBytes, stream,
                       false);
}

int qsa_sparse_attn_prefill(const qsa_dims *dims, const qsa_seqs *seqs, const float *q_dev,
                            const int32_t *q_seq_dev, int32_t n_q, const void *k_cache_dev,
                            const void *v_cache_dev, const int32_t *sel_cells_dev,
                            const int32_t *n_sel_dev, float *out_dev, void *ws_dev,
                            size_t ws_bytes, void *stream) {
    return attn_common(dims, seqs, q_dev, q_seq_dev, n_q, k_cache_dev, v_cache_dev,
                       sel_cells_dev, n_sel_dev, out_dev, ws_dev, ws_bytes, stream, true);
}

int qsa_decode_select_attend(const qsa_dims *dims, const qsa_seqs *seqs,
                             const int32_t *q_seq_dev, const int32_t *q_pos_dev, int32_t n_q,
                             int32_t nb_max, const float *scores_dev, int64_t ld_scores,
                             int32_t *sel_blocks_dev, int32_t *sel_cells_dev,
                             int32_t *n_sel_dev, const void *ws_idx_dev, size_t ws_idx_bytes,
                             const float *q_dev, const void *k_cache_dev,
                             const void *v_cache_dev, float *out_dev, void *ws_attn_dev,
                             size_t ws_attn_bytes, void *stream) {
    qsa::DecodeIdxArgs f;
    int rc = decode_idx_args(dims, seqs, nullptr, nullptr, 0, nullptr, nullptr, nullptr,
                             q_seq_dev, q_pos_dev, n_q, nb_max, (float *)scores_dev, ld_scores,
                             sel_blocks_dev, sel_cells_dev, n_sel_dev, (void *)ws_idx_dev,
                             ws_idx_bytes, false, true, &f);
    if (rc) return rc;
    if (nb_max > qsa::kSelAttnMaxBlocks)
        return fail(QSA_ENOTSUP, "nb_max %d above %d: use the separate calls", nb_max,
                    qsa::kSelAttnMaxBlocks);
    qsa::AttnArgs a;
    rc = attn_args(dims, seqs, q_dev, q_seq_dev, n_q, k_cache_dev, v_cache_dev, sel_cells_dev,
                   n_sel_dev, out_dev, ws_attn_dev, ws_attn_bytes, false, &a);
    if (rc) return rc;
    if (n_q == 0) return ok();
    return launched(qsa::launch_select_attn_decode(f, (void *)ws_idx_dev, a, (hipStream_t)stream),
                    "decode_select_attend");
}

// ---- memory-traffic probes (include/qsa_probe.h) ----

int qsa_probe_stream_read(const void *src_dev, size_t n_bytes, int32_t nontemporal,
                          uint32_t *sink_dev, int32_t n_sink, void *stream) {
    if (!src_dev || !aligned(src_dev, 16) || n_bytes % 16)
        return fail(QSA_EINVAL, "probe source NULL, not 16-byte aligned, or not whole 16-byte words");
    if (!sink_dev || !aligned(sink_dev, 4) || n_sink < 1)
        return fail(QSA_EINVAL, "probe sink NULL, misaligned or empty");
    if (n_bytes == 0) return ok();
    return launched(qsa::launch_probe_read(src_dev, n_bytes, nontemporal != 0, sink_dev, n_sink,
                                           (hipStream_t)stream),
                    "probe_stream_read");
}

int qsa_probe_gather_prefill(const qsa_dims *dims, const qsa_seqs *seqs,
                             const int32_t *q_seq_dev, int32_t n_q, const void *k_cache_dev,
                             const void *v_cache_dev, const int32_t *sel_cells_dev,
                             const int32_t *n_sel_dev, uint32_t *sink_dev, int32_t n_sink,
                             void *stream) {
    qsa::AttnArgs a;
    int rc = attn_args(dims, seqs, nullptr, q_seq_dev, n_q, k_cache_dev, v_cache_dev,
                       sel_cells_dev, n_sel_dev, nullptr, nullptr, 0, true, &a, true);
    if (rc) return rc;
    if (dims->kv_type != QSA_KV_Q8_0 || seqs->cell_rows_dev)
        return fail(QSA_ENOTSUP, "the gather probe follows the q8_0 kernel without a cell table");
    if (!sink_dev || !aligned(sink_dev, 4) || n_sink < 1)
        return fail(QSA_EINVAL, "probe sink NULL, misaligned or empty");
    if (n_q == 0) return ok();
    return launched(qsa::launch_probe_gather_prefill(a, sink_dev, n_sink, (hipStream_t)stream),
                    "probe_gather_prefill");
}

}  // extern "C"
