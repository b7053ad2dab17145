/*
 * qsa.h -- C ABI of libqsa, the QSA sparse-attention step on AMD Instinct
 * MI355X (gfx950).
 *
 * The step has four parts, each one call below:
 *   1. qsa_update_pooled_keys  -- persistent pooled block-key cache; only the
 *      dirtied blocks are recomputed.
 *   2. qsa_score_blocks        -- indexer score of every causal block.
 *   3. qsa_select_topk_blocks  -- top-k over whole blocks, expanded to cells,
 *      plus the incomplete tail block's cells.
 *   4. qsa_sparse_attn_decode / qsa_sparse_attn_prefill -- attention over the
 *      selected cells only.
 *
 * Sources (cited by page title and section):
 *   [ISSUE] llama.cpp issue #28734, "Eval bug: qwen4exp (Qwen3.8-Flash-Next)
 *           CUDA: decode slows linearly with context": the fix summary's
 *           sections lever1, lever3, lever2 and lever2b, and goodbadwolf's
 *           comment, paragraph "Why the two phases disagree".
 *   [DISC]  llama.cpp discussion #30071, "Qwen3.8-Flash-Next on 6x3090 and
 *           6x4090 without NVLink ...", the paragraph that separates the two
 *           problems (the compact-gather path that keeps q8_0 KV sparse).
 *
 * Conventions shared by every call
 * --------------------------------
 * Pointers named *_dev are device pointers (hipMalloc'd or equivalent);
 * the caller owns every buffer, including workspaces.  The library never
 * allocates, frees or synchronises: each call validates its host-side
 * arguments, enqueues kernels on `stream` (a hipStream_t; NULL = the default
 * stream) and returns.  On a validation error nothing is enqueued and no
 * output is touched.  Device faults surface at the caller's next
 * synchronisation.  No C++ exception crosses this boundary.  The library
 * keeps no state between calls (qsa_sparse_attn_decode_noalloc aside, which
 * uses a scratch array the library holds on each GPU); calls on different
 * streams may run concurrently if their outputs do not overlap.
 *
 * Sequences.  n_seq independent sequences each own a region of cap_cells
 * cells in every per-cell cache (cell index = token position in that
 * sequence).  n_cells_dev[s] (device, int32) is the number of cells present
 * in sequence s.  Block b of a sequence is cells b*r .. b*r+r-1.
 *
 * Queries.  Query i belongs to sequence q_seq_dev[i] and sits at position
 * q_pos_dev[i] (both device int32).  A query is valid when
 * 0 <= q_seq < n_seq and 0 <= q_pos < min(n_cells[q_seq], cap_cells).
 * An invalid query gets an all -inf score row, an empty selection
 * (n_sel = 0) and an all-zero attention output; no call reads or writes
 * outside the buffers on its behalf.
 *
 * Per query, nc = floor((q_pos+1)/r) complete blocks are visible; the tail
 * is the tail_len = q_pos+1 - r*nc (0 .. r-1) cells of the incomplete block
 * at the query position [ISSUE lever3: fully-future blocks are excluded and
 * the incomplete tail rides a per-token side input].
 *
 * Buffer layouts (all little-endian, row-major unless stated):
 *   kidx      float32, or bfloat16 bits when dims->kidx_type is QSA_KIDX_BF16
 *             (widened exactly before the mean), [n_seq][cap_cells][d_idx]:
 *             per-cell indexer keys
 *   pooled    float32 tiled: [n_seq][cap_blocks/64][d_idx/4][64][4];
 *             element (s, b, t) is at float offset
 *               ((s*(cap_blocks/64) + b/64) * (d_idx/4) + t/4) * 256
 *               + (b%64)*4 + t%4
 *             (64 blocks side by side per 16-byte dim quad, so 64 lanes read
 *             64 blocks with one 1 KiB coalesced load).  cap_blocks =
 *             cap_cells / r.
 *   pooled_bf16  uint16 (bfloat16 bits) [n_seq][cap_blocks][d_idx]: the same
 *             keys rounded to nearest even; the MFMA operand at prefill.
 *   scores    float32 [n_q][ld_scores]
 *   sel_blocks int32 [n_q][top_k/r]     ascending, padded with -1
 *   sel_cells  int32 [n_q][top_k+r-1]   ascending cell indices, padded -1;
 *             top_k + r - 1 is the largest possible set, n_kv_max
 *             [ISSUE, goodbadwolf: n_kv_max = min(n_kv, top_k + r - 1)]
 *   n_sel     int32 [n_q]               number of valid entries of sel_cells
 *   q_idx     float32 [n_q][d_idx]      indexer queries, not yet roped
 *   q         float32 [n_q][n_head][head_dim]   attention queries (already
 *             positioned; attention applies no RoPE)
 *   out       float32 [n_q][n_head][head_dim]
 *   K, V cache QSA_KV_F32:  float32 [n_seq][cap_cells][n_head_kv][head_dim]
 *             QSA_KV_F16:  binary16 [n_seq][cap_cells][n_head_kv][head_dim],
 *             value = float(h), exact (the KV type the fix of llama.cpp issue
 *             #28734 requires: its fix summary and the comment that times
 *             q8_0 KV against it)
 *             QSA_KV_Q8_0: bytes [n_seq][cap_cells][n_head_kv][head_dim/32*34];
 *             each 34-byte q8_0 block is a binary16 scale d followed by 32
 *             int8 q, value = float(d) * q.
 *
 * Supported geometry (else QSA_ENOTSUP): head_dim 256, d_idx 128,
 * n_head/n_head_kv in {1, 2, 4, 8}, 1 <= r <= 16, top_k % r == 0,
 * top_k/r <= 4096, cap_cells a multiple of 64*r.
 */
#ifndef QSA_H
#define QSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QSA_ABI_VERSION 3

/* Return codes.  0 is success; errors are negative. */
#define QSA_OK 0
#define QSA_EINVAL (-1)  /* bad pointer, size, alignment or geometry       */
#define QSA_ENOTSUP (-2) /* geometry outside what the library implements  */
#define QSA_EWS (-3)     /* workspace missing or smaller than required     */
#define QSA_EHIP (-4)    /* a HIP launch reported an error                 */

/* KV cache element types. */
#define QSA_KV_F32 0
#define QSA_KV_Q8_0 1
#define QSA_KV_F16 2

/* Per-cell indexer key storage (qsa_dims.kidx_type). */
#define QSA_KIDX_F32 0
#define QSA_KIDX_BF16 1

/* Score modes of qsa_score_blocks. */
#define QSA_SCORE_F32 0      /* decode: fp32, fixed summation order T      */
#define QSA_SCORE_BF16 1     /* prefill: bf16 operands, fp32 sum in order T */

/* Workspace owners for qsa_workspace_size. */
#define QSA_OP_SELECT 0
#define QSA_OP_ATTN_DECODE 1
#define QSA_OP_ATTN_PREFILL 2
#define QSA_OP_SCORE_BF16 3
#define QSA_OP_SCORE_SELECT 4
#define QSA_OP_SCORE_SELECT_PREFILL 5
#define QSA_OP_ATTN_DECODE_UNION 6 /* nb_max argument: tokens per group */

/* Model geometry and constants.
 *   kq_scale   attention logit scale; <= 0 means 1/sqrt(head_dim)
 *   rope_theta RoPE base of the indexer (split-half rotation of pairs
 *              (t, t + d_idx/2), inverse frequency theta^(-2t/d_idx))
 *   rms_eps    epsilon of the pooled-key RMS norm
 *   idx_norm_w_dev  optional device float32 [d_idx] RMS-norm weight (NULL =
 *              none)
 *   kidx_type  storage of the per-cell indexer keys: QSA_KIDX_F32 or
 *              QSA_KIDX_BF16 (the pages do not fix their dtype; bf16 halves
 *              the cache).  The pooled key is computed from the exactly
 *              widened values, so a bf16 cache gives the pooled keys of its
 *              f32 widening bit for bit. */
typedef struct qsa_dims {
    int32_t n_head;
    int32_t n_head_kv;
    int32_t head_dim;
    int32_t d_idx;
    int32_t r;
    int32_t top_k;
    int32_t kv_type;
    float kq_scale;
    float rope_theta;
    float rms_eps;
    const float *idx_norm_w_dev;
    int32_t kidx_type;
} qsa_dims;

/* Sequence geometry shared by every call.
 *   n_cells_dev      device int32 [n_seq]: cells (positions 0 .. n-1) present
 *   cell_rows_dev    optional device int32 [n_seq][cap_cells]: the row of
 *                    position p of sequence s in the per-cell arrays (kidx, K,
 *                    V), which then hold n_rows rows shared by all sequences
 *                    (a unified cache whose cells move under defrag and
 *                    sequence edits).  NULL: position p of sequence s is row
 *                    s*cap_cells + p.  Entries of present positions must lie in
 *                    [0, n_rows); others are read as row 0 and not used.
 *   n_rows           rows of the per-cell arrays when cell_rows_dev is given */
typedef struct qsa_seqs {
    int32_t n_seq;
    int64_t cap_cells;
    const int32_t *n_cells_dev;
    const int32_t *cell_rows_dev;
    int64_t n_rows;
} qsa_seqs;

/* Library version (QSA_ABI_VERSION). */
int qsa_version(void);

/* Message of the last error returned on the calling thread ("" if none). */
const char *qsa_last_error(void);

/* Bytes of workspace `op` needs for n_q queries whose scores are nb_max wide
 * (nb_max is ignored by ops that do not read scores).  Returns 0 and writes
 * *bytes, or an error code. */
int qsa_workspace_size(const qsa_dims *dims, int32_t op, int32_t n_q,
                       int32_t nb_max, size_t *bytes);

/* 0. Dirty blocks by structural compare  [ISSUE fix summary, lever2: a block
 * is recomputed when its member cells changed, found by comparing them with
 * the cells it was built from -- defrag, rollback and sequence edits need no
 * invalidation hooks].
 *
 * A block's members are the rows (through seqs->cell_rows_dev when given) of
 * its present positions block*r .. block*r+m-1, m = min(r, n_cells - block*r).
 * snapshot_dev: int32 [n_seq][cap_cells/r][r+1], owned by the caller and
 * zero-filled before the first call (every block empty), then kept by this
 * call: per block the member count and rows last reported.  Writes
 * dirty_dev[max_dirty][2]: the (seq, block) pairs of the changed non-empty
 * blocks, then (-1, -1) padding -- the list qsa_update_pooled_keys takes with
 * n_dirty = max_dirty, a fixed size a captured graph can keep -- and
 * *n_found_dev, the number of changed non-empty blocks found.  If that
 * exceeds max_dirty, the blocks the list has no room for keep their old
 * snapshot and are found again by the next call.  Blocks that became empty
 * are recorded, not listed.  Changes of a cell's contents in place are not
 * structural and are not seen (the caller lists such blocks itself).  Order
 * of the listed pairs is unspecified. */
int qsa_detect_dirty_blocks(const qsa_dims *dims, const qsa_seqs *seqs, int32_t *snapshot_dev,
                            int32_t *dirty_dev, int32_t max_dirty, uint32_t *n_found_dev,
                            void *stream);

/* 1. Pooled-key update  [ISSUE lever2; lever2b for the device-side block
 * membership: the members of block b are positions b*r .. b*r+r-1, read
 * through the cell table when the caller gives one].
 *
 * For every entry (seq, block) of dirty_dev (int32 pairs, n_dirty of them;
 * callers pad the list to a power of two >= 4 with (-1, -1) so a captured
 * graph keeps its shape): with m = min(r, n_cells[seq] - block*r) present
 * cells, the block's pooled key is
 *   a_t   = (kidx[c0][t] + ... + kidx[c0+m-1][t]) / m        (fp32, in order)
 *   ms    = T(a*a) / d_idx,  inv = 1 / sqrt(ms + rms_eps)   (correctly rounded)
 *   n_t   = a_t * inv  (* idx_norm_w[t] if given)
 *   key   = RoPE(n, position block*r)
 * where T is the stride-halving pairwise fp32 sum (h = d/2, d/4, ..., 1:
 * v[t] += v[t+h]).  The RoPE angle pos*omega_t and its cosine and sine are
 * evaluated in fp64 and rounded once to fp32; omega_t = theta^(-2t/d) is
 * formed in fp64 from nested square roots of theta multiplied over the set
 * bits of t.  Both `pooled_dev` and, if non-NULL, `pooled_bf16_dev` are
 * written.  Entries with seq < 0 or seq >= n_seq, or whose block has no
 * present cell or lies beyond cap_cells/r, are skipped.  The result does not
 * depend on the order of the list; listing a block twice recomputes it twice.
 * Listing every block of a sequence rebuilds it from scratch ("resume"). */
int qsa_update_pooled_keys(const qsa_dims *dims, const qsa_seqs *seqs,
                           const void *kidx_dev, const int32_t *dirty_dev,
                           int32_t n_dirty, float *pooled_dev,
                           uint16_t *pooled_bf16_dev, void *stream);

/* 2. Block scores  [ISSUE lever3; the device-side causal bias of the
 * llama.cpp-multigpu README, section 5, LLAMA_QSA_BIAS_DEVICE].
 *
 * For each query: q' = RoPE(q_idx, q_pos) (as above, in fp32);
 *   scores[i][b] = T(q' * pooled[q_seq][b])   for b < nc,
 *   scores[i][b] = -inf                       for nc <= b < nb_max.
 * mode QSA_SCORE_F32 multiplies in fp32 (each product rounded) and sums in
 * order T: the result is fixed to the last bit.  mode QSA_SCORE_BF16 rounds
 * q' and the keys to bf16 (pooled_bf16_dev) and contracts them on the matrix
 * cores with fp32 accumulation: products are exact, the sum order is the
 * hardware's, so each score is within 2*(d_idx-1)*2^-24*sum|q'_t k_t| of the
 * T-ordered bf16 score.  ld_scores >= nb_max; nb_max <= cap_cells/r.
 * Mode QSA_SCORE_BF16 needs the workspace QSA_OP_SCORE_BF16 reports (the
 * roped bf16 queries); mode QSA_SCORE_F32 needs none (ws may be NULL). */
int qsa_score_blocks(const qsa_dims *dims, const qsa_seqs *seqs,
                     const float *q_idx_dev, const int32_t *q_seq_dev,
                     const int32_t *q_pos_dev, int32_t n_q,
                     const float *pooled_dev, const uint16_t *pooled_bf16_dev,
                     int32_t nb_max, float *scores_dev, int64_t ld_scores,
                     int32_t mode, void *ws_dev, size_t ws_bytes, void *stream);

/* 3. Block top-k and expansion  [ISSUE lever3: blocks are selected first and
 * only the selected ones are expanded to cells; goodbadwolf's n_kv_max].
 *
 * Per query, the candidates are the blocks b < min(nc, nb_max) with a finite
 * score.  They are ranked by score, descending, ties to the lower block index
 * (-0 equals +0), and the first min(top_k/r, count) are kept.  Output:
 * sel_blocks in ascending order; sel_cells = each kept block's r cells,
 * ascending, then the tail cells r*nc .. q_pos; n_sel = r*kept + tail_len
 * (<= top_k + r - 1).  Unused entries are -1.  Exact: the set is the one the
 * ranking defines, bit for bit.  No workspace is needed (ws may be NULL). */
int qsa_select_topk_blocks(const qsa_dims *dims, const qsa_seqs *seqs,
                           const float *scores_dev, int64_t ld_scores,
                           const int32_t *q_seq_dev, const int32_t *q_pos_dev,
                           int32_t n_q, int32_t nb_max, int32_t *sel_blocks_dev,
                           int32_t *sel_cells_dev, int32_t *n_sel_dev, void *ws_dev,
                           size_t ws_bytes, void *stream);

/* 1+2+3 for prefill  [ISSUE lever2 and lever3]: the pooled-key update of the
 * dirty list (n_dirty may be 0), then for each query the exact top-k of
 * qsa_select_topk_blocks over the scores of mode QSA_SCORE_BF16 taken in the
 * canonical order T -- the bf16-rounded q' and keys, exact products, the T
 * sum -- without writing a score matrix.  The contraction runs on the matrix
 * cores; their sums differ from T's by at most Delta_i (a bound from |q'_i|
 * and the RMS-normed keys' norm), so a first pass keeps each query's
 * largest matrix-core score of every 16-block subgroup; tau_i, the
 * (top_k/r)-th largest of those, less 2 Delta_i is a threshold below which
 * no block of the exact top-k can score; a second pass marks the blocks
 * above it, and only those are rescored in order T for the exact selection:
 * sel_blocks, sel_cells and n_sel equal those of qsa_select_topk_blocks over
 * T-ordered bf16 scores bit for bit (ties to the lower block).  If a query
 * marks more than 4096 blocks it rescores every causal block (correct,
 * slower).
 *   pooled_bf16_dev: required (the update writes it; the scores read it).
 *   Workspace: qsa_workspace_size(QSA_OP_SCORE_SELECT_PREFILL, n_q, nb_max)
 *   bytes, 16-byte aligned, no initial contents required.
 * Needs nb_max <= 131072 (else QSA_ENOTSUP). */
int qsa_score_select_prefill(const qsa_dims *dims, const qsa_seqs *seqs, const void *kidx_dev,
                             const int32_t *dirty_dev, int32_t n_dirty, float *pooled_dev,
                             uint16_t *pooled_bf16_dev, const float *q_idx_dev,
                             const int32_t *q_seq_dev, const int32_t *q_pos_dev, int32_t n_q,
                             int32_t nb_max, int32_t *sel_blocks_dev, int32_t *sel_cells_dev,
                             int32_t *n_sel_dev, void *ws_dev, size_t ws_bytes, void *stream);

/* 1+2+3 for decode: the pooled-key update of the dirty list (n_dirty may be
 * 0), then exactly qsa_score_blocks (mode QSA_SCORE_F32) and
 * qsa_select_topk_blocks -- the same pooled keys, the same scores (written
 * to scores_dev) and the same selection, bit for bit -- in two launches,
 * also available as two calls:
 *   qsa_decode_score_candidates writes the dirty blocks and scores every
 *     block (a workgroup that holds a dirty block recomputes it in registers
 *     rather than reading it), keeping in the workspace the best keys of
 *     each group of 64 blocks (16 while nb_max <= 16384, 8 up to 32768, else
 *     4; when the call's queries overflow the fused selection + attention
 *     grid of qsa_decode_select_attend -- n_q * ceil((top_k + r - 1) / 32)
 *     * (4 for 16 heads over 2 KV heads) > 512 -- 16 up to 24576, 8 up to
 *     49152, else 6) and the largest key each group dropped;
 *   qsa_decode_select_candidates selects from those, re-admitting all keys
 *     of any group whose dropped key could compete (or re-reading the score
 *     row if more than 32 groups could), so the selection is exact.
 * Workspace: qsa_workspace_size(QSA_OP_SCORE_SELECT, n_q, nb_max) bytes,
 * 16-byte aligned, no initial contents required; the two calls must get the
 * same workspace, scores and geometry, and calls that share a workspace must
 * not overlap.  The split calls need nb_max <= 131072 (else QSA_ENOTSUP);
 * qsa_score_select_decode then falls back to the three general calls. */
int qsa_score_select_decode(const qsa_dims *dims, const qsa_seqs *seqs, const void *kidx_dev,
                            const int32_t *dirty_dev, int32_t n_dirty, float *pooled_dev,
                            uint16_t *pooled_bf16_dev, const float *q_idx_dev,
                            const int32_t *q_seq_dev, const int32_t *q_pos_dev, int32_t n_q,
                            int32_t nb_max, float *scores_dev, int64_t ld_scores,
                            int32_t *sel_blocks_dev, int32_t *sel_cells_dev,
                            int32_t *n_sel_dev, void *ws_dev, size_t ws_bytes, void *stream);

int qsa_decode_score_candidates(const qsa_dims *dims, const qsa_seqs *seqs,
                                const void *kidx_dev, const int32_t *dirty_dev,
                                int32_t n_dirty, float *pooled_dev, uint16_t *pooled_bf16_dev,
                                const float *q_idx_dev, const int32_t *q_seq_dev,
                                const int32_t *q_pos_dev, int32_t n_q, int32_t nb_max,
                                float *scores_dev, int64_t ld_scores, void *ws_dev,
                                size_t ws_bytes, void *stream);

int qsa_decode_select_candidates(const qsa_dims *dims, const qsa_seqs *seqs,
                                 const int32_t *q_seq_dev, const int32_t *q_pos_dev,
                                 int32_t n_q, int32_t nb_max, const float *scores_dev,
                                 int64_t ld_scores, int32_t *sel_blocks_dev,
                                 int32_t *sel_cells_dev, int32_t *n_sel_dev,
                                 const void *ws_dev, size_t ws_bytes, void *stream);

/* 4. Sparse attention  [ISSUE lever1: attention runs over the top-k set
 * only; DISC: q8_0 rows are dequantised inside the gather, never the whole
 * cache].
 *
 * For query i and head h (KV head h / (n_head/n_head_kv)), over the n_sel[i]
 * cells c_j listed in sel_cells[i]:
 *   l_j = kq_scale * <q[i][h], K[c_j]>,  w = softmax(l),
 *   out[i][h] = sum_j w_j * V[c_j]
 * Decode dequantises K and V to fp32 and accumulates in fp32.  Prefill runs
 * both products on the matrix cores with fp16 operands and fp32 sums (q *
 * kq_scale, P and V -- q8_0 V as int8 times its scale -- rounded to fp16;
 * q8_0 K enters as exact integers with its block scale applied to the fp32
 * partial sum; f32 K rounded to fp16), so it agrees with decode to about
 * 1e-3 absolute for unit-scale inputs.  Cells outside 0 ..
 * min(n_cells, cap_cells)-1 are ignored; an empty set gives zeros.  Decode is
 * tuned for few queries (split over cells, then a combine), prefill for many.
 * Both need the workspace qsa_workspace_size reports.  QSA_EINVAL if the
 * cache has 2^31 rows (n_seq * cap_cells * n_head_kv) or more. */
int qsa_sparse_attn_decode(const qsa_dims *dims, const qsa_seqs *seqs,
                           const float *q_dev, const int32_t *q_seq_dev,
                           int32_t n_q, const void *k_cache_dev,
                           const void *v_cache_dev, const int32_t *sel_cells_dev,
                           const int32_t *n_sel_dev, float *out_dev, void *ws_dev,
                           size_t ws_bytes, void *stream);

int qsa_sparse_attn_prefill(const qsa_dims *dims, const qsa_seqs *seqs,
                            const float *q_dev, const int32_t *q_seq_dev,
                            int32_t n_q, const void *k_cache_dev,
                            const void *v_cache_dev, const int32_t *sel_cells_dev,
                            const int32_t *n_sel_dev, float *out_dev, void *ws_dev,
                            size_t ws_bytes, void *stream);

/* 4 for several decode tokens per sequence over the union of their lists
 * [ISSUE goodbadwolf's comment, "Why the two phases disagree": with a few
 * query tokens per sequence -- a speculative verify step, the end of a chunk
 * -- each token has its own top-k set, and a gather per token reads the rows
 * their sets share once per token].  The same attention as
 * qsa_sparse_attn_prefill, per query, but each K/V row is loaded once for
 * every token of its group that lists it.
 *
 * Queries are taken t_group (1 .. 8) at a time in order (the last group may
 * be shorter).  Per group, the rows of every token's listed cells (cells in
 * 0 .. min(n_cells, cap_cells)-1 of its own sequence, first n_sel entries)
 * form one ascending list with a bit per token that holds the row; each row
 * is staged once per run of 128 and scored for every query head of the group,
 * a token's softmax skipping the rows it does not hold.  When the group's
 * tokens are in one sequence and each list strictly ascends (as the
 * selection calls produce them), equal cells fold into one entry; otherwise
 * the lists are concatenated (the same result, without the sharing).
 * Arithmetic as in prefill: fp16 operands on the matrix cores, fp32 sums.
 *
 *   t_group    tokens per group, 1 .. 8
 *   ws_dev     qsa_workspace_size(QSA_OP_ATTN_DECODE_UNION, n_q, t_group)
 *              bytes, 16-byte aligned
 * Other arguments as qsa_sparse_attn_decode.  QSA_EINVAL for t_group outside
 * 1 .. 8; QSA_ENOTSUP unless kv_type is QSA_KV_Q8_0, the sequences have no
 * cell table, cap_cells < 2^28, n_head / n_head_kv is 4, 8 or 16, and
 * t_group * (top_k + r - 1) <= 16448 (8 tokens of top_k 2048, r <= 9). */
int qsa_sparse_attn_decode_union(const qsa_dims *dims, const qsa_seqs *seqs,
                                 const float *q_dev, const int32_t *q_seq_dev, int32_t n_q,
                                 int32_t t_group, const void *k_cache_dev,
                                 const void *v_cache_dev, const int32_t *sel_cells_dev,
                                 const int32_t *n_sel_dev, float *out_dev, void *ws_dev,
                                 size_t ws_bytes, void *stream);

/* 4 for decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): exactly qsa_sparse_attn_decode -- the same
 * kernels, the same results bit for bit -- with the partial attention states
 * kept in a scratch array the library holds on each GPU (8 MiB: 65 runs x
 * n_head x 258 floats per query at top_k 2048, r 4 -- 7 queries of 16 heads).
 * Calls needing more return QSA_EWS.  The call allocates nothing; its first
 * call on a device looks up that device's scratch address (the current
 * device).  Every call on a GPU shares that GPU's array: calls that overlap
 * on one GPU (other streams, other threads) race and must be serialised by
 * the caller.  The scratch needs no initial contents. */
int qsa_sparse_attn_decode_noalloc(const qsa_dims *dims, const qsa_seqs *seqs,
                                   const float *q_dev, const int32_t *q_seq_dev, int32_t n_q,
                                   const void *k_cache_dev, const void *v_cache_dev,
                                   const int32_t *sel_cells_dev, const int32_t *n_sel_dev,
                                   float *out_dev, void *stream);

/* 3+4 for decode, fused  [ISSUE lever3 then lever1: the block top-k, expanded
 * to cells, is the set attention visits]: exactly qsa_decode_select_candidates
 * followed by qsa_sparse_attn_decode over its output, in one workgroup grid
 * plus the merge of partial states.  Every attention workgroup derives the
 * query's exact kept set from the candidates that qsa_decode_score_candidates
 * left in ws_idx (the set is unique, so all derive the same one) and takes
 * its 32 cells of the ascending cell list straight from on-chip memory; one
 * workgroup per query also writes sel_blocks, sel_cells and n_sel.  The
 * selection outputs equal the two calls' bit for bit, and so does out (the
 * same arithmetic in the same order).
 *   ws_idx:  the workspace qsa_decode_score_candidates filled (same n_q,
 *            nb_max, scores and geometry); read only.
 *   ws_attn: qsa_workspace_size(QSA_OP_ATTN_DECODE, n_q) bytes, 16-byte
 *            aligned, no initial contents required.
 * Needs nb_max <= 65536 (contexts up to 262144 cells), else QSA_ENOTSUP: use
 * the two calls.  Calls sharing a workspace must not overlap. */
int qsa_decode_select_attend(const qsa_dims *dims, const qsa_seqs *seqs,
                             const int32_t *q_seq_dev, const int32_t *q_pos_dev, int32_t n_q,
                             int32_t nb_max, const float *scores_dev, int64_t ld_scores,
                             int32_t *sel_blocks_dev, int32_t *sel_cells_dev,
                             int32_t *n_sel_dev, const void *ws_idx_dev, size_t ws_idx_bytes,
                             const float *q_dev, const void *k_cache_dev,
                             const void *v_cache_dev, float *out_dev, void *ws_attn_dev,
                             size_t ws_attn_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
