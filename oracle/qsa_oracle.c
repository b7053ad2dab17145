/*
 * qsa_oracle.c -- plain, slow CPU oracle for the QSA sparse-attention step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file; only the test-suite, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or constant generator
 * with the HIP library.
 *
 * Sources (web pages, cited by title and section):
 *   [ISSUE]  llama.cpp issue #28734, "Eval bug: qwen4exp (Qwen3.8-Flash-Next)
 *            CUDA: decode slows linearly with context", the LLM-generated fix
 *            summary and its sections lever1, lever3, lever2, lever2b; and the
 *            comment by goodbadwolf, "Why the two phases disagree".
 *   [DISC]   llama.cpp discussion #30071, "Qwen3.8-Flash-Next on 6x3090 and
 *            6x4090 without NVLink ...", the paragraph on the two problems.
 *
 * Floating point.  Everything that decides an integer (the block selection)
 * is computed in fp32 in one fixed, documented order, because the GPU takes
 * the same decision in fp32.  Attention, which decides no integer, is computed
 * in fp64.  Build with -ffp-contract=off and without fast-math: every fp32
 * multiply and add below must round separately.
 *
 * Readings of points the pages leave open:
 *   - RoPE is the split-half ("NeoX") form over all d dims, pairs (t, t+d/2),
 *     inverse frequency theta^(-2t/d), angle computed in fp64 and its cosine
 *     and sine rounded to fp32; a pooled block sits at position b*r.
 *   - The fixed fp32 summation order T is the stride-halving pairwise tree.
 *   - The score is a plain dot product of the roped query and the pooled key.
 *   - The incomplete tail block is never scored; its cells are always kept.
 *   - Ties in the block ranking go to the lower block index; -0 equals +0.
 *
 * Threads.  Built with OpenMP, three loops run their independent iterations
 * on several threads: the dirty entries of a pooled-key update, the blocks of
 * a score row and the heads of an attention call.  Each iteration computes
 * what it computes single-threaded, in the same order, so results do not
 * depend on the thread count (qo_set_threads; 1 by default).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define QO_MAX_D 1024

/* ------------------------------------------------------------------------ */
/* Threads                                                                   */
/* ------------------------------------------------------------------------ */

static int qo_threads = 1;

/* Threads the parallel loops use (n >= 1; capped by what OpenMP offers).
 * Returns the count now in force: 1 when built without OpenMP. */
int qo_set_threads(int n)
{
#ifdef _OPENMP
    if (n < 1)
        n = 1;
    int mx = omp_get_num_procs();
    qo_threads = n < mx ? n : mx;
#else
    (void)n;
    qo_threads = 1;
#endif
    return qo_threads;
}

/* ------------------------------------------------------------------------ */
/* Scalars                                                                   */
/* ------------------------------------------------------------------------ */

/* IEEE-754 binary16 -> binary32, exactly (every half is a float). */
float qo_half_to_float(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int mant = h & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)mant, -24); /* subnormal: mant * 2^-24 */
    else if (expo == 31)
        v = mant ? NAN : INFINITY;
    else
        v = ldexp((double)(mant + 1024), expo - 25); /* (1.mant) * 2^(e-15) */
    return (float)(sign ? -v : v);
}

/* fp32 -> bf16 with round-to-nearest-even, returned as the fp32 it denotes. */
float qo_round_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) /* NaN stays NaN */
        return x;
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    u &= 0xffff0000u;
    float y;
    memcpy(&y, &u, 4);
    return y;
}

/* ------------------------------------------------------------------------ */
/* T: the fixed fp32 summation order                                          */
/* ------------------------------------------------------------------------ */

/* Stride-halving pairwise sum of n (a power of two) fp32 values:
 * for h = n/2, n/4, ..., 1:  v[t] <- fl(v[t] + v[t+h]) for t < h; result v[0].
 * Overwrites v. */
float qo_tree_sum(float *v, int n)
{
    for (int h = n / 2; h >= 1; h /= 2)
        for (int t = 0; t < h; t++)
            v[t] = v[t] + v[t + h];
    return v[0];
}

/* T applied to the elementwise products a[t]*b[t] (each product rounded). */
float qo_tree_dot(const float *a, const float *b, int n)
{
    float p[QO_MAX_D];
    for (int t = 0; t < n; t++)
        p[t] = a[t] * b[t];
    return qo_tree_sum(p, n);
}

/* ------------------------------------------------------------------------ */
/* RoPE                                                                      */
/* ------------------------------------------------------------------------ */

/* Inverse frequencies omega_t = theta^(-2t/d), t < d/2, in fp64.
 * d/2 must be a power of two, 2^m.  Then theta^(-2t/d) = theta^(-t/2^m) is the
 * product, over the set bits k of t, of theta^(-1/2^(m-k)), and
 * theta^(1/2^j) is j nested square roots of theta.  Only correctly rounded
 * IEEE operations are used (sqrt, divide, multiply), in ascending k order, so
 * the value is fixed to the last bit.  Returns -1 if d/2 is not a power of two. */
int qo_inv_freq(double theta, int d, double *omega)
{
    int half = d / 2, m = 0;
    if (d <= 0 || d % 2)
        return -1;
    while ((1 << m) < half)
        m++;
    if ((1 << m) != half)
        return -1;
    double root[32];
    root[0] = theta;
    for (int j = 1; j <= m; j++)
        root[j] = sqrt(root[j - 1]);
    for (int t = 0; t < half; t++) {
        double w = 1.0;
        for (int k = 0; k < m; k++)
            if ((t >> k) & 1)
                w = w * (1.0 / root[m - k]);
        omega[t] = w;
    }
    return 0;
}

/* cos and sin of the angle pos*omega_t, angle and functions in fp64, each
 * result rounded once to fp32. */
int qo_rope_coeffs(double theta, int d, int64_t pos, float *c, float *s)
{
    double omega[QO_MAX_D / 2];
    if (qo_inv_freq(theta, d, omega))
        return -1;
    for (int t = 0; t < d / 2; t++) {
        double phi = (double)pos * omega[t];
        c[t] = (float)cos(phi);
        s[t] = (float)sin(phi);
    }
    return 0;
}

/* Split-half rotation of x (d values) to position pos, in fp32:
 *   out[t]     = x[t]*c_t     - x[t+d/2]*s_t
 *   out[t+d/2] = x[t+d/2]*c_t + x[t]*s_t
 * i.e. (x[t] + i x[t+d/2]) multiplied by exp(i * pos * omega_t). */
int qo_rope(const float *x, int d, int64_t pos, double theta, float *out)
{
    float c[QO_MAX_D / 2], s[QO_MAX_D / 2];
    if (qo_rope_coeffs(theta, d, pos, c, s))
        return -1;
    int half = d / 2;
    for (int t = 0; t < half; t++) {
        float a = x[t], b = x[t + half];
        float ac = a * c[t], bs = b * s[t];
        float bc = b * c[t], as = a * s[t];
        out[t] = ac - bs;
        out[t + half] = bc + as;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* O1: the pooled key of one block  [ISSUE lever2]                          */
/* ------------------------------------------------------------------------ */

/* cells: m rows of d fp32 (the block's present cells, in position order).
 * Mean over the m cells (left-to-right fp32 sum, then one divide by m), then
 * RMS-norm (mean of squares by T, divided by d; 1/sqrt(ms+eps) with correctly
 * rounded sqrt and divide; optional per-dim weight gamma), then RoPE at pos. */
int qo_pooled_key(const float *cells, int m, int d, float eps,
                  const float *gamma, int64_t pos, double theta, float *out)
{
    float a[QO_MAX_D], sq[QO_MAX_D], nrm[QO_MAX_D];
    if (m < 1 || d > QO_MAX_D)
        return -1;
    for (int t = 0; t < d; t++) {
        float acc = cells[t];
        for (int j = 1; j < m; j++)
            acc = acc + cells[(size_t)j * d + t];
        a[t] = acc / (float)m;
    }
    for (int t = 0; t < d; t++)
        sq[t] = a[t] * a[t];
    float ms = qo_tree_sum(sq, d) / (float)d;
    float inv = 1.0f / sqrtf(ms + eps);
    for (int t = 0; t < d; t++) {
        nrm[t] = a[t] * inv;
        if (gamma)
            nrm[t] = nrm[t] * gamma[t];
    }
    return qo_rope(nrm, d, pos, theta, out);
}

/* Pooled key of block b of a sequence whose per-cell keys are kidx[n_cells][d]
 * (block b covers cells b*r .. min(b*r+r, n_cells)-1). */
int qo_block_key(const float *kidx, int64_t n_cells, int d, int r, float eps,
                 const float *gamma, double theta, int64_t b, float *out)
{
    int64_t first = b * r;
    if (b < 0 || first >= n_cells)
        return -1;
    int m = (int)((n_cells - first) < r ? (n_cells - first) : r);
    return qo_pooled_key(kidx + (size_t)first * d, m, d, eps, gamma, first,
                         theta, out);
}

/* Apply a dirty list to a pooled cache.  kidx: [n_seq][cap_cells][d];
 * pooled: [n_seq][cap_blocks][d]; dirty: n_dirty (seq, block) pairs.  Pairs
 * with seq < 0, or whose block has no present cell, are skipped.  This is the
 * incremental form; re-running qo_block_key over every block is the slow form
 * it must equal bit for bit [ISSUE lever2]. */
int qo_update_pooled(const float *kidx, int64_t cap_cells, const int32_t *n_cells,
                     int n_seq, int d, int r, float eps, const float *gamma,
                     double theta, const int32_t *dirty, int n_dirty,
                     float *pooled, int64_t cap_blocks)
{
    int err = 0;
    /* (a block listed twice is written twice with the same value) */
#pragma omp parallel for num_threads(qo_threads) schedule(static) reduction(| : err)
    for (int i = 0; i < n_dirty; i++) {
        int32_t s = dirty[2 * i], b = dirty[2 * i + 1];
        if (s < 0 || s >= n_seq || b < 0 || b >= cap_blocks)
            continue;
        int64_t nc = n_cells[s];
        if ((int64_t)b * r >= nc)
            continue;
        if (qo_block_key(kidx + (size_t)s * cap_cells * d, nc, d, r, eps, gamma,
                         theta, b, pooled + ((size_t)s * cap_blocks + b) * d))
            err = 1;
    }
    return err ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* O2/O3: block scores  [ISSUE lever3]                                       */
/* ------------------------------------------------------------------------ */

/* Number of complete blocks visible from position pos: floor((pos+1)/r). */
int64_t qo_complete_blocks(int64_t pos, int r) { return (pos + 1) / r; }

/* Scores of one query at position pos against pooled[nb][d] (row-major):
 * q' = RoPE(q_idx, pos); s_b = T(q' * pooled_b) for b < nc, -inf for
 * nc <= b < nb_out.  If bf16 != 0, q' and each key are first rounded to bf16
 * (the prefill form; the products are then exact in fp32). */
int qo_score_query(const float *q_idx, int d, int64_t pos, double theta, int r,
                   const float *pooled, int64_t nb_avail, int64_t nb_out,
                   int bf16, float *scores)
{
    float qr[QO_MAX_D];
    if (qo_rope(q_idx, d, pos, theta, qr))
        return -1;
    if (bf16)
        for (int t = 0; t < d; t++)
            qr[t] = qo_round_bf16(qr[t]);
    int64_t nc = qo_complete_blocks(pos, r);
    if (nc > nb_avail)
        return -1;
#pragma omp parallel for num_threads(qo_threads) schedule(static)
    for (int64_t b = 0; b < nb_out; b++) {
        float k[QO_MAX_D];
        if (b >= nc) {
            scores[b] = -INFINITY;
            continue;
        }
        const float *kb = pooled + (size_t)b * d;
        for (int t = 0; t < d; t++)
            k[t] = bf16 ? qo_round_bf16(kb[t]) : kb[t];
        scores[b] = qo_tree_dot(qr, k, d);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* O4: block top-k and expansion  [ISSUE lever3, goodbadwolf's comment]      */
/* ------------------------------------------------------------------------ */

typedef struct {
    float s;
    int64_t b;
} qo_cand;

static int qo_cmp_rank(const void *x, const void *y)
{
    const qo_cand *a = (const qo_cand *)x, *b = (const qo_cand *)y;
    if (a->s > b->s) return -1; /* higher score first (-0 == +0 here) */
    if (a->s < b->s) return 1;
    return (a->b > b->b) - (a->b < b->b); /* then lower block index */
}

static int qo_cmp_i64(const void *x, const void *y)
{
    int64_t a = *(const int64_t *)x, b = *(const int64_t *)y;
    return (a > b) - (a < b);
}

/* Selection for one query at position pos.  Candidates are the complete
 * blocks b < floor((pos+1)/r) with a finite score.  They are ranked by score
 * (descending), ties to the lower block index, and the first min(top_k/r,
 * count) are kept, listed in ascending block order in sel_blocks.  sel_cells
 * gets each kept block's r cells in ascending order followed by the tail
 * cells r*nc .. pos.  Returns the number of cells (n_sel), writes the number
 * of blocks to *n_blocks; -1 on bad arguments. */
int qo_select(const float *scores, int64_t pos, int r, int top_k,
              int32_t *sel_blocks, int32_t *sel_cells, int32_t *n_blocks)
{
    if (pos < 0 || r < 1 || top_k < r || top_k % r)
        return -1;
    int64_t nc = qo_complete_blocks(pos, r);
    int64_t B = top_k / r;
    qo_cand *c = (qo_cand *)malloc(sizeof(qo_cand) * (size_t)(nc > 0 ? nc : 1));
    int64_t *keep = (int64_t *)malloc(sizeof(int64_t) * (size_t)(B > 0 ? B : 1));
    if (!c || !keep) {
        free(c);
        free(keep);
        return -1;
    }
    int64_t n = 0;
    for (int64_t b = 0; b < nc; b++)
        if (isfinite(scores[b])) {
            c[n].s = scores[b];
            c[n].b = b;
            n++;
        }
    qsort(c, (size_t)n, sizeof(qo_cand), qo_cmp_rank);
    int64_t nk = n < B ? n : B;
    for (int64_t j = 0; j < nk; j++)
        keep[j] = c[j].b;
    qsort(keep, (size_t)nk, sizeof(int64_t), qo_cmp_i64);
    int64_t nsel = 0;
    for (int64_t j = 0; j < nk; j++) {
        sel_blocks[j] = (int32_t)keep[j];
        for (int q = 0; q < r; q++)
            sel_cells[nsel++] = (int32_t)(keep[j] * r + q);
    }
    for (int64_t p = nc * r; p <= pos; p++) /* the tail rides along */
        sel_cells[nsel++] = (int32_t)p;
    *n_blocks = (int32_t)nk;
    free(c);
    free(keep);
    return (int)nsel;
}

/* The pages' slow form of the same selection: expand every complete block's
 * score to its r cells, sort all those cells by (score desc, cell asc), keep
 * the first r*min(top_k/r, count), then add the tail cells; output ascending.
 * It must equal qo_select [ISSUE lever3: selecting blocks first only shrinks
 * the sort]. */
int qo_select_dense_cells(const float *scores, int64_t pos, int r, int top_k,
                          int32_t *sel_cells)
{
    if (pos < 0 || r < 1 || top_k < r || top_k % r)
        return -1;
    int64_t nc = qo_complete_blocks(pos, r);
    int64_t ncell = nc * r;
    qo_cand *c = (qo_cand *)malloc(sizeof(qo_cand) * (size_t)(ncell > 0 ? ncell : 1));
    int64_t *keep = (int64_t *)malloc(sizeof(int64_t) * (size_t)(ncell + r + 1));
    if (!c || !keep) {
        free(c);
        free(keep);
        return -1;
    }
    int64_t n = 0, nfin = 0;
    for (int64_t cell = 0; cell < ncell; cell++) {
        float s = scores[cell / r];
        if (isfinite(s)) {
            c[n].s = s;
            c[n].b = cell;
            n++;
        }
    }
    nfin = n / r;
    qsort(c, (size_t)n, sizeof(qo_cand), qo_cmp_rank);
    int64_t B = top_k / r;
    int64_t nk = (nfin < B ? nfin : B) * r;
    for (int64_t j = 0; j < nk; j++)
        keep[j] = c[j].b;
    int64_t m = nk;
    for (int64_t p = ncell; p <= pos; p++)
        keep[m++] = p;
    qsort(keep, (size_t)m, sizeof(int64_t), qo_cmp_i64);
    for (int64_t j = 0; j < m; j++)
        sel_cells[j] = (int32_t)keep[j];
    free(c);
    free(keep);
    return (int)m;
}

/* ------------------------------------------------------------------------ */
/* O5: attention over the selected cells  [ISSUE lever1, DISC]              */
/* ------------------------------------------------------------------------ */

/* One KV row (one cell, one KV head) of D values, dequantised to fp32.
 * kv_type 0: fp32 row.  kv_type 1: q8_0 row, D/32 blocks of 34 bytes, each a
 * little-endian binary16 scale d followed by 32 int8 q; value = float(d)*q
 * (exact in fp32).  kv_type 2: D binary16 values, the KV type of the fix of
 * llama.cpp issue #28734 (fix summary); value = float(h), exact. */
static void qo_row(const void *cache, int kv_type, int64_t row, int D, float *out)
{
    if (kv_type == 0) {
        memcpy(out, (const float *)cache + (size_t)row * D, sizeof(float) * D);
        return;
    }
    if (kv_type == 2) {
        const uint16_t *h = (const uint16_t *)cache + (size_t)row * D;
        for (int i = 0; i < D; i++) out[i] = qo_half_to_float(h[i]);
        return;
    }
    const uint8_t *p = (const uint8_t *)cache + (size_t)row * (D / 32) * 34;
    for (int k = 0; k < D / 32; k++) {
        const uint8_t *blk = p + 34 * k;
        float dsc = qo_half_to_float((uint16_t)(blk[0] | (blk[1] << 8)));
        for (int i = 0; i < 32; i++)
            out[32 * k + i] = dsc * (float)(int8_t)blk[2 + i];
    }
}

/* Softmax attention of one query over a given cell list, all heads, in fp64.
 * q: [H][D] fp32.  k_cache, v_cache: one sequence, rows indexed by
 * cell*Hk + kvh.  Head h reads KV head h / (H/Hk).  l_j = scale*<q_h, K_j>,
 * w_j = exp(l_j - max l), out_h = sum w_j V_j / sum w_j, rounded to fp32.
 * scale <= 0 means 1/sqrt(D).  An empty list gives zeros. */
int qo_attend(const float *q, int H, int Hk, int D, const void *k_cache,
              const void *v_cache, int kv_type, const int32_t *cells, int n,
              float scale, float *out)
{
    if (H <= 0 || Hk <= 0 || H % Hk || D <= 0 || D > QO_MAX_D || kv_type < 0 ||
        kv_type > 2 || (kv_type == 1 && D % 32))
        return -1;
    int G = H / Hk;
    double sc = scale > 0.0f ? (double)scale : 1.0 / sqrt((double)D);
    int err = 0;
#pragma omp parallel for num_threads(qo_threads) schedule(static) reduction(| : err)
    for (int h = 0; h < H; h++) {
        double acc[QO_MAX_D];
        float kr[QO_MAX_D], vr[QO_MAX_D];
        double *lg = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        if (!lg) {
            err = 1;
            continue;
        }
        int kvh = h / G;
        const float *qh = q + (size_t)h * D;
        double mx = -INFINITY;
        for (int j = 0; j < n; j++) {
            qo_row(k_cache, kv_type, (int64_t)cells[j] * Hk + kvh, D, kr);
            double dot = 0.0;
            for (int t = 0; t < D; t++)
                dot += (double)qh[t] * (double)kr[t];
            lg[j] = sc * dot;
            if (lg[j] > mx)
                mx = lg[j];
        }
        double den = 0.0;
        for (int t = 0; t < D; t++)
            acc[t] = 0.0;
        for (int j = 0; j < n; j++) {
            double w = exp(lg[j] - mx);
            den += w;
            qo_row(v_cache, kv_type, (int64_t)cells[j] * Hk + kvh, D, vr);
            for (int t = 0; t < D; t++)
                acc[t] += w * (double)vr[t];
        }
        for (int t = 0; t < D; t++)
            out[(size_t)h * D + t] = n > 0 ? (float)(acc[t] / den) : 0.0f;
        free(lg);
    }
    return err ? -1 : 0;
}

/* The pages' slow form: dense causal attention over every cell 0..pos with
 * the logits of cells outside the selected set forced to -inf (a mask), in
 * fp64.  sel_mask[c] != 0 marks a selected cell.  Equals qo_attend up to
 * rounding [ISSUE lever1: the sparse set is the finite entries of the mask]. */
int qo_attend_dense_masked(const float *q, int H, int Hk, int D,
                           const void *k_cache, const void *v_cache,
                           int kv_type, const uint8_t *sel_mask, int64_t pos,
                           float scale, float *out)
{
    if (H <= 0 || Hk <= 0 || H % Hk || D <= 0 || D > QO_MAX_D || pos < 0 || kv_type < 0 ||
        kv_type > 2 || (kv_type == 1 && D % 32))
        return -1;
    int G = H / Hk;
    double sc = scale > 0.0f ? (double)scale : 1.0 / sqrt((double)D);
    int64_t n = pos + 1;
    double *lg = (double *)malloc(sizeof(double) * (size_t)n);
    double acc[QO_MAX_D];
    float kr[QO_MAX_D], vr[QO_MAX_D];
    if (!lg)
        return -1;
    for (int h = 0; h < H; h++) {
        int kvh = h / G;
        const float *qh = q + (size_t)h * D;
        double mx = -INFINITY;
        for (int64_t c = 0; c < n; c++) {
            qo_row(k_cache, kv_type, c * Hk + kvh, D, kr);
            double dot = 0.0;
            for (int t = 0; t < D; t++)
                dot += (double)qh[t] * (double)kr[t];
            lg[c] = sel_mask[c] ? sc * dot : -INFINITY;
            if (lg[c] > mx)
                mx = lg[c];
        }
        double den = 0.0;
        for (int t = 0; t < D; t++)
            acc[t] = 0.0;
        for (int64_t c = 0; c < n; c++) {
            if (lg[c] == -INFINITY)
                continue;
            double w = exp(lg[c] - mx);
            den += w;
            qo_row(v_cache, kv_type, c * Hk + kvh, D, vr);
            for (int t = 0; t < D; t++)
                acc[t] += w * (double)vr[t];
        }
        for (int t = 0; t < D; t++)
            out[(size_t)h * D + t] = den > 0.0 ? (float)(acc[t] / den) : 0.0f;
    }
    free(lg);
    return 0;
}
