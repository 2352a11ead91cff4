/*
 * mla_oracle.c -- plain, slow, fp64 CPU oracle for weight-absorbed MLA decode.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the bench's
 * CPU-baseline leg may load this library.  It shares no code, header, table or
 * helper with the HIP path, and the HIP path never calls it.
 *
 * What it computes, with the sources it follows:
 *   absorbed query   q_abs[h,m] = sum_d q_nope[h,d] W_UK[h,d,m]
 *                    ("DeepSeek-MLA-Principle", matrix absorption 3), key
 *                    absorption; "MLA Matrix Absorption" sec. 2.1 and the
 *                    fig. of sec. 4.2; weight layout [n_heads, d_head, d_latent]
 *                    of the PyTorch decode module on the "DeepSeek MLA 架构详解"
 *                    page)
 *   scores           z_t = scale * (q_abs . c_t + q_rope . k_pe_t),
 *                    scale = 1/sqrt(d_h + d_r)   ("MLA Matrix Absorption" 4.1;
 *                    "DeepSeek-MLA-Principle" sec. 2 score formula)
 *   softmax          over the visible positions, max-subtracted, two passes
 *                    ("DeepSeek-MLA-Principle" sec. 2, softmax over j)
 *   latent output    o'[m] = sum_t p_t c_t[m]  (value absorption, same pages)
 *   up-projection    out[h,d] = sum_m W_UV[h,d,m] o'[m]
 *   split partials   the same softmax restricted to a contiguous range of
 *                    whole pages, returned normalised with its log-sum-exp;
 *                    the merge is the textbook log-sum-exp combination (the
 *                    pages only name "split-KV" in FlashMLA's list of ideas).
 * Causal rule for Sq query rows: row s of sequence b sees positions
 * t <= seq_len[b] - Sq + s (the sum over j <= t of eq. (10), with the new tokens
 * already appended as in the decode module).
 *
 * Stored inputs are decoded exactly: fp32, bf16 (the upper half of a binary32),
 * and OCP FP8 E4M3 (bias 7, no infinities, S.1111.111 = NaN) times a per-token
 * fp32 scale.  Every sum is taken sequentially in ascending index order in
 * double precision.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_E4M3 = 2, ORC_F64 = 3 };

typedef struct {
    int32_t B, Sq, H, d_h, d_c, d_r;
    int32_t page_size;
    int32_t max_pages;   /* row stride of block_table */
    double scale;
} orc_dims;

/* ---- exact decoding of storage formats (from the format definitions) ---- */

double orc_bf16_value(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int e = (bits >> 7) & 0xFF;
    int m = bits & 0x7F;
    double v;
    if (e == 0xFF) v = m ? NAN : INFINITY;
    else if (e == 0) v = ldexp((double)m, -126 - 7);           /* subnormal */
    else v = ldexp(1.0 + (double)m / 128.0, e - 127);
    return sign ? -v : v;
}

double orc_e4m3_value(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double v;
    if (e == 0xF && m == 0x7) v = NAN;
    else if (e == 0) v = ldexp((double)m / 8.0, 1 - 7);          /* subnormal */
    else v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

static double ld(const void *p, int dt, int64_t i)
{
    switch (dt) {
    case ORC_F32: return (double)((const float *)p)[i];
    case ORC_BF16: return orc_bf16_value(((const uint16_t *)p)[i]);
    case ORC_E4M3: return orc_e4m3_value(((const uint8_t *)p)[i]);
    default: return ((const double *)p)[i];
    }
}

/* Bulk decode, used by tests to obtain the exact values the oracle sees. */
void orc_decode_array(const void *src, int dt, int64_t n, double *dst)
{
    for (int64_t i = 0; i < n; ++i) dst[i] = ld(src, dt, i);
}

/* ---- cache access ------------------------------------------------------- */

typedef struct {
    const orc_dims *D;
    const void *c_kv; int kv_dt; const float *kv_scale;
    const void *k_pe; int pe_dt;
    const int32_t *block_table;
} cache_t;

/* offset of token t of sequence b: (physical page, slot) -> row index */
static int64_t cache_row(const cache_t *C, int b, int64_t t)
{
    const orc_dims *D = C->D;
    int64_t page = C->block_table[(int64_t)b * D->max_pages + t / D->page_size];
    return page * D->page_size + t % D->page_size;
}

static double cache_c(const cache_t *C, int64_t row, int m)
{
    double v = ld(C->c_kv, C->kv_dt, row * C->D->d_c + m);
    if (C->kv_dt == ORC_E4M3) v *= (double)C->kv_scale[row];
    return v;
}

static double cache_r(const cache_t *C, int64_t row, int r)
{
    return ld(C->k_pe, C->pe_dt, row * C->D->d_r + r);
}

/* number of positions query row s of sequence b may see */
static int64_t visible(const orc_dims *D, const int32_t *seq_lens, int b, int s)
{
    int64_t n = (int64_t)seq_lens[b] - D->Sq + 1 + s;
    return n > 0 ? n : 0;
}

/* ---- step 1: key absorption -------------------------------------------- */

void orc_absorb_q(const orc_dims *D, const void *q_nope, int q_dt,
                  const void *W_UK, int w_dt, double *q_abs)
{
    int64_t rows = (int64_t)D->B * D->Sq * D->H;
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < rows; ++row) {
        int h = (int)(row % D->H);
        for (int m = 0; m < D->d_c; ++m) {
            double acc = 0.0;
            for (int d = 0; d < D->d_h; ++d)
                acc += ld(q_nope, q_dt, row * D->d_h + d) *
                       ld(W_UK, w_dt, ((int64_t)h * D->d_h + d) * D->d_c + m);
            q_abs[row * D->d_c + m] = acc;
        }
    }
}

/* ---- steps 2-4 for one query row over positions [t0, t1) --------------------
 * qa: absorbed query (d_c doubles), qr: rope query (d_r doubles).
 * Writes the normalised latent output o[d_c] and returns the log-sum-exp
 * (natural log); an empty range gives o = 0 and -inf. */
static double attend(const cache_t *C, int b, const double *qa, const double *qr,
                     int64_t t0, int64_t t1, double *z, double *o)
{
    const orc_dims *D = C->D;
    for (int m = 0; m < D->d_c; ++m) o[m] = 0.0;
    if (t1 <= t0) return -INFINITY;
    /* scores */
    for (int64_t t = t0; t < t1; ++t) {
        int64_t row = cache_row(C, b, t);
        double content = 0.0, rope = 0.0;
        for (int m = 0; m < D->d_c; ++m) content += qa[m] * cache_c(C, row, m);
        for (int r = 0; r < D->d_r; ++r) rope += qr[r] * cache_r(C, row, r);
        z[t - t0] = D->scale * (content + rope);
    }
    /* pass 1: maximum; pass 2: exponentials and their sum */
    double M = -INFINITY;
    for (int64_t t = t0; t < t1; ++t) if (z[t - t0] > M) M = z[t - t0];
    double Z = 0.0;
    for (int64_t t = t0; t < t1; ++t) { z[t - t0] = exp(z[t - t0] - M); Z += z[t - t0]; }
    /* latent-space weighted sum */
    for (int64_t t = t0; t < t1; ++t) {
        int64_t row = cache_row(C, b, t);
        double p = z[t - t0] / Z;
        for (int m = 0; m < D->d_c; ++m) o[m] += p * cache_c(C, row, m);
    }
    return M + log(Z);
}

static void load_row(const void *src, int dt, int64_t row, int n, double *dst)
{
    for (int i = 0; i < n; ++i) dst[i] = ld(src, dt, row * n + i);
}

/* ---- split-KV partials ---------------------------------------------------
 * Split c of sequence b covers the sequence's pages [c*split_pages,
 * (c+1)*split_pages); within it, positions below the row's visible count.
 * o_part [B,Sq,H,S,d_c], lse_part [B,Sq,H,S]. */
void orc_decode_splitkv(const orc_dims *D, const void *q_abs, int qa_dt,
                        const void *q_rope, int qr_dt,
                        const void *c_kv, int kv_dt, const float *kv_scale,
                        const void *k_pe, int pe_dt,
                        const int32_t *block_table, const int32_t *seq_lens,
                        int num_splits, int split_pages,
                        double *o_part, double *lse_part)
{
    cache_t C = {D, c_kv, kv_dt, kv_scale, k_pe, pe_dt, block_table};
    int64_t rows = (int64_t)D->B * D->Sq * D->H;
    int64_t maxlen = 0;
    for (int b = 0; b < D->B; ++b) if (seq_lens[b] > maxlen) maxlen = seq_lens[b];
#pragma omp parallel
    {
        double *qa = malloc(sizeof(double) * (D->d_c + 1));
        double *qr = malloc(sizeof(double) * (D->d_r + 1));
        double *z = malloc(sizeof(double) * (maxlen + 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t row = 0; row < rows; ++row) {
            int b = (int)(row / ((int64_t)D->Sq * D->H));
            int s = (int)((row / D->H) % D->Sq);
            load_row(q_abs, qa_dt, row, D->d_c, qa);
            load_row(q_rope, qr_dt, row, D->d_r, qr);
            int64_t n = visible(D, seq_lens, b, s);
            for (int c = 0; c < num_splits; ++c) {
                int64_t t0 = (int64_t)c * split_pages * D->page_size;
                int64_t t1 = t0 + (int64_t)split_pages * D->page_size;
                if (t1 > n) t1 = n;
                lse_part[row * num_splits + c] =
                    attend(&C, b, qa, qr, t0, t1, z, o_part + (row * num_splits + c) * D->d_c);
            }
        }
        free(qa); free(qr); free(z);
    }
}

/* ---- split partials over explicit page ranges ------------------------------
 * Split c of sequence b covers the sequence's pages [page_begin[b*S+c],
 * page_end[b*S+c]) (empty when begin >= end); within it, positions below the
 * row's visible count.  Same arithmetic as orc_decode_splitkv, for a split
 * plan given as data.  o_part [B,Sq,H,S,d_c], lse_part [B,Sq,H,S]. */
void orc_decode_page_ranges(const orc_dims *D, const void *q_abs, int qa_dt,
                            const void *q_rope, int qr_dt,
                            const void *c_kv, int kv_dt, const float *kv_scale,
                            const void *k_pe, int pe_dt,
                            const int32_t *block_table, const int32_t *seq_lens,
                            int num_splits, const int32_t *page_begin, const int32_t *page_end,
                            double *o_part, double *lse_part)
{
    cache_t C = {D, c_kv, kv_dt, kv_scale, k_pe, pe_dt, block_table};
    int64_t rows = (int64_t)D->B * D->Sq * D->H;
    int64_t maxlen = 0;
    for (int b = 0; b < D->B; ++b) if (seq_lens[b] > maxlen) maxlen = seq_lens[b];
#pragma omp parallel
    {
        double *qa = malloc(sizeof(double) * (D->d_c + 1));
        double *qr = malloc(sizeof(double) * (D->d_r + 1));
        double *z = malloc(sizeof(double) * (maxlen + 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t row = 0; row < rows; ++row) {
            int b = (int)(row / ((int64_t)D->Sq * D->H));
            int s = (int)((row / D->H) % D->Sq);
            load_row(q_abs, qa_dt, row, D->d_c, qa);
            load_row(q_rope, qr_dt, row, D->d_r, qr);
            int64_t n = visible(D, seq_lens, b, s);
            for (int c = 0; c < num_splits; ++c) {
                int64_t t0 = (int64_t)page_begin[b * num_splits + c] * D->page_size;
                int64_t t1 = (int64_t)page_end[b * num_splits + c] * D->page_size;
                if (t1 > n) t1 = n;
                lse_part[row * num_splits + c] =
                    attend(&C, b, qa, qr, t0, t1, z, o_part + (row * num_splits + c) * D->d_c);
            }
        }
        free(qa); free(qr); free(z);
    }
}

/* ---- log-sum-exp merge of split partials ---------------------------------
 * lse = M + ln sum_c exp(lse_c - M), o = sum_c exp(lse_c - lse) o_c with
 * M = max_c lse_c.  Splits with lse_c = -inf carry no weight and their o_c is
 * not read.  A row with no visible position gets o = 0, lse = -inf. */
void orc_combine_lse(const orc_dims *D, int num_splits, const void *o_part, int o_dt,
                     const double *lse_part, double *o_latent, double *lse_out)
{
    int64_t rows = (int64_t)D->B * D->Sq * D->H;
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < rows; ++row) {
        const double *l = lse_part + row * num_splits;
        double M = -INFINITY;
        for (int c = 0; c < num_splits; ++c) if (l[c] > M) M = l[c];
        double *o = o_latent + row * D->d_c;
        for (int m = 0; m < D->d_c; ++m) o[m] = 0.0;
        if (M == -INFINITY) { if (lse_out) lse_out[row] = -INFINITY; continue; }
        double S = 0.0;
        for (int c = 0; c < num_splits; ++c) if (l[c] != -INFINITY) S += exp(l[c] - M);
        double lse = M + log(S);
        for (int c = 0; c < num_splits; ++c) {
            if (l[c] == -INFINITY) continue;
            double w = exp(l[c] - lse);
            for (int m = 0; m < D->d_c; ++m)
                o[m] += w * ld(o_part, o_dt, (row * num_splits + c) * D->d_c + m);
        }
        if (lse_out) lse_out[row] = lse;
    }
}

/* ---- value up-projection ------------------------------------------------- */

void orc_up_v(const orc_dims *D, const void *o_latent, int o_dt,
              const void *W_UV, int w_dt, double *out)
{
    int64_t rows = (int64_t)D->B * D->Sq * D->H;
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < rows; ++row) {
        int h = (int)(row % D->H);
        for (int d = 0; d < D->d_h; ++d) {
            double acc = 0.0;
            for (int m = 0; m < D->d_c; ++m)
                acc += ld(W_UV, w_dt, ((int64_t)h * D->d_h + d) * D->d_c + m) *
                       ld(o_latent, o_dt, row * D->d_c + m);
            out[row * D->d_h + d] = acc;
        }
    }
}

/* ---- the whole decode step for selected query rows -------------------------
 * rows: n_rows flat indices into [B,Sq,H] (NULL = every row, in order).
 * Outputs are indexed by position in the list: out [n_rows,d_h],
 * o_latent [n_rows,d_c] (nullable), lse [n_rows] (nullable). */
void orc_decode(const orc_dims *D, const void *q_nope, const void *q_rope, int q_dt,
                const void *c_kv, int kv_dt, const float *kv_scale,
                const void *k_pe, int pe_dt,
                const void *W_UK, const void *W_UV, int w_dt,
                const int32_t *block_table, const int32_t *seq_lens,
                int64_t n_rows, const int64_t *rows,
                double *out, double *o_latent, double *lse)
{
    cache_t C = {D, c_kv, kv_dt, kv_scale, k_pe, pe_dt, block_table};
    int64_t maxlen = 0;
    for (int b = 0; b < D->B; ++b) if (seq_lens[b] > maxlen) maxlen = seq_lens[b];
#pragma omp parallel
    {
        double *qa = malloc(sizeof(double) * (D->d_c + 1));
        double *qr = malloc(sizeof(double) * (D->d_r + 1));
        double *o = malloc(sizeof(double) * (D->d_c + 1));
        double *z = malloc(sizeof(double) * (maxlen + 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_rows; ++i) {
            int64_t row = rows ? rows[i] : i;
            int b = (int)(row / ((int64_t)D->Sq * D->H));
            int s = (int)((row / D->H) % D->Sq);
            int h = (int)(row % D->H);
            for (int m = 0; m < D->d_c; ++m) {
                double acc = 0.0;
                for (int d = 0; d < D->d_h; ++d)
                    acc += ld(q_nope, q_dt, row * D->d_h + d) *
                           ld(W_UK, w_dt, ((int64_t)h * D->d_h + d) * D->d_c + m);
                qa[m] = acc;
            }
            load_row(q_rope, q_dt, row, D->d_r, qr);
            double l = attend(&C, b, qa, qr, 0, visible(D, seq_lens, b, s), z, o);
            for (int d = 0; d < D->d_h; ++d) {
                double acc = 0.0;
                for (int m = 0; m < D->d_c; ++m)
                    acc += ld(W_UV, w_dt, ((int64_t)h * D->d_h + d) * D->d_c + m) * o[m];
                out[i * D->d_h + d] = acc;
            }
            if (o_latent) memcpy(o_latent + i * D->d_c, o, sizeof(double) * D->d_c);
            if (lse) lse[i] = l;
        }
        free(qa); free(qr); free(o); free(z);
    }
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
