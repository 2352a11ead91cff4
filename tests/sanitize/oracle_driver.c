/* The oracle's C code under AddressSanitizer + UndefinedBehaviorSanitizer: every
 * entry point on small synthetic inputs (random values, random paging, ragged
 * lengths, empty sequences), with a check that the whole step equals the split
 * partials merged and up-projected. */
#include "../../oracle/mla_oracle.c"

#include <stdio.h>

static uint64_t st = 88172645463325252ull;
static double urand(void) {   /* xorshift64, in [-1, 1) */
    st ^= st << 13;
    st ^= st >> 7;
    st ^= st << 17;
    return (double)(st >> 11) / 4503599627370496.0 - 1.0;
}

int main(void) {
    const int B = 3, Sq = 2, H = 4, dh = 8, dc = 16, dr = 4, P = 64, mp = 5;
    orc_dims D = {B, Sq, H, dh, dc, dr, P, mp, 0.25};
    const int32_t lens[3] = {130, 0, 257};
    const int pages = 12;
    int32_t bt[3 * 5];
    int k = 0;
    for (int i = 0; i < B * mp; ++i) bt[i] = -1;
    for (int b = 0; b < B; ++b)
        for (int j = 0; j < (lens[b] + P - 1) / P; ++j) bt[b * mp + j] = (k++ * 7) % pages;
    const int rows = B * Sq * H;
    float *q_nope = malloc(sizeof(float) * rows * dh), *q_rope = malloc(sizeof(float) * rows * dr);
    float *ckv = malloc(sizeof(float) * pages * P * dc), *kpe = malloc(sizeof(float) * pages * P * dr);
    float *wuk = malloc(sizeof(float) * H * dh * dc), *wuv = malloc(sizeof(float) * H * dh * dc);
    for (int i = 0; i < rows * dh; ++i) q_nope[i] = (float)urand();
    for (int i = 0; i < rows * dr; ++i) q_rope[i] = (float)urand();
    for (int i = 0; i < pages * P * dc; ++i) ckv[i] = (float)urand();
    for (int i = 0; i < pages * P * dr; ++i) kpe[i] = (float)urand();
    for (int i = 0; i < H * dh * dc; ++i) { wuk[i] = (float)(0.1 * urand()); wuv[i] = (float)(0.1 * urand()); }
    double *qa = malloc(sizeof(double) * rows * dc);
    orc_absorb_q(&D, q_nope, ORC_F32, wuk, ORC_F32, qa);
    const int S = 3, sp = 2;
    double *op = malloc(sizeof(double) * rows * S * dc), *lp = malloc(sizeof(double) * rows * S);
    orc_decode_splitkv(&D, qa, ORC_F64, q_rope, ORC_F32, ckv, ORC_F32, NULL, kpe, ORC_F32, bt, lens, S, sp, op, lp);
    int32_t pb[9], pe[9];
    for (int b = 0; b < B; ++b)
        for (int c = 0; c < S; ++c) { pb[b * S + c] = c * sp; pe[b * S + c] = c * sp + sp; }
    double *op2 = malloc(sizeof(double) * rows * S * dc), *lp2 = malloc(sizeof(double) * rows * S);
    orc_decode_page_ranges(&D, qa, ORC_F64, q_rope, ORC_F32, ckv, ORC_F32, NULL, kpe, ORC_F32, bt, lens, S, pb, pe,
                           op2, lp2);
    double *ol = malloc(sizeof(double) * rows * dc), *lse = malloc(sizeof(double) * rows);
    orc_combine_lse(&D, S, op, ORC_F64, lp, ol, lse);
    double *out = malloc(sizeof(double) * rows * dh);
    orc_up_v(&D, ol, ORC_F64, wuv, ORC_F32, out);
    double *out2 = malloc(sizeof(double) * rows * dh), *ol2 = malloc(sizeof(double) * rows * dc);
    double *lse2 = malloc(sizeof(double) * rows);
    orc_decode(&D, q_nope, q_rope, ORC_F32, ckv, ORC_F32, NULL, kpe, ORC_F32, wuk, wuv, ORC_F32, bt, lens, rows, NULL,
               out2, ol2, lse2);
    double err = 0.0;
    for (int i = 0; i < rows * S; ++i)
        if (lp[i] != lp2[i] && !(isinf(lp[i]) && isinf(lp2[i]))) err = 1.0;
    for (int i = 0; i < rows * dh; ++i) err = fmax(err, fabs(out[i] - out2[i]));
    for (int i = 0; i < rows; ++i)
        if (!(lse[i] == lse2[i] || fabs(lse[i] - lse2[i]) < 1e-9)) err = fmax(err, 1.0);
    uint16_t bf = 0x3f80;
    uint8_t e = 0x38;
    if (orc_bf16_value(bf) != 1.0 || orc_e4m3_value(e) != 1.0) err = 1.0;
    free(q_nope); free(q_rope); free(ckv); free(kpe); free(wuk); free(wuv); free(qa); free(op); free(lp);
    free(op2); free(lp2); free(ol); free(lse); free(out); free(out2); free(ol2); free(lse2);
    if (err > 1e-9) {
        fprintf(stderr, "oracle driver: mismatch %g\n", err);
        return 1;
    }
    printf("oracle driver ok\n");
    return 0;
}
