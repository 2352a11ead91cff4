// Host-side exercise of the C ABI for the sanitizer build (AddressSanitizer +
// UndefinedBehaviorSanitizer on the host code of mla_api.cpp): parameter checks,
// the split planner, the default split count, the step workspace, and every
// entry point's argument-rejection path.  No call here reaches a GPU.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "mla.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd() {   // xorshift64*
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}

static mla_params_t v3(int B, int Sq, int max_pages) {
    mla_params_t p = {};
    p.B = B; p.Sq = Sq; p.H = 128; p.d_h = 128; p.d_c = 512; p.d_r = 64;
    p.page_size = 64; p.num_pages = B * max_pages; p.max_pages = max_pages;
    p.num_splits = 1; p.split_pages = max_pages; p.scale = 0.0721687836f;
    p.q_dtype = p.w_dtype = p.kv_dtype = p.pe_dtype = p.latent_dtype = MLA_BF16;
    p.out_dtype = MLA_F32;
    return p;
}

int main() {
    int failures = 0;
#define EXPECT(c)                                                  \
    do {                                                           \
        if (!(c)) {                                                \
            fprintf(stderr, "line %d: %s\n", __LINE__, #c);        \
            ++failures;                                            \
        }                                                          \
    } while (0)
    void *d = (void *)0x1000;
    // random parameter blocks through the validator (any field, any value)
    for (int i = 0; i < 20000; ++i) {
        mla_params_t p = v3(1 + rnd() % 200, 1 + rnd() % 8, 1 + rnd() % 300);
        int32_t *f = (int32_t *)&p;
        const int nf = (int)(sizeof(p) / 4);
        f[rnd() % nf] = (int32_t)rnd();
        const mla_status_t s = mla_check_params(&p);
        EXPECT(s >= MLA_OK && s <= MLA_ERR_UNSUPPORTED);
        (void)mla_status_string(s);
        (void)mla_last_error();
        (void)mla_decode_step_workspace(&p);
        (void)mla_prefer_absorbed(&p);
        (void)mla_prefill_lmax(&p);
        (void)mla_decode_kernel_name(&p);
    }
    // the planner and the default split count over random batches
    for (int i = 0; i < 20000; ++i) {
        const int B = 1 + rnd() % 4096;
        const int max_len = (int)(rnd() % 300000);
        mla_params_t p = v3(B, 1 + rnd() % 4, (max_len + 63) / 64 + 1);
        const int64_t total = (int64_t)(rnd() % (uint32_t)(max_len + 1)) * B;
        const mla_status_t s = mla_plan_splits(&p, max_len, total, 1 + rnd() % 512, 1 + rnd() % 64);
        if (s == MLA_OK) EXPECT(p.num_parts >= 1 && p.num_splits >= 1 && p.num_splits <= p.num_parts);
        const int32_t S = mla_default_num_splits(&p, max_len);
        EXPECT(max_len < 1 ? S == -1 : (S == -1 || S >= 1));
    }
    EXPECT(mla_plan_splits(NULL, 1, 1, 1, 1) == MLA_ERR_NULL);
    EXPECT(mla_default_num_splits(NULL, 1) == -1);
    // every entry point rejects NULL tensors and bad parameters before any launch
    mla_params_t p = v3(2, 1, 4);
    p.num_splits = 2;
    EXPECT(mla_absorb_q(&p, NULL, d, d, NULL) == MLA_ERR_NULL);
    const int32_t *di = (const int32_t *)d;
    EXPECT(mla_decode_splitkv(&p, d, d, NULL, d, NULL, di, di, d, (float *)d, NULL) == MLA_ERR_NULL);
    EXPECT(mla_combine_lse(&p, NULL, (const float *)d, d, NULL, NULL) == MLA_ERR_NULL);
    EXPECT(mla_up_v(&p, d, NULL, d, NULL) == MLA_ERR_NULL);
    EXPECT(mla_combine_up_v(&p, d, (const float *)d, NULL, d, NULL, NULL) == MLA_ERR_NULL);
    EXPECT(mla_expand_kv(&p, d, (const float *)d, d, NULL) == MLA_ERR_DTYPE);
    EXPECT(mla_append_kv(&p, NULL, d, NULL, NULL, (const int32_t *)d, (const int32_t *)d, d, d, NULL, NULL) ==
           MLA_ERR_NULL);
    EXPECT(mla_decompress_kv(&p, d, NULL, (const int32_t *)d, d, d, d, d, NULL) == MLA_ERR_NULL);
    EXPECT(mla_prefill_attention(&p, d, d, d, d, d, NULL, (const int32_t *)d, d, NULL) == MLA_ERR_NULL);
    const int64_t ws = mla_decode_step_workspace(&p);
    EXPECT(ws > 0);
    EXPECT(mla_decode_step(&p, d, d, d, d, NULL, (const int32_t *)d, (const int32_t *)d, d, d, d, NULL, NULL, ws,
                           NULL) == MLA_ERR_NULL);
    EXPECT(mla_decode_step(&p, d, d, d, d, NULL, (const int32_t *)d, (const int32_t *)d, d, d, d, NULL,
                           (void *)0x1008, ws, NULL) == MLA_ERR_SHAPE);
    EXPECT(mla_decode_step(&p, d, d, d, d, NULL, (const int32_t *)d, (const int32_t *)d, d, d, d, NULL, d, ws - 1,
                           NULL) == MLA_ERR_SHAPE);
    mla_params_t big = v3(64, 1, 16);
    big.num_splits = 16;
    EXPECT(mla_decode_step_noalloc(&big, d, d, d, d, NULL, (const int32_t *)d, (const int32_t *)d, d, d, d, NULL,
                                   NULL) == MLA_ERR_SHAPE);
    EXPECT(mla_device_errors(NULL, NULL) == MLA_ERR_NULL);
    p.Sq = 0;
    EXPECT(mla_absorb_q(&p, d, d, d, NULL) == MLA_ERR_SHAPE);
    EXPECT(mla_check_params(NULL) == MLA_ERR_NULL);
    if (failures) fprintf(stderr, "%d failures\n", failures);
    else printf("abi driver ok\n");
    return failures ? 1 : 0;
}
