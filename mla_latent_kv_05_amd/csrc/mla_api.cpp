// C ABI of libmla.so: host-side validation and kernel dispatch.
// Validation is pure host code (no HIP call), so it can be exercised on a
// machine without a GPU.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "mla.h"
#include "mla_internal.h"

namespace {

thread_local std::string g_last_error;

constexpr int kMaxSplits = 4096;   // the merge kernel keeps one weight per split in LDS
constexpr int kMaxParts = 1 << 20;

mla_status_t fail(mla_status_t s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
mla_status_t fail(mla_status_t s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

bool is_float_dtype(int dt) { return dt == MLA_F32 || dt == MLA_BF16; }

// fixed splits of one page each, one new token, bf16 partials, no forced kernel:
// the page kernel
bool use_page_kernel(const mla_params_t &p) {
    return !(p.flags & (MLA_FLAG_ROWS64 | MLA_FLAG_ROWS128 | MLA_FLAG_GENERIC)) && p.num_parts == 0 &&
           p.split_pages == 1 && mla::decode_page_supported(p);
}

// new tokens per sequence: at most kMaxAbsorbedSq on the absorbed path, kMaxPrefill on
// the non-absorbed one
constexpr int kMaxAbsorbedSq = 256;
// the absorbed path below, the non-absorbed one from here on: the two measure equal at
// 115 to 125 new tokens per sequence (4 x 4,096 and 16 x 2,048 cached positions), the
// absorbed path faster below (linear in the new tokens) and the non-absorbed one above
// (dominated by the decompression of every cached position)
constexpr int kSwitchSq = 120;
constexpr int kMaxPrefill = 65536;

mla_status_t check(const mla_params_t *p, int max_sq = kMaxAbsorbedSq) {
    if (!p) return fail(MLA_ERR_NULL, "params is NULL");
    if (p->B < 1 || p->Sq < 1 || p->Sq > max_sq || p->H < 1)
        return fail(MLA_ERR_SHAPE, "need B >= 1, 1 <= Sq <= %d, H >= 1 (got B=%d Sq=%d H=%d)", max_sq, p->B, p->Sq,
                    p->H);
    if (p->d_h < 1 || p->d_h > 256 || p->d_c < 1 || p->d_c > 1024 || p->d_r < 0 || p->d_r > 256)
        return fail(MLA_ERR_SHAPE, "need 1<=d_h<=256, 1<=d_c<=1024, 0<=d_r<=256 (got %d, %d, %d)", p->d_h, p->d_c, p->d_r);
    if (p->page_size != 64) return fail(MLA_ERR_SHAPE, "page_size must be 64 (got %d)", p->page_size);
    if (p->num_pages < 1 || p->max_pages < 1)
        return fail(MLA_ERR_SHAPE, "num_pages and max_pages must be >= 1 (got %d, %d)", p->num_pages, p->max_pages);
    if ((int64_t)p->B * p->Sq * p->H > (1ll << 28))
        return fail(MLA_ERR_SHAPE, "B*Sq*H too large");
    if (p->num_splits < 1 || p->num_splits > kMaxSplits)
        return fail(MLA_ERR_SPLITS, "num_splits must be in [1, %d] (got %d)", kMaxSplits, p->num_splits);
    if (p->num_parts < 0 || p->num_parts > kMaxParts)
        return fail(MLA_ERR_SPLITS, "num_parts must be in [0, %d] (got %d)", kMaxParts, p->num_parts);
    if (p->num_parts == 0) {
        if (p->split_pages < 1) return fail(MLA_ERR_SPLITS, "split_pages must be >= 1 (got %d)", p->split_pages);
        if ((int64_t)p->num_splits * p->split_pages < p->max_pages)
            return fail(MLA_ERR_SPLITS, "num_splits*split_pages = %lld < max_pages = %d",
                        (long long)p->num_splits * p->split_pages, p->max_pages);
        if ((int64_t)p->B * p->num_splits > (1ll << 31) / 64)
            return fail(MLA_ERR_SPLITS, "B*num_splits too large");
    }
    if (!(p->scale > 0.f) || !isfinite(p->scale)) return fail(MLA_ERR_SHAPE, "scale must be finite and > 0");
    if (!is_float_dtype(p->q_dtype)) return fail(MLA_ERR_DTYPE, "q_dtype must be F32 or BF16");
    if (!is_float_dtype(p->w_dtype)) return fail(MLA_ERR_DTYPE, "w_dtype must be F32 or BF16");
    if (!is_float_dtype(p->kv_dtype) && p->kv_dtype != MLA_FP8_E4M3)
        return fail(MLA_ERR_DTYPE, "kv_dtype must be F32, BF16 or FP8_E4M3");
    if (!is_float_dtype(p->pe_dtype)) return fail(MLA_ERR_DTYPE, "pe_dtype must be F32 or BF16");
    if (!is_float_dtype(p->latent_dtype)) return fail(MLA_ERR_DTYPE, "latent_dtype must be F32 or BF16");
    if (!is_float_dtype(p->out_dtype)) return fail(MLA_ERR_DTYPE, "out_dtype must be F32 or BF16");
    if (!is_float_dtype(p->part_dtype)) return fail(MLA_ERR_DTYPE, "part_dtype must be F32 or BF16");
    if (p->flags & ~static_cast<uint32_t>(MLA_FLAG_GENERIC | MLA_FLAG_ROWS64 | MLA_FLAG_ROWS128 | MLA_FLAG_POW2_SCALE))
        return fail(MLA_ERR_SHAPE, "unknown flag bits 0x%x", p->flags);
    if ((p->flags & MLA_FLAG_ROWS64) && (p->flags & MLA_FLAG_ROWS128))
        return fail(MLA_ERR_SHAPE, "MLA_FLAG_ROWS64 and MLA_FLAG_ROWS128 together");
    return MLA_OK;
}

mla_status_t hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return MLA_OK;
    return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t elem_bytes(int dt) { return dt == MLA_F32 ? 4 : dt == MLA_BF16 ? 2 : 1; }

int64_t align256(int64_t n) { return (n + 255) / 256 * 256; }

// Intermediates of the one-call decode step, at 256-byte aligned offsets of one
// workspace: q_abs, lse_part, o_part, then o_latent when the merge and the
// up-projection run as two launches.
struct StepLayout {
    int64_t q_abs, lse_part, o_part, o_latent, bytes;
};

StepLayout step_layout(const mla_params_t &p) {
    const int64_t rows = (int64_t)p.B * p.Sq * p.H;
    StepLayout l{};
    l.q_abs = 0;
    l.lse_part = align256(rows * p.d_c * (int64_t)elem_bytes(p.latent_dtype));
    l.o_part = l.lse_part + align256(rows * p.num_splits * 4);
    l.o_latent = l.o_part + align256(rows * p.num_splits * (int64_t)p.d_c * (int64_t)elem_bytes(p.part_dtype));
    l.bytes = mla::combine_up_v_supported(p) ? l.o_latent
                                             : l.o_latent + align256(rows * p.d_c * (int64_t)elem_bytes(p.latent_dtype));
    return l;
}

}  // namespace

extern "C" {

int32_t mla_abi_version(void) { return 3; }

const char *mla_status_string(mla_status_t s) {
    switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL: return "MLA_ERR_NULL";
    case MLA_ERR_SHAPE: return "MLA_ERR_SHAPE";
    case MLA_ERR_DTYPE: return "MLA_ERR_DTYPE";
    case MLA_ERR_SPLITS: return "MLA_ERR_SPLITS";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    }
    return "MLA_ERR_UNKNOWN";
}

const char *mla_last_error(void) { return g_last_error.c_str(); }

mla_status_t mla_check_params(const mla_params_t *p) { return check(p); }

const char *mla_decode_kernel_name(const mla_params_t *p) {
    if (!p || check(p) != MLA_OK) return "invalid";
    if (use_page_kernel(*p)) return "page_bf16";
    if (!mla::decode_mfma_supported(*p)) return "generic_f32";
    switch (mla::decode_kernel_for(*p)) {
    case mla::DecodeKernel::k128: return p->kv_dtype == MLA_FP8_E4M3 ? "mfma_fp8_128" : "mfma_bf16_128";
    case mla::DecodeKernel::k8: return "mfma_bf16_64";
    case mla::DecodeKernel::kMfma64: return "mfma_fp8_64";
    }
    return "invalid";
}

mla_status_t mla_plan_splits(mla_params_t *p, int32_t max_seq_len, int64_t total_tokens,
                             int32_t num_cus, int32_t min_splits) {
    if (!p) return fail(MLA_ERR_NULL, "params is NULL");
    if (max_seq_len < 0 || total_tokens < 0 || num_cus < 1 || min_splits < 1)
        return fail(MLA_ERR_SHAPE, "need max_seq_len >= 0, total_tokens >= 0, num_cus >= 1, min_splits >= 1");
    if (p->B < 1 || p->H < 1 || p->Sq < 1) return fail(MLA_ERR_SHAPE, "need B, Sq, H >= 1");
    const int64_t page = 64;
    const int64_t max_pages_seq = std::max<int64_t>(1, (max_seq_len + page - 1) / page);
    const int64_t pages_lo = (total_tokens + page - 1) / page;   // <= the batch's true page count
    // one workgroup per compute unit: each part is processed by Sq*H/64 workgroups
    // on the MFMA path (one per (row, split) on the generic path)
    // (the 128-row kernel's workgroups when it applies: a plan that leaves it few
    // workgroups sends a bf16 launch to the 64-row kernel, with twice as many)
    const bool mfma = mla::decode_mfma_supported(*p);
    // a small batch of single new tokens with bf16 partials: fixed splits of one page
    // each, on the page kernel (one workgroup per page and 32 heads, all launched at
    // once), when its workgroups stay within kPagePlanPerCu per compute unit
    {
        mla_params_t q = *p;
        q.num_parts = 0;
        q.split_pages = 1;
        q.num_splits = (int32_t)std::min<int64_t>(max_pages_seq, kMaxSplits);
        if (use_page_kernel(q) && max_pages_seq <= kMaxSplits &&
            (int64_t)p->B * ((max_pages_seq + 7) / 8 * 8) * (p->H / 32) <= mla::kPagePlanPerCu * num_cus) {
            p->num_parts = 0;
            p->split_pages = 1;
            p->num_splits = q.num_splits;
            return MLA_OK;
        }
    }
    const int64_t rows = (int64_t)p->Sq * p->H;
    const int64_t wg_per_part =
        mfma ? std::max<int64_t>(1, rows / (mla::decode128_supported(*p) ? mla::kDecodeRowsPerGroup
                                                                         : mla::kDecodeRowsPerBlock))
             : rows;
    int64_t P = std::max<int64_t>(1, num_cus / wg_per_part);
    if (!mfma) P = std::max<int64_t>(1, 2ll * num_cus / wg_per_part);
    // at least 8 parts even when that takes several rounds of workgroups (many query
    // rows per token): with 2 or 4 parts every page is read by all row groups at once
    // (measured at 4 x 4,096 positions: 64 new tokens, 2 parts 1.28 ms, 8 parts 0.44 ms)
    P = std::max<int64_t>(P, 8);
    // parts of at least 4 pages (2 with bf16 partials) keep the partials (d_c * 4 or 2
    // bytes per row) small next to the cache they summarise (measured at B = 1 with
    // fp32 partials: 4 pages per part beat 8, 2 and 1; with bf16 partials 2 beat 4 and 1)
    const int64_t min_pages = p->part_dtype == MLA_BF16 ? 2 : 4;
    P = std::min(P, std::max<int64_t>(1, pages_lo / min_pages));
    // a small batch whose plan leaves the 128-row kernel few workgroups runs on the
    // 64-row kernel (twice the workgroups): there, with bf16 partials, parts of one
    // unit each (at most one page) up to one 64-row workgroup per compute unit
    // (measured at B = 1, 4,096 positions: 128 parts 34 us per step, 32 parts 37 us)
    if (mfma && p->part_dtype == MLA_BF16 && mla::decode128_supported(*p) && mla::decode8_supported(*p) &&
        !(p->flags & MLA_FLAG_ROWS128) && P * wg_per_part <= mla::kSmallGrid128) {
        const int64_t units_lo = pages_lo + (int64_t)p->B * mla::kSeqStartCost;
        P = std::max(P, std::min(units_lo, std::max<int64_t>(1, num_cus / (2 * wg_per_part))));
    }
    P = std::max(P, std::min<int64_t>(min_splits, std::max<int64_t>(1, pages_lo)));
    P = std::min<int64_t>(P, kMaxParts);
    // a sequence of n pages touches at most ceil(n / q) + 1 parts of >= q pages, and
    // at most n parts
    const int64_t q_lo = pages_lo / P;
    int64_t S = q_lo >= 1 ? (max_pages_seq + q_lo - 1) / q_lo + 1 : max_pages_seq;
    S = std::min(S, max_pages_seq);
    S = std::min(S, P);
    S = std::max<int64_t>(S, 1);
    if (S > kMaxSplits) return fail(MLA_ERR_SPLITS, "planned num_splits %lld exceeds %d", (long long)S, kMaxSplits);
    p->num_parts = (int32_t)P;
    p->num_splits = (int32_t)S;
    if (p->split_pages < 1) p->split_pages = 1;   // unused with balanced splits
    return MLA_OK;
}

int32_t mla_default_num_splits(const mla_params_t *p, int32_t max_seq_len) {
    if (!p) {
        fail(MLA_ERR_NULL, "params is NULL");
        return -1;
    }
    if (max_seq_len < 1) {
        fail(MLA_ERR_SHAPE, "need max_seq_len >= 1 (got %d)", max_seq_len);
        return -1;
    }
    // the planner's part count for a batch of B sequences of max_seq_len tokens each,
    // on the 256 compute units of an MI355X; equal sequences share it evenly
    mla_params_t q = *p;
    if (mla_plan_splits(&q, max_seq_len, (int64_t)p->B * max_seq_len, 256, 1) != MLA_OK) return -1;
    const int64_t pages = (max_seq_len + 63) / 64;
    int64_t S = (q.num_parts + p->B - 1) / p->B;
    S = std::min<int64_t>(std::max<int64_t>(S, 1), std::min<int64_t>(pages, kMaxSplits));
    return (int32_t)S;
}

mla_status_t mla_absorb_q(const mla_params_t *p, const void *q_nope, const void *W_UK, void *q_abs,
                          void *stream) {
    mla_status_t s = check(p);
    if (s != MLA_OK) return s;
    if (!q_nope || !W_UK || !q_abs) return fail(MLA_ERR_NULL, "mla_absorb_q: NULL tensor pointer");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (!(p->flags & MLA_FLAG_GENERIC) && mla::absorb_rows_supported(*p))
        return hip_status(mla::launch_absorb_rows(*p, q_nope, W_UK, q_abs, st), "mla_absorb_q launch");
    if (mla::absorb_mfma_supported(*p))
        return hip_status(mla::launch_absorb_mfma(*p, q_nope, W_UK, q_abs, st), "mla_absorb_q launch");
    return hip_status(mla::launch_absorb_generic(*p, q_nope, W_UK, q_abs, st), "mla_absorb_q launch");
}

mla_status_t mla_decode_splitkv(const mla_params_t *p, const void *q_abs, const void *q_rope,
                                const void *c_kv, const void *k_pe, const float *kv_scale,
                                const int32_t *block_table, const int32_t *seq_lens, void *o_part,
                                float *lse_part, void *stream) {
    mla_status_t s = check(p);
    if (s != MLA_OK) return s;
    if (!q_abs || !c_kv || !block_table || !seq_lens || !o_part || !lse_part)
        return fail(MLA_ERR_NULL, "mla_decode_splitkv: NULL tensor pointer");
    if (p->d_r > 0 && (!q_rope || !k_pe)) return fail(MLA_ERR_NULL, "mla_decode_splitkv: NULL q_rope/k_pe with d_r > 0");
    if (p->kv_dtype == MLA_FP8_E4M3 && !kv_scale)
        return fail(MLA_ERR_NULL, "mla_decode_splitkv: kv_scale is required for an FP8_E4M3 cache");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (use_page_kernel(*p)) {
        if ((int64_t)p->B * ((p->num_splits + 7) / 8 * 8) * (p->H / 32) > 0x7fffffffll)
            return fail(MLA_ERR_SHAPE, "mla_decode_splitkv: grid too large");
        return hip_status(mla::launch_decode_page(*p, q_abs, q_rope, c_kv, k_pe, block_table, seq_lens, o_part,
                                                  lse_part, st),
                          "mla_decode_splitkv launch");
    }
    const int64_t rows = (int64_t)p->B * p->Sq * p->H;
    const int64_t parts = p->num_parts > 0 ? p->num_parts : (int64_t)p->B * p->num_splits;
    const int64_t grid = mla::decode_mfma_supported(*p)
                             ? (parts + 7) / 8 * 8 * (rows / p->B / mla::decode_rows_per_workgroup(*p))
                             : rows * p->num_splits;
    if (grid > 0x7fffffffll) return fail(MLA_ERR_SHAPE, "mla_decode_splitkv: grid of %lld workgroups too large", (long long)grid);
    if (mla::decode_mfma_supported(*p)) {
        const mla::DecodeKernel k = mla::decode_kernel_for(*p);
        if (((p->flags & MLA_FLAG_ROWS128) && k != mla::DecodeKernel::k128) ||
            ((p->flags & MLA_FLAG_ROWS64) && k != mla::DecodeKernel::k8))
            return fail(MLA_ERR_UNSUPPORTED, "mla_decode_splitkv: the forced attention kernel does not take these parameters");
        if (k == mla::DecodeKernel::k128)
            return hip_status(mla::launch_decode128(*p, q_abs, q_rope, c_kv, k_pe, kv_scale, block_table, seq_lens,
                                                    o_part, lse_part, st),
                              "mla_decode_splitkv launch");
        if (k == mla::DecodeKernel::k8)
            return hip_status(mla::launch_decode8(*p, q_abs, q_rope, c_kv, k_pe, block_table, seq_lens, o_part,
                                                  lse_part, st),
                              "mla_decode_splitkv launch");
        return hip_status(mla::launch_decode_mfma(*p, q_abs, q_rope, c_kv, k_pe, kv_scale, block_table,
                                                  seq_lens, o_part, lse_part, st),
                          "mla_decode_splitkv launch");
    }
    if (p->flags & (MLA_FLAG_ROWS64 | MLA_FLAG_ROWS128))
        return fail(MLA_ERR_UNSUPPORTED, "mla_decode_splitkv: a forced MFMA attention kernel does not take these parameters");
    return hip_status(mla::launch_decode_generic(*p, q_abs, q_rope, c_kv, k_pe, kv_scale, block_table,
                                                 seq_lens, o_part, lse_part, st),
                      "mla_decode_splitkv launch");
}

mla_status_t mla_combine_lse(const mla_params_t *p, const void *o_part, const float *lse_part,
                             void *o_latent, float *lse_out, void *stream) {
    mla_status_t s = check(p);
    if (s != MLA_OK) return s;
    if (!o_part || !lse_part || !o_latent) return fail(MLA_ERR_NULL, "mla_combine_lse: NULL tensor pointer");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (mla::combine_fast_supported(*p))
        return hip_status(mla::launch_combine_fast(*p, o_part, lse_part, o_latent, lse_out, st), "mla_combine_lse launch");
    return hip_status(mla::launch_combine(*p, o_part, lse_part, o_latent, lse_out, st), "mla_combine_lse launch");
}

mla_status_t mla_up_v(const mla_params_t *p, const void *o_latent, const void *W_UV, void *out,
                      void *stream) {
    mla_status_t s = check(p);
    if (s != MLA_OK) return s;
    if (!o_latent || !W_UV || !out) return fail(MLA_ERR_NULL, "mla_up_v: NULL tensor pointer");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (mla::up_v_mfma_supported(*p))
        return hip_status(mla::launch_up_v_mfma(*p, o_latent, W_UV, out, st), "mla_up_v launch");
    return hip_status(mla::launch_up_v_generic(*p, o_latent, W_UV, out, st), "mla_up_v launch");
}

mla_status_t mla_combine_up_v(const mla_params_t *p, const void *o_part, const float *lse_part, const void *W_UV,
                              void *out, float *lse_out, void *stream) {
    mla_status_t s = check(p);
    if (s != MLA_OK) return s;
    if (!o_part || !lse_part || !W_UV || !out) return fail(MLA_ERR_NULL, "mla_combine_up_v: NULL tensor pointer");
    if (!mla::combine_up_v_supported(*p))
        return fail(MLA_ERR_UNSUPPORTED, "mla_combine_up_v: kernels exist for d_h=128, d_c=512 with bf16 weights and "
                                         "latent_dtype bf16");
    hipStream_t st = static_cast<hipStream_t>(stream);
    return hip_status(mla::launch_combine_up_v(*p, o_part, lse_part, W_UV, out, lse_out, st), "mla_combine_up_v launch");
}

mla_status_t mla_expand_kv(const mla_params_t *p, const void *c_kv, const float *kv_scale, void *c_out,
                           void *stream) {
    mla_status_t s = check(p, kMaxPrefill);
    if (s != MLA_OK) return s;
    if (!c_kv || !kv_scale || !c_out) return fail(MLA_ERR_NULL, "mla_expand_kv: NULL tensor pointer");
    if (p->kv_dtype != MLA_FP8_E4M3) return fail(MLA_ERR_DTYPE, "mla_expand_kv: kv_dtype must be e4m3");
    if (p->d_c % 8 != 0) return fail(MLA_ERR_SHAPE, "mla_expand_kv: d_c must be a multiple of 8 (got %d)", p->d_c);
    if ((int64_t)p->num_pages * p->page_size * (p->d_c / 8) / 256 > 0x7fffffffll)
        return fail(MLA_ERR_SHAPE, "mla_expand_kv: cache too large for one launch");
    hipStream_t st = static_cast<hipStream_t>(stream);
    return hip_status(mla::launch_expand(*p, c_kv, kv_scale, c_out, st), "mla_expand_kv launch");
}

mla_status_t mla_append_kv(const mla_params_t *p, const void *c_new, const void *kpe_new, const void *q_rope_in,
                           void *q_rope_out, const int32_t *block_table, const int32_t *seq_lens, void *c_kv,
                           void *k_pe, float *kv_scale, void *stream) {
    mla_status_t s = check(p);
    if (s != MLA_OK) return s;
    if (!c_new || !block_table || !seq_lens || !c_kv) return fail(MLA_ERR_NULL, "mla_append_kv: NULL tensor pointer");
    if (p->d_r > 0 && (!kpe_new || !k_pe)) return fail(MLA_ERR_NULL, "mla_append_kv: NULL kpe_new/k_pe with d_r > 0");
    if (p->d_r % 2 != 0) return fail(MLA_ERR_SHAPE, "mla_append_kv: d_r must be even for the rotation (got %d)", p->d_r);
    if ((q_rope_in == nullptr) != (q_rope_out == nullptr))
        return fail(MLA_ERR_NULL, "mla_append_kv: q_rope_in and q_rope_out must be both given or both NULL");
    if (p->kv_dtype == MLA_FP8_E4M3 && !kv_scale)
        return fail(MLA_ERR_NULL, "mla_append_kv: kv_scale is required for an FP8_E4M3 cache");
    if ((int64_t)p->B * p->Sq > 0x7fffffffll) return fail(MLA_ERR_SHAPE, "mla_append_kv: B*Sq too large");
    hipStream_t st = static_cast<hipStream_t>(stream);
    return hip_status(mla::launch_append(*p, c_new, kpe_new, q_rope_in, q_rope_out, block_table, seq_lens, c_kv, k_pe,
                                         kv_scale, st),
                      "mla_append_kv launch");
}

int64_t mla_prefill_lmax(const mla_params_t *p) {
    if (check(p, kMaxPrefill) != MLA_OK) return -1;
    return mla::prefill_lmax(*p);
}

int32_t mla_prefer_absorbed(const mla_params_t *p) {
    if (check(p, kMaxPrefill) != MLA_OK) return -1;
    return p->Sq < kSwitchSq ? 1 : 0;
}

mla_status_t mla_decompress_kv(const mla_params_t *p, const void *c_kv, const int32_t *block_table,
                               const int32_t *seq_lens, const void *W_UK, const void *W_UV, void *k_nope,
                               void *v_t, void *stream) {
    mla_status_t s = check(p, kMaxPrefill);
    if (s != MLA_OK) return s;
    if (!c_kv || !block_table || !seq_lens || !W_UK || !W_UV || !k_nope || !v_t)
        return fail(MLA_ERR_NULL, "mla_decompress_kv: NULL tensor pointer");
    if (!mla::prefill_supported(*p))
        return fail(MLA_ERR_UNSUPPORTED, "mla_decompress_kv: kernels exist for d_h=128, d_c=512, d_r=64 with bf16 "
                                         "weights, cache and latent");
    if ((int64_t)p->B * ((p->max_pages + 3) / 4) * ((p->H + 15) / 16) > 0x7fffffffll)
        return fail(MLA_ERR_SHAPE, "mla_decompress_kv: grid too large");
    hipStream_t st = static_cast<hipStream_t>(stream);
    return hip_status(mla::launch_decompress(*p, c_kv, block_table, seq_lens, W_UK, W_UV, k_nope, v_t, st),
                      "mla_decompress_kv launch");
}

mla_status_t mla_prefill_attention(const mla_params_t *p, const void *q_nope, const void *q_rope,
                                   const void *k_nope, const void *v_t, const void *k_pe,
                                   const int32_t *block_table, const int32_t *seq_lens, void *out,
                                   void *stream) {
    mla_status_t s = check(p, kMaxPrefill);
    if (s != MLA_OK) return s;
    if (!q_nope || !q_rope || !k_nope || !v_t || !k_pe || !block_table || !seq_lens || !out)
        return fail(MLA_ERR_NULL, "mla_prefill_attention: NULL tensor pointer");
    if (!mla::prefill_supported(*p))
        return fail(MLA_ERR_UNSUPPORTED, "mla_prefill_attention: kernels exist for d_h=128, d_c=512, d_r=64 with "
                                         "bf16 queries, weights, cache and latent");
    if ((int64_t)p->B * p->H * ((p->Sq + 255) / 256) > 0x7fffffffll)
        return fail(MLA_ERR_SHAPE, "mla_prefill_attention: grid too large");
    hipStream_t st = static_cast<hipStream_t>(stream);
    return hip_status(mla::launch_prefill_attention(*p, q_nope, q_rope, k_nope, v_t, k_pe, block_table, seq_lens,
                                                    out, st),
                      "mla_prefill_attention launch");
}

mla_status_t mla_device_errors(uint32_t *bits, void *stream) {
    if (!bits) return fail(MLA_ERR_NULL, "mla_device_errors: bits is NULL");
    *bits = 0;
    hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
    if (e == hipSuccess) e = mla::take_errors_generic(bits);
    if (e == hipSuccess) e = mla::take_errors_decode_mfma(bits);
    if (e == hipSuccess) e = mla::take_errors_decode8(bits);
    if (e == hipSuccess) e = mla::take_errors_decode128(bits);
    if (e == hipSuccess) e = mla::take_errors_step_persistent(bits);
    return hip_status(e, "mla_device_errors");
}

int32_t mla_debug_bounds(void) {
#ifdef MLA_DEBUG_BOUNDS
    return 1;
#else
    return 0;
#endif
}

int64_t mla_decode_step_workspace(const mla_params_t *p) {
    if (check(p) != MLA_OK) return -1;
    return step_layout(*p).bytes;
}

}  // extern "C"

namespace {

// absorb, attention, then the merge and up-projection (one launch where the fused
// tail applies) on the intermediates at ws
mla_status_t run_step(const mla_params_t *p, const void *q_nope, const void *q_rope, const void *c_kv,
                      const void *k_pe, const float *kv_scale, const int32_t *block_table, const int32_t *seq_lens,
                      const void *W_UK, const void *W_UV, void *out, float *lse_out, char *ws, void *stream) {
    const StepLayout l = step_layout(*p);
    void *q_abs = ws + l.q_abs;
    float *lse_part = reinterpret_cast<float *>(ws + l.lse_part);
    void *o_part = ws + l.o_part;
    mla_status_t s = mla_absorb_q(p, q_nope, W_UK, q_abs, stream);
    if (s != MLA_OK) return s;
    s = mla_decode_splitkv(p, q_abs, q_rope, c_kv, k_pe, kv_scale, block_table, seq_lens, o_part, lse_part, stream);
    if (s != MLA_OK) return s;
    if (mla::combine_up_v_supported(*p)) return mla_combine_up_v(p, o_part, lse_part, W_UV, out, lse_out, stream);
    void *o_latent = ws + l.o_latent;
    s = mla_combine_lse(p, o_part, lse_part, o_latent, lse_out, stream);
    if (s != MLA_OK) return s;
    return mla_up_v(p, o_latent, W_UV, out, stream);
}

mla_status_t check_step(const mla_params_t *p, const void *q_nope, const void *c_kv, const int32_t *block_table,
                        const int32_t *seq_lens, const void *W_UK, const void *W_UV, void *out, const char *who) {
    mla_status_t s = check(p);
    if (s != MLA_OK) return s;
    if (!q_nope || !c_kv || !block_table || !seq_lens || !W_UK || !W_UV || !out)
        return fail(MLA_ERR_NULL, "%s: NULL tensor pointer", who);
    return MLA_OK;
}

}  // namespace

// The no-allocation step's intermediates live in this file-scope device array (one
// copy per GPU, alive until the process ends).  Host code never passes the array's
// name to a kernel or a copy: it uses the device address hipGetSymbolAddress gives,
// looked up once per device with that device current.
constexpr int64_t kScratchBytes = 160ll << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

mla_status_t scratch_of_current_device(char **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "mla_decode_step_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(MLA_ERR_HIP, "mla_decode_step_noalloc: device %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *a = nullptr;
        e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !a)
            return fail(MLA_ERR_HIP, "mla_decode_step_noalloc: hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = a;
    }
    *ptr = static_cast<char *>(g_scratch_ptr[dev]);
    return MLA_OK;
}

}  // namespace

extern "C" {

mla_status_t mla_decode_step(const mla_params_t *p, const void *q_nope, const void *q_rope, const void *c_kv,
                             const void *k_pe, const float *kv_scale, const int32_t *block_table,
                             const int32_t *seq_lens, const void *W_UK, const void *W_UV, void *out, float *lse_out,
                             void *workspace, int64_t workspace_bytes, void *stream) {
    mla_status_t s = check_step(p, q_nope, c_kv, block_table, seq_lens, W_UK, W_UV, out, "mla_decode_step");
    if (s != MLA_OK) return s;
    if (!workspace) return fail(MLA_ERR_NULL, "mla_decode_step: NULL workspace");
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
        return fail(MLA_ERR_SHAPE, "mla_decode_step: workspace must be 256-byte aligned");
    const int64_t need = step_layout(*p).bytes;
    if (workspace_bytes < need)
        return fail(MLA_ERR_SHAPE, "mla_decode_step: workspace of %lld bytes, need %lld (mla_decode_step_workspace)",
                    (long long)workspace_bytes, (long long)need);
    return run_step(p, q_nope, q_rope, c_kv, k_pe, kv_scale, block_table, seq_lens, W_UK, W_UV, out, lse_out,
                    static_cast<char *>(workspace), stream);
}

mla_status_t mla_decode_step_noalloc(const mla_params_t *p, const void *q_nope, const void *q_rope, const void *c_kv,
                                     const void *k_pe, const float *kv_scale, const int32_t *block_table,
                                     const int32_t *seq_lens, const void *W_UK, const void *W_UV, void *out,
                                     float *lse_out, void *stream) {
    mla_status_t s = check_step(p, q_nope, c_kv, block_table, seq_lens, W_UK, W_UV, out, "mla_decode_step_noalloc");
    if (s != MLA_OK) return s;
    const int64_t need = step_layout(*p).bytes;
    if (need > kScratchBytes)
        return fail(MLA_ERR_SHAPE,
                    "mla_decode_step_noalloc: the step needs %lld bytes of scratch, the static scratch holds %lld "
                    "(use mla_decode_step with a workspace)",
                    (long long)need, (long long)kScratchBytes);
    char *ws = nullptr;
    s = scratch_of_current_device(&ws);
    if (s != MLA_OK) return s;
    return run_step(p, q_nope, q_rope, c_kv, k_pe, kv_scale, block_table, seq_lens, W_UK, W_UV, out, lse_out, ws,
                    stream);
}

int64_t mla_decode_step_persistent_workspace(const mla_params_t *p) {
    if (check(p) != MLA_OK || !mla::step_persistent_supported(*p)) return -1;
    return mla::step_persistent_layout(*p).bytes;
}

mla_status_t mla_decode_step_persistent(const mla_params_t *p, const void *q_nope, const void *q_rope,
                                        const void *c_kv, const void *k_pe, const int32_t *block_table,
                                        const int32_t *seq_lens, const void *W_UK, const void *W_UV, void *out,
                                        float *lse_out, void *workspace, int64_t workspace_bytes, void *stream) {
    mla_status_t s = check_step(p, q_nope, c_kv, block_table, seq_lens, W_UK, W_UV, out,
                                "mla_decode_step_persistent");
    if (s != MLA_OK) return s;
    if (!q_rope || !k_pe) return fail(MLA_ERR_NULL, "mla_decode_step_persistent: NULL q_rope or k_pe");
    if (!mla::step_persistent_supported(*p))
        return fail(MLA_ERR_UNSUPPORTED,
                    "mla_decode_step_persistent: needs Sq = 1, B <= 8, H a multiple of 32 up to 128, d_h = 128, "
                    "d_c = 512, d_r = 64, bf16 q, weights, cache, RoPE keys and q_abs, bf16 or f32 out, "
                    "max_pages <= %d",
                    mla::kStepPersistentMaxPages);
    if (!workspace) return fail(MLA_ERR_NULL, "mla_decode_step_persistent: NULL workspace");
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
        return fail(MLA_ERR_SHAPE, "mla_decode_step_persistent: workspace must be 256-byte aligned");
    const int64_t need = mla::step_persistent_layout(*p).bytes;
    if (workspace_bytes < need)
        return fail(MLA_ERR_SHAPE,
                    "mla_decode_step_persistent: workspace of %lld bytes, need %lld "
                    "(mla_decode_step_persistent_workspace)",
                    (long long)workspace_bytes, (long long)need);
    return hip_status(mla::launch_step_persistent(*p, q_nope, q_rope, c_kv, k_pe, block_table, seq_lens, W_UK, W_UV,
                                                  out, lse_out, static_cast<char *>(workspace),
                                                  static_cast<hipStream_t>(stream)),
                      "mla_decode_step_persistent launch");
}

}  // extern "C"
