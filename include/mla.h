/*
 * mla.h -- C ABI of libmla.so: weight-absorbed Multi-Head Latent Attention
 * (MLA) decode over a paged latent KV cache, hand-written HIP kernels for
 * AMD Instinct MI355X (gfx950).
 *
 * The new tokens enter the cache with mla_append_kv (RoPE, optional e4m3
 * quantisation); one decode step is then four stream-ordered calls:
 *
 *   mla_absorb_q        q_abs  = q_nope . W_UK            (key absorption)
 *   mla_decode_splitkv  per split c: scores, softmax, latent sum -> (O_c, lse_c)
 *   mla_combine_lse     log-sum-exp merge of the splits   -> o_latent (+ lse)
 *   mla_up_v            out    = o_latent . W_UV^T        (value up-projection)
 *   mla_combine_up_v    the last two in one launch
 *
 * Sources ("the pages"): "MLA 矩阵吸收 & 吸收分离 原理详解" (MLA Matrix
 * Absorption), sections 2.1, 4.1, 4.2; "DeepSeek-MLA-Principle", section 2
 * (score scale, softmax, eq. (10)) and section 3, matrix absorption 3) (key
 * absorption and value absorption) and "does down/up-projection save..." 3.
 * (FlashMLA: no K/V materialisation, tiling with online softmax and split-KV,
 * paged cache with a block table); "DeepSeek MLA 架构详解" section 3 and its
 * PyTorch decode module (tensor layouts [n_heads, d_head, d_latent]).
 *
 * Conventions for every entry point
 *   - Tensors are dense, row-major, contiguous, in DEVICE memory owned by the
 *     caller.  The library never allocates, frees or synchronises; it only
 *     enqueues kernels on `stream` (a hipStream_t; NULL = the null stream).
 *   - Arguments are validated on the host before anything is enqueued; a
 *     failed check returns an error status and launches nothing.  A launch
 *     failure returns MLA_ERR_HIP.  mla_last_error() gives a message for the
 *     calling thread's most recent failure.
 *   - Contents of seq_lens and block_table are NOT checked (they live on the
 *     device): every referenced page id must lie in [0, num_pages) and
 *     0 <= seq_lens[b] <= max_pages * page_size.  Violations are undefined.
 *   - Calls on different streams share no state and may run concurrently.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MLA_F32 = 0,
    MLA_BF16 = 1,
    MLA_FP8_E4M3 = 2   /* OCP E4M3 (bias 7, max 448, no infinities); c_kv only */
} mla_dtype_t;

typedef enum {
    MLA_OK = 0,
    MLA_ERR_NULL = 1,        /* a required pointer is NULL */
    MLA_ERR_SHAPE = 2,       /* a dimension is out of range */
    MLA_ERR_DTYPE = 3,       /* unsupported dtype or dtype combination */
    MLA_ERR_SPLITS = 4,      /* split plan out of range (see num_splits / split_pages / num_parts) */
    MLA_ERR_HIP = 5,         /* a HIP runtime call or kernel launch failed */
    MLA_ERR_UNSUPPORTED = 6  /* a valid request no kernel here implements */
} mla_status_t;

/* Bits of the device error word (mla_device_errors). */
#define MLA_DEVERR_SPLITS 1u  /* a sequence had pages in more parts than num_splits (stale plan): pages skipped */
#define MLA_DEVERR_SYNC 2u    /* a bounded wait between the waves of a workgroup gave up */
#define MLA_DEVERR_PAGE 4u    /* (MLA_DEBUG_BOUNDS build) block_table entry outside [0, num_pages) */
#define MLA_DEVERR_SEQLEN 8u  /* (MLA_DEBUG_BOUNDS build) seq_lens entry outside [0, max_pages * 64] */
#define MLA_DEVERR_SCALE 16u  /* (MLA_DEBUG_BOUNDS build) MLA_FLAG_POW2_SCALE with a scale that is no power of two */

/* Flags (mla_params_t.flags). */
#define MLA_FLAG_GENERIC 1u  /* use the fp32 VALU kernels even where MFMA kernels apply */
/* Attention kernel for a bf16 cache where both MFMA kernels apply (Sq*H a multiple
 * of 128).  By default the four-wave kernel (128 query rows per workgroup) runs,
 * unless its grid would hold at most 128 workgroups (a small batch): the eight-wave
 * kernel (64 rows per workgroup, twice the workgroups) then runs instead.  These
 * bits force one of them (not both; a forced kernel that cannot take *p makes
 * mla_decode_splitkv return MLA_ERR_UNSUPPORTED).  Both compute the same softmax
 * and partials up to rounding. */
#define MLA_FLAG_ROWS64 2u   /* the eight-wave kernel (bf16 cache, Sq*H a multiple of 64) */
#define MLA_FLAG_ROWS128 4u  /* the four-wave kernel (bf16 or e4m3 cache, Sq*H a multiple of 128) */
/* e4m3 cache: every kv_scale entry of a position a sequence holds is a power of two
 * (mla_append_kv writes only such scales).  The four-wave kernel then widens the
 * codes with gfx950's MX-style conversion, one instruction per two codes, instead
 * of widening, multiplying and rounding: the same values, bit for bit.  A scale
 * that is no power of two gives wrong values for its row (the conversion uses only
 * the scale's exponent); the MLA_DEBUG_BOUNDS build raises MLA_DEVERR_SCALE. */
#define MLA_FLAG_POW2_SCALE 8u

/*
 * Problem description shared by the four calls.
 *
 *   B           sequences in the batch                          >= 1
 *   Sq          new query tokens per sequence (causal among them) 1..256
 *               (1..65,536 for mla_append_kv, mla_decompress_kv and
 *               mla_prefill_attention)
 *   H           attention heads n_h (DeepSeek-V3: 128)           >= 1
 *   d_h         per-head non-RoPE query/key dim = value dim (128)  1..256
 *   d_c         latent dim kv_lora_rank (512)                    1..1024
 *   d_r         decoupled RoPE dim d_h^R (64)                    0..256
 *   page_size   tokens per cache page; must be 64
 *   num_pages   physical pages in c_kv / k_pe / kv_scale          >= 1
 *   max_pages   row stride of block_table                         >= 1
 *   num_splits  S: split slots per sequence (stride of o_part / lse_part) >= 1
 *   split_pages fixed splits (num_parts == 0): pages per split; split c of
 *               sequence b covers its pages [c*split_pages, (c+1)*split_pages).
 *               Requires num_splits * split_pages >= max_pages.
 *   num_parts   0 for fixed splits; P >= 1 for balanced splits, which give
 *               every part the same amount of work whatever the length mix.
 *               Work is counted in units: sequence b with n_b = ceil(seq_lens[b]
 *               / 64) > 0 pages costs u_b = 6 + n_b units (a start cost of 6,
 *               for its query loads, first copies and partial output, then one
 *               unit per page); an empty sequence costs 0.  With U = sum_b u_b and
 *               off_b = u_0 + ... + u_{b-1}, the batch's units taken in order are
 *               cut into P parts, part j holding units [floor(j*U/P),
 *               floor((j+1)*U/P)); page i of sequence b is unit off_b + 6 + i.
 *               Split c of sequence b is its pages in part j0(b) + c, where j0(b)
 *               is the part holding its first page (a sequence's pages lie in
 *               consecutive parts, one split each).  split_pages is ignored.
 *               Requires num_splits >= the largest number of parts holding pages
 *               of one sequence, which mla_plan_splits guarantees; a split index
 *               at or past num_splits is not computed.
 *   scale       softmax scale, 1/sqrt(d_h + d_r) ("DeepSeek-MLA-Principle"
 *               sec. 2; the decode module's self.scale)
 *   q_dtype     q_nope, q_rope            F32 | BF16
 *   w_dtype     W_UK, W_UV                F32 | BF16
 *   kv_dtype    c_kv                      F32 | BF16 | FP8_E4M3
 *   pe_dtype    k_pe                      F32 | BF16
 *   latent_dtype q_abs and o_latent       F32 | BF16
 *   out_dtype   out                       F32 | BF16
 *   flags       MLA_FLAG_* bits
 *   part_dtype  o_part (the split partials)  F32 | BF16 (0 = F32).  BF16 halves
 *               the bytes the attention writes and the merge reads; each partial
 *               row is rounded once (to nearest even) after its normalisation.
 */
typedef struct {
    int32_t B, Sq, H, d_h, d_c, d_r;
    int32_t page_size;
    int32_t num_pages;
    int32_t max_pages;
    int32_t num_splits;
    int32_t split_pages;
    float scale;
    int32_t q_dtype, w_dtype, kv_dtype, pe_dtype, latent_dtype, out_dtype;
    uint32_t flags;
    int32_t num_parts;
    int32_t part_dtype;
} mla_params_t;

/*
 * mla_absorb_q -- key absorption ("DeepSeek-MLA-Principle", matrix absorption
 * 3) (1); "MLA Matrix Absorption" sec. 2.1, Q' = Q x W_UK^T):
 *
 *   q_abs[b,s,h,m] = sum_{d < d_h} q_nope[b,s,h,d] * W_UK[h,d,m]
 *
 *   q_nope [B,Sq,H,d_h]  q_dtype       (in)
 *   W_UK   [H,d_h,d_c]   w_dtype       (in)
 *   q_abs  [B,Sq,H,d_c]  latent_dtype  (out)
 * Accumulates in fp32; rounds once to latent_dtype.
 */
mla_status_t mla_absorb_q(const mla_params_t *p, const void *q_nope, const void *W_UK,
                          void *q_abs, void *stream);

/*
 * mla_decode_splitkv -- attention over the paged latent cache, one partial
 * per split ("MLA Matrix Absorption" sec. 4.1-4.2: score = Q'_nope c^T +
 * Q_rope k_pe^T; "DeepSeek-MLA-Principle" sec. 2 scale and softmax, value
 * absorption m = sum alpha c; FlashMLA's tiling / online softmax / split-KV /
 * paged cache).  For row (b,s,h) and split c, with
 *   n = seq_lens[b] - Sq + 1 + s          (causal: position t visible iff t < n)
 *   T = positions t < n on the sequence's pages [c*split_pages, (c+1)*split_pages)
 *   z_t = scale * (q_abs[b,s,h,:] . C_t + q_rope[b,s,h,:] . k_pe_t)
 * where token t lives at page block_table[b, t/64], slot t%64, and
 * C_t = c_kv row (fp8: decoded code * kv_scale of that token):
 *   lse_part[b,s,h,c]  = ln sum_{t in T} exp(z_t)          (-inf if T empty)
 *   o_part[b,s,h,c,:]  = sum_{t in T} exp(z_t - lse) C_t   (normalised; left
 *                        unwritten when T is empty)
 * With balanced splits, "the sequence's pages" of split c are those given
 * under num_parts above.  In both modes every lse_part slot c < num_splits of
 * every row is written.
 *
 *   q_abs     [B,Sq,H,d_c]          latent_dtype (in)
 *   q_rope    [B,Sq,H,d_r]          q_dtype      (in)
 *   c_kv      [num_pages,64,d_c]    kv_dtype     (in)
 *   k_pe      [num_pages,64,d_r]    pe_dtype     (in, already rotated)
 *   kv_scale  [num_pages,64] fp32   (in; required iff kv_dtype == FP8_E4M3, else ignored)
 *   block_table [B,max_pages] int32 (in; entries past a sequence's last page unread)
 *   seq_lens  [B] int32             (in; tokens per sequence incl. the Sq new ones)
 *   o_part    [B,Sq,H,num_splits,d_c] part_dtype (out)
 *   lse_part  [B,Sq,H,num_splits]     fp32 (out)
 * Cache slots at or beyond seq_lens[b] in a sequence's last page are read but
 * contribute exactly zero, whatever they hold (non-finite values included).
 * An e4m3 cache enters the products as bf16(code * kv_scale) (one fp32 product,
 * rounded to nearest even: the values mla_expand_kv writes) in the four-wave
 * 128-row kernel; the 64-row e4m3 kernel multiplies the content score and the
 * weight by kv_scale in fp32 instead.  MLA_FLAG_ROWS64 / MLA_FLAG_ROWS128 pick
 * the bf16 kernel (see the flags above).
 */
mla_status_t mla_decode_splitkv(const mla_params_t *p, const void *q_abs, const void *q_rope,
                                const void *c_kv, const void *k_pe, const float *kv_scale,
                                const int32_t *block_table, const int32_t *seq_lens,
                                void *o_part, float *lse_part, void *stream);

/*
 * mla_combine_lse -- log-sum-exp merge of split partials (the merge that
 * split-KV implies; the pages only name split-KV):
 *   M = max_c lse_c,  lse = M + ln sum_c exp(lse_c - M),
 *   o_latent = sum_c exp(lse_c - lse) * o_part_c
 * Splits with lse_c = -inf carry no weight and their o_part is not read.  A
 * row whose splits are all empty gets o_latent = 0 and lse = -inf.
 *
 *   o_part   [B,Sq,H,num_splits,d_c] part_dtype (in)
 *   lse_part [B,Sq,H,num_splits]     fp32 (in)
 *   o_latent [B,Sq,H,d_c]  latent_dtype  (out)
 *   lse_out  [B,Sq,H] fp32 (out; may be NULL)
 */
mla_status_t mla_combine_lse(const mla_params_t *p, const void *o_part, const float *lse_part,
                             void *o_latent, float *lse_out, void *stream);

/*
 * mla_up_v -- value up-projection after the latent-space sum
 * ("DeepSeek-MLA-Principle", matrix absorption 3) (2): o = W_i^UV m;
 * "MLA Matrix Absorption" sec. 2.1, O = O' x W_UV):
 *
 *   out[b,s,h,d] = sum_{m < d_c} o_latent[b,s,h,m] * W_UV[h,d,m]
 *
 *   o_latent [B,Sq,H,d_c]  latent_dtype (in)
 *   W_UV     [H,d_h,d_c]   w_dtype      (in)
 *   out      [B,Sq,H,d_h]  out_dtype    (out)
 */
mla_status_t mla_up_v(const mla_params_t *p, const void *o_latent, const void *W_UV,
                      void *out, void *stream);

/*
 * mla_combine_up_v -- mla_combine_lse followed by mla_up_v in one launch, the
 * merged latent rows kept on chip: the fusion of the decode step's tail that the
 * value absorption allows ("DeepSeek-MLA-Principle", matrix absorption 3) (2):
 * the up-projection needs only the merged latent row of its own query row).
 * The merged rows are rounded to bf16 as mla_combine_lse rounds o_latent, and
 * the result is bit for bit that of the two calls with latent_dtype = bf16.
 * Kernels exist for d_h = 128, d_c = 512, bf16 weights and latent_dtype = bf16;
 * other parameters return MLA_ERR_UNSUPPORTED.
 *
 *   o_part   [B,Sq,H,num_splits,d_c] part_dtype (in)
 *   lse_part [B,Sq,H,num_splits]     fp32 (in)
 *   W_UV     [H,d_h,d_c]   w_dtype      (in)
 *   out      [B,Sq,H,d_h]  out_dtype    (out)
 *   lse_out  [B,Sq,H] fp32 (out; may be NULL)
 */
mla_status_t mla_combine_up_v(const mla_params_t *p, const void *o_part, const float *lse_part, const void *W_UV,
                              void *out, float *lse_out, void *stream);

/*
 * mla_decode_step -- the whole absorbed decode step in one call: mla_absorb_q,
 * mla_decode_splitkv, then mla_combine_up_v where it applies (else mla_combine_lse
 * and mla_up_v), all on `stream`, with the intermediates (q_abs, the partials, and
 * o_latent when the merge and the up-projection are two launches) in a workspace
 * the caller owns ("DeepSeek-MLA-Principle", matrix absorption 3): the query is
 * absorbed once, attention runs in latent space, the output is up-projected once).
 * The output equals that of the separate calls bit for bit.
 *
 *   q_nope, q_rope, c_kv, k_pe, kv_scale, block_table, seq_lens, W_UK, W_UV
 *                as for the separate calls (in)
 *   out        [B,Sq,H,d_h] out_dtype (out)
 *   lse_out    [B,Sq,H] fp32 (out; may be NULL)
 *   workspace  device memory of at least mla_decode_step_workspace(p) bytes,
 *              256-byte aligned (scratch: its contents on entry do not matter and
 *              are overwritten; two calls in flight at once need two workspaces)
 * Returns MLA_ERR_NULL / MLA_ERR_SHAPE (workspace NULL, misaligned or too small)
 * without launching anything, else the first failing call's status.
 */
mla_status_t mla_decode_step(const mla_params_t *p, const void *q_nope, const void *q_rope, const void *c_kv,
                             const void *k_pe, const float *kv_scale, const int32_t *block_table,
                             const int32_t *seq_lens, const void *W_UK, const void *W_UV, void *out, float *lse_out,
                             void *workspace, int64_t workspace_bytes, void *stream);

/* Workspace bytes mla_decode_step needs for *p (host-only; -1 for invalid p). */
int64_t mla_decode_step_workspace(const mla_params_t *p);

/*
 * mla_decode_step_noalloc -- mla_decode_step for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same calls and the same output bit for bit, with
 * the intermediates in a static scratch array of the library instead of a
 * caller's workspace.  It allocates nothing (no hipMalloc / hipFree, no
 * allocating library routine).
 *   - The scratch holds 160 MiB (167,772,160 bytes) per GPU, reserved when the
 *     library's code is loaded on that GPU and held until the process ends.
 *     Parameters whose mla_decode_step_workspace exceeds it return MLA_ERR_SHAPE
 *     without launching anything (B = 64, Sq = 1, num_splits = 8 at the
 *     DeepSeek-V3 shapes needs 143 MB).
 *   - Every call on one GPU shares that GPU's scratch, which keeps the last
 *     call's contents (nothing in it needs to start at zero).  Calls that overlap
 *     on one GPU (other streams, other threads) race on it: serialise them.
 *   - The scratch's device address is looked up on the first call on each device
 *     (the device current at the call); a failure returns MLA_ERR_HIP.
 * Arguments as for mla_decode_step, without the workspace.
 */
mla_status_t mla_decode_step_noalloc(const mla_params_t *p, const void *q_nope, const void *q_rope, const void *c_kv,
                                     const void *k_pe, const float *kv_scale, const int32_t *block_table,
                                     const int32_t *seq_lens, const void *W_UK, const void *W_UV, void *out,
                                     float *lse_out, void *stream);

/*
 * mla_decode_step_persistent -- the step of mla_decode_step for a small batch
 * of single new tokens, in one launch: absorb, attention and the merge with the
 * up-projection run as one kernel ("DeepSeek-MLA-Principle", matrix absorption
 * 3): the query is absorbed once, attention runs in latent space, the output is
 * up-projected once; "DeepSeek MLA 架构详解" sec. 3, the decode module).
 * Workgroups take one of three roles by index (absorb, attention per page and
 * 32 heads, merge and up-projection per head and 64 rows); a workgroup waits
 * only for workgroups of lower index through counters in the workspace, so the
 * launch drains however many of them are resident at once.
 *
 * Computes what mla_decode_step computes, within rounding (not bit for bit: q_abs
 * and the partials are summed in another order).  Each page of 64 positions is
 * one split; its partial is normalised and rounded once to bf16, as with
 * part_dtype = BF16.  num_splits, split_pages, num_parts, part_dtype and the flags
 * are ignored.  On an MI355X this one launch is slower than mla_decode_step's
 * three (the waits between its roles cross the compute dies' L2 caches); it is
 * for callers that want a single launch.  It suits short contexts only.  Every
 * page is one attention workgroup and one partial per head, so the work grows
 * with the pages: 4 sequences of 131,072 positions take about 4.9 ms, against
 * 0.18 ms for mla_decode_step.
 *
 * Supported (else MLA_ERR_UNSUPPORTED): Sq = 1, 1 <= B <= 8, H a multiple of 32
 * up to 128, d_h = 128, d_c = 512, d_r = 64, q_dtype = w_dtype = kv_dtype =
 * pe_dtype = latent_dtype = BF16, out_dtype BF16 or F32, max_pages <= 4096.
 *
 *   q_nope, q_rope, c_kv, k_pe, block_table, seq_lens, W_UK, W_UV
 *                as for mla_decode_step (in; q_rope and k_pe not NULL)
 *   out        [B,1,H,d_h] out_dtype (out)
 *   lse_out    [B,1,H] fp32 (out; may be NULL; -inf for an empty sequence, whose
 *              out rows are zero)
 *   workspace  device memory of at least mla_decode_step_persistent_workspace(p)
 *              bytes, 256-byte aligned.  Its first 256 bytes are the kernel's
 *              counters: they must be zero before the workspace's first use with
 *              this call (allocate it zeroed), and every call leaves them zero.  The
 *              rest is scratch.  Calls that share a workspace must not overlap.
 * The waits between workgroups are bounded: one that gives up sets
 * MLA_DEVERR_SYNC (mla_device_errors) and the kernel still ends.
 * Returns MLA_ERR_NULL / MLA_ERR_SHAPE / MLA_ERR_UNSUPPORTED without launching
 * anything, MLA_ERR_HIP if the launch fails.
 */
mla_status_t mla_decode_step_persistent(const mla_params_t *p, const void *q_nope, const void *q_rope,
                                        const void *c_kv, const void *k_pe, const int32_t *block_table,
                                        const int32_t *seq_lens, const void *W_UK, const void *W_UV, void *out,
                                        float *lse_out, void *workspace, int64_t workspace_bytes, void *stream);

/* Workspace bytes mla_decode_step_persistent needs for *p (host-only; -1 for an
 * invalid or unsupported p). */
int64_t mla_decode_step_persistent_workspace(const mla_params_t *p);

/*
 * mla_append_kv -- write the Sq new tokens of every sequence into the paged
 * cache, rotating the shared RoPE key at each token's position; optionally
 * rotate the query's RoPE part at the same positions.  The decode module of
 * "DeepSeek MLA 架构详解" computes the new token's latent row and RoPE key,
 * rotates the key at the token's position and appends both to the caches
 * before attending; "DeepSeek-MLA-Principle" sec. 3 (why RoPE) gives the
 * rotation's relative-position property.
 *
 * Token s of sequence b takes position pos = seq_lens[b] - Sq + s (seq_lens
 * already counts the new tokens, as for mla_decode_splitkv) and cache row
 * block_table[b, pos / 64] * 64 + pos % 64.  RoPE, rotate-half form, base 10000:
 * with half = d_r / 2 and theta_i = pos * 10000^(-i / half), i < half,
 *   y[i]        = x[i] cos theta_i - x[i + half] sin theta_i
 *   y[i + half] = x[i + half] cos theta_i + x[i] sin theta_i
 * computed in fp64, rounded once to fp32, then to the destination format.
 * Latent rows are stored in kv_dtype (round to nearest even from fp32).  For an
 * FP8_E4M3 cache, per token: s0 = max(amax, 2^-20) / 448 (a correctly rounded
 * fp32 division), scale = the smallest power of two >= s0, r_j = x_j / scale
 * (exact), code_j = the E4M3 value nearest to r_j (ties to even, |r_j| > 448
 * saturating to 448, sign kept), and the token's kv_scale entry = scale.  Every
 * scale written is a power of two, so a cache filled only by this call may be
 * read with MLA_FLAG_POW2_SCALE.
 *
 *   c_new      [B,Sq,d_c]    q_dtype  (in: latent rows of the new tokens)
 *   kpe_new    [B,Sq,d_r]    q_dtype  (in: RoPE keys before rotation; may be NULL iff d_r == 0)
 *   q_rope_in  [B,Sq,H,d_r]  q_dtype  (in, may be NULL: query RoPE parts before rotation)
 *   q_rope_out [B,Sq,H,d_r]  q_dtype  (out; NULL iff q_rope_in is NULL; may equal q_rope_in)
 *   block_table, seq_lens    as for mla_decode_splitkv; seq_lens[b] >= Sq
 *   c_kv       [num_pages,64,d_c] kv_dtype (in/out: only the new tokens' rows are written)
 *   k_pe       [num_pages,64,d_r] pe_dtype (in/out: likewise)
 *   kv_scale   [num_pages,64] fp32 (out for the new rows; required iff kv_dtype == FP8_E4M3)
 * d_r must be even.  Two new tokens must not map to the same cache row
 * (distinct pages per sequence), else the result is undefined.
 */
mla_status_t mla_append_kv(const mla_params_t *p, const void *c_new, const void *kpe_new,
                           const void *q_rope_in, void *q_rope_out, const int32_t *block_table,
                           const int32_t *seq_lens, void *c_kv, void *k_pe, float *kv_scale,
                           void *stream);

/*
 * mla_expand_kv -- a bf16 copy of an e4m3 latent cache with each token's scale
 * applied (the cache's value semantics: c = code * kv_scale, "DeepSeek-MLA-
 * Principle" sec. 3 on the cache footprint; the per-token quantisation is that of
 * mla_append_kv):
 *   c_out[page, slot, m] = bf16_rne(float(e4m3(c_kv[page, slot, m])) * kv_scale[page, slot])
 * (one fp32 product, then rounding to nearest even).  Every page is expanded.
 * mla_decode_splitkv on the bf16 copy (kv_dtype = bf16, the 128-row kernel) gives
 * the same partials, bit for bit, as on the e4m3 cache directly; the direct call
 * needs no bf16 workspace and measured faster (B = 128, Sq = 4: 1.43-1.47 ms
 * against 1.52-1.59 ms with the expansion), so this entry point is an option, not
 * the default route.
 *
 *   c_kv     [num_pages,64,d_c]  e4m3 codes  (in; kv_dtype must be MLA_FP8_E4M3)
 *   kv_scale [num_pages,64]      fp32        (in)
 *   c_out    [num_pages,64,d_c]  bf16        (out)
 */
mla_status_t mla_expand_kv(const mla_params_t *p, const void *c_kv, const float *kv_scale, void *c_out,
                           void *stream);

/*
 * The non-absorbed path, for many new tokens per sequence (prefill, chunked
 * prefill).  "MLA Matrix Absorption" sec. 6 describes the switch: with x new tokens
 * per sequence at or above a threshold (about 64) the per-head keys and values are
 * decompressed from the latent cache and a standard attention runs; below it the
 * absorbed path (the four calls above) wins.  "DeepSeek-MLA-Principle" eqs. (2),
 * (4), (10): k_{t,h} = [W_UK[h] c_t ; k_pe_t], v_{t,h} = W_UV[h] c_t.  Both paths
 * compute the same attention (absorption is an exact re-association).
 *
 * These entry points take Sq = x new tokens per sequence with 1 <= x <= 65536
 * (token s of sequence b at position seq_lens[b] - x + s, as for the decode).
 * Kernels exist for d_h = 128, d_c = 512, d_r = 64 with bf16 queries, weights,
 * latent cache and RoPE keys; other requests return MLA_ERR_UNSUPPORTED.
 * Lmax = mla_prefill_lmax(p) (max_pages * 64 rounded up to a multiple of 256) is
 * the row stride of the decompressed tensors.
 */

/*
 * mla_decompress_kv -- per-head keys (content part) and values of every cached
 * position t < seq_lens[b]:
 *   k_nope[b, t, h, d] = sum_m W_UK[h,d,m] c_t[m]
 *   v_t[b, h, d, t]    = sum_m W_UV[h,d,m] c_t[m]      (values stored transposed)
 * accumulated in fp32, rounded once to latent_dtype.  Positions from seq_lens[b]
 * up to the next multiple of 256 are written with zeros; later positions are not
 * written.
 *
 *   c_kv, block_table, seq_lens   as for mla_decode_splitkv (bf16 cache)
 *   W_UK, W_UV  [H,d_h,d_c]         w_dtype        (in)
 *   k_nope      [B,Lmax,H,d_h]      latent_dtype   (out)
 *   v_t         [B,H,d_h,Lmax]      latent_dtype   (out)
 */
mla_status_t mla_decompress_kv(const mla_params_t *p, const void *c_kv, const int32_t *block_table,
                               const int32_t *seq_lens, const void *W_UK, const void *W_UV, void *k_nope,
                               void *v_t, void *stream);

/*
 * mla_prefill_attention -- standard causal attention of the Sq new tokens of
 * every sequence with the decompressed keys and values: for row (b,s,h),
 * n = seq_lens[b] - Sq + 1 + s visible positions,
 *   z_t = scale * (q_nope[b,s,h,:] . k_nope[b,t,h,:] + q_rope[b,s,h,:] . k_pe_t),  t < n
 *   out[b,s,h,:] = sum_{t<n} softmax(z)_t v[b,t,h,:]
 * (out = 0 when n <= 0).  The weights are rounded to bf16 for the value product
 * and the sum is normalised by the weights as rounded.
 *
 *   q_nope [B,Sq,H,d_h], q_rope [B,Sq,H,d_r]   q_dtype       (in)
 *   k_nope [B,Lmax,H,d_h], v_t [B,H,d_h,Lmax]  latent_dtype  (in: from mla_decompress_kv)
 *   k_pe, block_table, seq_lens                as for mla_decode_splitkv
 *   out    [B,Sq,H,d_h]                        out_dtype     (out)
 */
mla_status_t mla_prefill_attention(const mla_params_t *p, const void *q_nope, const void *q_rope,
                                   const void *k_nope, const void *v_t, const void *k_pe,
                                   const int32_t *block_table, const int32_t *seq_lens, void *out,
                                   void *stream);

/* Row stride Lmax (positions) of the decompressed tensors for *p: max_pages * 64
 * rounded up to a multiple of 256 (host-only; -1 for invalid parameters). */
int64_t mla_prefill_lmax(const mla_params_t *p);

/* The switch of "MLA Matrix Absorption" sec. 6 (host-only): 1 when Sq new tokens
 * per sequence are served faster by the absorbed path, 0 when by the non-absorbed
 * one; -1 for invalid parameters.  The pages put the crossover near 64 new tokens;
 * with these kernels the two paths measure equal near 120, so the switch is at
 * Sq = 120 (absorbed below).  Both paths accept 1 <= Sq <= 256 and agree there;
 * the non-absorbed path accepts up to 65,536. */
int32_t mla_prefer_absorbed(const mla_params_t *p);

/* Host-only validation of *p (no GPU needed).  Returns MLA_OK or the first error. */
mla_status_t mla_check_params(const mla_params_t *p);

/*
 * Host-only split planner.  Given the longest sequence (tokens), the total
 * tokens of the batch and the number of compute units to fill, chooses
 * balanced splits: sets p->num_parts (P: one attention workgroup per compute
 * unit, at least 8 parts, parts of at least 4 pages on average (2 with bf16
 * partials), at least
 * `min_splits` parts when the batch has that many pages) and p->num_splits, the
 * bound on the parts one sequence can touch.  It extends mla_default_num_splits
 * (uniform lengths, fixed splits) to any mix of lengths.  max_seq_len must not be
 * below, and total_tokens not above, the true values; the plan depends on
 * seq_lens through them, so it must be recomputed whenever a sequence grows past
 * max_seq_len (a split index at or past num_splits is not computed).
 * Reads B, Sq, H, max_pages, the dtypes and flags.  Returns MLA_OK or an error.
 */
mla_status_t mla_plan_splits(mla_params_t *p, int32_t max_seq_len, int64_t total_tokens,
                             int32_t num_cus, int32_t min_splits);

/*
 * Host-only default split count for fixed splits (num_parts == 0): the number of
 * KV chunks per sequence that fills the 256 compute units of an MI355X when all
 * B sequences hold max_seq_len tokens, i.e. ceil(P / B) for the part count P that
 * mla_plan_splits picks for that batch, clamped to [1, ceil(max_seq_len / 64)].
 * Use it with split_pages = ceil(ceil(max_seq_len / 64) / S).  Reads the same
 * fields as mla_plan_splits.  Returns S >= 1, or -1 (mla_last_error says why) for
 * a NULL or invalid p or max_seq_len < 1.
 */
int32_t mla_default_num_splits(const mla_params_t *p, int32_t max_seq_len);

/*
 * mla_device_errors -- synchronises `stream`, then returns in *bits the OR of the
 * MLA_DEVERR_* bits the attention kernels of this process raised on the current
 * device since the previous call, and clears them.  The kernels never stop or
 * fault on these conditions: a stale plan's extra pages are skipped (their rows'
 * results are then wrong), a wait that gives up continues with the data at hand,
 * and (MLA_DEBUG_BOUNDS build, libmla_debug.so) an out-of-range page or length is
 * replaced by page 0 or clamped.  The one entry point that synchronises.
 * Returns MLA_OK, MLA_ERR_NULL or MLA_ERR_HIP.
 */
mla_status_t mla_device_errors(uint32_t *bits, void *stream);

/* 1 when this library was built with the MLA_DEBUG_BOUNDS device checks, else 0. */
int32_t mla_debug_bounds(void);

/* Name of the attention kernel mla_decode_splitkv would launch for *p (host-only):
 * "mfma_bf16_128" / "mfma_fp8_128" (four waves, 128 query rows per workgroup),
 * "mfma_bf16_64" (eight waves, 64 rows), "mfma_fp8_64" (e4m3 cache, four waves, 64
 * rows), "generic_f32" (fp32 VALU), or "invalid" (bad parameters or flags). */
const char *mla_decode_kernel_name(const mla_params_t *p);

/* Static string for a status code. */
const char *mla_status_string(mla_status_t s);

/* Message describing the calling thread's most recent failed call ("" if none). */
const char *mla_last_error(void);

/* ABI version: bumped when mla_params_t or a signature changes. */
int32_t mla_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
