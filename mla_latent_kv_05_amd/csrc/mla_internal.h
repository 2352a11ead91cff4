// Internal launcher interface between the C ABI (mla_api.cpp) and the HIP
// kernel translation units.  Every launcher enqueues on `stream` and returns
// the launch status; arguments were validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla.h"

namespace mla {

// fp32 VALU kernels for any supported shape / dtype (kernels_generic.hip)
hipError_t launch_absorb_generic(const mla_params_t &p, const void *q_nope, const void *W_UK,
                                 void *q_abs, hipStream_t stream);
hipError_t launch_decode_generic(const mla_params_t &p, const void *q_abs, const void *q_rope,
                                 const void *c_kv, const void *k_pe, const float *kv_scale,
                                 const int32_t *block_table, const int32_t *seq_lens,
                                 void *o_part, float *lse_part, hipStream_t stream);
hipError_t launch_up_v_generic(const mla_params_t &p, const void *o_latent, const void *W_UV,
                               void *out, hipStream_t stream);
hipError_t launch_combine(const mla_params_t &p, const void *o_part, const float *lse_part,
                          void *o_latent, float *lse_out, hipStream_t stream);

// kernels for the DeepSeek-V3 head shapes (kernels_mfma.hip, kernels_decode.hip: both cache
// dtypes)
bool decode_mfma_supported(const mla_params_t &p);
hipError_t launch_decode_mfma(const mla_params_t &p, const void *q_abs, const void *q_rope,
                              const void *c_kv, const void *k_pe, const float *kv_scale,
                              const int32_t *block_table, const int32_t *seq_lens,
                              void *o_part, float *lse_part, hipStream_t stream);
// bf16 cache: eight-wave attention kernel (kernels_decode8.hip)
bool decode8_supported(const mla_params_t &p);
hipError_t launch_decode8(const mla_params_t &p, const void *q_abs, const void *q_rope, const void *c_kv,
                          const void *k_pe, const int32_t *block_table, const int32_t *seq_lens, void *o_part,
                          float *lse_part, hipStream_t stream);
bool absorb_mfma_supported(const mla_params_t &p);
hipError_t launch_absorb_mfma(const mla_params_t &p, const void *q_nope, const void *W_UK,
                              void *q_abs, hipStream_t stream);
bool up_v_mfma_supported(const mla_params_t &p);
bool combine_fast_supported(const mla_params_t &p);
bool combine_up_v_supported(const mla_params_t &p);
hipError_t launch_expand(const mla_params_t &p, const void *c_kv, const float *kv_scale, void *c_out,
                         hipStream_t stream);
hipError_t launch_combine_up_v(const mla_params_t &p, const void *o_part, const float *lse_part, const void *W_UV,
                               void *out, float *lse_out, hipStream_t stream);
hipError_t launch_combine_fast(const mla_params_t &p, const void *o_part, const float *lse_part,
                               void *o_latent, float *lse_out, hipStream_t stream);
hipError_t launch_up_v_mfma(const mla_params_t &p, const void *o_latent, const void *W_UV,
                            void *out, hipStream_t stream);

// cache append with RoPE and the e4m3 quantiser (kernels_append.hip)
hipError_t launch_append(const mla_params_t &p, const void *c_new, const void *kpe_new, const void *q_rope_in,
                         void *q_rope_out, const int32_t *block_table, const int32_t *seq_lens, void *c_kv,
                         void *k_pe, float *kv_scale, hipStream_t stream);

// non-absorbed path for many new tokens (kernels_prefill.hip)
bool prefill_supported(const mla_params_t &p);
// Row stride (positions) of the decompressed keys and values: max_pages * 64 rounded
// up to a whole number of 256-position decompression tiles.
__host__ __device__ inline int64_t prefill_lmax(const mla_params_t &p) { return (static_cast<int64_t>(p.max_pages) * 64 + 255) / 256 * 256; }
hipError_t launch_decompress(const mla_params_t &p, const void *c_kv, const int32_t *block_table,
                             const int32_t *seq_lens, const void *W_UK, const void *W_UV, void *k_nope, void *v_t,
                             hipStream_t stream);
hipError_t launch_prefill_attention(const mla_params_t &p, const void *q_nope, const void *q_rope,
                                    const void *k_nope, const void *v_t, const void *k_pe,
                                    const int32_t *block_table, const int32_t *seq_lens, void *out,
                                    hipStream_t stream);

// Heads x query rows handled by one attention workgroup of the e4m3 kernel
// (kernels_decode.hip) and of the eight-wave bf16 kernel (kernels_decode8.hip).
constexpr int kDecodeRowsPerBlock = 64;
// ... of the four-wave kernel (kernels_decode128.hip; bf16 and e4m3 caches).
constexpr int kDecodeRowsPerGroup = 128;
bool decode128_supported(const mla_params_t &p);
hipError_t launch_decode128(const mla_params_t &p, const void *q_abs, const void *q_rope, const void *c_kv,
                            const void *k_pe, const float *kv_scale, const int32_t *block_table,
                            const int32_t *seq_lens, void *o_part, float *lse_part, hipStream_t stream);
// Balanced parts are cut in units of work: a sequence with n > 0 pages costs
// kSeqStartCost + n units, its start cost first, then one unit per page; an empty
// sequence costs nothing.  The batch's units, taken in sequence order, are cut into
// num_parts equal parts, so a part that also starts a sequence (one more segment:
// its query loads, its first copies and its partial output) streams fewer pages.
constexpr int kSeqStartCost = 6;
// the whole step of a small batch in one cooperative launch (kernels_step_persistent.hip)
constexpr int kStepPersistentMaxPages = 4096;          // merge weights of one sequence in LDS
struct StepPersistentLayout {
    int64_t q_abs, lse_part, o_part, bytes;             // byte offsets in the workspace; counters at 0
};
bool step_persistent_supported(const mla_params_t &p);
StepPersistentLayout step_persistent_layout(const mla_params_t &p);
hipError_t launch_step_persistent(const mla_params_t &p, const void *q_nope, const void *q_rope, const void *c_kv,
                                  const void *k_pe, const int32_t *block_table, const int32_t *seq_lens,
                                  const void *W_UK, const void *W_UV, void *out, float *lse_out, char *ws,
                                  hipStream_t stream);
hipError_t take_errors_step_persistent(uint32_t *bits);
// each attention unit's device error word: OR it into *bits, then clear it
hipError_t take_errors_generic(uint32_t *bits);
hipError_t take_errors_decode_mfma(uint32_t *bits);
hipError_t take_errors_decode8(uint32_t *bits);
hipError_t take_errors_decode128(uint32_t *bits);
// the attention kernel mla_decode_splitkv launches for p on the MFMA path: the
// four-wave 128-row kernel, else the eight-wave 64-row kernel (bf16), else the
// four-wave 64-row kernel (e4m3).  Before that path: with fixed splits of one
// page each, a single new token and bf16 partials, the page kernel (one
// workgroup per page and 32 heads, kernels_step_persistent.hip).
enum class DecodeKernel { k128, k8, kMfma64 };
bool decode_page_supported(const mla_params_t &p);
// mla_absorb_q for at most 8 query rows: one workgroup per head and column half,
// fp32 VALU sums (kernels_step_persistent.hip)
bool absorb_rows_supported(const mla_params_t &p);
hipError_t launch_absorb_rows(const mla_params_t &p, const void *q_nope, const void *W_UK, void *q_abs,
                              hipStream_t stream);
hipError_t launch_decode_page(const mla_params_t &p, const void *q_abs, const void *q_rope, const void *c_kv,
                              const void *k_pe, const int32_t *block_table, const int32_t *seq_lens, void *o_part,
                              float *lse_part, hipStream_t stream);
// Batches of single new tokens whose one-page plan has at most this many page
// workgroups (pages x H / 32) per compute unit are planned with one-page splits.
constexpr int64_t kPagePlanPerCu = 2;
// Workgroups of the 128-row kernel at or below which a bf16 launch goes to the
// eight-wave kernel: with at most one 128-row workgroup per two compute units, twice
// as many 64-row workgroups (each loading half the query rows and storing half the
// partials) still fit at once and finish sooner (B = 1, 4,096 positions, 32 parts:
// 18 us against 26 us).
constexpr int64_t kSmallGrid128 = 128;
DecodeKernel decode_kernel_for(const mla_params_t &p);
// query rows per attention workgroup of that kernel
int decode_rows_per_workgroup(const mla_params_t &p);

}  // namespace mla
