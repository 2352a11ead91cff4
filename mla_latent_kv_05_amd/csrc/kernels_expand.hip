// mla_expand_kv: a bf16 copy of an e4m3 latent cache with each token's scale
// applied, gfx950 / CDNA4.  An e4m3 cache stores each latent row as codes with
// one fp32 scale per token (the per-token quantisation of the cache append); the
// row's values are code * scale.  When a decode step is bound by the matrix cores
// (many query rows per cached token), expanding the rows once per step and running
// the bf16 attention kernel is faster than converting inside the attention.
//
// One thread per 8 codes: the codes are widened to fp32 (v_cvt_pk_f32_fp8, OCP
// e4m3 on gfx950), multiplied by the token's scale (one fp32 rounding) and
// rounded to bf16 (nearest even).
#include <hip/hip_runtime.h>

#include "gfx950.h"
#include "mla_internal.h"

namespace mla {
namespace {

using namespace gfx;

__global__ __launch_bounds__(256) void expand_kernel(int64_t n_chunks, int chunks_per_row,
                                                     const uint8_t *__restrict__ codes,
                                                     const float *__restrict__ scales, uint16_t *__restrict__ out) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n_chunks) return;
    const float sc = scales[i / chunks_per_row];
    const u32x2 v = *reinterpret_cast<const u32x2 *>(codes + i * 8);
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(v[w], false);   // codes 4w, 4w+1
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(v[w], true);    // codes 4w+2, 4w+3
        o[2 * w] = cvt_pk_bf16(lo[0] * sc, lo[1] * sc);
        o[2 * w + 1] = cvt_pk_bf16(hi[0] * sc, hi[1] * sc);
    }
    *reinterpret_cast<u32x4 *>(out + i * 8) = o;
}

}  // namespace

hipError_t launch_expand(const mla_params_t &p, const void *c_kv, const float *kv_scale, void *c_out,
                         hipStream_t stream) {
    const int chunks_per_row = p.d_c / 8;
    const int64_t n_chunks = static_cast<int64_t>(p.num_pages) * p.page_size * chunks_per_row;
    const int64_t blocks = (n_chunks + 255) / 256;
    hipLaunchKernelGGL(expand_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, n_chunks,
                       chunks_per_row, static_cast<const uint8_t *>(c_kv), kv_scale, static_cast<uint16_t *>(c_out));
    return hipGetLastError();
}

}  // namespace mla
