// bf16 MFMA kernels for the two per-head projections of absorbed-MLA decode at
// the DeepSeek-V3 head shapes (d_h = 128, d_c = 512), gfx950 / CDNA4:
// mla_absorb_q (q_abs = q_nope . W_UK) and mla_up_v (out = o_latent . W_UV^T).
// Both are per-head batched GEMMs with a small row count (B*Sq), bound by
// reading the weights; each wave streams a slice of one head's weight matrix
// once and applies it to up to 64 rows on v_mfma_f32_16x16x32_bf16.
#include <hip/hip_runtime.h>

#include "gfx950.h"
#include "mla_internal.h"

namespace mla {
namespace {

using namespace gfx;

constexpr int kDc = 512;

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) { return cvt_pk_bf16(a, b); }

// ---------------------------------------------------------------------------
// mla_absorb_q: q_abs[r, h, m] = sum_d q_nope[r, h, d] W_UK[h, d, m]
// One wave per (head, 64-row chunk, 128-column quarter of d_c).
// D^T[m, r] = W^T[m, d] . q^T[d, r]: W rows are read 8 at a time (16 bytes
// each) and transposed in registers into 8 A operands covering 128 columns.
// ---------------------------------------------------------------------------
template <int kDh>
__global__ __launch_bounds__(64) void absorb_mfma_kernel(
    const mla_params_t p, const uint16_t *__restrict__ q_nope, const uint16_t *__restrict__ W_UK,
    uint16_t *__restrict__ q_abs) {
    const int lane = threadIdx.x, r16 = lane & 15, g = lane >> 4;
    const int R = p.B * p.Sq;
    const int h = blockIdx.x % p.H;
    const int rest = blockIdx.x / p.H;
    const int cq = rest & 3;                      // 128-column quarter of d_c
    const int r0 = (rest >> 2) * 64;              // first row of the chunk
    const int col0 = cq * 128 + r16 * 8;          // this lane's 8 columns in A
    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) acc[i][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint16_t *W = W_UK + static_cast<int64_t>(h) * kDh * kDc;
#pragma unroll 1
    for (int ks = 0; ks < kDh / 32; ++ks) {
        u32x4 rows[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            rows[e] = *reinterpret_cast<const u32x4 *>(W + static_cast<int64_t>(ks * 32 + g * 8 + e) * kDc + col0);
        bf16x8 bq[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const int r = r0 + rt * 16 + r16;
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (r < R) v = *reinterpret_cast<const u32x4 *>(q_nope + (static_cast<int64_t>(r) * p.H + h) * kDh + ks * 32 + g * 8);
            bq[rt] = as_bf16x8(v);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            u32x4 a;
#pragma unroll
            for (int k2 = 0; k2 < 4; ++k2)
                a[k2] = (i & 1) ? pack_hi(rows[2 * k2][i >> 1], rows[2 * k2 + 1][i >> 1])
                                : pack_lo(rows[2 * k2][i >> 1], rows[2 * k2 + 1][i >> 1]);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) acc[i][rt] = mfma16(as_bf16x8(a), bq[rt], acc[i][rt]);
        }
    }
    // acc[i][rt][j]: row r0 + rt*16 + r16, column cq*128 + 8*(4g + j) + i
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        const int r = r0 + rt * 16 + r16;
        if (r >= R) continue;
        uint16_t *dst = q_abs + (static_cast<int64_t>(r) * p.H + h) * kDc + cq * 128;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u32x4 v;
#pragma unroll
            for (int k2 = 0; k2 < 4; ++k2) v[k2] = pack_bf16x2(acc[2 * k2][rt][j], acc[2 * k2 + 1][rt][j]);
            *reinterpret_cast<u32x4 *>(dst + (g * 4 + j) * 8) = v;
        }
    }
}

// ---------------------------------------------------------------------------
// mla_up_v: out[r, h, d] = sum_m o_latent[r, h, m] W_UV[h, d, m]
// One wave per (head, 64-row chunk, 32-row quarter of d_h... generalised to
// d_h/4 rows): D^T[d, r] = W_UV[d, m] . o^T[m, r]; both operands are
// contiguous along m, so no transpose is needed.
// ---------------------------------------------------------------------------
template <int kDh, bool kOutBf16>
__global__ __launch_bounds__(64) void up_v_mfma_kernel(
    const mla_params_t p, const uint16_t *__restrict__ o_latent, const uint16_t *__restrict__ W_UV,
    void *__restrict__ out) {
    constexpr int kDt = kDh / 4 / 16;             // 16-row d tiles per wave
    const int lane = threadIdx.x, r16 = lane & 15, g = lane >> 4;
    const int R = p.B * p.Sq;
    const int h = blockIdx.x % p.H;
    const int rest = blockIdx.x / p.H;
    const int dq = rest & 3;
    const int r0 = (rest >> 2) * 64;
    const int d0 = dq * (kDh / 4);
    f32x4 acc[kDt][4];
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) acc[dt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint16_t *W = W_UV + static_cast<int64_t>(h) * kDh * kDc;
    bool rvalid[4];
    const uint16_t *orow[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        const int r = r0 + rt * 16 + r16;
        rvalid[rt] = r < R;
        orow[rt] = o_latent + (static_cast<int64_t>(rvalid[rt] ? r : 0) * p.H + h) * kDc;
    }
#pragma unroll 2
    for (int ks = 0; ks < kDc / 32; ++ks) {
        bf16x8 bo[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (rvalid[rt]) v = *reinterpret_cast<const u32x4 *>(orow[rt] + ks * 32 + g * 8);
            bo[rt] = as_bf16x8(v);
        }
#pragma unroll
        for (int dt = 0; dt < kDt; ++dt) {
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(W + static_cast<int64_t>(d0 + dt * 16 + r16) * kDc + ks * 32 + g * 8);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) acc[dt][rt] = mfma16(a, bo[rt], acc[dt][rt]);
        }
    }
    // acc[dt][rt][j]: row r0 + rt*16 + r16, d = d0 + dt*16 + 4g + j
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        if (!rvalid[rt]) continue;
        const int64_t base = (static_cast<int64_t>(r0 + rt * 16 + r16) * p.H + h) * kDh + d0;
#pragma unroll
        for (int dt = 0; dt < kDt; ++dt) {
            if constexpr (kOutBf16) {
                uint16_t *o = static_cast<uint16_t *>(out) + base + dt * 16 + g * 4;
                *reinterpret_cast<u32x2 *>(o) = u32x2{pack_bf16x2(acc[dt][rt][0], acc[dt][rt][1]),
                                                      pack_bf16x2(acc[dt][rt][2], acc[dt][rt][3])};
            } else {
                float *o = static_cast<float *>(out) + base + dt * 16 + g * 4;
                *reinterpret_cast<f32x4 *>(o) = acc[dt][rt];
            }
        }
    }
}

}  // namespace

bool absorb_mfma_supported(const mla_params_t &p) {
    if (p.flags & MLA_FLAG_GENERIC) return false;
    return p.d_c == kDc && p.d_h == 128 && p.q_dtype == MLA_BF16 && p.w_dtype == MLA_BF16 &&
           p.latent_dtype == MLA_BF16;
}

hipError_t launch_absorb_mfma(const mla_params_t &p, const void *q_nope, const void *W_UK,
                              void *q_abs, hipStream_t stream) {
    const int64_t R = static_cast<int64_t>(p.B) * p.Sq;
    const int64_t blocks = static_cast<int64_t>(p.H) * 4 * ((R + 63) / 64);
    hipLaunchKernelGGL(absorb_mfma_kernel<128>, dim3(static_cast<unsigned>(blocks)), dim3(64), 0, stream, p,
                       static_cast<const uint16_t *>(q_nope), static_cast<const uint16_t *>(W_UK),
                       static_cast<uint16_t *>(q_abs));
    return hipGetLastError();
}

bool up_v_mfma_supported(const mla_params_t &p) {
    if (p.flags & MLA_FLAG_GENERIC) return false;
    return p.d_c == kDc && p.d_h == 128 && p.latent_dtype == MLA_BF16 && p.w_dtype == MLA_BF16;
}

hipError_t launch_up_v_mfma(const mla_params_t &p, const void *o_latent, const void *W_UV,
                            void *out, hipStream_t stream) {
    const int64_t R = static_cast<int64_t>(p.B) * p.Sq;
    const int64_t blocks = static_cast<int64_t>(p.H) * 4 * ((R + 63) / 64);
    const auto ol = static_cast<const uint16_t *>(o_latent);
    const auto w = static_cast<const uint16_t *>(W_UV);
    if (p.out_dtype == MLA_BF16)
        hipLaunchKernelGGL((up_v_mfma_kernel<128, true>), dim3(static_cast<unsigned>(blocks)), dim3(64), 0, stream,
                           p, ol, w, out);
    else
        hipLaunchKernelGGL((up_v_mfma_kernel<128, false>), dim3(static_cast<unsigned>(blocks)), dim3(64), 0, stream,
                           p, ol, w, out);
    return hipGetLastError();
}

}  // namespace mla
