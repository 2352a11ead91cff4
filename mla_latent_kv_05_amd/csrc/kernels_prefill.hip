// The non-absorbed path for many new tokens per sequence, gfx950 / CDNA4:
// mla_decompress_kv and mla_prefill_attention at d_h = 128, d_c = 512, d_r = 64,
// bf16 operands, v_mfma_f32_32x32x16_bf16.
//
// "MLA Matrix Absorption" sec. 6: with many new tokens x per sequence (prefill),
// the per-head keys and values are decompressed from the latent cache once and a
// standard attention runs over them (large dense products); with few (decode)
// the absorbed form wins.  "DeepSeek-MLA-Principle" eqs. (2), (4), (10): the key
// of head h at position t is [W_UK[h] c_t ; k_pe_t], its value W_UV[h] c_t, the
// score scale 1/sqrt(d_h + d_r), and row s attends to positions t <= its own.
//
// Decompress: one workgroup (4 waves) per (sequence, 32-position tile, group of 8
// heads).  Every wave holds the tile's latent rows as MFMA operands (128 VGPRs)
// and, for each head of the group, forms its 32 output dims of the keys
// K[t, d] = c_t . W_UK[h, d, :] and of the transposed values V^T[d, t] =
// W_UV[h, d, :] . c_t: the latent row is the A operand of the first product and
// the B operand of the second, with the same register contents (both read 8
// consecutive latent values per lane), so each value row lands contiguous along
// t.  The weights are read from L2.
//
// Attention: one workgroup (4 waves) per (sequence, head, 128 new tokens); wave w
// takes 32 of them.  Per tile of 32 positions:
//   S^T[t, q] = K_tile . Q^T over the 192 dims (12 MFMAs; Q^T in registers).  Tile
//   row r holds position swap23(r) (bits 2 and 3 of r exchanged), so that the 16
//   weights a lane holds for query q are, as the B operand of the next product,
//   positions 16ks + 8g + e in order;
//   online softmax per query in the exp2 domain (a lane pair per query);
//   O^T[d, q] += V^T[d, t] . P^T[t, q] (8 MFMAs; V^T rows read 16 bytes at a time
//   from the transposed values).
// Positions at or past seq_len inside the last tile are masked in the scores and
// zeroed in the value operand (the decompressed tensors are not written there).
#include <hip/hip_runtime.h>
#include <math.h>

#include "gfx950.h"
#include "mla_internal.h"

namespace mla {
namespace {

using namespace gfx;

constexpr int kDh = 128;
constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kHeadsPerWg = 8;                 // heads of one decompress workgroup
constexpr int kQPerWg = 128;                   // new tokens of one attention workgroup
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ uint16_t bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);           // round to nearest even (finite values)
    return static_cast<uint16_t>(u >> 16);
}

// tile row r holds position swap23(r) of the tile
__device__ __forceinline__ int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void decompress_kernel(const mla_params_t p, const uint16_t *__restrict__ c_kv,
                                                         const int32_t *__restrict__ block_table,
                                                         const int32_t *__restrict__ seq_lens,
                                                         const uint16_t *__restrict__ W_UK,
                                                         const uint16_t *__restrict__ W_UV,
                                                         uint16_t *__restrict__ k_nope, uint16_t *__restrict__ v_t) {
    const int lane = threadIdx.x & 63, t32 = lane & 31, g = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n_hg = (p.H + kHeadsPerWg - 1) / kHeadsPerWg;
    const int64_t lmax = static_cast<int64_t>(p.max_pages) * 64;
    const int tiles = p.max_pages * 2;
    int64_t bid = blockIdx.x;
    const int hg = static_cast<int>(bid % n_hg);
    bid /= n_hg;
    const int tile = static_cast<int>(bid % tiles);
    const int b = static_cast<int>(bid / tiles);
    const int L = seq_lens[b];
    const int t0 = tile * 32;
    if (t0 >= L) return;
    // the latent row of position t0 + t32: dims 16ks + 8g .. 16ks + 8g + 7
    const int t = t0 + t32;
    const bool valid = t < L;
    int64_t crow = 0;
    if (valid) crow = static_cast<int64_t>(block_table[static_cast<int64_t>(b) * p.max_pages + t / 64]) * 64 + t % 64;
    bf16x8 cop[kDc / 16];
#pragma unroll
    for (int ks = 0; ks < kDc / 16; ++ks) {
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (valid) v = *reinterpret_cast<const u32x4 *>(c_kv + crow * kDc + ks * 16 + g * 8);
        cop[ks] = as_bf16x8(v);
    }
    const int d = 32 * w + t32;                // this lane's weight row (operand) / output dim
    for (int hh = 0; hh < kHeadsPerWg; ++hh) {
        const int h = hg * kHeadsPerWg + hh;
        if (h >= p.H) break;
        const uint16_t *wk = W_UK + (static_cast<int64_t>(h) * kDh + d) * kDc + g * 8;
        const uint16_t *wv = W_UV + (static_cast<int64_t>(h) * kDh + d) * kDc + g * 8;
        f32x16 ak, av;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            ak[j] = 0.f;
            av[j] = 0.f;
        }
#pragma unroll
        for (int ks = 0; ks < kDc / 16; ++ks) {
            const bf16x8 bk = as_bf16x8(*reinterpret_cast<const u32x4 *>(wk + ks * 16));
            const bf16x8 bv = as_bf16x8(*reinterpret_cast<const u32x4 *>(wv + ks * 16));
            ak = mfma32(cop[ks], bk, ak);      // D[position, d]
            av = mfma32(bv, cop[ks], av);      // D[d, position]
        }
        // ak[j]: position t0 + 8(j/4) + 4g + j%4, dim d;  av[j]: dim 32w + 8(j/4) + 4g + j%4, position t
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int r = 8 * (j >> 2) + 4 * g + (j & 3);
            if (t0 + r < L) k_nope[((static_cast<int64_t>(b) * lmax + t0 + r) * p.H + h) * kDh + d] = bf16_bits(ak[j]);
            if (valid) v_t[((static_cast<int64_t>(b) * p.H + h) * kDh + 32 * w + r) * lmax + t] = bf16_bits(av[j]);
        }
    }
}

// ---------------------------------------------------------------------------
template <bool kOutBf16>
__global__ __launch_bounds__(256) void prefill_attention_kernel(
    const mla_params_t p, const uint16_t *__restrict__ q_nope, const uint16_t *__restrict__ q_rope,
    const uint16_t *__restrict__ k_nope, const uint16_t *__restrict__ v_t, const uint16_t *__restrict__ k_pe,
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ seq_lens, void *__restrict__ out) {
    const int lane = threadIdx.x & 63, t32 = lane & 31, g = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n_qb = (p.Sq + kQPerWg - 1) / kQPerWg;
    const int64_t lmax = static_cast<int64_t>(p.max_pages) * 64;
    int64_t bid = blockIdx.x;
    const int qb = static_cast<int>(bid % n_qb);
    bid /= n_qb;
    const int h = static_cast<int>(bid % p.H);
    const int b = static_cast<int>(bid / p.H);
    const int s0 = qb * kQPerWg + 32 * w;      // this wave's first new token
    if (s0 >= p.Sq) return;
    const int L = seq_lens[b];
    const int base = L - p.Sq;                 // position of new token 0
    const int s = s0 + t32;                    // this lane's query
    const bool q_ok = s < p.Sq;
    const int pos_q = base + s;                // last visible position of the query
    // last visible position of any query of the wave (uniform)
    const int pos_max = __builtin_amdgcn_readfirstlane(base + min(s0 + 31, p.Sq - 1));
    const int64_t qrow = (static_cast<int64_t>(b) * p.Sq + (q_ok ? s : s0)) * p.H + h;
    // Q^T (B operand): k-steps 0..7 the content dims, 8..11 the RoPE dims
    bf16x8 qreg[12];
#pragma unroll
    for (int ks = 0; ks < 12; ++ks) {
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (q_ok) {
            if (ks < 8) v = *reinterpret_cast<const u32x4 *>(q_nope + qrow * kDh + ks * 16 + g * 8);
            else v = *reinterpret_cast<const u32x4 *>(q_rope + qrow * kDr + (ks - 8) * 16 + g * 8);
        }
        qreg[ks] = as_bf16x8(v);
    }
    const float zscale = p.scale * kLog2e;
    float m_run = -INFINITY;                   // running maximum (log2 domain), same in the lane pair
    float l_run = 0.f;                         // this lane's share of the sum of bf16-rounded weights
    f32x16 o[4];                               // O^T tiles: dims 32dt .., query t32
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[dt][j] = 0.f;
    const uint16_t *vrow = v_t + ((static_cast<int64_t>(b) * p.H + h) * kDh + t32) * lmax;   // + 32dt*lmax
    const int32_t *bt = block_table + static_cast<int64_t>(b) * p.max_pages;
    const int n_tiles = pos_max >= 0 ? pos_max / 32 + 1 : 0;
    for (int kt = 0; kt < n_tiles; ++kt) {
        const int k0 = kt * 32;
        // K operand: tile row t32 holds position k0 + swap23(t32)
        const int key = k0 + swap23(t32);
        const bool key_ok = key < L;
        const int kk = key_ok ? key : L - 1;
        const uint16_t *krow = k_nope + ((static_cast<int64_t>(b) * lmax + kk) * p.H + h) * kDh + g * 8;
        const int64_t prow = static_cast<int64_t>(bt[kk / 64]) * 64 + kk % 64;
        const uint16_t *rrow = k_pe + prow * kDr + g * 8;
        f32x16 sacc;
#pragma unroll
        for (int j = 0; j < 16; ++j) sacc[j] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 12; ++ks) {
            const u32x4 a = ks < 8 ? *reinterpret_cast<const u32x4 *>(krow + ks * 16)
                                   : *reinterpret_cast<const u32x4 *>(rrow + (ks - 8) * 16);
            sacc = mfma32(as_bf16x8(a), qreg[ks], sacc);
        }
        // sacc[j]: position k0 + swap23(8(j/4) + 4g + j%4) = k0 + 16(j/8) + 8g + (j%8), query t32
        float sc[16];
        float mloc = -INFINITY;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int pos = k0 + 16 * (j >> 3) + 8 * g + (j & 7);
            sc[j] = (pos <= pos_q && pos < L) ? sacc[j] * zscale : -INFINITY;
            mloc = fmaxf(mloc, sc[j]);
        }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
        const float m_new = fmaxf(m_run, mloc);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;   // nothing visible yet: weights 0
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);   // 0 on the first visible tile
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int j = 0; j < 16; ++j) o[dt][j] *= alpha;
        // weights, rounded to bf16 for the value product; B operand of k-step kp:
        // positions k0 + 16kp + 8g + e, e < 8
        uint32_t pk[2][4];
#pragma unroll
        for (int kp = 0; kp < 2; ++kp)
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const float p0 = __builtin_amdgcn_exp2f(sc[8 * kp + 2 * e2] - m_use);
                const float p1 = __builtin_amdgcn_exp2f(sc[8 * kp + 2 * e2 + 1] - m_use);
                const uint32_t pr = cvt_pk_bf16(p0, p1);
                pk[kp][e2] = pr;
                l_run += __uint_as_float(pr << 16) + __uint_as_float(pr & 0xffff0000u);
            }
        // O^T += V^T . P^T: A operand of dim tile dt, k-step kp: dims 32dt + t32,
        // positions k0 + 16kp + 8g .. +7 (zero past the sequence end)
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
            const int pv0 = k0 + 16 * kp + 8 * g;
            const bf16x8 pb = as_bf16x8(u32x4{pk[kp][0], pk[kp][1], pk[kp][2], pk[kp][3]});
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                u32x4 va = *reinterpret_cast<const u32x4 *>(vrow + static_cast<int64_t>(32 * dt) * lmax + pv0);
                if (pv0 + 8 > L) {
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2) {
                        const uint32_t lo_ok = pv0 + 2 * e2 < L ? 0x0000ffffu : 0u;
                        const uint32_t hi_ok = pv0 + 2 * e2 + 1 < L ? 0xffff0000u : 0u;
                        va[e2] &= lo_ok | hi_ok;
                    }
                }
                o[dt] = mfma32(as_bf16x8(va), pb, o[dt]);
            }
        }
    }
    if (!q_ok) return;
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    // o[dt][j]: dim 32dt + 8(j/4) + 4g + j%4, query s
    const int64_t orow = ((static_cast<int64_t>(b) * p.Sq + s) * p.H + h) * kDh;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int d0 = 32 * dt + 8 * q4 + 4 * g;
            const f32x4 v = f32x4{o[dt][4 * q4], o[dt][4 * q4 + 1], o[dt][4 * q4 + 2], o[dt][4 * q4 + 3]} * inv;
            if constexpr (kOutBf16) {
                uint16_t *dst = static_cast<uint16_t *>(out) + orow + d0;
                *reinterpret_cast<u32x2 *>(dst) = u32x2{cvt_pk_bf16(v[0], v[1]), cvt_pk_bf16(v[2], v[3])};
            } else {
                *reinterpret_cast<f32x4 *>(static_cast<float *>(out) + orow + d0) = v;
            }
        }
}

}  // namespace

bool prefill_supported(const mla_params_t &p) {
    return p.d_h == kDh && p.d_c == kDc && p.d_r == kDr && p.page_size == 64 && p.q_dtype == MLA_BF16 &&
           p.w_dtype == MLA_BF16 && p.kv_dtype == MLA_BF16 && p.pe_dtype == MLA_BF16 && p.latent_dtype == MLA_BF16;
}

hipError_t launch_decompress(const mla_params_t &p, const void *c_kv, const int32_t *block_table,
                             const int32_t *seq_lens, const void *W_UK, const void *W_UV, void *k_nope, void *v_t,
                             hipStream_t stream) {
    const int64_t n_hg = (p.H + kHeadsPerWg - 1) / kHeadsPerWg;
    const int64_t blocks = static_cast<int64_t>(p.B) * p.max_pages * 2 * n_hg;
    hipLaunchKernelGGL(decompress_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, p,
                       static_cast<const uint16_t *>(c_kv), block_table, seq_lens,
                       static_cast<const uint16_t *>(W_UK), static_cast<const uint16_t *>(W_UV),
                       static_cast<uint16_t *>(k_nope), static_cast<uint16_t *>(v_t));
    return hipGetLastError();
}

hipError_t launch_prefill_attention(const mla_params_t &p, const void *q_nope, const void *q_rope,
                                    const void *k_nope, const void *v_t, const void *k_pe,
                                    const int32_t *block_table, const int32_t *seq_lens, void *out,
                                    hipStream_t stream) {
    const int64_t blocks = static_cast<int64_t>(p.B) * p.H * ((p.Sq + kQPerWg - 1) / kQPerWg);
    const auto qn = static_cast<const uint16_t *>(q_nope);
    const auto qr = static_cast<const uint16_t *>(q_rope);
    const auto kn = static_cast<const uint16_t *>(k_nope);
    const auto vt = static_cast<const uint16_t *>(v_t);
    const auto kp = static_cast<const uint16_t *>(k_pe);
    if (p.out_dtype == MLA_BF16)
        hipLaunchKernelGGL(prefill_attention_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                           p, qn, qr, kn, vt, kp, block_table, seq_lens, out);
    else
        hipLaunchKernelGGL(prefill_attention_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                           p, qn, qr, kn, vt, kp, block_table, seq_lens, out);
    return hipGetLastError();
}

}  // namespace mla
