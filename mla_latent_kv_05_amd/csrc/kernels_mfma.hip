// bf16 MFMA kernels for absorbed-MLA decode at the DeepSeek-V3 head shapes
// (d_c = 512 latent, d_r = 64 RoPE key, page = 64 tokens), gfx950 / CDNA4.
//
// Attention ("MLA Matrix Absorption" sec. 4.1-4.2; "DeepSeek-MLA-Principle"
// sec. 2 and matrix absorption 3)): every head of a sequence attends to the
// same latent cache row c_t (the MQA form of the absorbed computation), so for
// one page the scores of 16 heads are a dense [64 tokens x 576] x [576 x 16]
// product and the latent update is a dense [512 x 64] x [64 x 16] product.
// Both run on v_mfma_f32_16x16x32_bf16.
//
// Work decomposition of mla_decode_splitkv
//   workgroup = 4 waves = 64 query rows (s, h) of one sequence b and one
//               split c; wave w owns 16 heads of a single query row s.
//   grid      = B * num_splits * (Sq*H/64) workgroups, numbered so that the
//               Sq*H/64 workgroups reading the same pages land on the same
//               XCD (workgroup i runs on XCD i % 8) back to back, letting the
//               second read of a page hit that XCD's L2.
//   page loop = each 64-token page (c_kv 64 KiB + k_pe 8 KiB in bf16) is
//               copied global->LDS with global_load_lds_dwordx4 (no VGPR
//               staging), double-buffered: page i+1 streams in while page i
//               is multiplied.  The 16-byte chunks of each LDS row are
//               XOR-swizzled with the row index so that the MFMA operand
//               reads of 16 different rows hit distinct banks.
//   scores    = S^T[token, head] = K[token, 576] . Q^T[576, head]: K from LDS
//               (A operand), the wave's 16 query rows held in registers
//               (B operand, 18 k-steps of 32).
//   softmax   = online, in the exp2 domain; a head's 64 scores sit in 4 lanes
//               (xor 16, 32), so the row max needs two cross-lane steps and
//               the running sum stays per lane until the end.
//   latent PV = O^T[latent, head] += V^T[latent, token] . P^T[token, head].
//               P^T comes straight from the score accumulators (same lane =
//               same head, tokens permuted consistently); V^T is read from
//               the row-major page as 8x8 bf16 blocks and transposed in
//               registers with v_perm_b32, so LDS reads stay 16 bytes wide.
//   output    = normalised partial O_c (fp32) and its log-sum-exp per row.
// fp8 cache: the e4m3 page (32 KiB) is copied raw into LDS, converted once
// per workgroup into the same bf16 layout (e4m3 values are exact in bf16);
// the per-token scale multiplies the content score before the RoPE term is
// added and the weight p_t before it is rounded to bf16.
#include <hip/hip_runtime.h>
#include <math.h>

#include "dtype.h"
#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kPage = 64;
constexpr int kThreads = 256;
constexpr int kCkvRow = kDc * 2;                       // bf16 bytes per latent row
constexpr int kKpeRow = kDr * 2;                       // bf16 bytes per RoPE-key row
constexpr int kCkvBytes = kPage * kCkvRow;             // 65536
constexpr int kKpeBytes = kPage * kKpeRow;             // 8192
// bf16 cache: two page buffers [c_kv | k_pe]
constexpr int kBufBf16 = kCkvBytes + kKpeBytes;        // 73728
constexpr int kSmemBf16 = 2 * kBufBf16;                // 147456
// fp8 cache: two raw buffers [e4m3 c_kv | k_pe | scales] + one converted bf16 c_kv
constexpr int kRawCkv = kPage * kDc;                   // 32768
constexpr int kRawBuf = kRawCkv + kKpeBytes + kPage * 4;  // 41216
constexpr int kSmemFp8 = 2 * kRawBuf + kCkvBytes;      // 147968
constexpr int kLoadsBf16 = (kCkvBytes + kKpeBytes) / 1024 / 4;  // 18 per wave per page
constexpr int kLoadsFp8 = (kRawCkv + kKpeBytes) / 1024 / 4 + 1;  // 11 per wave per page
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier without the release fence of __syncthreads(): the fence
// would wait for the in-flight prefetch (vmcnt(0)).  LDS reads are drained
// first so a buffer can be refilled safely after the barrier.
__device__ __forceinline__ void barrier_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ void load_lds16(const void *g, LDS_AS void *l) {
    __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
}
__device__ __forceinline__ void load_lds4(const void *g, LDS_AS void *l) {
    __builtin_amdgcn_global_load_lds(g, l, 4, 0, 0);
}

// generic pointer to a __shared__ object -> explicit LDS address-space pointer
__device__ __forceinline__ LDS_AS char *lds_ptr(char *p) { return (LDS_AS char *)(p); }

template <typename T>
__device__ __forceinline__ T lds_read(const LDS_AS char *p) {
    return *reinterpret_cast<const LDS_AS T *>(p);
}

// physical byte offset of logical 16-byte chunk `lc` of latent row `tok`
__device__ __forceinline__ int ckv_off(int tok, int lc) { return tok * kCkvRow + ((lc ^ (tok & 15)) << 4); }
// ... and of RoPE-key row `tok`
__device__ __forceinline__ int kpe_off(int tok, int lc) { return tok * kKpeRow + ((lc ^ (tok & 7)) << 4); }

__device__ __forceinline__ uint32_t pack_lo(uint32_t lo_src, uint32_t hi_src) {
    return __builtin_amdgcn_perm(hi_src, lo_src, 0x05040100u);   // {lo_src.lo16, hi_src.lo16}
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t lo_src, uint32_t hi_src) {
    return __builtin_amdgcn_perm(hi_src, lo_src, 0x07060302u);   // {lo_src.hi16, hi_src.hi16}
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return static_cast<uint32_t>(f32_to_bf16_bits(a)) | (static_cast<uint32_t>(f32_to_bf16_bits(b)) << 16);
}

// ---------------------------------------------------------------------------
// mla_decode_splitkv
// ---------------------------------------------------------------------------
template <bool kFp8>
__global__ __launch_bounds__(kThreads, 1) void decode_mfma_kernel(
    const mla_params_t p, const uint16_t *__restrict__ q_abs, const uint16_t *__restrict__ q_rope,
    const void *__restrict__ c_kv, const uint16_t *__restrict__ k_pe,
    const float *__restrict__ kv_scale, const int32_t *__restrict__ block_table,
    const int32_t *__restrict__ seq_lens, float *__restrict__ o_part, float *__restrict__ lse_part) {
    __shared__ __attribute__((aligned(1024))) char smem[kFp8 ? kSmemFp8 : kSmemBf16];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r16 = lane & 15;
    const int g = lane >> 4;
    const int S = p.num_splits;

    // workgroup -> (item u = b*S + c, row group rg); items are spread over the
    // 8 XCDs, the row groups of one item share an XCD.
    const int n_rg = (p.Sq * p.H) / 64;
    const int xcd = blockIdx.x & 7;
    const int q = blockIdx.x >> 3;
    const int rg = q % n_rg;
    const int64_t u = static_cast<int64_t>(q / n_rg) * 8 + xcd;
    if (u >= static_cast<int64_t>(p.B) * S) return;
    const int b = static_cast<int>(u / S);
    const int c = static_cast<int>(u % S);

    const int seq_len = seq_lens[b];
    const int n_pages_seq = (seq_len + kPage - 1) / kPage;
    const int pg0 = c * p.split_pages;
    const int pg1 = min(pg0 + p.split_pages, n_pages_seq);

    const int row0 = rg * 64 + wave * 16;          // first (s,h) row of this wave
    const int s = row0 / p.H;
    const int h = row0 % p.H + r16;                // this lane's head
    const int64_t qrow = (static_cast<int64_t>(b) * p.Sq + s) * p.H + h;
    const int n_vis = seq_len - p.Sq + 1 + s;      // positions this wave's rows may see
    const int64_t out_row = qrow * S + c;

    if (pg0 >= pg1) {                              // split past the sequence's last page
        if (g == 0) lse_part[out_row] = -INFINITY;
        return;
    }

    // query operands (B of the score product): 16 k-steps of latent, 2 of RoPE
    bf16x8 qreg[18];
#pragma unroll
    for (int ks = 0; ks < 16; ++ks)
        qreg[ks] = *reinterpret_cast<const bf16x8 *>(q_abs + qrow * kDc + ks * 32 + g * 8);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
        qreg[16 + ks] = *reinterpret_cast<const bf16x8 *>(q_rope + qrow * kDr + ks * 32 + g * 8);

    const int32_t *bt = block_table + static_cast<int64_t>(b) * p.max_pages;

    auto issue_page = [&](int pg, int bi) {
        const int64_t phys = bt[pg];
        if constexpr (!kFp8) {
            LDS_AS char *base = lds_ptr(smem) + bi * kBufBf16;
            const char *gc = static_cast<const char *>(c_kv) + phys * kCkvBytes;
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {          // latent rows wave*16 .. +15, one 1 KiB row each
                const int j = wave * 16 + jj;
                load_lds16(gc + j * kCkvRow + ((lane ^ (j & 15)) << 4), base + j * kCkvRow);
            }
            const char *gr = reinterpret_cast<const char *>(k_pe) + phys * kKpeBytes;
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {           // RoPE rows, 8 per instruction
                const int qi = wave * 2 + qq;
                const int r = qi * 8 + (lane >> 3);
                load_lds16(gr + r * kKpeRow + (((lane & 7) ^ (r & 7)) << 4), base + kCkvBytes + qi * 1024);
            }
        } else {
            LDS_AS char *base = lds_ptr(smem) + bi * kRawBuf;
            const char *gc = static_cast<const char *>(c_kv) + phys * kRawCkv;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {           // raw e4m3 rows, linear layout
                const int j = wave * 8 + jj;
                load_lds16(gc + j * 1024 + lane * 16, base + j * 1024);
            }
            const char *gr = reinterpret_cast<const char *>(k_pe) + phys * kKpeBytes;
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
                const int qi = wave * 2 + qq;
                const int r = qi * 8 + (lane >> 3);
                load_lds16(gr + r * kKpeRow + (((lane & 7) ^ (r & 7)) << 4), base + kRawCkv + qi * 1024);
            }
            const float *gs = kv_scale + phys * kPage;
            if (lane < 16) load_lds4(gs + wave * 16 + lane, base + kRawCkv + kKpeBytes + wave * 64);
        }
    };

    float m_run = -INFINITY;   // running max (log2 domain), identical in the 4 lanes of a head
    float l_run = 0.f;         // this lane's share of the running sum of exp2 weights (-> lse)
    float lw_run = 0.f;        // ... of the same weights as rounded for the PV product (-> O)
    f32x4 oacc[4][8];
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int i = 0; i < 8; ++i) oacc[st][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    const float zscale = p.scale * kLog2e;
    const int valid_last = seq_len - (n_pages_seq - 1) * kPage;   // valid slots of the last page

    issue_page(pg0, 0);
    for (int pg = pg0; pg < pg1; ++pg) {
        const int cur = (pg - pg0) & 1;
        if (pg + 1 < pg1) {
            issue_page(pg + 1, cur ^ 1);
            if constexpr (kFp8) wait_vmcnt<kLoadsFp8>(); else wait_vmcnt<kLoadsBf16>();
        } else {
            wait_vmcnt<0>();
        }
        barrier_lds();                                   // page pg is in LDS for every wave

        const bool last_partial = (pg == n_pages_seq - 1) && (valid_last < kPage);
        const LDS_AS char *ckv;
        const LDS_AS char *kpe;
        const LDS_AS float *scl = nullptr;
        if constexpr (!kFp8) {
            ckv = lds_ptr(smem) + cur * kBufBf16;
            kpe = ckv + kCkvBytes;
        } else {
            // convert the raw e4m3 page into the swizzled bf16 layout; slots past the
            // sequence end become zero so whatever they held cannot reach the sums
            const LDS_AS char *raw = lds_ptr(smem) + cur * kRawBuf;
            LDS_AS char *dst = lds_ptr(smem) + 2 * kRawBuf;
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const int unit = threadIdx.x + k * kThreads;   // 8 latents of one token
                const int tok = unit >> 6, lc = unit & 63;
                const u32x2 v = lds_read<u32x2>(raw + tok * 512 + lc * 8);
                u32x4 o;
#pragma unroll
                for (int hw = 0; hw < 2; ++hw) {
                    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(v[hw], false);
                    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(v[hw], true);
                    // e4m3 values are exact in bf16: keep the upper halves
                    o[hw * 2 + 0] = pack_hi(__float_as_uint(lo[0]), __float_as_uint(lo[1]));
                    o[hw * 2 + 1] = pack_hi(__float_as_uint(hi[0]), __float_as_uint(hi[1]));
                }
                if (last_partial && tok >= valid_last) o = u32x4{0u, 0u, 0u, 0u};
                *reinterpret_cast<LDS_AS u32x4 *>(dst + ckv_off(tok, lc)) = o;
            }
            barrier_lds();
            ckv = dst;
            kpe = raw + kRawCkv;
            scl = reinterpret_cast<const LDS_AS float *>(raw + kRawCkv + kKpeBytes);
        }

        // ---- scores S^T[token, head] for the 4 token tiles of the page
        f32x4 sacc[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) sacc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const int tok = tt * 16 + r16;
                const bf16x8 a = lds_read<bf16x8>(ckv + ckv_off(tok, ks * 4 + g));
                sacc[tt] = mfma16(a, qreg[ks], sacc[tt]);
            }
        }
        f32x4 tscale[4];                              // fp8: per-token scale of my 16 tokens
        if constexpr (kFp8) {
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                tscale[tt] = *reinterpret_cast<const LDS_AS f32x4 *>(scl + tt * 16 + g * 4);
                if (last_partial) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (tt * 16 + g * 4 + j >= valid_last) tscale[tt][j] = 0.f;
                }
                sacc[tt] *= tscale[tt];
            }
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const int tok = tt * 16 + r16;
                const bf16x8 a = lds_read<bf16x8>(kpe + kpe_off(tok, ks * 4 + g));
                sacc[tt] = mfma16(a, qreg[16 + ks], sacc[tt]);
            }
        }

        // ---- online softmax (log2 domain); lane holds tokens tt*16 + 4g + j of head r16
        const int tbase = pg * kPage;
        const bool need_mask = tbase + kPage > n_vis;
        float z[4][4];
        float mloc = -INFINITY;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float v = sacc[tt][j] * zscale;
                if (need_mask && tbase + tt * 16 + g * 4 + j >= n_vis) v = -INFINITY;
                z[tt][j] = v;
                mloc = fmaxf(mloc, v);
            }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
        const float m_new = fmaxf(m_run, mloc);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;   // nothing visible yet
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        m_run = m_new;
        // Two sums: the exact weights give the log-sum-exp; the weights exactly as
        // the PV product sees them (after bf16 rounding) normalise O, so every
        // partial is a true convex combination of latent rows.
        float psum = 0.f, pwsum = 0.f;
        uint32_t pk[2][4];                               // P^T operands, bf16 pairs
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            uint32_t pb[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float pv = __builtin_amdgcn_exp2f(z[tt][j] - m_use);
                if constexpr (kFp8) {
                    // weight of the e4m3 code = p * scale; a zero scale (or a masked
                    // slot) still counts p in the sum, its latent being zero
                    const float sc = tscale[tt][j];
                    pb[j] = f32_to_bf16_bits(pv * sc);
                    pwsum += (sc > 0.f) ? bf16_bits_to_f32(static_cast<uint16_t>(pb[j])) / sc : pv;
                } else {
                    pb[j] = f32_to_bf16_bits(pv);
                    pwsum += bf16_bits_to_f32(static_cast<uint16_t>(pb[j]));
                }
                psum += pv;
            }
            pk[tt >> 1][(tt & 1) * 2 + 0] = pb[0] | (pb[1] << 16);
            pk[tt >> 1][(tt & 1) * 2 + 1] = pb[2] | (pb[3] << 16);
        }
        l_run = l_run * alpha + psum;
        lw_run = lw_run * alpha + pwsum;
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int i = 0; i < 8; ++i) oacc[st][i] *= alpha;

        // ---- latent update O^T[latent, head] += V^T[latent, token] P^T[token, head]
        // k-step kk covers tokens 32kk + {4g..4g+3} and 32kk + 16 + {4g..4g+3} for lane group g
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const bf16x8 pb = as_bf16x8(u32x4{pk[kk][0], pk[kk][1], pk[kk][2], pk[kk][3]});
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                u32x4 rows[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int tok = kk * 32 + (e >> 2) * 16 + g * 4 + (e & 3);
                    rows[e] = lds_read<u32x4>(ckv + ckv_off(tok, st * 16 + r16));
                    if constexpr (!kFp8) {
                        if (last_partial && tok >= valid_last) rows[e] = u32x4{0u, 0u, 0u, 0u};
                    }
                }
                // 8x8 bf16 transpose: A_i[e] = rows[e].bf16[i]
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    u32x4 a;
#pragma unroll
                    for (int k2 = 0; k2 < 4; ++k2)
                        a[k2] = (i & 1) ? pack_hi(rows[2 * k2][i >> 1], rows[2 * k2 + 1][i >> 1])
                                        : pack_lo(rows[2 * k2][i >> 1], rows[2 * k2 + 1][i >> 1]);
                    oacc[st][i] = mfma16(as_bf16x8(a), pb, oacc[st][i]);
                }
            }
        }
        barrier_lds();                                   // buffer `cur` may be refilled next
    }

    // ---- epilogue: total sum of the head's 4 lanes, normalised partial + lse
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    float lw_tot = lw_run + __shfl_xor(lw_run, 16);
    lw_tot += __shfl_xor(lw_tot, 32);
    if (l_tot == 0.f) {                                  // no visible position in this split
        if (g == 0) lse_part[out_row] = -INFINITY;
        return;
    }
    const float inv = 1.f / lw_tot;
    float *dst = o_part + out_row * kDc;
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = st * 128 + (g * 4 + j) * 8;
            f32x4 v0, v1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v0[i] = oacc[st][i][j] * inv;
                v1[i] = oacc[st][i + 4][j] * inv;
            }
            *reinterpret_cast<f32x4 *>(dst + col) = v0;
            *reinterpret_cast<f32x4 *>(dst + col + 4) = v1;
        }
    if (g == 0) lse_part[out_row] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
}

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

bool decode_mfma_supported(const mla_params_t &p) {
    if (p.flags & MLA_FLAG_GENERIC) return false;
    if (p.d_c != kDc || p.d_r != kDr || p.page_size != kPage) return false;
    if (p.latent_dtype != MLA_BF16 || p.q_dtype != MLA_BF16 || p.pe_dtype != MLA_BF16) return false;
    if (p.kv_dtype != MLA_BF16 && p.kv_dtype != MLA_FP8_E4M3) return false;
    if (p.H % 16 != 0 || (p.Sq * p.H) % kDecodeRowsPerBlock != 0) return false;
    return true;
}

hipError_t launch_decode_mfma(const mla_params_t &p, const void *q_abs, const void *q_rope,
                              const void *c_kv, const void *k_pe, const float *kv_scale,
                              const int32_t *block_table, const int32_t *seq_lens,
                              float *o_part, float *lse_part, hipStream_t stream) {
    const int64_t items = static_cast<int64_t>(p.B) * p.num_splits;
    const int64_t n_rg = (static_cast<int64_t>(p.Sq) * p.H) / kDecodeRowsPerBlock;
    const int64_t blocks = ((items + 7) / 8) * 8 * n_rg;
    const auto qa = static_cast<const uint16_t *>(q_abs);
    const auto qr = static_cast<const uint16_t *>(q_rope);
    const auto kp = static_cast<const uint16_t *>(k_pe);
    if (p.kv_dtype == MLA_FP8_E4M3)
        hipLaunchKernelGGL(decode_mfma_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream,
                           p, qa, qr, c_kv, kp, kv_scale, block_table, seq_lens, o_part, lse_part);
    else
        hipLaunchKernelGGL(decode_mfma_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream,
                           p, qa, qr, c_kv, kp, kv_scale, block_table, seq_lens, o_part, lse_part);
    return hipGetLastError();
}

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
