// mla_append_kv: write the Sq new tokens of every sequence into the paged
// latent cache, rotating the shared RoPE key (and, if asked, the query's RoPE
// part) at each token's position, gfx950 / CDNA4.
//
// The decode module of "DeepSeek MLA 架构详解" computes the new token's latent
// row and RoPE key, rotates the key at the token's position and appends both to
// the caches before attending; "DeepSeek-MLA-Principle" sec. 3 (why RoPE) gives
// the rotation's relative-position property.  Rotation, rotate-half form, base
// 10000, with half = d_r / 2 and theta_i = pos * 10000^(-i / half), i < half:
//   y[i] = x[i] cos theta_i - x[i + half] sin theta_i
//   y[i + half] = x[i + half] cos theta_i + x[i] sin theta_i
//
// Tokens are numbered tok = b * Sq + s, at position pos = seq_lens[b] - Sq + s,
// cache row block_table[b, pos / 64] * 64 + pos % 64.  One launch, two kinds of
// workgroups (256 threads each):
//   rows     the latent row (8 consecutive values per lane, 16-byte accesses)
//            and the RoPE key: at d_c = 512, d_r = 64 one wave takes 4 tokens
//            (rows_v3), else one wave per token with lane i < half rotating pair i.
//   queries  (only with a query to rotate) one token per workgroup: thread
//            (wave w, lane l) rotates pairs i = l % 32 (+ 32 j) of 1/8 of the
//            heads, so 32 lanes read a head's low (or high) values together.
// Every thread that rotates computes its own angle in fp64 (positions reach
// 10^5 and more, where an fp32 angle would be off by ~1e-2 rad).  One thread
// reads and writes both members of a rotated pair, so the query may be rotated
// in place.  y is formed in fp64, rounded once to fp32 and then to the
// destination format (bf16: round to nearest even).  For an e4m3 cache the wave
// reduces its row's amax; s0 = max(amax, 2^-20) / 448 is a correctly rounded fp32
// division, the scale is the smallest power of two >= s0 (per-token power-of-two
// scales, which the decode kernel widens with one MX-style conversion per two
// codes), r = x / scale, and each r goes to the nearest e4m3 value
// (ties to even, magnitudes above 448 saturating) by an exact power-of-two
// scaling and rint; the row's kv_scale entry gets the scale.
// Bound: HBM (a few KB per token, no reuse).
#include <hip/hip_runtime.h>
#include <math.h>

#include "dtype.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kThreads = 256;

// nearest OCP e4m3 code to r: ties to even, |r| >= 448 (and NaN) -> 448, sign kept
__device__ __forceinline__ uint8_t f32_to_e4m3_sat(float r) {
    const uint32_t sign = (__float_as_uint(r) >> 24) & 0x80u;
    const float a = fabsf(r);
    uint32_t code;
    if (!(a < 448.f)) {
        code = 0x7eu;
    } else if (a < 0.015625f) {                // below the smallest normal: multiples of 2^-9
        code = static_cast<uint32_t>(rintf(a * 512.f));   // 8 is the smallest normal's code
    } else {
        const int e = static_cast<int>((__float_as_uint(a) >> 23) & 0xffu) - 127;   // -6 .. 8
        const uint32_t q = static_cast<uint32_t>(rintf(ldexpf(a, 3 - e)));          // 8 .. 16
        code = (static_cast<uint32_t>(e + 7) << 3) + q - 8u;   // q = 16 carries into the exponent
        if (code > 0x7eu) code = 0x7eu;
    }
    return static_cast<uint8_t>(code | sign);
}

// the token scale: the smallest power of two >= max(amax, 2^-20) / 448 (s0 is a
// positive normal float: a power of two has no mantissa bits; otherwise the next
// binade's power)
__device__ __forceinline__ float pow2_scale(float amax) {
    const uint32_t b = __float_as_uint(__fdiv_rn(fmaxf(amax, 0x1p-20f), 448.f));
    return __uint_as_float((b & 0x7fffffu) ? (b & 0xff800000u) + 0x800000u : b);
}

// (x_lo, x_hi) rotated by the angle with cosine c and sine s, stored as `dt`
__device__ __forceinline__ void rotate_store(void *dst, int dt, int64_t i_lo, int64_t i_hi, float x_lo,
                                             float x_hi, double c, double s) {
    const double y_lo = static_cast<double>(x_lo) * c - static_cast<double>(x_hi) * s;
    const double y_hi = static_cast<double>(x_hi) * c + static_cast<double>(x_lo) * s;
    store_elem(dst, dt, i_lo, static_cast<float>(y_lo));
    store_elem(dst, dt, i_hi, static_cast<float>(y_hi));
}

// cosine and sine of pos * 10000^(-i / half), in fp64
__device__ __forceinline__ void rope_angle(int pos, int i, int half, double &c, double &s) {
    const double freq = exp(-log(10000.0) * static_cast<double>(i) / static_cast<double>(half));
    sincos(static_cast<double>(pos) * freq, &s, &c);
}

struct TokenRow {
    int pos;
    int64_t crow;      // cache row
};

__device__ __forceinline__ TokenRow token_row(const mla_params_t &p, const int32_t *block_table,
                                              const int32_t *seq_lens, int64_t tok) {
    const int b = static_cast<int>(tok / p.Sq);
    const int s = static_cast<int>(tok % p.Sq);
    const int pos = seq_lens[b] - p.Sq + s;
    const int64_t page = block_table[static_cast<int64_t>(b) * p.max_pages + pos / 64];
    return TokenRow{pos, page * 64 + pos % 64};
}

// 8 consecutive values of a row as floats (f32 or bf16 storage)
__device__ __forceinline__ void load8(const void *base, int dt, int64_t i, float *v) {
    if (dt == MLA_F32) {
        const float4 *q = reinterpret_cast<const float4 *>(static_cast<const float *>(base) + i);
        const float4 a = q[0], b = q[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
        const uint4 u = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) + i);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = __uint_as_float(w[k] << 16);
            v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
        }
    }
}

__device__ __forceinline__ void store8(void *base, int dt, int64_t i, const float *v) {
    if (dt == MLA_F32) {
        float4 *q = reinterpret_cast<float4 *>(static_cast<float *>(base) + i);
        q[0] = make_float4(v[0], v[1], v[2], v[3]);
        q[1] = make_float4(v[4], v[5], v[6], v[7]);
    } else {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            w[k] = static_cast<uint32_t>(f32_to_bf16_bits(v[2 * k])) |
                   (static_cast<uint32_t>(f32_to_bf16_bits(v[2 * k + 1])) << 16);
        *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(base) + i) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// e4m3 codes of 8 values, packed little-endian
__device__ __forceinline__ uint2 e4m3x8(const float *v, float scale) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        lo |= static_cast<uint32_t>(f32_to_e4m3_sat(__fdiv_rn(v[k], scale))) << (8 * k);
        hi |= static_cast<uint32_t>(f32_to_e4m3_sat(__fdiv_rn(v[4 + k], scale))) << (8 * k);
    }
    return make_uint2(lo, hi);
}

// Latent row of one token by one wave: 8 consecutive values per lane when `vec`
// (d_c % 8 == 0 and 16-byte aligned tensors), else one value per lane at a time.
__device__ __forceinline__ void latent_row(const mla_params_t &p, bool vec, const void *c_new, void *c_kv,
                                           float *kv_scale, int64_t tok, int64_t crow, int lane) {
    const int64_t src = tok * p.d_c, dst = crow * p.d_c;
    if (p.kv_dtype == MLA_FP8_E4M3) {
        float amax = 0.f;
        if (vec) {
            for (int m = 8 * lane; m < p.d_c; m += 512) {
                float v[8];
                load8(c_new, p.q_dtype, src + m, v);
#pragma unroll
                for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(v[k]));
            }
        } else {
            for (int m = lane; m < p.d_c; m += 64) amax = fmaxf(amax, fabsf(load_elem(c_new, p.q_dtype, src + m)));
        }
        for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
        const float scale = pow2_scale(amax);
        if (vec) {
            for (int m = 8 * lane; m < p.d_c; m += 512) {
                float v[8];
                load8(c_new, p.q_dtype, src + m, v);
                *reinterpret_cast<uint2 *>(static_cast<uint8_t *>(c_kv) + dst + m) = e4m3x8(v, scale);
            }
        } else {
            for (int m = lane; m < p.d_c; m += 64)
                static_cast<uint8_t *>(c_kv)[dst + m] = f32_to_e4m3_sat(__fdiv_rn(load_elem(c_new, p.q_dtype, src + m), scale));
        }
        if (lane == 0) kv_scale[crow] = scale;
    } else if (vec) {
        for (int m = 8 * lane; m < p.d_c; m += 512) {
            float v[8];
            load8(c_new, p.q_dtype, src + m, v);
            store8(c_kv, p.kv_dtype, dst + m, v);
        }
    } else {
        for (int m = lane; m < p.d_c; m += 64) store_elem(c_kv, p.kv_dtype, dst + m, load_elem(c_new, p.q_dtype, src + m));
    }
}

// Rows of 4 consecutive tokens by one wave at d_c = 512, d_r = 64 (16-byte aligned
// tensors): every load is issued before any arithmetic (4 latent chunks of 16
// bytes per lane, 2 RoPE pairs per lane, the 4 cache rows looked up by lanes 0-3),
// the frequency of pair i = l % 32 is
// computed once, and each lane rotates pair i of tokens l / 32 and 2 + l / 32, so
// all 64 lanes take part in the fp64 angle work.
constexpr int kFastTok = 4;

__device__ __forceinline__ void rows_v3(const mla_params_t &p, const void *c_new, const void *kpe_new,
                                        const int32_t *block_table, const int32_t *seq_lens, void *c_kv,
                                        void *k_pe, float *kv_scale, int64_t tok0, int64_t n_tok, int lane) {
    TokenRow tr[kFastTok];
    float v[kFastTok][8];
#pragma unroll
    for (int t = 0; t < kFastTok; ++t) {
        const int64_t tok = min(tok0 + t, n_tok - 1);     // a missing token repeats the last one (not stored)
        load8(c_new, p.q_dtype, tok * 512 + 8 * lane, v[t]);
    }
    {
        // lane t < kFastTok looks up the cache row of token tok0 + t (one pair of
        // dependent loads for the wave instead of one per token), then broadcasts it
        // (measured: bulk append 241 -> 187 us)
        const int64_t tok = min(tok0 + min(lane, kFastTok - 1), n_tok - 1);
        const TokenRow mine = token_row(p, block_table, seq_lens, tok);
        const int lo = static_cast<int>(mine.crow & 0xffffffff), hi = static_cast<int>(mine.crow >> 32);
#pragma unroll
        for (int t = 0; t < kFastTok; ++t) {
            tr[t].pos = __builtin_amdgcn_readlane(mine.pos, t);
            tr[t].crow = (static_cast<int64_t>(__builtin_amdgcn_readlane(hi, t)) << 32) |
                         static_cast<uint32_t>(__builtin_amdgcn_readlane(lo, t));
        }
    }
    const int i = lane & 31;
    float x_lo[2], x_hi[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int64_t tok = min(tok0 + 2 * r + (lane >> 5), n_tok - 1);
        x_lo[r] = load_elem(kpe_new, p.q_dtype, tok * 64 + i);
        x_hi[r] = load_elem(kpe_new, p.q_dtype, tok * 64 + i + 32);
    }
    const double freq = exp(-log(10000.0) * static_cast<double>(i) / 32.0);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int t = 2 * r + (lane >> 5);
        double c, s;
        sincos(static_cast<double>(tr[t].pos) * freq, &s, &c);
        if (tok0 + t < n_tok) {
            const int64_t w0 = tr[t].crow * 64;
            rotate_store(k_pe, p.pe_dtype, w0 + i, w0 + i + 32, x_lo[r], x_hi[r], c, s);
        }
    }
#pragma unroll
    for (int t = 0; t < kFastTok; ++t) {
        if (tok0 + t >= n_tok) break;
        const int64_t dst = tr[t].crow * 512 + 8 * lane;
        if (p.kv_dtype == MLA_FP8_E4M3) {
            float amax = 0.f;
#pragma unroll
            for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(v[t][k]));
            for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
            const float scale = pow2_scale(amax);
            *reinterpret_cast<uint2 *>(static_cast<uint8_t *>(c_kv) + dst) = e4m3x8(v[t], scale);
            if (lane == 0) kv_scale[tr[t].crow] = scale;
        } else {
            store8(c_kv, p.kv_dtype, dst, v[t]);
        }
    }
}

// Workgroups [0, n_row_blocks): rows (4 tokens per workgroup, or 16 on the
// DeepSeek-V3 fast path); then, with a query to rotate, one query workgroup per
// token.
__global__ __launch_bounds__(kThreads) void append_kernel(
    const mla_params_t p, int64_t n_row_blocks, bool vec, bool fast, const void *__restrict__ c_new, const void *__restrict__ kpe_new,
    const void *q_rope_in, void *q_rope_out, const int32_t *__restrict__ block_table,
    const int32_t *__restrict__ seq_lens, void *__restrict__ c_kv, void *__restrict__ k_pe,
    float *__restrict__ kv_scale) {
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int64_t n_tok = static_cast<int64_t>(p.B) * p.Sq;
    const int half = p.d_r / 2;
    if (static_cast<int64_t>(blockIdx.x) < n_row_blocks && fast) {
        const int64_t tok0 = (static_cast<int64_t>(blockIdx.x) * 4 + w) * kFastTok;
        if (tok0 < n_tok)
            rows_v3(p, c_new, kpe_new, block_table, seq_lens, c_kv, k_pe, kv_scale, tok0, n_tok, lane);
        return;
    }
    if (static_cast<int64_t>(blockIdx.x) < n_row_blocks) {
        const int64_t tok = static_cast<int64_t>(blockIdx.x) * 4 + w;
        if (tok >= n_tok) return;
        const TokenRow tr = token_row(p, block_table, seq_lens, tok);
        latent_row(p, vec, c_new, c_kv, kv_scale, tok, tr.crow, lane);
        // RoPE key: lane i rotates pair (i, i + half)
        for (int i = lane; i < half; i += 64) {
            double c, s;
            rope_angle(tr.pos, i, half, c, s);
            const int64_t r0 = tok * p.d_r, w0 = tr.crow * p.d_r;
            rotate_store(k_pe, p.pe_dtype, w0 + i, w0 + i + half, load_elem(kpe_new, p.q_dtype, r0 + i),
                         load_elem(kpe_new, p.q_dtype, r0 + i + half), c, s);
        }
        return;
    }
    // query RoPE parts of one token: thread (w, l) takes pairs i = l % 32 (+ 32 j) of
    // the heads of half-wave 2w + l / 32 (an eighth of them)
    const int64_t tok = static_cast<int64_t>(blockIdx.x) - n_row_blocks;
    if (tok >= n_tok || q_rope_in == nullptr) return;
    const TokenRow tr = token_row(p, block_table, seq_lens, tok);
    const int h_per = (p.H + 7) / 8;
    const int h0 = (2 * w + (lane >> 5)) * h_per;
    const int h1 = min(h0 + h_per, p.H);
    constexpr int kG = 16;                         // heads loaded together
    for (int i = lane & 31; i < half; i += 32) {
        double c, s;
        rope_angle(tr.pos, i, half, c, s);
        for (int hg = h0; hg < h1; hg += kG) {
            float x_lo[kG], x_hi[kG];
#pragma unroll
            for (int k = 0; k < kG; ++k) {
                const int h = min(hg + k, h1 - 1);
                const int64_t q0 = (tok * p.H + h) * p.d_r;
                x_lo[k] = load_elem(q_rope_in, p.q_dtype, q0 + i);
                x_hi[k] = load_elem(q_rope_in, p.q_dtype, q0 + i + half);
            }
#pragma unroll
            for (int k = 0; k < kG; ++k) {
                if (hg + k >= h1) break;
                const int64_t q0 = (tok * p.H + hg + k) * p.d_r;
                rotate_store(q_rope_out, p.q_dtype, q0 + i, q0 + i + half, x_lo[k], x_hi[k], c, s);
            }
        }
    }
}

}  // namespace

hipError_t launch_append(const mla_params_t &p, const void *c_new, const void *kpe_new, const void *q_rope_in,
                         void *q_rope_out, const int32_t *block_table, const int32_t *seq_lens, void *c_kv,
                         void *k_pe, float *kv_scale, hipStream_t stream) {
    const int64_t n_tok = static_cast<int64_t>(p.B) * p.Sq;
    const bool vec = p.d_c % 8 == 0 && reinterpret_cast<uintptr_t>(c_new) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(c_kv) % 16 == 0;
    const bool fast = vec && p.d_c == 512 && p.d_r == 64;
    const int64_t per_block = fast ? 4 * kFastTok : 4;
    const int64_t row_blocks = (n_tok + per_block - 1) / per_block;
    const int64_t blocks = row_blocks + (q_rope_in != nullptr ? n_tok : 0);
    hipLaunchKernelGGL(append_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream, p, row_blocks,
                       vec, fast, c_new, kpe_new, q_rope_in, q_rope_out, block_table, seq_lens, c_kv, k_pe, kv_scale);
    return hipGetLastError();
}

}  // namespace mla
