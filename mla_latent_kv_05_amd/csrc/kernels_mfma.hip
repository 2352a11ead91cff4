// Kernels around the attention at the DeepSeek-V3 head shapes (d_h = 128,
// d_c = 512), gfx950 / CDNA4: the two per-head projections mla_absorb_q
// (q_abs = q_nope . W_UK) and mla_up_v (out = o_latent . W_UV^T), bf16 MFMA
// (v_mfma_f32_16x16x32_bf16), and the split merge mla_combine_lse.  The
// projections are per-head batched GEMMs with a small row count (B*Sq), bound
// by reading the weights: each wave reads a slice of one head's weight matrix
// once, with all its loads in flight together, and applies it to every row.
#include <hip/hip_runtime.h>

#include "gfx950.h"
#include "mla_internal.h"

namespace mla {
namespace {

using namespace gfx;

constexpr int kDc = 512;

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) { return cvt_pk_bf16(a, b); }
// eight bf16 (16 bytes) -> two f32x4 (elements 0..3, 4..7)
__device__ __forceinline__ void unpack_bf16x8(const u32x4 &v, f32x4 &lo, f32x4 &hi) {
    lo = f32x4{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xffff0000u), __uint_as_float(v[1] << 16),
               __uint_as_float(v[1] & 0xffff0000u)};
    hi = f32x4{__uint_as_float(v[2] << 16), __uint_as_float(v[2] & 0xffff0000u), __uint_as_float(v[3] << 16),
               __uint_as_float(v[3] & 0xffff0000u)};
}

// ---------------------------------------------------------------------------
// mla_absorb_q: q_abs[r, h, m] = sum_d q_nope[r, h, d] W_UK[h, d, m]
// One wave per (head, 64-column eighth of d_c): the wave reads its 128 x 64
// slice of W_UK[h] once, all loads in flight together, keeps it in registers
// as MFMA operands and applies it to the rows 64 at a time (1024 waves at the
// DeepSeek-V3 shapes: four per compute unit, so that loads and stores overlap).
// D^T[m, r] = W^T[m, d] . q^T[d, r]: each lane reads 4 columns of 8 W rows
// (8 bytes each) and transposes them in registers into 4 A operands; MFMA i of
// a k-step covers column col0 + i of the 16 lanes' column groups.
// ---------------------------------------------------------------------------
template <int kDh>
__global__ __launch_bounds__(64) void absorb_mfma_kernel(
    const mla_params_t p, const uint16_t *__restrict__ q_nope, const uint16_t *__restrict__ W_UK,
    uint16_t *__restrict__ q_abs) {
    constexpr int kKs = kDh / 32;                 // 32-deep k-steps
    const int lane = threadIdx.x, r16 = lane & 15, g = lane >> 4;
    const int R = p.B * p.Sq;
    // workgroups are dealt to the 8 XCDs in turn (XCD = blockIdx % 8): the eight
    // column slices of a head go to one XCD, whose L2 then serves the head's query
    // rows to all eight after the first load
    const int hpx = (p.H + 7) / 8;                // heads per XCD
    const int k8 = blockIdx.x >> 3;
    const int h = (blockIdx.x & 7) * hpx + (k8 >> 3);
    const int c8 = k8 & 7;                        // 64-column eighth of d_c
    if (h >= p.H) return;
    const int col0 = c8 * 64 + r16 * 4;           // this lane's 4 columns
    const uint16_t *W = W_UK + static_cast<int64_t>(h) * kDh * kDc;
    u32x2 rows[kKs][8];
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            rows[ks][e] = *reinterpret_cast<const u32x2 *>(W + static_cast<int64_t>(ks * 32 + g * 8 + e) * kDc + col0);
    // the first row chunk's query loads go out with the weight loads
    auto load_q = [&](int r0, bf16x8 (&bq)[kKs][4]) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const int r = r0 + rt * 16 + r16;
            const uint16_t *src = q_nope + (static_cast<int64_t>(r < R ? r : 0) * p.H + h) * kDh + g * 8;
#pragma unroll
            for (int ks = 0; ks < kKs; ++ks) {
                u32x4 v = *reinterpret_cast<const u32x4 *>(src + ks * 32);
                if (r >= R) v = u32x4{0u, 0u, 0u, 0u};
                bq[ks][rt] = as_bf16x8(v);
            }
        }
    };
    bf16x8 bq[kKs][4];
    load_q(0, bq);
    // A operand i: column col0 + i, d = ks*32 + g*8 + 0..7
    bf16x8 a[kKs][4];
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            u32x4 v;
#pragma unroll
            for (int k2 = 0; k2 < 4; ++k2)
                v[k2] = (i & 1) ? pack_hi(rows[ks][2 * k2][i >> 1], rows[ks][2 * k2 + 1][i >> 1])
                                : pack_lo(rows[ks][2 * k2][i >> 1], rows[ks][2 * k2 + 1][i >> 1]);
            a[ks][i] = as_bf16x8(v);
        }
    for (int r0 = 0; r0 < R; r0 += 64) {
        f32x4 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) acc[i][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) acc[i][rt] = mfma16(a[ks][i], bq[ks][rt], acc[i][rt]);
        if (r0 + 64 < R) load_q(r0 + 64, bq);          // next chunk, in flight under the stores
        // acc[i][rt][j]: row r0 + rt*16 + r16, column c8*64 + 4*(4g + j) + i
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const int r = r0 + rt * 16 + r16;
            if (r >= R) continue;
            uint16_t *dst = q_abs + (static_cast<int64_t>(r) * p.H + h) * kDc + c8 * 64;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<u32x2 *>(dst + (g * 4 + j) * 4) =
                    u32x2{pack_bf16x2(acc[0][rt][j], acc[1][rt][j]), pack_bf16x2(acc[2][rt][j], acc[3][rt][j])};
        }
    }
}

// ---------------------------------------------------------------------------
// mla_up_v: out[r, h, d] = sum_m o_latent[r, h, m] W_UV[h, d, m]
// One workgroup of 4 waves per (head, 32-row chunk): the chunk's latent rows go
// to LDS once (16-byte chunks XOR-swizzled by row, so that the 16 rows an MFMA
// operand reads at one column hit distinct banks); wave w holds the weight rows
// d = 32w .. 32w+31 in registers (all loads in flight together) and forms
// D^T[d, r] = W_UV[d, m] . o^T[m, r]; both operands are contiguous along m.  The
// two chunks of a head run on the same XCD, so the second weight read hits L2.
// ---------------------------------------------------------------------------
constexpr int kUpRows = 32;                       // rows per workgroup

template <int kDh, bool kOutBf16>
__global__ __launch_bounds__(256) void up_v_mfma_kernel(
    const mla_params_t p, const uint16_t *__restrict__ o_latent, const uint16_t *__restrict__ W_UV,
    void *__restrict__ out) {
    static_assert(kDh == 128, "four waves of 32 output rows");
    __shared__ __attribute__((aligned(16))) char smem[kUpRows * kDc * 2];
    const int lane = threadIdx.x & 63, r16 = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int R = p.B * p.Sq;
    const int n_rc = (R + kUpRows - 1) / kUpRows;
    // workgroup -> (head, row chunk): consecutive chunks of a head are 8 workgroups
    // apart (workgroup i runs on XCD i % 8)
    const int q = blockIdx.x >> 3;
    const int rc = q % n_rc;
    const int h = (q / n_rc) * 8 + (blockIdx.x & 7);
    if (h >= p.H) return;                         // grid rounded up to 8 heads
    const int r0 = rc * kUpRows;
    const int d0 = w * 32;
    const uint32_t sm = lds_addr(smem);
    // this wave's weights: d-tile dt (16 rows), k-step ks (32 columns m)
    const uint16_t *W = W_UV + static_cast<int64_t>(h) * kDh * kDc;
    bf16x8 wa[kDc / 32][2];
#pragma unroll
    for (int ks = 0; ks < kDc / 32; ++ks)
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
            wa[ks][dt] = *reinterpret_cast<const bf16x8 *>(W + static_cast<int64_t>(d0 + dt * 16 + r16) * kDc + ks * 32 + g * 8);
    // the chunk's latent rows into LDS: row rr, 16-byte chunk c at rr*1024 + ((c ^ (rr % 16)) << 4)
#pragma unroll
    for (int k = threadIdx.x; k < kUpRows * 64; k += 256) {
        const int rr = k >> 6, c = k & 63;
        const int r = r0 + rr;
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (r < R) v = *reinterpret_cast<const u32x4 *>(o_latent + (static_cast<int64_t>(r) * p.H + h) * kDc + c * 8);
        lds_store<u32x4>(sm + rr * 1024 + ((c ^ (rr & 15)) << 4), v);
    }
    __syncthreads();
    constexpr int kRt = kUpRows / 16;             // 16-row tiles
    f32x4 acc[2][kRt];                            // [dt][rt]
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int rt = 0; rt < kRt; ++rt) acc[dt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kDc / 32; ++ks)
#pragma unroll
        for (int rt = 0; rt < kRt; ++rt) {
            const int rr = rt * 16 + r16, c = ks * 4 + g;
            const bf16x8 bo = as_bf16x8(lds_load<u32x4>(sm + rr * 1024 + ((c ^ (rr & 15)) << 4)));
#pragma unroll
            for (int dt = 0; dt < 2; ++dt) acc[dt][rt] = mfma16(wa[ks][dt], bo, acc[dt][rt]);
        }
    // acc[dt][rt][j]: row r0 + rt*16 + r16, d = d0 + dt*16 + 4g + j
#pragma unroll
    for (int rt = 0; rt < kRt; ++rt) {
        const int r = r0 + rt * 16 + r16;
        if (r >= R) continue;
        const int64_t base = (static_cast<int64_t>(r) * p.H + h) * kDh + d0;
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
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

// ---------------------------------------------------------------------------
// mla_combine_lse at d_c = 512: one wave per (b,s,h) row, 8 latent columns per
// lane, four rows per workgroup.  The lanes read the row's split log-sum-exps
// 64 at a time; the weighted sum visits only the splits with weight.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// live splits whose partial loads are issued together: the merge kernel (one row
// per wave) and the fused tail's single-row path
constexpr int kMergeBatch = 4;
constexpr int kMergeBatchRow = 8;

template <bool kBf16Out, bool kPartBf16>
__global__ __launch_bounds__(256) void combine_kernel_512(
    const mla_params_t p, const void *__restrict__ o_part, const float *__restrict__ lse_part,
    void *__restrict__ o_latent, float *__restrict__ lse_out) {
    const int lane = threadIdx.x & 63;
    const int64_t rows = static_cast<int64_t>(p.B) * p.Sq * p.H;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= rows) return;
    const int S = p.num_splits;
    const float *l = lse_part + row * S;
    float mx = -INFINITY;
    for (int c0 = 0; c0 < S; c0 += 64) mx = fmaxf(mx, c0 + lane < S ? l[c0 + lane] : -INFINITY);
    mx = wave_max_f(mx);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float sum = 0.f;
    if (mx != -INFINITY) {
        const int64_t op = row * static_cast<int64_t>(S) * kDc + lane * 8;     // element index
        for (int c0 = 0; c0 < S; c0 += 64) {
            const float lc = c0 + lane < S ? l[c0 + lane] : -INFINITY;
            const float w = lc == -INFINITY ? 0.f : __expf(lc - mx);
            sum += w;
            uint64_t live = __builtin_amdgcn_ballot_w64(w != 0.f);
            // up to kMergeBatch live splits per round: their loads first, then the sums
            // in split order (the same order as one split at a time)
            while (live) {
                int kq[kMergeBatch];
                bool vq[kMergeBatch];
#pragma unroll
                for (int q = 0; q < kMergeBatch; ++q) {
                    vq[q] = live != 0;
                    kq[q] = vq[q] ? __builtin_ctzll(live) : 0;
                    live &= live - 1;
                }
                f32x4 v0[kMergeBatch], v1[kMergeBatch];
#pragma unroll
                for (int q = 0; q < kMergeBatch; ++q) {
                    if (!vq[q]) continue;
                    const int64_t e = op + static_cast<int64_t>(c0 + kq[q]) * kDc;
                    if constexpr (kPartBf16) {
                        unpack_bf16x8(*reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(o_part) + e), v0[q],
                                      v1[q]);
                    } else {
                        const f32x4 *src = reinterpret_cast<const f32x4 *>(static_cast<const float *>(o_part) + e);
                        v0[q] = src[0];
                        v1[q] = src[1];
                    }
                }
#pragma unroll
                for (int q = 0; q < kMergeBatch; ++q) {
                    if (!vq[q]) continue;
                    const float wk = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(w), kq[q]));
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        acc[j] = __builtin_fmaf(wk, v0[q][j], acc[j]);
                        acc[4 + j] = __builtin_fmaf(wk, v1[q][j], acc[4 + j]);
                    }
                }
            }
        }
        sum = wave_sum_f(sum);
    }
    const float inv = sum > 0.f ? 1.f / sum : 0.f;
    if constexpr (kBf16Out) {
        u32x4 o;
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = pack_bf16x2(acc[2 * k] * inv, acc[2 * k + 1] * inv);
        *reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(o_latent) + row * kDc + lane * 8) = o;
    } else {
        f32x4 *dst = reinterpret_cast<f32x4 *>(static_cast<float *>(o_latent) + row * kDc + lane * 8);
        dst[0] = f32x4{acc[0], acc[1], acc[2], acc[3]} * inv;
        dst[1] = f32x4{acc[4], acc[5], acc[6], acc[7]} * inv;
    }
    if (lse_out && lane == 0) lse_out[row] = mx == -INFINITY ? -INFINITY : mx + __logf(sum);
}

// ---------------------------------------------------------------------------
// mla_combine_up_v: the split merge and the up-projection in one launch, without
// the merged latent rows leaving the chip.  One workgroup of 8 waves per (head,
// 32-row chunk), as for up_v: wave w first merges rows w, w+8, w+16, w+24 of the chunk
// from their split partials (the arithmetic and order of combine_kernel_512, four
// rows at a time so that their loads overlap), rounds them to bf16 into the
// swizzled LDS layout of up_v, and then forms output dims 16w .. 16w+15 from its
// weight rows, which were loaded before the merge.
// ---------------------------------------------------------------------------
constexpr int kCuRowsPerWave = kUpRows / 8;
constexpr int kFewRows = 8;                      // rows per head up to which the whole workgroup merges one row
constexpr int kFewSplit = 2;                     // ... and workgroups per head then (one per CU at 225 VGPRs)

template <bool kOutBf16, bool kPartBf16, bool kFew>
__global__ __launch_bounds__(512) void combine_up_v_kernel(
    const mla_params_t p, const void *__restrict__ o_part, const float *__restrict__ lse_part,
    const uint16_t *__restrict__ W_UV, void *__restrict__ out, float *__restrict__ lse_out) {
    constexpr int kDh = 128;
    constexpr int kEb = kPartBf16 ? 2 : 4;
    // kFew (at most kFewRows rows per head): partial rows staged in LDS, kSlots at a time
    constexpr int kSlots = kPartBf16 ? 64 : 32;
    constexpr int kStageBytes = kFew ? kSlots * kDc * kEb : 0;
    constexpr int kLatRows = kFew ? 16 : kUpRows;  // merged rows held for the up-projection
    __shared__ __attribute__((aligned(16))) char smem[kLatRows * kDc * 2 + kStageBytes];
    const int lane = threadIdx.x & 63, r16 = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int R = p.B * p.Sq;
    const int n_rc = (R + kUpRows - 1) / kUpRows;
    const int q = blockIdx.x >> 3;
    // kFew: kFewSplit workgroups per head on one XCD (low bits of q), each forming
    // kDh / kFewSplit of the output dims with its first waves (all of them merge the
    // rows: the later ones' partial reads mostly hit the shared L2), so that no
    // compute unit has to pull all of a head's weights through alone
    constexpr int kProjWaves = kFew ? 8 / kFewSplit : 8;
    const int half = kFew ? (q % kFewSplit) : 0;
    const int qh = kFew ? (q / kFewSplit) : q;
    const int rc = kFew ? 0 : qh % n_rc;
    const int h = (kFew ? qh : qh / n_rc) * 8 + (blockIdx.x & 7);
    if (h >= p.H) return;                         // grid rounded up to 8 heads
    const int r0 = rc * kUpRows;
    const bool proj = w < kProjWaves;             // waves that form output dims
    const int d0 = kFew ? half * (kDh / kFewSplit) + w * 16 : w * 16;
    const uint32_t sm = lds_addr(smem);
    const int S = p.num_splits;
    // this wave's weights (16 rows d0 ..), in flight during the merge
    const uint16_t *W = W_UV + static_cast<int64_t>(h) * kDh * kDc;
    bf16x8 wa[kDc / 32];
    auto load_weights = [&] {
        if (!proj) return;
#pragma unroll
        for (int ks = 0; ks < kDc / 32; ++ks)
            wa[ks] = *reinterpret_cast<const bf16x8 *>(W + static_cast<int64_t>(d0 + r16) * kDc + ks * 32 + g * 8);
    };
    if constexpr (kFew) {
        // At most kFewRows rows (r0 = 0), one at a time, with the whole workgroup: every
        // wave finds the row's live splits from its lse values, the waves load the
        // partial rows into LDS together (with at most kSlots splits, all of them, issued
        // with the lse values: one round trip per row), and lane l of wave w then sums
        // latent column 64w + l over the live ones in split order -- per column the
        // arithmetic and order of combine_kernel_512.
        const uint32_t stg = sm + kLatRows * kDc * 2;
        const int col = w * 64 + lane;
        const bool one_round = S <= kSlots;
        auto lse_at = [&](int64_t rowi, int c0) {
            const float v = lse_part[rowi * S + min(c0 + lane, S - 1)];
            return c0 + lane < S ? v : -INFINITY;
        };
        // wave w's staged splits: c0 + cb + 8q + w
        u32x4 x[kSlots / 8][kEb / 2];
        auto load_part = [&](int64_t rowi, int c, int q) {
            const char *src = static_cast<const char *>(o_part) + ((rowi * S + c) * kDc + lane * 8) * kEb;
#pragma unroll
            for (int e = 0; e < kEb / 2; ++e) x[q][e] = reinterpret_cast<const u32x4 *>(src)[e];
        };
        auto stage_part = [&](int k, int q) {
#pragma unroll
            for (int e = 0; e < kEb / 2; ++e) lds_store<u32x4>(stg + (k * kDc + lane * 8) * kEb + 16 * e, x[q][e]);
        };
        // the weighted sum of the staged live splits lv (bit k: slot k, lse lane cb + k),
        // over every slot in order with the dead ones' weight and value replaced by
        // zero (a zero term leaves the sum unchanged, bit for bit), so that the LDS
        // reads need not wait for each other
        auto sum_staged = [&](uint64_t lv, int cb, float wt, float &acc) {
#pragma unroll
            for (int k = 0; k < kSlots; ++k) {
                const bool on = (lv >> k) & 1;
                float v;
                if constexpr (kPartBf16)
                    v = __uint_as_float(static_cast<uint32_t>(lds_load<uint16_t>(stg + (k * kDc + col) * 2)) << 16);
                else
                    v = lds_load<float>(stg + (k * kDc + col) * 4);
                const float wk = on ? __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(wt), (cb + k) & 63)) : 0.f;
                acc = __builtin_fmaf(wk, on ? v : 0.f, acc);
            }
        };
        for (int rr = 0; rr < R; ++rr) {
            const int64_t rowi = static_cast<int64_t>(rr) * p.H + h;
            // loads complete in order: the lse values first, then the partials, then
            // (first row) the weights
            const float l_c0 = lse_at(rowi, 0);
            if (one_round) {
#pragma unroll
                for (int q = 0; q < kSlots / 8; ++q)
                    if (8 * q + w < S) load_part(rowi, 8 * q + w, q);
            }
            if (rr == 0) load_weights();
            float mx = l_c0;
            for (int c0 = 64; c0 < S; c0 += 64) mx = fmaxf(mx, lse_at(rowi, c0));
            mx = wave_max_f(mx);
            float sum = 0.f, acc = 0.f;
            for (int c0 = 0; c0 < S; c0 += 64) {
                const float lc = c0 == 0 ? l_c0 : lse_at(rowi, c0);
                const float wt = (lc == -INFINITY || mx == -INFINITY) ? 0.f : __expf(lc - mx);
                sum += wt;
                const uint64_t live = __builtin_amdgcn_ballot_w64(wt != 0.f);
                if (one_round) {
                    __syncthreads();                   // the previous row's LDS reads are done
#pragma unroll
                    for (int q = 0; q < kSlots / 8; ++q)
                        if (8 * q + w < S) stage_part(8 * q + w, q);
                    __syncthreads();
                    sum_staged(live, 0, wt, acc);
                    continue;
                }
#pragma unroll
                for (int cb = 0; cb < 64; cb += kSlots) {
                    const uint64_t lv = (live >> cb) & (kSlots == 64 ? ~0ull : (1ull << kSlots) - 1);
                    if (!lv) continue;
                    __syncthreads();                   // the previous round's LDS reads are done
#pragma unroll
                    for (int q = 0; q < kSlots / 8; ++q)
                        if ((lv >> (8 * q + w)) & 1) load_part(rowi, c0 + cb + 8 * q + w, q);
#pragma unroll
                    for (int q = 0; q < kSlots / 8; ++q)
                        if ((lv >> (8 * q + w)) & 1) stage_part(8 * q + w, q);
                    __syncthreads();
                    sum_staged(lv, cb, wt, acc);
                }
            }
            const float tot = wave_sum_f(sum);
            const float inv = tot > 0.f ? 1.f / tot : 0.f;
            lds_store<uint16_t>(sm + rr * 1024 + (((col >> 3) ^ (rr & 15)) << 4) + (col & 7) * 2,
                                static_cast<uint16_t>(pack_bf16x2(acc * inv, 0.f) & 0xffffu));
            if (lse_out && half == 0 && w == 0 && lane == 0)
                lse_out[rowi] = mx == -INFINITY ? -INFINITY : mx + __logf(tot);
        }
        for (int rr = R + w; rr < kLatRows; rr += 8) lds_store<u32x4>(sm + rr * 1024 + 16 * lane, u32x4{0u, 0u, 0u, 0u});
    } else {
    // merge rows rr = w + 8i: lane owns latent columns 8 lane .. 8 lane + 7
    int64_t row[kCuRowsPerWave];
    bool ok[kCuRowsPerWave];
    float mx[kCuRowsPerWave], sum[kCuRowsPerWave], acc[kCuRowsPerWave][8];
#pragma unroll
    for (int i = 0; i < kCuRowsPerWave; ++i) {
        const int r = r0 + w + 8 * i;             // strided: few rows still spread over the waves
        ok[i] = r < R;
        row[i] = static_cast<int64_t>(ok[i] ? r : 0) * p.H + h;
        mx[i] = -INFINITY;
        sum[i] = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
    }
    // split lse values, 64 at a time (lane = split); the first 64 are kept for the
    // second pass.  Loads use a clamped index and a select, so all rows' loads issue
    // together.
    auto lse_of = [&](int i, int c0) {
        const float v = lse_part[row[i] * S + min(c0 + lane, S - 1)];
        return ok[i] && c0 + lane < S ? v : -INFINITY;
    };
    // each row's partials as a raw buffer of S * d_c elements
    __amdgpu_buffer_rsrc_t prow[kCuRowsPerWave];
#pragma unroll
    for (int i = 0; i < kCuRowsPerWave; ++i)
        prow[i] = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char *>(static_cast<const char *>(o_part)) + row[i] * S * kDc * kEb, 0,
            ok[i] ? S * kDc * kEb : 0, 0x20000);
    float l0[kCuRowsPerWave];
#pragma unroll
    for (int i = 0; i < kCuRowsPerWave; ++i) l0[i] = lse_part[row[i] * S + min(lane, S - 1)];
#pragma unroll
    for (int i = 0; i < kCuRowsPerWave; ++i) {
        l0[i] = ok[i] && lane < S ? l0[i] : -INFINITY;
        mx[i] = l0[i];
    }
    // the weights, issued after the split lse values (loads complete in order:
    // waiting for the lse values does not wait for the weights)
    load_weights();
    for (int c0 = 64; c0 < S; c0 += 64)
#pragma unroll
        for (int i = 0; i < kCuRowsPerWave; ++i) mx[i] = fmaxf(mx[i], lse_of(i, c0));
#pragma unroll
    for (int i = 0; i < kCuRowsPerWave; ++i) mx[i] = wave_max_f(mx[i]);
    for (int c0 = 0; c0 < S; c0 += 64) {
        float wt[kCuRowsPerWave];
        uint64_t live = 0;
#pragma unroll
        for (int i = 0; i < kCuRowsPerWave; ++i) {
            const float lc = c0 == 0 ? l0[i] : lse_of(i, c0);
            wt[i] = (lc == -INFINITY || mx[i] == -INFINITY) ? 0.f : __expf(lc - mx[i]);
            sum[i] += wt[i];
            live |= __builtin_amdgcn_ballot_w64(wt[i] != 0.f);
        }
        if (R - r0 <= 8) {
            // at most one row per wave (row w of the chunk): up to kMergeBatchRow live
            // splits per round, loads first, then the sums in split order
            while (live) {
                int kq[kMergeBatchRow];
                bool vq[kMergeBatchRow];
#pragma unroll
                for (int qq = 0; qq < kMergeBatchRow; ++qq) {
                    vq[qq] = live != 0;
                    kq[qq] = vq[qq] ? __builtin_ctzll(live) : 0;
                    live &= live - 1;
                }
                f32x4 v0[kMergeBatchRow], v1[kMergeBatchRow];
#pragma unroll
                for (int qq = 0; qq < kMergeBatchRow; ++qq) {
                    const uint32_t off = vq[qq] ? ((c0 + kq[qq]) * kDc + lane * 8) * static_cast<uint32_t>(kEb) : 0x80000000u;
                    if constexpr (kPartBf16) {
                        unpack_bf16x8(__builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(prow[0], off, 0, 0)),
                                      v0[qq], v1[qq]);
                    } else {
                        v0[qq] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(prow[0], off, 0, 0));
                        v1[qq] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(prow[0], off + 16u, 0, 0));
                    }
                }
#pragma unroll
                for (int qq = 0; qq < kMergeBatchRow; ++qq) {
                    if (!vq[qq]) continue;
                    const float wk = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(wt[0]), kq[qq]));
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        acc[0][j] = __builtin_fmaf(wk, v0[qq][j], acc[0][j]);
                        acc[0][4 + j] = __builtin_fmaf(wk, v1[qq][j], acc[0][4 + j]);
                    }
                }
            }
            continue;
        }
        // kSr live splits per round (four with bf16 partials, two with fp32): the
        // loads of all rows and splits first, then the sums in split order; a row
        // without weight on a split (or a missing split) loads past its buffer's
        // end, which returns zeros without a memory access
        constexpr int kSr = kPartBf16 ? 4 : 2;
        while (live) {
            int kq[kSr];
            bool vq[kSr];
#pragma unroll
            for (int qq = 0; qq < kSr; ++qq) {
                vq[qq] = live != 0;
                kq[qq] = vq[qq] ? __builtin_ctzll(live) : 0;
                live &= live - 1;
            }
            float wq[kCuRowsPerWave][kSr];
            u32x4 x0[kCuRowsPerWave][kSr], x1[kCuRowsPerWave][kSr];
#pragma unroll
            for (int i = 0; i < kCuRowsPerWave; ++i)
#pragma unroll
                for (int qq = 0; qq < kSr; ++qq) {
                    wq[i][qq] = vq[qq] ? __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(wt[i]), kq[qq])) : 0.f;
                    const uint32_t off =
                        wq[i][qq] != 0.f ? ((c0 + kq[qq]) * kDc + lane * 8) * static_cast<uint32_t>(kEb) : 0x80000000u;
                    x0[i][qq] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(prow[i], off, 0, 0));
                    if constexpr (!kPartBf16)
                        x1[i][qq] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(prow[i], off + 16u, 0, 0));
                }
#pragma unroll
            for (int i = 0; i < kCuRowsPerWave; ++i)
#pragma unroll
                for (int qq = 0; qq < kSr; ++qq) {
                    if (wq[i][qq] == 0.f) continue;
                    f32x4 v0, v1;
                    if constexpr (kPartBf16) {
                        unpack_bf16x8(x0[i][qq], v0, v1);
                    } else {
                        v0 = __builtin_bit_cast(f32x4, x0[i][qq]);
                        v1 = __builtin_bit_cast(f32x4, x1[i][qq]);
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        acc[i][j] = __builtin_fmaf(wq[i][qq], v0[j], acc[i][j]);
                        acc[i][4 + j] = __builtin_fmaf(wq[i][qq], v1[j], acc[i][4 + j]);
                    }
                }
        }
    }
#pragma unroll
    for (int i = 0; i < kCuRowsPerWave; ++i) {
        const float tot = wave_sum_f(sum[i]);
        const float inv = tot > 0.f ? 1.f / tot : 0.f;
        const int rr = w + 8 * i;
        u32x4 o;
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = pack_bf16x2(acc[i][2 * k] * inv, acc[i][2 * k + 1] * inv);
        lds_store<u32x4>(sm + rr * 1024 + ((lane ^ (rr & 15)) << 4), o);     // zero rows past R
        if (lse_out && ok[i] && lane == 0) lse_out[row[i]] = mx[i] == -INFINITY ? -INFINITY : mx[i] + __logf(tot);
    }
    }
    __syncthreads();

    if (!proj) return;
    // 16-row tiles (kFew: at most kFewRows rows, one tile)
    constexpr int kRt = kFew ? 1 : kUpRows / 16;
    static_assert(!kFew || kFewRows <= 16, "one tile holds the few rows");
    f32x4 acc2[kRt];
#pragma unroll
    for (int rt = 0; rt < kRt; ++rt) acc2[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kDc / 32; ++ks)
#pragma unroll
        for (int rt = 0; rt < kRt; ++rt) {
            const int rr = rt * 16 + r16, c = ks * 4 + g;
            const bf16x8 bo = as_bf16x8(lds_load<u32x4>(sm + rr * 1024 + ((c ^ (rr & 15)) << 4)));
            acc2[rt] = mfma16(wa[ks], bo, acc2[rt]);
        }
    // acc2[rt][j]: row r0 + rt*16 + r16, d = d0 + 4g + j
#pragma unroll
    for (int rt = 0; rt < kRt; ++rt) {
        const int r = r0 + rt * 16 + r16;
        if (r >= R) continue;
        const int64_t base = (static_cast<int64_t>(r) * p.H + h) * kDh + d0 + g * 4;
        if constexpr (kOutBf16) {
            *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(out) + base) =
                u32x2{pack_bf16x2(acc2[rt][0], acc2[rt][1]), pack_bf16x2(acc2[rt][2], acc2[rt][3])};
        } else {
            *reinterpret_cast<f32x4 *>(static_cast<float *>(out) + base) = acc2[rt];
        }
    }
}

}  // namespace

bool combine_up_v_supported(const mla_params_t &p) {
    if (p.flags & MLA_FLAG_GENERIC) return false;
    return p.d_c == kDc && p.d_h == 128 && p.latent_dtype == MLA_BF16 && p.w_dtype == MLA_BF16;
}

hipError_t launch_combine_up_v(const mla_params_t &p, const void *o_part, const float *lse_part, const void *W_UV,
                               void *out, float *lse_out, hipStream_t stream) {
    const int64_t R = static_cast<int64_t>(p.B) * p.Sq;
    const dim3 grid(static_cast<unsigned>((static_cast<int64_t>(p.H) + 7) / 8 * 8 * ((R + kUpRows - 1) / kUpRows)));
    const auto w = static_cast<const uint16_t *>(W_UV);
    const bool ob = p.out_dtype == MLA_BF16, pb = p.part_dtype == MLA_BF16;
    const bool few = R <= kFewRows;
    const dim3 grid_few(static_cast<unsigned>((static_cast<int64_t>(p.H) + 7) / 8 * 8 * kFewSplit));
#define MLA_CUV(OB, PB)                                                                                          \
    if (few)                                                                                                     \
        hipLaunchKernelGGL((combine_up_v_kernel<OB, PB, true>), grid_few, dim3(512), 0, stream, p, o_part,       \
                           lse_part, w, out, lse_out);                                                           \
    else                                                                                                         \
        hipLaunchKernelGGL((combine_up_v_kernel<OB, PB, false>), grid, dim3(512), 0, stream, p, o_part, lse_part, \
                           w, out, lse_out);
    if (ob && pb) {
        MLA_CUV(true, true)
    } else if (ob) {
        MLA_CUV(true, false)
    } else if (pb) {
        MLA_CUV(false, true)
    } else {
        MLA_CUV(false, false)
    }
#undef MLA_CUV
    return hipGetLastError();
}

bool absorb_mfma_supported(const mla_params_t &p) {
    if (p.flags & MLA_FLAG_GENERIC) return false;
    return p.d_c == kDc && p.d_h == 128 && p.q_dtype == MLA_BF16 && p.w_dtype == MLA_BF16 &&
           p.latent_dtype == MLA_BF16;
}

hipError_t launch_absorb_mfma(const mla_params_t &p, const void *q_nope, const void *W_UK,
                              void *q_abs, hipStream_t stream) {
    const int64_t blocks = (static_cast<int64_t>(p.H) + 7) / 8 * 64;
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
    const int64_t blocks = (static_cast<int64_t>(p.H) + 7) / 8 * 8 * ((R + kUpRows - 1) / kUpRows);
    const auto ol = static_cast<const uint16_t *>(o_latent);
    const auto w = static_cast<const uint16_t *>(W_UV);
    if (p.out_dtype == MLA_BF16)
        hipLaunchKernelGGL((up_v_mfma_kernel<128, true>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                           p, ol, w, out);
    else
        hipLaunchKernelGGL((up_v_mfma_kernel<128, false>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                           p, ol, w, out);
    return hipGetLastError();
}

bool combine_fast_supported(const mla_params_t &p) {
    if (p.flags & MLA_FLAG_GENERIC) return false;
    return p.d_c == kDc && (p.latent_dtype == MLA_BF16 || p.latent_dtype == MLA_F32);
}

hipError_t launch_combine_fast(const mla_params_t &p, const void *o_part, const float *lse_part,
                               void *o_latent, float *lse_out, hipStream_t stream) {
    const int64_t rows = static_cast<int64_t>(p.B) * p.Sq * p.H;
    const dim3 grid(static_cast<unsigned>((rows + 3) / 4));
    const bool lb = p.latent_dtype == MLA_BF16, pb = p.part_dtype == MLA_BF16;
    if (lb && pb)
        hipLaunchKernelGGL((combine_kernel_512<true, true>), grid, dim3(256), 0, stream, p, o_part, lse_part, o_latent, lse_out);
    else if (lb)
        hipLaunchKernelGGL((combine_kernel_512<true, false>), grid, dim3(256), 0, stream, p, o_part, lse_part, o_latent, lse_out);
    else if (pb)
        hipLaunchKernelGGL((combine_kernel_512<false, true>), grid, dim3(256), 0, stream, p, o_part, lse_part, o_latent, lse_out);
    else
        hipLaunchKernelGGL((combine_kernel_512<false, false>), grid, dim3(256), 0, stream, p, o_part, lse_part, o_latent, lse_out);
    return hipGetLastError();
}

}  // namespace mla
