// mla_decode_step_persistent: the whole absorbed decode step of a small batch
// (one new token per sequence, DeepSeek-V3 head shapes, bf16) in one launch.
//
// What is computed: the three stages of the absorbed decode ("DeepSeek-MLA-
// Principle" matrix absorption 3): the query is absorbed into latent space,
// q_abs = q_nope W_UK; every head attends to the shared cached latent rows and
// RoPE keys (the MQA form, "MLA Matrix Absorption" sec. 4.1-4.2); the merged
// latent output is up-projected once, out = W_UV o ("DeepSeek MLA 架构详解"
// sec. 3, the decode module).  At a small batch the two weight matrices are most
// of the bytes and each stage is short, so three launches spend much of their
// time filling and draining the GPU; here the stages overlap in one launch.
//
// Work decomposition: workgroups of four waves in three roles, by index:
//   absorb     [0, 2H): item (h, column half): q_abs[b, h, 256 half ..] for every
//              b from W_UK[h][:, 256 half ..] (64 KiB, read once).  Adds 1 to
//              count[0].
//   attention  [2H, 2H + A): item (page, quarter of 32 heads): the 64 positions of
//              a page for 32 heads; scores on v_mfma_f32_16x16x32_bf16, softmax
//              within the page, latent sum on v_mfma_f32_32x32x16_bf16, a
//              normalised bf16 partial and its log-sum-exp.  Copies its page into
//              LDS first, then waits for count[0] = 2H (every q_abs row).  Adds 1
//              to count[1].
//   tail       [2H + A, 4H + A): item (h, row half): copies rows 64 half .. + 63 of
//              W_UV[h] into LDS first, then waits for count[1] = every attention
//              item, merges head h's page partials of every b and multiplies.
// A workgroup waits only for workgroups of lower index, and workgroups are
// dispatched in index order, so the grid drains whatever number of them is
// resident at once (no co-residency is assumed).  Two fit on a compute unit (LDS
// and registers are sized for it), so on an idle GPU the absorb and attention
// workgroups start together, the pages stream in under the absorb, and the tail
// workgroups take the compute units the absorb frees and stream W_UV in under the
// attention.  The workgroup that finishes last sets the counters back to zero
// (count[2] counts finished workgroups).  Every wait is bounded: a wait that gives
// up sets MLA_DEVERR_SYNC and goes on.
//
// Cross-workgroup data (q_abs, the partials and their lse values) is written with
// device-scope stores and published with one agent-scope release per workgroup;
// readers acquire at agent scope, which orders it across the compute dies'
// separate L2 caches.  Loads of cross-workgroup data are vector loads (never the
// scalar cache, which the acquire does not invalidate).
#include <hip/hip_runtime.h>
#include <math.h>

#include "decode_common.h"

namespace mla {
namespace {

using namespace gfx;

constexpr int kThreads = 256;
constexpr int kDh = 128;
constexpr int kMaxB = 8;
// attention workgroup: the page (latent rows of 1 KiB, then RoPE rows of 128
// bytes), the weights P[32 heads][64 tokens] in bf16 (rows of 144 bytes), the
// softmax maxima and sums of the four waves
constexpr int kRopeOff = dec::kPage * dec::kCkvRow;   // 65536
constexpr int kPOff = kRopeOff + dec::kPage * dec::kKpeRow;   // 73728
constexpr int kPRow = 144;
constexpr int kStatOff = kPOff + 32 * kPRow;          // 78336
constexpr int kAttnSmem = kStatOff + 768;             // 79104
// tail workgroup: 64 rows of W_UV[h] (1 KiB each), then o_b (512 fp32)
constexpr int kObufOff = 64 * dec::kCkvRow;           // 65536
constexpr int kTailSmem = kObufOff + 2048;            // 67584
constexpr int kSmem = kAttnSmem > kTailSmem ? kAttnSmem : kTailSmem;
constexpr uint32_t kSpinLimit = 1u << 22;             // bound of a counter wait (never reached)
static_assert(2 * kSmem <= 160 * 1024, "two workgroups per compute unit");

struct Args {
    mla_params_t p;
    const uint16_t *q_nope, *q_rope, *c_kv, *k_pe, *W_UK, *W_UV;
    const int32_t *block_table, *seq_lens;
    void *out;
    float *lse_out;
    uint32_t *count;           // [0] absorb items done, [1] attention items done, [2] workgroups finished
    uint16_t *q_abs;           // [B][H][512] bf16
    float *lse_part;           // [B][H][max_pages]
    uint16_t *o_part;          // [B][H][max_pages][512] bf16
    int n_att_wg;              // attention workgroups launched (a bound on the items)
};

// Swizzle of the 16-byte chunks of latent row r: logical chunk c sits at position
// c ^ lat_swz(r), a bijection of r % 16 onto 0..15.  The 16 rows a 16-lane group
// reads for one K operand then fill the 16 bank groups once, and so do the four
// rows x two chunks of a group's transposing V read (their swizzles 2j + const).
__device__ __forceinline__ int lat_swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1) | (r & 8); }
// ... of RoPE row r (rows of 8 chunks)
__device__ __forceinline__ int rope_swz(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ uint16_t bf16_bits(float x) { return static_cast<uint16_t>(cvt_pk_bf16(x, 0.f) & 0xffffu); }

// One global -> LDS copy of up to 1 KiB: lane i's 16 bytes from src + voff_i land
// at LDS address lds + 16 i.  src and lds are wave-uniform.
__device__ __forceinline__ void dma_1k(const void *src, uint32_t bytes, uint32_t lds, uint32_t voff) {
    const u32x4 r{dec::lo32(src), dec::hi32(src) & 0xffffu, static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(bytes)),
                  0x20000u};
    asm volatile("s_mov_b32 m0, %[l]\n\ts_nop 0\n\tbuffer_load_dwordx4 %[v], %[r], %[so] offen lds"
                 :: [r] "s"(r), [l] "s"(__builtin_amdgcn_readfirstlane(lds)), [so] "s"(0u), [v] "v"(voff)
                 : "memory", "m0");
}

// Stores of data that other workgroups read carry device scope (relaxed
// agent-scope atomic stores: sc1): they are written through this die's L2, so the
// L2 holds no dirty lines of theirs and the release below, which writes back the
// whole L2, has little to write.
__device__ __forceinline__ void store_dev_u16(uint16_t *p, uint16_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev_f32(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev_x4(void *p, const u32x4 &v) {
    uint64_t *q = static_cast<uint64_t *>(p);
    __hip_atomic_store(q, (static_cast<uint64_t>(v[1]) << 32) | v[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + 1, (static_cast<uint64_t>(v[3]) << 32) | v[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// a device-scope vector load of a value other workgroups wrote
__device__ __forceinline__ float load_dev_f32(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Publish: each wave waits for its own stores (and any copy in flight), the
// workgroup meets, then one lane adds 1 to the counter with an agent-scope release.
__device__ __forceinline__ void signal(uint32_t *c) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until *c >= target: one lane polls, then acquires at agent scope (the
// invalidation is of the caches the whole workgroup reads through), and the
// workgroup meets.  The poll is a compare-and-swap that never matches (no count
// reaches 0xffffffff): an atomic is performed where the die L2s are coherent,
// while a plain load of the counter may be served by this die's L2 from a line
// that another die's increments have made stale (measured: such polls saw the
// final count up to 20 us late).
__device__ __forceinline__ void wait_count(uint32_t *c, uint32_t target) {
    if (threadIdx.x == 0) {
        uint32_t spin = 0;
        for (; spin < kSpinLimit; ++spin) {
            uint32_t cur = 0xffffffffu;
            __hip_atomic_compare_exchange_strong(c, &cur, 0xffffffffu, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
            if (cur >= target) break;
            __builtin_amdgcn_s_sleep(1);
        }
        if (spin == kSpinLimit) raise_error(MLA_DEVERR_SYNC);   // gave up: flagged, never a hang
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// absorb item (h, ch): q_abs[r, h, m] = sum_d q_nope[r, h, d] W_UK[h, d, m] for
// m in [256 ch, 256 ch + 256), every query row r < R (R <= 8).  Wave w takes
// columns 256 ch + 64 w .. + 63; lane l sums rows 16 (l / 8) .. + 15 of the 8
// columns 8 (l % 8) .. + 7 in fp32, then the eight row groups are added across
// lanes (l ^ 32, l ^ 16, l ^ 8).  store(index, value) writes one q_abs element.
// ---------------------------------------------------------------------------
template <typename Store>
__device__ __forceinline__ void absorb_rows(const mla_params_t &p, const uint16_t *__restrict__ q_nope,
                                            const uint16_t *__restrict__ W_UK, int R, int item, Store &&store) {
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = item >> 1, ch = item & 1;
    const int rg = lane >> 3;
    const int col = 256 * ch + 64 * w + 8 * (lane & 7);
    const uint16_t *wk = W_UK + (static_cast<int64_t>(h) * kDh + 16 * rg) * dec::kDc + col;
    u32x4 wv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) wv[r] = *reinterpret_cast<const u32x4 *>(wk + r * dec::kDc);
    const bool b5 = lane & 32, b4 = lane & 16, b3 = lane & 8;
    const int e_out = 4 * b5 + 2 * b4 + b3;           // the column this lane ends with
#pragma unroll
    for (int b = 0; b < kMaxB; ++b) {
        if (b >= R) break;
        const uint16_t *qn = q_nope + (static_cast<int64_t>(b) * p.H + h) * kDh + 16 * rg;
        const u32x4 q0 = *reinterpret_cast<const u32x4 *>(qn), q1 = *reinterpret_cast<const u32x4 *>(qn + 8);
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const uint32_t qw = r < 8 ? q0[r >> 1] : q1[(r - 8) >> 1];
            const float qv = (r & 1) ? bf_hi(qw) : bf_lo(qw);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] = fmaf(qv, bf_lo(wv[r][e]), acc[2 * e]);
                acc[2 * e + 1] = fmaf(qv, bf_hi(wv[r][e]), acc[2 * e + 1]);
            }
        }
        // add the row groups: each step keeps half of the columns and takes the
        // partner's sum of them
        float v4[4], v2[2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float send = b5 ? acc[i] : acc[i + 4];
            v4[i] = (b5 ? acc[i + 4] : acc[i]) + __shfl_xor(send, 32);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const float send = b4 ? v4[i] : v4[i + 2];
            v2[i] = (b4 ? v4[i + 2] : v4[i]) + __shfl_xor(send, 16);
        }
        const float send = b3 ? v2[0] : v2[1];
        const float v1 = (b3 ? v2[1] : v2[0]) + __shfl_xor(send, 8);
        store((static_cast<int64_t>(b) * p.H + h) * dec::kDc + col + e_out, v1);
    }
}

// ---------------------------------------------------------------------------
// attention item: page j of sequence b (positions 64 j .. 64 j + n_valid - 1),
// heads 32 hq .. 32 hq + 31
// ---------------------------------------------------------------------------
// copy the page into LDS: wave w copies latent rows 16 w .. 16 w + 15 (one 1 KiB
// instruction each) and RoPE rows 16 w .. 16 w + 15 (two instructions of 8 rows);
// latent rows past the sequence's end are zeroed instead, so that the latent sum
// meets only finite values (their weights are zero; a cache slot past the end may
// hold anything)
struct PageSrc {
    const uint16_t *c_kv, *k_pe;
    const int32_t *block_table;
};

__device__ __forceinline__ void issue_page(const mla_params_t &p, const PageSrc &a, uint32_t sm, int b, int j,
                                           int n_valid) {
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    n_valid = __builtin_amdgcn_readfirstlane(n_valid);
    const int64_t page = __builtin_amdgcn_readfirstlane(
        checked_page(p, a.block_table[static_cast<int64_t>(b) * p.max_pages + j]));
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = 16 * w + i;
        if (r < n_valid)
            dma_1k(a.c_kv + (page * dec::kPage + r) * dec::kDc, 1024u, sm + r * dec::kCkvRow,
                   static_cast<uint32_t>(lane ^ lat_swz(r)) << 4);
        else
            lds_store<u32x4>(sm + r * dec::kCkvRow + 16 * lane, u32x4{0u, 0u, 0u, 0u});
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int r0 = 16 * w + 8 * q;
        const int rows = min(max(n_valid - r0, 0), 8);
        if (rows > 0) {
            const int rr = r0 + (lane >> 3);
            dma_1k(a.k_pe + (page * dec::kPage + r0) * dec::kDr, static_cast<uint32_t>(rows) * dec::kKpeRow,
                   sm + kRopeOff + r0 * dec::kKpeRow,
                   static_cast<uint32_t>((lane >> 3) * dec::kKpeRow + (((lane & 7) ^ rope_swz(rr)) << 4)));
        }
    }
}

// Where an attention item reads its query and writes its partial: split j of
// head h of sequence b is row (b H + h) * split_stride + j of o_part (512 bf16)
// and of lse_part.  kDev: device-scope stores (read by other workgroups of the
// same launch), else plain stores.
struct AttnIo {
    const uint16_t *q_abs, *q_rope;
    uint16_t *o_part;
    float *lse_part;
    int split_stride;
};

// Scores of one half of the 576 dims for one head block (16 heads) over the page's
// 64 tokens: S^T[token, head] = K Q^T in four 16-token blocks, 9 steps of 32 dims
// (step ks = 9 KH + s: latent chunk group ks < 16, RoPE ks - 16).  The wave loads
// only its half of the query rows, then waits for them and the page copy.
template <int KH>
__device__ __forceinline__ void score_half(const AttnIo &a, uint32_t sm, int64_t qrow, int lane, f32x4 (&sc)[4]) {
    const int l16 = lane & 15, q4 = lane >> 4;            // 16x16 operand lane: row / column l16, k-group q4
    // query operand (B): head row qrow, dims 32 ks + 8 q4 .. + 7
    bf16x8 qreg[9];
    {
        const uint16_t *qa = a.q_abs + qrow * dec::kDc + 8 * q4;
        const uint16_t *qr = a.q_rope + qrow * dec::kDr + 8 * q4;
#pragma unroll
        for (int s = 0; s < 9; ++s) {
            const int ks = 9 * KH + s;
            qreg[s] = *reinterpret_cast<const bf16x8 *>(ks < 16 ? qa + 32 * ks : qr + 32 * (ks - 16));
        }
    }
    wait_vmcnt<0>();                                      // the query rows and the page
    __syncthreads();
    // K operand (A): token row 16 tb + l16, logical chunk 4 ks + q4 (latent, ks = 4 m +
    // k0: at kx[k0] + 256 m) or 4 (ks - 16) + q4 (RoPE); the swizzles depend on l16 only
    const int sw = lat_swz(l16);
    uint32_t kx[4], kp[2];
#pragma unroll
    for (int k0 = 0; k0 < 4; ++k0) kx[k0] = sm + l16 * dec::kCkvRow + (((4 * k0 + q4) ^ sw) << 4);
#pragma unroll
    for (int k = 0; k < 2; ++k) kp[k] = sm + kRopeOff + l16 * dec::kKpeRow + (((4 * k + q4) ^ rope_swz(l16)) << 4);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) sc[tb] = f32x4{};
#pragma unroll
    for (int s = 0; s < 9; ++s) {
        const int ks = 9 * KH + s;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            const uint32_t addr = ks < 16 ? kx[ks & 3] + 256 * (ks >> 2) + tb * 16 * dec::kCkvRow
                                          : kp[ks - 16] + tb * 16 * dec::kKpeRow;
            sc[tb] = mfma16(as_bf16x8(dec::ld128(addr)), qreg[s], sc[tb]);
        }
    }
}

// q_abs is readable; the page copy may still be in flight.
//   scores   wave w: head block hb = w % 2 (16 heads) and half kh = w / 2 of the
//            576 dims (kh = 0: latent 0 .. 287; kh = 1: latent 288 .. 511 and the
//            RoPE key), all 64 tokens (score_half): each query element is loaded
//            by one wave of the workgroup
//   softmax  the kh = 1 wave of a head block passes its partial scores through LDS
//            (the RoPE rows, dead once every score step is done); the kh = 0 wave
//            adds them, takes the maximum, weights and sums over the page and writes
//            the bf16 weights to LDS as P[head][token]
//   latent   wave w: latent columns 128 w .. 128 w + 127 of all 32 heads:
//            O^T += V^T P^T, V^T by transposing reads, tokens in natural order
template <bool kDev>
__device__ __forceinline__ void attend_quarter(const mla_params_t &p, const AttnIo &a, uint32_t sm, int b, int j,
                                               int n_valid, int hq) {
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hb = w & 1, kh = w >> 1;
    const int l16 = lane & 15, q4 = lane >> 4;
    const int h0 = 32 * hq;                               // first head of the quarter
    const int64_t qrow = static_cast<int64_t>(b) * p.H + h0 + 16 * hb + l16;
    f32x4 sc[4];
    if (kh == 0) score_half<0>(a, sm, qrow, lane, sc);
    else score_half<1>(a, sm, qrow, lane, sc);
    // lane holds head 16 hb + l16, tokens 16 tb + 4 q4 + i (partial over its half)
    __syncthreads();                                      // every score step is done: the RoPE rows are free
    const uint32_t xs = sm + kRopeOff + hb * 4096 + 16 * lane;
    if (kh == 1) {
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) lds_store<f32x4>(xs + 1024 * tb, sc[tb]);
    }
    __syncthreads();
    // stats: [512, 768) the sums of the rounded weights per head of the quarter
    const uint32_t st = sm + kStatOff;
    float m = -INFINITY, ls = 0.f;
    if (kh == 0) {
        const float zs = p.scale * dec::kLog2e;
        float z[4][4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            const f32x4 o1 = lds_load<f32x4>(xs + 1024 * tb);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = 16 * tb + 4 * q4 + i;
                z[tb][i] = tok < n_valid ? (sc[tb][i] + o1[i]) * zs : -INFINITY;
                m = fmaxf(m, z[tb][i]);
            }
        }
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));                  // finite: position 0 of the page is valid
        float lw = 0.f;
        uint32_t pk[4][2];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
                const float p0 = exp2f(z[tb][i] - m), p1 = exp2f(z[tb][i + 1] - m);
                ls += p0 + p1;
                const uint32_t u = cvt_pk_bf16(p0, p1);
                lw += bf_lo(u) + bf_hi(u);
                pk[tb][i >> 1] = u;
            }
#pragma unroll
        for (int o = 16; o <= 32; o <<= 1) {
            ls += __shfl_xor(ls, o);
            lw += __shfl_xor(lw, o);
        }
        if (q4 == 0) lds_store<float>(st + 512 + 4 * (16 * hb + l16), lw);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
            lds_store<u32x2>(sm + kPOff + (16 * hb + l16) * kPRow + 2 * (16 * tb + 4 * q4), u32x2{pk[tb][0], pk[tb][1]});
    }
    __syncthreads();
    // latent sum: lane (n, g): head n of the quarter, k = 8 g + e <-> token 16 kk + 8 g
    // + e.  Transposing read hl of lane (q16, i16): row 16 kk + 8 g + 4 hl + i16 / 4,
    // latent columns 128 w + 32 cb + 16 (q16 % 2) + 4 (i16 % 4) .. + 3 (logical chunk
    // 16 w + 4 cb + c2); the row's swizzle does not depend on kk.
    const int n = lane & 31, g = lane >> 5;
    const int i16 = lane & 15, q16 = lane >> 4;
    const int c2 = 2 * (q16 & 1) + ((i16 & 3) >> 1);
    uint32_t vb[2][4];
#pragma unroll
    for (int hl = 0; hl < 2; ++hl) {
        const int row = 8 * g + 4 * hl + (i16 >> 2);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
            vb[hl][cb] = sm + row * dec::kCkvRow + (((16 * w + 4 * cb + c2) ^ lat_swz(row)) << 4) + 8 * (i16 & 1);
    }
    const uint32_t pb = sm + kPOff + n * kPRow + 16 * g;
    f32x16 o[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 bw = as_bf16x8(dec::ld128(pb + 32 * kk));
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const v4i16 lo = dec::ld_tr16(vb[0][cb] + 16 * kk * dec::kCkvRow);
            const v4i16 hi = dec::ld_tr16(vb[1][cb] + 16 * kk * dec::kCkvRow);
            const bf16x8 av = __builtin_bit_cast(bf16x8, v8i16{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
            o[cb] = mfma32(av, bw, o[cb]);
        }
    }
    // head n's total of its rounded weights
    const int hbn = n >> 4, ln = n & 15;
    const float lw_tot = lds_load<float>(st + 512 + 4 * (16 * hbn + ln));
    const float inv = 1.f / lw_tot;
    const int64_t prow = (static_cast<int64_t>(b) * p.H + h0 + n) * a.split_stride + j;
    uint16_t *dst = a.o_part + prow * dec::kDc + 128 * w;
    // lane (n, g) holds latent columns 32 cb + 8 k + 4 g .. + 3 (k = 0..3); lanes n and
    // n ^ 32 exchange halves so that each stores 16 contiguous bytes
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
            uint32_t u0[2], u1[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                u0[t] = cvt_pk_bf16(o[cb][8 * pr + 2 * t] * inv, o[cb][8 * pr + 2 * t + 1] * inv);
                u1[t] = cvt_pk_bf16(o[cb][8 * pr + 4 + 2 * t] * inv, o[cb][8 * pr + 4 + 2 * t + 1] * inv);
            }
            u32x4 v;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const auto r = __builtin_amdgcn_permlane32_swap(u0[t], u1[t], false, false);
                v[t] = r[0];
                v[2 + t] = r[1];
            }
            if constexpr (kDev) store_dev_x4(dst + 32 * cb + 16 * pr + 8 * g, v);
            else *reinterpret_cast<u32x4 *>(dst + 32 * cb + 16 * pr + 8 * g) = v;
        }
    if (kh == 0 && q4 == 0) {                                  // head 16 w + l16: maximum and sum
        const float l_tot = ls;
        const int64_t prow_h = (static_cast<int64_t>(b) * p.H + h0 + 16 * w + l16) * a.split_stride + j;
        const float lse = (m + __log2f(l_tot)) * dec::kLn2;
        if constexpr (kDev) store_dev_f32(a.lse_part + prow_h, lse);
        else a.lse_part[prow_h] = lse;
    }
}

// ---------------------------------------------------------------------------
// tail item (h, rh): out[b, h, 64 rh + i] = sum_m W_UV[h, 64 rh + i, m] o_b[m],
// o_b = the merge of head h's page partials of sequence b
// ---------------------------------------------------------------------------
__device__ __forceinline__ void issue_wuv(const Args &a, uint32_t sm, int item) {
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = item >> 1, rh = item & 1;
    const uint16_t *src = a.W_UV + (static_cast<int64_t>(h) * kDh + 64 * rh) * dec::kDc;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = 16 * w + i;
        dma_1k(src + r * dec::kDc, 1024u, sm + r * dec::kCkvRow, static_cast<uint32_t>(lane) << 4);
    }
}

__device__ __forceinline__ void tail_item(const Args &a, uint32_t sm, int item, const int (&pages)[kMaxB]) {
    const mla_params_t &p = a.p;
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), t = threadIdx.x;
    const int h = item >> 1, rh = item & 1;
    // this wave's 16 rows of the slice, lane l's 16 bytes of each
    u32x4 wv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) wv[r] = lds_load<u32x4>(sm + (16 * w + r) * dec::kCkvRow + 16 * lane);
    const uint32_t obuf = sm + kObufOff;
#pragma unroll
    for (int b = 0; b < kMaxB; ++b) {
        if (b >= p.B) break;
        const int np = pages[b];
        const int64_t prow0 = (static_cast<int64_t>(b) * p.H + h) * p.max_pages;
        // the page partials' weights exp(lse_j - max) / total: every wave finds the
        // same maximum and total, every thread recomputes the weights it uses
        float mx = -INFINITY;
        for (int j0 = 0; j0 < np; j0 += 64)
            mx = fmaxf(mx, j0 + lane < np ? load_dev_f32(a.lse_part + prow0 + j0 + lane) : -INFINITY);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        float tot = 0.f;
        for (int j0 = 0; j0 < np; j0 += 64)
            tot += j0 + lane < np ? __expf(load_dev_f32(a.lse_part + prow0 + j0 + lane) - mx) : 0.f;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) tot += __shfl_xor(tot, o);
        // o_b[2 t], o_b[2 t + 1]: 32 pages' loads in flight at a time
        float o0 = 0.f, o1 = 0.f;
        const uint32_t *src = reinterpret_cast<const uint32_t *>(a.o_part + prow0 * dec::kDc) + t;
        for (int j0 = 0; j0 < np; j0 += 32) {
            uint32_t v[32];
            float l[32];
#pragma unroll
            for (int u = 0; u < 32; ++u) {
                v[u] = j0 + u < np ? src[(j0 + u) * (dec::kDc / 2)] : 0u;
                l[u] = j0 + u < np ? load_dev_f32(a.lse_part + prow0 + j0 + u) : -INFINITY;
            }
#pragma unroll
            for (int u = 0; u < 32; ++u) {
                const float wj = __expf(l[u] - mx);
                o0 = fmaf(wj, bf_lo(v[u]), o0);
                o1 = fmaf(wj, bf_hi(v[u]), o1);
            }
        }
        const float inv = np > 0 ? 1.f / tot : 0.f;
        lds_store<f32x2>(obuf + 8 * t, f32x2{o0 * inv, o1 * inv});
        __syncthreads();
        // rows 16 w + r: lane l's 8 columns 8 l .. 8 l + 7, then the 64 lanes added
        const f32x4 oa = lds_load<f32x4>(obuf + 32 * lane), ob = lds_load<f32x4>(obuf + 32 * lane + 16);
        float v16[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float s = 0.f;
            s = fmaf(bf_lo(wv[r][0]), oa[0], s);
            s = fmaf(bf_hi(wv[r][0]), oa[1], s);
            s = fmaf(bf_lo(wv[r][1]), oa[2], s);
            s = fmaf(bf_hi(wv[r][1]), oa[3], s);
            s = fmaf(bf_lo(wv[r][2]), ob[0], s);
            s = fmaf(bf_hi(wv[r][2]), ob[1], s);
            s = fmaf(bf_lo(wv[r][3]), ob[2], s);
            s = fmaf(bf_hi(wv[r][3]), ob[3], s);
            v16[r] = s;
        }
        const bool b5 = lane & 32, b4 = lane & 16, b3 = lane & 8, b2 = lane & 4;
        float v8[8], v4[4], v2[2];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float send = b5 ? v16[i] : v16[i + 8];
            v8[i] = (b5 ? v16[i + 8] : v16[i]) + __shfl_xor(send, 32);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float send = b4 ? v8[i] : v8[i + 4];
            v4[i] = (b4 ? v8[i + 4] : v8[i]) + __shfl_xor(send, 16);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const float send = b3 ? v4[i] : v4[i + 2];
            v2[i] = (b3 ? v4[i + 2] : v4[i]) + __shfl_xor(send, 8);
        }
        float v1 = (b2 ? v2[1] : v2[0]) + __shfl_xor(b2 ? v2[0] : v2[1], 4);
        v1 += __shfl_xor(v1, 2);
        v1 += __shfl_xor(v1, 1);
        const int row = 64 * rh + 16 * w + 8 * b5 + 4 * b4 + 2 * b3 + b2;
        if ((lane & 3) == 0) {
            const int64_t oi = (static_cast<int64_t>(b) * p.H + h) * kDh + row;
            if (p.out_dtype == MLA_BF16) static_cast<uint16_t *>(a.out)[oi] = bf16_bits(v1);
            else static_cast<float *>(a.out)[oi] = v1;
        }
        if (a.lse_out && rh == 0 && t == 0)
            a.lse_out[static_cast<int64_t>(b) * p.H + h] = np > 0 ? mx + __logf(tot) : -INFINITY;
        __syncthreads();                      // o_b is rewritten for the next b
    }
}

__global__ __launch_bounds__(kThreads, 2) void step_persistent_kernel(const Args a) {
    __shared__ __attribute__((aligned(1024))) char smem[kSmem];
    const mla_params_t &p = a.p;
    const int wg = blockIdx.x;
    const uint32_t sm = lds_addr(smem);

    // pages of each sequence
    int pages[kMaxB];
    int n_att = 0;
#pragma unroll
    for (int b = 0; b < kMaxB; ++b) {
        pages[b] = b < p.B ? seq_pages(p, a.seq_lens[b]) : 0;
        n_att += pages[b];
    }
    const int n_q = p.H / 32, n_absorb = 2 * p.H;
    const int n_items = n_att * n_q;

    if (wg < n_absorb) {
        absorb_rows(p, a.q_nope, a.W_UK, p.B, wg,
                    [&](int64_t i, float v) { store_dev_u16(a.q_abs + i, bf16_bits(v)); });
        signal(&a.count[0]);
    } else if (wg < n_absorb + a.n_att_wg) {
        // attention item i: page (i % 8) + 8 ((i / 8) / n_q), pages counted in sequence
        // order, quarter (i / 8) % n_q: the quarters of a page run on one compute die
        // (workgroup k goes to die k % 8, and 2H is a multiple of 8) and share the page
        // through its L2
        const int i = wg - n_absorb;
        const int r = i >> 3, hq = r % n_q;
        const int pi = (i & 7) + 8 * (r / n_q);
        if (pi < n_att) {
            int base = 0, b = 0, j = 0;
#pragma unroll
            for (int bb = 0; bb < kMaxB; ++bb) {
                if (pi >= base && pi < base + pages[bb]) {
                    b = bb;
                    j = pi - base;
                }
                base += pages[bb];
            }
            const int nv = min(dec::kPage, a.seq_lens[b] - dec::kPage * j);
            issue_page(p, PageSrc{a.c_kv, a.k_pe, a.block_table}, sm, b, j, nv);
            wait_count(&a.count[0], static_cast<uint32_t>(n_absorb));
            attend_quarter<true>(p, AttnIo{a.q_abs, a.q_rope, a.o_part, a.lse_part, p.max_pages}, sm, b, j, nv, hq);
            signal(&a.count[1]);
        }
    } else {
        const int u = wg - n_absorb - a.n_att_wg;
        issue_wuv(a, sm, u);
        wait_count(&a.count[1], static_cast<uint32_t>(n_items));
        wait_vmcnt<0>();
        __syncthreads();
        tail_item(a, sm, u, pages);
    }

    // the last workgroup to finish sets the counters back to zero
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t done = __hip_atomic_fetch_add(&a.count[2], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (done == gridDim.x - 1u) {
            __hip_atomic_store(&a.count[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&a.count[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&a.count[2], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ---------------------------------------------------------------------------
// mla_absorb_q for at most 8 query rows (B * Sq <= 8) at the DeepSeek-V3 head
// shapes: the absorb item above, one workgroup per (head, column half), every
// weight load in flight at once; fp32 sums, one rounding to latent_dtype.
// ---------------------------------------------------------------------------
template <bool kOutBf16>
__global__ __launch_bounds__(kThreads) void absorb_rows_kernel(const mla_params_t p, const uint16_t *__restrict__ q_nope,
                                                               const uint16_t *__restrict__ W_UK, void *__restrict__ q_abs) {
    absorb_rows(p, q_nope, W_UK, p.B * p.Sq, blockIdx.x, [&](int64_t i, float v) {
        if constexpr (kOutBf16) static_cast<uint16_t *>(q_abs)[i] = bf16_bits(v);
        else static_cast<float *>(q_abs)[i] = v;
    });
}

// ---------------------------------------------------------------------------
// mla_decode_splitkv with fixed splits of one page each (the plan of a small batch
// of single new tokens): one workgroup per (sequence, page, quarter of 32 heads),
// the attention item above with plain stores.  A split past the sequence's pages
// gets lse = -inf.  The quarters of a page are consecutive-by-8 workgroups (one
// compute die) and share the page through its L2.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads, 2) void decode_page_kernel(const mla_params_t p, const uint16_t *__restrict__ q_abs,
                                                                   const uint16_t *__restrict__ q_rope,
                                                                   const uint16_t *__restrict__ c_kv,
                                                                   const uint16_t *__restrict__ k_pe,
                                                                   const int32_t *__restrict__ block_table,
                                                                   const int32_t *__restrict__ seq_lens,
                                                                   uint16_t *__restrict__ o_part,
                                                                   float *__restrict__ lse_part) {
    __shared__ __attribute__((aligned(1024))) char smem[kAttnSmem];
    const int n_q = p.H / 32;
    const int S = p.num_splits;
    const int per_seq = (S + 7) / 8 * 8 * n_q;        // workgroups of one sequence
    const int b = blockIdx.x / per_seq, i = blockIdx.x % per_seq;
    const int r = i >> 3, hq = r % n_q;
    const int j = (i & 7) + 8 * (r / n_q);            // the split (= page) of this workgroup
    if (j >= S) return;
    const int len = seq_lens[b];
    const int pages = seq_pages(p, len);
    if (j == 0 && hq == 0 && threadIdx.x == 0 && pages > S) raise_error(MLA_DEVERR_SPLITS);
    if (j >= pages) {                                  // no page: an empty split
        if (threadIdx.x < 32)
            lse_part[(static_cast<int64_t>(b) * p.H + 32 * hq + threadIdx.x) * S + j] = -INFINITY;
        return;
    }
    const uint32_t sm = lds_addr(smem);
    const int nv = min(dec::kPage, len - dec::kPage * j);
    issue_page(p, PageSrc{c_kv, k_pe, block_table}, sm, b, j, nv);
    attend_quarter<false>(p, AttnIo{q_abs, q_rope, o_part, lse_part, S}, sm, b, j, nv, hq);
}

}  // namespace

bool absorb_rows_supported(const mla_params_t &p) {
    return static_cast<int64_t>(p.B) * p.Sq <= kMaxB && p.d_h == kDh && p.d_c == dec::kDc && p.q_dtype == MLA_BF16 &&
           p.w_dtype == MLA_BF16 && (p.latent_dtype == MLA_BF16 || p.latent_dtype == MLA_F32);
}

hipError_t launch_absorb_rows(const mla_params_t &p, const void *q_nope, const void *W_UK, void *q_abs,
                              hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(2 * p.H));
    const auto qn = static_cast<const uint16_t *>(q_nope);
    const auto wk = static_cast<const uint16_t *>(W_UK);
    if (p.latent_dtype == MLA_BF16)
        hipLaunchKernelGGL((absorb_rows_kernel<true>), grid, dim3(kThreads), 0, stream, p, qn, wk, q_abs);
    else
        hipLaunchKernelGGL((absorb_rows_kernel<false>), grid, dim3(kThreads), 0, stream, p, qn, wk, q_abs);
    return hipGetLastError();
}

bool decode_page_supported(const mla_params_t &p) {
    return p.Sq == 1 && p.H >= 32 && p.H % 32 == 0 && p.d_c == dec::kDc && p.d_r == dec::kDr &&
           p.page_size == dec::kPage && p.q_dtype == MLA_BF16 && p.kv_dtype == MLA_BF16 && p.pe_dtype == MLA_BF16 &&
           p.latent_dtype == MLA_BF16 && p.part_dtype == MLA_BF16;
}

hipError_t launch_decode_page(const mla_params_t &p, const void *q_abs, const void *q_rope, const void *c_kv,
                              const void *k_pe, const int32_t *block_table, const int32_t *seq_lens, void *o_part,
                              float *lse_part, hipStream_t stream) {
    const int64_t per_seq = (static_cast<int64_t>(p.num_splits) + 7) / 8 * 8 * (p.H / 32);
    hipLaunchKernelGGL(decode_page_kernel, dim3(static_cast<unsigned>(p.B * per_seq)), dim3(kThreads), 0, stream, p,
                       static_cast<const uint16_t *>(q_abs), static_cast<const uint16_t *>(q_rope),
                       static_cast<const uint16_t *>(c_kv), static_cast<const uint16_t *>(k_pe), block_table, seq_lens,
                       static_cast<uint16_t *>(o_part), lse_part);
    return hipGetLastError();
}

bool step_persistent_supported(const mla_params_t &p) {
    return p.Sq == 1 && p.B >= 1 && p.B <= kMaxB && p.H >= 32 && p.H <= 128 && p.H % 32 == 0 && p.d_h == kDh &&
           p.d_c == dec::kDc && p.d_r == dec::kDr && p.page_size == dec::kPage && p.q_dtype == MLA_BF16 &&
           p.w_dtype == MLA_BF16 && p.kv_dtype == MLA_BF16 && p.pe_dtype == MLA_BF16 && p.latent_dtype == MLA_BF16 &&
           (p.out_dtype == MLA_BF16 || p.out_dtype == MLA_F32) && p.max_pages <= kStepPersistentMaxPages;
}

StepPersistentLayout step_persistent_layout(const mla_params_t &p) {
    auto align256 = [](int64_t x) { return (x + 255) / 256 * 256; };
    const int64_t rows = static_cast<int64_t>(p.B) * p.H;
    StepPersistentLayout l{};
    l.q_abs = 256;
    l.lse_part = l.q_abs + align256(rows * dec::kDc * 2);
    l.o_part = l.lse_part + align256(rows * p.max_pages * 4);
    l.bytes = l.o_part + align256(rows * p.max_pages * dec::kDc * 2);
    return l;
}

hipError_t launch_step_persistent(const mla_params_t &p, const void *q_nope, const void *q_rope, const void *c_kv,
                                  const void *k_pe, const int32_t *block_table, const int32_t *seq_lens,
                                  const void *W_UK, const void *W_UV, void *out, float *lse_out, char *ws,
                                  hipStream_t stream) {
    const StepPersistentLayout l = step_persistent_layout(p);
    // attention workgroups: every page a batch of B sequences of max_pages pages can
    // have, in groups of 8 pages, times the head quarters
    const int64_t pages_max = static_cast<int64_t>(p.B) * p.max_pages;
    const int n_att_wg = static_cast<int>((pages_max + 7) / 8 * 8 * (p.H / 32));
    Args a{p,
           static_cast<const uint16_t *>(q_nope), static_cast<const uint16_t *>(q_rope),
           static_cast<const uint16_t *>(c_kv), static_cast<const uint16_t *>(k_pe),
           static_cast<const uint16_t *>(W_UK), static_cast<const uint16_t *>(W_UV),
           block_table, seq_lens, out, lse_out,
           reinterpret_cast<uint32_t *>(ws), reinterpret_cast<uint16_t *>(ws + l.q_abs),
           reinterpret_cast<float *>(ws + l.lse_part), reinterpret_cast<uint16_t *>(ws + l.o_part), n_att_wg};
    const dim3 grid(static_cast<unsigned>(2 * p.H + n_att_wg + 2 * p.H));
    hipLaunchKernelGGL(step_persistent_kernel, grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t take_errors_step_persistent(uint32_t *bits) { return take_unit_errors(bits); }

}  // namespace mla
