// mla_decode_splitkv on bf16 MFMA for a bf16 latent cache: eight waves per
// workgroup with split roles, gfx950 / CDNA4.
//
// What is computed is the same as in kernels_decode.hip ("MLA Matrix
// Absorption" sec. 4.1-4.2; "DeepSeek-MLA-Principle" sec. 2 and matrix
// absorption 3)): for a tile of 32 cache tokens the scores of 32 heads are a
// dense [32 x 576] x [576 x 32] product (latent + RoPE key), the latent update a
// dense [512 x 32] x [32 x 32] product, both on v_mfma_f32_32x32x16_bf16.
//
// Work decomposition (64 query rows = two head blocks hb of 32 per workgroup)
//   score waves 0..3   wave s = (hb, kh): the scores of head block hb over half kh
//                      of the 576 dims (kh = 0: latent 0..287; kh = 1: latent
//                      288..511 and the RoPE key), query operands in 72 VGPRs.
//                      The two fp32 partials of a head block meet in LDS (a flag
//                      per wave, no workgroup barrier); wave (hb, kh) then owns
//                      heads 16kh .. 16kh+15 of the block: it sums both partials,
//                      keeps their running maximum and sums, and publishes the
//                      bf16 weights P and the rescale factors.
//   latent waves 4..7  wave v accumulates latent columns 128v .. 128v+127 for all
//                      64 heads (8 accumulator tiles, 128 registers), so every
//                      transposed V read feeds two MFMAs, and issues the tile
//                      copies (global -> LDS, 3-stage ring).
//   Wave w and wave w+4 run on the same SIMD: each SIMD holds one score wave and
//   one latent wave, whose MFMAs (18 and 16 per tile) share its matrix core while
//   the score wave's LDS traffic and softmax arithmetic issue under the latent
//   wave's MFMAs.
// Pipeline: iteration i (one workgroup barrier at its end) computes the scores and
// weights of tile i+1 in the score waves and the latent update of tile i in the
// latent waves; once its V reads of tile i are in, latent wave v refills its
// column block of that stage with tile i+3 (copies run two to three tiles ahead).
// Layouts of the latent / RoPE rows in a stage and the token order are those of
// decode_common.h.  The output is the normalised partial O_c (fp32) and its
// log-sum-exp per row, as for every other decode kernel.
#include <hip/hip_runtime.h>
#include <math.h>

#include "decode_common.h"

namespace mla {
namespace {

using namespace gfx;
using namespace dec;

constexpr int kThreads = 512;
constexpr int kRows = kDecodeRowsPerBlock;              // 64 query rows: two head blocks of 32
// LDS: the latent rows of tile t in stage t % 3, column-blocked: physical chunk p of
// row r at (p / 16) * 8192 + r * 256 + (p % 16) * 16, so that latent wave v reads (as
// V), and refills, block v alone; the RoPE rows of tile t in slot t % 3
constexpr int kStages = 3;
constexpr int kBlock = kTile * 256;                     // one column block (16 chunks) of a tile
constexpr int kOffRope = kStages * kTileCkv;            // 98304
constexpr int kPartWave = 64 * 16 * 4;                  // one score wave's partial scores (fp32)
constexpr int kOffPart = kOffRope + kStages * kTileKpe; // 110592
constexpr int kOffP = kOffPart + 4 * kPartWave;         // 126976
constexpr int kPBuf = 2 * 2 * 2 * 32 * 16;              // bf16 weights: [hb][k-step][g2][head] x 16 B
constexpr int kOffAlpha = kOffP + 2 * kPBuf;            // 135168: rescale factors [buf][head][hb]
constexpr int kABuf = 64 * 4;
constexpr int kOffFin = kOffAlpha + 2 * kABuf;          // 135680: 1 / sum of weights [head][hb]
constexpr int kOffFlag = kOffFin + kABuf;               // 135936: partial-ready counters of the score waves
constexpr int kSmem = kOffFlag + 64;                    // 136000
constexpr int kSSteps = 18;                             // score k-steps per score wave per tile
constexpr int kKAhead = 8;                              // K reads in flight
constexpr int kLoads = 9;                               // copy instructions per latent wave per tile
constexpr uint32_t kSpinLimit = 1u << 22;               // bound of the flag wait (never reached)
static_assert(kSmem <= 160 * 1024, "LDS budget");
static_assert(kRows == 64, "two head blocks of 32");

// K operand of score step k for half KH of the 576 dims:
//   KH = 0: latent chunk 2k + g2 (dims 16k ..), k < 18
//   KH = 1: latent chunk 2k + 36 + g2 (dims 288 + 16k ..) for k < 14, then RoPE chunk 2(k-14) + g2
// kb[u]: tile base + lane offset of chunk column u; kp[r]: RoPE chunk r
template <int KH, int k>
__device__ __forceinline__ u32x4 k_operand(const uint32_t *kb, const uint32_t *kp) {
    if constexpr (KH == 1 && k >= 14) {
        return ld128(kp[k - 14]);
    } else {
        constexpr int chunk = 2 * k + 36 * KH;
        return ld128(kb[(chunk >> 1) & 7] + (chunk >> 4) * kBlock);
    }
}

// Partial scores S^T[token, head] of one tile over half KH of the dims: one MFMA
// chain of 18 steps with the K operands read kKAhead steps ahead (the compiler's
// counted waits keep them in flight).
template <int KH>
__device__ __forceinline__ f32x16 score_tile(const uint32_t *kb, const uint32_t *kp, const bf16x8 *qreg) {
    u32x4 a[kSSteps];
    f32x16 acc;
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = 0.f;
#define MLA_KREAD(k) a[k] = k_operand<KH, k>(kb, kp);
    MLA_KREAD(0) MLA_KREAD(1) MLA_KREAD(2) MLA_KREAD(3) MLA_KREAD(4) MLA_KREAD(5) MLA_KREAD(6) MLA_KREAD(7)
    pin();
#define MLA_KSTEP(k)                                                                   \
    {                                                                                  \
        acc = mfma32(as_bf16x8(a[k]), qreg[k], acc);                                   \
        if constexpr ((k) + kKAhead < kSSteps) MLA_KREAD((k) + kKAhead)                \
        pin();                                                                         \
    }
    MLA_KSTEP(0) MLA_KSTEP(1) MLA_KSTEP(2) MLA_KSTEP(3) MLA_KSTEP(4) MLA_KSTEP(5)
    MLA_KSTEP(6) MLA_KSTEP(7) MLA_KSTEP(8) MLA_KSTEP(9) MLA_KSTEP(10) MLA_KSTEP(11)
    MLA_KSTEP(12) MLA_KSTEP(13) MLA_KSTEP(14) MLA_KSTEP(15) MLA_KSTEP(16) MLA_KSTEP(17)
#undef MLA_KSTEP
#undef MLA_KREAD
    return acc;
}


__device__ __forceinline__ bf16x8 tr_op(const v4i16 &lo, const v4i16 &hi) {
    return __builtin_bit_cast(bf16x8, v8i16{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
}

// reductions over the 4 lanes of a DPP quad
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xf, 0xf, false));
}
__device__ __forceinline__ float max4(float v) {
    v = fmaxf(v, dpp<0xB1>(v));          // quad_perm [1,0,3,2]
    return fmaxf(v, dpp<0x4E>(v));       // quad_perm [2,3,0,1]
}
__device__ __forceinline__ float sum4(float v) {
    v += dpp<0xB1>(v);
    return v + dpp<0x4E>(v);
}

// Values of one segment shared by both roles (all wave-uniform).
struct SegInfo {
    int t_begin;       // first token (page aligned)
    int n_tiles;       // >= 1
    int last_valid;    // rows of the last tile inside the sequence
    int64_t row_wg;    // first query row of the workgroup
    int seq_len;
};

__device__ __forceinline__ SegInfo seg_info(const mla_params_t &p, const Segment &seg, int rg, int seq_len) {
    SegInfo si;
    si.seq_len = __builtin_amdgcn_readfirstlane(seq_len);
    si.t_begin = __builtin_amdgcn_readfirstlane(seg.pa * kPage);
    const int t_end = __builtin_amdgcn_readfirstlane(min(seg.pb * kPage, si.seq_len));
    si.n_tiles = __builtin_amdgcn_readfirstlane((t_end - si.t_begin + kTile - 1) / kTile);
    si.last_valid = __builtin_amdgcn_readfirstlane(t_end - (si.t_begin + (si.n_tiles - 1) * kTile));
    si.row_wg = static_cast<int64_t>(seg.b) * p.Sq * p.H + rg * kRows;
    return si;
}

// ---------------------------------------------------------------------------
// Score wave (hb, KH) for one segment.  Barriers: two in the prologue, one per
// tile after the first, one before the epilogue's output (matching latent_role).
// `gen` counts the tiles this wave has scored since the kernel started; the
// partial-ready flag of a wave holds the count of its last published partial.
// ---------------------------------------------------------------------------
template <int KH>
__device__ __forceinline__ void score_role(char *smem, const mla_params_t &p, const uint16_t *__restrict__ q_abs,
                                           const uint16_t *__restrict__ q_rope, const Segment &seg, const SegInfo &si,
                                           int rg, float *__restrict__ lse_part, uint32_t &gen) {
    // lane-dependent offsets are computed per segment: opaque to loop-invariant
    // code motion, so that neither role's offsets stay live across the other's code
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const int s = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // 0..3
    const int hb = s >> 1;
    const int t32 = lane & 31, g2 = lane >> 5;
    const int S = p.num_splits;
    const int s_q = (rg * kRows + 32 * hb) / p.H;                       // query position of the block
    const int n_vis = __builtin_amdgcn_readfirstlane(si.seq_len - p.Sq + 1 + s_q);
    wait_vmcnt<0>();

    // query operands (B of the score product): this wave's half of the 576 dims
    const int64_t qrow = si.row_wg + 32 * hb + t32;
    bf16x8 qreg[kSSteps];
#pragma unroll
    for (int ks = 0; ks < kSSteps; ++ks) {
        const uint16_t *src;
        if (KH == 0) src = q_abs + qrow * kDc + ks * 16 + g2 * 8;
        else if (ks < 14) src = q_abs + qrow * kDc + 288 + ks * 16 + g2 * 8;
        else src = q_rope + qrow * kDr + (ks - 14) * 16 + g2 * 8;
        qreg[ks] = *reinterpret_cast<const bf16x8 *>(src);
    }
#pragma unroll
    for (int ks = 0; ks < kSSteps; ++ks) asm volatile("" : "+v"(qreg[ks]));

    const uint32_t sm = lds_addr(smem);
    // K operand: row perm_tok(t32); in each column block, chunk column u holds logical
    // chunk (2u + g2) ^ (row % 16)
    const int krow = perm_tok(t32);
    uint32_t kx[8], kpx[4];
#pragma unroll
    for (int u = 0; u < 8; ++u) kx[u] = krow * 256 + ((((2 * u + g2) & 15) ^ (krow & 15)) << 4);
#pragma unroll
    for (int r = 0; r < 4; ++r) kpx[r] = krow * kKpeRow + (((2 * r + g2) ^ ((krow >> 1) & 7)) << 4);
    // partial scores: chunk q of lane l (D rows 8q + 4(l/32) ..) in slot
    // q*64 + (l & ~15) + ((l + 4(l/32) + 8(q/2)) % 16) of the wave's area
    auto pslot = [](int l, int q) -> uint32_t {
        return (q * 64 + (l & ~15) + ((l + 4 * (l >> 5) + 8 * (q >> 1)) & 15)) * 16;
    };
    const uint32_t pw_base = sm + kOffPart + s * kPartWave;
    // owner view: head n = 16 KH + lane/4 of the block; m = lane % 4 -> k-step kq = m/2,
    // B-operand lane half g = m % 2; its 8 weights are D rows 16kq + 8(e/4) + 4g + e%4
    const int n = 16 * KH + (lane >> 2);
    const int kq = (lane & 3) >> 1, gq = lane & 1;
    const uint32_t pr_addr = sm + kOffPart + 2 * hb * kPartWave + pslot(n + 32 * gq, 2 * kq);   // + 1024: chunk 2kq+1
    const int pgrp = kq * 2 + gq;
    const uint32_t pw_off = hb * 2048 + (pgrp * 32 + (n ^ (4 * pgrp))) * 16;
    const uint32_t aw_off = (n * 2 + hb) * 4;
    int rtok[8];                                        // tile position of weight e
#pragma unroll
    for (int e = 0; e < 8; ++e) rtok[e] = perm_tok(16 * kq + 8 * (e >> 2) + 4 * gq + (e & 3));

    float m_ref = -INFINITY;   // reference maximum (log2 domain), equal in the head's 4 lanes
    float l_run = 0.f;         // this lane's share of the sum of exp2 weights (-> lse)
    float lw_run = 0.f;        // ... of the weights as rounded to bf16 for the product (-> O)
    const float zscale = p.scale * kLog2e;
    const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);

    // scores, exchange and softmax of tile t
    auto score_and_weights = [&](int t) {
        gen += 1;
        uint32_t kb[8], kp[4];
        const uint32_t lst = sm + (t % kStages) * kTileCkv;
        const uint32_t rst = sm + kOffRope + (t % kStages) * kTileKpe;
#pragma unroll
        for (int u = 0; u < 8; ++u) kb[u] = lst + kx[u];
#pragma unroll
        for (int r = 0; r < 4; ++r) kp[r] = rst + kpx[r];
        const f32x16 acc = score_tile<KH>(kb, kp, qreg);
        // publish the partial: plain stores (the compiler keeps the wait states an MFMA
        // result needs before a store reads it), then the flag once they completed
#pragma unroll
        for (int q = 0; q < 4; ++q)
            lds_store<f32x4>(pw_base + pslot(lane, q), f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]});
        asm volatile("s_waitcnt lgkmcnt(0)\n\tds_write_b32 %0, %1" ::"v"(sm + kOffFlag + s * 4), "v"(gen) : "memory");
        // wait for the other half's partial of this tile (bounded: the partner always
        // publishes, the bound only keeps a wave from spinning forever)
        uint32_t spin = 0;
        for (; spin < kSpinLimit; ++spin) {
            uint32_t f;
            asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(f) : "v"(sm + kOffFlag + (s ^ 1) * 4) : "memory");
            if (__builtin_amdgcn_readfirstlane(f) == gen) break;
            __builtin_amdgcn_s_sleep(1);
        }
        if (spin == kSpinLimit && lane == 0) raise_error(MLA_DEVERR_SYNC);   // gave up: flagged, never a hang
        // both partials of the owned heads, in the owner layout
        const u32x4 x0 = ld128(pr_addr), x1 = ld128(pr_addr + 1024);
        const u32x4 y0 = ld128(pr_addr + kPartWave), y1 = ld128(pr_addr + kPartWave + 1024);
        float sc[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sc[e] = __uint_as_float(x0[e]) + __uint_as_float(y0[e]);
            sc[4 + e] = __uint_as_float(x1[e]) + __uint_as_float(y1[e]);
        }
        const int tbase = si.t_begin + t * kTile;
        if (tbase + kTile > n_vis) {                   // causal bound or sequence end inside the tile
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (tbase + rtok[e] >= n_vis) sc[e] = -INFINITY;
        }
        float mloc = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
        mloc = max4(mloc) * zscale;                    // zscale > 0: max commutes with it
        // raise the reference only when a weight would exceed 2^kRescaleSlack
        const bool raise = mloc > m_ref + kRescaleSlack;
        const float alpha = raise ? __builtin_amdgcn_exp2f(m_ref - mloc) : 1.f;   // 0 when m_ref = -inf
        l_run *= alpha;
        lw_run *= alpha;
        m_ref = raise ? mloc : m_ref;
        const uint32_t buf = (t & 1);
        if ((lane & 3) == 0) lds_store<float>(sm + kOffAlpha + buf * kABuf + aw_off, alpha);
        const float m_use = m_ref == -INFINITY ? 0.f : m_ref;   // nothing visible yet: weights 0
        float pe[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pe[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e], zscale, -m_use));
        l_run += ((pe[0] + pe[1]) + (pe[2] + pe[3])) + ((pe[4] + pe[5]) + (pe[6] + pe[7]));
        // (a scalar array: with a u32x4 element here the compiler has fed the same
        // pair to all four dot products)
        uint32_t pk[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            pk[h] = cvt_pk_bf16(pe[2 * h], pe[2 * h + 1]);
            // the sum of the weights exactly as the latent product sees them
            lw_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[h]), ones, lw_run, false);
        }
        lds_store<u32x4>(sm + kOffP + buf * kPBuf + pw_off, u32x4{pk[0], pk[1], pk[2], pk[3]});
    };

    // prologue: tile 0 lands (barrier), scores of tile 0, its weights visible (barrier)
    barrier_lds();
    score_and_weights(0);
    barrier_lds();
    for (int i = 0; i + 1 < si.n_tiles; ++i) {
        score_and_weights(i + 1);
        barrier_lds();
    }
    // epilogue: per head 1 / sum of weights for the latent waves, lse
    const float l_tot = sum4(l_run);
    const float lw_tot = sum4(lw_run);
    if ((lane & 3) == 0) {
        const bool empty = l_tot == 0.f;               // no visible position in this split
        lds_store<float>(sm + kOffFin + aw_off, empty ? 0.f : 1.f / lw_tot);
        lse_part[(si.row_wg + 32 * hb + n) * S + seg.c] = empty ? -INFINITY : (m_ref + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
    barrier_lds();
}

// ---------------------------------------------------------------------------
// Latent wave v for one segment: copies, latent update of columns 128v .., output.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void latent_role(char *smem, const mla_params_t &p, const char *__restrict__ c_kv,
                                            const uint16_t *__restrict__ k_pe, const int32_t *__restrict__ bt,
                                            const Segment &seg, const SegInfo &si, void *__restrict__ o_part) {
    int lane = threadIdx.x & 63;                       // opaque, as in score_role
    asm volatile("" : "+v"(lane));
    const int v = __builtin_amdgcn_readfirstlane((threadIdx.x >> 6) - 4);   // 0..3
    const int t32 = lane & 31, g2 = lane >> 5;
    const int S = p.num_splits;
    const int n_tiles = si.n_tiles;
    // earlier stores and copies (a previous segment's) complete before the counted
    // waits on this segment's copies begin
    wait_vmcnt<0>();
    const int n_pages = __builtin_amdgcn_readfirstlane(seg.pb - seg.pa);
    const int32_t *seg_bt = bt + __builtin_amdgcn_readfirstlane(seg.pa);
    int pl_base = 0;                                   // pages pl_base .. pl_base+63 of the segment, one per lane
    int plist = checked_page(p, seg_bt[min(lane, n_pages - 1)]);
    asm volatile("" : "+v"(plist));

    const uint32_t sm = lds_addr(smem);
    // copies of block v: instruction m covers rows 4m .. 4m+3 (16 lanes per row); lane l
    // lands in physical chunk 16v + l % 16 of row 4m + l / 16 and fetches logical chunk
    // 16v + ((l % 16) ^ (row % 16)); the global lane offset depends on m % 4 only
    uint32_t vo[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int r = 4 * m + (lane >> 4);
        vo[m] = (lane >> 4) * kCkvRow + (16 * v + ((lane & 15) ^ (r & 15))) * 16;
    }
    // RoPE rows 8v .. 8v+7 (8 lanes per row)
    const int kpe_r = 8 * v + (lane >> 3);
    const uint32_t voff_kpe = kpe_r * kKpeRow + (((lane & 7) ^ ((kpe_r >> 1) & 7)) << 4);
    // transposed V read of half h2 (tokens 8h2 ..), column block cb (latent 128v + 32cb ..):
    // row 4*((lane&15)/4) + 2h2 + g2, logical chunk 16v + 4cb + 2*((lane>>4)&1) + (lane&3)/2
    uint32_t vx[8];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const int rv = 4 * ((lane & 15) >> 2) + 2 * h2 + g2;
            const int cl = 4 * cb + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
            vx[h2 * 4 + cb] = v * kBlock + rv * 256 + ((cl ^ (rv & 15)) << 4) + (lane & 1) * 8;
        }
    // weights of k-step kq for B-operand lane (t32, g2): slot (2kq + g2)*32 + (t32 ^ 4(2kq + g2))
    const uint32_t pr0 = (g2 * 32 + (t32 ^ (4 * g2))) * 16;
    const uint32_t pr1 = ((2 + g2) * 32 + (t32 ^ (4 * (2 + g2)))) * 16;
    const uint32_t ar_off = t32 * 8;                   // rescale factors of head t32 in both blocks

    auto stage_of = [&](int t) -> uint32_t { return sm + (t % kStages) * kTileCkv; };
    auto page_of = [&](int t) -> int64_t { return __builtin_amdgcn_readlane(plist, (t >> 1) - pl_base); };
    // Copies of tile t into block v of its stage (two instructions of four) and RoPE
    // rows 8v .. 8v+7 into its slot (one).  A tile past the segment's end (real =
    // false) gets a zero-length buffer: its loads move no memory, so every iteration
    // issues the same copies and the vmcnt accounting is the same in all of them.
    struct TileSrc {
        const char *ckv;
        const uint16_t *kpe;
        uint32_t ckv_bytes, kpe_bytes, st, rope;
    };
    auto tile_src = [&](int t) -> TileSrc {
        const bool real = t < n_tiles;
        if (real && (t >> 1) - pl_base >= 64) {
            // the next 64 pages: a load and its wait in one statement (the wait also
            // drains the copies in flight; once per 64 pages)
            pl_base = t >> 1;
            const int32_t *src = seg_bt + min(pl_base + lane, n_pages - 1);
            asm volatile("global_load_dword %0, %1, off\n\ts_waitcnt vmcnt(0)" : "=v"(plist) : "v"(src) : "memory");
            plist = checked_page(p, plist);
        }
        const int64_t phys = real ? page_of(t) : 0;
        const int64_t crow0 = phys * kPage + (t & 1) * kTile;   // first cache row of the tile
        return TileSrc{c_kv + crow0 * kCkvRow, k_pe + crow0 * kDr, real ? kTileCkv : 0u, real ? kTileKpe : 0u,
                       stage_of(t) + v * kBlock, sm + kOffRope + (t % kStages) * kTileKpe + v * 1024};
    };
    // part 0: rows 0..15, part 1: rows 16..31, part 2: RoPE rows
    auto copy_part = [&](const TileSrc &ts, int part) {
        if (part < 2)
            dma_blk4(ts.ckv, ts.ckv_bytes, ts.st + part * 4096, part * 16 * kCkvRow, vo[0], vo[1], vo[2], vo[3]);
        else
            dma_x4(ts.kpe, ts.kpe_bytes, ts.rope, 0, voff_kpe);
    };
    auto issue_tile = [&](int t) {
        const TileSrc ts = tile_src(t);
        copy_part(ts, 0);
        copy_part(ts, 1);
        copy_part(ts, 2);
    };
    // rows past the sequence end in a partial last tile: zero, so that their (zero)
    // weights never meet stale values in the latent product
    auto zero_tail = [&](int t) {
        const uint32_t st = stage_of(t) + v * kBlock;  // this wave's block
        for (int k = lane; k < (kTile - si.last_valid) * 16; k += 64)
            lds_store<u32x4>(st + (si.last_valid + (k >> 4)) * 256 + (k & 15) * 16, u32x4{0u, 0u, 0u, 0u});
    };

    f32x16 oacc[2][4];                 // [hb][cb]: latent 128v + 32cb .., heads 32hb + t32
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[hb][cb][e] = 0.f;

    // latent update of tile t: 21 LDS reads (rescale factors, weights, transposed V of
    // block v), all complete before the MFMAs, so that copy(g), run after MFMA group g,
    // may refill block v of this stage
    auto latent_tile = [&](int t, auto &&copy) {
        const uint32_t vb = stage_of(t);
        const uint32_t pb = sm + kOffP + (t & 1) * kPBuf;
        const u32x2 al = lds_load<u32x2>(sm + kOffAlpha + (t & 1) * kABuf + ar_off);
        const u32x4 pw00 = ld128(pb + pr0), pw10 = ld128(pb + pr0 + 2048);
        const u32x4 pw01 = ld128(pb + pr1), pw11 = ld128(pb + pr1 + 2048);
        v4i16 lo[2][4], hi[2][4];
#define MLA_VR(kq)                                                                                     \
        lo[kq][0] = ld_tr16(vb + vx[0] + (kq) * 4096); hi[kq][0] = ld_tr16(vb + vx[4] + (kq) * 4096); \
        lo[kq][1] = ld_tr16(vb + vx[1] + (kq) * 4096); hi[kq][1] = ld_tr16(vb + vx[5] + (kq) * 4096); \
        lo[kq][2] = ld_tr16(vb + vx[2] + (kq) * 4096); hi[kq][2] = ld_tr16(vb + vx[6] + (kq) * 4096); \
        lo[kq][3] = ld_tr16(vb + vx[3] + (kq) * 4096); hi[kq][3] = ld_tr16(vb + vx[7] + (kq) * 4096);
        MLA_VR(0)
        MLA_VR(1)
#undef MLA_VR
        // every read of block v has completed before copy() may refill it
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        // rescale (rare: the first tiles)
        {
            const float a0 = __uint_as_float(al[0]), a1 = __uint_as_float(al[1]);
            if (__builtin_amdgcn_ballot_w64(a0 != 1.f || a1 != 1.f)) {
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) {
                    oacc[0][cb] *= a0;
                    oacc[1][cb] *= a1;
                }
            }
        }
        pin();
#define MLA_PV(kq, cb, p0, p1)                                                                           \
        oacc[0][cb] = mfma32(tr_op(lo[kq][cb], hi[kq][cb]), as_bf16x8(p0), oacc[0][cb]);              \
        oacc[1][cb] = mfma32(tr_op(lo[kq][cb], hi[kq][cb]), as_bf16x8(p1), oacc[1][cb]);              \
        copy((kq) * 4 + (cb));                                                                           \
        pin();
        MLA_PV(0, 0, pw00, pw10) MLA_PV(0, 1, pw00, pw10) MLA_PV(0, 2, pw00, pw10) MLA_PV(0, 3, pw00, pw10)
        MLA_PV(1, 0, pw01, pw11) MLA_PV(1, 1, pw01, pw11) MLA_PV(1, 2, pw01, pw11) MLA_PV(1, 3, pw01, pw11)
#undef MLA_PV
    };
    auto no_copy = [](int) {};

    // prologue: copies of tiles 0, 1, 2; tile 0 lands (barrier); tile 1 lands and the
    // weights of tile 0 are out (barrier)
    issue_tile(0);
    issue_tile(1);
    issue_tile(2);
    wait_vmcnt<2 * kLoads>();                          // tile 0 landed
    barrier_lds();
    if (n_tiles == 1 && si.last_valid < kTile) zero_tail(0);
    if (n_tiles > 1) wait_vmcnt<kLoads>();             // tile 1 landed
    barrier_lds();
    for (int i = 0; i + 1 < n_tiles; ++i) {
        // latent update of tile i; block v of its stage takes tile i+3 once the V reads
        // are in, the RoPE slot of tile i (last read in the previous iteration) too
        const TileSrc ts = tile_src(i + 3);
        latent_tile(i, [&](int g) {
            if (g < 3) copy_part(ts, g);
        });
        if (i + 2 == n_tiles && si.last_valid < kTile) zero_tail(i + 1);   // before its V reads
        if (i + 2 < n_tiles) wait_vmcnt<kLoads>();     // tile i+2 landed (tile i+3 in flight)
        barrier_lds();
    }
    latent_tile(n_tiles - 1, no_copy);
    barrier_lds();                                     // the owners' 1 / sums are out
    const u32x2 inv = lds_load<u32x2>(sm + kOffFin + ar_off);
    // oacc[hb][cb][e]: head 32hb + t32, latent 128v + 32cb + 8*(e/4) + 4*g2 + e%4
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
        const float sc = __uint_as_float(inv[hb]);
        const int64_t dst = ((si.row_wg + 32 * hb + t32) * S + seg.c) * kDc + 128 * v + 4 * g2;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 o = f32x4{oacc[hb][cb][4 * q], oacc[hb][cb][4 * q + 1], oacc[hb][cb][4 * q + 2],
                                      oacc[hb][cb][4 * q + 3]} * sc;
                store_part4(o_part, p.part_dtype, dst + 32 * cb + 8 * q, o);
            }
    }
}

__global__ __launch_bounds__(kThreads) void decode8_kernel(
    const mla_params_t p, const uint16_t *__restrict__ q_abs, const uint16_t *__restrict__ q_rope,
    const char *__restrict__ c_kv, const uint16_t *__restrict__ k_pe, const int32_t *__restrict__ block_table,
    const int32_t *__restrict__ seq_lens, void *__restrict__ o_part, float *__restrict__ lse_part) {
    __shared__ __attribute__((aligned(1024))) char smem[kSmem];
    // workgroup -> (part, row group rg); parts are spread over the 8 XCDs, the row
    // groups of one part share an XCD (the second read of a page hits its L2)
    const int n_rg = (p.Sq * p.H) / kRows;
    const int qq = blockIdx.x >> 3;
    const int rg = qq % n_rg;
    const int part = (qq / n_rg) * 8 + (blockIdx.x & 7);
    const int n_parts = p.num_parts > 0 ? p.num_parts : p.B * p.num_splits;
    if (part >= n_parts) return;                       // grid rounded up to 8 XCDs
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = p.num_splits;
    uint32_t gen = 0;
    // the score waves' partial-ready counters start at 0 (ordered before any wait
    // on them by the first barrier of the first segment)
    if (w < 4 && lane == 0) lds_store<uint32_t>(lds_addr(smem) + kOffFlag + w * 4, 0u);
    bool first = true;
    // slots [c0, c1) of every row of this row group of sequence b: empty
    auto fill = [&](int b, int c0, int c1) {
        const int64_t row = static_cast<int64_t>(b) * p.Sq * p.H + rg * kRows + w * 8 + (lane >> 3);
        for (int c = c0 + (lane & 7); c < c1; c += 8) lse_part[row * S + c] = -INFINITY;
    };
    auto run = [&](const Segment &seg) {
        if (seg.pa >= seg.pb) {                        // an empty part inside the sequence's range
            if (seg.c < S) fill(seg.b, seg.c, seg.c + 1);
        } else if (seg.c < S) {
            if (!first) barrier_lds();                 // the previous segment's LDS traffic is done
            first = false;
            const SegInfo si = seg_info(p, seg, rg, seq_lens[seg.b]);
            if (w >= 4)
                latent_role(smem, p, c_kv, k_pe, block_table + static_cast<int64_t>(seg.b) * p.max_pages, seg, si, o_part);
            else if (w & 1)
                score_role<1>(smem, p, q_abs, q_rope, seg, si, rg, lse_part, gen);
            else
                score_role<0>(smem, p, q_abs, q_rope, seg, si, rg, lse_part, gen);
        } else if (threadIdx.x == 0) {
            raise_error(MLA_DEVERR_SPLITS);            // num_splits below the plan's bound
        }
        if (seg.last) fill(seg.b, seg.c + 1, S);       // slots after the last split carry no weight
    };
    for_each_segment(p, seq_lens, part, run, fill);
}

}  // namespace

bool decode8_supported(const mla_params_t &p) {
    return decode_mfma_supported(p) && p.kv_dtype == MLA_BF16;
}

hipError_t launch_decode8(const mla_params_t &p, const void *q_abs, const void *q_rope, const void *c_kv,
                          const void *k_pe, const int32_t *block_table, const int32_t *seq_lens, void *o_part,
                          float *lse_part, hipStream_t stream) {
    const int64_t parts = p.num_parts > 0 ? p.num_parts : static_cast<int64_t>(p.B) * p.num_splits;
    const int64_t n_rg = (static_cast<int64_t>(p.Sq) * p.H) / kRows;
    const int64_t blocks = ((parts + 7) / 8) * 8 * n_rg;
    hipLaunchKernelGGL(decode8_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream, p,
                       static_cast<const uint16_t *>(q_abs), static_cast<const uint16_t *>(q_rope),
                       static_cast<const char *>(c_kv), static_cast<const uint16_t *>(k_pe), block_table, seq_lens,
                       o_part, lse_part);
    return hipGetLastError();
}

hipError_t take_errors_decode8(uint32_t *bits) { return take_unit_errors(bits); }

}  // namespace mla
