// mla_decode_splitkv on bf16 MFMA: absorbed-MLA attention over the paged
// latent cache at the DeepSeek-V3 head shapes (d_c = 512 latent, d_r = 64
// RoPE key, page = 64 tokens), gfx950 / CDNA4.  Launched for the e4m3 cache
// (a bf16 cache runs on the eight-wave kernel of kernels_decode8.hip, so only
// the kFp8 = true instance of the template is built).
//
// Attention ("MLA Matrix Absorption" sec. 4.1-4.2; "DeepSeek-MLA-Principle"
// sec. 2 and matrix absorption 3)): every head of a sequence attends to the
// same latent cache row c_t (the MQA form of the absorbed computation), so for
// a tile of 32 tokens the scores of 32 heads are a dense [32 x 576] x [576 x 32]
// product and the latent update a dense [512 x 32] x [32 x 32] product.  Both
// run on v_mfma_f32_32x32x16_bf16.
//
// Work decomposition
//   workgroup = 4 waves = 64 query rows (s, h) of one row group rg, working
//               through the segments of one work part (below).  Waves 2p and
//               2p+1 form a pair that owns 32 heads of one query row s:
//                 scores: each wave contracts half of the 576 dims (wave 0 of
//                         the pair latent 0..287, wave 1 latent 288..511 and
//                         the RoPE key); the fp32 partial scores are swapped
//                         through LDS and added, so both hold the full scores;
//                 softmax: computed identically by both waves;
//                 latent: each wave accumulates half of the 512 latent columns.
//               Per wave this keeps 72 VGPRs of query and 128 AGPRs of output.
//   work part = fixed splits: one (sequence, split) item, pages
//               [c*split_pages, (c+1)*split_pages) of sequence b;
//               balanced: one of num_parts equal shares of the batch's pages
//               taken in order (sequence 0's pages, then sequence 1's, ...),
//               cut into one segment per sequence it touches.  Every
//               workgroup then streams the same number of pages.
//   grid      = parts x row groups, numbered so that the row groups of one
//               part run on the same XCD (workgroup i runs on XCD i % 8) at
//               the same time: the second read of a page hits that XCD's L2.
//   pipeline  = 32-token tiles.  Iteration i overlaps the score MFMAs of tile
//               i+1 with the softmax of tile i, then runs the latent MFMAs of
//               tile i while the partner's partial scores of tile i+1 land in
//               LDS.  Tiles are copied global->LDS by buffer_load ... lds (no
//               VGPR staging) into a ring (bf16: 4 stages, copies issued 3
//               tiles ahead, one instruction per odd score MFMA).  The 16-byte chunks
//               of each latent row are XOR-swizzled with (row % 16), which
//               keeps both the K-operand reads (16 rows, one column) and the
//               transposing V reads (4 rows x 64 bytes per 16 lanes) free of
//               bank conflicts.  The K operands are read 8 steps ahead of
//               their MFMA (the compiler places the counted waits).
//   scores    = S^T[token, head] = K[token, k] . Q^T[k, head]: K from LDS
//               (A operand), the query rows in registers (B operand).
//   softmax   = online, in the exp2 domain; a head's 32 scores of a tile sit
//               in lanes l and l^32.  The reference maximum is only raised
//               (and O rescaled) when a score exceeds it by more than 2^8.
//   latent PV = O^T[latent, head] += V^T[latent, token] . P^T[token, head]:
//               P^T straight from the score accumulators (same lane = same
//               head), V^T from ds_read_b64_tr_b16 transposing LDS reads.
//   output    = normalised partial O_c (fp32) and its log-sum-exp per row.
// fp8 cache: the e4m3 tile (16 KiB) is copied raw into LDS and converted once
// per workgroup into the same bf16 layout (e4m3 values are exact in bf16);
// the per-token scale multiplies the content score before the RoPE term is
// added and the weight p_t before it is rounded to bf16.
#include <hip/hip_runtime.h>
#include <math.h>

#include "decode_common.h"

namespace mla {
namespace {

using namespace gfx;
using namespace dec;

constexpr int kThreads = 256;
constexpr int kRows = kDecodeRowsPerBlock;             // query rows per workgroup
// bf16 cache: 4-stage ring of [c_kv | k_pe] tiles, then the score exchange area
constexpr int kStagesBf16 = 4;
constexpr int kStageBf16 = kTileCkv + kTileKpe;        // 36864
// fp8 cache: 3-stage ring of raw [e4m3 c_kv | k_pe | scales] tiles, 2 converted bf16 tiles
constexpr int kStagesFp8 = 3;
constexpr int kRawCkv = kTile * kDc;                   // 16384
constexpr int kStageFp8 = kRawCkv + kTileKpe + kTile * 4;  // 20608
constexpr int kXchgWave = 64 * 16 * 4;                 // 16 fp32 per lane
constexpr int kXchg = 4 * kXchgWave;                   // one slot per wave
constexpr int kSmemBf16 = kStagesBf16 * kStageBf16 + kXchg;                 // 163840
constexpr int kSmemFp8 = kStagesFp8 * kStageFp8 + 2 * kTileCkv + kXchg;     // 143744
constexpr int kLoadsBf16 = (kTileCkv + kTileKpe) / 1024 / 4;                // 9 per wave per tile
constexpr int kLoadsFp8 = (kRawCkv + kTileKpe) / 1024 / 4 + 1;              // 6 per wave per tile
constexpr int kSteps = 18;                             // 32x32x16 MFMA k-steps per wave per tile
constexpr int kReadAhead = 8;                          // K-operand reads in flight
static_assert(kSmemBf16 <= 160 * 1024, "LDS budget");
static_assert(kRows == 64, "four waves of 32 heads in pairs");

// O^T[256 latent columns of this wave, 32 heads] += V^T[., 16 tokens] P^T[16 tokens, heads]
// for one 16-token k-step kq of a tile: 16 transposing reads, then per column
// block the MFMA and fill(blk) (VALU work slotted under the MFMAs).  vx[h*4 +
// b4]: lane address of the transposing read of half h (tokens 8h..) for column
// blocks blk = b4, b4+4.
template <int kq, typename Fill>
__device__ __forceinline__ void latent_step(uint32_t base, const uint32_t *vx, bf16x8 pb, f32x16 *oacc,
                                            Fill &&fill) {
    constexpr int kq_off = kq * 16 * kCkvRow;
    v4i16 lo[8], hi[8];
#define MLA_TR(blk) \
    lo[blk] = ld_tr16(base + vx[(blk) & 3] + kq_off + ((blk) >> 2) * 256); \
    hi[blk] = ld_tr16(base + vx[4 + ((blk) & 3)] + kq_off + ((blk) >> 2) * 256);
    MLA_TR(0) MLA_TR(1) MLA_TR(2) MLA_TR(3) MLA_TR(4) MLA_TR(5) MLA_TR(6) MLA_TR(7)
#undef MLA_TR
    pin();
#define MLA_PV(blk)                                                                                 \
    oacc[blk] = mfma32(__builtin_bit_cast(bf16x8, v8i16{lo[blk][0], lo[blk][1], lo[blk][2], lo[blk][3], \
                                                        hi[blk][0], hi[blk][1], hi[blk][2], hi[blk][3]}), \
                       pb, oacc[blk]);                                                              \
    fill(blk);                                                                                      \
    pin();
    MLA_PV(0) MLA_PV(1) MLA_PV(2) MLA_PV(3) MLA_PV(4) MLA_PV(5) MLA_PV(6) MLA_PV(7)
#undef MLA_PV
}

// K operand of score step k for this wave's half (KH) of the 576 dims:
//   KH = 0: latent chunk 2k + g2 (dims 16k ..), k < 18
//   KH = 1: latent chunk 2k + 36 + g2 (dims 288 + 16k ..) for k < 14, then RoPE chunk 2(k-14) + g2
// kb[u]: tile base + lane offset of chunk column u (see the layout above); kp[r]: RoPE chunk r
template <int KH, int k>
__device__ __forceinline__ u32x4 k_operand(const uint32_t *kb, const uint32_t *kp) {
    if constexpr (KH == 1 && k >= 14) {
        return ld128(kp[k - 14]);
    } else {
        constexpr int chunk = 2 * k + 36 * KH;             // logical chunk for g2 = 0
        return ld128(kb[(chunk >> 1) & 7] + ((chunk & ~15) << 4));
    }
}

// Partial scores of one tile over this wave's half of the 576 dims (one MFMA
// chain of 18 steps; K operands read 8 steps ahead), with copy(part) of a
// later tile's part (k-1)/2 after every odd step k and fill(k) after every MFMA.
//   tsc (fp8): per-D-element token scales, multiplied in before the RoPE term
template <int KH, bool kFp8, typename Copy, typename Fill>
__device__ __forceinline__ f32x16 score_tile(const uint32_t *kb, const uint32_t *kp, const bf16x8 *qreg,
                                             const float *tsc, Copy &&copy, Fill &&fill) {
    constexpr int kContent = KH == 0 ? kSteps : 14;
    u32x4 a[kSteps];
    f32x16 acc;
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = 0.f;
#define MLA_KREAD(k) a[k] = k_operand<KH, k>(kb, kp);
    MLA_KREAD(0) MLA_KREAD(1) MLA_KREAD(2) MLA_KREAD(3) MLA_KREAD(4) MLA_KREAD(5) MLA_KREAD(6) MLA_KREAD(7)
    pin();
    // step k: wait for read k (reads up to k+7 may be in flight), MFMA, read k+8
#define MLA_KSTEP(k)                                                                   \
    {                                                                                  \
        if constexpr (kFp8 && (k) == kContent) {                                       \
            for (int j = 0; j < 16; ++j) acc[j] *= tsc[j];                              \
        }                                                                              \
        acc = mfma32(as_bf16x8(a[k]), qreg[k], acc);                                   \
        if constexpr ((k) + kReadAhead < kSteps) a[(k) + kReadAhead] = k_operand<KH, (k) + kReadAhead>(kb, kp); \
        if constexpr ((k) & 1) copy((k) >> 1);                                         \
        fill(k);                                                                       \
        pin();                                                                         \
    }
    MLA_KSTEP(0) MLA_KSTEP(1) MLA_KSTEP(2) MLA_KSTEP(3) MLA_KSTEP(4) MLA_KSTEP(5)
    MLA_KSTEP(6) MLA_KSTEP(7) MLA_KSTEP(8) MLA_KSTEP(9) MLA_KSTEP(10) MLA_KSTEP(11)
    MLA_KSTEP(12) MLA_KSTEP(13) MLA_KSTEP(14) MLA_KSTEP(15) MLA_KSTEP(16) MLA_KSTEP(17)
#undef MLA_KSTEP
#undef MLA_KREAD
    if constexpr (kFp8 && KH == 0) {
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[j] *= tsc[j];
    }
    return acc;
}

// ---------------------------------------------------------------------------
// Steady-state phases with reads issued one phase ahead (cross-phase pipeline).
// Per tile, a wave's LDS operations are issued in this order:
//   score phase: K reads R0..R17 (8 ahead); in slots 10..17 also the transposing
//                reads T0..T15 of the first latent k-step (two per slot)
//   exchange writes W0..W3
//   first latent k-step: slot b waits for T(2b, 2b+1) and issues U(2b, 2b+1), the
//                reads of the second k-step
//   barrier (after W3 completed), exchange reads X0..X3
//   second latent k-step: uses U, then X
// The reads are plain loads: the compiler's counted waits before each use keep the
// later ones in flight.
// ---------------------------------------------------------------------------
// transposing reads of column block blk (halves lo / hi) of k-step kq
#define MLA_TR_PAIR(kq, blk, lo, hi, base, vx)                                                         \
    lo = ld_tr16((base) + (vx)[(blk) & 3] + (kq) * 16 * kCkvRow + ((blk) >> 2) * 256);                 \
    hi = ld_tr16((base) + (vx)[4 + ((blk) & 3)] + (kq) * 16 * kCkvRow + ((blk) >> 2) * 256);

__device__ __forceinline__ bf16x8 tr_operand(const v4i16 &lo, const v4i16 &hi) {
    return __builtin_bit_cast(bf16x8, v8i16{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
}

// Score phase with the first latent k-step's reads (of the tile at vbase) in slots 10..17.
template <int KH, bool kFp8, typename Copy, typename Fill>
__device__ __forceinline__ f32x16 score_tile_ahead(const uint32_t *kb, const uint32_t *kp, const bf16x8 *qreg,
                                                   const float *tsc, Copy &&copy, Fill &&fill, uint32_t vbase,
                                                   const uint32_t *vx, v4i16 *tlo, v4i16 *thi) {
    constexpr int kContent = KH == 0 ? kSteps : 14;
    u32x4 a[kSteps];
    f32x16 acc;
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = 0.f;
#define MLA_KREAD(k) a[k] = k_operand<KH, k>(kb, kp);
    MLA_KREAD(0) MLA_KREAD(1) MLA_KREAD(2) MLA_KREAD(3) MLA_KREAD(4) MLA_KREAD(5) MLA_KREAD(6) MLA_KREAD(7)
    pin();
    // slot k waits for R(k): younger are R(k+1..min(k+7,17)) and the T pairs of slots 10..k-1
#define MLA_KSTEP(k)                                                                   \
    {                                                                                  \
        if constexpr (kFp8 && (k) == kContent) {                                       \
            for (int j = 0; j < 16; ++j) acc[j] *= tsc[j];                              \
        }                                                                              \
        acc = mfma32(as_bf16x8(a[k]), qreg[k], acc);                                   \
        if constexpr ((k) + kReadAhead < kSteps) a[(k) + kReadAhead] = k_operand<KH, (k) + kReadAhead>(kb, kp); \
        if constexpr ((k) >= 10) { MLA_TR_PAIR(0, (k) - 10, tlo[(k) - 10], thi[(k) - 10], vbase, vx) } \
        if constexpr ((k) & 1) copy((k) >> 1);                                         \
        fill(k);                                                                       \
        pin();                                                                         \
    }
    MLA_KSTEP(0) MLA_KSTEP(1) MLA_KSTEP(2) MLA_KSTEP(3) MLA_KSTEP(4) MLA_KSTEP(5)
    MLA_KSTEP(6) MLA_KSTEP(7) MLA_KSTEP(8) MLA_KSTEP(9) MLA_KSTEP(10) MLA_KSTEP(11)
    MLA_KSTEP(12) MLA_KSTEP(13) MLA_KSTEP(14) MLA_KSTEP(15) MLA_KSTEP(16) MLA_KSTEP(17)
#undef MLA_KSTEP
#undef MLA_KREAD
    if constexpr (kFp8 && KH == 0) {
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[j] *= tsc[j];
    }
    return acc;
}

// First latent k-step on the reads T issued in the score phase (the four exchange
// writes follow them); slot b issues the reads U of the second k-step.
__device__ __forceinline__ void latent_first(const v4i16 *tlo, const v4i16 *thi, bf16x8 pb, f32x16 *oacc,
                                             uint32_t vbase, const uint32_t *vx, v4i16 *ulo, v4i16 *uhi) {
#define MLA_B1(blk)                                                                    \
    {                                                                                  \
        v4i16 lo = tlo[blk], hi = thi[blk];                                            \
        oacc[blk] = mfma32(tr_operand(lo, hi), pb, oacc[blk]);                         \
        MLA_TR_PAIR(1, blk, ulo[blk], uhi[blk], vbase, vx)                             \
        pin();                                                                         \
    }
    MLA_B1(0) MLA_B1(1) MLA_B1(2) MLA_B1(3) MLA_B1(4) MLA_B1(5) MLA_B1(6) MLA_B1(7)
#undef MLA_B1
}

// Second latent k-step on the reads U, with the exchange reads X0..X3 issued after
// them; fill(b) runs after MFMA b.
template <typename Fill>
__device__ __forceinline__ void latent_second(const v4i16 *ulo, const v4i16 *uhi, bf16x8 pb, f32x16 *oacc,
                                              u32x4 *xr, Fill &&fill) {
#define MLA_B2(blk)                                                                    \
    {                                                                                  \
        v4i16 lo = ulo[blk], hi = uhi[blk];                                            \
        oacc[blk] = mfma32(tr_operand(lo, hi), pb, oacc[blk]);                         \
        fill(blk);                                                                     \
        pin();                                                                         \
    }
    MLA_B2(0) MLA_B2(1) MLA_B2(2) MLA_B2(3) MLA_B2(4) MLA_B2(5) MLA_B2(6) MLA_B2(7)
#undef MLA_B2
}

// ---------------------------------------------------------------------------
// One segment for one wave: rows of pair (wave >> 1) of row group rg, tokens
// [t_begin, t_end) of sequence b, partial written to split slot c.
// KH (= wave % 2, the wave's half of the pair's work) is a template parameter
// so that each wave's loop is straight-line code the scheduler can interleave.
// ---------------------------------------------------------------------------
template <bool kFp8, int KH>
__device__ __forceinline__ void attend_segment(
    char *smem, const mla_params_t &p, const uint16_t *__restrict__ q_abs, const uint16_t *__restrict__ q_rope,
    const void *__restrict__ c_kv, const uint16_t *__restrict__ k_pe,
    const float *__restrict__ kv_scale, const int32_t *__restrict__ bt, int seq_len,
    const Segment &seg, int rg, void *__restrict__ o_part, float *__restrict__ lse_part) {
    constexpr int kNst = kFp8 ? kStagesFp8 : kStagesBf16;     // raw ring depth
    constexpr int kAhead = kNst - 1;                          // tiles copied ahead of the one finishing
    constexpr int kLoads = kFp8 ? kLoadsFp8 : kLoadsBf16;
    constexpr int kStage = kFp8 ? kStageFp8 : kStageBf16;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int t32 = lane & 31;          // A/B operand row, D column (= head of the pair)
    const int g2 = lane >> 5;           // k-group of the operands, row group of D
    constexpr int kh = KH;              // which half of the contraction / latent columns
    const int S = p.num_splits;

    seq_len = __builtin_amdgcn_readfirstlane(seq_len);              // wave-uniform scalars
    const int t_begin = __builtin_amdgcn_readfirstlane(seg.pa * kPage);                 // page aligned
    const int t_end = __builtin_amdgcn_readfirstlane(min(seg.pb * kPage, seq_len));     // past the last stored token
    const int row0 = rg * kRows + (wave >> 1) * 32;    // first (s,h) row of this wave pair
    const int s = row0 / p.H;
    const int h = row0 % p.H + t32;                    // this lane's head
    const int64_t qrow = (static_cast<int64_t>(seg.b) * p.Sq + s) * p.H + h;
    const int n_vis = __builtin_amdgcn_readfirstlane(seq_len - p.Sq + 1 + s);   // positions these rows may see
    const int64_t out_row = qrow * S + seg.c;
    const int n_tiles = __builtin_amdgcn_readfirstlane((t_end - t_begin + kTile - 1) / kTile);   // >= 1
    const int last_valid = __builtin_amdgcn_readfirstlane(t_end - (t_begin + (n_tiles - 1) * kTile));  // rows of the last tile
    // earlier stores (a previous segment's partials) complete before the counted
    // waits on this segment's copies begin
    wait_vmcnt<0>();

    // query operands (B of the score product) for this wave's half of the 576 dims
    bf16x8 qreg[kSteps];
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) {
        const uint16_t *src;
        if (kh == 0) src = q_abs + qrow * kDc + ks * 16 + g2 * 8;                   // latent 0..287
        else if (ks < 14) src = q_abs + qrow * kDc + 288 + ks * 16 + g2 * 8;         // latent 288..511
        else src = q_rope + qrow * kDr + (ks - 14) * 16 + g2 * 8;                    // RoPE 0..63
        qreg[ks] = *reinterpret_cast<const bf16x8 *>(src);
    }
    // the segment's pages, one per lane (refilled every 64 pages)
    const int n_pages = __builtin_amdgcn_readfirstlane(seg.pb - seg.pa);
    const int32_t *seg_bt = bt + __builtin_amdgcn_readfirstlane(seg.pa);
    int pl_base = 0;
    int plist = checked_page(p, seg_bt[min(lane, n_pages - 1)]);
    // Consume the loads here: otherwise the compiler places their vmcnt
    // waits at the first use inside the tile loop, where (re-executed every
    // iteration) they would also wait for the tile copies in flight.
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) asm volatile("" : "+v"(qreg[ks]));
    asm volatile("" : "+v"(plist));

    const uint32_t sm = lds_addr(smem);
    const uint32_t xchg = sm + (kFp8 ? kStagesFp8 * kStageFp8 + 2 * kTileCkv : kStagesBf16 * kStageBf16);
    const uint32_t conv0 = sm + kStagesFp8 * kStageFp8;                  // fp8: converted tiles

    // ---- loop-invariant lane offsets
    // copies: latent row r = wave*8 + jj stores logical chunk lane^(r%16) in physical chunk lane
    uint32_t vd[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) vd[jj] = (lane ^ ((kh << 3) | jj)) << 4;
    const int kpe_r = wave * 8 + (lane >> 3);          // RoPE rows: 8 per instruction
    const uint32_t voff_kpe = kpe_r * kKpeRow + (((lane & 7) ^ ((kpe_r >> 1) & 7)) << 4);
    // K operand: row perm_tok(t32), chunk column u holds logical chunk (2u + g2) ^ (row % 16)
    const int krow = perm_tok(t32);
    uint32_t kx[8], kpx[4];
#pragma unroll
    for (int u8 = 0; u8 < 8; ++u8) kx[u8] = krow * kCkvRow + ((((2 * u8 + g2) & 15) ^ (krow & 15)) << 4);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kpx[ks] = krow * kKpeRow + (((2 * ks + g2) ^ ((krow >> 1) & 7)) << 4);
    // transposing V read of half h, column block b4 (+4): row 4*((lane&15)/4) + 2h + g2,
    // logical chunk 32kh + 4*b4 + 2*((lane>>4)&1) + (lane&3)/2, byte 8*(lane&1)
    uint32_t vx[8];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) {
            const int rv = 4 * ((lane & 15) >> 2) + 2 * hh + g2;
            const int cl = 4 * b4 + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
            vx[hh * 4 + b4] = rv * kCkvRow + ((cl ^ (rv & 15)) << 4) + (lane & 1) * 8 + kh * 512;
        }

    auto stage_of = [&](int t) -> uint32_t { return sm + (t % kNst) * kStage; };
    // LDS addresses of tile t's latent rows (bf16 layout) and RoPE rows
    auto ckv_of = [&](int t) -> uint32_t { return kFp8 ? conv0 + (t & 1) * kTileCkv : stage_of(t); };
    auto kpe_of = [&](int t) -> uint32_t { return stage_of(t) + (kFp8 ? kRawCkv : kTileCkv); };

    // physical page of tile t (pages are listed from the segment's first page)
    auto page_of = [&](int t) -> int64_t {
        const int k = t >> 1;
        if (k - pl_base >= 64) {
            // the next 64 pages (segments of more than 4096 tokens): a load and its
            // wait in one statement, so that no wait for it lands on the common path
            // (the wait also drains the copies in flight; this is rare)
            pl_base = k & ~63;
            const int32_t *src = seg_bt + min(pl_base + lane, n_pages - 1);
            asm volatile("global_load_dword %0, %1, off\n\ts_waitcnt vmcnt(0)" : "=v"(plist) : "v"(src) : "memory");
            plist = checked_page(p, plist);
        }
        return __builtin_amdgcn_readlane(plist, k - pl_base);
    };
    // copy of tile t (tokens t_begin + 32t ...) from page `phys` into its ring stage, in
    // three parts 0, 1, 2.  Every position of the ring schedule issues its copies, so
    // the vmcnt accounting is the same in every iteration: a tile past the segment's
    // end (real = false) gets a zero-length buffer, whose loads move no memory and
    // fill the (unused) stage with zeros.
    auto copy_part = [&](int t, int64_t phys, int part, bool real) {
        const int64_t crow0 = phys * kPage + (t & 1) * kTile;   // first cache row of the tile
        const uint32_t base = stage_of(t);
        const uint32_t live = real ? ~0u : 0u;
        if constexpr (!kFp8) {
            // parts 0..7: latent row wave*8 + part; part 8: the wave's 8 RoPE-key rows
            if (part < 8) {
                const uint32_t r = wave * 8 + part;
                dma_x4(static_cast<const char *>(c_kv) + crow0 * kCkvRow, kTileCkv & live, base + r * kCkvRow,
                       r * kCkvRow, vd[part]);
            } else {
                dma_x4(k_pe + crow0 * kDr, kTileKpe & live, base + kTileCkv + wave * 1024, 0, voff_kpe);
            }
        } else {
            // parts 0..3: one KiB of the wave's 4 KiB of codes; 4: RoPE keys; 5: scales
            if (part < 4) {
                const uint32_t o = wave * 4096 + part * 1024;
                dma_x4(static_cast<const char *>(c_kv) + crow0 * kDc, kRawCkv & live, base + o, o, lane * 16);
            } else if (part == 4) {
                dma_x4(k_pe + crow0 * kDr, kTileKpe & live, base + kRawCkv + wave * 1024, 0, voff_kpe);
            } else if (lane < 8) {
                dma_x1(kv_scale + crow0, (kTile * 4) & live, base + kRawCkv + kTileKpe + wave * 32, wave * 32, lane * 4);
            }
        }
    };
    auto issue_tile = [&](int t) {
        const bool real = t < n_tiles;
        const int64_t phys = real ? page_of(t) : 0;
#pragma unroll
        for (int part = 0; part < kLoads; ++part) copy_part(t, phys, part, real);
    };

    // make tile t (just landed) ready for the MFMAs: fp8 -> bf16 conversion, or (bf16)
    // zeroing of the rows past the sequence end in a partial last tile; returns
    // whether a barrier is needed before reading it
    auto prepare_tile = [&](int t) -> bool {
        const int valid = t == n_tiles - 1 ? last_valid : kTile;
        if constexpr (kFp8) {
            const uint32_t raw = stage_of(t);
            const uint32_t dst = ckv_of(t);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int unit = threadIdx.x + k * kThreads;   // 8 latents of one token
                const int tok = unit >> 6, lc = unit & 63;
                const u32x2 v = lds_load<u32x2>(raw + tok * kDc + lc * 8);
                u32x4 o;
#pragma unroll
                for (int hw = 0; hw < 2; ++hw) {
                    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(v[hw], false);
                    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(v[hw], true);
                    // e4m3 values are exact in bf16: keep the upper halves
                    o[hw * 2 + 0] = pack_hi(__float_as_uint(lo[0]), __float_as_uint(lo[1]));
                    o[hw * 2 + 1] = pack_hi(__float_as_uint(hi[0]), __float_as_uint(hi[1]));
                }
                if (tok >= valid) o = u32x4{0u, 0u, 0u, 0u};   // past the sequence end
                lds_store<u32x4>(dst + tok * kCkvRow + ((lc ^ (tok & 15)) << 4), o);
            }
            return true;
        } else {
            if (valid == kTile) return false;
            const uint32_t w = stage_of(t);
            for (int k = threadIdx.x; k < (kTile - valid) * 64; k += kThreads)
                lds_store<u32x4>(w + (valid + (k >> 6)) * kCkvRow + (k & 63) * 16, u32x4{0u, 0u, 0u, 0u});
            return true;
        }
    };

    // per-D-element token scales of tile t (fp8), zero past the sequence end
    auto token_scales = [&](int t, float *tsc) {
        const int valid = t == n_tiles - 1 ? last_valid : kTile;
        const uint32_t sc = stage_of(t) + kRawCkv + kTileKpe;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int tok = perm_tok((j >> 2) * 8 + g2 * 4 + (j & 3));
            tsc[j] = tok < valid ? lds_load<float>(sc + tok * 4) : 0.f;
        }
    };

    // partial scores of tile t (tsc: its token scales, fp8), with copy(part) and
    // fill(k) slotted between the MFMAs
    auto partial_scores = [&](int t, const float *tsc, auto &&copy, auto &&fill) -> f32x16 {
        uint32_t kb[8], kp[4];
        const uint32_t ckv = ckv_of(t), kpe = kpe_of(t);
#pragma unroll
        for (int u = 0; u < 8; ++u) kb[u] = ckv + kx[u];
#pragma unroll
        for (int r = 0; r < 4; ++r) kp[r] = kpe + kpx[r];
        return score_tile<KH, kFp8>(kb, kp, qreg, tsc, copy, fill);
    };
    auto partial_scores_ahead = [&](int t, const float *tsc, auto &&copy, auto &&fill, uint32_t vbase,
                                    v4i16 *tlo, v4i16 *thi) -> f32x16 {
        uint32_t kb[8], kp[4];
        const uint32_t ckv = ckv_of(t), kpe = kpe_of(t);
#pragma unroll
        for (int u = 0; u < 8; ++u) kb[u] = ckv + kx[u];
#pragma unroll
        for (int r = 0; r < 4; ++r) kp[r] = kpe + kpx[r];
        return score_tile_ahead<KH, kFp8>(kb, kp, qreg, tsc, copy, fill, vbase, vx, tlo, thi);
    };

    // partial scores are swapped with the other wave of the pair through LDS: four
    // asm writes / reads each (slot of wave w: lane l's floats 4jq.. at jq*1024 + 16l)
    auto exchange_write = [&](const f32x16 &sp) {
        const uint32_t w = xchg + wave * kXchgWave + lane * 16;
#define MLA_XW(jq) \
        lds_store<u32x4>(w + (jq) * 1024, u32x4{__float_as_uint(sp[4 * (jq)]), __float_as_uint(sp[4 * (jq) + 1]), \
                                                __float_as_uint(sp[4 * (jq) + 2]), __float_as_uint(sp[4 * (jq) + 3])});
        MLA_XW(0) MLA_XW(1) MLA_XW(2) MLA_XW(3)
#undef MLA_XW
    };
    u32x4 xr[4];                                       // the partner's partial scores, as read
    auto exchange_read = [&]() {
        const uint32_t r = xchg + (wave ^ 1) * kXchgWave + lane * 16;
        xr[0] = ld128(r);
        xr[1] = ld128(r + 1024);
        xr[2] = ld128(r + 2048);
        xr[3] = ld128(r + 3072);
    };

    float m_ref = -INFINITY;   // reference maximum (log2 domain), identical in a head's lanes
    float l_run = 0.f;         // this lane's share of the sum of exp2 weights (-> lse)
    float lw_run = 0.f;        // ... of the weights as rounded for the PV product (-> O; bf16 cache)
    f32x16 oacc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[i][j] = 0.f;
    const float zscale = p.scale * kLog2e;
    const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);

    // Full scores and running maximum of tile t, in five pieces slotted under the
    // MFMAs of a latent phase (piece 0 needs the partner's scores in xr):
    //   0, 1: sc = own + partner (commutative: the same sum in both waves)
    //   2: mask positions past the causal bound / sequence end
    //   3: maximum of the lane's 16 scores;  4: of the head's 32, raise decision
    f32x16 sc;
    float mloc = 0.f;
    bool raise = false;
    uint64_t any_raise = 0;
    auto max_piece = [&](int t, const f32x16 &own, int piece) {
        if (piece == 0 || piece == 1) {
#pragma unroll
            for (int j = 8 * piece; j < 8 * piece + 8; ++j) sc[j] = own[j] + __uint_as_float(xr[j >> 2][j & 3]);
        } else if (piece == 2) {
            const int tbase = t_begin + t * kTile;
            if (tbase + kTile > n_vis) {               // causal bound or sequence end inside the tile
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    if (tbase + perm_tok((j >> 2) * 8 + g2 * 4 + (j & 3)) >= n_vis) sc[j] = -INFINITY;
            }
        } else if (piece == 3) {
            float m = fmaxf(fmaxf(sc[0], sc[1]), sc[2]);
#pragma unroll
            for (int j = 3; j < 15; j += 2) m = fmaxf(fmaxf(m, sc[j]), sc[j + 1]);
            mloc = fmaxf(m, sc[15]);
        } else if (piece == 4) {
            mloc = pair_max(mloc) * zscale;            // zscale > 0: max commutes with it
            // raise the reference only when a weight would exceed 2^kRescaleSlack
            raise = mloc > m_ref + kRescaleSlack;
            any_raise = __builtin_amdgcn_ballot_w64(raise);
        }
    };
    // after the latent phase: rescale O when the reference rises; returns the
    // reference the tile's weights are taken against
    auto max_finish = [&]() -> float {
        if (any_raise) {
            // the latent MFMAs just issued write oacc: let them finish before the
            // accumulators are read back
            asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
            const float m_new = raise ? mloc : m_ref;
            const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);   // 0 when m_ref = -inf
            l_run *= alpha;
            lw_run *= alpha;
            // element-wise in place: the accumulators stay in AGPRs (VALU cannot
            // read AGPRs, so a plain multiply would pull all 128 into VGPRs)
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    float v = oacc[i][j];
                    scale_agpr(v, alpha);
                    oacc[i][j] = v;
                }
            m_ref = m_new;
        }
        return (m_ref == -INFINITY) ? 0.f : m_ref;     // nothing visible yet: weights 0
    };
    // weight of score j of the current tile, 2^(z - m): pieces j = 0..15 slotted under
    // the score MFMAs of the next tile; odd j also packs the pair into the bf16 P^T
    // operand and adds it to the sums.  Masked scores are -inf: exp2(-inf) = 0.
    auto weight_piece = [&](int j, float m_use, const float *tsc, float *pw, uint32_t *pk) {
        pw[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[j], zscale, -m_use));
        if (j & 1) {
            l_run += pw[j - 1] + pw[j];
            if constexpr (kFp8) {
                pk[j >> 1] = cvt_pk_bf16(pw[j - 1] * tsc[j - 1], pw[j] * tsc[j]);
            } else {
                pk[j >> 1] = cvt_pk_bf16(pw[j - 1], pw[j]);
                // the sum of the weights exactly as the PV product sees them
                lw_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[j >> 1]), ones, lw_run, false);
            }
        }
    };
    auto no_copy = [](int) {};
    auto no_fill = [](int) {};
    float tsc_cur[16], tsc_next[16];                  // token scales (fp8) of tiles i and i+1

    // ---- prologue: copies of tiles 0 .. kAhead-1; scores, exchange and maximum of tile 0
#pragma unroll
    for (int t = 0; t < kAhead; ++t) issue_tile(t);
    wait_vmcnt<(kAhead - 1) * kLoads>();               // tile 0 landed; tiles 1 .. kAhead-1 in flight
    barrier_lds();
    if (prepare_tile(0)) barrier_lds();
    if constexpr (kFp8) token_scales(0, tsc_cur);
    f32x16 own = partial_scores(0, tsc_cur, no_copy, no_fill);
    exchange_write(own);
    barrier_lds();
    exchange_read();
#pragma unroll
    for (int piece = 0; piece < 5; ++piece) max_piece(0, own, piece);
    float m_use = max_finish();
    if (n_tiles > 1) {                                 // tile 1 landed; tiles 2 .. kAhead-1 in flight
        wait_vmcnt<(kAhead - 2) * kLoads>();
        barrier_lds();
    }

    // ---- steady state: tiles 0 .. n-2 (the next tile exists)
    for (int i = 0; i + 1 < n_tiles; ++i) {
        // tile i+1 has landed and is visible; every wave is done with tile i-1
        if (prepare_tile(i + 1)) barrier_lds();
        if constexpr (kFp8) token_scales(i + 1, tsc_next);
        // copies of tile i+kAhead into the stage of tile i-1
        const int t_copy = i + kAhead;
        const bool copy_real = t_copy < n_tiles;
        const int64_t phys = copy_real ? page_of(t_copy) : 0;
        auto copy = [&](int part) {
            if (part < kLoads) copy_part(t_copy, phys, part, copy_real);
        };
        // score MFMAs of tile i+1, with the weights of tile i under them and the
        // first latent k-step's reads of tile i in the last slots
        float pw[16];
        uint32_t pk[8];
        const float m_cur = m_use;
        const uint32_t vbase = ckv_of(i);
        v4i16 tlo[8], thi[8], ulo[8], uhi[8];
        own = partial_scores_ahead(i + 1, tsc_next, copy, [&](int k) {
            if (k < 16) weight_piece(k, m_cur, tsc_cur, pw, pk);
        }, vbase, tlo, thi);
        exchange_write(own);
        pin();                                         // the writes precede the reads U
        // latent MFMAs of tile i, first k-step (issuing the second k-step's reads)
        latent_first(tlo, thi, as_bf16x8(u32x4{pk[0], pk[1], pk[2], pk[3]}), oacc, vbase, vx, ulo, uhi);
        // the exchange writes have completed (they precede the 16 reads U, and LDS
        // operations complete in order): partner may read
        asm volatile("s_waitcnt lgkmcnt(15)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        exchange_read();
        // second k-step, with the full scores and maximum of tile i+1 under its last MFMAs
        latent_second(ulo, uhi, as_bf16x8(u32x4{pk[4], pk[5], pk[6], pk[7]}), oacc, xr, [&](int blk) {
            if (blk == 4) { max_piece(i + 1, own, 0); max_piece(i + 1, own, 1); }
            if (blk == 5) { max_piece(i + 1, own, 2); max_piece(i + 1, own, 3); }
            if (blk == 6) max_piece(i + 1, own, 4);
        });
        m_use = max_finish();
        if (i + 2 < n_tiles) {                         // tile i+2 landed; later copies in flight
            wait_vmcnt<(kAhead - 2) * kLoads>();
            barrier_lds();
        }
        if constexpr (kFp8) {
#pragma unroll
            for (int j = 0; j < 16; ++j) tsc_cur[j] = tsc_next[j];
        }
    }
    // ---- last tile: weights and latent update
    {
        const int i = n_tiles - 1;
        float pw[16];
        uint32_t pk[8];
#pragma unroll
        for (int j = 0; j < 16; ++j) weight_piece(j, m_use, tsc_cur, pw, pk);
        const uint32_t vbase = ckv_of(i);
        latent_step<0>(vbase, vx, as_bf16x8(u32x4{pk[0], pk[1], pk[2], pk[3]}), oacc, no_fill);
        latent_step<1>(vbase, vx, as_bf16x8(u32x4{pk[4], pk[5], pk[6], pk[7]}), oacc, no_fill);
    }

    // ---- epilogue: sums of the head's two lanes, normalised partial + lse
    const float l_tot = pair_sum(l_run);
    if (l_tot == 0.f) {                                  // no visible position in this split
        if (kh == 0 && g2 == 0) lse_part[out_row] = -INFINITY;
        return;
    }
    const float norm = kFp8 ? l_tot : pair_sum(lw_run);
    const float inv = 1.f / norm;
    const int64_t dst = out_row * kDc + kh * 256;
    // oacc[blk][j]: head t32, latent 256kh + 32*blk + 8*(j/4) + 4*g2 + j%4
#pragma unroll
    for (int blk = 0; blk < 8; ++blk)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
            const f32x4 v = f32x4{oacc[blk][jq * 4], oacc[blk][jq * 4 + 1], oacc[blk][jq * 4 + 2],
                                  oacc[blk][jq * 4 + 3]} * inv;
            store_part4(o_part, p.part_dtype, dst + blk * 32 + jq * 8 + g2 * 4, v);
        }
    if (kh == 0 && g2 == 0) lse_part[out_row] = (m_ref + __builtin_amdgcn_logf(l_tot)) * kLn2;
}

template <bool kFp8, int KH>
__device__ __forceinline__ void decode_wave(
    char *smem, const mla_params_t &p, int part, int rg, const uint16_t *__restrict__ q_abs,
    const uint16_t *__restrict__ q_rope, const void *__restrict__ c_kv, const uint16_t *__restrict__ k_pe,
    const float *__restrict__ kv_scale, const int32_t *__restrict__ block_table,
    const int32_t *__restrict__ seq_lens, void *__restrict__ o_part, float *__restrict__ lse_part) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = p.num_splits;
    bool first = true;
    // slots [c0, c1) of every row of this row group of sequence b: empty
    auto fill = [&](int b, int c0, int c1) {
        const int64_t row = (static_cast<int64_t>(b) * p.Sq * p.H) + rg * kRows + wave * 16 + (lane >> 2);
        for (int c = c0 + (lane & 3); c < c1; c += 4) lse_part[row * S + c] = -INFINITY;
    };
    auto run = [&](const Segment &seg) {
        if (seg.pa >= seg.pb) {                        // an empty part inside the sequence's range
            if (seg.c < S) fill(seg.b, seg.c, seg.c + 1);
        } else if (seg.c < S) {
            if (!first) barrier_lds();                 // the previous segment's LDS reads are done
            first = false;
            attend_segment<kFp8, KH>(smem, p, q_abs, q_rope, c_kv, k_pe, kv_scale,
                                     block_table + static_cast<int64_t>(seg.b) * p.max_pages,
                                     seq_lens[seg.b], seg, rg, o_part, lse_part);
        } else if (threadIdx.x == 0) {
            raise_error(MLA_DEVERR_SPLITS);            // num_splits below the plan's bound
        }
        if (seg.last) fill(seg.b, seg.c + 1, S);       // slots after the last split carry no weight
    };
    for_each_segment(p, seq_lens, part, run, fill);
}

template <bool kFp8>
__global__ __launch_bounds__(kThreads, 1) void decode_mfma_kernel(
    const mla_params_t p, const uint16_t *__restrict__ q_abs, const uint16_t *__restrict__ q_rope,
    const void *__restrict__ c_kv, const uint16_t *__restrict__ k_pe,
    const float *__restrict__ kv_scale, const int32_t *__restrict__ block_table,
    const int32_t *__restrict__ seq_lens, void *__restrict__ o_part, float *__restrict__ lse_part) {
    __shared__ __attribute__((aligned(1024))) char smem[kFp8 ? kSmemFp8 : kSmemBf16];
    // workgroup -> (part, row group rg); parts are spread over the 8 XCDs, the row
    // groups of one part share an XCD
    const int n_rg = (p.Sq * p.H) / kRows;
    const int q = blockIdx.x >> 3;
    const int rg = q % n_rg;
    const int part = (q / n_rg) * 8 + (blockIdx.x & 7);
    const int n_parts = p.num_parts > 0 ? p.num_parts : p.B * p.num_splits;
    if (part >= n_parts) return;                       // grid rounded up to 8 XCDs
    if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & 1)
        decode_wave<kFp8, 1>(smem, p, part, rg, q_abs, q_rope, c_kv, k_pe, kv_scale, block_table, seq_lens,
                             o_part, lse_part);
    else
        decode_wave<kFp8, 0>(smem, p, part, rg, q_abs, q_rope, c_kv, k_pe, kv_scale, block_table, seq_lens,
                             o_part, lse_part);
}

}  // namespace

bool decode_mfma_supported(const mla_params_t &p) {
    if (p.flags & MLA_FLAG_GENERIC) return false;
    if (p.d_c != kDc || p.d_r != kDr || p.page_size != kPage) return false;
    if (p.latent_dtype != MLA_BF16 || p.q_dtype != MLA_BF16 || p.pe_dtype != MLA_BF16) return false;
    if (p.kv_dtype != MLA_BF16 && p.kv_dtype != MLA_FP8_E4M3) return false;
    if (p.H % 32 != 0 || (p.Sq * p.H) % kRows != 0) return false;
    return true;
}

hipError_t launch_decode_mfma(const mla_params_t &p, const void *q_abs, const void *q_rope,
                              const void *c_kv, const void *k_pe, const float *kv_scale,
                              const int32_t *block_table, const int32_t *seq_lens,
                              void *o_part, float *lse_part, hipStream_t stream) {
    const int64_t parts = p.num_parts > 0 ? p.num_parts : static_cast<int64_t>(p.B) * p.num_splits;
    const int64_t n_rg = (static_cast<int64_t>(p.Sq) * p.H) / kRows;
    const int64_t blocks = ((parts + 7) / 8) * 8 * n_rg;
    const auto qa = static_cast<const uint16_t *>(q_abs);
    const auto qr = static_cast<const uint16_t *>(q_rope);
    const auto kp = static_cast<const uint16_t *>(k_pe);
    // a bf16 cache runs on the eight-wave kernel (kernels_decode8.hip); this one
    // serves the e4m3 cache
    if (p.kv_dtype != MLA_FP8_E4M3) return hipErrorInvalidValue;
    hipLaunchKernelGGL(decode_mfma_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream,
                       p, qa, qr, c_kv, kp, kv_scale, block_table, seq_lens, o_part, lse_part);
    return hipGetLastError();
}

hipError_t take_errors_decode_mfma(uint32_t *bits) { return take_unit_errors(bits); }

}  // namespace mla
