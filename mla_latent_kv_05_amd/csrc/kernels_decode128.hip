// mla_decode_splitkv for the DeepSeek-V3 head shapes (d_c = 512, d_r = 64,
// pages of 64 tokens): one workgroup of four waves per work part and row group
// of 128 query rows, gfx950 / CDNA4.
//
// What is computed ("MLA Matrix Absorption" sec. 4.1-4.2; "DeepSeek-MLA-Principle"
// sec. 2 and matrix absorption 3)): every head of a sequence attends to the same
// cached latent row c_t and RoPE key k_pe_t (the MQA form of the absorbed
// computation), so for a tile of 32 cache tokens the scores of 32 heads are a
// dense [32 x 576] x [576 x 32] product and their latent update a dense
// [512 x 32] x [32 x 32] product, both on v_mfma_f32_32x32x16_bf16.
//
// Work decomposition
//   workgroup  4 waves; wave w owns the 32 query rows 32w .. 32w+31 of its row
//              group (at H = 128 and one new token: heads 32w .. 32w+31) from end
//              to end: scores over all 576 dims, softmax, and the latent sum over
//              all 512 columns.  No partial result crosses waves; the waves share
//              only the cache tiles in LDS.  Per wave: the 36 query operands in
//              144 VGPRs, the 512 x 32 latent accumulator in 256 AGPRs.
//   row group  128 query rows (s, h) of one sequence; a page is copied into LDS
//              once per row group, so at Sq = 1 (128 rows per token) once in all.
//   work part  as for every attention kernel here (decode_common.h): a fixed
//              split, or one of num_parts equal shares of the batch's pages.
//   grid       parts x row groups; the row groups of one part share an XCD.
//   pipeline   32-token tiles in a 4-stage LDS ring, copied global -> LDS by
//              buffer_load ... lds with the non-temporal hint (the cache is read
//              once per step), two tiles ahead.  Iteration t runs the score
//              MFMAs of tile t, then the latent MFMAs of tile t-1 with the softmax
//              of tile t issued between them; one workgroup barrier per tile.
//   scores     S^T[token, head] = K[token, k] . Q^T[k, head]: K from LDS (A
//              operand), the query rows in registers (B operand).  MFMA row x
//              holds tile token tok_of(x) (bits 2 and 3 of x exchanged), which
//              puts every lane's weights exactly where the latent product wants
//              its B operand.
//   softmax    online, exp2 domain; a head's 32 scores sit in lanes l and l^32.
//              The reference maximum is raised (and O rescaled) only when a score
//              exceeds it by more than 2^8.
//   latent PV  O^T[latent, head] += V^T[latent, token] . P^T[token, head], V^T by
//              transposing LDS reads (ds_read_b64_tr_b16).
//   output     the normalised partial O_c and its log-sum-exp per row.
//
// LDS layout of a stage (38 KiB): 32 latent rows at a stride of 1088 bytes (1 KiB
// of data and 64 bytes of padding), then 32 RoPE rows of 128 bytes.  The 16-byte
// chunk c of latent row r sits at chunk position c ^ ((r / 4) % 4), and chunk c
// (< 8) of RoPE row r at c ^ ((r / 2) % 8).  With the padding, the rows of a
// 16-row block start in four different bank quads; together with the swizzle the
// 16 rows a 16-lane group reads for one K operand fill 16 distinct bank quads, and
// so do the 4 rows x 64 bytes of a half-wave's transposing V read.  Both read
// patterns are free of bank conflicts, every operand address is a per-lane base
// plus a constant, and a copy instruction still fills one whole row.
#include <hip/hip_runtime.h>
#include <math.h>

#include <type_traits>

#include "decode_common.h"

namespace mla {
namespace {

using namespace gfx;
using namespace dec;

constexpr int kThreads = 256;
constexpr int kRows = kDecodeRowsPerGroup;              // 128 query rows: four waves of 32
constexpr int kStages = 4;
constexpr int kLRow = kCkvRow + 64;                     // LDS stride of a latent row
constexpr int kStageKpe = kTile * kLRow;                // 34816: RoPE rows of a stage
constexpr int kStage = kStageKpe + kTileKpe;            // 38912
constexpr int kSmemStages = kStages * kStage;           // 155648
constexpr int kSmem = kSmemStages + 8 * 1024;           // + one buffer of the weights (8 slots of 1 KiB)
constexpr int kSteps = 36;                              // score k-steps: 576 / 16
constexpr int kCopies = 9;                              // copy instructions per wave per tile
constexpr float kSlack = 64.f;                          // log2 units a score may exceed the reference by
constexpr int kORow = 256 * 4 + 16;                     // LDS stride of an output row (fp32, padded)
constexpr int kORowBf16 = 256 * 2 + 16;                 // ... bf16
constexpr int kOutArea = 32 * kORow;                    // a wave's output area: one head block
static_assert(4 * kOutArea <= kSmemStages, "output areas inside the stages");
static_assert(kSmem <= 160 * 1024, "LDS budget");
static_assert(kRows == 128, "four waves of 32 rows");

__device__ __forceinline__ int tok_of(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }
// swizzle of the 16-byte chunks of latent row r
__device__ __forceinline__ int lat_swz(int r) { return (r >> 2) & 3; }
// ... of RoPE row r
__device__ __forceinline__ int rope_swz(int r) { return (r >> 1) & 7; }

// ---------------------------------------------------------------------------
// Copies (global -> LDS), non-temporal.  One instruction fills 1 KiB of LDS:
// lane i's 16 bytes from base + soff + voff_i land at M0 + 16 i.
// ---------------------------------------------------------------------------
// The buffer descriptor of a copy source (base address, byte count; raw buffer) is
// built once per tile in SGPRs; each copy then sets M0 and issues one instruction.
__device__ __forceinline__ u32x4 copy_rsrc(const void *base, uint32_t bytes) {
    return u32x4{lo32(base), hi32(base) & 0xffffu, static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(bytes)), 0x20000u};
}
// kNt: non-temporal (the bf16 stream, read once; the e4m3 stream is read again by
// the other row groups of a part at Sq > 1, and its loads without the hint measured
// 3 % faster there, 6 % slower for bf16 at Sq = 1)
template <bool kNt = true>
__device__ __forceinline__ void copy_1k(const u32x4 &rsrc, uint32_t l, uint32_t soff, uint32_t v) {
    // (one wait state between the M0 write and the copy that reads it)
    if constexpr (kNt)
        asm volatile("s_mov_b32 m0, %[l]\n\ts_nop 0\n\tbuffer_load_dwordx4 %[v], %[r], %[so] offen nt lds"
                     :: [r] "s"(rsrc), [l] "s"(__builtin_amdgcn_readfirstlane(l)),
                        [so] "s"(__builtin_amdgcn_readfirstlane(soff)), [v] "v"(v)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %[l]\n\ts_nop 0\n\tbuffer_load_dwordx4 %[v], %[r], %[so] offen lds"
                     :: [r] "s"(rsrc), [l] "s"(__builtin_amdgcn_readfirstlane(l)),
                        [so] "s"(__builtin_amdgcn_readfirstlane(soff)), [v] "v"(v)
                     : "memory", "m0");
}

// One instruction copying 256 bytes: lane i's 4 bytes from base + soff + voff_i land at
// M0 + 4 i (lanes past the buffer's end read zeros).
__device__ __forceinline__ void copy_256(const u32x4 &rsrc, uint32_t l, uint32_t soff, uint32_t v) {
    asm volatile("s_mov_b32 m0, %[l]\n\ts_nop 0\n\tbuffer_load_dword %[v], %[r], %[so] offen lds"
                 :: [r] "s"(rsrc), [l] "s"(__builtin_amdgcn_readfirstlane(l)),
                    [so] "s"(__builtin_amdgcn_readfirstlane(soff)), [v] "v"(v)
                 : "memory", "m0");
}

// LDS layout by cache type.  bf16: 4 stages of 38 KiB, weight buffer 0 in the stage
// row padding, buffer 1 after the stages.  e4m3: 3 bf16 stages (filled by the
// conversion of the raw codes and by the RoPE copies), 2 raw stages (32 rows of 512
// codes, then each wave's copy of the 32 token scales), buffer 0's slots 6 and 7
// (there is no fourth stage's padding), then buffer 1.
template <bool kFp8>
struct Lds {
    static constexpr int kStages = kFp8 ? 3 : 4;
    static constexpr int kRawCodes = kTile * kDc;                   // 16384
    static constexpr int kRawStage = kRawCodes + 4 * 256;
    static constexpr int kRawBase = kStages * kStage;
    static constexpr int kW0Extra = kRawBase + 2 * kRawStage;
    static constexpr int kW1Base = kFp8 ? kW0Extra + 2048 : kSmemStages;
    static constexpr int kEnd = kW1Base + 8192;
    static_assert(kEnd <= kSmem, "LDS budget");
};

// s_waitcnt lgkmcnt(n) that the compiler sees (it then adds no wait of its own for
// the LDS reads it covers); vmcnt and expcnt are left at their maxima
template <int N>
__device__ __forceinline__ void wait_lgkm() {
    static_assert(N >= 0 && N < 16, "lgkmcnt range");
    __builtin_amdgcn_s_waitcnt(0xC07F | (N << 8));
}

// The score product's MFMAs as inline asm with the accumulator in VGPRs ("v"
// constraints), so that all 256 AGPRs are left to the latent accumulators.  A chain
// on one accumulator needs no wait states between its MFMAs (same destination, same
// operation); score_done() holds back a VALU read of the result that follows the
// last MFMA directly until the MFMA has written it.
__device__ __forceinline__ void score_mfma_first(f32x16 &d, const u32x4 &a, const bf16x8 &b) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void score_mfma(f32x16 &d, const u32x4 &a, const bf16x8 &b) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void score_done(f32x16 &d) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(d));
}

__device__ __forceinline__ bf16x8 tr_op(const v4i16 &lo, const v4i16 &hi) {
    return __builtin_bit_cast(bf16x8, v8i16{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
}

// ---------------------------------------------------------------------------
// One wave's part of one segment.
// ---------------------------------------------------------------------------
template <bool kFp8, bool kPow2>
__device__ __forceinline__ void attend_segment(char *smem, const mla_params_t &p, const uint16_t *__restrict__ q_abs,
                                               const uint16_t *__restrict__ q_rope, const char *__restrict__ c_kv,
                                               const uint16_t *__restrict__ k_pe, const float *__restrict__ kv_scale,
                                               const int32_t *__restrict__ seg_bt,
                                               const Segment &seg, int seq_len, int rg, void *__restrict__ o_part,
                                               float *__restrict__ lse_part) {
    // lane-dependent values are recomputed per segment (opaque to code motion, so
    // that they do not stay live across the segment loop)
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 31, g = lane >> 5;
    const int S = p.num_splits;
    const uint32_t sm = lds_addr(smem);
    using L = Lds<kFp8>;
    constexpr int kNst = L::kStages;

    seq_len = __builtin_amdgcn_readfirstlane(seq_len);
    const int t_begin = __builtin_amdgcn_readfirstlane(seg.pa * kPage);
    const int t_end = __builtin_amdgcn_readfirstlane(min(seg.pb * kPage, seq_len));
    const int n_tiles = __builtin_amdgcn_readfirstlane((t_end - t_begin + kTile - 1) / kTile);
    const int last_valid = __builtin_amdgcn_readfirstlane(t_end - (t_begin + (n_tiles - 1) * kTile));
    const int n_pages = __builtin_amdgcn_readfirstlane(seg.pb - seg.pa);
    const int64_t row_w = static_cast<int64_t>(seg.b) * p.Sq * p.H + rg * kRows + 32 * w;   // first row of the wave
    const int s_q = (rg * kRows + 32 * w) / p.H;                                              // its query position
    const int n_vis = __builtin_amdgcn_readfirstlane(seq_len - p.Sq + 1 + s_q);

    // LDS address of tile t's bf16 stage, made a scalar explicitly (with three stages
    // the compiler otherwise keeps the modulo in vector registers and spills)
    auto stage_addr = [&](int t) -> uint32_t {
        return sm + __builtin_amdgcn_readfirstlane((t % kNst) * kStage);
    };
    // ---- copies: latent rows 8w .. 8w+7 and RoPE rows 8w .. 8w+7 of a tile
    // page list of the segment: lanes hold pages pl_base .. pl_base + 63
    int pl_base = 0;
    int plist = checked_page(p, seg_bt[min(lane, n_pages - 1)]);
    asm volatile("" : "+v"(plist));
    auto tile_page = [&](int t) -> int64_t {
        if ((t >> 1) - pl_base >= 64) {
            // the next 64 pages (a load and its wait in one statement, once per 64 pages;
            // the wait also drains the copies in flight)
            pl_base = t >> 1;
            const int32_t *src = seg_bt + min(pl_base + lane, n_pages - 1);
            asm volatile("global_load_dword %0, %1, off\n\ts_waitcnt vmcnt(0)" : "=v"(plist) : "v"(src) : "memory");
            plist = checked_page(p, plist);
        }
        return __builtin_amdgcn_readlane(plist, (t >> 1) - pl_base);
    };
    // lane offsets of the copies: latent row 8w + i lands whole (64 lanes x 16 B),
    // lane p fetching the logical chunk stored at position p (rows 8w .. 8w+3 and
    // 8w+4 .. 8w+7 share a swizzle); the RoPE instruction covers rows 8w .. 8w+7
    // (8 lanes per row)
    const uint32_t lat_v0 = static_cast<uint32_t>(lane ^ lat_swz(8 * w)) << 4;
    const uint32_t lat_v1 = static_cast<uint32_t>(lane ^ lat_swz(8 * w + 4)) << 4;
    const int rr = 8 * w + (lane >> 3);
    const uint32_t rope_voff = (lane >> 3) * kKpeRow + (((lane & 7) ^ rope_swz(rr)) << 4);
    // copies of tile t, one instruction at a time: i < 8 latent row 8w + i, i = 8 the
    // RoPE rows 8w .. 8w+7.  A tile past the segment's end gets a zero-length buffer:
    // its instructions move nothing, so that every tile issues the same copies and
    // the vmcnt accounting is the same for all of them.  e4m3: the codes of rows
    // 8w .. 8w+7 (two rows per instruction) and the 32 token scales go to the tile's
    // raw stage, the RoPE rows to its bf16 stage.
    struct TileSrc {
        u32x4 ckv, kpe, scl;   // buffer descriptors of the tile's latent rows, RoPE rows, scales
        uint32_t st, raw;      // its bf16 stage and (e4m3) raw stage
    };
    auto tile_src = [&](int t) -> TileSrc {
        const bool real = t < n_tiles;
        const int64_t phys = real ? tile_page(t) : 0;
        const int64_t crow0 = phys * kPage + (t & 1) * kTile;
        constexpr int kRowBytes = kFp8 ? kDc : kCkvRow;
        return TileSrc{copy_rsrc(c_kv + crow0 * kRowBytes, real ? kTile * kRowBytes : 0u),
                       copy_rsrc(k_pe + crow0 * kDr, real ? kTileKpe : 0u),
                       copy_rsrc(kFp8 ? kv_scale + crow0 : nullptr, kFp8 && real ? kTile * 4 : 0u),
                       stage_addr(t), sm + L::kRawBase + (t & 1) * L::kRawStage};
    };
    auto copy_one = [&](const TileSrc &ts, int i) {
        if (i < 8)
            copy_1k(ts.ckv, ts.st + (8 * w + i) * kLRow, (8 * w + i) * kCkvRow, i < 4 ? lat_v0 : lat_v1);
        else
            copy_1k(ts.kpe, ts.st + kStageKpe + w * 1024, w * 1024, rope_voff);
    };
    auto issue_tile = [&](int t) {
        const TileSrc ts = tile_src(t);
#pragma unroll
        for (int i = 0; i < kCopies; ++i) copy_one(ts, i);
    };
    // e4m3: codes copy i < 4 (rows 8w + 2i, 8w + 2i + 1), i = 4 the scales (each wave
    // its own copy); the RoPE rows of a tile separately (rope_copy)
    const uint32_t lane16 = static_cast<uint32_t>(lane) << 4, lane4 = static_cast<uint32_t>(lane) << 2;
    auto raw_copy = [&](const TileSrc &ts, int i) {
        if (i < 4)
            copy_1k<false>(ts.ckv, ts.raw + (8 * w + 2 * i) * kDc, (8 * w + 2 * i) * kDc, lane16);
        else
            copy_256(ts.scl, ts.raw + L::kRawCodes + w * 256, 0u, lane4);
    };
    auto rope_copy = [&](const TileSrc &ts) { copy_1k<false>(ts.kpe, ts.st + kStageKpe + w * 1024, w * 1024, rope_voff); };
    // e4m3 conversion of rows 8w .. 8w+7 of tile t from its raw stage into its bf16
    // stage: bf16(float(code) * scale), one fp32 product rounded to nearest even (the
    // value mla_expand_kv gives).  One row at a time: lane l reads codes 8l .. 8l+7 of
    // the row (512 contiguous bytes over the wave) and writes their bf16 values as the
    // row's logical 16-byte chunk l (a permutation of the row's chunks over the
    // lanes), so that neither access has bank conflicts; conv_read issues the reads of
    // row 8w + j, conv_write converts and stores it.
    struct ConvIn {
        u32x2 codes;
        float scale;
    };
    auto conv_read = [&](int t, int j) -> ConvIn {
        const uint32_t raw = sm + L::kRawBase + (t & 1) * L::kRawStage;
        return ConvIn{lds_load<u32x2>(raw + (8 * w + j) * kDc + 8 * lane),
                      lds_load<float>(raw + L::kRawCodes + w * 256 + (8 * w + j) * 4)};
    };
    // kPow2 (MLA_FLAG_POW2_SCALE: the caller states that every valid row's scale is a
    // power of two, as mla_append_kv writes them): code * scale is then exact in bf16,
    // and gfx950's MX-style conversion applies such a scale itself, one instruction
    // per two codes.  It uses only the scale's exponent, so any other scale needs
    // the widening, the two products and the rounding.  The MLA_DEBUG_BOUNDS build
    // checks the statement for the rows it converts (MLA_DEVERR_SCALE).
    auto conv_write = [&](int t, int j, const ConvIn &v) {
        const int r = 8 * w + j;
        u32x4 o;
        if constexpr (kPow2) {
#ifdef MLA_DEBUG_BOUNDS
            const bool valid = t < n_tiles - 1 || (t == n_tiles - 1 && r < last_valid);
            if (valid && lane == 0 && (__float_as_uint(v.scale) & 0x7fffffu) != 0u) raise_error(MLA_DEVERR_SCALE);
#endif
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                o[2 * e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.codes[e], v.scale, false));
                o[2 * e + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.codes[e], v.scale, true));
            }
        } else {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(v.codes[e], false);
                const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(v.codes[e], true);
                o[2 * e] = cvt_pk_bf16(lo[0] * v.scale, lo[1] * v.scale);
                o[2 * e + 1] = cvt_pk_bf16(hi[0] * v.scale, hi[1] * v.scale);
            }
        }
        lds_store<u32x4>(stage_addr(t) + r * kLRow + ((lane ^ lat_swz(r)) << 4), o);
    };
    auto convert_tile = [&](int t) {
#pragma unroll
        for (int j = 0; j < 8; ++j) conv_write(t, j, conv_read(t, j));
    };

    // ---- query operands (B of the score product): k-step k < 32 latent dims
    // 16k + 8g .., k >= 32 RoPE dims 16(k - 32) + 8g .., of row row_w + n
    bf16x8 qreg[kSteps];
    {
        const uint16_t *qa = q_abs + (row_w + n) * kDc + 8 * g;
        const uint16_t *qr = q_rope + (row_w + n) * kDr + 8 * g;
#pragma unroll
        for (int k = 0; k < 32; ++k) qreg[k] = *reinterpret_cast<const bf16x8 *>(qa + 16 * k);
#pragma unroll
        for (int k = 0; k < 4; ++k) qreg[32 + k] = *reinterpret_cast<const bf16x8 *>(qr + 16 * k);
    }

    // ---- operand addresses (relative to a stage)
    // K operand, lane (n, g): MFMA row n holds token r = tok_of(n); step k = 2m + k0
    // (k < 32) reads latent chunk 2k + g at kx[k0] + 64 m, RoPE step k'' at kp[k'']
    const int r = tok_of(n);
    uint32_t kx[2], kp[4];
#pragma unroll
    for (int k0 = 0; k0 < 2; ++k0) kx[k0] = r * kLRow + (((2 * k0 + g) ^ lat_swz(r)) << 4);
#pragma unroll
    for (int k = 0; k < 4; ++k) kp[k] = kStageKpe + r * kKpeRow + (((2 * k + g) ^ rope_swz(r)) << 4);
    // V^T operand of column block cb (of the wave's half kh: latent columns 256kh ..),
    // k-step kk, half h: lane (group gq of 16, index a in it) addresses row
    // 16kk + 8g + a/4 + 4h, latent columns 32cb + 16(gq & 1) + 4(a % 4) .. + 3, at
    // vx[h] + 64 cb + 16 kLRow kk
    const int kh = w & 1, pr = w >> 1;                  // column half and head-block pair of the latent sum
    uint32_t vx[2];
    {
        const int a = lane & 15, hh = (lane >> 4) & 1;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = 8 * g + (a >> 2) + 4 * h;
            const int c = 2 * hh + ((a & 3) >> 1);                  // chunk within the block's four
            vx[h] = row * kLRow + ((c ^ lat_swz(row)) << 4) + (a & 1) * 8 + kh * 512;
        }
    }
    // weights (B operands of the latent product) of head block hb and k-step kk:
    // slot s = 2hb + kk of 64 cells of 16 bytes, lane l's operand in cell l.  Buffer 0
    // is spread over the padding of the stage rows (slot s: rows 16(s & 1) .. +15 of
    // stage s / 2, four cells per row); buffer 1 follows the stages.
    auto cell = [&](int buf, int slot, int idx) -> uint32_t {
        if (buf) return sm + L::kW1Base + slot * 1024 + idx * 16;
        if (kFp8 && slot >= 2 * kNst) return sm + L::kW0Extra + (slot - 2 * kNst) * 1024 + idx * 16;
        return sm + (slot >> 1) * kStage + (16 * (slot & 1) + (idx >> 2)) * kLRow + kCkvRow + (idx & 3) * 16;
    };
    auto pslot = [&](int buf, int slot) -> uint32_t { return cell(buf, slot, lane); };

    // ---- softmax state.  The reference maximum of a row is fixed for the whole
    // segment: the maximum of its first tile with a visible position.  Weights are
    // exp2 of the scores above it (in log2 units) and may exceed 1, so O never
    // needs rescaling.  A score more than kSlack above the reference would risk
    // overflow: the segment is then computed again with the reference set to the
    // maximum of all its scores, found in the first pass (a second pass is needed
    // only for scores that grow by more than 2^64 along a split).
    const float zscale = p.scale * kLog2e;
    const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);
    float m_ref = -INFINITY;   // reference maximum (log2 domain), equal in lanes n and n^32
    float m_all = -INFINITY;   // maximum of the scores seen
    float l_run = 0.f;         // this lane's share of the sum of exp2 weights (-> lse)
    float lw_run = 0.f;        // ... of the weights as rounded to bf16 (-> normalisation of O)
    bool over = false;         // a score above m_ref + kSlack
    f32x16 oacc[2][8];         // O^T[256kh + 32cb + D row, head n of block 2pr + j]

    // ---- score product of tile t (its stage has landed): 36 MFMAs on one
    // accumulator, each K operand read eight MFMAs ahead
    auto score = [&](int t, const TileSrc *cp, const TileSrc *rp = nullptr) -> f32x16 {
        const uint32_t st = stage_addr(t);
        // e4m3: the conversion of tile t + 1 (row 8w + j read at step 4j + 1, converted
        // and stored at 4j + 3), the raw copies of tile t + 2 and the RoPE copy of tile t + 1
        // (a tile past the end is converted too: its stage is not read again in the
        // segment, and its zero-length copies move nothing)
        ConvIn cv{};
        auto fp8_step = [&](auto K) {
            constexpr int k = decltype(K)::value;
            if constexpr (k % 4 == 1 && k < 32) {
                cv = conv_read(t + 1, k / 4);
            } else if constexpr (k % 4 == 3 && k < 32) {
                conv_write(t + 1, k / 4, cv);
            } else if constexpr (k % 4 == 2 && k <= 18) {
                raw_copy(*cp, (k - 2) / 4);
            } else if constexpr (k == 22) {
                rope_copy(*rp);
            }
        };
        const uint32_t kb0 = st + kx[0], kb1 = st + kx[1];
        uint32_t kpb[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) kpb[k] = st + kp[k];
        f32x16 acc;
        u32x4 a[kSteps];
#define D128_KADDR(k) ((k) < 32 ? ((k) & 1 ? kb1 : kb0) + ((k) >> 1) * 64 : kpb[(k) - 32])
#define D128_KREAD(k) a[k] = ld128(D128_KADDR(k));
        // groups of four MFMAs; the reads of group g+2 are issued during group g, and
        // one wait per group covers its four operands
        D128_KREAD(0) D128_KREAD(1) D128_KREAD(2) D128_KREAD(3)
        D128_KREAD(4) D128_KREAD(5) D128_KREAD(6) D128_KREAD(7)
        pin();
#define D128_KSTEP(k)                                                 \
        if constexpr ((k) == 0) score_mfma_first(acc, a[k], qreg[k]); \
        else score_mfma(acc, a[k], qreg[k]);                          \
        if constexpr ((k) + 8 < kSteps) D128_KREAD((k) + 8)           \
        if constexpr (kFp8) fp8_step(std::integral_constant<int, (k)>{}); \
        else if constexpr ((k) % 4 == 2) if (cp) copy_one(*cp, (k) / 4); \
        pin();
#define D128_KGROUP(g)                                                \
        if constexpr (4 * (g) + 4 < kSteps) wait_lgkm<4>();           \
        else wait_lgkm<0>();                                          \
        D128_KSTEP(4 * (g)) D128_KSTEP(4 * (g) + 1) D128_KSTEP(4 * (g) + 2) D128_KSTEP(4 * (g) + 3)
        D128_KGROUP(0) D128_KGROUP(1) D128_KGROUP(2) D128_KGROUP(3) D128_KGROUP(4) D128_KGROUP(5) D128_KGROUP(6)
        D128_KGROUP(7) D128_KGROUP(8)
#undef D128_KGROUP
#undef D128_KSTEP
#undef D128_KREAD
#undef D128_KADDR
        return acc;
    };

    // ---- mask of tile t: positions past the causal bound or the sequence end
    auto mask = [&](int t, f32x16 &sc) {
        const int tbase = t_begin + t * kTile;
        if (tbase + kTile > n_vis) {
            score_done(sc);                        // the last MFMA has written the scores
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int i = e >> 2, j = e & 3;
                const int tok = 16 * (i >> 1) + 8 * g + 4 * (i & 1) + j;
                if (tbase + tok >= n_vis) sc[e] = -INFINITY;
            }
        }
    };

    // ---- softmax of masked scores -> bf16 weights (B operands of the two latent
    // k-steps) and the running sums, cut into 17 steps so that they can be slotted
    // between the latent MFMAs of the previous tile: step k of Softmax::step
    struct Softmax {
        f32x16 sc;
        int buf;               // weight buffer of the tile
        float m[5], mloc, m_use;
        float pe[16];
        uint32_t pk[8];
    };
    auto sm_step = [&](Softmax &x, auto K, u32x4 &pb0, u32x4 &pb1) {
        constexpr int k = decltype(K)::value;
        if constexpr (k == 0) {
            x.m[0] = fmaxf(fmaxf(x.sc[0], x.sc[1]), x.sc[2]);
            x.m[1] = fmaxf(fmaxf(x.sc[3], x.sc[4]), x.sc[5]);
        } else if constexpr (k == 1) {
            x.m[2] = fmaxf(fmaxf(x.sc[6], x.sc[7]), x.sc[8]);
            x.m[3] = fmaxf(fmaxf(x.sc[9], x.sc[10]), x.sc[11]);
        } else if constexpr (k == 2) {
            x.m[4] = fmaxf(fmaxf(x.sc[12], x.sc[13]), x.sc[14]);
            x.m[0] = fmaxf(fmaxf(x.m[0], x.m[1]), x.m[2]);
        } else if constexpr (k == 3) {
            x.mloc = fmaxf(fmaxf(x.m[0], x.m[3]), fmaxf(x.m[4], x.sc[15]));
        } else if constexpr (k == 4) {
            const float ml = pair_max(x.mloc) * zscale;   // zscale > 0: the maximum commutes with it
            m_all = fmaxf(m_all, ml);
            m_ref = m_ref == -INFINITY ? ml : m_ref;      // the first tile with a visible position
            over |= ml > m_ref + kSlack;
            x.m_use = m_ref == -INFINITY ? 0.f : m_ref;   // nothing visible yet: weights 0
        } else if constexpr (k >= 5 && k < 13) {
            constexpr int e = 2 * (k - 5);
            x.pe[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x.sc[e], zscale, -x.m_use));
            x.pe[e + 1] = __builtin_amdgcn_exp2f(__builtin_fmaf(x.sc[e + 1], zscale, -x.m_use));
        } else if constexpr (k == 13) {
            l_run += ((x.pe[0] + x.pe[1]) + (x.pe[2] + x.pe[3])) + ((x.pe[4] + x.pe[5]) + (x.pe[6] + x.pe[7]));
        } else if constexpr (k == 14) {
            l_run += ((x.pe[8] + x.pe[9]) + (x.pe[10] + x.pe[11])) + ((x.pe[12] + x.pe[13]) + (x.pe[14] + x.pe[15]));
        } else if constexpr (k == 15 || k == 16) {
            constexpr int h0 = 4 * (k - 15);
#pragma unroll
            for (int h = h0; h < h0 + 4; ++h) {
                x.pk[h] = cvt_pk_bf16(x.pe[2 * h], x.pe[2 * h + 1]);
                // the sum of the weights exactly as the latent product sees them
                lw_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x.pk[h]), ones, lw_run, false);
            }
            if constexpr (k == 15) pb0 = u32x4{x.pk[0], x.pk[1], x.pk[2], x.pk[3]};
            else pb1 = u32x4{x.pk[4], x.pk[5], x.pk[6], x.pk[7]};
            // the partner wave of the latent sum reads them in the next iteration
            lds_store<u32x4>(pslot(x.buf, 2 * w + (k - 15)), k == 15 ? pb0 : pb1);
        }
    };
    constexpr int kSmSteps = 17;
    auto softmax = [&](Softmax &x, u32x4 &pb0, u32x4 &pb1) {
#define D128_SM(k) sm_step(x, std::integral_constant<int, k>{}, pb0, pb1);
        D128_SM(0) D128_SM(1) D128_SM(2) D128_SM(3) D128_SM(4) D128_SM(5) D128_SM(6) D128_SM(7) D128_SM(8)
        D128_SM(9) D128_SM(10) D128_SM(11) D128_SM(12) D128_SM(13) D128_SM(14) D128_SM(15) D128_SM(16)
#undef D128_SM
    };

    // ---- latent update of the wave's 64 heads x 256 columns with the weights of
    // tile t (stage of tile t; weights of both head blocks read from buffer `buf`):
    // 16 V reads (pairs), each feeding the MFMAs of both head blocks, read three
    // pairs ahead; with `x`, the softmax steps of the next tile are issued between
    // the MFMAs (step k after MFMA k + 2)
    auto latent = [&](int t, int buf, auto WithSm, Softmax &x, u32x4 &pn0, u32x4 &pn1) {
        constexpr bool kWithSm = decltype(WithSm)::value;
        const uint32_t st = stage_addr(t);
        const uint32_t vb0 = st + vx[0], vb1 = st + vx[1];
        u32x4 pw[2][2];                                  // [head block][k-step]
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) pw[j][kk] = ld128(pslot(buf, 2 * (2 * pr + j) + kk));
        v4i16 lo[16], hi[16];
#define D128_VREAD(j)                                                                        \
        {                                                                                    \
            constexpr int kk = (j) >> 3, cb = (j) & 7;                                       \
            lo[j] = ld_tr16(vb0 + cb * 64 + kk * 16 * kLRow);                                \
            hi[j] = ld_tr16(vb1 + cb * 64 + kk * 16 * kLRow);                                \
        }
#define D128_SM(m)                                                                           \
            if constexpr (kWithSm && (m) >= 2 && (m) - 2 < kSmSteps)                         \
                sm_step(x, std::integral_constant<int, (m) - 2>{}, pn0, pn1);
#define D128_PV(j)                                                                           \
        {                                                                                    \
            constexpr int kk = (j) >> 3, cb = (j) & 7;                                       \
            const bf16x8 v = tr_op(lo[j], hi[j]);                                            \
            oacc[0][cb] = mfma32(v, as_bf16x8(pw[0][kk]), oacc[0][cb]);                      \
            if constexpr ((j) + 3 < 16) D128_VREAD((j) + 3)                                  \
            D128_SM(2 * (j))                                                                 \
            pin();                                                                           \
            oacc[1][cb] = mfma32(v, as_bf16x8(pw[1][kk]), oacc[1][cb]);                      \
            D128_SM(2 * (j) + 1)                                                             \
            pin();                                                                           \
        }
        // one wait per V pair covers its two reads (and, before the first, the weights)
#define D128_PVW(j)                                                                          \
        if constexpr ((j) + 3 < 16) wait_lgkm<6>();                                         \
        else if constexpr ((j) + 2 < 16) wait_lgkm<4>();                                    \
        else if constexpr ((j) + 1 < 16) wait_lgkm<2>();                                    \
        else wait_lgkm<0>();                                                                 \
        D128_PV(j)
        D128_VREAD(0) D128_VREAD(1) D128_VREAD(2)
        pin();
        D128_PVW(0) D128_PVW(1) D128_PVW(2) D128_PVW(3) D128_PVW(4) D128_PVW(5) D128_PVW(6) D128_PVW(7)
        D128_PVW(8) D128_PVW(9) D128_PVW(10) D128_PVW(11) D128_PVW(12) D128_PVW(13) D128_PVW(14) D128_PVW(15)
#undef D128_PVW
#undef D128_PV
#undef D128_SM
#undef D128_VREAD
    };

    int xb = 0;                // the weight buffer free at the end of the tile loop
    for (int pass = 0;; ++pass) {
        l_run = 0.f;
        lw_run = 0.f;
        over = false;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int cb = 0; cb < 8; ++cb)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[j][cb][e] = 0.f;

        // ---- the tile loop.  Iteration t: scores of tile t (copies of tile t+2
        // between its MFMAs), then the latent sum of tile t-1 with the softmax of
        // tile t between its MFMAs.  The weights of tile t go to buffer t & 1.
        if constexpr (kFp8) {
            // tile 0's RoPE rows, codes and scales and tile 1's codes and scales in
            // flight; tile 0 converted before its scores
            {
                const TileSrc t0 = tile_src(0), t1 = tile_src(1);
                rope_copy(t0);
#pragma unroll
                for (int i = 0; i < 5; ++i) raw_copy(t0, i);
#pragma unroll
                for (int i = 0; i < 5; ++i) raw_copy(t1, i);
            }
            wait_vmcnt<0>();                             // query loads, tiles 0 and 1 landed
            barrier_lds();
            convert_tile(0);
            barrier_lds();
        } else {
            issue_tile(0);
            issue_tile(1);
            wait_vmcnt<kCopies>();                       // query loads and tile 0 landed
            barrier_lds();
            issue_tile(2);
        }
        {
            Softmax x;
            x.buf = 0;
            if constexpr (kFp8) {
                const TileSrc r1 = tile_src(1), c2 = tile_src(2);   // ascending: tile_page moves forward
                x.sc = score(0, &c2, &r1);               // converts tile 1, copies tiles 1 (RoPE) and 2
            } else {
                x.sc = score(0, nullptr);
            }
            score_done(x.sc);
            mask(0, x.sc);
            u32x4 pn0, pn1;
#define D128_SM(k) sm_step(x, std::integral_constant<int, k>{}, pn0, pn1);
            D128_SM(0) D128_SM(1) D128_SM(2) D128_SM(3) D128_SM(4) D128_SM(5) D128_SM(6) D128_SM(7) D128_SM(8)
            D128_SM(9) D128_SM(10) D128_SM(11) D128_SM(12) D128_SM(13) D128_SM(14) D128_SM(15) D128_SM(16)
#undef D128_SM
        }
        for (int t = 1; t < n_tiles; ++t) {
            Softmax x;
            x.buf = t & 1;
            if constexpr (kFp8) {
                wait_vmcnt<0>();                         // tile t's RoPE rows and tile t+1's codes landed
                barrier_lds();                           // ... and tile t converted, for every wave
                const TileSrc r = tile_src(t + 1), c = tile_src(t + 2);   // ascending (page list window)
                x.sc = score(t, &c, &r);
            } else {
                wait_vmcnt<kCopies>();                   // tile t landed (tile t+1 may be in flight)
                barrier_lds();                           // ... for every wave, and the weights of tile t-1
                const TileSrc next = tile_src(t + 2);
                x.sc = score(t, &next);                  // copies tile t+2 between its MFMAs
            }
            mask(t, x.sc);                               // (softmax reads the scores two MFMAs later)
            u32x4 pn0, pn1;
            latent(t - 1, (t - 1) & 1, std::true_type{}, x, pn0, pn1);
        }
        if (last_valid < kTile) {
            // rows past the sequence end in the last tile: zero, so that their zero
            // weights never meet non-finite values in the latent product.  Each wave
            // clears its own rows once its copies of the tile have landed; other waves
            // may still read them for scores, which are masked there whatever they hold.
            const uint32_t st = stage_addr(n_tiles - 1);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (8 * w + i >= last_valid) lds_store<u32x4>(st + (8 * w + i) * kLRow + 16 * lane, u32x4{0u, 0u, 0u, 0u});
        }
        barrier_lds();                                   // the weights of the last tile (and the zeros)
        {
            Softmax x;
            u32x4 pn0, pn1;
            latent(n_tiles - 1, (n_tiles - 1) & 1, std::false_type{}, x, pn0, pn1);
        }
        // the other weight buffer is free: each wave publishes its per-head
        // normalisation (1 / sum of the weights as rounded; slot hb, cell n) and whether
        // any score exceeded its reference by more than kSlack (slot 4, cell w)
        xb = n_tiles & 1;
        {
            const float l_tot = pair_sum(l_run);
            const float lw_tot = pair_sum(lw_run);
            if (lane < 32) lds_store<float>(cell(xb, w, n), l_tot == 0.f ? 0.f : 1.f / lw_tot);
        }
        {
            // the ballot runs with every lane active (inside `lane == 0` it would see
            // lane 0's flag only)
            const int any_over = __builtin_amdgcn_ballot_w64(over) != 0;
            if (lane == 0) lds_store<int>(cell(xb, 4, w), any_over);
        }
        barrier_lds();
        const int ov = lds_load<int>(cell(xb, 4, 0)) | lds_load<int>(cell(xb, 4, 1)) | lds_load<int>(cell(xb, 4, 2)) |
                       lds_load<int>(cell(xb, 4, 3));
        if (pass == 1 || !__builtin_amdgcn_readfirstlane(ov)) break;
        // second pass: every wave (the waves share the copies), each row with its own
        // maximum as the reference
        m_ref = m_all;
        pl_base = 0;
        plist = checked_page(p, seg_bt[min(lane, n_pages - 1)]);
        wait_vmcnt<0>();
        barrier_lds();
    }

    // ---- output: lse of the wave's head block; O of its 64 heads x 256 columns,
    // normalised by the sums the score waves published.  A lane holds 16 columns of
    // one row in groups of four, so O goes out through LDS: each head block is
    // written to a wave-private area of 32 rows and read back a row at a time, and
    // every store then writes 1 KiB (bf16: 512 bytes) of one row, instead of 32
    // rows x 32 bytes.
    const float inv0 = lds_load<float>(cell(xb, 2 * pr, n));
    const float inv1 = lds_load<float>(cell(xb, 2 * pr + 1, n));
    wait_vmcnt<0>();           // the copies of tiles past the end (zero-length) are done too
    barrier_lds();             // every wave has its sums: the stage area is free
    {
        const float l_tot = pair_sum(l_run);
        if (g == 0)
            lse_part[(row_w + n) * S + seg.c] = l_tot == 0.f ? -INFINITY : (m_ref + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
    const uint32_t ob = sm + w * kOutArea;
    const bool part_bf16 = p.part_dtype == MLA_BF16;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int hb = 2 * pr + j;
        const float inv = j ? inv1 : inv0;
        const int64_t dst = ((static_cast<int64_t>(seg.b) * p.Sq * p.H + rg * kRows + 32 * hb) * S + seg.c) * kDc +
                            256 * kh;
        // oacc[j][cb][4i + e]: latent column 256kh + 32cb + 8i + 4g + e of head n of block hb
        if (part_bf16) {
#pragma unroll
            for (int cb = 0; cb < 8; ++cb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    lds_store<u32x2>(ob + n * kORowBf16 + (32 * cb + 8 * i + 4 * g) * 2,
                                     u32x2{cvt_pk_bf16(oacc[j][cb][4 * i] * inv, oacc[j][cb][4 * i + 1] * inv),
                                           cvt_pk_bf16(oacc[j][cb][4 * i + 2] * inv, oacc[j][cb][4 * i + 3] * inv)});
            // row x of the block: lane l stores columns 4l .. 4l + 3 of the wave's half
            uint16_t *d = static_cast<uint16_t *>(o_part) + dst + 4 * lane;
#pragma unroll
            for (int x = 0; x < 32; ++x)
                *reinterpret_cast<u32x2 *>(d + static_cast<int64_t>(x) * S * kDc) =
                    lds_load<u32x2>(ob + x * kORowBf16 + 8 * lane);
        } else {
#pragma unroll
            for (int cb = 0; cb < 8; ++cb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    lds_store<f32x4>(ob + n * kORow + (32 * cb + 8 * i + 4 * g) * 4,
                                     f32x4{oacc[j][cb][4 * i], oacc[j][cb][4 * i + 1], oacc[j][cb][4 * i + 2],
                                           oacc[j][cb][4 * i + 3]} * inv);
            float *d = static_cast<float *>(o_part) + dst + 4 * lane;
#pragma unroll
            for (int x = 0; x < 32; ++x)
                *reinterpret_cast<f32x4 *>(d + static_cast<int64_t>(x) * S * kDc) =
                    lds_load<f32x4>(ob + x * kORow + 16 * lane);
        }
    }
}

template <bool kFp8, bool kPow2>
__global__ __launch_bounds__(kThreads, 1) void decode128_kernel(
    const mla_params_t p, const uint16_t *__restrict__ q_abs, const uint16_t *__restrict__ q_rope,
    const char *__restrict__ c_kv, const uint16_t *__restrict__ k_pe, const float *__restrict__ kv_scale,
    const int32_t *__restrict__ block_table,
    const int32_t *__restrict__ seq_lens, void *__restrict__ o_part, float *__restrict__ lse_part) {
    __shared__ __attribute__((aligned(1024))) char smem[kSmem];
    // workgroup -> (part, row group rg).  Workgroups are dealt to the 8 XCDs in turn
    // (XCD = blockIdx % 8); each XCD takes a contiguous run of parts, so that the
    // parts of one sequence mostly share an XCD and its L2 serves their query rows
    // after the first load, and the row groups of one part share an XCD too.
    const int n_rg = (p.Sq * p.H) / kRows;
    const int n_parts = p.num_parts > 0 ? p.num_parts : p.B * p.num_splits;
    const int per_xcd = (n_parts + 7) / 8;
    const int qq = blockIdx.x >> 3;
    const int rg = qq % n_rg;
    const int part = (blockIdx.x & 7) * per_xcd + qq / n_rg;
    if (part >= n_parts) return;                       // grid rounded up to 8 XCDs
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = p.num_splits;
    bool first = true;
    // slots [c0, c1) of every row of this row group of sequence b: empty
    auto fill = [&](int b, int c0, int c1) {
        const int64_t row = static_cast<int64_t>(b) * p.Sq * p.H + rg * kRows + 32 * w + (lane >> 1);
        for (int c = c0 + (lane & 1); c < c1; c += 2) lse_part[row * S + c] = -INFINITY;
    };
    auto run = [&](const Segment &seg) {
        if (seg.pa >= seg.pb) {                        // an empty part inside the sequence's range
            if (seg.c < S) fill(seg.b, seg.c, seg.c + 1);
        } else if (seg.c < S) {
            if (!first) barrier_lds();                 // the previous segment's LDS reads are done
            first = false;
            wait_vmcnt<0>();                           // its stores too (the copy waits count from here)
            attend_segment<kFp8, kPow2>(smem, p, q_abs, q_rope, c_kv, k_pe, kv_scale,
                                 block_table + static_cast<int64_t>(seg.b) * p.max_pages + seg.pa, seg,
                           seq_lens[seg.b], rg, o_part, lse_part);
        } else if (threadIdx.x == 0) {
            raise_error(MLA_DEVERR_SPLITS);            // num_splits below the plan's bound
        }
        if (seg.last) fill(seg.b, seg.c + 1, S);       // slots after the last split carry no weight
    };
    for_each_segment(p, seq_lens, part, run, fill);
}

}  // namespace

DecodeKernel decode_kernel_for(const mla_params_t &p) {
    const bool k128 = decode128_supported(p), k8 = decode8_supported(p);
    if (k128 && (p.flags & MLA_FLAG_ROWS128)) return DecodeKernel::k128;
    if (k8 && (p.flags & MLA_FLAG_ROWS64)) return DecodeKernel::k8;
    if (k128 && k8) {
        const int64_t parts = p.num_parts > 0 ? p.num_parts : static_cast<int64_t>(p.B) * p.num_splits;
        return parts * ((static_cast<int64_t>(p.Sq) * p.H) / kRows) <= kSmallGrid128 ? DecodeKernel::k8
                                                                                        : DecodeKernel::k128;
    }
    return k128 ? DecodeKernel::k128 : k8 ? DecodeKernel::k8 : DecodeKernel::kMfma64;
}

int decode_rows_per_workgroup(const mla_params_t &p) {
    return decode_kernel_for(p) == DecodeKernel::k128 ? kRows : kDecodeRowsPerBlock;
}

bool decode128_supported(const mla_params_t &p) {
    return decode_mfma_supported(p) && (p.kv_dtype == MLA_BF16 || p.kv_dtype == MLA_FP8_E4M3) &&
           (p.Sq * p.H) % kRows == 0;
}

hipError_t launch_decode128(const mla_params_t &p, const void *q_abs, const void *q_rope, const void *c_kv,
                            const void *k_pe, const float *kv_scale, const int32_t *block_table,
                            const int32_t *seq_lens, void *o_part, float *lse_part, hipStream_t stream) {
    const int64_t parts = p.num_parts > 0 ? p.num_parts : static_cast<int64_t>(p.B) * p.num_splits;
    const int64_t n_rg = (static_cast<int64_t>(p.Sq) * p.H) / kRows;
    const dim3 grid(static_cast<unsigned>(((parts + 7) / 8) * 8 * n_rg));
    const auto qa = static_cast<const uint16_t *>(q_abs);
    const auto qr = static_cast<const uint16_t *>(q_rope);
    const auto kv = static_cast<const char *>(c_kv);
    const auto kp = static_cast<const uint16_t *>(k_pe);
    if (p.kv_dtype == MLA_FP8_E4M3 && (p.flags & MLA_FLAG_POW2_SCALE))
        hipLaunchKernelGGL((decode128_kernel<true, true>), grid, dim3(kThreads), 0, stream, p, qa, qr, kv, kp,
                           kv_scale, block_table, seq_lens, o_part, lse_part);
    else if (p.kv_dtype == MLA_FP8_E4M3)
        hipLaunchKernelGGL((decode128_kernel<true, false>), grid, dim3(kThreads), 0, stream, p, qa, qr, kv, kp,
                           kv_scale, block_table, seq_lens, o_part, lse_part);
    else
        hipLaunchKernelGGL((decode128_kernel<false, false>), grid, dim3(kThreads), 0, stream, p, qa, qr, kv, kp,
                           kv_scale, block_table, seq_lens, o_part, lse_part);
    return hipGetLastError();
}

hipError_t take_errors_decode128(uint32_t *bits) { return take_unit_errors(bits); }

}  // namespace mla
