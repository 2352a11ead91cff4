// bf16 MFMA kernels for absorbed-MLA decode at the DeepSeek-V3 head shapes
// (d_c = 512 latent, d_r = 64 RoPE key, page = 64 tokens), gfx950 / CDNA4.
//
// Attention ("MLA Matrix Absorption" sec. 4.1-4.2; "DeepSeek-MLA-Principle"
// sec. 2 and matrix absorption 3)): every head of a sequence attends to the
// same latent cache row c_t (the MQA form of the absorbed computation), so for
// a tile of 32 tokens the scores of 32 heads are a dense [32 x 576] x [576 x 32]
// product and the latent update a dense [512 x 32] x [32 x 32] product.  Both
// run on v_mfma_f32_32x32x16_bf16.
//
// Work decomposition of mla_decode_splitkv
//   workgroup = 4 waves = 64 query rows (s, h) of one sequence b and one
//               split c.  Waves 2p and 2p+1 form a pair that owns 32 heads of
//               one query row s:
//                 scores: each wave contracts half of the 576 dims (wave 0 of
//                         the pair latent 0..287, wave 1 latent 288..511 and
//                         the RoPE key); the fp32 partial scores are swapped
//                         through LDS and added, so both hold the full scores;
//                 softmax: computed identically by both waves;
//                 latent: each wave accumulates half of the 512 latent columns.
//               Per wave this keeps 72 VGPRs of query and 128 AGPRs of output.
//   grid      = B * num_splits * (Sq*H/64) workgroups, numbered so that the
//               Sq*H/64 workgroups reading the same pages land on the same
//               XCD (workgroup i runs on XCD i % 8) back to back, letting the
//               second read of a page hit that XCD's L2.
//   pipeline  = 32-token tiles.  Iteration i overlaps the score MFMAs of tile
//               i+1 with the softmax of tile i, then runs the latent MFMAs of
//               tile i while the partner's partial scores of tile i+1 land in
//               LDS.  Tiles are copied global->LDS by buffer_load ... lds (no
//               VGPR staging) into a ring (bf16: 4 stages, copies issued 3
//               tiles ahead).  The 16-byte chunks of each latent row are
//               XOR-swizzled with (row % 16), which keeps both the K-operand
//               reads (16 rows, one column) and the transposing V reads
//               (4 rows x 64 bytes per 16 lanes) free of bank conflicts.
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

#include "dtype.h"
#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kPage = 64;
constexpr int kTile = 32;                              // tokens per pipeline stage
constexpr int kThreads = 256;
constexpr int kCkvRow = kDc * 2;                       // bf16 bytes per latent row
constexpr int kKpeRow = kDr * 2;                       // bf16 bytes per RoPE-key row
constexpr int kTileCkv = kTile * kCkvRow;              // 32768
constexpr int kTileKpe = kTile * kKpeRow;              // 4096
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
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.f;                   // log2 units
static_assert(kSmemBf16 <= 160 * 1024, "LDS budget");

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier without the release fence of __syncthreads(): the fence
// would wait for the in-flight prefetch (vmcnt(0)).  LDS traffic is drained
// first so a buffer can be rewritten safely after the barrier.
__device__ __forceinline__ void barrier_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// generic pointer to a __shared__ object -> explicit LDS address-space pointer
__device__ __forceinline__ LDS_AS char *lds_ptr(char *p) { return (LDS_AS char *)(p); }

template <typename T>
__device__ __forceinline__ T lds_at(uint32_t addr) {
    return *reinterpret_cast<const LDS_AS T *>(static_cast<uintptr_t>(addr));
}

__device__ __forceinline__ uint32_t pack_lo(uint32_t lo_src, uint32_t hi_src) {
    return __builtin_amdgcn_perm(hi_src, lo_src, 0x05040100u);   // {lo_src.lo16, hi_src.lo16}
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t lo_src, uint32_t hi_src) {
    return __builtin_amdgcn_perm(hi_src, lo_src, 0x07060302u);   // {lo_src.hi16, hi_src.hi16}
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// acc *= s for an accumulator held in an AGPR, through one temporary VGPR
__device__ __forceinline__ void scale_agpr(float &acc, float s) {
    float t;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(acc), "=&v"(t)
                 : "v"(s));
}

// two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) { return cvt_pk_bf16(a, b); }

// ---------------------------------------------------------------------------
// Direct global->LDS copies (buffer_load_dword{,x4} ... lds): lane i's bytes from
// base + soff + voff_i land at LDS address M0 + 4*i (dword) or M0 + 16*i (dwordx4).
// Issued as inline asm so that the compiler, which cannot tell LDS-DMA targets
// from the operand reads, does not add its own waits on the copies in flight;
// every vmcnt wait in the attention loop is explicit.  Each statement builds a
// raw buffer descriptor (base, 48-bit address, stride 0, `bytes` records) in
// s[48:51] and issues its copies back to back.  Offsets are in range by
// construction (the caller's block-table precondition).
// ---------------------------------------------------------------------------
#define MLA_DMA_SETUP                                   \
    "s_mov_b32 s48, %[lo]\n\t"                         \
    "s_and_b32 s49, %[hi], 0xffff\n\t"                 \
    "s_mov_b32 s50, %[n]\n\t"                          \
    "s_mov_b32 s51, 0x20000\n\t"                       \
    "s_mov_b32 m0, %[l]\n\t"                           \
    "s_mov_b32 s52, %[so]\n\t"
#define MLA_DMA_X4(v) "buffer_load_dwordx4 %[" #v "], s[48:51], s52 offen lds\n\t"
#define MLA_DMA_STEP(lstride, gstride) "s_add_u32 m0, m0, " #lstride "\n\ts_add_u32 s52, s52, " #gstride "\n\t"
#define MLA_DMA_CLOBBERS "memory", "m0", "s48", "s49", "s50", "s51", "s52", "scc"

__device__ __forceinline__ uint32_t lo32(const void *p) {
    return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p)));
}
__device__ __forceinline__ uint32_t hi32(const void *p) {
    return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p) >> 32));
}

// 8 rows of 1 KiB: global rows soff, soff+1024, ...; LDS rows l, l+1024, ...; row jj's lane
// offsets v<jj> (the XOR swizzle makes them differ per row)
__device__ __forceinline__ void dma_rows8(const void *base, uint32_t bytes, uint32_t l, const uint32_t *v,
                                          uint32_t soff) {
    asm volatile(MLA_DMA_SETUP
                 MLA_DMA_X4(v0) MLA_DMA_STEP(1024, 1024) MLA_DMA_X4(v1) MLA_DMA_STEP(1024, 1024)
                 MLA_DMA_X4(v2) MLA_DMA_STEP(1024, 1024) MLA_DMA_X4(v3) MLA_DMA_STEP(1024, 1024)
                 MLA_DMA_X4(v4) MLA_DMA_STEP(1024, 1024) MLA_DMA_X4(v5) MLA_DMA_STEP(1024, 1024)
                 MLA_DMA_X4(v6) MLA_DMA_STEP(1024, 1024) MLA_DMA_X4(v7)
                 :: [lo] "s"(lo32(base)), [hi] "s"(hi32(base)), [n] "s"(bytes), [l] "s"(l),
                    [v0] "v"(v[0]), [v1] "v"(v[1]), [v2] "v"(v[2]), [v3] "v"(v[3]),
                    [v4] "v"(v[4]), [v5] "v"(v[5]), [v6] "v"(v[6]), [v7] "v"(v[7]), [so] "s"(soff)
                 : MLA_DMA_CLOBBERS);
}
// 4 consecutive KiB, same lane offsets: global soff, soff+1024, ...; LDS l, l+1024, ...
__device__ __forceinline__ void dma_kib4(const void *base, uint32_t bytes, uint32_t l, uint32_t voff,
                                         uint32_t soff) {
    asm volatile(MLA_DMA_SETUP
                 MLA_DMA_X4(v) MLA_DMA_STEP(1024, 1024) MLA_DMA_X4(v) MLA_DMA_STEP(1024, 1024)
                 MLA_DMA_X4(v) MLA_DMA_STEP(1024, 1024) MLA_DMA_X4(v)
                 :: [lo] "s"(lo32(base)), [hi] "s"(hi32(base)), [n] "s"(bytes), [l] "s"(l),
                    [v] "v"(voff), [so] "s"(soff)
                 : MLA_DMA_CLOBBERS);
}
// one 16-byte-per-lane copy
__device__ __forceinline__ void dma_x4(const void *base, uint32_t bytes, uint32_t l, uint32_t voff,
                                       uint32_t soff) {
    asm volatile(MLA_DMA_SETUP MLA_DMA_X4(v)
                 :: [lo] "s"(lo32(base)), [hi] "s"(hi32(base)), [n] "s"(bytes), [l] "s"(l),
                    [v] "v"(voff), [so] "s"(soff)
                 : MLA_DMA_CLOBBERS);
}
// one 4-byte-per-lane copy (lanes inactive in exec copy nothing)
__device__ __forceinline__ void dma_x1(const void *base, uint32_t bytes, uint32_t l, uint32_t voff,
                                       uint32_t soff) {
    asm volatile(MLA_DMA_SETUP "buffer_load_dword %[v], s[48:51], s52 offen lds\n\t"
                 :: [lo] "s"(lo32(base)), [hi] "s"(hi32(base)), [n] "s"(bytes), [l] "s"(l),
                    [v] "v"(voff), [so] "s"(soff)
                 : MLA_DMA_CLOBBERS);
}

// ---------------------------------------------------------------------------
// LDS layouts of a tile
//   latent row r (1 KiB, 64 chunks of 16 bytes): logical chunk c at
//       r*1024 + ((c ^ (r % 16)) << 4)
//   RoPE-key row r (128 bytes, 8 chunks): logical chunk c at
//       r*128 + ((c ^ ((r / 2) % 8)) << 4)
// Token order: MFMA row x of the score product (and D row x of S^T) holds
// tile token perm_tok(x) with x = 16kq + 8h + 4g + j -> 16kq + 4j + 2h + g.
// The 16 rows a 16-lane group reads for the K operand are then 16 distinct
// rows, and the 4 rows one 16-lane group of a transposing V read touches are
// 4 apart, which keeps both read patterns conflict-free under the swizzle.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int perm_tok(int x) {
    return (x & 16) | ((x & 3) << 2) | (((x >> 3) & 1) << 1) | ((x >> 2) & 1);
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each 16-lane group, lane i
// receives element i%4 of the 8-byte chunks addressed by lanes 4j + i/4,
// j = 0..3.  Issued as inline asm (see the copies above); the caller waits on
// lgkmcnt before using the result, and the memory clobbers keep every other
// memory operation (scalar loads count in lgkmcnt too) out of the window
// between the reads and their waits.
template <int kOff>
__device__ __forceinline__ v4i16 lds_read_tr16(uint32_t addr) {
    v4i16 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(kOff) : "memory");
    return r;
}
template <int N>
__device__ __forceinline__ void wait_lgkm_tied(v4i16 &a, v4i16 &b) {
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "n"(N) : "memory");
}

// O^T[256 latent columns of this wave, 32 heads] += V^T[., 16 tokens] P^T[16 tokens, heads]
// for one 16-token k-step kq of a tile.  vx[h*4 + b4]: lane address of the
// transposing read of half h (tokens 8h..) for column blocks blk = b4, b4+4.
template <int kq>
__device__ __forceinline__ void latent_step(uint32_t base, const uint32_t *vx, bf16x8 pb, f32x16 *oacc) {
    constexpr int kq_off = kq * 16 * kCkvRow;
    v4i16 lo[8], hi[8];
#define MLA_TR(blk) \
    lo[blk] = lds_read_tr16<kq_off + ((blk) >> 2) * 256>(base + vx[(blk) & 3]); \
    hi[blk] = lds_read_tr16<kq_off + ((blk) >> 2) * 256>(base + vx[4 + ((blk) & 3)]);
    MLA_TR(0) MLA_TR(1) MLA_TR(2) MLA_TR(3) MLA_TR(4) MLA_TR(5) MLA_TR(6) MLA_TR(7)
#undef MLA_TR
#define MLA_PV(blk, n)                                                                              \
    wait_lgkm_tied<n>(lo[blk], hi[blk]);                                                            \
    oacc[blk] = mfma32(__builtin_bit_cast(bf16x8, v8i16{lo[blk][0], lo[blk][1], lo[blk][2], lo[blk][3], \
                                                        hi[blk][0], hi[blk][1], hi[blk][2], hi[blk][3]}), \
                       pb, oacc[blk]);
    MLA_PV(0, 14) MLA_PV(1, 12) MLA_PV(2, 10) MLA_PV(3, 8) MLA_PV(4, 6) MLA_PV(5, 4) MLA_PV(6, 2) MLA_PV(7, 0)
#undef MLA_PV
}

// Partial scores of one tile over this wave's half of the 576 dims.
//   ckv: LDS address of the tile's latent rows; kpe: of its RoPE-key rows
//   kx[u]: lane offset of the K chunk for k-steps with (ks + 18*KH) % 8 == u
//   kpx[ks]: lane offset of RoPE chunk 2ks+g (KH = 1 only)
//   tsc (fp8): per-D-element token scales, multiplied in before the RoPE term
template <int KH, bool kFp8>
__device__ __forceinline__ f32x16 score_tile(uint32_t ckv, uint32_t kpe, const uint32_t *kx, const uint32_t *kpx,
                                             const bf16x8 *qreg, const float *tsc) {
    constexpr int N = KH == 0 ? 18 : 14;
    f32x16 sa, sb;
#pragma unroll
    for (int j = 0; j < 16; ++j) { sa[j] = 0.f; sb[j] = 0.f; }
    bf16x8 a[N];
#pragma unroll
    for (int ks = 0; ks < N; ++ks)
        a[ks] = lds_at<bf16x8>(ckv + kx[(ks + 18 * KH) & 7] + ((((2 * ks + 36 * KH) & ~15)) << 4));
#pragma unroll
    for (int ks = 0; ks < N; ++ks) {
        if (ks & 1) sb = mfma32(a[ks], qreg[ks], sb);
        else sa = mfma32(a[ks], qreg[ks], sa);
    }
    f32x16 s = sa + sb;
    if constexpr (kFp8) {
#pragma unroll
        for (int j = 0; j < 16; ++j) s[j] *= tsc[j];
    }
    if constexpr (KH == 1) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) s = mfma32(lds_at<bf16x8>(kpe + kpx[ks]), qreg[14 + ks], s);
    }
    return s;
}

// ---------------------------------------------------------------------------
// mla_decode_splitkv
// ---------------------------------------------------------------------------
// Instruction schedule of the block holding the score MFMAs of the next tile
// and the softmax VALU of the current one: four K-operand reads up front, then
// each MFMA followed by the next read and a few VALU instructions, so that LDS
// latency and the VALU work hide under the MFMAs.
template <int KH>
__device__ __forceinline__ void shape_scores_softmax() {
    constexpr int N = KH == 0 ? 18 : 14;               // content k-steps (KH = 1 adds 4 RoPE steps)
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // DS read
#pragma unroll
    for (int k = 0; k < N - 4; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    }
}

// The body of the attention kernel for one wave; KH (= wave % 2, the wave's half
// of the pair's work) is a template parameter so that each wave's loop is
// straight-line code the scheduler can interleave.
template <bool kFp8, int KH>
__device__ __forceinline__ void decode_wave(
    char *smem, const mla_params_t &p, const uint16_t *__restrict__ q_abs, const uint16_t *__restrict__ q_rope,
    const void *__restrict__ c_kv, const uint16_t *__restrict__ k_pe,
    const float *__restrict__ kv_scale, const int32_t *__restrict__ block_table,
    const int32_t *__restrict__ seq_lens, float *__restrict__ o_part, float *__restrict__ lse_part) {
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

    // workgroup -> (item u = b*S + c, row group rg); items are spread over the
    // 8 XCDs, the row groups of one item share an XCD.
    const int n_rg = (p.Sq * p.H) / 64;
    const int xcd = blockIdx.x & 7;
    const int q = blockIdx.x >> 3;
    const int rg = q % n_rg;
    const int64_t u = static_cast<int64_t>(q / n_rg) * 8 + xcd;
    const int b = static_cast<int>(u / S);
    const int c = static_cast<int>(u % S);

    const int seq_len = seq_lens[b];
    const int t_begin = c * p.split_pages * kPage;                       // first position of the split
    const int t_end = min(t_begin + p.split_pages * kPage, seq_len);     // one past the last stored one
    const int row0 = rg * 64 + (wave >> 1) * 32;       // first (s,h) row of this wave pair
    const int s = row0 / p.H;
    const int h = row0 % p.H + t32;                    // this lane's head
    const int64_t qrow = (static_cast<int64_t>(b) * p.Sq + s) * p.H + h;
    const int n_vis = seq_len - p.Sq + 1 + s;          // positions this pair's rows may see
    const int64_t out_row = qrow * S + c;

    if (t_begin >= t_end) {                            // split past the sequence's end
        if (kh == 0 && g2 == 0) lse_part[out_row] = -INFINITY;
        return;
    }
    const int n_tiles = (t_end - t_begin + kTile - 1) / kTile;
    const int last_valid = t_end - (t_begin + (n_tiles - 1) * kTile);   // stored rows of the last tile

    // query operands (B of the score product) for this wave's half of the 576 dims
    bf16x8 qreg[18];
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
        const uint16_t *src;
        if (kh == 0) src = q_abs + qrow * kDc + ks * 16 + g2 * 8;                   // latent 0..287
        else if (ks < 14) src = q_abs + qrow * kDc + 288 + ks * 16 + g2 * 8;         // latent 288..511
        else src = q_rope + qrow * kDr + (ks - 14) * 16 + g2 * 8;                    // RoPE 0..63
        qreg[ks] = *reinterpret_cast<const bf16x8 *>(src);
    }
    // Consume the query loads here: otherwise the compiler places their vmcnt
    // waits at the first use inside the tile loop, where (re-executed every
    // iteration) they would also wait for the tile copies in flight.
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) asm volatile("" : "+v"(qreg[ks]));

    const int32_t *bt = block_table + static_cast<int64_t>(b) * p.max_pages;
    const uint32_t sm = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_ptr(smem)));
    const uint32_t xchg = sm + (kFp8 ? kStagesFp8 * kStageFp8 + 2 * kTileCkv : kStagesBf16 * kStageBf16);
    const uint32_t conv0 = sm + kStagesFp8 * kStageFp8;                  // fp8: converted tiles

    // ---- loop-invariant lane offsets
    // copies: latent row r = wave*8 + jj stores logical chunk lane^(r%16) in physical chunk lane
    uint32_t vd[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) vd[jj] = (lane ^ ((kh << 3) | jj)) << 4;
    const int kpe_r = wave * 8 + (lane >> 3);          // RoPE rows: 8 per instruction
    const uint32_t voff_kpe = kpe_r * kKpeRow + (((lane & 7) ^ ((kpe_r >> 1) & 7)) << 4);
    // K operand: row perm_tok(t32), logical chunk 2ks + 36kh + g2
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

    // copy tile t (tokens t_begin + 32t ...) whose page is `phys` into its ring stage
    auto issue_tile = [&](int t, int64_t phys) {
        const int tok0 = t_begin + t * kTile;          // multiple of 32
        const int64_t crow0 = phys * kPage + (tok0 % kPage);   // first cache row of the tile
        const uint32_t base = stage_of(t);
        if constexpr (!kFp8) {
            dma_rows8(static_cast<const char *>(c_kv) + crow0 * kCkvRow, kTileCkv, base + wave * 8 * kCkvRow,
                      vd, wave * 8 * kCkvRow);
            dma_x4(k_pe + crow0 * kDr, kTileKpe, base + kTileCkv + wave * 1024, voff_kpe, 0);
        } else {
            dma_kib4(static_cast<const char *>(c_kv) + crow0 * kDc, kRawCkv, base + wave * 4 * 1024, lane * 16,
                     wave * 4 * 1024);
            dma_x4(k_pe + crow0 * kDr, kTileKpe, base + kRawCkv + wave * 1024, voff_kpe, 0);
            if (lane < 8) dma_x1(kv_scale + crow0, kTile * 4, base + kRawCkv + kTileKpe + wave * 32, lane * 4, wave * 32);
        }
    };
    auto page_of = [&](int t) -> int64_t { return bt[(t_begin + t * kTile) / kPage]; };

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
                const u32x2 v = lds_at<u32x2>(raw + tok * kDc + lc * 8);
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
                *reinterpret_cast<LDS_AS u32x4 *>(static_cast<uintptr_t>(dst + tok * kCkvRow + ((lc ^ (tok & 15)) << 4))) = o;
            }
            return true;
        } else {
            if (valid == kTile) return false;
            const uint32_t w = stage_of(t);
            for (int k = threadIdx.x; k < (kTile - valid) * 64; k += kThreads)
                *reinterpret_cast<LDS_AS u32x4 *>(static_cast<uintptr_t>(w + (valid + (k >> 6)) * kCkvRow + (k & 63) * 16)) =
                    u32x4{0u, 0u, 0u, 0u};
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
            tsc[j] = tok < valid ? lds_at<float>(sc + tok * 4) : 0.f;
        }
    };

    auto partial_scores = [&](int t) -> f32x16 {
        float tsc[16];
        if constexpr (kFp8) token_scales(t, tsc);
        return score_tile<KH, kFp8>(ckv_of(t), kpe_of(t), kx, kpx, qreg, tsc);
    };

    // swap partial scores with the other wave of the pair: write, barrier, read + add
    auto exchange_write = [&](const f32x16 &sp) {
#pragma unroll
        for (int jq = 0; jq < 4; ++jq)
            *reinterpret_cast<LDS_AS f32x4 *>(static_cast<uintptr_t>(xchg + wave * kXchgWave + (jq * 64 + lane) * 16)) =
                f32x4{sp[jq * 4], sp[jq * 4 + 1], sp[jq * 4 + 2], sp[jq * 4 + 3]};
    };
    auto exchange_read = [&](f32x16 &sp) {
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
            const f32x4 o = lds_at<f32x4>(xchg + (wave ^ 1) * kXchgWave + (jq * 64 + lane) * 16);
#pragma unroll
            for (int j = 0; j < 4; ++j) sp[jq * 4 + j] += o[j];   // commutative: same sum in both waves
        }
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

    // softmax, first part: scale, mask, running maximum (rescales O when it jumps)
    auto softmax_max = [&](int t, const f32x16 &sfull, float *z) -> float {
        const int tbase = t_begin + t * kTile;
#pragma unroll
        for (int j = 0; j < 16; ++j) z[j] = sfull[j] * zscale;
        if (tbase + kTile > n_vis) {                   // causal bound or sequence end inside the tile
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (tbase + perm_tok((j >> 2) * 8 + g2 * 4 + (j & 3)) >= n_vis) z[j] = -INFINITY;
        }
        float mloc = z[0];
#pragma unroll
        for (int j = 1; j < 16; ++j) mloc = fmaxf(mloc, z[j]);
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
        // raise the reference only when a weight would exceed 2^kRescaleSlack
        const bool raise = mloc > m_ref + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(raise)) {
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
    // softmax, second part: weights, their sums, bf16 P^T operands (pairs j, j+1)
    auto softmax_weights = [&](int t, const float *z, float m_use, uint32_t *pk) {
        float tsc[16];
        if constexpr (kFp8) token_scales(t, tsc);
#pragma unroll
        for (int j = 0; j < 16; j += 2) {
            const float p0 = __builtin_amdgcn_exp2f(z[j] - m_use);
            const float p1 = __builtin_amdgcn_exp2f(z[j + 1] - m_use);
            l_run += p0 + p1;
            if constexpr (kFp8) {
                pk[j >> 1] = cvt_pk_bf16(p0 * tsc[j], p1 * tsc[j + 1]);
            } else {
                pk[j >> 1] = cvt_pk_bf16(p0, p1);
                // the sum of the weights exactly as the PV product sees them
                lw_run += __uint_as_float(pk[j >> 1] << 16) + __uint_as_float(pk[j >> 1] & 0xffff0000u);
            }
        }
    };
    auto latent_update = [&](int t, const uint32_t *pk) {
        const uint32_t base = ckv_of(t);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // counted waits below see only these reads
        latent_step<0>(base, vx, as_bf16x8(u32x4{pk[0], pk[1], pk[2], pk[3]}), oacc);
        latent_step<1>(base, vx, as_bf16x8(u32x4{pk[4], pk[5], pk[6], pk[7]}), oacc);
    };

    // ---- prologue: copies of tiles 0 .. kAhead-1, scores of tile 0
    int64_t phys_next = 0;                             // page of tile kAhead (+ i), read one iteration early
#pragma unroll
    for (int t = 0; t < kAhead; ++t)
        if (t < n_tiles) issue_tile(t, page_of(t));
    if (kAhead < n_tiles) phys_next = page_of(kAhead);
    // wait for tile 0: the copies of tiles 1 .. kAhead-1 may stay in flight
    {
        const int inflight = min(kAhead, n_tiles) - 1;
        if (inflight >= 2) wait_vmcnt<2 * kLoads>();
        else if (inflight == 1) wait_vmcnt<kLoads>();
        else wait_vmcnt<0>();
    }
    barrier_lds();
    if (prepare_tile(0)) barrier_lds();
    f32x16 sfull = partial_scores(0);
    exchange_write(sfull);
    barrier_lds();
    exchange_read(sfull);

    // ---- steady state: tiles 0 .. n-2 (the next tile exists)
    for (int i = 0; i + 1 < n_tiles; ++i) {
        // tile i+1 has landed; tiles up to i+kAhead-1 may stay in flight
        if constexpr (kFp8) {
            wait_vmcnt<0>();
        } else {
            if (i + 2 < n_tiles) wait_vmcnt<kLoads>(); else wait_vmcnt<0>();
        }
        barrier_lds();                                 // tile i+1 visible; iteration i-1 finished
        // copy tile i+kAhead into the stage of tile i-1 (free: every wave passed the barrier)
        if (i + kAhead < n_tiles) {
            issue_tile(i + kAhead, phys_next);
            if (i + kAhead + 1 < n_tiles) phys_next = page_of(i + kAhead + 1);
        }
        if (prepare_tile(i + 1)) barrier_lds();

        float z[16];
        const float m_use = softmax_max(i, sfull, z);
        uint32_t pk[8];
        // score MFMAs of tile i+1 and the softmax VALU of tile i are independent
        f32x16 snext = partial_scores(i + 1);
        softmax_weights(i, z, m_use, pk);
        shape_scores_softmax<KH>();
        exchange_write(snext);
        latent_update(i, pk);
        barrier_lds();                                 // partner's partial scores of tile i+1 written
        exchange_read(snext);
        sfull = snext;
    }
    // ---- last tile
    {
        const int i = n_tiles - 1;
        float z[16];
        const float m_use = softmax_max(i, sfull, z);
        uint32_t pk[8];
        softmax_weights(i, z, m_use, pk);
        latent_update(i, pk);
    }

    // ---- epilogue: sums of the head's two lanes, normalised partial + lse
    float l_tot = l_run + __shfl_xor(l_run, 32);
    if (l_tot == 0.f) {                                  // no visible position in this split
        if (kh == 0 && g2 == 0) lse_part[out_row] = -INFINITY;
        return;
    }
    float norm = l_tot;
    if constexpr (!kFp8) norm = lw_run + __shfl_xor(lw_run, 32);
    const float inv = 1.f / norm;
    float *dst = o_part + out_row * kDc + kh * 256;
    // oacc[blk][j]: head t32, latent 256kh + 32*blk + 8*(j/4) + 4*g2 + j%4
#pragma unroll
    for (int blk = 0; blk < 8; ++blk)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
            const f32x4 v = f32x4{oacc[blk][jq * 4], oacc[blk][jq * 4 + 1], oacc[blk][jq * 4 + 2],
                                  oacc[blk][jq * 4 + 3]} * inv;
            *reinterpret_cast<f32x4 *>(dst + blk * 32 + jq * 8 + g2 * 4) = v;
        }
    if (kh == 0 && g2 == 0) lse_part[out_row] = (m_ref + __builtin_amdgcn_logf(l_tot)) * kLn2;
}

template <bool kFp8>
__global__ __launch_bounds__(kThreads, 1) void decode_mfma_kernel(
    const mla_params_t p, const uint16_t *__restrict__ q_abs, const uint16_t *__restrict__ q_rope,
    const void *__restrict__ c_kv, const uint16_t *__restrict__ k_pe,
    const float *__restrict__ kv_scale, const int32_t *__restrict__ block_table,
    const int32_t *__restrict__ seq_lens, float *__restrict__ o_part, float *__restrict__ lse_part) {
    __shared__ __attribute__((aligned(1024))) char smem[kFp8 ? kSmemFp8 : kSmemBf16];
    // workgroups past the last (sequence, split) item (grid rounded up to 8 XCDs)
    const int n_rg = (p.Sq * p.H) / 64;
    const int64_t u = static_cast<int64_t>((blockIdx.x >> 3) / n_rg) * 8 + (blockIdx.x & 7);
    if (u >= static_cast<int64_t>(p.B) * p.num_splits) return;
    if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & 1)
        decode_wave<kFp8, 1>(smem, p, q_abs, q_rope, c_kv, k_pe, kv_scale, block_table, seq_lens, o_part, lse_part);
    else
        decode_wave<kFp8, 0>(smem, p, q_abs, q_rope, c_kv, k_pe, kv_scale, block_table, seq_lens, o_part, lse_part);
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
    if (p.H % 32 != 0 || (p.Sq * p.H) % kDecodeRowsPerBlock != 0) return false;
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
