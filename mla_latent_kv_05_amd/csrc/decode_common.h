// Device code shared by the two attention kernels (kernels_decode.hip,
// kernels_decode8.hip): tile constants, the global->LDS copy instructions, the
// LDS tile layout and its operand reads, and the walk over the segments of a
// work part.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

#include "dev_errors.h"
#include "gfx950.h"
#include "mla_internal.h"

namespace mla {
namespace dec {

using namespace gfx;

constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kPage = 64;
constexpr int kTile = 32;                              // tokens per pipeline stage
constexpr int kCkvRow = kDc * 2;                       // bf16 bytes per latent row
constexpr int kKpeRow = kDr * 2;                       // bf16 bytes per RoPE-key row
constexpr int kTileCkv = kTile * kCkvRow;              // 32768
constexpr int kTileKpe = kTile * kKpeRow;              // 4096
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.f;                   // log2 units

// acc *= s for an accumulator held in an AGPR, through one temporary VGPR
__device__ __forceinline__ void scale_agpr(float &acc, float s) {
    float t;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(acc), "=&v"(t)
                 : "v"(s));
}

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
#define MLA_DMA_BASE(base, bytes, l, soff)                                                 \
    [lo] "s"(lo32(base)), [hi] "s"(hi32(base)), [n] "s"(__builtin_amdgcn_readfirstlane(bytes)), \
        [l] "s"(__builtin_amdgcn_readfirstlane(l)), [so] "s"(__builtin_amdgcn_readfirstlane(soff))

__device__ __forceinline__ uint32_t lo32(const void *p) {
    return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p)));
}
__device__ __forceinline__ uint32_t hi32(const void *p) {
    return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p) >> 32));
}

// two / four rows of 1 KiB: global soff, soff+1024, ...; LDS l, l+1024, ...; row j's lane offset v<j>
__device__ __forceinline__ void dma_rows2(const void *base, uint32_t bytes, uint32_t l, uint32_t soff,
                                          uint32_t v0, uint32_t v1) {
    asm volatile(MLA_DMA_SETUP MLA_DMA_X4(v0) MLA_DMA_STEP(1024, 1024) MLA_DMA_X4(v1)
                 :: MLA_DMA_BASE(base, bytes, l, soff), [v0] "v"(v0), [v1] "v"(v1)
                 : MLA_DMA_CLOBBERS);
}
// four rows of 1 KiB
__device__ __forceinline__ void dma_rows4(const void *base, uint32_t bytes, uint32_t l, uint32_t soff,
                                          uint32_t v0, uint32_t v1, uint32_t v2, uint32_t v3) {
    asm volatile(MLA_DMA_SETUP MLA_DMA_X4(v0) MLA_DMA_STEP(1024, 1024) MLA_DMA_X4(v1) MLA_DMA_STEP(1024, 1024)
                 MLA_DMA_X4(v2) MLA_DMA_STEP(1024, 1024) MLA_DMA_X4(v3)
                 :: MLA_DMA_BASE(base, bytes, l, soff), [v0] "v"(v0), [v1] "v"(v1), [v2] "v"(v2), [v3] "v"(v3)
                 : MLA_DMA_CLOBBERS);
}
// four 1 KiB pieces to consecutive LDS KiB from global offsets soff, soff+4096, ...
// (four rows of 256 bytes each, of a tile whose rows are 1 KiB apart)
__device__ __forceinline__ void dma_blk4(const void *base, uint32_t bytes, uint32_t l, uint32_t soff,
                                         uint32_t v0, uint32_t v1, uint32_t v2, uint32_t v3) {
    asm volatile(MLA_DMA_SETUP MLA_DMA_X4(v0) MLA_DMA_STEP(1024, 4096) MLA_DMA_X4(v1) MLA_DMA_STEP(1024, 4096)
                 MLA_DMA_X4(v2) MLA_DMA_STEP(1024, 4096) MLA_DMA_X4(v3)
                 :: MLA_DMA_BASE(base, bytes, l, soff), [v0] "v"(v0), [v1] "v"(v1), [v2] "v"(v2), [v3] "v"(v3)
                 : MLA_DMA_CLOBBERS);
}
// one 16-byte-per-lane copy
__device__ __forceinline__ void dma_x4(const void *base, uint32_t bytes, uint32_t l, uint32_t soff, uint32_t v) {
    asm volatile(MLA_DMA_SETUP MLA_DMA_X4(v)
                 :: MLA_DMA_BASE(base, bytes, l, soff), [v] "v"(v)
                 : MLA_DMA_CLOBBERS);
}
// one 4-byte-per-lane copy (lanes inactive in exec copy nothing)
__device__ __forceinline__ void dma_x1(const void *base, uint32_t bytes, uint32_t l, uint32_t soff, uint32_t v) {
    asm volatile(MLA_DMA_SETUP "buffer_load_dword %[v], s[48:51], s52 offen lds\n\t"
                 :: MLA_DMA_BASE(base, bytes, l, soff), [v] "v"(v)
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

// LDS operand reads are plain loads: the compiler places a counted lgkmcnt wait
// before each use (LDS operations complete in issue order; it counts the ones it
// issued, and LDS operations written as inline asm elsewhere only make those waits
// stricter) and keeps each value in its registers until it has landed.
__device__ __forceinline__ u32x4 ld128(uint32_t addr) { return lds_load<u32x4>(addr); }

// four consecutive elements of a split partial (element index e) in the partials'
// storage type: fp32, or bf16 rounded to nearest even
__device__ __forceinline__ void store_part4(void *o_part, int part_dtype, int64_t e, const f32x4 &v) {
    if (part_dtype == MLA_BF16)
        *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(o_part) + e) = u32x2{cvt_pk_bf16(v[0], v[1]), cvt_pk_bf16(v[2], v[3])};
    else
        *reinterpret_cast<f32x4 *>(static_cast<float *>(o_part) + e) = v;
}
// Transposing LDS read (ds_read_b64_tr_b16).  Within each 16-lane group, lane i
// receives element i%4 of the 8-byte chunks addressed by lanes 4j + i/4, j = 0..3.
__device__ __forceinline__ v4i16 ld_tr16(uint32_t addr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<MLA_LDS_AS v4i16 *>(static_cast<uintptr_t>(addr)));
}
// Nothing moves across: the instruction order of a phase is the source order.
__device__ __forceinline__ void pin() { __builtin_amdgcn_sched_barrier(0); }

// ---------------------------------------------------------------------------
// Work parts.  A segment is the part of one sequence b that a work part
// covers: pages [pa, pb) of b, producing split slot c of b's rows.
// ---------------------------------------------------------------------------
struct Segment {
    int b, c, pa, pb;
    bool last;         // the part holding b's last page: fills the later slots with -inf
};

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(v, o);
        if (lane >= o) v += t;
    }
    return v;
}

// Calls f(seg) for the segments of work part `part`, in sequence order (a
// segment has no pages when the part is an empty one inside the sequence's
// range, which happens with more parts than pages), and fill(b, c0, c1) for
// each empty sequence this part owns.
// Every value is wave-uniform (each wave of the workgroup walks identically).
template <typename F, typename Fill>
__device__ __forceinline__ void for_each_segment(const mla_params_t &p, const int32_t *__restrict__ seq_lens,
                                                 int part, F &&f, Fill &&fill) {
    const int lane = threadIdx.x & 63;
    if (p.num_parts == 0) {                            // fixed splits: part = b * S + c
        const int b = part / p.num_splits;
        const int c = part % p.num_splits;
        const int pages = seq_pages(p, seq_lens[b]);
        const int pa = c * p.split_pages;
        const int pb = min(pa + p.split_pages, pages);
        if (pa < pb) f(Segment{b, c, pa, pb, false});
        else fill(b, c, c + 1);
        return;
    }
    auto cost = [](int pages) { return pages > 0 ? pages + kSeqStartCost : 0; };
    const int64_t P = p.num_parts;
    int64_t T = 0;                                     // units of the whole batch
    for (int b0 = 0; b0 < p.B; b0 += 64) {
        const int b = b0 + lane;
        T += wave_sum(b < p.B ? cost(seq_pages(p, seq_lens[b])) : 0);
    }
    const int64_t pg0 = part * T / P, pg1 = (part + 1) * T / P;   // this part's units
    int64_t base = 0;                                  // units before sequence b0
    for (int b0 = 0; b0 < p.B; b0 += 64) {
        const int b = b0 + lane;
        const int pages = b < p.B ? seq_pages(p, seq_lens[b]) : 0;
        const int units = cost(pages);
        const int incl = wave_inclusive_scan(units);
        const int chunk = __builtin_amdgcn_readlane(incl, 63);
        if (base > pg1) break;                         // every later sequence starts past this part
        if (base + chunk >= pg0) {
            const int64_t off = base + incl - units;   // the sequence's first unit
            const int64_t first = off + kSeqStartCost; // ... and the unit of its first page
            // sequences with pages in the part; empty sequences are owned by the part
            // whose range holds their position (the last part owns those at the very end)
            const bool mine = b < p.B && (pages > 0 ? (first < pg1 && first + pages > pg0)
                                                    : ((off >= pg0 && off < pg1) || (part == P - 1 && off >= T)));
            uint64_t m = __builtin_amdgcn_ballot_w64(mine);
            while (m) {
                const int k = __builtin_ctzll(m);
                m &= m - 1;
                const int bb = b0 + k;
                const int pg_b = __builtin_amdgcn_readlane(pages, k);
                const int64_t off_b = base + __builtin_amdgcn_readlane(incl, k) - cost(pg_b);
                if (pg_b == 0) {
                    fill(bb, 0, p.num_splits);
                    continue;
                }
                const int64_t f_b = off_b + kSeqStartCost;
                const int64_t j0 = ((f_b + 1) * P - 1) / T;             // part holding the first page
                const int64_t jl = ((f_b + pg_b) * P - 1) / T;          // part holding the last page
                const int c = static_cast<int>(part - j0);
                const int pa = static_cast<int>(max<int64_t>(pg0 - f_b, 0));
                const int pb = static_cast<int>(min<int64_t>(pg1 - f_b, pg_b));
                f(Segment{bb, c, pa, pb, part == jl});
            }
        }
        base += chunk;
    }
}

}  // namespace dec
}  // namespace mla
