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
// Decompress: one workgroup (8 waves) per (group of 16 heads, sequence, 256
// positions); wave w holds the latent rows of 32 of the positions as MFMA operands
// (128 VGPRs) for the whole workgroup.  The weights stream through LDS in passes
// of 64 rows (output dims) of one head, W_UK[h] then W_UV[h], each pass in chunks
// of 256 latent dims (direct global->LDS copies into a ring of three buffers, two
// chunks ahead, shared by the 8 waves; the blocks running together on an XCD start
// at different passes):
//   keys:   D[d, t] = W_UK[h] . c^T (weight rows as the A operand, latent rows as B),
//   values: D[t, d] = c . W_UV[h]^T (latent rows as A, weight rows as B),
// the latent registers serving both roles unchanged (both operands take 8
// consecutive latent dims per lane).  A-operand rows are taken in swap23 order,
// so each lane ends with 8 consecutive output rows twice per 32-row tile: the keys
// are written 8 dims (16 bytes) and the transposed values 8 positions at a time.
// Blocks are ordered head group first, and with a multiple of 8 blocks XCD x gets
// one contiguous range, so each XCD's L2 serves few head groups' weights.
//
// Attention: one workgroup (8 waves) per (sequence, head, 256 new tokens); wave w
// takes 32 of them.  Keys and transposed values of 64 positions (one page) at a
// time are staged in LDS once per workgroup, double-buffered, and read by every
// wave.  Per staged tile, in two halves of 32 positions, each wave forms
//   S^T[t, q] = K_half . Q^T over the 192 dims (12 MFMAs; Q^T in registers).
//   Row r of the half holds position swap23(r) (bits 2 and 3 of r exchanged), so
//   that the 16 weights a lane holds for query q are, as the B operand of the
//   value product, positions 16k + 8g + e in order;
//   the online softmax per query in the exp2 domain (a lane pair per query); the
//   running maximum only moves when exceeded by more than 2^8, so the rescale of
//   the accumulators is skipped on most halves;
//   O^T[d, q] += V^T[d, t] . P^T[t, q] (8 MFMAs).
// Positions past a query's own or past seq_len are masked in the scores; values
// past seq_len are zeroed when staged.
#include <hip/hip_runtime.h>
#include <math.h>

#include "decode_common.h"
#include "gfx950.h"
#include "mla_internal.h"

namespace mla {
namespace {

using namespace gfx;

// Four 16-byte-per-lane direct copies (buffer_load_dwordx4 ... lds) to consecutive
// KiB of LDS from l on; copy i reads base + soff + v<i> in each lane (inline asm, as
// in the attention kernels, so the compiler adds no waits of its own on them).
__device__ __forceinline__ void dma_rows4_fixed(const void *base, uint32_t bytes, uint32_t l, uint32_t soff,
                                                uint32_t v0, uint32_t v1, uint32_t v2, uint32_t v3) {
    using dec::hi32;
    using dec::lo32;
    asm volatile(MLA_DMA_SETUP MLA_DMA_X4(v0) "s_add_u32 m0, m0, 1024\n\t" MLA_DMA_X4(v1)
                 "s_add_u32 m0, m0, 1024\n\t" MLA_DMA_X4(v2) "s_add_u32 m0, m0, 1024\n\t" MLA_DMA_X4(v3)
                 :: MLA_DMA_BASE(base, bytes, l, soff), [v0] "v"(v0), [v1] "v"(v1), [v2] "v"(v2), [v3] "v"(v3)
                 : MLA_DMA_CLOBBERS);
}

constexpr int kDh = 128;
constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kDecHeads = 16;                  // heads of one decompress workgroup
constexpr int kDecWaves = 8;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDecPos = 32 * kDecWaves;        // positions of one decompress workgroup (32 per wave)
constexpr int kDecRows = 64;                   // weight rows (output dims) of one pass
constexpr int kWChunk = 256;                   // latent dims of one staged weight chunk
constexpr int kWStage = kDecRows * kWChunk * 2;  // one staged chunk: 64 rows of 512 bytes (swizzled)
constexpr int kWBufs = 3;                      // staged chunks: in use, landed, in flight
// The 32 blocks that run at once on one XCD share a head group; block j of them
// starts at pass kDecRot * j (mod the pass count), so that they do not all ask
// the XCD's L2 for the same weight chunk at the same moment (in lockstep they
// fetched at about 2 TB/s overall and took 1.0-1.1 ms at 4 x 4,096 positions;
// staggered, 0.66-0.70 ms).
constexpr int kDecRot = 2;
static_assert(kDecPos == 256, "prefill_lmax rounds the row stride to whole decompression tiles");
static_assert(kDecWaves * 4 * 1024 == kWStage, "four 1 KiB copies per wave fill one staged chunk");
constexpr float kLog2e = 1.4426950408889634f;

// Instruction order of one staged chunk's 32 operand reads and 32 MFMAs: the first
// kReadAhead reads, then one MFMA and one read in turn, so that each read is issued
// kReadAhead MFMAs before its product (the default schedule issues it just before).
constexpr int kReadAhead = 6;
__device__ __forceinline__ void read_ahead_schedule() {
    constexpr int kN = 2 * (kWChunk / 16);
    __builtin_amdgcn_sched_group_barrier(0x100, kReadAhead, 0);     // DS reads
#pragma unroll
    for (int i = 0; i < kN - kReadAhead; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kReadAhead, 0);
}

// tile row r holds position swap23(r) of the tile
__device__ __forceinline__ int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kDecThreads) void decompress_kernel(
    const mla_params_t p, const uint16_t *__restrict__ c_kv, const int32_t *__restrict__ block_table,
    const int32_t *__restrict__ seq_lens, const uint16_t *__restrict__ W_UK, const uint16_t *__restrict__ W_UV,
    uint16_t *__restrict__ k_nope, uint16_t *__restrict__ v_t) {
    // 1 KiB alignment: the operand addresses XOR bits 5..8 of buffer offsets
    __shared__ __attribute__((aligned(1024))) char lds[kWBufs * kWStage];
    const int tid = threadIdx.x, lane = tid & 63, t32 = lane & 31, g = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t lmax = prefill_lmax(p);               // a multiple of kDecPos
    const int n_pt = static_cast<int>(lmax / kDecPos);
    const int64_t nblk = gridDim.x;
    int64_t lb = blockIdx.x;
    if ((nblk & 7) == 0) lb = (lb & 7) * (nblk >> 3) + (lb >> 3);
    const int lb_run = static_cast<int>(lb & 31);           // position among concurrent blocks
    const int pt = static_cast<int>(lb % n_pt);
    lb /= n_pt;
    const int b = static_cast<int>(lb % p.B);
    const int hg = static_cast<int>(lb / p.B);
    const int L = seq_lens[b];
    const int t0 = pt * kDecPos;
    if (t0 >= L) return;
    // this lane's latent row: position t0 + 32w + swap23(t32), dims 16ks + 8g .. +7
    const int tw = t0 + 32 * w;
    const int pos = tw + swap23(t32);
    const bool valid = pos < L;
    bf16x8 cop[kDc / 16];
    {
        int64_t crow = 0;
        if (valid) crow = static_cast<int64_t>(block_table[static_cast<int64_t>(b) * p.max_pages + pos / 64]) * 64 + pos % 64;
#pragma unroll
        for (int ks = 0; ks < kDc / 16; ++ks) {
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (valid) v = *reinterpret_cast<const u32x4 *>(c_kv + crow * kDc + ks * 16 + g * 8);
            cop[ks] = as_bf16x8(v);
        }
    }

    // Weight chunks reach LDS by direct copies (buffer_load ... lds), three buffers:
    // stage st (pass st / kChunks, chunk st % kChunks) in buffer st % 3, copied two
    // stages ahead.  Row R of a chunk (512 bytes, 32 chunks of 16 bytes) holds
    // logical chunk c at physical chunk c ^ (R % 32); one copy instruction of wave w
    // fills rows 8w + 2i and 8w + 2i + 1, lane l taking physical chunk l % 32 of row
    // 8w + 2i + l / 32.
    const uint32_t lds0 = lds_addr(lds);
    uint32_t voff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int R = 8 * w + 2 * i + (lane >> 5);
        voff[i] = static_cast<uint32_t>(R * kDc * 2 + (((lane & 31) ^ (R & 31)) << 4));
    }
    // passes: (head, keys | values, row half); pass ps covers rows kDecRows*(ps % 2) ..
    constexpr int kHalves = kDh / kDecRows;
    const int h0 = hg * kDecHeads;
    const int n_ps = 2 * kHalves * min(kDecHeads, p.H - h0);
    constexpr int kChunks = kDc / kWChunk;               // stages per pass
    const int n_st = n_ps * kChunks;
    const int rot = (kDecRot * lb_run) % n_ps;
    auto pass_of = [&](int i) { const int q = i + rot; return q >= n_ps ? q - n_ps : q; };
    // copy stage s2 (clamped to the last: the copy past the end refills a buffer no
    // stage reads, so that every stage issues the same number of copies) into buffer
    // `buf`; the descriptor covers one head's matrix
    auto copy_stage = [&](int s2, int buf) {
        s2 = min(s2, n_st - 1);
        const int ps2 = pass_of(s2 / kChunks), hk = ps2 / kHalves;
        const uint16_t *Wh = ((hk & 1) ? W_UV : W_UK) + static_cast<int64_t>(h0 + (hk >> 1)) * kDh * kDc;
        const uint32_t soff = static_cast<uint32_t>((kDecRows * (ps2 % kHalves) * kDc + (s2 % kChunks) * kWChunk) * 2);
        dma_rows4_fixed(Wh, kDh * kDc * 2, lds0 + buf * kWStage + w * 4096, soff, voff[0], voff[1], voff[2], voff[3]);
    };
    // MFMA operand reads: row R = 32dt + x (x = swap23(t32) for the keys' A operand,
    // t32 for the values' B operand), logical chunk 2ks + g -> physical
    // (2ks + g) ^ x, at R*512 + physical*16 = (base ^ (ks << 5)) + dt*16384 with
    // base = x*512 + ((x & 30) << 4) + (((g ^ x) & 1) << 4)
    auto rbase = [&](int x) -> uint32_t {
        return static_cast<uint32_t>(x * 512 + ((x & 30) << 4) + (((g ^ x) & 1) << 4));
    };
    const uint32_t a_base = rbase(swap23(t32));
    const uint32_t b_base = rbase(t32);

    copy_stage(0, 0);
    copy_stage(1, 1);
    for (int ps = 0; ps < n_ps; ++ps) {
        const int pe = pass_of(ps);
        const bool is_v = (pe / kHalves) & 1;
        f32x16 acc[kDecRows / 32];
#pragma unroll
        for (int dt = 0; dt < kDecRows / 32; ++dt)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[dt][j] = 0.f;
#pragma unroll
        for (int kc = 0; kc < kChunks; ++kc) {
            const int st = ps * kChunks + kc;
            // this wave's copies of stage st are complete once at most the copies
            // issued after them are outstanding: those of stage st + 1 (4) and, from
            // the second pass on, the 4 output stores of the pass before
            if (ps == 0) wait_vmcnt<4>();
            else wait_vmcnt<8>();
            // every wave's copies have landed, and every wave is done with buffer
            // (st + 2) % 3 = (st - 1) % 3
            barrier_lds();
            copy_stage(st + 2, (st + 2) % kWBufs);
            const uint32_t buf = lds0 + (st % kWBufs) * kWStage;
            if (is_v) {
                const uint32_t base = buf + b_base;
#pragma unroll
                for (int ks = 0; ks < kWChunk / 16; ++ks)
#pragma unroll
                    for (int dt = 0; dt < kDecRows / 32; ++dt) {
                        const u32x4 wb = lds_load<u32x4>((base ^ (ks << 5)) + dt * 32 * 512);
                        acc[dt] = mfma32(cop[kc * (kWChunk / 16) + ks], as_bf16x8(wb), acc[dt]);
                    }
                read_ahead_schedule();
            } else {
                const uint32_t base = buf + a_base;
#pragma unroll
                for (int ks = 0; ks < kWChunk / 16; ++ks)
#pragma unroll
                    for (int dt = 0; dt < kDecRows / 32; ++dt) {
                        const u32x4 wa = lds_load<u32x4>((base ^ (ks << 5)) + dt * 32 * 512);
                        acc[dt] = mfma32(as_bf16x8(wa), cop[kc * (kWChunk / 16) + ks], acc[dt]);
                    }
                read_ahead_schedule();
            }
        }
        const int h = h0 + pe / (2 * kHalves);
        const int d_base = kDecRows * (pe % kHalves);
        // acc[dt][8hf + e]: keys: dim d_base + 32dt + 16hf + 8g + e of position pos;
        //                   values: position tw + 16hf + 8g + e of dim d_base + 32dt + t32
#pragma unroll
        for (int dt = 0; dt < kDecRows / 32; ++dt)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const u32x4 v = u32x4{cvt_pk_bf16(acc[dt][8 * hf], acc[dt][8 * hf + 1]),
                                      cvt_pk_bf16(acc[dt][8 * hf + 2], acc[dt][8 * hf + 3]),
                                      cvt_pk_bf16(acc[dt][8 * hf + 4], acc[dt][8 * hf + 5]),
                                      cvt_pk_bf16(acc[dt][8 * hf + 6], acc[dt][8 * hf + 7])};
                // unconditional (positions past seq_len hold zero latents, so their rows
                // are written as zeros; the tile ends inside lmax): every pass issues
                // the same 4 stores, which the copy waits above count
                if (!is_v) {
                    *reinterpret_cast<u32x4 *>(k_nope + ((static_cast<int64_t>(b) * lmax + pos) * p.H + h) * kDh +
                                               d_base + 32 * dt + 16 * hf + 8 * g) = v;
                } else {
                    *reinterpret_cast<u32x4 *>(v_t + ((static_cast<int64_t>(b) * p.H + h) * kDh + d_base + 32 * dt + t32) *
                                                         lmax +
                                               tw + 16 * hf + 8 * g) = v;
                }
            }
    }
    // the copies past the end are still in flight: no wave may end (and free the
    // workgroup's LDS) before they have landed
    wait_vmcnt<0>();
}

// ---------------------------------------------------------------------------
// Attention: one workgroup of 8 waves per (sequence, head, 256 new tokens); wave
// w takes 32 of them.  Keys ([content ; RoPE], 192 dims) and transposed values of
// 64 positions at a time are staged once per workgroup in LDS (two stages: the
// next tile's global loads are in flight while the current one is used) and read
// by all 8 waves.
constexpr int kQPerWg = 256;                         // new tokens of one workgroup
constexpr int kKvTile = 64;                          // positions of one stage
constexpr int kKStride = 2 * (kDh + kDr) + 16;       // bytes per key row in LDS (padded: no bank conflicts)
constexpr int kVStride = 2 * kKvTile + 16;           // bytes per value row in LDS (padded)
constexpr int kKBytes = kKvTile * kKStride;
constexpr int kStageBytes = kKBytes + kDh * kVStride;
constexpr float kRescaleLog2 = 8.f;                  // running maximum moves when exceeded by more than this
#ifndef MLA_PREFILL_QT
#define MLA_PREFILL_QT 1
#endif
constexpr int kQT = MLA_PREFILL_QT;                  // 32-query tiles per wave
constexpr int kAttWaves = kQPerWg / (32 * kQT);
constexpr int kAttThreads = 64 * kAttWaves;

template <bool kOutBf16>
__global__ __launch_bounds__(kAttThreads) void prefill_attention_kernel(
    const mla_params_t p, const uint16_t *__restrict__ q_nope, const uint16_t *__restrict__ q_rope,
    const uint16_t *__restrict__ k_nope, const uint16_t *__restrict__ v_t, const uint16_t *__restrict__ k_pe,
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ seq_lens, void *__restrict__ out) {
    __shared__ __attribute__((aligned(16))) char lds[2 * kStageBytes];
    const int tid = threadIdx.x, lane = tid & 63, t32 = lane & 31, g = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n_qb = (p.Sq + kQPerWg - 1) / kQPerWg;
    const int64_t lmax = prefill_lmax(p);
    // Block order: the blocks of one (sequence, head) are consecutive and the
    // heaviest (latest new tokens) first; with a multiple of 8 blocks, XCD x (which
    // receives blocks x, x+8, ...) gets one contiguous range of that order, so the
    // blocks sharing a head's keys and values run together on one L2.
    const int64_t nblk = gridDim.x;
    int64_t lb = blockIdx.x;
    if ((nblk & 7) == 0) lb = (lb & 7) * (nblk >> 3) + (lb >> 3);
    const int qb = n_qb - 1 - static_cast<int>(lb % n_qb);
    lb /= n_qb;
    const int h = static_cast<int>(lb % p.H);
    const int b = static_cast<int>(lb / p.H);
    const int L = seq_lens[b];
    const int base = L - p.Sq;                           // position of new token 0
    const int q0 = qb * kQPerWg;
    const int s0 = q0 + 32 * kQT * w;                    // this wave's first new token; tile qt: s0 + 32 qt
    const int pos_wave = base + min(s0 + 32 * kQT - 1, p.Sq - 1);  // last position any query of the wave sees
    const int pos_wg = base + min(q0 + kQPerWg - 1, p.Sq - 1);
    const int n_tiles = pos_wg >= 0 ? pos_wg / kKvTile + 1 : 0;
    int pos_q[kQT];                                      // last position this lane's query of tile qt sees
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) pos_q[qt] = base + s0 + 32 * qt + t32;

    auto store_out = [&](int qt, const f32x16 *o, float inv) {
        const int s = s0 + 32 * qt + t32;
        if (s >= p.Sq) return;
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
    };
    f32x16 o[kQT][4];                                    // O^T tiles: dims 32dt + .., query of tile qt
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int j = 0; j < 16; ++j) o[qt][dt][j] = 0.f;
    if (n_tiles == 0) {                                  // no new token of the block sees any position
#pragma unroll
        for (int qt = 0; qt < kQT; ++qt) store_out(qt, o[qt], 0.f);
        return;
    }

    // Q^T (B operand) of each tile: k-steps 0..7 the content dims, 8..11 the RoPE dims
    bf16x8 qreg[kQT][12];
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) {
        const int s = s0 + 32 * qt + t32;
        const bool q_ok = s < p.Sq;
        const int64_t qrow = (static_cast<int64_t>(b) * p.Sq + (q_ok ? s : 0)) * p.H + h;
#pragma unroll
        for (int ks = 0; ks < 12; ++ks) {
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (q_ok) {
                if (ks < 8) v = *reinterpret_cast<const u32x4 *>(q_nope + qrow * kDh + ks * 16 + g * 8);
                else v = *reinterpret_cast<const u32x4 *>(q_rope + qrow * kDr + (ks - 8) * 16 + g * 8);
            }
            qreg[qt][ks] = as_bf16x8(v);
        }
    }

    // Staging: a tile is 64 key rows of 16 content chunks and 8 RoPE chunks, and 128
    // value rows of 8 chunks (16 bytes each); thread tid moves content chunk tid%16
    // of rows tid/16 + (T/16)i, RoPE chunk tid%8 of rows tid/8 + (T/8)i and value
    // chunk tid%8 of rows tid/8 + (T/8)i (T threads).  Every row of a tile lies
    // inside lmax; rows past seq_len are masked in the scores (keys) or zeroed when
    // staged (values), and a tile is one page, so its RoPE rows are rows of that page.
    constexpr int kNK = 1024 / kAttThreads, kNR = 512 / kAttThreads, kNV = 1024 / kAttThreads;
    const int32_t *bt = block_table + static_cast<int64_t>(b) * p.max_pages;
    const int kr = tid >> 4, kc = tid & 15, rr = tid >> 3, rc = tid & 7;
    const int64_t kstride = static_cast<int64_t>(p.H) * kDh;      // elements per key position
    const uint16_t *kptr = k_nope + (static_cast<int64_t>(b) * lmax * p.H + h) * kDh + kr * kstride + kc * 8;
    const uint16_t *vptr = v_t + ((static_cast<int64_t>(b) * p.H + h) * kDh + rr) * lmax + rc * 8;
    const uint16_t *rptr = k_pe + rr * kDr + rc * 8;
    u32x4 stg_k[kNK], stg_r[kNR], stg_v[kNV];
    auto load_tile = [&](int k0, int page) {
        const uint16_t *kp = kptr + k0 * kstride;
#pragma unroll
        for (int i = 0; i < kNK; ++i)
            stg_k[i] = *reinterpret_cast<const u32x4 *>(kp + (kAttThreads / 16) * i * kstride);
#pragma unroll
        for (int i = 0; i < kNR; ++i)
            stg_r[i] = *reinterpret_cast<const u32x4 *>(rptr + (static_cast<int64_t>(page) * 64 + (kAttThreads / 8) * i) * kDr);
#pragma unroll
        for (int i = 0; i < kNV; ++i)
            stg_v[i] = *reinterpret_cast<const u32x4 *>(vptr + (kAttThreads / 8) * i * lmax + k0);
    };
    const uint32_t lds0 = lds_addr(lds);
    auto store_tile = [&](int k0, int stage) {
        const int pv = k0 + rc * 8;
        if (pv + 8 > L) {                                // values past the sequence end: zeros (finite)
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const uint32_t keep = (pv + 2 * e2 < L ? 0x0000ffffu : 0u) | (pv + 2 * e2 + 1 < L ? 0xffff0000u : 0u);
#pragma unroll
                for (int i = 0; i < kNV; ++i) stg_v[i][e2] &= keep;
            }
        }
        const uint32_t st = lds0 + stage * kStageBytes;
#pragma unroll
        for (int i = 0; i < kNK; ++i) lds_store<u32x4>(st + (kr + (kAttThreads / 16) * i) * kKStride + kc * 16, stg_k[i]);
#pragma unroll
        for (int i = 0; i < kNR; ++i)
            lds_store<u32x4>(st + (rr + (kAttThreads / 8) * i) * kKStride + 2 * kDh + rc * 16, stg_r[i]);
#pragma unroll
        for (int i = 0; i < kNV; ++i)
            lds_store<u32x4>(st + kKBytes + (rr + (kAttThreads / 8) * i) * kVStride + rc * 16, stg_v[i]);
    };

    const float zscale = p.scale * kLog2e;
    float m_run[kQT], l_run[kQT];                        // running maximum (log2 domain) and weight sum
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) {
        m_run[qt] = -INFINITY;
        l_run[qt] = 0.f;
    }
    // key operand rows of this lane: tile rows swap23(t32) and 32 + swap23(t32)
    const uint32_t k_off = swap23(t32) * kKStride + g * 16;
    const uint32_t v_off = kKBytes + t32 * kVStride + g * 16;

    load_tile(0, bt[0]);
    int page_next = n_tiles > 1 ? bt[1] : 0;             // page of the next tile, read one tile ahead
    store_tile(0, 0);
    __syncthreads();
    for (int kt = 0; kt < n_tiles; ++kt) {
        const int k0 = kt * kKvTile;
        const bool more = kt + 1 < n_tiles;
        if (more) load_tile(k0 + kKvTile, page_next);
        if (s0 < p.Sq && k0 <= pos_wave) {
            const uint32_t st = lds0 + (kt & 1) * kStageBytes;
            // the tile in two halves of 32 positions: scores, softmax, value product
#pragma unroll
            for (int ps = 0; ps < 2; ++ps) {
                const int kh = k0 + 32 * ps;                 // first position of the half
                // S^T[t, q] for positions kh + swap23(row); each key operand serves
                // every query tile of the wave
                f32x16 sacc[kQT];
#pragma unroll
                for (int qt = 0; qt < kQT; ++qt)
#pragma unroll
                    for (int j = 0; j < 16; ++j) sacc[qt][j] = 0.f;
#pragma unroll
                for (int ks = 0; ks < 12; ++ks) {
                    const u32x4 a = lds_load<u32x4>(st + k_off + ps * 32 * kKStride + ks * 32);
#pragma unroll
                    for (int qt = 0; qt < kQT; ++qt) sacc[qt] = mfma32(as_bf16x8(a), qreg[qt][ks], sacc[qt]);
                }
                uint32_t pk[kQT][2][4];
#pragma unroll
                for (int qt = 0; qt < kQT; ++qt) {
                    // sacc[qt][j]: position kh + 16(j/8) + 8g + (j%8); the maximum is
                    // taken on the raw scores (the scale is positive)
                    float mt = -INFINITY;
                    if (kh + 31 > base + s0 + 32 * qt || kh + 32 > L) {
                        // the half reaches past the tile's first query position or the sequence end
                        const int lim = min(pos_q[qt], L - 1) - (kh + 8 * g);
#pragma unroll
                        for (int j = 0; j < 16; ++j) {
                            const int rel = 16 * (j >> 3) + (j & 7);
                            sacc[qt][j] = rel <= lim ? sacc[qt][j] : -INFINITY;
                            mt = fmaxf(mt, sacc[qt][j]);
                        }
                    } else {
#pragma unroll
                        for (int j = 0; j < 16; ++j) mt = fmaxf(mt, sacc[qt][j]);
                    }
                    mt = pair_max(mt) * zscale;          // log2 domain
                    // the running maximum moves only when this half's exceeds it by more
                    // than kRescaleLog2, so the weights stay below 2^kRescaleLog2 and the
                    // rescale of the accumulators is skipped on most halves
                    const bool grow = mt > m_run[qt] + kRescaleLog2;
                    if (__builtin_amdgcn_ballot_w64(grow)) {
                        const float alpha = grow ? __builtin_amdgcn_exp2f(m_run[qt] - mt) : 1.f;   // 0 the first time
                        m_run[qt] = grow ? mt : m_run[qt];
                        l_run[qt] *= alpha;
#pragma unroll
                        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                            for (int j = 0; j < 16; ++j) o[qt][dt][j] *= alpha;
                    }
                    const float m_neg = m_run[qt] == -INFINITY ? 0.f : -m_run[qt];   // nothing visible yet: weights 0
                    // weights exp2(scale * z - m), rounded to bf16; k-step kk of the value
                    // product takes positions kh + 16kk + 8g + e, which are sacc[qt][8kk + e]
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                        for (int e2 = 0; e2 < 4; ++e2) {
                            const int j = 8 * kk + 2 * e2;
                            const uint32_t pr =
                                cvt_pk_bf16(__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qt][j], zscale, m_neg)),
                                            __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qt][j + 1], zscale, m_neg)));
                            pk[qt][kk][e2] = pr;
                            l_run[qt] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pr),
                                                                        bf16x2{(__bf16)1.f, (__bf16)1.f}, l_run[qt],
                                                                        false);
                        }
                }
                // O^T[d, q] += V^T[d, t] . P^T[t, q]; each value operand serves every query tile
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt) {
                        const u32x4 a = lds_load<u32x4>(st + v_off + dt * 32 * kVStride + (2 * ps + kk) * 32);
#pragma unroll
                        for (int qt = 0; qt < kQT; ++qt)
                            o[qt][dt] = mfma32(
                                as_bf16x8(a),
                                as_bf16x8(u32x4{pk[qt][kk][0], pk[qt][kk][1], pk[qt][kk][2], pk[qt][kk][3]}),
                                o[qt][dt]);
                    }
            }
        }
        if (more) {
            page_next = kt + 2 < n_tiles ? bt[kt + 2] : 0;
            store_tile(k0 + kKvTile, (kt + 1) & 1);
        }
        __syncthreads();
    }
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) {
        const float l_tot = pair_sum(l_run[qt]);
        store_out(qt, o[qt], l_tot > 0.f ? 1.f / l_tot : 0.f);
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
    const int64_t n_hg = (p.H + kDecHeads - 1) / kDecHeads;
    const int64_t n_pt = (static_cast<int64_t>(p.max_pages) * 64 + kDecPos - 1) / kDecPos;
    const int64_t blocks = n_hg * p.B * n_pt;
    hipLaunchKernelGGL(decompress_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kDecThreads), 0, stream, p,
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
    static_assert(kQPerWg == 256, "the host's grid check assumes 256 new tokens per workgroup");
    const auto qn = static_cast<const uint16_t *>(q_nope);
    const auto qr = static_cast<const uint16_t *>(q_rope);
    const auto kn = static_cast<const uint16_t *>(k_nope);
    const auto vt = static_cast<const uint16_t *>(v_t);
    const auto kp = static_cast<const uint16_t *>(k_pe);
    if (p.out_dtype == MLA_BF16)
        hipLaunchKernelGGL(prefill_attention_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(kAttThreads), 0, stream,
                           p, qn, qr, kn, vt, kp, block_table, seq_lens, out);
    else
        hipLaunchKernelGGL(prefill_attention_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(kAttThreads), 0, stream,
                           p, qn, qr, kn, vt, kp, block_table, seq_lens, out);
    return hipGetLastError();
}

}  // namespace mla
