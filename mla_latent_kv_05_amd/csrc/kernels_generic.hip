// fp32 VALU kernels for absorbed-MLA decode: any supported dims and dtypes.
//
// These serve shapes the MFMA kernels do not cover (e.g. H=8, d_h=32,
// d_c=64, d_r=16 in fp32) and act as a second, independently written HIP
// implementation that tests can force with MLA_FLAG_GENERIC.  They are plain
// and correct rather than fast; the DeepSeek-V3 shapes use kernels_mfma.hip.
#include <hip/hip_runtime.h>
#include <math.h>

#include "dev_errors.h"
#include "dtype.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxDc = 1024;
constexpr int kMaxDr = 256;
constexpr int kMaxDh = 256;
constexpr int kColsPerThread = kMaxDc / kThreads;

__device__ __forceinline__ float block_reduce_max(float v, float *red) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float r = red[0];
    for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, red[i]);
    return r;
}

__device__ __forceinline__ float block_reduce_sum(float v, float *red) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float r = red[0];
    for (int i = 1; i < kThreads / 64; ++i) r += red[i];
    return r;
}

__device__ __forceinline__ int64_t block_reduce_sum_i64(int64_t v, int64_t *red) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    int64_t r = red[0];
    for (int i = 1; i < kThreads / 64; ++i) r += red[i];
    return r;
}

// Pages [*pa, *pb) of sequence b that split c covers (empty when *pa >= *pb).
// Fixed splits: [c*split_pages, (c+1)*split_pages).  Balanced splits: the
// batch's work units (kSeqStartCost + n for a sequence of n > 0 pages, start cost
// first) in sequence order are cut into num_parts parts, part j holding units
// [floor(j*T/P), floor((j+1)*T/P)); split c of b is its pages in part j0 + c, j0
// being the part that holds b's first page.
__device__ void split_pages_of(const mla_params_t &p, const int32_t *__restrict__ seq_lens, int b, int c,
                               int64_t *pa, int64_t *pb, int64_t *red) {
    const int64_t pages = seq_pages(p, seq_lens[b]);
    if (p.num_parts == 0) {
        *pa = static_cast<int64_t>(c) * p.split_pages;
        *pb = *pa + p.split_pages;
        if (*pb > pages) *pb = pages;
        return;
    }
    int64_t tot = 0, before = 0;
    for (int i = threadIdx.x; i < p.B; i += kThreads) {
        const int64_t n = seq_pages(p, seq_lens[i]);
        const int64_t units = n > 0 ? n + kSeqStartCost : 0;
        tot += units;
        if (i < b) before += units;
    }
    const int64_t T = block_reduce_sum_i64(tot, red);
    const int64_t off = block_reduce_sum_i64(before, red) + kSeqStartCost;   // unit of b's first page
    *pa = 0;
    *pb = 0;
    if (pages == 0) return;
    const int64_t P = p.num_parts;
    const int64_t j0 = ((off + 1) * P - 1) / T;           // part holding b's first page
    if (c == p.num_splits - 1 && threadIdx.x == 0 && ((off + pages) * P - 1) / T - j0 >= p.num_splits)
        raise_error(MLA_DEVERR_SPLITS);                   // pages in more parts than num_splits
    const int64_t j = j0 + c;
    if (j >= P) return;
    const int64_t lo = j * T / P - off, hi = (j + 1) * T / P - off;
    *pa = lo > 0 ? lo : 0;
    *pb = hi < pages ? hi : pages;
}

// q_abs[row, m] = sum_d q_nope[row, d] * W_UK[h, d, m]; one block per (b,s,h) row.
__global__ __launch_bounds__(kThreads) void absorb_generic_kernel(
    mla_params_t p, const void *__restrict__ q_nope, const void *__restrict__ W_UK,
    void *__restrict__ q_abs) {
    __shared__ float q[kMaxDh];
    const int64_t row = blockIdx.x;
    const int h = static_cast<int>(row % p.H);
    for (int d = threadIdx.x; d < p.d_h; d += kThreads)
        q[d] = load_elem(q_nope, p.q_dtype, row * p.d_h + d);
    __syncthreads();
    for (int m = threadIdx.x; m < p.d_c; m += kThreads) {
        float acc = 0.f;
        for (int d = 0; d < p.d_h; ++d)
            acc += q[d] * load_elem(W_UK, p.w_dtype, (static_cast<int64_t>(h) * p.d_h + d) * p.d_c + m);
        store_elem(q_abs, p.latent_dtype, row * p.d_c + m, acc);
    }
}

// One block per ((b,s,h) row, split).  Positions are processed 256 at a time:
// every thread scores one position, the block updates a running max / sum
// (online softmax) and every thread accumulates its own latent columns.
__global__ __launch_bounds__(kThreads) void decode_generic_kernel(
    mla_params_t p, const void *__restrict__ q_abs, const void *__restrict__ q_rope,
    const void *__restrict__ c_kv, const void *__restrict__ k_pe,
    const float *__restrict__ kv_scale, const int32_t *__restrict__ block_table,
    const int32_t *__restrict__ seq_lens, void *__restrict__ o_part,
    float *__restrict__ lse_part) {
    __shared__ float qa[kMaxDc];
    __shared__ float qr[kMaxDr];
    __shared__ float pw[kThreads];
    __shared__ int64_t prow[kThreads];
    __shared__ float red[kThreads / 64];
    __shared__ int64_t red64[kThreads / 64];

    const int S = p.num_splits;
    const int64_t row = blockIdx.x / S;
    const int c = static_cast<int>(blockIdx.x % S);
    const int b = static_cast<int>(row / (static_cast<int64_t>(p.Sq) * p.H));
    const int s = static_cast<int>((row / p.H) % p.Sq);
    const int64_t n = static_cast<int64_t>(seq_lens[b]) - p.Sq + 1 + s;   // visible positions
    int64_t pa, pb;
    split_pages_of(p, seq_lens, b, c, &pa, &pb, red64);
    const int64_t t0 = pa * p.page_size;
    int64_t t1 = pb * p.page_size;
    if (t1 > n) t1 = n;
    const int64_t out_idx = row * S + c;
    if (t1 <= t0) {
        if (threadIdx.x == 0) lse_part[out_idx] = -INFINITY;
        return;
    }
    for (int m = threadIdx.x; m < p.d_c; m += kThreads) qa[m] = load_elem(q_abs, p.latent_dtype, row * p.d_c + m);
    for (int r = threadIdx.x; r < p.d_r; r += kThreads) qr[r] = load_elem(q_rope, p.q_dtype, row * p.d_r + r);
    __syncthreads();

    float acc[kColsPerThread];
#pragma unroll
    for (int k = 0; k < kColsPerThread; ++k) acc[k] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const int32_t *bt = block_table + static_cast<int64_t>(b) * p.max_pages;

    for (int64_t tb = t0; tb < t1; tb += kThreads) {
        const int64_t t = tb + threadIdx.x;
        float z = -INFINITY;
        int64_t crow = 0;
        if (t < t1) {
            crow = static_cast<int64_t>(checked_page(p, bt[t / p.page_size])) * p.page_size + t % p.page_size;
            float content = 0.f, rope = 0.f;
            for (int m = 0; m < p.d_c; ++m) content += qa[m] * load_elem(c_kv, p.kv_dtype, crow * p.d_c + m);
            if (p.kv_dtype == MLA_FP8_E4M3) content *= kv_scale[crow];
            for (int r = 0; r < p.d_r; ++r) rope += qr[r] * load_elem(k_pe, p.pe_dtype, crow * p.d_r + r);
            z = p.scale * (content + rope);
        }
        const float cmax = block_reduce_max(z, red);
        const float m_new = fmaxf(m_run, cmax);                 // finite: t0 < t1
        const float alpha = __expf(m_run - m_new);              // 0 on the first chunk
        const float pt = (t < t1) ? __expf(z - m_new) : 0.f;
        const float csum = block_reduce_sum(pt, red);
        l_run = l_run * alpha + csum;
        m_run = m_new;
        // fp8: fold the token's scale into its weight
        pw[threadIdx.x] = (t < t1 && p.kv_dtype == MLA_FP8_E4M3) ? pt * kv_scale[crow] : pt;
        prow[threadIdx.x] = crow;
        __syncthreads();
        const int cnt = static_cast<int>((t1 - tb) < kThreads ? (t1 - tb) : kThreads);
#pragma unroll
        for (int k = 0; k < kColsPerThread; ++k) {
            const int m = threadIdx.x + k * kThreads;
            if (m < p.d_c) {
                float a = acc[k] * alpha;
                for (int j = 0; j < cnt; ++j) a += pw[j] * load_elem(c_kv, p.kv_dtype, prow[j] * p.d_c + m);
                acc[k] = a;
            }
        }
        __syncthreads();
    }
    const float inv = 1.f / l_run;
#pragma unroll
    for (int k = 0; k < kColsPerThread; ++k) {
        const int m = threadIdx.x + k * kThreads;
        if (m < p.d_c) store_elem(o_part, p.part_dtype, out_idx * p.d_c + m, acc[k] * inv);
    }
    if (threadIdx.x == 0) lse_part[out_idx] = m_run + logf(l_run);
}

// out[row, d] = sum_m o_latent[row, m] * W_UV[h, d, m]; one wave per output element.
__global__ __launch_bounds__(kThreads) void up_v_generic_kernel(
    mla_params_t p, const void *__restrict__ o_latent, const void *__restrict__ W_UV,
    void *__restrict__ out) {
    __shared__ float o[kMaxDc];
    const int64_t row = blockIdx.x;
    const int h = static_cast<int>(row % p.H);
    for (int m = threadIdx.x; m < p.d_c; m += kThreads) o[m] = load_elem(o_latent, p.latent_dtype, row * p.d_c + m);
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int d = wave; d < p.d_h; d += kThreads / 64) {
        const int64_t wbase = (static_cast<int64_t>(h) * p.d_h + d) * p.d_c;
        float acc = 0.f;
        for (int m = lane; m < p.d_c; m += 64) acc += o[m] * load_elem(W_UV, p.w_dtype, wbase + m);
        for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
        if (lane == 0) store_elem(out, p.out_dtype, row * p.d_h + d, acc);
    }
}

// Log-sum-exp merge: one block per (b,s,h) row.
constexpr int kMaxSplits = 4096;

__global__ __launch_bounds__(kThreads) void combine_kernel(
    mla_params_t p, const void *__restrict__ o_part, const float *__restrict__ lse_part,
    void *__restrict__ o_latent, float *__restrict__ lse_out) {
    __shared__ float w[kMaxSplits];
    __shared__ float red[kThreads / 64];
    const int S = p.num_splits;
    const int64_t row = blockIdx.x;
    const float *l = lse_part + row * S;
    float mx = -INFINITY;
    for (int c = threadIdx.x; c < S; c += kThreads) mx = fmaxf(mx, l[c]);
    mx = block_reduce_max(mx, red);
    if (mx == -INFINITY) {                                   // nothing visible
        for (int m = threadIdx.x; m < p.d_c; m += kThreads) store_elem(o_latent, p.latent_dtype, row * p.d_c + m, 0.f);
        if (lse_out && threadIdx.x == 0) lse_out[row] = -INFINITY;
        return;
    }
    float sum = 0.f;
    for (int c = threadIdx.x; c < S; c += kThreads) {
        const float e = (l[c] == -INFINITY) ? 0.f : __expf(l[c] - mx);
        w[c] = e;
        sum += e;
    }
    sum = block_reduce_sum(sum, red);                        // also orders the w[] writes
    const float inv = 1.f / sum;
    const int64_t op = row * static_cast<int64_t>(S) * p.d_c;
    for (int m = threadIdx.x; m < p.d_c; m += kThreads) {
        float acc = 0.f;
        for (int c = 0; c < S; ++c)
            if (w[c] != 0.f) acc += w[c] * load_elem(o_part, p.part_dtype, op + static_cast<int64_t>(c) * p.d_c + m);
        store_elem(o_latent, p.latent_dtype, row * p.d_c + m, acc * inv);
    }
    if (lse_out && threadIdx.x == 0) lse_out[row] = mx + logf(sum);
}

}  // namespace

static_assert(kMaxSplits >= 1, "");

hipError_t launch_absorb_generic(const mla_params_t &p, const void *q_nope, const void *W_UK,
                                 void *q_abs, hipStream_t stream) {
    const int64_t rows = static_cast<int64_t>(p.B) * p.Sq * p.H;
    hipLaunchKernelGGL(absorb_generic_kernel, dim3(static_cast<unsigned>(rows)), dim3(kThreads), 0, stream,
                       p, q_nope, W_UK, q_abs);
    return hipGetLastError();
}

hipError_t launch_decode_generic(const mla_params_t &p, const void *q_abs, const void *q_rope,
                                 const void *c_kv, const void *k_pe, const float *kv_scale,
                                 const int32_t *block_table, const int32_t *seq_lens,
                                 void *o_part, float *lse_part, hipStream_t stream) {
    const int64_t blocks = static_cast<int64_t>(p.B) * p.Sq * p.H * p.num_splits;
    hipLaunchKernelGGL(decode_generic_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream,
                       p, q_abs, q_rope, c_kv, k_pe, kv_scale, block_table, seq_lens, o_part, lse_part);
    return hipGetLastError();
}

hipError_t launch_up_v_generic(const mla_params_t &p, const void *o_latent, const void *W_UV,
                               void *out, hipStream_t stream) {
    const int64_t rows = static_cast<int64_t>(p.B) * p.Sq * p.H;
    hipLaunchKernelGGL(up_v_generic_kernel, dim3(static_cast<unsigned>(rows)), dim3(kThreads), 0, stream,
                       p, o_latent, W_UV, out);
    return hipGetLastError();
}

hipError_t launch_combine(const mla_params_t &p, const void *o_part, const float *lse_part,
                          void *o_latent, float *lse_out, hipStream_t stream) {
    const int64_t rows = static_cast<int64_t>(p.B) * p.Sq * p.H;
    hipLaunchKernelGGL(combine_kernel, dim3(static_cast<unsigned>(rows)), dim3(kThreads), 0, stream,
                       p, o_part, lse_part, o_latent, lse_out);
    return hipGetLastError();
}

hipError_t take_errors_generic(uint32_t *bits) { return take_unit_errors(bits); }

}  // namespace mla
