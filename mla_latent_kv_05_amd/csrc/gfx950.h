// Device helpers shared by the MFMA kernels (gfx950 / CDNA4): vector types,
// MFMA wrappers, bf16 packing, LDS address-space access and waits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {
namespace gfx {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
#define MLA_LDS_AS __attribute__((address_space(3)))

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_lo(uint32_t lo_src, uint32_t hi_src) {
    return __builtin_amdgcn_perm(hi_src, lo_src, 0x05040100u);   // {lo_src.lo16, hi_src.lo16}
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t lo_src, uint32_t hi_src) {
    return __builtin_amdgcn_perm(hi_src, lo_src, 0x07060302u);   // {lo_src.hi16, hi_src.hi16}
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// generic pointer to a __shared__ object -> LDS byte address
__device__ __forceinline__ uint32_t lds_addr(void *p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((MLA_LDS_AS char *)(p)));
}

template <typename T>
__device__ __forceinline__ T lds_load(uint32_t addr) {
    return *reinterpret_cast<const MLA_LDS_AS T *>(static_cast<uintptr_t>(addr));
}
template <typename T>
__device__ __forceinline__ void lds_store(uint32_t addr, const T &v) {
    *reinterpret_cast<MLA_LDS_AS T *>(static_cast<uintptr_t>(addr)) = v;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier without the release fence of __syncthreads(): the fence
// would also wait for the global->LDS copies in flight (vmcnt(0)).  The
// wave's own LDS traffic is drained first, so after the barrier every wave's
// earlier LDS reads and writes are complete.
__device__ __forceinline__ void barrier_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Reductions over lanes l and l ^ 32 with v_permlane32_swap (no LDS round
// trip).  Swapping a register with itself leaves, in every lane, x[l] in one
// of the two results and x[l ^ 32] in the other; a symmetric operation on the
// pair gives the same value in both lanes.
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace gfx
}  // namespace mla
