// Element loads/stores for the storage formats of the C ABI (device side).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// bf16 is the upper half of an IEEE binary32.
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// OCP E4M3 (bias 7, no infinities; S.1111.111 is NaN) -> fp32, exact.
__device__ __forceinline__ float e4m3_to_f32(uint8_t c) {
    const uint32_t sign = static_cast<uint32_t>(c & 0x80u) << 24;
    const uint32_t e = (c >> 3) & 0xfu;
    const uint32_t m = c & 0x7u;
    float v;
    if (e == 0) {
        v = static_cast<float>(m) * 0.001953125f;          // m * 2^-9
    } else if (e == 0xfu && m == 0x7u) {
        v = __uint_as_float(0x7fc00000u);
    } else {
        v = __uint_as_float(((e + 120u) << 23) | (m << 20));  // (1 + m/8) * 2^(e-7)
    }
    return __uint_as_float(__float_as_uint(v) | sign);
}

// Load element i of a tensor stored as dtype `dt` (MLA_F32 / MLA_BF16 / MLA_FP8_E4M3).
__device__ __forceinline__ float load_elem(const void *p, int dt, int64_t i) {
    if (dt == 0) return static_cast<const float *>(p)[i];
    if (dt == 1) return bf16_bits_to_f32(static_cast<const uint16_t *>(p)[i]);
    return e4m3_to_f32(static_cast<const uint8_t *>(p)[i]);
}

__device__ __forceinline__ void store_elem(void *p, int dt, int64_t i, float v) {
    if (dt == 0) static_cast<float *>(p)[i] = v;
    else static_cast<uint16_t *>(p)[i] = f32_to_bf16_bits(v);
}

}  // namespace mla
