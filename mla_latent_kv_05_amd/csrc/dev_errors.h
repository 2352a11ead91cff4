// Device error word of the kernels of one translation unit (bits MLA_DEVERR_* of
// mla.h).  Kernels set bits with raise_error; mla_device_errors reads and clears
// the word of every unit through its take_errors_* function.  Each unit that
// includes this header has its own word.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla.h"

namespace mla {

static __device__ uint32_t dev_errors;

__device__ __forceinline__ void raise_error(uint32_t bit) { atomicOr(&dev_errors, bit); }

// Pages of a sequence of `len` tokens (pages of 64).  The MLA_DEBUG_BOUNDS build
// checks len against a block-table row (0 .. max_pages pages), flags a violation
// and clamps it.
__device__ __forceinline__ int seq_pages(const mla_params_t &p, int len) {
#ifdef MLA_DEBUG_BOUNDS
    if (len < 0 || len > p.max_pages * 64) {
        raise_error(MLA_DEVERR_SEQLEN);
        len = len < 0 ? 0 : p.max_pages * 64;
    }
#else
    (void)p;
#endif
    return (len + 63) / 64;
}

// A physical page from the block table.  The MLA_DEBUG_BOUNDS build checks it
// against the cache's pages, flags a violation and substitutes page 0.
__device__ __forceinline__ int checked_page(const mla_params_t &p, int page) {
#ifdef MLA_DEBUG_BOUNDS
    if (page < 0 || page >= p.num_pages) {
        raise_error(MLA_DEVERR_PAGE);
        page = 0;
    }
#else
    (void)p;
#endif
    return page;
}

// Host side: this unit's word, then zero it (synchronous copies).
static inline hipError_t take_unit_errors(uint32_t *bits) {
    uint32_t v = 0, zero = 0;
    hipError_t e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(dev_errors), sizeof(v), 0, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return e;
    if (v) e = hipMemcpyToSymbol(HIP_SYMBOL(dev_errors), &zero, sizeof(zero), 0, hipMemcpyHostToDevice);
    *bits |= v;
    return e;
}

}  // namespace mla
