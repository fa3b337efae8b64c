// Byte layout of one packed expert ("slot image"); the public description is in moe.h.
// Shared by the host packer, the cache and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// bytes of one 16-row block of a [R, K] matrix (fragments, then int4 scales)
__host__ __device__ inline size_t rowblock_bytes(int K, moe_dtype w) {
    switch (w) {
        case MOE_F32: return (size_t)16 * K * 4;
        case MOE_BF16: return (size_t)16 * K * 2;
        case MOE_INT4_G128: return (size_t)8 * K + (size_t)32 * (K / 128);
    }
    return 0;
}

// offset of the gate (which=0) or up (which=1) block b of the [f, d] matrices
__host__ __device__ inline size_t gu_block_offset(int b, int which, int d, moe_dtype w) {
    return (size_t)(2 * b + which) * rowblock_bytes(d, w);
}

// offset of block b of the [d, f] down matrix
__host__ __device__ inline size_t down_block_offset(int b, int d, int f, moe_dtype w) {
    return (size_t)(2 * (f / 16)) * rowblock_bytes(d, w) + (size_t)b * rowblock_bytes(f, w);
}

inline bool slot_shape_ok(int d, int f, moe_dtype w) {
    int q = (w == MOE_INT4_G128) ? 128 : 32;
    if (w != MOE_F32 && w != MOE_BF16 && w != MOE_INT4_G128) return false;
    return d >= 64 && f >= 64 && d <= 16384 && f <= 16384 && d % q == 0 && f % q == 0;
}

inline size_t slot_bytes_raw(int d, int f, moe_dtype w) {
    return (size_t)(2 * (f / 16)) * rowblock_bytes(d, w) + (size_t)(d / 16) * rowblock_bytes(f, w);
}

}  // namespace moe
