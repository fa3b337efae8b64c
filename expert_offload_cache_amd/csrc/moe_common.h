// Shared host/device helpers of libmoe (gfx950).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "moe.h"

namespace moe {

// ---- error reporting -------------------------------------------------------------------------
moe_status set_error(moe_status code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
moe_status hip_error(hipError_t e, const char* what);

#define MOE_HIP(call)                                      \
    do {                                                   \
        hipError_t e_ = (call);                            \
        if (e_ != hipSuccess) return moe::hip_error(e_, #call); \
    } while (0)

#define MOE_CHECK(cond, code, ...)                                  \
    do {                                                            \
        if (!(cond)) return moe::set_error((code), __VA_ARGS__);    \
    } while (0)

// Check the launch that just happened (launch-configuration errors only; faults are async).
moe_status check_launch(const char* kernel);

// ---- kernel timing (moe_profile_*) -----------------------------------------------------------
bool profiling_on();
void prof_begin(const char* kernel, hipStream_t s);
void prof_end(hipStream_t s);

struct ProfScope {
    hipStream_t s;
    bool on;
    ProfScope(const char* kernel, hipStream_t st) : s(st), on(profiling_on()) {
        if (on) prof_begin(kernel, s);
    }
    ~ProfScope() {
        if (on) prof_end(s);
    }
};

// ---- number formats ----------------------------------------------------------------------------
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));  // native vector: stays in registers

__host__ __device__ inline float as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__host__ __device__ inline uint32_t as_u32(float f) { return __builtin_bit_cast(uint32_t, f); }
__host__ __device__ inline float bf16_lo(uint32_t w) { return as_f32(w << 16); }
__host__ __device__ inline float bf16_hi(uint32_t w) { return as_f32(w & 0xFFFF0000u); }
__host__ __device__ inline float bf16_to_f32(uint16_t h) { return as_f32(((uint32_t)h) << 16); }

// round to nearest even; NaN stays NaN
__host__ __device__ inline uint16_t f32_to_bf16(float f) {
    uint32_t u = as_u32(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---- cross-lane sums without LDS (gfx950) -------------------------------------------------------
// Each returns v[lane] + v[lane ^ s] in every lane.  Floating-point addition is commutative, so the
// two lanes of a pair hold identical bits afterwards, which the fixed-order reductions rely on.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float pair_sum1(float v) { return v + dpp_move<0xB1>(v); }  // quad_perm [1,0,3,2]
__device__ __forceinline__ float pair_sum2(float v) { return v + dpp_move<0x4E>(v); }  // quad_perm [2,3,0,1]
// lane i <-> 7-i within 8 lanes: the partner quad; valid when each quad is already uniform
__device__ __forceinline__ float pair_sum4_uniform(float v) { return v + dpp_move<0x141>(v); }
// lane i <-> 15-i within 16 lanes: the partner 8-lane group; valid when each group is uniform
__device__ __forceinline__ float pair_sum8_uniform(float v) { return v + dpp_move<0x140>(v); }
// v_permlane16/32_swap exchange rows of two registers.  Swapping v against a zero register
// gives, in each result pair, v of a row and v of its partner row, so r0 + r1 is the pair sum in
// the lanes that keep their own row: lanes 0-15 and 32-47 (stride 16), lanes 0-31 (stride 32).
// (The two results are copied to scalars before reinterpreting: a bit cast applied directly to
// a vector-element expression picked up element 0 for both.)
__device__ __forceinline__ float pair_sum16_low(float v) {
    auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, v), 0u, false, false);
    const unsigned r0 = r[0], r1 = r[1];
    return as_f32(r0) + as_f32(r1);
}
__device__ __forceinline__ float pair_sum32_low(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v), 0u, false, false);
    const unsigned r0 = r[0], r1 = r[1];
    return as_f32(r0) + as_f32(r1);
}
// Sum of the four row quarters (lanes r, r+16, r+32, r+48), valid in lanes 0-15.
__device__ __forceinline__ float quarter_sum_low(float v) { return pair_sum32_low(pair_sum16_low(v)); }
// Pairwise sum of the 64 lane values, neighbours first (strides 1, 2, ..., 32), valid in
// lanes 0-15: level m+1 of the tree adds the two level-m sums of adjacent 2^m-lane groups.
__device__ __forceinline__ float wave_tree_sum(float v) {
    v = pair_sum1(v);
    v = pair_sum2(v);
    v = pair_sum4_uniform(v);
    v = pair_sum8_uniform(v);
    return pair_sum32_low(pair_sum16_low(v));
}

constexpr int kWave = 64;

}  // namespace moe
