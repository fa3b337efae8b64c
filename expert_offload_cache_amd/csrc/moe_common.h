// Shared host/device helpers of libmoe (gfx950).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/moe.h"

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

constexpr int kWave = 64;

}  // namespace moe
