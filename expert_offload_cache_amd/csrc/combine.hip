// moe_combine: y[t] = sum_j g[t,j] * y_perm[inv_perm[t*k+j]] (+ shared expert row), j ascending,
// binary32 accumulation, one rounding to the output type.  The pages do not give the combine;
// a gate-weighted sum of the selected experts' outputs is the plain reading.
// Memory-bound: every thread owns 4 consecutive columns of one token (16-byte loads of binary32
// rows, 8-byte loads of bf16 rows).
#include <hip/hip_runtime.h>

#include "moe_common.h"

namespace moe {
namespace {

// four consecutive elements of a y_perm row, widened to binary32 (bf16 -> binary32 is exact)
__device__ __forceinline__ float4 load_row4(const float* p) { return *(const float4*)p; }
__device__ __forceinline__ float4 load_row4(const uint16_t* p) {
    const uint2 v = *(const uint2*)p;
    return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u), __uint_as_float(v.y << 16),
                       __uint_as_float(v.y & 0xffff0000u));
}

template <bool kBf16Out, typename YT>
__global__ __launch_bounds__(256) void combine_kernel(const YT* __restrict__ yp, const float* __restrict__ g,
                                                      const int32_t* __restrict__ inv, int T, int k, int d,
                                                      int has_shared, void* __restrict__ y) {
    const int t = blockIdx.y;
    const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (c >= d) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    // 8 experts at a time: their indices and gates, then their rows, are loaded together; the
    // products are added in ascending j as before
    for (int j0 = 0; j0 < k; j0 += 8) {
        int idx[8];
        float gj[8];
        float4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int j = min(j0 + u, k - 1);
            idx[u] = inv[(size_t)t * k + j];
            gj[u] = g[(size_t)t * k + j];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = load_row4(yp + (size_t)idx[u] * d + c);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (j0 + u < k) {
                acc.x = __builtin_fmaf(gj[u], v[u].x, acc.x);
                acc.y = __builtin_fmaf(gj[u], v[u].y, acc.y);
                acc.z = __builtin_fmaf(gj[u], v[u].z, acc.z);
                acc.w = __builtin_fmaf(gj[u], v[u].w, acc.w);
            }
        }
    }
    if (has_shared) {
        const float4 v = load_row4(yp + ((size_t)T * k + t) * d + c);
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    if constexpr (kBf16Out) {
        uint2 o;
        o.x = (uint32_t)f32_to_bf16(acc.x) | ((uint32_t)f32_to_bf16(acc.y) << 16);
        o.y = (uint32_t)f32_to_bf16(acc.z) | ((uint32_t)f32_to_bf16(acc.w) << 16);
        *(uint2*)((uint16_t*)y + (size_t)t * d + c) = o;
    } else {
        *(float4*)((float*)y + (size_t)t * d + c) = acc;
    }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_combine(const void* y_perm, moe_dtype y_dtype, const float* topk_w,
                                  const int32_t* inv_perm, int T, int k, int d, int has_shared, void* y,
                                  moe_dtype out, moe_stream s) {
    MOE_CHECK(T >= 0 && k >= 1 && d >= 4 && d % 4 == 0, MOE_ESHAPE, "moe_combine: bad shape T=%d k=%d d=%d", T, k, d);
    if (T == 0) return MOE_OK;
    MOE_CHECK(T <= 65535, MOE_ESHAPE, "moe_combine: T=%d too large", T);
    MOE_CHECK(out == MOE_F32 || out == MOE_BF16, MOE_EDTYPE, "moe_combine: output must be F32 or BF16");
    MOE_CHECK(y_dtype == MOE_F32 || y_dtype == MOE_BF16, MOE_EDTYPE, "moe_combine: y_perm must be F32 or BF16");
    MOE_CHECK(y_perm && topk_w && inv_perm && y, MOE_EINVAL, "moe_combine: NULL pointer");
    MOE_CHECK((uintptr_t)y_perm % 16 == 0 && (uintptr_t)y % 8 == 0, MOE_EINVAL, "moe_combine: misaligned buffers");
    hipStream_t st = (hipStream_t)s;
    dim3 grid((unsigned)((d / 4 + 255) / 256), (unsigned)T);
    ProfScope p("combine", st);
    const float* yf = (const float*)y_perm;
    const uint16_t* yh = (const uint16_t*)y_perm;
    if (out == MOE_BF16) {
        if (y_dtype == MOE_BF16) combine_kernel<true><<<grid, 256, 0, st>>>(yh, topk_w, inv_perm, T, k, d, has_shared, y);
        else combine_kernel<true><<<grid, 256, 0, st>>>(yf, topk_w, inv_perm, T, k, d, has_shared, y);
    } else {
        if (y_dtype == MOE_BF16) combine_kernel<false><<<grid, 256, 0, st>>>(yh, topk_w, inv_perm, T, k, d, has_shared, y);
        else combine_kernel<false><<<grid, 256, 0, st>>>(yf, topk_w, inv_perm, T, k, d, has_shared, y);
    }
    return check_launch("combine");
}
