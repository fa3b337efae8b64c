// Internal interface between the moe_expert_ffn_grouped dispatcher and its kernels.
#pragma once

#include <algorithm>

#include "moe_common.h"

namespace moe {

struct FfnArgs {
    const void* x;               // [T, d] activations
    int T, d, f, E, k;
    const int32_t* perm;         // [T*k]
    const int32_t* offsets;      // [E+1]
    const int32_t* counts;       // [E]
    const int32_t* slot_of_expert;  // [E]
    int n_slots;
    const uint8_t* pool;         // slot pool
    size_t stride;               // bytes per slot
    const uint8_t* shared_w;     // shared expert image or nullptr
    void* h;                     // [rows, f] intermediate (bf16 for bf16 activations, else f32)
    void* y_perm;                // [rows, d], binary32 or (y_bf16) bf16
    int y_bf16;                  // y_perm rows are bf16 (each sum rounded once) instead of binary32
    int32_t* status;             // sticky error word
    void* plan;                  // scratch for the prefill tile schedule
    int n_lo = 1, n_hi = 1 << 30;  // a launch covers the experts with n_lo <= n_e <= n_hi tokens
};

enum { kGateUp = 0, kDown = 1 };  // the two projections of a grouped call

constexpr size_t kWsHeader = 256;
constexpr size_t kPlanBytes = 1 << 16;

// Upper bound on the work items (expert, chunk of ntg tokens) of a launch over the experts in
// [n_lo, n_hi] (grid rows; the items past the real count exit at once).
inline int64_t work_items(const FfnArgs& a, int ntg) {
    const int64_t tk = (int64_t)a.T * a.k;
    const int64_t nexp = std::min<int64_t>(std::min<int64_t>(a.E, tk), tk / std::max(a.n_lo, 1));
    int64_t routed = (tk + ntg - 1) / ntg + nexp;
    if (a.n_hi < (1 << 30)) routed = std::min<int64_t>(routed, nexp * ((a.n_hi + ntg - 1) / ntg));
    const bool sh = a.shared_w && a.T >= a.n_lo && a.T <= a.n_hi;
    return routed + (sh ? (a.T + ntg - 1) / ntg : 0);
}

// Argument checks of moe_expert_ffn_grouped except the workspace; fills every field of `a` but
// status, plan and h (left NULL).  T == 0 returns MOE_OK with nothing to run.  `fn` names the
// caller in error messages.
moe_status ffn_prepare(FfnArgs& a, const char* fn, const void* x, moe_dtype act, int T, int d, int f, int E, int k,
                       const int32_t* perm, const int32_t* offsets, const int32_t* counts,
                       const int32_t* slot_of_expert, int n_slots, const void* slot_pool, size_t slot_stride,
                       moe_dtype w, const void* shared_w, void* y_perm, moe_dtype y_dtype);
// Launch the grouped experts: the prefill MFMA GEMM where it applies, else the decode GEMVs.
moe_status ffn_run(const FfnArgs& a, moe_dtype act, moe_dtype w, hipStream_t st);
// moe_expert_ffn_grouped with the absent-slot flag going to `status` (device int32) instead of the
// workspace's status word when `status` is not NULL (ffn_dispatch.cpp)
moe_status ffn_grouped_status(const void* x, moe_dtype act, int T, int d, int f, int E, int k, const int32_t* perm,
                              const int32_t* offsets, const int32_t* counts, const int32_t* slot_of_expert,
                              int n_slots, const void* slot_pool, size_t slot_stride, moe_dtype w,
                              const void* shared_w, void* y_perm, moe_dtype y_dtype, void* ws, size_t ws_bytes,
                              int32_t* status, moe_stream s);

// decode path: grouped GEMV kernels (ffn_gemv.hip), both projections or one (mode kGateUp = 0,
// kDown = 1)
moe_status ffn_gemv(const FfnArgs& a, moe_dtype act, moe_dtype w, hipStream_t st);
moe_status ffn_gemv_proj(const FfnArgs& a, moe_dtype act, moe_dtype w, int mode, hipStream_t st);
// The decode kernels below launch one projection (mode kGateUp = 0 or kDown = 1) and return
// MOE_EDTYPE, with nothing launched, for shapes they do not cover.
// bf16 x bf16, weights held in registers, inputs split over the waves (ffn_gemv_mfma.hip)
moe_status ffn_gemv_mfma(const FfnArgs& a, int mode, hipStream_t st);
// bf16 or int4 weights x bf16 activations, K streamed through each wave (ffn_gemv_ks.hip)
moe_status ffn_gemv_ks(const FfnArgs& a, int mode, moe_dtype w, hipStream_t st);
// bf16 or int4 weights x bf16 activations, a few tokens, every weight load of a wave issued at once
// (ffn_gemv_deep.hip)
moe_status ffn_gemv_deep(const FfnArgs& a, int mode, moe_dtype w, hipStream_t st);
// prefill path: MFMA grouped GEMM (ffn_mfma.hip), both projections or one; MOE_EDTYPE when it
// does not apply
moe_status ffn_mfma(const FfnArgs& a, moe_dtype act, moe_dtype w, hipStream_t st);
moe_status ffn_mfma_proj(const FfnArgs& a, moe_dtype act, moe_dtype w, int mode, hipStream_t st);

}  // namespace moe
