// Internal interface between the moe_expert_ffn_grouped dispatcher and its kernels.
#pragma once

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
    float* y_perm;               // [rows, d]
    int32_t* status;             // sticky error word
    void* plan;                  // scratch for the prefill tile schedule
};

constexpr size_t kWsHeader = 256;
constexpr size_t kPlanBytes = 1 << 16;

// decode path: grouped GEMV kernels (ffn_gemv.hip)
moe_status ffn_gemv(const FfnArgs& a, moe_dtype act, moe_dtype w, hipStream_t st);
// The decode kernels below launch one projection (mode kGateUp = 0 or kDown = 1) and return
// MOE_EDTYPE, with nothing launched, for shapes they do not cover.
// bf16 x bf16, weights held in registers, inputs split over the waves (ffn_gemv_mfma.hip)
moe_status ffn_gemv_mfma(const FfnArgs& a, int mode, hipStream_t st);
// bf16 or int4 weights x bf16 activations, K streamed through each wave (ffn_gemv_ks.hip)
moe_status ffn_gemv_ks(const FfnArgs& a, int mode, moe_dtype w, hipStream_t st);
// prefill path: MFMA grouped GEMM (ffn_mfma.hip); returns MOE_EDTYPE when it does not apply
moe_status ffn_mfma(const FfnArgs& a, moe_dtype act, moe_dtype w, hipStream_t st);

}  // namespace moe
