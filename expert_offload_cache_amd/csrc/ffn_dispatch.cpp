// moe_expert_ffn_grouped: argument checks, workspace layout, and the choice between the
// decode GEMV kernels and the prefill MFMA grouped GEMM.
#include <hip/hip_runtime.h>

#include "ffn.h"
#include "slot_layout.h"

using namespace moe;

namespace {
size_t h_bytes(int T, int f, int k, int has_shared, moe_dtype act) {
    size_t rows = (size_t)T * k + (has_shared ? (size_t)T : 0);
    return align_up(rows * f * (act == MOE_BF16 ? 2 : 4), 256);
}
}  // namespace

extern "C" {

size_t moe_workspace_bytes(int T, int d, int f, int E, int k, int has_shared, moe_dtype act, moe_dtype w) {
    (void)d;
    (void)E;
    (void)w;
    if (T < 0 || f <= 0 || k <= 0) return 0;
    return kWsHeader + kPlanBytes + h_bytes(T, f, k, has_shared, act);
}

moe_status moe_expert_ffn_grouped(const void* x, moe_dtype act, int T, int d, int f, int E, int k,
                                  const int32_t* perm, const int32_t* offsets, const int32_t* counts,
                                  const int32_t* slot_of_expert, int n_slots, const void* slot_pool,
                                  size_t slot_stride, moe_dtype w, const void* shared_w, float* y_perm,
                                  void* ws, size_t ws_bytes, moe_stream s) {
    MOE_CHECK(T >= 0, MOE_ESHAPE, "moe_expert_ffn_grouped: T=%d < 0", T);
    if (T == 0) return MOE_OK;
    MOE_CHECK(act == MOE_F32 || act == MOE_BF16, MOE_EDTYPE, "moe_expert_ffn_grouped: bad activation dtype");
    MOE_CHECK(w != MOE_INT4_G128 || act == MOE_BF16, MOE_EDTYPE, "moe_expert_ffn_grouped: int4 needs bf16 activations");
    MOE_CHECK(w == MOE_INT4_G128 || w == act, MOE_EDTYPE,
              "moe_expert_ffn_grouped: dense weights must have the activation dtype");
    MOE_CHECK(slot_shape_ok(d, f, w), MOE_ESHAPE, "moe_expert_ffn_grouped: unsupported d=%d f=%d for dtype %d", d,
              f, (int)w);
    MOE_CHECK(E >= 1 && E <= 1024 && k >= 1 && k <= E, MOE_ESHAPE, "moe_expert_ffn_grouped: need 1 <= k <= E <= 1024");
    MOE_CHECK((int64_t)T * k <= (1 << 24), MOE_ESHAPE, "moe_expert_ffn_grouped: T*k too large");
    MOE_CHECK(x && perm && offsets && counts && slot_of_expert && slot_pool && y_perm && ws, MOE_EINVAL,
              "moe_expert_ffn_grouped: NULL pointer");
    MOE_CHECK(n_slots >= 1, MOE_EINVAL, "moe_expert_ffn_grouped: n_slots must be >= 1");
    MOE_CHECK(slot_stride >= moe_slot_bytes(d, f, w) && slot_stride % 256 == 0, MOE_EINVAL,
              "moe_expert_ffn_grouped: slot_stride %zu smaller than a slot (%zu) or not 256-aligned", slot_stride,
              moe_slot_bytes(d, f, w));
    MOE_CHECK((uintptr_t)slot_pool % 256 == 0 && (!shared_w || (uintptr_t)shared_w % 256 == 0), MOE_EINVAL,
              "moe_expert_ffn_grouped: slot pool / shared expert must be 256-byte aligned");
    MOE_CHECK((uintptr_t)x % 16 == 0 && (uintptr_t)y_perm % 16 == 0, MOE_EINVAL,
              "moe_expert_ffn_grouped: x and y_perm must be 16-byte aligned");
    MOE_CHECK((uintptr_t)ws % 256 == 0, MOE_EINVAL, "moe_expert_ffn_grouped: workspace must be 256-byte aligned");
    const int has_shared = shared_w != nullptr;
    size_t need = moe_workspace_bytes(T, d, f, E, k, has_shared, act, w);
    MOE_CHECK(ws_bytes >= need, MOE_ENOMEM, "moe_expert_ffn_grouped: workspace %zu < %zu bytes", ws_bytes, need);

    FfnArgs a;
    a.x = x;
    a.T = T;
    a.d = d;
    a.f = f;
    a.E = E;
    a.k = k;
    a.perm = perm;
    a.offsets = offsets;
    a.counts = counts;
    a.slot_of_expert = slot_of_expert;
    a.n_slots = n_slots;
    a.pool = (const uint8_t*)slot_pool;
    a.stride = slot_stride;
    a.shared_w = (const uint8_t*)shared_w;
    a.status = (int32_t*)ws;
    a.plan = (uint8_t*)ws + kWsHeader;
    a.h = (uint8_t*)ws + kWsHeader + kPlanBytes;
    a.y_perm = y_perm;
    hipStream_t st = (hipStream_t)s;

    moe_status r = ffn_mfma(a, act, w, st);
    if (r != MOE_EDTYPE) return r;
    return ffn_gemv(a, act, w, st);
}

}  // extern "C"
