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

namespace moe {

moe_status ffn_prepare(FfnArgs& a, const char* fn, const void* x, moe_dtype act, int T, int d, int f, int E, int k,
                       const int32_t* perm, const int32_t* offsets, const int32_t* counts,
                       const int32_t* slot_of_expert, int n_slots, const void* slot_pool, size_t slot_stride,
                       moe_dtype w, const void* shared_w, void* y_perm, moe_dtype y_dtype) {
    MOE_CHECK(T >= 0, MOE_ESHAPE, "%s: T=%d < 0", fn, T);
    if (T == 0) return MOE_OK;
    MOE_CHECK(act == MOE_F32 || act == MOE_BF16, MOE_EDTYPE, "%s: bad activation dtype", fn);
    MOE_CHECK(w != MOE_INT4_G128 || act == MOE_BF16, MOE_EDTYPE, "%s: int4 needs bf16 activations", fn);
    MOE_CHECK(w == MOE_INT4_G128 || w == act, MOE_EDTYPE, "%s: dense weights must have the activation dtype", fn);
    MOE_CHECK(y_dtype == MOE_F32 || (y_dtype == MOE_BF16 && act == MOE_BF16), MOE_EDTYPE,
              "%s: y_perm must be F32, or BF16 with bf16 activations", fn);
    MOE_CHECK(slot_shape_ok(d, f, w), MOE_ESHAPE, "%s: unsupported d=%d f=%d for dtype %d", fn, d, f, (int)w);
    MOE_CHECK(E >= 1 && E <= 1024 && k >= 1 && k <= E, MOE_ESHAPE, "%s: need 1 <= k <= E <= 1024", fn);
    MOE_CHECK((int64_t)T * k <= (1 << 24), MOE_ESHAPE, "%s: T*k too large", fn);
    MOE_CHECK(x && perm && offsets && counts && slot_of_expert && slot_pool && y_perm, MOE_EINVAL,
              "%s: NULL pointer", fn);
    MOE_CHECK(n_slots >= 1, MOE_EINVAL, "%s: n_slots must be >= 1", fn);
    MOE_CHECK(slot_stride >= moe_slot_bytes(d, f, w) && slot_stride % 256 == 0, MOE_EINVAL,
              "%s: slot_stride %zu smaller than a slot (%zu) or not 256-aligned", fn, slot_stride,
              moe_slot_bytes(d, f, w));
    MOE_CHECK((uintptr_t)slot_pool % 256 == 0 && (!shared_w || (uintptr_t)shared_w % 256 == 0), MOE_EINVAL,
              "%s: slot pool / shared expert must be 256-byte aligned", fn);
    MOE_CHECK((uintptr_t)x % 16 == 0 && (uintptr_t)y_perm % 16 == 0, MOE_EINVAL,
              "%s: x and y_perm must be 16-byte aligned", fn);
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
    a.y_perm = y_perm;
    a.y_bf16 = y_dtype == MOE_BF16;
    a.status = nullptr;
    a.plan = nullptr;
    a.h = nullptr;
    return MOE_OK;
}

// experts with fewer tokens than this run on the decode kernels in prefill (int4: measured on the
// DeepSeek-V4-Flash shaped layer, FFN 1082 -> 685 us at 512 tokens, 1811 -> 1377 us at 2048 with
// 32; 28 then measured 8 % faster at 512 tokens and 2-5 % at 2048 than 32, 20 and 24 in between,
// equal at 8192: an expert holding 28-31 tokens fills two 16-token items of the decode kernel and
// reads its weights twice; bf16 weights gain nothing, the light experts' launch is bound by HBM
// either way)
#ifndef MOE_SPLIT_INT4
#define MOE_SPLIT_INT4 28
#endif
// bf16: experts with fewer than 8 tokens, while the call averages at most 64 tokens an expert
// (T*k <= 64*E): measured on the DeepSeek-V4-Flash shaped layer, FFN 1,272 -> 1,174 us at 512
// tokens and 2,025 -> 1,942 at 2048 (4 and 12 tokens measured slower); above, few experts are that
// light and the second launch, mostly empty, only costs time (dense routing at 2048 tokens: 705 ->
// 740 us)
#ifndef MOE_SPLIT_BF16
#define MOE_SPLIT_BF16 8
#endif

int prefill_split(moe_dtype w) { return w == MOE_INT4_G128 ? MOE_SPLIT_INT4 : w == MOE_BF16 ? MOE_SPLIT_BF16 : 0; }

// the split for this call (0: none)
static int prefill_split_for(const FfnArgs& a, moe_dtype w) {
    if (w == MOE_BF16 && (int64_t)a.T * a.k > (int64_t)64 * a.E) return 0;
    return prefill_split(w);
}

moe_status ffn_run(const FfnArgs& a, moe_dtype act, moe_dtype w, hipStream_t st) {
    // Prefill with few tokens on most experts: the experts holding fewer than `split` tokens go to
    // the decode kernels (their weights are streamed once, no 128-token tiles to fill), the others
    // and the shared expert to the matrix-core GEMM; both gate/up launches precede both down
    // launches.  0 = one launch per projection.
    const int split = prefill_split_for(a, w);
    if (split > 1 && act == MOE_BF16 && a.T > 64) {
        FfnArgs heavy = a, light = a;
        heavy.n_lo = split;
        light.n_hi = split - 1;
        for (int mode = kGateUp; mode <= kDown; ++mode) {
            moe_status r = ffn_mfma_proj(heavy, act, w, mode, st);
            if (r == MOE_EDTYPE) return ffn_gemv(a, act, w, st);  // the GEMM does not take this shape
            if (r != MOE_OK) return r;
            r = ffn_gemv_proj(light, act, w, mode, st);
            if (r != MOE_OK) return r;
        }
        return MOE_OK;
    }
    moe_status r = ffn_mfma(a, act, w, st);
    if (r != MOE_EDTYPE) return r;
    return ffn_gemv(a, act, w, st);
}

}  // namespace moe

extern "C" {

int moe_prefill_gemv_tokens(moe_dtype w) {
    const int s = moe::prefill_split(w);
    return s > 1 ? s - 1 : 0;
}

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
                                  size_t slot_stride, moe_dtype w, const void* shared_w, void* y_perm,
                                  moe_dtype y_dtype, void* ws, size_t ws_bytes, moe_stream s) {
    return moe::ffn_grouped_status(x, act, T, d, f, E, k, perm, offsets, counts, slot_of_expert, n_slots, slot_pool,
                                   slot_stride, w, shared_w, y_perm, y_dtype, ws, ws_bytes, nullptr, s);
}

}  // extern "C"

namespace moe {
moe_status ffn_grouped_status(const void* x, moe_dtype act, int T, int d, int f, int E, int k, const int32_t* perm,
                              const int32_t* offsets, const int32_t* counts, const int32_t* slot_of_expert,
                              int n_slots, const void* slot_pool, size_t slot_stride, moe_dtype w,
                              const void* shared_w, void* y_perm, moe_dtype y_dtype, void* ws, size_t ws_bytes,
                              int32_t* status, moe_stream s) {
    FfnArgs a;
    moe_status r = ffn_prepare(a, "moe_expert_ffn_grouped", x, act, T, d, f, E, k, perm, offsets, counts,
                               slot_of_expert, n_slots, slot_pool, slot_stride, w, shared_w, y_perm, y_dtype);
    if (r != MOE_OK || T == 0) return r;
    MOE_CHECK(ws, MOE_EINVAL, "moe_expert_ffn_grouped: NULL workspace");
    MOE_CHECK((uintptr_t)ws % 256 == 0, MOE_EINVAL, "moe_expert_ffn_grouped: workspace must be 256-byte aligned");
    size_t need = moe_workspace_bytes(T, d, f, E, k, shared_w != nullptr, act, w);
    MOE_CHECK(ws_bytes >= need, MOE_ENOMEM, "moe_expert_ffn_grouped: workspace %zu < %zu bytes", ws_bytes, need);
    a.status = status ? status : (int32_t*)ws;
    a.plan = (uint8_t*)ws + kWsHeader;
    a.h = (uint8_t*)ws + kWsHeader + kPlanBytes;
    return ffn_run(a, act, w, (hipStream_t)s);
}
}  // namespace moe
