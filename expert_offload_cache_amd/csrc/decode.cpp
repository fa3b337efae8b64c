// Native decode driver of the offloaded stack: one call runs every MoE layer of one decode step
// through the slot cache (FreeToken linux guide, "MoE memory handling": per layer the router
// picks the experts, the GPU-resident ones are used from their slots and a miss is copied from
// the pinned host pool first; FreeToken GGUF page, offload backend).
//
// Per layer, on the compute stream: route -> permute -> ids copied to pinned host memory and the
// stream waited for (the cache decides on the host, with no lookahead) -> distinct ids, lookup,
// fill (copies on the copy stream, compute waits) -> grouped experts through the layer's
// slot-table row -> combine -> mark_read.  The same calls, in the same order, as a caller would
// make one by one; only the host-side marshalling between them is gone.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>

#include "moe_common.h"

using namespace moe;

extern "C" moe_status moe_decode_step(moe_cache* cache, int n_layers, const moe_decode_layer* layers, int T, int d,
                                      int f, int E, int k, moe_dtype act, moe_dtype w, const void* slot_pool,
                                      int n_slots, size_t slot_stride, const int32_t* slot_table, int32_t* topk_idx,
                                      float* topk_w, float* logits, int32_t* counts, int32_t* offsets, int32_t* perm,
                                      int32_t* inv_perm, float* y_perm, void* ws, size_t ws_bytes, int32_t* host_idx,
                                      moe_stream compute, moe_stream copy) {
    MOE_CHECK(cache && layers && slot_table && host_idx, MOE_EINVAL, "moe_decode_step: NULL pointer");
    MOE_CHECK(n_layers >= 0 && T >= 1 && k >= 1 && k <= E, MOE_ESHAPE,
              "moe_decode_step: need n_layers >= 0, T >= 1, 1 <= k <= E (n_layers=%d T=%d k=%d E=%d)", n_layers, T,
              k, E);
    hipStream_t cs = (hipStream_t)compute;
    std::vector<int32_t> ids((size_t)T * k), slots((size_t)T * k);
    for (int i = 0; i < n_layers; ++i) {
        const moe_decode_layer& ly = layers[i];
        MOE_CHECK(ly.x && ly.w_router && ly.y, MOE_EINVAL, "moe_decode_step: layer %d: NULL pointer", i);
        moe_status r = moe_route(ly.x, act, T, d, ly.w_router, ly.bias, E, k, ly.forced_idx, topk_idx, topk_w,
                                 logits, compute);
        if (r != MOE_OK) return r;
        r = moe_permute(topk_idx, T, k, E, counts, offsets, perm, inv_perm, nullptr, 0, compute);
        if (r != MOE_OK) return r;
        MOE_HIP(hipMemcpyAsync(host_idx, topk_idx, sizeof(int32_t) * (size_t)T * k, hipMemcpyDeviceToHost, cs));
        MOE_HIP(hipStreamSynchronize(cs));
        std::copy(host_idx, host_idx + (size_t)T * k, ids.begin());
        std::sort(ids.begin(), ids.end());
        const int n = (int)(std::unique(ids.begin(), ids.end()) - ids.begin());
        int32_t n_miss = 0;
        r = moe_cache_lookup(cache, ly.layer, ids.data(), n, slots.data(), &n_miss);
        if (r != MOE_OK) return r;
        r = moe_cache_fill(cache, copy, compute);
        if (r != MOE_OK) return r;
        r = moe_expert_ffn_grouped(ly.x, act, T, d, f, E, k, perm, offsets, counts, slot_table + (size_t)ly.layer * E,
                                   n_slots, slot_pool, slot_stride, w, ly.shared_w, y_perm, ws, ws_bytes, compute);
        if (r != MOE_OK) return r;
        r = moe_combine(y_perm, topk_w, inv_perm, T, k, d, ly.shared_w != nullptr, ly.y, act, compute);
        if (r != MOE_OK) return r;
        r = moe_cache_mark_read(cache, ly.layer, compute);
        if (r != MOE_OK) return r;
    }
    return MOE_OK;
}
