// Native decode loop of the offloaded stack: one call runs every MoE layer of one decode step
// through the slot cache (FreeToken linux guide, "MoE memory handling": per layer the router
// picks the experts, the GPU-resident ones are used from their slots and a miss is copied from
// the pinned host pool first; FreeToken GGUF page, offload backend).
//
// Per layer, on the compute stream: route + permute (one call) -> ids copied to pinned host
// memory; the host waits for the copy (the cache decides on the host, with no lookahead) ->
// distinct ids, lookup, fill (copies on the copy stream, compute waits) -> grouped experts
// through the layer's slot-table row -> combine -> mark_read.  The same calls as a caller would
// make one by one; only the host-side marshalling between them is gone.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>

#include "moe_common.h"

using namespace moe;

namespace {
// Event marking the ids' arrival in host memory (created per call, released on every return).
struct IdsEvent {
    hipEvent_t e = nullptr;
    hipError_t status;
    IdsEvent() : status(hipEventCreateWithFlags(&e, hipEventDisableTiming)) {}
    ~IdsEvent() {
        if (e) (void)hipEventDestroy(e);
    }
};
}  // namespace

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
    for (int i = 0; i < n_layers; ++i)  // every layer is checked before anything is enqueued
        MOE_CHECK(layers[i].x && layers[i].w_router && layers[i].y, MOE_EINVAL,
                  "moe_decode_step: layer %d: NULL pointer", i);
    if (n_layers == 0) return MOE_OK;
    hipStream_t cs = (hipStream_t)compute;
    std::vector<int32_t> ids((size_t)T * k), slots((size_t)T * k);
    IdsEvent ev;
    MOE_HIP(ev.status);
    for (int i = 0; i < n_layers; ++i) {
        const moe_decode_layer& ly = layers[i];
        moe_status r = moe_route_permute(ly.x, act, T, d, ly.w_router, ly.bias, E, k, ly.forced_idx, topk_idx,
                                         topk_w, logits, counts, offsets, perm, inv_perm, compute);
        if (r != MOE_OK) return r;
        MOE_HIP(hipMemcpyAsync(host_idx, topk_idx, sizeof(int32_t) * (size_t)T * k, hipMemcpyDeviceToHost, cs));
        MOE_HIP(hipEventRecord(ev.e, cs));
        MOE_HIP(hipEventSynchronize(ev.e));
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

namespace moe {
const void* cache_host_image(const moe_cache* c, int layer, int expert);  // cache.cpp
}

namespace {
// Misses of one layer to run on the host: the n minimising max((m - n) / pcie_rate, n / cpu_rate),
// ties to fewer on the host (FreeToken RTX 5090 page, miss split; stork.ai article, miss policy).
int hybrid_split(int m, double cpu_rate, double pcie_rate) {
    if (cpu_rate <= 0.0 || m <= 0) return 0;
    int best = 0;
    double best_t = m / pcie_rate;
    for (int n = 1; n <= m; ++n) {
        const double t = std::max((m - n) / pcie_rate, n / cpu_rate);
        if (t < best_t - 1e-15) {
            best = n;
            best_t = t;
        }
    }
    return best;
}
}  // namespace

extern "C" moe_status moe_decode_step_hybrid(
    moe_cache* cache, int n_layers, const moe_decode_layer* layers, int d, int f, int E, int k, moe_dtype act,
    moe_dtype w, const void* slot_pool, int n_slots, size_t slot_stride, const int32_t* slot_table, int32_t* topk_idx,
    float* topk_w, float* logits, int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm, float* y_perm,
    void* ws, size_t ws_bytes, int32_t* host_idx, void* host_x, float* host_y, int32_t* host_table,
    int32_t* dev_table, double cpu_rate, double pcie_rate, int copy_too, int cpu_threads, int64_t* n_cpu_out,
    moe_stream compute, moe_stream copy) {
    MOE_CHECK(cache && layers && slot_table && host_idx && host_x && host_y && host_table && dev_table, MOE_EINVAL,
              "moe_decode_step_hybrid: NULL pointer");
    MOE_CHECK(n_layers >= 0 && k >= 1 && k <= E && act == MOE_BF16, MOE_ESHAPE,
              "moe_decode_step_hybrid: need n_layers >= 0, 1 <= k <= E and bf16 activations");
    hipStream_t cs = (hipStream_t)compute;
    const int T = 1;  // one token: a pair's row of y_perm is the rank of its expert id
    for (int i = 0; i < n_layers; ++i)  // every layer is checked before anything is enqueued
        MOE_CHECK(layers[i].x && layers[i].w_router && layers[i].y, MOE_EINVAL,
                  "moe_decode_step_hybrid: layer %d: NULL pointer", i);
    if (n_layers == 0) return MOE_OK;
    std::vector<int32_t> ids(k), slots(k), miss, on_cpu, gpu_ids;
    int64_t n_cpu_total = 0;
    IdsEvent ev;
    MOE_HIP(ev.status);
    for (int i = 0; i < n_layers; ++i) {
        const moe_decode_layer& ly = layers[i];
        moe_status r = moe_route_permute(ly.x, act, T, d, ly.w_router, ly.bias, E, k, ly.forced_idx, topk_idx,
                                         topk_w, logits, counts, offsets, perm, inv_perm, compute);
        if (r != MOE_OK) return r;
        MOE_HIP(hipMemcpyAsync(host_idx, topk_idx, sizeof(int32_t) * k, hipMemcpyDeviceToHost, cs));
        MOE_HIP(hipEventRecord(ev.e, cs));
        // the event also retires the previous layer's table and row copies (earlier on the stream)
        MOE_HIP(hipEventSynchronize(ev.e));
        std::copy(host_idx, host_idx + k, ids.begin());
        std::sort(ids.begin(), ids.end());
        const int n = (int)(std::unique(ids.begin(), ids.end()) - ids.begin());
        miss.clear();
        for (int j = 0; j < n; ++j) {
            int32_t sl = -1;
            r = moe_cache_slot_of(cache, ly.layer, ids[j], &sl);
            if (r != MOE_OK) return r;
            if (sl < 0) miss.push_back(ids[j]);
        }
        const int n_cpu = hybrid_split((int)miss.size(), cpu_rate, pcie_rate);
        if (n_cpu == 0) {
            // nothing for the host in this layer: the plain step (the cache's own slot-table row,
            // no table or activation copies), with the same cache decisions and outputs
            int32_t n_miss = 0;
            r = moe_cache_lookup(cache, ly.layer, ids.data(), n, slots.data(), &n_miss);
            if (r != MOE_OK) return r;
            r = moe_cache_fill(cache, copy, compute);
            if (r != MOE_OK) return r;
            r = moe_expert_ffn_grouped(ly.x, act, T, d, f, E, k, perm, offsets, counts,
                                       slot_table + (size_t)ly.layer * E, n_slots, slot_pool, slot_stride, w,
                                       ly.shared_w, y_perm, ws, ws_bytes, compute);
            if (r != MOE_OK) return r;
            r = moe_combine(y_perm, topk_w, inv_perm, T, k, d, ly.shared_w != nullptr, ly.y, act, compute);
            if (r != MOE_OK) return r;
            r = moe_cache_mark_read(cache, ly.layer, compute);
            if (r != MOE_OK) return r;
            continue;
        }
        // the host's experts need the activation row; it crosses while the cache decides
        MOE_HIP(hipMemcpyAsync(host_x, ly.x, sizeof(uint16_t) * d, hipMemcpyDeviceToHost, cs));
        MOE_HIP(hipEventRecord(ev.e, cs));
        on_cpu.assign(miss.end() - n_cpu, miss.end());  // the highest-numbered misses
        gpu_ids.clear();
        for (int j = 0; j < n; ++j)
            if (copy_too || std::find(on_cpu.begin(), on_cpu.end(), ids[j]) == on_cpu.end()) gpu_ids.push_back(ids[j]);
        int32_t n_miss = 0;
        r = moe_cache_lookup(cache, ly.layer, gpu_ids.data(), (int)gpu_ids.size(), slots.data(), &n_miss);
        if (r != MOE_OK) return r;
        r = copy_too ? moe_cache_fill_split(cache, on_cpu.data(), (int)on_cpu.size(), copy, compute)
                     : moe_cache_fill(cache, copy, compute);
        if (r != MOE_OK) return r;
        std::fill(host_table, host_table + E, -1);
        for (size_t j = 0; j < gpu_ids.size(); ++j) host_table[gpu_ids[j]] = slots[j];
        for (int e : on_cpu) host_table[e] = MOE_SLOT_ELSEWHERE;
        MOE_HIP(hipMemcpyAsync(dev_table, host_table, sizeof(int32_t) * E, hipMemcpyHostToDevice, cs));
        r = moe_expert_ffn_grouped(ly.x, act, T, d, f, E, k, perm, offsets, counts, dev_table, n_slots, slot_pool,
                                   slot_stride, w, ly.shared_w, y_perm, ws, ws_bytes, compute);
        if (r != MOE_OK) return r;
        // the host's experts run while the copies and the GPU's experts do
        MOE_HIP(hipEventSynchronize(ev.e));  // host_x has arrived
        for (int e : on_cpu) {
            const int row = (int)(std::lower_bound(ids.begin(), ids.begin() + n, e) - ids.begin());
            const void* img = cache_host_image(cache, ly.layer, e);
            MOE_CHECK(img, MOE_ESTATE, "moe_decode_step_hybrid: the cache has no host image of (%d,%d)", ly.layer, e);
            r = moe_cpu_expert_ffn(img, w, d, f, host_x, 1, host_y + (size_t)row * d, cpu_threads);
            if (r != MOE_OK) return r;
            MOE_HIP(hipMemcpyAsync(y_perm + (size_t)row * d, host_y + (size_t)row * d, sizeof(float) * d,
                                   hipMemcpyHostToDevice, cs));
        }
        n_cpu_total += n_cpu;
        r = moe_combine(y_perm, topk_w, inv_perm, T, k, d, ly.shared_w != nullptr, ly.y, act, compute);
        if (r != MOE_OK) return r;
        r = moe_cache_mark_read(cache, ly.layer, compute);
        if (r != MOE_OK) return r;
    }
    if (n_cpu_out) *n_cpu_out += n_cpu_total;
    return MOE_OK;
}

extern "C" moe_status moe_decode_step_split(moe_cache* cache, int n_layers, const moe_decode_layer* layers, int T,
                                            int d, int f, int E, int k, moe_dtype act, moe_dtype w,
                                            const void* slot_pool, int n_slots, size_t slot_stride,
                                            const int32_t* slot_table, int32_t* topk_idx, float* topk_w,
                                            float* logits, int32_t* counts, int32_t* offsets, int32_t* perm,
                                            int32_t* inv_perm, float* y_perm, void* ws, size_t ws_bytes,
                                            int32_t* host_idx, int32_t* host_tables, int32_t* dev_tables,
                                            moe_stream compute, moe_stream copy) {
    MOE_CHECK(cache && layers && slot_table && host_idx && host_tables && dev_tables, MOE_EINVAL,
              "moe_decode_step_split: NULL pointer");
    MOE_CHECK(n_layers >= 0 && T >= 1 && k >= 1 && k <= E, MOE_ESHAPE,
              "moe_decode_step_split: need n_layers >= 0, T >= 1, 1 <= k <= E (n_layers=%d T=%d k=%d E=%d)",
              n_layers, T, k, E);
    for (int i = 0; i < n_layers; ++i)  // every layer is checked before anything is enqueued
        MOE_CHECK(layers[i].x && layers[i].w_router && layers[i].y, MOE_EINVAL,
                  "moe_decode_step_split: layer %d: NULL pointer", i);
    if (n_layers == 0) return MOE_OK;
    hipStream_t cs = (hipStream_t)compute;
    std::vector<int32_t> ids((size_t)T * k), slots((size_t)T * k);
    std::vector<char> missed((size_t)T * k);
    IdsEvent ev;
    MOE_HIP(ev.status);
    for (int i = 0; i < n_layers; ++i) {
        const moe_decode_layer& ly = layers[i];
        moe_status r = moe_route_permute(ly.x, act, T, d, ly.w_router, ly.bias, E, k, ly.forced_idx, topk_idx,
                                         topk_w, logits, counts, offsets, perm, inv_perm, compute);
        if (r != MOE_OK) return r;
        MOE_HIP(hipMemcpyAsync(host_idx, topk_idx, sizeof(int32_t) * (size_t)T * k, hipMemcpyDeviceToHost, cs));
        MOE_HIP(hipEventRecord(ev.e, cs));
        // also retires the previous layer's table copy (earlier on the stream)
        MOE_HIP(hipEventSynchronize(ev.e));
        std::copy(host_idx, host_idx + (size_t)T * k, ids.begin());
        std::sort(ids.begin(), ids.end());
        const int n = (int)(std::unique(ids.begin(), ids.end()) - ids.begin());
        int n_missed = 0;
        for (int j = 0; j < n; ++j) {
            int32_t sl = -1;
            r = moe_cache_slot_of(cache, ly.layer, ids[j], &sl);
            if (r != MOE_OK) return r;
            missed[j] = sl < 0;
            n_missed += missed[j];
        }
        int32_t n_miss = 0;
        r = moe_cache_lookup(cache, ly.layer, ids.data(), n, slots.data(), &n_miss);
        if (r != MOE_OK) return r;
        if (n_missed == 0) {
            r = moe_cache_fill(cache, copy, compute);
            if (r == MOE_OK)
                r = moe_expert_ffn_grouped(ly.x, act, T, d, f, E, k, perm, offsets, counts,
                                           slot_table + (size_t)ly.layer * E, n_slots, slot_pool, slot_stride, w,
                                           ly.shared_w, y_perm, ws, ws_bytes, compute);
        } else {
            // row 0: the resident experts (missed ones produced elsewhere), row 1: the missed ones
            int32_t* hit_row = host_tables;
            int32_t* miss_row = host_tables + E;
            std::fill(host_tables, host_tables + 2 * (size_t)E, -1);
            for (int j = 0; j < n; ++j) {
                hit_row[ids[j]] = missed[j] ? MOE_SLOT_ELSEWHERE : slots[j];
                miss_row[ids[j]] = missed[j] ? slots[j] : MOE_SLOT_ELSEWHERE;
            }
            MOE_HIP(hipMemcpyAsync(dev_tables, host_tables, sizeof(int32_t) * 2 * (size_t)E, hipMemcpyHostToDevice,
                                   cs));
            // the resident experts run while the misses are copied in
            r = moe_expert_ffn_grouped(ly.x, act, T, d, f, E, k, perm, offsets, counts, dev_tables, n_slots,
                                       slot_pool, slot_stride, w, ly.shared_w, y_perm, ws, ws_bytes, compute);
            if (r == MOE_OK) r = moe_cache_fill(cache, copy, compute);
            if (r == MOE_OK)
                r = moe_expert_ffn_grouped(ly.x, act, T, d, f, E, k, perm, offsets, counts, dev_tables + E, n_slots,
                                           slot_pool, slot_stride, w, nullptr, y_perm, ws, ws_bytes, compute);
        }
        if (r != MOE_OK) return r;
        r = moe_combine(y_perm, topk_w, inv_perm, T, k, d, ly.shared_w != nullptr, ly.y, act, compute);
        if (r != MOE_OK) return r;
        r = moe_cache_mark_read(cache, ly.layer, compute);
        if (r != MOE_OK) return r;
    }
    return MOE_OK;
}
