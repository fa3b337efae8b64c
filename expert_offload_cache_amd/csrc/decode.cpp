// Native decode loop of the offloaded stack: one call runs every MoE layer of one decode step
// through the slot cache (FreeToken linux guide, "MoE memory handling": per layer the router
// picks the experts, the GPU-resident ones are used from their slots and a miss is copied from
// the pinned host pool first; FreeToken GGUF page, offload backend).
//
// Per layer, on the compute stream (moe_decode_step): route + permute (one call) -> grouped experts
// through the layer's slot-table row as it stands and the combine, enqueued at once -> the host
// reads the ids (at one token the route kernel stores them straight into coherent host memory; the
// cache decides on the host, with no lookahead) -> distinct ids, lookup, fill (copies on the copy
// stream, compute waits) -> for a layer with misses, the missed experts again after their copies,
// and the combine again -> mark_read.  The cache's decisions and the outputs are those of the calls
// made one by one; the GPU runs the resident experts while the host decides.  The hybrid and
// split-launch steps decide before launching any expert.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <climits>
#include <vector>

#include "moe_common.h"

using namespace moe;

namespace moe {
moe_status route_permute_publish(const void* x, moe_dtype act, int T, int d, const void* w_router, const float* bias,
                                 int E, int k, const int32_t* forced_idx, int32_t* topk_idx, float* topk_w,
                                 float* logits, int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                                 void* ws, size_t ws_bytes, int32_t* publish, moe_stream s);  // route.hip
moe_status ffn_grouped_status(const void* x, moe_dtype act, int T, int d, int f, int E, int k, const int32_t* perm,
                              const int32_t* offsets, const int32_t* counts, const int32_t* slot_of_expert,
                              int n_slots, const void* slot_pool, size_t slot_stride, moe_dtype w,
                              const void* shared_w, void* y_perm, moe_dtype y_dtype, void* ws, size_t ws_bytes,
                              int32_t* status, moe_stream s);  // ffn_dispatch.cpp
}

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

// Per host thread (a thread runs one decode step at a time) and device, allocated on first use and
// held until the process ends: coherent host memory that the one-token route kernel stores the
// ids into, and a slot-table row (pinned host, device) for a layer's second launch.  NULL when any
// of them cannot be allocated (the steps then take the copy-and-wait path).
constexpr int kMaxE = 1024;  // k <= E <= 1024
constexpr int kScratchDevices = 64;
struct StepScratch {
    int32_t* mirror = nullptr;    // [kMaxE] coherent host
    int32_t* host_row = nullptr;  // [kMaxE] pinned host
    int32_t* dev_row = nullptr;   // [kMaxE + 64] device: a slot-table row, then the first launch's
                                  // absent-slot flag (never read)
    bool failed = false;
};
StepScratch* step_scratch() {
    thread_local StepScratch scratch[kScratchDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return nullptr;
    StepScratch& sc = scratch[dev];
    if (sc.failed) return nullptr;
    if (!sc.dev_row) {
        void *m = nullptr, *h = nullptr, *dv = nullptr;
        const size_t bytes = sizeof(int32_t) * kMaxE;
        if (hipHostMalloc(&m, bytes, hipHostMallocCoherent) != hipSuccess || hipHostMalloc(&h, bytes) != hipSuccess ||
            hipMalloc(&dv, bytes + 256) != hipSuccess) {
            if (m) (void)hipHostFree(m);
            if (h) (void)hipHostFree(h);
            sc.failed = true;
            return nullptr;
        }
        sc.mirror = (int32_t*)m;
        sc.host_row = (int32_t*)h;
        sc.dev_row = (int32_t*)dv;
    }
    return &sc;
}

// Enqueues route + permute of one layer on `compute` and starts the ids' way to the host: with a
// `mirror` (one token only) the route kernel also stores the k ids into it, with system scope,
// after the host has set it to INT_MIN; without one, topk_idx is copied to host_idx and an event
// recorded after the copy.
moe_status route_start(const moe_decode_layer& ly, moe_dtype act, int T, int d, int E, int k, int32_t* topk_idx,
                       float* topk_w, float* logits, int32_t* counts, int32_t* offsets, int32_t* perm,
                       int32_t* inv_perm, int32_t* mirror, int32_t* host_idx, IdsEvent& ev, moe_stream compute) {
    hipStream_t cs = (hipStream_t)compute;
    if (mirror)
        for (int j = 0; j < k; ++j) __atomic_store_n(mirror + j, INT_MIN, __ATOMIC_RELAXED);
    moe_status r = route_permute_publish(ly.x, act, T, d, ly.w_router, ly.bias, E, k, ly.forced_idx, topk_idx, topk_w,
                                         logits, counts, offsets, perm, inv_perm, nullptr, 0, mirror, compute);
    if (r != MOE_OK || mirror) return r;
    MOE_HIP(hipMemcpyAsync(host_idx, topk_idx, sizeof(int32_t) * (size_t)T * k, hipMemcpyDeviceToHost, cs));
    MOE_HIP(hipEventRecord(ev.e, cs));
    return MOE_OK;
}

// Waits until the layer's T*k ids are in host memory and leaves them in host_idx.  When it returns
// OK, everything enqueued on `compute` before the route launch has completed.  With a mirror the
// host polls it; a poll that sees the stream finished, or a stream error, without every id
// arriving returns MOE_EHIP (the kernel's stores are posted before its completion).
moe_status ids_wait(int T, int k, int32_t* mirror, int32_t* host_idx, IdsEvent& ev, moe_stream compute) {
    if (!mirror) {
        MOE_HIP(hipEventSynchronize(ev.e));
        return MOE_OK;
    }
    hipStream_t cs = (hipStream_t)compute;
    auto arrived = [&] {
        int j = 0;
        while (j < k && __atomic_load_n(mirror + j, __ATOMIC_ACQUIRE) != INT_MIN) ++j;
        return j == k;
    };
    const auto t0 = std::chrono::steady_clock::now();
    for (unsigned spin = 0; !arrived(); ++spin) {
        if ((spin & 1023u) == 1023u) {
            const hipError_t q = hipStreamQuery(cs);
            if (q == hipSuccess) {
                if (arrived()) break;
                return set_error(MOE_EHIP, "decode step: the route kernel finished without publishing its ids");
            }
            if (q != hipErrorNotReady) return hip_error(q, "decode step: route kernel");
            if (std::chrono::steady_clock::now() - t0 > std::chrono::seconds(30))
                return set_error(MOE_EHIP, "decode step: the layer's ids did not arrive within 30 s");
        }
        __builtin_ia32_pause();
    }
    for (int j = 0; j < T * k; ++j) host_idx[j] = mirror[j];
    return MOE_OK;
}

// route_start + ids_wait (the steps that decide before launching any expert)
moe_status route_ids_to_host(const moe_decode_layer& ly, moe_dtype act, int T, int d, int E, int k, int32_t* topk_idx,
                             float* topk_w, float* logits, int32_t* counts, int32_t* offsets, int32_t* perm,
                             int32_t* inv_perm, int32_t* host_idx, IdsEvent& ev, moe_stream compute) {
    StepScratch* sc = T == 1 ? step_scratch() : nullptr;
    int32_t* mirror = sc ? sc->mirror : nullptr;
    moe_status r = route_start(ly, act, T, d, E, k, topk_idx, topk_w, logits, counts, offsets, perm, inv_perm, mirror,
                               host_idx, ev, compute);
    if (r != MOE_OK) return r;
    return ids_wait(T, k, mirror, host_idx, ev, compute);
}
}  // namespace

namespace moe {
moe_status cache_wait_background(moe_cache* c, hipStream_t compute);  // cache.cpp
}

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
    std::vector<int32_t> ids((size_t)T * k), slots((size_t)T * k), missed;
    IdsEvent ev;
    MOE_HIP(ev.status);
    StepScratch* sc = E <= kMaxE ? step_scratch() : nullptr;
    for (int i = 0; i < n_layers; ++i) {
        const moe_decode_layer& ly = layers[i];
        const int32_t* row = slot_table + (size_t)ly.layer * E;
        int32_t* mirror = (sc && T == 1) ? sc->mirror : nullptr;
        moe_status r = route_start(ly, act, T, d, E, k, topk_idx, topk_w, logits, counts, offsets, perm, inv_perm,
                                   mirror, host_idx, ev, compute);
        if (r != MOE_OK) return r;
        if (sc) {
            // the experts and the combine go ahead through the slot table as it stands while the host
            // reads the ids and decides: a resident expert's rows are final; a missed expert's rows
            // (its slot absent, or being refilled) are recomputed below once its copy has landed.
            // This launch's absent-slot flag goes to a word of the library: the workspace's status
            // word is the final launches' to set.
            r = cache_wait_background(cache, cs);
            if (r != MOE_OK) return r;
            r = ffn_grouped_status(ly.x, act, T, d, f, E, k, perm, offsets, counts, row, n_slots, slot_pool,
                                   slot_stride, w, ly.shared_w, y_perm, MOE_F32, ws, ws_bytes, sc->dev_row + kMaxE, compute);
            if (r != MOE_OK) return r;
            r = moe_combine(y_perm, MOE_F32, topk_w, inv_perm, T, k, d, ly.shared_w != nullptr, ly.y, act, compute);
            if (r != MOE_OK) return r;
        }
        r = ids_wait(T, k, mirror, host_idx, ev, compute);
        if (r != MOE_OK) return r;
        std::copy(host_idx, host_idx + (size_t)T * k, ids.begin());
        std::sort(ids.begin(), ids.end());
        const int n = (int)(std::unique(ids.begin(), ids.end()) - ids.begin());
        missed.clear();
        if (sc)
            for (int j = 0; j < n; ++j) {
                int32_t sl = -1;
                r = moe_cache_slot_of(cache, ly.layer, ids[j], &sl);
                if (r != MOE_OK) return r;
                if (sl < 0) missed.push_back(j);
            }
        int32_t n_miss = 0;
        r = moe_cache_lookup(cache, ly.layer, ids.data(), n, slots.data(), &n_miss);
        if (r != MOE_OK) return r;
        r = moe_cache_fill(cache, copy, compute);
        if (r != MOE_OK) return r;
        if (!sc) {
            r = moe_expert_ffn_grouped(ly.x, act, T, d, f, E, k, perm, offsets, counts, row, n_slots, slot_pool,
                                       slot_stride, w, ly.shared_w, y_perm, MOE_F32, ws, ws_bytes, compute);
            if (r != MOE_OK) return r;
            r = moe_combine(y_perm, MOE_F32, topk_w, inv_perm, T, k, d, ly.shared_w != nullptr, ly.y, act, compute);
            if (r != MOE_OK) return r;
        } else if (!missed.empty()) {
            // the missed experts again, after their copies (the fill made `compute` wait for them):
            // a row with only them in their new slots, every other expert produced elsewhere (and
            // the shared expert's rows kept); then the combine again.  The next layer's ids arriving
            // retires this row's copy before the host writes the row again.
            for (int e = 0; e < E; ++e) sc->host_row[e] = MOE_SLOT_ELSEWHERE;
            for (int j : missed) sc->host_row[ids[j]] = slots[j];
            MOE_HIP(hipMemcpyAsync(sc->dev_row, sc->host_row, sizeof(int32_t) * E, hipMemcpyHostToDevice, cs));
            r = moe_expert_ffn_grouped(ly.x, act, T, d, f, E, k, perm, offsets, counts, sc->dev_row, n_slots,
                                       slot_pool, slot_stride, w, nullptr, y_perm, MOE_F32, ws, ws_bytes, compute);
            if (r != MOE_OK) return r;
            r = moe_combine(y_perm, MOE_F32, topk_w, inv_perm, T, k, d, ly.shared_w != nullptr, ly.y, act, compute);
            if (r != MOE_OK) return r;
        }
        r = moe_cache_mark_read(cache, ly.layer, compute);
        if (r != MOE_OK) return r;
    }
    return MOE_OK;
}

namespace moe {
const void* cache_host_image(const moe_cache* c, int layer, int expert);  // cache.cpp
}

namespace {
// Misses of one layer to run on the host (FreeToken RTX 5090 page, miss split: the split follows the
// measured host and PCIe bandwidths; stork.ai article, miss policy).  With n of the m misses on the
// host the layer's miss work takes t(0) = m / pcie_rate, or t(n) = max((m - n) / pcie_rate,
// host_fixed_s + n / cpu_rate) for n >= 1, where host_fixed_s is the host path's cost that does not
// grow with n (activation row to the host, thread wake-up, output rows back).  The smallest t wins;
// ties go to fewer on the host.
int hybrid_split(int m, double cpu_rate, double pcie_rate, double host_fixed_s) {
    if (cpu_rate <= 0.0 || m <= 0) return 0;
    int best = 0;
    double best_t = m / pcie_rate;
    for (int n = 1; n <= m; ++n) {
        const double t = std::max((m - n) / pcie_rate, host_fixed_s + n / cpu_rate);
        if (t < best_t) {
            best = n;
            best_t = t;
        }
    }
    return best;
}
}  // namespace

extern "C" moe_status moe_hybrid_split(int m, double cpu_rate, double pcie_rate, double host_fixed_s,
                                       int32_t* n_host) {
    MOE_CHECK(n_host, MOE_EINVAL, "moe_hybrid_split: n_host is NULL");
    MOE_CHECK(m >= 0 && pcie_rate > 0.0 && cpu_rate >= 0.0 && host_fixed_s >= 0.0, MOE_EINVAL,
              "moe_hybrid_split: need m >= 0, pcie_rate > 0, cpu_rate >= 0, host_fixed_s >= 0");
    *n_host = hybrid_split(m, cpu_rate, pcie_rate, host_fixed_s);
    return MOE_OK;
}

extern "C" moe_status moe_decode_step_hybrid(
    moe_cache* cache, int n_layers, const moe_decode_layer* layers, int d, int f, int E, int k, moe_dtype act,
    moe_dtype w, const void* slot_pool, int n_slots, size_t slot_stride, const int32_t* slot_table, int32_t* topk_idx,
    float* topk_w, float* logits, int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm, float* y_perm,
    void* ws, size_t ws_bytes, int32_t* host_idx, void* host_x, float* host_y, int32_t* host_table,
    int32_t* dev_table, double cpu_rate, double pcie_rate, double host_fixed_s, int copy_too, int cpu_threads,
    int64_t* n_cpu_out, moe_stream compute, moe_stream copy) {
    MOE_CHECK(cache && layers && slot_table && host_idx && host_x && host_y && host_table && dev_table, MOE_EINVAL,
              "moe_decode_step_hybrid: NULL pointer");
    MOE_CHECK(n_layers >= 0 && k >= 1 && k <= E && act == MOE_BF16, MOE_ESHAPE,
              "moe_decode_step_hybrid: need n_layers >= 0, 1 <= k <= E and bf16 activations");
    MOE_CHECK(pcie_rate > 0.0 && cpu_rate >= 0.0 && host_fixed_s >= 0.0, MOE_EINVAL,
              "moe_decode_step_hybrid: need pcie_rate > 0, cpu_rate >= 0, host_fixed_s >= 0");
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
    StepScratch* sc = E <= kMaxE ? step_scratch() : nullptr;
    for (int i = 0; i < n_layers; ++i) {
        const moe_decode_layer& ly = layers[i];
        const int32_t* row = slot_table + (size_t)ly.layer * E;
        int32_t* mirror = sc ? sc->mirror : nullptr;
        moe_status r = route_start(ly, act, T, d, E, k, topk_idx, topk_w, logits, counts, offsets, perm, inv_perm,
                                   mirror, host_idx, ev, compute);
        if (r != MOE_OK) return r;
        if (sc) {
            // as moe_decode_step: the experts and the combine through the slot table as it stands
            // while the host decides; every miss's rows are produced again below (by the host or
            // after its copy)
            r = cache_wait_background(cache, cs);
            if (r != MOE_OK) return r;
            r = ffn_grouped_status(ly.x, act, T, d, f, E, k, perm, offsets, counts, row, n_slots, slot_pool,
                                   slot_stride, w, ly.shared_w, y_perm, MOE_F32, ws, ws_bytes, sc->dev_row + kMaxE, compute);
            if (r != MOE_OK) return r;
            r = moe_combine(y_perm, MOE_F32, topk_w, inv_perm, T, k, d, ly.shared_w != nullptr, ly.y, act, compute);
            if (r != MOE_OK) return r;
        }
        // the ids' arrival also retires the previous layer's table and row copies (earlier on the
        // stream than the route kernel)
        r = ids_wait(T, k, mirror, host_idx, ev, compute);
        if (r != MOE_OK) return r;
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
        const int n_cpu = hybrid_split((int)miss.size(), cpu_rate, pcie_rate, host_fixed_s);
        if (n_cpu == 0) {
            // nothing for the host in this layer: the plain step (the cache's own slot-table row,
            // no table or activation copies), with the same cache decisions and outputs
            int32_t n_miss = 0;
            r = moe_cache_lookup(cache, ly.layer, ids.data(), n, slots.data(), &n_miss);
            if (r != MOE_OK) return r;
            r = moe_cache_fill(cache, copy, compute);
            if (r != MOE_OK) return r;
            if (!sc) {
                r = moe_expert_ffn_grouped(ly.x, act, T, d, f, E, k, perm, offsets, counts, row, n_slots, slot_pool,
                                           slot_stride, w, ly.shared_w, y_perm, MOE_F32, ws, ws_bytes, compute);
                if (r != MOE_OK) return r;
                r = moe_combine(y_perm, MOE_F32, topk_w, inv_perm, T, k, d, ly.shared_w != nullptr, ly.y, act, compute);
                if (r != MOE_OK) return r;
            } else if (!miss.empty()) {
                // the missed experts again after their copies, then the combine again
                for (int e = 0; e < E; ++e) sc->host_row[e] = MOE_SLOT_ELSEWHERE;
                for (int e : miss) sc->host_row[e] = slots[std::lower_bound(ids.begin(), ids.begin() + n, e) - ids.begin()];
                MOE_HIP(hipMemcpyAsync(sc->dev_row, sc->host_row, sizeof(int32_t) * E, hipMemcpyHostToDevice, cs));
                r = moe_expert_ffn_grouped(ly.x, act, T, d, f, E, k, perm, offsets, counts, sc->dev_row, n_slots,
                                           slot_pool, slot_stride, w, nullptr, y_perm, MOE_F32, ws, ws_bytes, compute);
                if (r != MOE_OK) return r;
                r = moe_combine(y_perm, MOE_F32, topk_w, inv_perm, T, k, d, ly.shared_w != nullptr, ly.y, act, compute);
                if (r != MOE_OK) return r;
            }
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
        if (!sc) {
            std::fill(host_table, host_table + E, -1);
            for (size_t j = 0; j < gpu_ids.size(); ++j) host_table[gpu_ids[j]] = slots[j];
            for (int e : on_cpu) host_table[e] = MOE_SLOT_ELSEWHERE;
            MOE_HIP(hipMemcpyAsync(dev_table, host_table, sizeof(int32_t) * E, hipMemcpyHostToDevice, cs));
            r = moe_expert_ffn_grouped(ly.x, act, T, d, f, E, k, perm, offsets, counts, dev_table, n_slots,
                                       slot_pool, slot_stride, w, ly.shared_w, y_perm, MOE_F32, ws, ws_bytes, compute);
            if (r != MOE_OK) return r;
        } else {
            // the first launch produced the resident experts; the GPU's misses again after their
            // copies (every other expert produced elsewhere), the host's below
            std::fill(host_table, host_table + E, MOE_SLOT_ELSEWHERE);
            int n_gpu_miss = 0;
            for (size_t j = 0; j < gpu_ids.size(); ++j) {
                const int e = gpu_ids[j];
                if (std::find(miss.begin(), miss.end(), e) != miss.end() &&
                    std::find(on_cpu.begin(), on_cpu.end(), e) == on_cpu.end()) {
                    host_table[e] = slots[j];
                    ++n_gpu_miss;
                }
            }
            if (n_gpu_miss > 0) {
                MOE_HIP(hipMemcpyAsync(dev_table, host_table, sizeof(int32_t) * E, hipMemcpyHostToDevice, cs));
                r = moe_expert_ffn_grouped(ly.x, act, T, d, f, E, k, perm, offsets, counts, dev_table, n_slots,
                                           slot_pool, slot_stride, w, nullptr, y_perm, MOE_F32, ws, ws_bytes, compute);
                if (r != MOE_OK) return r;
            }
        }
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
        r = moe_combine(y_perm, MOE_F32, topk_w, inv_perm, T, k, d, ly.shared_w != nullptr, ly.y, act, compute);
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
        // the ids' arrival also retires the previous layer's table copy (earlier on the stream than
        // the route kernel)
        moe_status r = route_ids_to_host(ly, act, T, d, E, k, topk_idx, topk_w, logits, counts, offsets, perm,
                                         inv_perm, host_idx, ev, compute);
        if (r != MOE_OK) return r;
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
                                           ly.shared_w, y_perm, MOE_F32, ws, ws_bytes, compute);
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
            // the resident experts run while the misses are copied in; copies deferred by an earlier
            // split fill (hybrid handling) may have filled some of them, so those are waited for
            r = cache_wait_background(cache, cs);
            if (r == MOE_OK)
                r = moe_expert_ffn_grouped(ly.x, act, T, d, f, E, k, perm, offsets, counts, dev_tables, n_slots,
                                       slot_pool, slot_stride, w, ly.shared_w, y_perm, MOE_F32, ws, ws_bytes, compute);
            if (r == MOE_OK) r = moe_cache_fill(cache, copy, compute);
            if (r == MOE_OK)
                r = moe_expert_ffn_grouped(ly.x, act, T, d, f, E, k, perm, offsets, counts, dev_tables + E, n_slots,
                                           slot_pool, slot_stride, w, nullptr, y_perm, MOE_F32, ws, ws_bytes, compute);
        }
        if (r != MOE_OK) return r;
        r = moe_combine(y_perm, MOE_F32, topk_w, inv_perm, T, k, d, ly.shared_w != nullptr, ly.y, act, compute);
        if (r != MOE_OK) return r;
        r = moe_cache_mark_read(cache, ly.layer, compute);
        if (r != MOE_OK) return r;
    }
    return MOE_OK;
}
