// Expert-slot cache shared by all MoE layers: LRU over (layer, expert) keys, slot table,
// fills from the pinned host pool on a copy stream with write-after-read guards.
//
// The pages (FreeToken linux guide, "MoE memory handling" and its mechanism table; FreeToken
// GGUF page, offload backend) fix: GPU expert slots, the full routed pool in host RAM, one LRU
// shared across MoE layers, misses copied over PCIe and kept, and prefill streaming of the
// next layer's experts during the current layer.  The request semantics (hits promoted in
// ascending id, then misses in ascending id taking the lowest free slot or the LRU victim's
// slot) are this library's reading; the oracle's simulator follows the same reading.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <functional>
#include <queue>
#include <vector>

#include "moe_common.h"

using namespace moe;

namespace {
constexpr int kReadRing = 256;  // mark_read events kept; older reads are known complete
constexpr int kStage = 4;       // pinned staging buffers for slot-table uploads

struct SlotInfo {
    int32_t key = -1;   // layer*E + expert, -1 = free
    int32_t prev = -1;  // LRU list (towards older)
    int32_t next = -1;  // LRU list (towards newer)
    int64_t read_seq = -1;
    bool pinned = false;
};

struct PendingCopy {
    int32_t slot, key;
    int64_t wait_seq;
};
}  // namespace

struct moe_cache {
    int L = 0, E = 0, C = 0;
    size_t stride = 0;
    uint8_t* pool = nullptr;
    int32_t* dtable = nullptr;
    const void* const* host = nullptr;
    bool policy_only = true;

    std::vector<int32_t> table;  // key -> slot
    std::vector<SlotInfo> slots;
    int32_t lru_head = -1, lru_tail = -1;  // oldest, newest
    std::priority_queue<int32_t, std::vector<int32_t>, std::greater<int32_t>> free_slots;
    std::vector<std::vector<int32_t>> pinned_by_layer;
    std::vector<PendingCopy> pending;
    bool table_dirty = false;

    int64_t stats[6] = {0, 0, 0, 0, 0, 0};
    std::vector<uint8_t> trace;
    std::vector<int64_t> copy_log;
    int inject_failures = 0;

    int64_t read_seq = 0;
    int64_t shrink_seq = -1;  // reads up to this one may still touch slots removed by a shrink
    hipEvent_t read_ev[kReadRing] = {};
    hipEvent_t fill_ev = nullptr;
    hipEvent_t bg_ev = nullptr;  // end of the copies compute has not waited for yet
    bool bg_pending = false;
    int last_layer = -1;  // layer of the last request
    int32_t* stage[kStage] = {};
    hipEvent_t stage_ev[kStage] = {};
    bool stage_used[kStage] = {};
    int stage_next = 0;

    void unlink(int32_t s) {
        SlotInfo& x = slots[s];
        if (x.prev >= 0) slots[x.prev].next = x.next; else lru_head = x.next;
        if (x.next >= 0) slots[x.next].prev = x.prev; else lru_tail = x.prev;
        x.prev = x.next = -1;
    }
    void push_newest(int32_t s) {
        SlotInfo& x = slots[s];
        x.prev = lru_tail;
        x.next = -1;
        if (lru_tail >= 0) slots[lru_tail].next = s; else lru_head = s;
        lru_tail = s;
    }
};

static moe_status request(moe_cache* c, int layer, const int32_t* ids, int n, int32_t* slots_out,
                          int32_t* n_miss_out, bool prefill) {
    MOE_CHECK(layer >= 0 && layer < c->L, MOE_EINVAL, "cache: layer %d out of [0,%d)", layer, c->L);
    MOE_CHECK(n >= 0 && (n == 0 || ids), MOE_EINVAL, "cache: bad id list");
    MOE_CHECK(n <= c->C, MOE_ECAPACITY, "cache: request of %d experts exceeds %d slots", n, c->C);
    std::vector<int32_t> order(n);
    for (int i = 0; i < n; ++i) {
        MOE_CHECK(ids[i] >= 0 && ids[i] < c->E, MOE_EINVAL, "cache: expert id %d out of [0,%d)", ids[i], c->E);
        order[i] = i;
    }
    std::sort(order.begin(), order.end(), [&](int a, int b) { return ids[a] < ids[b]; });
    for (int i = 1; i < n; ++i)
        MOE_CHECK(ids[order[i]] != ids[order[i - 1]], MOE_EINVAL, "cache: duplicate expert id %d", ids[order[i]]);

    const int32_t base = layer * c->E;
    c->last_layer = layer;
    // plan: victims are the oldest residents outside the request's hits; refuse pinned ones
    int n_miss = 0;
    std::vector<char> is_hit(n, 0);
    for (int i = 0; i < n; ++i) {
        is_hit[i] = c->table[base + ids[order[i]]] >= 0;
        n_miss += !is_hit[i];
    }
    int need_evict = std::max(0, n_miss - (int)c->free_slots.size());
    if (need_evict > 0) {
        std::vector<char> hit_slot(c->C, 0);
        for (int i = 0; i < n; ++i)
            if (is_hit[i]) hit_slot[c->table[base + ids[order[i]]]] = 1;
        int found = 0;
        for (int32_t s = c->lru_head; s >= 0 && found < need_evict; s = c->slots[s].next) {
            if (hit_slot[s]) continue;
            MOE_CHECK(!c->slots[s].pinned, MOE_ESTATE,
                      "cache: evicting slot %d (layer %d expert %d) that is not marked read yet", s,
                      c->slots[s].key / c->E, c->slots[s].key % c->E);
            ++found;
        }
        MOE_CHECK(found == need_evict, MOE_ECAPACITY, "cache: not enough evictable slots");
    }
    // hits first, ascending id
    for (int i = 0; i < n; ++i) {
        if (!is_hit[i]) continue;
        int32_t s = c->table[base + ids[order[i]]];
        c->unlink(s);
        c->push_newest(s);
    }
    // then misses, ascending id
    for (int i = 0; i < n; ++i) {
        if (is_hit[i]) continue;
        int32_t key = base + ids[order[i]];
        int32_t s;
        if (!c->free_slots.empty()) {
            s = c->free_slots.top();
            c->free_slots.pop();
        } else {
            s = c->lru_head;
            c->unlink(s);
            c->table[c->slots[s].key] = -1;
        }
        c->slots[s].key = key;
        c->table[key] = s;
        c->push_newest(s);
        c->pending.push_back({s, key, c->slots[s].read_seq});
        c->table_dirty = true;
    }
    // pin, report, count
    for (int i = 0; i < n; ++i) {
        int32_t s = c->table[base + ids[order[i]]];
        if (!c->slots[s].pinned) {
            c->slots[s].pinned = true;
            c->pinned_by_layer[layer].push_back(s);
        }
        if (slots_out) slots_out[order[i]] = s;
        c->trace.push_back(is_hit[i] ? 1 : 0);
    }
    if (prefill) {
        c->stats[3] += n;
        c->stats[4] += n_miss;
    } else {
        c->stats[0] += n;
        c->stats[1] += n - n_miss;
        c->stats[2] += n_miss;
    }
    if (n_miss_out) *n_miss_out = n_miss;
    return MOE_OK;
}

static void drop_entry(moe_cache* c, const PendingCopy& p) {
    // the copy never happened: the entry must not look resident
    if (c->table[p.key] == p.slot) c->table[p.key] = -1;
    SlotInfo& x = c->slots[p.slot];
    if (x.key == p.key) {
        c->unlink(p.slot);
        x.key = -1;
        if (x.pinned) {
            // the freed slot no longer belongs to the requesting layer: a later mark_read of that
            // layer must not unpin it (or stamp its read sequence) once another layer owns it
            std::vector<int32_t>& pl = c->pinned_by_layer[p.key / c->E];
            pl.erase(std::remove(pl.begin(), pl.end(), p.slot), pl.end());
        }
        x.pinned = false;
        c->free_slots.push(p.slot);
    }
    c->table_dirty = true;
}

// Make `compute` wait for copies it has not waited for yet (fill_split's deferred copies).
static moe_status wait_background(moe_cache* c, hipStream_t compute) {
    if (c->policy_only || !c->bg_pending) return MOE_OK;
    MOE_HIP(hipStreamWaitEvent(compute, c->bg_ev, 0));
    c->bg_pending = false;
    return MOE_OK;
}

static hipEvent_t read_event_for(moe_cache* c, int64_t seq) {
    // events older than the ring are complete (checked before each ring entry is reused)
    if (seq <= 0 || seq <= c->read_seq - kReadRing) return nullptr;
    return c->read_ev[seq % kReadRing];
}

extern "C" {

moe_status moe_cache_create(int L, int E, int n_slots, size_t slot_stride, void* slot_pool,
                            int32_t* slot_table, const void* const* host_expert, moe_cache** out) {
    MOE_CHECK(out, MOE_EINVAL, "moe_cache_create: out is NULL");
    *out = nullptr;
    MOE_CHECK(L >= 1 && E >= 1 && E <= 4096 && (int64_t)L * E <= (1 << 24), MOE_ESHAPE,
              "moe_cache_create: bad L=%d E=%d", L, E);
    MOE_CHECK(n_slots >= 1, MOE_ECAPACITY, "moe_cache_create: n_slots must be >= 1");
    bool policy = slot_pool == nullptr;
    if (policy) {
        MOE_CHECK(!slot_table && !host_expert, MOE_EINVAL,
                  "moe_cache_create: policy-only mode takes no slot table or host pool");
    } else {
        MOE_CHECK(slot_table && host_expert && slot_stride > 0, MOE_EINVAL,
                  "moe_cache_create: slot table, host pool and stride are required");
        for (int64_t i = 0; i < (int64_t)L * E; ++i)
            MOE_CHECK(host_expert[i], MOE_EINVAL, "moe_cache_create: host_expert[%lld] is NULL", (long long)i);
    }
    moe_cache* c = new (std::nothrow) moe_cache();
    MOE_CHECK(c, MOE_ENOMEM, "moe_cache_create: out of host memory");
    c->L = L;
    c->E = E;
    c->C = n_slots;
    c->stride = slot_stride;
    c->pool = (uint8_t*)slot_pool;
    c->dtable = slot_table;
    c->host = host_expert;
    c->policy_only = policy;
    c->table.assign((size_t)L * E, -1);
    c->slots.assign(n_slots, SlotInfo());
    for (int s = 0; s < n_slots; ++s) c->free_slots.push(s);
    c->pinned_by_layer.assign(L, {});
    if (!policy) {
        moe_status st = MOE_OK;
        auto fail = [&](hipError_t e, const char* w) {
            st = hip_error(e, w);
        };
        hipError_t e;
        for (int i = 0; i < kReadRing && st == MOE_OK; ++i)
            if ((e = hipEventCreateWithFlags(&c->read_ev[i], hipEventDisableTiming)) != hipSuccess)
                fail(e, "hipEventCreate");
        if (st == MOE_OK && (e = hipEventCreateWithFlags(&c->fill_ev, hipEventDisableTiming)) != hipSuccess)
            fail(e, "hipEventCreate");
        if (st == MOE_OK && (e = hipEventCreateWithFlags(&c->bg_ev, hipEventDisableTiming)) != hipSuccess)
            fail(e, "hipEventCreate");
        for (int i = 0; i < kStage && st == MOE_OK; ++i) {
            if ((e = hipHostMalloc((void**)&c->stage[i], (size_t)L * E * 4, hipHostMallocDefault)) != hipSuccess)
                fail(e, "hipHostMalloc");
            else if ((e = hipEventCreateWithFlags(&c->stage_ev[i], hipEventDisableTiming)) != hipSuccess)
                fail(e, "hipEventCreate");
        }
        if (st == MOE_OK) {
            std::fill(c->stage[0], c->stage[0] + (size_t)L * E, -1);
            if ((e = hipMemcpy(slot_table, c->stage[0], (size_t)L * E * 4, hipMemcpyHostToDevice)) != hipSuccess)
                fail(e, "hipMemcpy(slot_table)");
        }
        if (st != MOE_OK) {
            moe_cache_destroy(c);
            return st;
        }
    }
    *out = c;
    return MOE_OK;
}

moe_status moe_cache_lookup(moe_cache* c, int layer, const int32_t* ids, int n, int32_t* slots_out,
                            int32_t* n_miss_out) {
    MOE_CHECK(c, MOE_EINVAL, "moe_cache_lookup: NULL cache");
    return request(c, layer, ids, n, slots_out, n_miss_out, false);
}

}  // extern "C"

// Enqueue the copies of `todo` on cs (each after the last read of its slot); failed copies leave
// their entries non-resident.  Returns the first error.
static moe_status copy_entries(moe_cache* c, const std::vector<PendingCopy>& todo, hipStream_t cs) {
    moe_status result = MOE_OK;
    int n_copied = 0;
    for (const PendingCopy& p : todo) {
        c->copy_log.push_back(p.slot);
        c->copy_log.push_back(p.key);
        c->copy_log.push_back(p.wait_seq);
        if (c->inject_failures > 0) {
            --c->inject_failures;
            drop_entry(c, p);
            result = set_error(MOE_EHIP, "moe_cache_fill: injected copy failure (slot %d)", p.slot);
            continue;
        }
        if (c->policy_only) {
            ++n_copied;
            continue;
        }
        hipError_t e = hipSuccess;
        hipEvent_t w = read_event_for(c, p.wait_seq);
        if (w) e = hipStreamWaitEvent(cs, w, 0);
        if (e == hipSuccess)
            e = hipMemcpyAsync(c->pool + (size_t)p.slot * c->stride, c->host[p.key], c->stride,
                               hipMemcpyHostToDevice, cs);
        if (e != hipSuccess) {
            drop_entry(c, p);
            result = hip_error(e, "moe_cache_fill: copy");
            continue;
        }
        ++n_copied;
    }
    c->stats[5] += (int64_t)n_copied * (int64_t)c->stride;
    return result;
}

// Upload the whole host table on cs from a staging buffer whose previous upload has finished.
static moe_status upload_table(moe_cache* c, hipStream_t cs) {
    int i = c->stage_next;
    c->stage_next = (i + 1) % kStage;
    if (c->stage_used[i]) MOE_HIP(hipEventSynchronize(c->stage_ev[i]));
    memcpy(c->stage[i], c->table.data(), c->table.size() * 4);
    MOE_HIP(hipMemcpyAsync(c->dtable, c->stage[i], c->table.size() * 4, hipMemcpyHostToDevice, cs));
    MOE_HIP(hipEventRecord(c->stage_ev[i], cs));
    c->stage_used[i] = true;
    c->table_dirty = false;
    return MOE_OK;
}

static moe_status fill_impl(moe_cache* c, hipStream_t cs, hipStream_t compute, const int32_t* later, int n_later) {
    std::vector<PendingCopy> todo, bg;
    for (const PendingCopy& p : c->pending) {
        bool is_later = false;
        for (int i = 0; i < n_later && !is_later; ++i) is_later = p.key % c->E == later[i] && p.key / c->E == c->last_layer;
        (is_later ? bg : todo).push_back(p);
    }
    c->pending.clear();
    moe_status result = copy_entries(c, todo, cs);
    if (c->policy_only) {
        moe_status r2 = copy_entries(c, bg, cs);
        return result != MOE_OK ? result : r2;
    }
    // compute waits for this request's copies and for earlier copies it has not waited for
    if (c->table_dirty || !todo.empty() || c->bg_pending) {
        if (c->table_dirty) {
            moe_status r = upload_table(c, cs);
            if (r != MOE_OK) return r;
        }
        MOE_HIP(hipEventRecord(c->fill_ev, cs));
        MOE_HIP(hipStreamWaitEvent(compute, c->fill_ev, 0));
        c->bg_pending = false;
    }
    if (!bg.empty()) {
        moe_status r2 = copy_entries(c, bg, cs);
        if (result == MOE_OK) result = r2;
        if (c->table_dirty) {
            moe_status r = upload_table(c, cs);
            if (r != MOE_OK) return r;
        }
        MOE_HIP(hipEventRecord(c->bg_ev, cs));
        c->bg_pending = true;
    }
    return result;
}

extern "C" {

moe_status moe_cache_fill(moe_cache* c, moe_stream copy, moe_stream compute) {
    MOE_CHECK(c, MOE_EINVAL, "moe_cache_fill: NULL cache");
    return fill_impl(c, (hipStream_t)copy, (hipStream_t)compute, nullptr, 0);
}

moe_status moe_cache_fill_split(moe_cache* c, const int32_t* later, int n_later, moe_stream copy,
                                moe_stream compute) {
    MOE_CHECK(c, MOE_EINVAL, "moe_cache_fill_split: NULL cache");
    MOE_CHECK(n_later >= 0 && (n_later == 0 || later), MOE_EINVAL, "moe_cache_fill_split: bad id list");
    return fill_impl(c, (hipStream_t)copy, (hipStream_t)compute, later, n_later);
}

moe_status moe_cache_prefetch_layer(moe_cache* c, int layer, moe_stream copy, moe_stream compute) {
    MOE_CHECK(c, MOE_EINVAL, "moe_cache_prefetch_layer: NULL cache");
    std::vector<int32_t> ids(c->E);
    for (int e = 0; e < c->E; ++e) ids[e] = e;
    moe_status st = request(c, layer, ids.data(), c->E, nullptr, nullptr, true);
    if (st != MOE_OK) return st;
    return moe_cache_fill(c, copy, compute);
}

moe_status moe_cache_mark_read(moe_cache* c, int layer, moe_stream compute) {
    MOE_CHECK(c, MOE_EINVAL, "moe_cache_mark_read: NULL cache");
    MOE_CHECK(layer >= 0 && layer < c->L, MOE_EINVAL, "moe_cache_mark_read: layer %d out of range", layer);
    int64_t seq = c->read_seq + 1;
    if (!c->policy_only) {
        hipEvent_t ev = c->read_ev[seq % kReadRing];
        if (seq > kReadRing) MOE_HIP(hipEventSynchronize(ev));  // the read it recorded is complete
        MOE_HIP(hipEventRecord(ev, (hipStream_t)compute));
    }
    c->read_seq = seq;
    for (int32_t s : c->pinned_by_layer[layer]) {
        c->slots[s].read_seq = seq;
        c->slots[s].pinned = false;
    }
    c->pinned_by_layer[layer].clear();
    return MOE_OK;
}

moe_status moe_cache_resize(moe_cache* c, int n_slots, moe_stream copy, moe_stream compute) {
    MOE_CHECK(c, MOE_EINVAL, "moe_cache_resize: NULL cache");
    MOE_CHECK(n_slots >= 1, MOE_ECAPACITY, "moe_cache_resize: n_slots must be >= 1");
    MOE_CHECK(c->pending.empty(), MOE_ESTATE, "moe_cache_resize: call moe_cache_fill for the pending misses first");
    for (int l = 0; l < c->L; ++l)
        MOE_CHECK(c->pinned_by_layer[l].empty(), MOE_ESTATE,
                  "moe_cache_resize: layer %d is not marked read (resize only at a safe point)", l);
    if (n_slots >= c->C) {
        // grow: new slots are free
        for (int s = c->C; s < n_slots; ++s) {
            SlotInfo fresh;
            fresh.read_seq = c->shrink_seq;  // a regrown slot may still be read by older kernels
            c->slots.push_back(fresh);
            c->free_slots.push(s);
        }
        c->C = n_slots;
        return wait_background(c, (hipStream_t)compute);
    }
    // shrink: keep the n_slots most recently used entries
    c->shrink_seq = c->read_seq;
    int resident = 0;
    for (const SlotInfo& x : c->slots) resident += x.key >= 0;
    while (resident > n_slots) {
        const int32_t s = c->lru_head;
        c->unlink(s);
        c->table[c->slots[s].key] = -1;
        c->slots[s].key = -1;
        --resident;
        c->table_dirty = true;
    }
    // kept entries in removed slots move to the lowest free slots below n_slots, taken in
    // ascending old-slot order; each copy waits for the last read of the slot it overwrites
    std::vector<int32_t> free_low;
    for (int s = 0; s < n_slots; ++s)
        if (c->slots[s].key < 0) free_low.push_back(s);
    size_t next_free = 0;
    std::vector<std::pair<int32_t, int32_t>> moves;  // (old, new)
    for (int s = n_slots; s < c->C; ++s)
        if (c->slots[s].key >= 0) moves.push_back({s, free_low[next_free++]});
    hipStream_t cs = (hipStream_t)copy;
    for (auto [from, to] : moves) {
        if (!c->policy_only) {
            hipEvent_t w = read_event_for(c, c->slots[to].read_seq);
            if (w) MOE_HIP(hipStreamWaitEvent(cs, w, 0));
            MOE_HIP(hipMemcpyAsync(c->pool + (size_t)to * c->stride, c->pool + (size_t)from * c->stride, c->stride,
                                   hipMemcpyDeviceToDevice, cs));
        }
        // the moved entry takes the old slot's place in the LRU list
        SlotInfo& dst = c->slots[to];
        SlotInfo& src = c->slots[from];
        dst.key = src.key;
        dst.read_seq = src.read_seq;
        dst.pinned = false;
        dst.prev = src.prev;
        dst.next = src.next;
        if (src.prev >= 0) c->slots[src.prev].next = to; else c->lru_head = to;
        if (src.next >= 0) c->slots[src.next].prev = to; else c->lru_tail = to;
        c->table[dst.key] = to;
        src = SlotInfo();
        c->copy_log.push_back(to);
        c->copy_log.push_back(dst.key);
        c->copy_log.push_back(-2 - (int64_t)from);  // a move: -2 - source slot
        c->table_dirty = true;
    }
    c->slots.resize(n_slots);
    c->C = n_slots;
    decltype(c->free_slots) fresh;
    for (int s = 0; s < n_slots; ++s)
        if (c->slots[s].key < 0) fresh.push(s);
    c->free_slots.swap(fresh);
    if (c->policy_only || !c->table_dirty) return wait_background(c, (hipStream_t)compute);
    // Evicted entries leave the table as -1.  Kernels enqueued before this call may still read the
    // table row of their layer (mark_read is asynchronous), so the upload waits for every read
    // recorded so far, not only for the reads of the move targets.
    if (hipEvent_t w = read_event_for(c, c->read_seq)) MOE_HIP(hipStreamWaitEvent(cs, w, 0));
    int i = c->stage_next;
    c->stage_next = (i + 1) % kStage;
    if (c->stage_used[i]) MOE_HIP(hipEventSynchronize(c->stage_ev[i]));
    memcpy(c->stage[i], c->table.data(), c->table.size() * 4);
    MOE_HIP(hipMemcpyAsync(c->dtable, c->stage[i], c->table.size() * 4, hipMemcpyHostToDevice, cs));
    MOE_HIP(hipEventRecord(c->stage_ev[i], cs));
    c->stage_used[i] = true;
    c->table_dirty = false;
    MOE_HIP(hipEventRecord(c->fill_ev, cs));
    MOE_HIP(hipStreamWaitEvent((hipStream_t)compute, c->fill_ev, 0));
    c->bg_pending = false;  // the deferred copies ran on cs before fill_ev
    return MOE_OK;
}

moe_status moe_cache_stats(const moe_cache* c, int64_t out[6]) {
    MOE_CHECK(c && out, MOE_EINVAL, "moe_cache_stats: NULL argument");
    for (int i = 0; i < 6; ++i) out[i] = c->stats[i];
    return MOE_OK;
}

moe_status moe_cache_trace(const moe_cache* c, uint8_t* hitmiss, int64_t cap, int64_t* n) {
    MOE_CHECK(c && n && (cap <= 0 || hitmiss), MOE_EINVAL, "moe_cache_trace: bad arguments");
    int64_t tot = (int64_t)c->trace.size();
    if (cap > 0) memcpy(hitmiss, c->trace.data(), (size_t)std::min(cap, tot));
    *n = tot;
    return MOE_OK;
}

moe_status moe_cache_copy_log(const moe_cache* c, int64_t* out, int64_t cap, int64_t* n) {
    MOE_CHECK(c && n && (cap <= 0 || out), MOE_EINVAL, "moe_cache_copy_log: bad arguments");
    int64_t tot = (int64_t)c->copy_log.size() / 3;
    if (cap > 0) memcpy(out, c->copy_log.data(), (size_t)std::min(cap, tot) * 3 * sizeof(int64_t));
    *n = tot;
    return MOE_OK;
}

moe_status moe_cache_inject_copy_failures(moe_cache* c, int n) {
    MOE_CHECK(c && n >= 0, MOE_EINVAL, "moe_cache_inject_copy_failures: bad arguments");
    c->inject_failures = n;
    return MOE_OK;
}

moe_status moe_cache_slot_of(const moe_cache* c, int layer, int expert, int32_t* slot) {
    MOE_CHECK(c && slot, MOE_EINVAL, "moe_cache_slot_of: NULL argument");
    MOE_CHECK(layer >= 0 && layer < c->L && expert >= 0 && expert < c->E, MOE_EINVAL,
              "moe_cache_slot_of: (%d,%d) out of range", layer, expert);
    *slot = c->table[(size_t)layer * c->E + expert];
    return MOE_OK;
}

}  // extern "C"

namespace moe {
// Library-internal: make `compute` wait for deferred (fill_split) copies before a launch that may
// read their slots ahead of the next fill.
moe_status cache_wait_background(moe_cache* c, hipStream_t compute) { return wait_background(c, compute); }

// Pinned host image of (layer, expert), or nullptr (policy-only cache).  Library-internal.
const void* cache_host_image(const moe_cache* c, int layer, int expert) {
    if (!c || !c->host || layer < 0 || layer >= c->L || expert < 0 || expert >= c->E) return nullptr;
    return c->host[(size_t)layer * c->E + expert];
}
}  // namespace moe

extern "C" {
void moe_cache_destroy(moe_cache* c) {
    if (!c) return;
    if (!c->policy_only) {
        for (int i = 0; i < kStage; ++i) {
            if (c->stage_ev[i]) {
                (void)hipEventSynchronize(c->stage_ev[i]);
                (void)hipEventDestroy(c->stage_ev[i]);
            }
            if (c->stage[i]) (void)hipHostFree(c->stage[i]);
        }
        if (c->fill_ev) {
            (void)hipEventSynchronize(c->fill_ev);
            (void)hipEventDestroy(c->fill_ev);
        }
        if (c->bg_ev) {
            (void)hipEventSynchronize(c->bg_ev);
            (void)hipEventDestroy(c->bg_ev);
        }
        for (int i = 0; i < kReadRing; ++i)
            if (c->read_ev[i]) (void)hipEventDestroy(c->read_ev[i]);
    }
    delete c;
}

}  // extern "C"
