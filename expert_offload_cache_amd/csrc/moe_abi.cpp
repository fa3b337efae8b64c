// Host-side entry points of libmoe: errors, version, slot packing, workspace sizing,
// pinned memory and kernel timing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <functional>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "moe_common.h"
#include "slot_layout.h"

namespace moe {

static thread_local std::string g_last_error;

moe_status set_error(moe_status code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

moe_status hip_error(hipError_t e, const char* what) {
    return set_error(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

moe_status check_launch(const char* kernel) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return set_error(MOE_EHIP, "launch of %s: %s", kernel, hipGetErrorString(e));
    return MOE_OK;
}

// ---- kernel timing -----------------------------------------------------------------------------
namespace {
struct Pending {
    std::string name;
    hipEvent_t a, b;
};
struct Total {
    std::string name;
    double ms;
    int64_t n;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<hipEvent_t> g_ev_pool;
std::vector<Pending> g_pending;
std::vector<Total> g_totals;
thread_local std::vector<std::pair<std::string, hipEvent_t>> t_open;

hipEvent_t take_event() {
    if (!g_ev_pool.empty()) {
        hipEvent_t e = g_ev_pool.back();
        g_ev_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}
}  // namespace

bool profiling_on() { return g_prof_on; }

void prof_begin(const char* kernel, hipStream_t s) {
    std::lock_guard<std::mutex> g(g_prof_mu);
    hipEvent_t a = take_event();
    if (a) (void)hipEventRecord(a, s);
    t_open.emplace_back(kernel, a);
}

void prof_end(hipStream_t s) {
    std::lock_guard<std::mutex> g(g_prof_mu);
    if (t_open.empty()) return;
    auto top = t_open.back();
    t_open.pop_back();
    hipEvent_t b = take_event();
    if (!top.second || !b) return;
    (void)hipEventRecord(b, s);
    g_pending.push_back({top.first, top.second, b});
}

}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_last_error(void) { return g_last_error.c_str(); }
const char* moe_version(void) { return "libmoe 0.1 gfx950"; }

size_t moe_slot_bytes(int d, int f, moe_dtype w) {
    if (!slot_shape_ok(d, f, w)) return 0;
    return align_up(slot_bytes_raw(d, f, w), 256);
}

// ---- packing ------------------------------------------------------------------------------------
// Runs fn(i) for i in [0, n) on up to 16 host threads.
static void parallel_for(int n, const std::function<void(int)>& fn) {
    int nt = (int)std::min<unsigned>(16u, std::max(1u, std::thread::hardware_concurrency()));
    nt = std::min(nt, n);
    if (nt <= 1) {
        for (int i = 0; i < n; ++i) fn(i);
        return;
    }
    std::vector<std::thread> th;
    for (int t = 0; t < nt; ++t)
        th.emplace_back([&, t] {
            for (int i = t; i < n; i += nt) fn(i);
        });
    for (auto& x : th) x.join();
}

// one 16-row block of a dense [R, K] matrix: fragment kb, lane l <- row 16rb + l%16,
// inputs 32kb + 8(l/16) .. +7
static void pack_dense_block(const uint8_t* src, int rb, int K, int esz, uint8_t* blk) {
    for (int kb = 0; kb < K / 32; ++kb) {
        uint8_t* frag = blk + (size_t)kb * 512 * esz;
        for (int l = 0; l < 64; ++l) {
            int r = rb * 16 + (l % 16), k0 = kb * 32 + 8 * (l / 16);
            memcpy(frag + (size_t)8 * l * esz, src + ((size_t)r * K + k0) * esz, (size_t)8 * esz);
        }
    }
}

static inline int nib(const uint8_t* row, int e) {
    uint8_t b = row[e >> 1];
    return (e & 1) ? (b >> 4) : (b & 0xF);
}

// one 16-row block of an int4 [R, K] matrix: K/128 fragments, then bf16 scales [16][K/128]
static void pack_int4_block(const uint8_t* q, const uint16_t* sc, int rb, int K, uint8_t* blk) {
    int G = K / 128;
    for (int g = 0; g < G; ++g)
        for (int l = 0; l < 64; ++l) {
            int r = rb * 16 + (l % 16), qq = l / 16;
            const uint8_t* row = q + (size_t)r * (K / 2);
            uint32_t words[4];
            for (int s = 0; s < 4; ++s) {
                int k0 = g * 128 + 32 * s + 8 * qq;
                uint32_t w = 0;
                for (int p = 0; p < 4; ++p) {
                    w |= (uint32_t)nib(row, k0 + 2 * p) << (4 * p);
                    w |= (uint32_t)nib(row, k0 + 2 * p + 1) << (16 + 4 * p);
                }
                words[s] = w;
            }
            memcpy(blk + (size_t)g * 1024 + 16 * l, words, 16);
        }
    uint16_t* sdst = (uint16_t*)(blk + (size_t)G * 1024);
    for (int r = 0; r < 16; ++r) memcpy(sdst + r * G, sc + (size_t)(rb * 16 + r) * G, (size_t)G * 2);
}

moe_status moe_pack_expert(moe_dtype w, int d, int f, const void* wg, const void* wu, const void* wd,
                           const void* sg, const void* su, const void* sd, void* slot_out) {
    MOE_CHECK(slot_shape_ok(d, f, w), MOE_ESHAPE, "moe_pack_expert: unsupported shape d=%d f=%d dtype=%d", d,
              f, (int)w);
    MOE_CHECK(wg && wu && wd && slot_out, MOE_EINVAL, "moe_pack_expert: NULL weight or output");
    const bool i4 = w == MOE_INT4_G128;
    if (i4) MOE_CHECK(sg && su && sd, MOE_EINVAL, "moe_pack_expert: int4 needs scales");
    else MOE_CHECK(!sg && !su && !sd, MOE_EINVAL, "moe_pack_expert: scales only for int4");
    uint8_t* out = (uint8_t*)slot_out;
    size_t total = moe_slot_bytes(d, f, w);
    memset(out + slot_bytes_raw(d, f, w), 0, total - slot_bytes_raw(d, f, w));
    const int esz = (w == MOE_F32) ? 4 : 2;
    const int ngu = f / 16, ndn = d / 16;
    // work items: gate block b, up block b (b < f/16), then down block b (b < d/16)
    parallel_for(2 * ngu + ndn, [&](int i) {
        if (i < 2 * ngu) {
            int b = i / 2, which = i % 2;
            const void* m = which ? wu : wg;
            uint8_t* blk = out + gu_block_offset(b, which, d, w);
            if (i4) pack_int4_block((const uint8_t*)m, (const uint16_t*)(which ? su : sg), b, d, blk);
            else pack_dense_block((const uint8_t*)m, b, d, esz, blk);
        } else {
            int b = i - 2 * ngu;
            uint8_t* blk = out + down_block_offset(b, d, f, w);
            if (i4) pack_int4_block((const uint8_t*)wd, (const uint16_t*)sd, b, f, blk);
            else pack_dense_block((const uint8_t*)wd, b, f, esz, blk);
        }
    });
    return MOE_OK;
}

// ---- pinned memory ------------------------------------------------------------------------------
moe_status moe_pinned_alloc(size_t bytes, void** out) {
    MOE_CHECK(out && bytes > 0, MOE_EINVAL, "moe_pinned_alloc: bad arguments");
    *out = nullptr;
    hipError_t e = hipHostMalloc(out, bytes, hipHostMallocDefault);
    if (e != hipSuccess) {
        *out = nullptr;
        return set_error(MOE_ENOMEM, "hipHostMalloc(%zu): %s", bytes, hipGetErrorString(e));
    }
    return MOE_OK;
}

void moe_pinned_free(void* p) {
    if (p) (void)hipHostFree(p);
}

// ---- timing -------------------------------------------------------------------------------------
void moe_profile_enable(int on) {
    std::lock_guard<std::mutex> g(g_prof_mu);
    g_prof_on = on != 0;
}

moe_status moe_profile_collect(void) {
    std::lock_guard<std::mutex> g(g_prof_mu);
    for (auto& p : g_pending) {
        MOE_HIP(hipEventSynchronize(p.b));
        float ms = 0.f;
        MOE_HIP(hipEventElapsedTime(&ms, p.a, p.b));
        bool found = false;
        for (auto& t : g_totals)
            if (t.name == p.name) {
                t.ms += ms;
                t.n += 1;
                found = true;
                break;
            }
        if (!found) g_totals.push_back({p.name, (double)ms, 1});
        g_ev_pool.push_back(p.a);
        g_ev_pool.push_back(p.b);
    }
    g_pending.clear();
    return MOE_OK;
}

moe_status moe_profile_get(int i, char* name, int name_cap, double* total_ms, int64_t* launches) {
    std::lock_guard<std::mutex> g(g_prof_mu);
    MOE_CHECK(i >= 0 && i < (int)g_totals.size(), MOE_EINVAL, "moe_profile_get: index %d out of range", i);
    if (name && name_cap > 0) {
        strncpy(name, g_totals[i].name.c_str(), (size_t)name_cap - 1);
        name[name_cap - 1] = 0;
    }
    if (total_ms) *total_ms = g_totals[i].ms;
    if (launches) *launches = g_totals[i].n;
    return MOE_OK;
}

void moe_profile_reset(void) {
    std::lock_guard<std::mutex> g(g_prof_mu);
    g_totals.clear();
}

}  // extern "C"
