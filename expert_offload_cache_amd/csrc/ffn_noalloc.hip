// moe_expert_ffn_grouped_noalloc: the grouped experts with their scratch (the intermediate h and
// the status word) in a fixed device array of this library instead of a caller workspace, for
// callers that cannot allocate device memory.  Same checks and kernels as moe_expert_ffn_grouped.
//
// The array below exists once per GPU the library runs on and lives until the process ends.  In
// host code its name is only a host-side stand-in, so its device address is looked up once per
// device (hipGetSymbolAddress, with that device current) and only that address is handed to the
// kernels.  Nothing in it needs to start at zero: h is written before it is read, and the status
// word is used only when the caller passes no status pointer (it is then never read back).
#include <hip/hip_runtime.h>

#include <mutex>

#include "ffn.h"

using namespace moe;

namespace {

static_assert(MOE_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static_assert(MOE_NOALLOC_SCRATCH_BYTES > kWsHeader + kPlanBytes, "scratch size");

__device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
uint8_t* g_scratch[kMaxDevices] = {};  // device address of `scratch` on each device, once looked up

// Device address of this device's scratch array (looked up on the first call on the device).
moe_status scratch_on_current_device(uint8_t** out) {
    int dev = -1;
    MOE_HIP(hipGetDevice(&dev));
    MOE_CHECK(dev >= 0 && dev < kMaxDevices, MOE_EINVAL, "moe_expert_ffn_grouped_noalloc: device %d out of range",
              dev);
    std::lock_guard<std::mutex> g(g_lock);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_error(e, "hipGetSymbolAddress(scratch)");
        MOE_CHECK(p && (uintptr_t)p % 256 == 0, MOE_EHIP, "moe_expert_ffn_grouped_noalloc: bad scratch address");
        g_scratch[dev] = (uint8_t*)p;
    }
    *out = g_scratch[dev];
    return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_expert_ffn_grouped_noalloc(const void* x, moe_dtype act, int T, int d, int f, int E, int k,
                                                     const int32_t* perm, const int32_t* offsets,
                                                     const int32_t* counts, const int32_t* slot_of_expert,
                                                     int n_slots, const void* slot_pool, size_t slot_stride,
                                                     moe_dtype w, const void* shared_w, void* y_perm,
                                                     moe_dtype y_dtype, int32_t* status, moe_stream s) {
    FfnArgs a;
    moe_status r = ffn_prepare(a, "moe_expert_ffn_grouped_noalloc", x, act, T, d, f, E, k, perm, offsets, counts,
                               slot_of_expert, n_slots, slot_pool, slot_stride, w, shared_w, y_perm, y_dtype);
    if (r != MOE_OK || T == 0) return r;
    MOE_CHECK(!status || (uintptr_t)status % 4 == 0, MOE_EINVAL,
              "moe_expert_ffn_grouped_noalloc: status must be 4-byte aligned");
    const size_t need = moe_workspace_bytes(T, d, f, E, k, shared_w != nullptr, act, w);
    MOE_CHECK(need <= MOE_NOALLOC_SCRATCH_BYTES, MOE_ENOMEM,
              "moe_expert_ffn_grouped_noalloc: this call needs %zu bytes of scratch, more than the %zu the library "
              "holds per GPU (use moe_expert_ffn_grouped with a workspace)",
              need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
    uint8_t* base = nullptr;
    r = scratch_on_current_device(&base);
    if (r != MOE_OK) return r;
    a.status = status ? status : (int32_t*)base;
    a.plan = base + kWsHeader;
    a.h = base + kWsHeader + kPlanBytes;
    return ffn_run(a, act, w, (hipStream_t)s);
}
