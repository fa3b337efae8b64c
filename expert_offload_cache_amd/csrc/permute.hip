// moe_permute: stable counting sort of the T*k (token, choice) pairs by expert id.
//
// The pages do not describe this step; the plain reading is a counting sort of the flat pair
// ids t*k + j, stable within an expert.  One workgroup of 16 waves does it without atomics on
// positions, so the result is deterministic:
//   1. wave w owns a contiguous stretch of pairs and counts it per expert into its own LDS row
//      (within a wave, equal ids are found with ballots over the id bits; one lane per
//      distinct id writes, so no two lanes touch the same counter);
//   2. per expert: counts = sum over waves, offsets = exclusive scan over experts, and the
//      start of wave w's run = offset + counts of waves before w;
//   3. each wave walks its stretch again in order and writes pair i to position
//      start + (equal ids on lower lanes of the same batch), advancing its run starts.
#include <hip/hip_runtime.h>

#include "moe_common.h"

namespace moe {
namespace {

constexpr int kWaves = 16;
constexpr int kMaxE = 1024;

__device__ __forceinline__ uint64_t match_mask(int e, int nbits, uint64_t active) {
    uint64_t m = active;
    for (int b = 0; b < nbits; ++b) {
        bool bit = (e >> b) & 1;
        uint64_t bal = __ballot(bit);
        m &= bit ? bal : ~bal;
    }
    return m;
}

__global__ __launch_bounds__(1024) void permute_kernel(const int32_t* __restrict__ ids, int N, int E,
                                                       int nbits, int32_t* __restrict__ counts,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ perm,
                                                       int32_t* __restrict__ inv_perm) {
    __shared__ int32_t run[kWaves][kMaxE];
    __shared__ int32_t scan_tmp[1024];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    for (int i = tid; i < kWaves * kMaxE; i += 1024) (&run[0][0])[i] = 0;
    __syncthreads();

    const int per = ((N + kWaves - 1) / kWaves + 63) / 64 * 64;  // stretch length, whole batches
    const int lo = min(N, w * per), hi = min(N, lo + per);
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    // 1. per-wave counts
    for (int b = lo; b < hi; b += 64) {
        int i = b + lane;
        bool act = i < hi;
        uint64_t active = __ballot(act);
        int e = act ? min(max(ids[i], 0), E - 1) : 0;  // out-of-range ids are misfiled, never out of bounds
        uint64_t m = match_mask(e, nbits, active);
        if (act && (m >> lane) == 1ull) run[w][e] += __popcll(m);  // highest lane of its group
    }
    __syncthreads();

    // 2. counts, offsets, run starts (thread e owns expert e)
    int c = 0;
    if (tid < E)
        for (int v = 0; v < kWaves; ++v) c += run[v][tid];
    scan_tmp[tid] = (tid < E) ? c : 0;
    __syncthreads();
    for (int s = 1; s < 1024; s <<= 1) {  // inclusive Hillis-Steele scan (integer: order-free)
        int v = (tid >= s) ? scan_tmp[tid - s] : 0;
        __syncthreads();
        scan_tmp[tid] += v;
        __syncthreads();
    }
    if (tid < E) {
        int off = scan_tmp[tid] - c;
        counts[tid] = c;
        offsets[tid] = off;
        if (tid == E - 1) offsets[E] = scan_tmp[tid];
        for (int v = 0; v < kWaves; ++v) {
            int n = run[v][tid];
            run[v][tid] = off;
            off += n;
        }
    }
    __syncthreads();

    // 3. stable scatter
    for (int b = lo; b < hi; b += 64) {
        int i = b + lane;
        bool act = i < hi;
        uint64_t active = __ballot(act);
        int e = act ? min(max(ids[i], 0), E - 1) : 0;
        uint64_t m = match_mask(e, nbits, active);
        if (act) {
            int pos = run[w][e] + __popcll(m & lt);
            perm[pos] = i;
            inv_perm[i] = pos;
        }
        // every lane has read its run start before the group's last lane advances it
        __builtin_amdgcn_wave_barrier();
        if (act && (m >> lane) == 1ull) run[w][e] += __popcll(m);
        __builtin_amdgcn_wave_barrier();
    }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_permute(const int32_t* topk_idx, int T, int k, int E, int32_t* counts,
                                  int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* ws,
                                  size_t ws_bytes, moe_stream s) {
    (void)ws;
    (void)ws_bytes;
    MOE_CHECK(T >= 0 && k >= 1 && E >= 1 && E <= kMaxE && k <= E, MOE_ESHAPE,
              "moe_permute: need T >= 0, 1 <= k <= E <= %d (T=%d k=%d E=%d)", kMaxE, T, k, E);
    MOE_CHECK((int64_t)T * k <= (1 << 24), MOE_ESHAPE, "moe_permute: T*k too large");
    MOE_CHECK(counts && offsets && (T == 0 || (topk_idx && perm && inv_perm)), MOE_EINVAL,
              "moe_permute: NULL pointer");
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    hipStream_t st = (hipStream_t)s;
    ProfScope p("permute", st);
    permute_kernel<<<1, 1024, 0, st>>>(topk_idx, T * k, E, nbits, counts, offsets, perm, inv_perm);
    return check_launch("permute");
}
