// moe_permute: stable counting sort of the T*k (token, choice) pairs by expert id.
//
// The pages do not describe this step; the plain reading is a counting sort of the flat pair
// ids t*k + j, stable within an expert.  One workgroup does it without atomics on
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

template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void permute_kernel(const int32_t* __restrict__ ids, int N, int E,
                                                             int nbits, int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ perm,
                                                             int32_t* __restrict__ inv_perm) {
    constexpr int NT = WAVES * 64;
    constexpr int EPT = (kMaxE + NT - 1) / NT;  // experts per thread in the scan
    __shared__ int32_t run[WAVES][kMaxE];
    __shared__ int32_t s_wave[WAVES];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    for (int i = tid; i < WAVES * E; i += NT) run[i / E][i % E] = 0;
    __syncthreads();

    const int per = ((N + WAVES - 1) / WAVES + 63) / 64 * 64;  // stretch length, whole batches
    const int lo = min(N, w * per), hi = min(N, lo + per);
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    // 1. per-wave counts
    for (int b = lo; b < hi; b += 64) {
        const int i = b + lane;
        const bool act = i < hi;
        const uint64_t active = __ballot(act);
        const int e = act ? min(max(ids[i], 0), E - 1) : 0;  // out-of-range ids are misfiled, never out of bounds
        const uint64_t m = match_mask(e, nbits, active);
        if (act && (m >> lane) == 1ull) run[w][e] += __popcll(m);  // highest lane of its group
    }
    __syncthreads();

    // 2. counts and offsets: thread tid owns experts [tid*EPT, tid*EPT + EPT)
    int c[EPT];
    int own = 0;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int e = tid * EPT + j;
        int v = 0;
        if (e < E)
            for (int ww = 0; ww < WAVES; ++ww) v += run[ww][e];
        c[j] = v;
        own += v;
    }
    int incl = own;  // integer scans: order does not matter
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
        const int v = __shfl_up(incl, sh, 64);
        if (lane >= sh) incl += v;
    }
    if (lane == 63) s_wave[w] = incl;
    __syncthreads();
    int base = incl - own;
    for (int ww = 0; ww < w; ++ww) base += s_wave[ww];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int e = tid * EPT + j;
        if (e < E) {
            counts[e] = c[j];
            offsets[e] = base;
            int off = base;
            for (int ww = 0; ww < WAVES; ++ww) {  // start of wave ww's run of expert e
                const int n = run[ww][e];
                run[ww][e] = off;
                off += n;
            }
            base += c[j];
            if (e == E - 1) offsets[E] = base;
        }
    }
    __syncthreads();

    // 3. stable scatter
    for (int b = lo; b < hi; b += 64) {
        const int i = b + lane;
        const bool act = i < hi;
        const uint64_t active = __ballot(act);
        const int e = act ? min(max(ids[i], 0), E - 1) : 0;
        const uint64_t m = match_mask(e, nbits, active);
        if (act) {
            const int pos = run[w][e] + __popcll(m & lt);
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
    const int N = T * k;
    if (N <= 4096) permute_kernel<4><<<1, 256, 0, st>>>(topk_idx, N, E, nbits, counts, offsets, perm, inv_perm);
    else permute_kernel<16><<<1, 1024, 0, st>>>(topk_idx, N, E, nbits, counts, offsets, perm, inv_perm);
    return check_launch("permute");
}
