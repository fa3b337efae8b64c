// moe_permute: stable counting sort of the T*k (token, choice) pairs by expert id.
//
// The pages do not describe this step; the plain reading is a counting sort of the flat pair
// ids t*k + j, stable within an expert, done without atomics on positions (permute_block in
// select_permute.h; for many pairs split over workgroups, below), so the result is deterministic.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "moe_common.h"
#include "select_permute.h"

namespace moe {
namespace {

constexpr int kMaxE = kPermMaxE;
// the split sort: one workgroup per kSplitPairs pairs, at most kSplitMaxGroups (beyond 8192 pairs
// one workgroup is the slower: at 49,152 pairs it takes 77 us)
constexpr int kSplitPairs = 2048;
constexpr int kSplitMaxGroups = 256;
constexpr int kSplitMinPairs = 8192;

template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void permute_kernel(const int32_t* __restrict__ ids, int N, int E,
                                                             int nbits, int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ perm,
                                                             int32_t* __restrict__ inv_perm) {
    __shared__ int32_t run[WAVES * kMaxE];
    __shared__ int32_t s_wave[WAVES];
    permute_block<WAVES>(ids, N, E, nbits, counts, offsets, perm, inv_perm, run, s_wave);
}

// Many pairs: the same counting sort over G workgroups, still without atomics on positions.
// Workgroup g owns the pairs [g*CH, min(N, (g+1)*CH)).
//   permute_count: its waves count their stretches per expert (count_stretch) and the workgroup's
//     counts go to table[g][e] (the caller's workspace);
//   permute_place: every workgroup reads the whole table: expert totals (counts), their exclusive
//     scan over experts (offsets), and its own start per expert = offset + the counts of the
//     workgroups before it; its waves' run starts follow from their own counts, and the pairs are
//     placed in order (place_stretch).  Workgroup 0 writes counts and offsets.
// The result is the one-workgroup sort's: every pair's position is (pairs of smaller experts) +
// (pairs of its expert earlier in the flat order).
template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void permute_count(const int32_t* __restrict__ ids, int N, int E, int nbits,
                                                            int CH, int32_t* __restrict__ table) {
    __shared__ int32_t run[WAVES * kMaxE];
    const int tid = threadIdx.x, w = tid >> 6;
    for (int i = tid; i < WAVES * E; i += WAVES * 64) run[i] = 0;
    __syncthreads();
    const int lo_g = blockIdx.x * CH, hi_g = min(N, lo_g + CH);
    const int per = ((hi_g - lo_g + WAVES - 1) / WAVES + 63) / 64 * 64;
    const int lo = min(hi_g, lo_g + w * per), hi = min(hi_g, lo + per);
    count_stretch(ids, lo, hi, E, nbits, run + w * E);
    __syncthreads();
    for (int e = tid; e < E; e += WAVES * 64) {
        int c = 0;
        for (int ww = 0; ww < WAVES; ++ww) c += run[ww * E + e];
        table[(size_t)blockIdx.x * E + e] = c;
    }
}

template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void permute_place(const int32_t* __restrict__ ids, int N, int E, int nbits,
                                                            int CH, int G, const int32_t* __restrict__ table,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ perm,
                                                            int32_t* __restrict__ inv_perm) {
    constexpr int NT = WAVES * 64;
    constexpr int EPT = (kMaxE + NT - 1) / NT;  // experts per thread in the scan
    __shared__ int32_t run[WAVES * kMaxE];
    __shared__ int32_t s_start[kMaxE];
    __shared__ int32_t s_wave[WAVES];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = blockIdx.x;
    for (int i = tid; i < WAVES * E; i += NT) run[i] = 0;
    // expert totals and the counts of the workgroups before this one
    int tot[EPT], before[EPT], own = 0;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int e = tid * EPT + j;
        int t = 0, b = 0;
        if (e < E) {
#pragma unroll 8
            for (int gg = 0; gg < G; ++gg) {  // independent loads, eight in flight
                const int c = table[(size_t)gg * E + e];
                t += c;
                b += gg < g ? c : 0;
            }
        }
        tot[j] = t;
        before[j] = b;
        own += t;
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
            if (g == 0) {
                counts[e] = tot[j];
                offsets[e] = base;
                if (e == E - 1) offsets[E] = base + tot[j];
            }
            s_start[e] = base + before[j];
            base += tot[j];
        }
    }
    // this workgroup's pairs: per-wave counts, then each wave's run start per expert
    const int lo_g = g * CH, hi_g = min(N, lo_g + CH);
    const int per = ((hi_g - lo_g + WAVES - 1) / WAVES + 63) / 64 * 64;
    const int lo = min(hi_g, lo_g + w * per), hi = min(hi_g, lo + per);
    count_stretch(ids, lo, hi, E, nbits, run + w * E);
    __syncthreads();
    for (int e = tid; e < E; e += NT) {
        int off = s_start[e];
        for (int ww = 0; ww < WAVES; ++ww) {
            const int n = run[ww * E + e];
            run[ww * E + e] = off;
            off += n;
        }
    }
    __syncthreads();
    place_stretch(ids, lo, hi, E, nbits, run + w * E, perm, inv_perm);
}

// workgroups of the split sort for N pairs over E experts (0 or 1: one workgroup sorts)
int split_groups(int64_t N, int E) {
    const int64_t g = std::min<int64_t>((N + kSplitPairs - 1) / kSplitPairs, kSplitMaxGroups);
    return (int)std::max<int64_t>(g, 1);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_permute_workspace_bytes(int T, int k, int E) {
    if (T <= 0 || k <= 0 || E <= 0 || E > kMaxE || (int64_t)T * k <= kSplitMinPairs) return 0;
    return (size_t)split_groups((int64_t)T * k, E) * E * sizeof(int32_t);
}

extern "C" moe_status moe_permute(const int32_t* topk_idx, int T, int k, int E, int32_t* counts,
                                  int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* ws,
                                  size_t ws_bytes, moe_stream s) {
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
    const int G = split_groups(N, E);
    if (N > kSplitMinPairs && G > 1 && ws && ws_bytes >= (size_t)G * E * sizeof(int32_t) && (uintptr_t)ws % 4 == 0) {
        // many pairs and a workspace for the per-workgroup counts: the split sort
        const int CH = (N + G - 1) / G;
        permute_count<8><<<G, 512, 0, st>>>(topk_idx, N, E, nbits, CH, (int32_t*)ws);
        moe_status r = check_launch("permute_count");
        if (r != MOE_OK) return r;
        permute_place<8><<<G, 512, 0, st>>>(topk_idx, N, E, nbits, CH, G, (const int32_t*)ws, counts, offsets, perm,
                                            inv_perm);
        return check_launch("permute_place");
    }
    // 8 waves up to 4096 pairs (4.1 us at 512 pairs against 4.5 with 4 waves, 6.8 with 2), 16 above
    if (N <= 4096) permute_kernel<8><<<1, 512, 0, st>>>(topk_idx, N, E, nbits, counts, offsets, perm, inv_perm);
    else permute_kernel<16><<<1, 1024, 0, st>>>(topk_idx, N, E, nbits, counts, offsets, perm, inv_perm);
    return check_launch("permute");
}
