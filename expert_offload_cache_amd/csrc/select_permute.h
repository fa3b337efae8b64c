// Device code shared by the router's top-k selection and the permutation by expert: the order
// that ranks experts, and the one-workgroup stable counting sort of (token, choice) pairs.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {

constexpr int kPermMaxE = 1024;

// expert i with logit v beats expert bi with logit bv: larger logit, or equal logit and lower id
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
}

// lanes of `active` whose e equals this lane's e (ballots over the id bits)
__device__ __forceinline__ uint64_t match_mask(int e, int nbits, uint64_t active) {
    uint64_t m = active;
    for (int b = 0; b < nbits; ++b) {
        bool bit = (e >> b) & 1;
        uint64_t bal = __ballot(bit);
        m &= bit ? bal : ~bal;
    }
    return m;
}

// One wave counts the pairs [lo, hi) per expert into its own LDS row my_run (within a wave, equal ids
// are found with ballots over the id bits; one lane per distinct id writes).
__device__ __forceinline__ void count_stretch(const int32_t* ids, int lo, int hi, int E, int nbits, int32_t* my_run) {
    const int lane = threadIdx.x & 63;
    for (int b = lo; b < hi; b += 64) {
        const int i = b + lane;
        const bool act = i < hi;
        const uint64_t active = __ballot(act);
        const int e = act ? min(max(ids[i], 0), E - 1) : 0;
        const uint64_t m = match_mask(e, nbits, active);
        if (act && (m >> lane) == 1ull) my_run[e] += __popcll(m);  // highest lane of its group
    }
}

// One wave places the pairs [lo, hi) in order: pair i goes to my_run[e] + (equal ids on lower lanes of
// the same batch), and the run starts advance.
__device__ __forceinline__ void place_stretch(const int32_t* ids, int lo, int hi, int E, int nbits, int32_t* my_run,
                                              int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm) {
    const int lane = threadIdx.x & 63;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int b = lo; b < hi; b += 64) {
        const int i = b + lane;
        const bool act = i < hi;
        const uint64_t active = __ballot(act);
        const int e = act ? min(max(ids[i], 0), E - 1) : 0;
        const uint64_t m = match_mask(e, nbits, active);
        if (act) {
            const int pos = my_run[e] + __popcll(m & lt);
            perm[pos] = i;
            inv_perm[i] = pos;
        }
        // every lane has read its run start before the group's last lane advances it
        __builtin_amdgcn_wave_barrier();
        if (act && (m >> lane) == 1ull) my_run[e] += __popcll(m);
        __builtin_amdgcn_wave_barrier();
    }
}

// Stable counting sort of the N flat pair ids t*k + j by expert id ids[i], run by one workgroup
// of WAVES waves, without atomics on positions (so the result is deterministic):
//   1. wave w owns a contiguous stretch of pairs and counts it per expert into its own LDS row
//      (within a wave, equal ids are found with ballots over the id bits; one lane per distinct id
//      writes, so no two lanes touch the same counter);
//   2. per expert: counts = sum over waves, offsets = exclusive scan over experts, and the start
//      of wave w's run = offset + counts of waves before w;
//   3. each wave walks its stretch again in order and writes pair i to position
//      start + (equal ids on lower lanes of the same batch), advancing its run starts.
// `ids` may point to global memory or LDS; `run` is LDS of WAVES * E ints, `s_wave` of WAVES.
// Out-of-range ids are clamped into [0, E) (misfiled, never out of bounds).
template <int WAVES>
__device__ void permute_block(const int32_t* ids, int N, int E, int nbits, int32_t* __restrict__ counts,
                              int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                              int32_t* __restrict__ inv_perm, int32_t* run, int32_t* s_wave) {
    constexpr int NT = WAVES * 64;
    constexpr int EPT = (kPermMaxE + NT - 1) / NT;  // experts per thread in the scan
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    for (int i = tid; i < WAVES * E; i += NT) run[i] = 0;
    __syncthreads();

    const int per = ((N + WAVES - 1) / WAVES + 63) / 64 * 64;  // stretch length, whole batches
    const int lo = min(N, w * per), hi = min(N, lo + per);
    int32_t* my_run = run + w * E;

    // 1. per-wave counts
    count_stretch(ids, lo, hi, E, nbits, my_run);
    __syncthreads();

    // 2. counts and offsets: thread tid owns experts [tid*EPT, tid*EPT + EPT)
    int c[EPT];
    int own = 0;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int e = tid * EPT + j;
        int v = 0;
        if (e < E)
            for (int ww = 0; ww < WAVES; ++ww) v += run[ww * E + e];
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
                const int n = run[ww * E + e];
                run[ww * E + e] = off;
                off += n;
            }
            base += c[j];
            if (e == E - 1) offsets[E] = base;
        }
    }
    __syncthreads();

    // 3. stable scatter
    place_stretch(ids, lo, hi, E, nbits, my_run, perm, inv_perm);
}

}  // namespace moe
