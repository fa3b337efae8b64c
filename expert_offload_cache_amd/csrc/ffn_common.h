// Device code shared by the grouped expert kernels (GEMV and MFMA).
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "ffn.h"
#include "slot_layout.h"

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// streaming 16-byte load (weights are read once per call)
__device__ __forceinline__ uint4 load_stream(const void* p) {
    u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// Stores into y_perm row `row`, column `c`: binary32, or with YB bf16 (round to nearest even), the
// element type the call asked for (a.y_bf16).  The decode kernels pick YB once, outside their
// store loops (a test of the flag at every store measured 2 % slower at a few tokens); the other
// kernels test the flag per store (store_y, store_y4).
template <bool YB>
__device__ __forceinline__ void store_y_as(const FfnArgs& a, size_t row, int c, float v) {
    if constexpr (YB) ((uint16_t*)a.y_perm)[row * a.d + c] = f32_to_bf16(v);
    else ((float*)a.y_perm)[row * a.d + c] = v;
}
// four consecutive columns c .. c+3 (c a multiple of 4)
template <bool YB>
__device__ __forceinline__ void store_y4_as(const FfnArgs& a, size_t row, int c, float v0, float v1, float v2,
                                            float v3) {
    if constexpr (YB) {
        uint2 o;
        o.x = (uint32_t)f32_to_bf16(v0) | ((uint32_t)f32_to_bf16(v1) << 16);
        o.y = (uint32_t)f32_to_bf16(v2) | ((uint32_t)f32_to_bf16(v3) << 16);
        *(uint2*)((uint16_t*)a.y_perm + row * a.d + c) = o;
    } else {
        *(float4*)((float*)a.y_perm + row * a.d + c) = make_float4(v0, v1, v2, v3);
    }
}
__device__ __forceinline__ void store_y(const FfnArgs& a, size_t row, int c, float v) {
    if (a.y_bf16) store_y_as<true>(a, row, c, v);
    else store_y_as<false>(a, row, c, v);
}
__device__ __forceinline__ void store_y4(const FfnArgs& a, size_t row, int c, float v0, float v1, float v2, float v3) {
    if (a.y_bf16) store_y4_as<true>(a, row, c, v0, v1, v2, v3);
    else store_y4_as<false>(a, row, c, v0, v1, v2, v3);
}
// Runs f(std::true_type) when the call's y_perm rows are bf16 (only the down projection stores
// them), else f(std::false_type): one test of the flag for a whole store loop.
template <int MODE, typename F>
__device__ __forceinline__ void with_y_type(const FfnArgs& a, F&& f) {
    if (MODE == kDown && a.y_bf16) f(std::true_type{});
    else f(std::false_type{});
}

// Work item a of the launch -> (expert, token chunk).  Expert e contributes ceil(n_e / ntg)
// chunks, in ascending expert id; the shared expert's ceil(T / ntg) chunks come last (e = -1).
// Only experts whose token count lies in [n_lo, n_hi] take part (the shared expert counts T
// tokens): a grouped call can run its heavy and its light experts in different launches.
// Returns false when a is past the last item.  Every lane of the calling wave agrees.
__device__ __forceinline__ bool find_work(const int32_t* __restrict__ counts, int E, int T, int ntg, bool has_shared, int a,
                          int& e_out, int& chunk_out, int n_lo, int n_hi) {
    const int lane = threadIdx.x & 63;
    const int per = (E + 63) / 64;
    has_shared = has_shared && T >= n_lo && T <= n_hi;
    auto chunks = [&](int n) { return (n >= n_lo && n <= n_hi) ? (n + ntg - 1) / ntg : 0; };
    int nz = 0;
    for (int i = 0; i < per; ++i) {
        int e = lane * per + i;
        if (e < E) nz += chunks(counts[e]);
    }
    int incl = nz;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
        int v = __shfl_up(incl, s, 64);
        if (lane >= s) incl += v;
    }
    const int total = __shfl(incl, 63, 64);
    if (a >= total) {
        const int c = a - total;
        if (!has_shared || c >= (T + ntg - 1) / ntg) return false;
        e_out = -1;
        chunk_out = __builtin_amdgcn_readfirstlane(c);
        return true;
    }
    const int excl = incl - nz;
    int found = -1, chunk = 0;
    if (a >= excl && a < incl) {
        int r = a - excl;
        for (int i = 0; i < per; ++i) {
            int e = lane * per + i;
            if (e >= E) break;
            int ce = chunks(counts[e]);
            if (r < ce) {
                found = e;
                chunk = r;
                break;
            }
            r -= ce;
        }
    }
    const int src = (int)__builtin_ctzll(__ballot(found >= 0));
    // wave-uniform results, so the caller's loops branch on scalars
    e_out = __builtin_amdgcn_readfirstlane(__shfl(found, src, 64));
    chunk_out = __builtin_amdgcn_readfirstlane(__shfl(chunk, src, 64));
    return true;
}

// find_work that also returns the item's slot, token count and first sorted row (the shared expert:
// slot -1, T tokens, row T*k).  The counts and the slot-table row are loaded together, and the
// expert's first row is the exclusive prefix sum of the counts (what offsets holds), so the item's
// weights can be addressed after one round of loads instead of two.
// (MAXPER experts a lane at most: E <= 64 * MAXPER)
template <int kMaxPer>
__device__ __forceinline__ bool find_work_slot(const int32_t* __restrict__ counts, const int32_t* __restrict__ slots,
                                               int E, int T, int k, int ntg, bool has_shared, int a, int& e_out,
                                               int& chunk_out, int& slot_out, int& n_out, int& p0_out, int n_lo,
                                               int n_hi) {
    const int lane = threadIdx.x & 63;
    const int per = (E + 63) / 64;
    has_shared = has_shared && T >= n_lo && T <= n_hi;
    auto chunks = [&](int n) { return (n >= n_lo && n <= n_hi) ? (n + ntg - 1) / ntg : 0; };
    int cnt[kMaxPer], sl[kMaxPer];
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
        const int e = lane * per + i;
        const bool in = i < per && e < E;
        cnt[i] = in ? counts[e] : 0;
        sl[i] = in ? slots[e] : 0;
    }
    int nz = 0, rows = 0;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
        nz += chunks(cnt[i]);
        rows += cnt[i];
    }
    int incl = nz, rincl = rows;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
        const int v = __shfl_up(incl, s, 64), rv = __shfl_up(rincl, s, 64);
        if (lane >= s) {
            incl += v;
            rincl += rv;
        }
    }
    const int total = __shfl(incl, 63, 64);
    if (a >= total) {
        const int c = a - total;
        if (!has_shared || c >= (T + ntg - 1) / ntg) return false;
        e_out = -1;
        chunk_out = __builtin_amdgcn_readfirstlane(c);
        slot_out = -1;
        n_out = T;
        p0_out = T * k;
        return true;
    }
    const int excl = incl - nz;
    int found = -1, chunk = 0, fslot = 0, fn = 0, fp0 = 0;
    if (a >= excl && a < incl) {
        int r = a - excl, row = rincl - rows;  // this lane's first expert's first sorted row
#pragma unroll
        for (int i = 0; i < kMaxPer; ++i) {
            const int ce = chunks(cnt[i]);
            if (found < 0) {
                if (r < ce) {
                    found = lane * per + i;
                    chunk = r;
                    fslot = sl[i];
                    fn = cnt[i];
                    fp0 = row;
                } else {
                    r -= ce;
                    row += cnt[i];
                }
            }
        }
    }
    const int src = (int)__builtin_ctzll(__ballot(found >= 0));
    e_out = __builtin_amdgcn_readfirstlane(__shfl(found, src, 64));
    chunk_out = __builtin_amdgcn_readfirstlane(__shfl(chunk, src, 64));
    slot_out = __builtin_amdgcn_readfirstlane(__shfl(fslot, src, 64));
    n_out = __builtin_amdgcn_readfirstlane(__shfl(fn, src, 64));
    p0_out = __builtin_amdgcn_readfirstlane(__shfl(fp0, src, 64));
    return true;
}

// Work item `a` of a launch -> (expert, chunk, slot, tokens of the expert, its first sorted row):
// find_work_slot where a lane covers at most 4 experts (E <= 256), else find_work and then the
// expert's slot, count and offset.
__device__ __forceinline__ bool find_item(const FfnArgs& f, int ntg, int a, int& e, int& chunk, int& slot, int& n,
                                          int& p0) {
    if (f.E <= 256)
        return find_work_slot<4>(f.counts, f.slot_of_expert, f.E, f.T, f.k, ntg, f.shared_w != nullptr, a, e, chunk,
                                 slot, n, p0, f.n_lo, f.n_hi);
    if (!find_work(f.counts, f.E, f.T, ntg, f.shared_w != nullptr, a, e, chunk, f.n_lo, f.n_hi)) return false;
    const bool shared = e == -1;
    slot = shared ? -1 : __builtin_amdgcn_readfirstlane(f.slot_of_expert[e]);
    n = __builtin_amdgcn_readfirstlane(shared ? f.T : f.counts[e]);
    p0 = __builtin_amdgcn_readfirstlane(shared ? f.T * f.k : f.offsets[e]);
    return true;
}

template <int W>
struct Frag;
template <>
struct Frag<MOE_BF16> {
    static constexpr int kIn = 32, kBytes = 1024, kLaneVec = 1;  // 16-byte vectors per lane
};
template <>
struct Frag<MOE_F32> {
    static constexpr int kIn = 32, kBytes = 2048, kLaneVec = 2;
};
template <>
struct Frag<MOE_INT4_G128> {
    static constexpr int kIn = 128, kBytes = 1024, kLaneVec = 1;
};

constexpr uint32_t kMagic = 0x43004300u;  // bf16 pair (128, 128)
constexpr uint32_t kOnes = 0x3F803F80u;   // bf16 pair (1, 1)

// int4 word (8 nibbles, input pair p at bits 4p and 16+4p) -> 4 bf16 pairs (128 + u)
__device__ __forceinline__ void int4_word_to_bf16(uint32_t w, uint32_t* out) {
    out[0] = (w & 0x000F000Fu) | kMagic;
    out[1] = ((w >> 4) & 0x000F000Fu) | kMagic;
    out[2] = ((w >> 8) & 0x000F000Fu) | kMagic;
    out[3] = ((w >> 12) & 0x000F000Fu) | kMagic;
}


// One token group of one item: acc[i][m] = this lane's partial dot products of its weight share
// (fragments f0 .. f0+nmine-1 of matrix m, already in registers) with token i's staged row.
template <int W, bool kBf16Act, int FPW, int NTG, int NM>
__device__ __forceinline__ void gemv_group(const uint4 (&wreg)[FPW][NM][Frag<W>::kLaneVec],
                                           const float (&sc)[FPW][NM], const uint8_t* s_x, size_t row_bytes,
                                           int f0, int nmine, int nt, int q, float (&acc)[NTG][NM]) {
    constexpr int LV = Frag<W>::kLaneVec;
#pragma unroll
    for (int i = 0; i < NTG; ++i)
#pragma unroll
        for (int m = 0; m < NM; ++m) acc[i][m] = 0.f;
#pragma unroll
    for (int c = 0; c < FPW; ++c) {
        if (c < nmine) {
            const int fr = f0 + c;
            if constexpr (W == MOE_INT4_G128 && NTG <= 4) {
                // few tokens: widen one word (32 inputs) at a time, so only 4 bf16 pairs per
                // matrix are live (fewer registers, more resident waves); the sums run in the
                // same order as in the general branch below
                float xs[NTG], p[NTG][NM];
#pragma unroll
                for (int i = 0; i < NTG; ++i) {
                    xs[i] = 0.f;
#pragma unroll
                    for (int m = 0; m < NM; ++m) p[i][m] = 0.f;
                }
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    uint32_t wb[NM][4];
#pragma unroll
                    for (int m = 0; m < NM; ++m) {
                        const uint4 wv = wreg[c][m][0];
                        const uint32_t w = s == 0 ? wv.x : s == 1 ? wv.y : s == 2 ? wv.z : wv.w;
                        int4_word_to_bf16(w, &wb[m][0]);
                    }
#pragma unroll
                    for (int i = 0; i < NTG; ++i) {
                        if (i < nt) {
                            const uint16_t* xr = (const uint16_t*)(s_x + (size_t)i * row_bytes) + fr * 128 + 8 * q;
                            const uint4 xv = *(const uint4*)(xr + 32 * s);
                            const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                            for (int pp = 0; pp < 4; ++pp) {
                                xs[i] = dot2(kOnes, xw[pp], xs[i]);
#pragma unroll
                                for (int m = 0; m < NM; ++m) p[i][m] = dot2(wb[m][pp], xw[pp], p[i][m]);
                            }
                        }
                    }
                }
#pragma unroll
                for (int i = 0; i < NTG; ++i)
                    if (i < nt)
#pragma unroll
                        for (int m = 0; m < NM; ++m)
                            acc[i][m] = __builtin_fmaf(sc[c][m], __builtin_fmaf(-136.0f, xs[i], p[i][m]), acc[i][m]);
            } else if constexpr (W == MOE_INT4_G128) {
                uint32_t wb[NM][16];
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    int4_word_to_bf16(wreg[c][m][0].x, &wb[m][0]);
                    int4_word_to_bf16(wreg[c][m][0].y, &wb[m][4]);
                    int4_word_to_bf16(wreg[c][m][0].z, &wb[m][8]);
                    int4_word_to_bf16(wreg[c][m][0].w, &wb[m][12]);
                }
#pragma unroll
                for (int i = 0; i < NTG; ++i) {
                    if (i < nt) {
                        const uint16_t* xr = (const uint16_t*)(s_x + (size_t)i * row_bytes) + fr * 128 + 8 * q;
                        float xs = 0.f, p[NM];
#pragma unroll
                        for (int m = 0; m < NM; ++m) p[m] = 0.f;
#pragma unroll
                        for (int s = 0; s < 4; ++s) {
                            const uint4 xv = *(const uint4*)(xr + 32 * s);
                            const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                            for (int pp = 0; pp < 4; ++pp) {
                                xs = dot2(kOnes, xw[pp], xs);
#pragma unroll
                                for (int m = 0; m < NM; ++m) p[m] = dot2(wb[m][4 * s + pp], xw[pp], p[m]);
                            }
                        }
#pragma unroll
                        for (int m = 0; m < NM; ++m)
                            acc[i][m] = __builtin_fmaf(sc[c][m], __builtin_fmaf(-136.0f, xs, p[m]), acc[i][m]);
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < NTG; ++i) {
                    if (i < nt) {
                        if constexpr (W == MOE_BF16) {
                            const uint4 xv =
                                *(const uint4*)((const uint16_t*)(s_x + (size_t)i * row_bytes) + fr * 32 + 8 * q);
#pragma unroll
                            for (int m = 0; m < NM; ++m) {
                                float t = acc[i][m];
                                t = dot2(wreg[c][m][0].x, xv.x, t);
                                t = dot2(wreg[c][m][0].y, xv.y, t);
                                t = dot2(wreg[c][m][0].z, xv.z, t);
                                t = dot2(wreg[c][m][0].w, xv.w, t);
                                acc[i][m] = t;
                            }
                        } else {  // f32 weights and activations
                            const float* xr = (const float*)(s_x + (size_t)i * row_bytes) + fr * 32 + 8 * q;
                            const float4 xa = *(const float4*)xr, xb = *(const float4*)(xr + 4);
#pragma unroll
                            for (int m = 0; m < NM; ++m) {
                                float t = acc[i][m];
                                const uint4 wa = wreg[c][m][0], wb2 = wreg[c][m][LV - 1];
                                t = __builtin_fmaf(as_f32(wa.x), xa.x, t);
                                t = __builtin_fmaf(as_f32(wa.y), xa.y, t);
                                t = __builtin_fmaf(as_f32(wa.z), xa.z, t);
                                t = __builtin_fmaf(as_f32(wa.w), xa.w, t);
                                t = __builtin_fmaf(as_f32(wb2.x), xb.x, t);
                                t = __builtin_fmaf(as_f32(wb2.y), xb.y, t);
                                t = __builtin_fmaf(as_f32(wb2.z), xb.z, t);
                                t = __builtin_fmaf(as_f32(wb2.w), xb.w, t);
                                acc[i][m] = t;
                            }
                        }
                    }
                }
            }
        }
    }
}

}  // namespace moe
