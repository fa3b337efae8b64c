// moe_route: router logits in one fixed binary32 order, top-k selection, renormalised gates.
//
// The pages (FreeToken linux guide, "MoE memory handling") state only that a router activates
// a few experts per token.  The summation order is this library's reading, chosen so that the
// selected ids are reproducible bit for bit: 64 contiguous segments of d/64 elements, each
// summed from +0 in ascending index, joined pairwise neighbours first, bias added last.
//
// Two logits kernels implement that one order:
//   * few tokens (decode): one wave per (expert, group of 8 tokens); lane j owns segment j and
//     the pairwise join is the xor butterfly with strides 1, 2, 4, ..., 32 (a + b == b + a, so
//     every lane ends with the same bits);
//   * many tokens (prefill): an LDS-tiled VALU product, each thread owning 4 tokens x 4
//     experts, running the segments one after another and joining segment sums with a
//     binary-counter stack (the same neighbours-first tree).
// The top-k kernel gives one wave to each token.
#include <hip/hip_runtime.h>

#include "moe_common.h"

namespace moe {
namespace {

constexpr int kTokGroup = 8;

// acc + a*b with two roundings (a*b exact for bf16 inputs, so a fused form gives the same bits)
template <bool kBf16>
__device__ __forceinline__ float madd(float acc, float a, float b) {
    if constexpr (kBf16) {
        return __builtin_fmaf(a, b, acc);
    } else {
#pragma clang fp contract(off)
        float p = a * b;
        return acc + p;
    }
}

template <bool kBf16>
__device__ __forceinline__ float load_elem(const void* base, size_t i) {
    if constexpr (kBf16) return bf16_to_f32(((const uint16_t*)base)[i]);
    else return ((const float*)base)[i];
}

// ---- decode logits: one wave per (expert, token group) --------------------------------------
template <bool kBf16>
__global__ __launch_bounds__(256) void route_logits_wave(const void* __restrict__ x,
                                                          const void* __restrict__ w,
                                                          const float* __restrict__ bias, int T,
                                                          int d, int E, float* __restrict__ logits) {
    const int lane = threadIdx.x & 63;
    const long gw = (long)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
    const int e = (int)(gw % E);
    const int t0 = (int)(gw / E) * kTokGroup;
    if (t0 >= T) return;
    const int nt = min(kTokGroup, T - t0);
    const int S = d / 64;
    const size_t seg = (size_t)lane * S;
    float acc[kTokGroup];
#pragma unroll
    for (int t = 0; t < kTokGroup; ++t) acc[t] = 0.0f;

    if (kBf16 && (S % 8) == 0) {
        const uint4* wr = (const uint4*)((const uint16_t*)w + (size_t)e * d + seg);
        for (int c = 0; c < S / 8; ++c) {
            uint4 wv = wr[c];
            float wf[8] = {bf16_lo(wv.x), bf16_hi(wv.x), bf16_lo(wv.y), bf16_hi(wv.y),
                           bf16_lo(wv.z), bf16_hi(wv.z), bf16_lo(wv.w), bf16_hi(wv.w)};
#pragma unroll
            for (int t = 0; t < kTokGroup; ++t) {
                if (t < nt) {
                    uint4 xv = ((const uint4*)((const uint16_t*)x + (size_t)(t0 + t) * d + seg))[c];
                    float xf[8] = {bf16_lo(xv.x), bf16_hi(xv.x), bf16_lo(xv.y), bf16_hi(xv.y),
                                   bf16_lo(xv.z), bf16_hi(xv.z), bf16_lo(xv.w), bf16_hi(xv.w)};
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[t] = madd<true>(acc[t], xf[i], wf[i]);
                }
            }
        }
    } else {
        for (int i = 0; i < S; ++i) {
            float wf = load_elem<kBf16>(w, (size_t)e * d + seg + i);
#pragma unroll
            for (int t = 0; t < kTokGroup; ++t)
                if (t < nt) acc[t] = madd<kBf16>(acc[t], load_elem<kBf16>(x, (size_t)(t0 + t) * d + seg + i), wf);
        }
    }
    // neighbours-first pairwise join of the 64 segment sums
#pragma unroll
    for (int t = 0; t < kTokGroup; ++t) {
#pragma unroll
        for (int s = 1; s < 64; s <<= 1) acc[t] = acc[t] + __shfl_xor(acc[t], s, 64);
    }
    if (lane < nt) {
        float v = acc[0];
#pragma unroll
        for (int t = 1; t < kTokGroup; ++t)
            if (lane == t) v = acc[t];
        logits[(size_t)(t0 + lane) * E + e] = bias ? v + bias[e] : v;
    }
}

// ---- prefill logits: LDS tiles, 64 tokens x 64 experts per block ------------------------------
constexpr int kTT = 64;  // tokens per tile
constexpr int kTE = 64;  // experts per tile
constexpr int kKT = 32;  // inputs per LDS stage

template <bool kBf16>
__global__ __launch_bounds__(256) void route_logits_tiled(const void* __restrict__ x,
                                                           const void* __restrict__ w,
                                                           const float* __restrict__ bias, int T,
                                                           int d, int E, float* __restrict__ logits) {
    __shared__ float xs[kKT][kTT + 4];
    __shared__ float ws[kKT][kTE + 4];
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;  // tx -> experts, ty -> tokens
    const int tb = blockIdx.y * kTT, eb = blockIdx.x * kTE;
    const int S = d / 64;

    float acc[4][4], stk[6][4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = 0.f;

    int seg_pos = 0, seg_idx = 0;
    for (int k0 = 0; k0 < d; k0 += kKT) {
        const int kk = min(kKT, d - k0);
        // stage: 64 rows x kk inputs of x and of w, converted to binary32
        for (int i = tid; i < kTT * kKT; i += 256) {
            int r = i / kKT, c = i % kKT;
            float xv = 0.f, wv = 0.f;
            if (c < kk) {
                if (tb + r < T) xv = load_elem<kBf16>(x, (size_t)(tb + r) * d + k0 + c);
                if (eb + r < E) wv = load_elem<kBf16>(w, (size_t)(eb + r) * d + k0 + c);
            }
            xs[c][r] = xv;
            ws[c][r] = wv;
        }
        __syncthreads();
        for (int c = 0; c < kk; ++c) {
            float4 xv = *(const float4*)&xs[c][ty * 4];
            float4 wv = *(const float4*)&ws[c][tx * 4];
            float xa[4] = {xv.x, xv.y, xv.z, xv.w}, wa[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) acc[a][b] = madd<kBf16>(acc[a][b], xa[a], wa[b]);
            if (++seg_pos == S) {
                // close segment seg_idx: binary-counter join (left sibling + right)
                seg_pos = 0;
                int n = seg_idx++;
#pragma unroll
                for (int lv = 0; lv < 6; ++lv) {
                    if (n & (1 << lv)) {
#pragma unroll
                        for (int a = 0; a < 4; ++a)
#pragma unroll
                            for (int b = 0; b < 4; ++b) acc[a][b] = stk[lv][a][b] + acc[a][b];
                    } else {
#pragma unroll
                        for (int a = 0; a < 4; ++a)
#pragma unroll
                            for (int b = 0; b < 4; ++b) stk[lv][a][b] = acc[a][b];
                        break;
                    }
                }
                if (n != 63) {
#pragma unroll
                    for (int a = 0; a < 4; ++a)
#pragma unroll
                        for (int b = 0; b < 4; ++b) acc[a][b] = 0.f;
                }
            }
        }
        __syncthreads();
    }
    // after segment 63 the joined sum is in acc
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        int t = tb + ty * 4 + a;
        if (t >= T) continue;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            int e = eb + tx * 4 + b;
            if (e < E) logits[(size_t)t * E + e] = bias ? acc[a][b] + bias[e] : acc[a][b];
        }
    }
}

// ---- top-k and gates: one wave per token -------------------------------------------------------
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
}

__global__ __launch_bounds__(256) void route_topk(const float* __restrict__ logits, int T, int E, int k,
                                                  const int32_t* __restrict__ forced,
                                                  int32_t* __restrict__ topk_idx,
                                                  float* __restrict__ topk_w) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
    if (t >= T) return;
    const float* row = logits + (size_t)t * E;
    __shared__ float sel_v_all[4][1024];
    __shared__ int sel_i_all[4][1024];
    float* sel_v = sel_v_all[threadIdx.x >> 6];
    int* sel_i = sel_i_all[threadIdx.x >> 6];

    if (forced) {
        for (int j = lane; j < k; j += 64) {
            int id = forced[(size_t)t * k + j];
            int safe = min(max(id, 0), E - 1);
            sel_i[j] = id;
            sel_v[j] = row[safe];
        }
    } else {
        float v[16];
        unsigned taken = 0;
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            int e = lane + 64 * m;
            v[m] = (e < E) ? row[e] : 0.f;
            if (e >= E) taken |= 1u << m;
        }
        for (int j = 0; j < k; ++j) {
            float bv = 0.f;
            int bi = 0x7FFFFFFF;
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                int e = lane + 64 * m;
                if (!(taken & (1u << m)) && (bi == 0x7FFFFFFF || better(v[m], e, bv, bi))) {
                    bv = v[m];
                    bi = e;
                }
            }
#pragma unroll
            for (int s = 32; s >= 1; s >>= 1) {
                float ov = __shfl_xor(bv, s, 64);
                int oi = __shfl_xor(bi, s, 64);
                if (oi != 0x7FFFFFFF && (bi == 0x7FFFFFFF || better(ov, oi, bv, bi))) {
                    bv = ov;
                    bi = oi;
                }
            }
            if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
            if (lane == 0) {
                sel_i[j] = bi;
                sel_v[j] = bv;
            }
        }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    // gates: softmax over the selected logits in binary64, rounded once
    double m = -INFINITY;
    for (int j = 0; j < k; ++j) m = fmax(m, (double)sel_v[j]);
    double den = 0.0;
    for (int j = 0; j < k; ++j) den += exp((double)sel_v[j] - m);
    for (int j = lane; j < k; j += 64) {
        topk_idx[(size_t)t * k + j] = sel_i[j];
        topk_w[(size_t)t * k + j] = (float)(exp((double)sel_v[j] - m) / den);
    }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_route(const void* x, moe_dtype act, int T, int d, const void* w_router,
                                const float* bias, int E, int k, const int32_t* forced_idx,
                                int32_t* topk_idx, float* topk_w, float* logits, moe_stream s) {
    MOE_CHECK(T >= 0, MOE_ESHAPE, "moe_route: T=%d < 0", T);
    if (T == 0) return MOE_OK;
    MOE_CHECK(act == MOE_F32 || act == MOE_BF16, MOE_EDTYPE, "moe_route: activations must be F32 or BF16");
    MOE_CHECK(E >= 1 && E <= 1024 && k >= 1 && k <= E, MOE_ESHAPE, "moe_route: need 1 <= k <= E <= 1024 (k=%d E=%d)", k, E);
    MOE_CHECK(d >= 64 && d <= 16384 && d % 64 == 0, MOE_ESHAPE, "moe_route: d=%d must be a multiple of 64 in [64,16384]", d);
    MOE_CHECK(x && w_router && topk_idx && topk_w && logits, MOE_EINVAL, "moe_route: NULL pointer");
    MOE_CHECK(T <= (1 << 24), MOE_ESHAPE, "moe_route: T=%d too large", T);
    hipStream_t st = (hipStream_t)s;
    const bool bf = act == MOE_BF16;
    const int S = d / 64;
    const bool vec_ok = !bf || (S % 8 == 0 && ((uintptr_t)x % 16 == 0) && ((uintptr_t)w_router % 16 == 0));
    if (T <= 64 || !vec_ok) {
        long waves = (long)E * ((T + kTokGroup - 1) / kTokGroup);
        dim3 grid((unsigned)((waves + 3) / 4));
        ProfScope p("route_logits_wave", st);
        if (bf) route_logits_wave<true><<<grid, 256, 0, st>>>(x, w_router, bias, T, d, E, logits);
        else route_logits_wave<false><<<grid, 256, 0, st>>>(x, w_router, bias, T, d, E, logits);
    } else {
        dim3 grid((unsigned)((E + kTE - 1) / kTE), (unsigned)((T + kTT - 1) / kTT));
        ProfScope p("route_logits_tiled", st);
        if (bf) route_logits_tiled<true><<<grid, 256, 0, st>>>(x, w_router, bias, T, d, E, logits);
        else route_logits_tiled<false><<<grid, 256, 0, st>>>(x, w_router, bias, T, d, E, logits);
    }
    moe_status r = check_launch("route_logits");
    if (r != MOE_OK) return r;
    {
        ProfScope p("route_topk", st);
        route_topk<<<(T + 3) / 4, 256, 0, st>>>(logits, T, E, k, forced_idx, topk_idx, topk_w);
    }
    return check_launch("route_topk");
}
