// Grouped SwiGLU experts for few tokens per expert (decode): streaming GEMV over expert slots.
//
// Expert weights are reached through the slot table (FreeToken GGUF page, "MoE backends",
// offload backend: GPU expert slots; FreeToken linux guide, memory tier table).  The expert
// form (SwiGLU, no biases) is the plain reading; the pages do not give it.
//
// Work decomposition.  A workgroup owns one 16-row block of one expert (gate+up pair for the
// first kernel, a W_d block for the second) and splits the inputs K among its KS waves.  The
// slot layout stores each 16-row block as fragments of 16 rows x 32 inputs (bf16/f32) or
// 16 x 128 (int4) in lane order, so every wave load is 1 KB contiguous (16 bytes per lane) and
// each lane always works on one row: lane l holds row l%16 and input quarter q = l/16.  A
// lane's partial sums are joined over the four quarters with two shuffles and over the waves
// through LDS.  Activations are read from L1/L2 (16 lanes share every 16-byte chunk).
//
// Arithmetic: bf16 x bf16 pairs with v_dot2_f32_bf16 (binary32 accumulation).  int4 nibbles u
// become the bf16 value 128 + u with one AND-OR per pair (u sits in the low mantissa bits of
// 0x4300), so the dot gives sum (136 + q) x; subtracting 136 * sum x per 128-input group and
// multiplying by the group scale gives sum q*s*x without any per-weight subtraction.
#include <hip/hip_runtime.h>

#include "ffn.h"
#include "slot_layout.h"

namespace moe {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// Find the a-th expert with a nonzero count (ascending id).  Returns its id, or -1 if a == U,
// or -2 if a > U.  Every lane of the calling wave gets the same answer.
__device__ int find_active(const int32_t* __restrict__ counts, int E, int a) {
    const int lane = threadIdx.x & 63;
    const int per = (E + 63) / 64;
    int nz = 0;
    for (int i = 0; i < per; ++i) {
        int e = lane * per + i;
        nz += (e < E && counts[e] > 0);
    }
    int incl = nz;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
        int v = __shfl_up(incl, s, 64);
        if (lane >= s) incl += v;
    }
    int U = __shfl(incl, 63, 64);
    if (a > U) return -2;
    if (a == U) return -1;
    int excl = incl - nz;
    int found = -1;
    if (a >= excl && a < incl) {
        int r = a - excl;
        for (int i = 0; i < per; ++i) {
            int e = lane * per + i;
            if (e < E && counts[e] > 0) {
                if (r == 0) {
                    found = e;
                    break;
                }
                --r;
            }
        }
    }
    uint64_t who = __ballot(found >= 0);
    return __shfl(found, (int)__builtin_ctzll(who), 64);
}

// per-matrix element traits
template <int W>
struct Frag;
template <>
struct Frag<MOE_BF16> {
    static constexpr int kIn = 32;          // inputs per fragment
    static constexpr int kBytes = 1024;     // bytes per fragment
    static constexpr int kLaneBytes = 16;   // bytes per lane
};
template <>
struct Frag<MOE_F32> {
    static constexpr int kIn = 32;
    static constexpr int kBytes = 2048;
    static constexpr int kLaneBytes = 32;
};
template <>
struct Frag<MOE_INT4_G128> {
    static constexpr int kIn = 128;
};

// Activation chunk: the 8 inputs lane quarter q uses from one fragment sub-step.
template <bool kBf16Act>
struct XChunk {
    uint4 v;  // 8 bf16
};
template <>
struct XChunk<false> {
    float4 a, b;  // 8 f32
};

template <bool kBf16Act>
__device__ __forceinline__ XChunk<kBf16Act> load_x(const void* row, int k0) {
    XChunk<kBf16Act> c;
    if constexpr (kBf16Act) c.v = *(const uint4*)((const uint16_t*)row + k0);
    else {
        c.a = *(const float4*)((const float*)row + k0);
        c.b = *(const float4*)((const float*)row + k0 + 4);
    }
    return c;
}

// dot of one lane's dense fragment share (8 weights) with its 8 activations
template <int W, bool kBf16Act>
__device__ __forceinline__ float dot8(const uint4* wv, const XChunk<kBf16Act>& x, float acc) {
    if constexpr (W == MOE_BF16) {
        acc = dot2(wv[0].x, x.v.x, acc);
        acc = dot2(wv[0].y, x.v.y, acc);
        acc = dot2(wv[0].z, x.v.z, acc);
        acc = dot2(wv[0].w, x.v.w, acc);
    } else {  // f32 weights, f32 activations
        acc = __builtin_fmaf(__uint_as_float(wv[0].x), x.a.x, acc);
        acc = __builtin_fmaf(__uint_as_float(wv[0].y), x.a.y, acc);
        acc = __builtin_fmaf(__uint_as_float(wv[0].z), x.a.z, acc);
        acc = __builtin_fmaf(__uint_as_float(wv[0].w), x.a.w, acc);
        acc = __builtin_fmaf(__uint_as_float(wv[1].x), x.b.x, acc);
        acc = __builtin_fmaf(__uint_as_float(wv[1].y), x.b.y, acc);
        acc = __builtin_fmaf(__uint_as_float(wv[1].z), x.b.z, acc);
        acc = __builtin_fmaf(__uint_as_float(wv[1].w), x.b.w, acc);
    }
    return acc;
}

constexpr uint32_t kMagic = 0x43004300u;  // bf16 pair (128, 128)
constexpr uint32_t kOnes = 0x3F803F80u;   // bf16 pair (1, 1)

// int4 word (8 nibbles, pairs at bits 4p / 16+4p) -> 4 bf16 pairs of (128 + u)
__device__ __forceinline__ void int4_word_to_bf16(uint32_t w, uint32_t out[4]) {
    out[0] = (w & 0x000F000Fu) | kMagic;
    out[1] = ((w >> 4) & 0x000F000Fu) | kMagic;
    out[2] = ((w >> 8) & 0x000F000Fu) | kMagic;
    out[3] = ((w >> 12) & 0x000F000Fu) | kMagic;
}

enum { kGateUp = 0, kDown = 1 };

template <int MODE, int W, bool kBf16Act, int NT>
__global__ __launch_bounds__(256) void ffn_gemv_kernel(FfnArgs a) {
    constexpr int NM = (MODE == kGateUp) ? 2 : 1;  // matrices sharing the activations
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int KS = blockDim.x >> 6;
    const int q = lane >> 4, r16 = lane & 15;
    const int rb = blockIdx.x;  // 16-row block
    const int ai = blockIdx.y;  // active expert index

    __shared__ int s_tok[NT];
    __shared__ float s_red[4][NT][NM][16];

    int e = find_active(a.counts, a.E, ai);
    if (e == -2 || (e == -1 && !a.shared_w)) return;
    const bool shared = (e == -1);
    const int n = shared ? a.T : a.counts[e];
    const int p0 = shared ? a.T * a.k : a.offsets[e];
    const uint8_t* base;
    if (shared) {
        base = a.shared_w;
    } else {
        int slot = a.slot_of_expert[e];
        if (slot < 0 || slot >= a.n_slots) {
            // absent or invalid slot: flag it and give the expert's rows zeros
            if (threadIdx.x == 0) *a.status = 1;
            const int K_out = (MODE == kGateUp) ? 16 : 16;
            for (int i = threadIdx.x; i < n * K_out; i += blockDim.x) {
                int row = p0 + i / K_out, c = rb * 16 + i % K_out;
                if (MODE == kGateUp) {
                    if (kBf16Act) ((uint16_t*)a.h)[(size_t)row * a.f + c] = 0;
                    else ((float*)a.h)[(size_t)row * a.f + c] = 0.f;
                } else {
                    a.y_perm[(size_t)row * a.d + c] = 0.f;
                }
            }
            return;
        }
        base = a.pool + (size_t)slot * a.stride;
    }

    const int K = (MODE == kGateUp) ? a.d : a.f;
    const int nfrag = K / Frag<W>::kIn;
    const int f0 = wv * nfrag / KS, f1 = (wv + 1) * nfrag / KS;
    const uint8_t* mats[NM];
    if constexpr (MODE == kGateUp) {
        mats[0] = base + gu_block_offset(rb, 0, a.d, (moe_dtype)W);
        mats[NM - 1] = base + gu_block_offset(rb, 1, a.d, (moe_dtype)W);
    } else {
        mats[0] = base + down_block_offset(rb, a.d, a.f, (moe_dtype)W);
    }
    const size_t in_stride = (size_t)K * (kBf16Act ? 2 : 4);
    const uint8_t* in_base = (MODE == kGateUp) ? (const uint8_t*)a.x : (const uint8_t*)a.h;

    for (int i0 = 0; i0 < n; i0 += NT) {
        const int nt = min(NT, n - i0);
        __syncthreads();
        for (int i = threadIdx.x; i < nt; i += blockDim.x) {
            if (MODE == kGateUp) s_tok[i] = shared ? (i0 + i) : (a.perm[p0 + i0 + i] / a.k);
            else s_tok[i] = p0 + i0 + i;  // rows of h in sorted order
        }
        __syncthreads();

        float acc[NT][NM];
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int m = 0; m < NM; ++m) acc[i][m] = 0.f;

        if constexpr (W == MOE_INT4_G128) {
            const int G = K / 128;
            for (int fr = f0; fr < f1; ++fr) {
                uint4 wraw[NM];
                float sc[NM];
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    wraw[m] = *(const uint4*)(mats[m] + (size_t)fr * 1024 + 16 * lane);
                    sc[m] = bf16_to_f32(*(const uint16_t*)(mats[m] + (size_t)G * 1024 + ((size_t)r16 * G + fr) * 2));
                }
                uint32_t wb[NM][16];
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    int4_word_to_bf16(wraw[m].x, &wb[m][0]);
                    int4_word_to_bf16(wraw[m].y, &wb[m][4]);
                    int4_word_to_bf16(wraw[m].z, &wb[m][8]);
                    int4_word_to_bf16(wraw[m].w, &wb[m][12]);
                }
#pragma unroll
                for (int i = 0; i < NT; ++i) {
                    if (i < nt) {
                        const uint8_t* row = in_base + (size_t)s_tok[i] * in_stride;
                        float xs = 0.f, p[NM];
#pragma unroll
                        for (int m = 0; m < NM; ++m) p[m] = 0.f;
#pragma unroll
                        for (int s = 0; s < 4; ++s) {
                            uint4 xv = *(const uint4*)((const uint16_t*)row + fr * 128 + 32 * s + 8 * q);
                            uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                            for (int pp = 0; pp < 4; ++pp) {
                                xs = dot2(kOnes, xw[pp], xs);
#pragma unroll
                                for (int m = 0; m < NM; ++m) p[m] = dot2(wb[m][4 * s + pp], xw[pp], p[m]);
                            }
                        }
#pragma unroll
                        for (int m = 0; m < NM; ++m)
                            acc[i][m] = __builtin_fmaf(sc[m], __builtin_fmaf(-136.0f, xs, p[m]), acc[i][m]);
                    }
                }
            }
        } else {
            constexpr int CH = (NT >= 32) ? 2 : 4;  // fragments in flight per matrix
            constexpr int LV = Frag<W>::kLaneBytes / 16;
            for (int fr = f0; fr < f1; fr += CH) {
                uint4 wl[CH][NM][LV];
#pragma unroll
                for (int c = 0; c < CH; ++c)
                    if (fr + c < f1)
#pragma unroll
                        for (int m = 0; m < NM; ++m)
#pragma unroll
                            for (int v = 0; v < LV; ++v)
                                wl[c][m][v] = *(const uint4*)(mats[m] + (size_t)(fr + c) * Frag<W>::kBytes +
                                                              (size_t)lane * Frag<W>::kLaneBytes + 16 * v);
#pragma unroll
                for (int i = 0; i < NT; ++i) {
                    if (i < nt) {
                        const uint8_t* row = in_base + (size_t)s_tok[i] * in_stride;
#pragma unroll
                        for (int c = 0; c < CH; ++c) {
                            if (fr + c < f1) {
                                XChunk<kBf16Act> xc = load_x<kBf16Act>(row, (fr + c) * 32 + 8 * q);
#pragma unroll
                                for (int m = 0; m < NM; ++m) acc[i][m] = dot8<W, kBf16Act>(wl[c][m], xc, acc[i][m]);
                            }
                        }
                    }
                }
            }
        }

        // join the four input quarters (lanes r, r+16, r+32, r+48), then the waves
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            if (i < nt) {
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    float v = acc[i][m];
                    v += __shfl_xor(v, 16, 64);
                    v += __shfl_xor(v, 32, 64);
                    if (lane < 16) s_red[wv][i][m][lane] = v;
                }
            }
        }
        __syncthreads();
        for (int idx = threadIdx.x; idx < nt * 16; idx += blockDim.x) {
            const int i = idx >> 4, r = idx & 15;
            float v[NM];
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                float s = 0.f;
                for (int w2 = 0; w2 < KS; ++w2) s += s_red[w2][i][m][r];
                v[m] = s;
            }
            if constexpr (MODE == kGateUp) {
                const size_t row = (size_t)(p0 + i0 + i);
                const float h = silu_mul(v[0], v[NM - 1]);
                if (kBf16Act) ((uint16_t*)a.h)[row * a.f + rb * 16 + r] = f32_to_bf16(h);
                else ((float*)a.h)[row * a.f + rb * 16 + r] = h;
            } else {
                a.y_perm[(size_t)(p0 + i0 + i) * a.d + rb * 16 + r] = v[0];
            }
        }
    }
}

template <int MODE, int W, bool kBf16Act>
moe_status launch_nt(const FfnArgs& a, int nt_max, int KS, dim3 grid, hipStream_t st, const char* name) {
    ProfScope p(name, st);
    dim3 block(64 * KS);
#define MOE_GEMV_CASE(NTV) \
    case NTV: ffn_gemv_kernel<MODE, W, kBf16Act, NTV><<<grid, block, 0, st>>>(a); break;
    switch (nt_max) {
        MOE_GEMV_CASE(1)
        MOE_GEMV_CASE(2)
        MOE_GEMV_CASE(4)
        MOE_GEMV_CASE(8)
        MOE_GEMV_CASE(16)
        MOE_GEMV_CASE(32)
        default: ffn_gemv_kernel<MODE, W, kBf16Act, 64><<<grid, block, 0, st>>>(a); break;
    }
#undef MOE_GEMV_CASE
    return check_launch(name);
}

int pick_ks(int nfrag) {
    for (int ks = 4; ks > 1; ks >>= 1)
        if (nfrag % ks == 0 && nfrag / ks >= 1) return ks;
    return 1;
}

}  // namespace

moe_status ffn_gemv(const FfnArgs& a, moe_dtype act, moe_dtype w, int grid_experts, hipStream_t st) {
    int nt_max = 1;
    while (nt_max < a.T && nt_max < 64) nt_max <<= 1;
    const int kin = (w == MOE_INT4_G128) ? 128 : 32;
    const int ks1 = pick_ks(a.d / kin), ks2 = pick_ks(a.f / kin);
    dim3 g1((unsigned)(a.f / 16), (unsigned)grid_experts), g2((unsigned)(a.d / 16), (unsigned)grid_experts);
    moe_status r;
    if (w == MOE_BF16 && act == MOE_BF16) {
        r = launch_nt<kGateUp, MOE_BF16, true>(a, nt_max, ks1, g1, st, "ffn_gemv_gateup_bf16");
        if (r == MOE_OK) r = launch_nt<kDown, MOE_BF16, true>(a, nt_max, ks2, g2, st, "ffn_gemv_down_bf16");
    } else if (w == MOE_INT4_G128 && act == MOE_BF16) {
        r = launch_nt<kGateUp, MOE_INT4_G128, true>(a, nt_max, ks1, g1, st, "ffn_gemv_gateup_int4");
        if (r == MOE_OK) r = launch_nt<kDown, MOE_INT4_G128, true>(a, nt_max, ks2, g2, st, "ffn_gemv_down_int4");
    } else if (w == MOE_F32 && act == MOE_F32) {
        r = launch_nt<kGateUp, MOE_F32, false>(a, nt_max, ks1, g1, st, "ffn_gemv_gateup_f32");
        if (r == MOE_OK) r = launch_nt<kDown, MOE_F32, false>(a, nt_max, ks2, g2, st, "ffn_gemv_down_f32");
    } else {
        return set_error(MOE_EDTYPE, "moe_expert_ffn_grouped: unsupported act/weight dtypes (%d,%d)", (int)act, (int)w);
    }
    return r;
}

}  // namespace moe
