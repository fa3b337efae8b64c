// Grouped SwiGLU experts for few tokens per expert (decode): streaming GEMV over expert slots.
//
// Expert weights are reached through the slot table (FreeToken GGUF page, "MoE backends",
// offload backend: GPU expert slots; FreeToken linux guide, memory tier table).  The expert
// form (SwiGLU, no biases) is the plain reading; the pages do not give it.
//
// Work decomposition (weights stationary, activations streamed through LDS):
//   * a workgroup owns one 16-row block of one expert -- the gate and up blocks of the same
//     16 outputs in the first kernel, one W_d block in the second -- and splits its inputs K
//     among KS waves;
//   * the slot layout stores a 16-row block as fragments of 16 rows x 32 inputs (bf16, f32) or
//     16 x 128 (int4) in lane order, so every weight load is 1 KB contiguous per wave (16 bytes
//     per lane); each wave issues all of its fragment loads at once into registers, which keeps
//     several KB in flight per wave from the first cycle;
//   * the expert's tokens are processed in groups of NTG: the group's activation rows are
//     staged in LDS once per workgroup, and lanes read them as 16-byte broadcasts (the 16 lanes
//     of a row quarter share an address);
//   * lane l always works on row l%16 and input quarter l/16, so a lane's partial sums are
//     joined over the four quarters with two shuffles and over the waves through LDS.
//
// Arithmetic: bf16 x bf16 pairs with v_dot2_f32_bf16 (binary32 accumulation).  An int4 nibble
// u becomes the bf16 value 128 + u with one AND-OR per pair (u fills the low mantissa bits of
// 0x4300), so the dot gives sum (136 + q) x; subtracting 136 * sum x per 128-input group and
// multiplying by the group scale gives sum q*s*x without a per-weight subtraction.
#include <hip/hip_runtime.h>

#include "ffn.h"
#include "ffn_common.h"
#include "slot_layout.h"

#include <algorithm>

namespace moe {
namespace {

// LDS layout: [NTG][K] activations, then [KS][NTG][NM][16] partial sums
template <int MODE, int W, bool kBf16Act, int FPW, int NTG>
__global__ __launch_bounds__(512) void ffn_gemv_kernel(FfnArgs a) {
    constexpr int NM = (MODE == kGateUp) ? 2 : 1;
    constexpr int LV = Frag<W>::kLaneVec;
    constexpr int ESZ = kBf16Act ? 2 : 4;
    extern __shared__ __align__(16) uint8_t smem[];

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int KS = blockDim.x >> 6;
    const int q = lane >> 4, r16 = lane & 15;
    const int rb = blockIdx.x;
    const int K = (MODE == kGateUp) ? a.d : a.f;
    const int nfrag = K / Frag<W>::kIn;
    uint8_t* s_x = smem;
    float* s_red = (float*)(smem + (size_t)NTG * K * ESZ);

    int e, chunk;
    if (!find_work(a.counts, a.E, a.T, NTG, a.shared_w != nullptr, blockIdx.y, e, chunk)) return;
    const bool shared = (e == -1);
    const int n_all = __builtin_amdgcn_readfirstlane(shared ? a.T : a.counts[e]);
    const int i0 = chunk * NTG;                 // this workgroup's tokens: i0 .. i0 + nt - 1
    const int nt = __builtin_amdgcn_readfirstlane(min(NTG, n_all - i0));
    const int p0 = __builtin_amdgcn_readfirstlane(shared ? a.T * a.k : a.offsets[e]);
    const uint8_t* base;
    if (shared) {
        base = a.shared_w;
    } else {
        const int slot = __builtin_amdgcn_readfirstlane(a.slot_of_expert[e]);
        if (slot < 0 || slot >= a.n_slots) {
            // absent or invalid slot: flag it and give the expert's rows zeros; nothing is read
            if (threadIdx.x == 0) *a.status = 1;
            for (int i = threadIdx.x; i < nt * 16; i += blockDim.x) {
                const size_t row = (size_t)(p0 + i0 + i / 16);
                const int c = rb * 16 + i % 16;
                if (MODE == kGateUp) {
                    if (kBf16Act) ((uint16_t*)a.h)[row * a.f + c] = 0;
                    else ((float*)a.h)[row * a.f + c] = 0.f;
                } else {
                    a.y_perm[row * a.d + c] = 0.f;
                }
            }
            return;
        }
        base = a.pool + (size_t)slot * a.stride;
    }

    // ---- this wave's fragments: issue every load now ---------------------------------------
    const int per = (nfrag + KS - 1) / KS;
    const int f0 = __builtin_amdgcn_readfirstlane(wv * per);
    const int nmine = __builtin_amdgcn_readfirstlane(max(0, min(per, nfrag - f0)));
    const uint8_t* mats[NM];
    if constexpr (MODE == kGateUp) {
        mats[0] = base + gu_block_offset(rb, 0, a.d, (moe_dtype)W);
        mats[NM - 1] = base + gu_block_offset(rb, 1, a.d, (moe_dtype)W);
    } else {
        mats[0] = base + down_block_offset(rb, a.d, a.f, (moe_dtype)W);
    }
    uint4 wreg[FPW][NM][LV];
    float sc[FPW][NM];
#pragma unroll
    for (int c = 0; c < FPW; ++c) {
        const int fr = f0 + min(c, max(nmine - 1, 0));  // clamped: loads stay inside the block
#pragma unroll
        for (int m = 0; m < NM; ++m) {
#pragma unroll
            for (int v = 0; v < LV; ++v)
                wreg[c][m][v] = load_stream(mats[m] + (size_t)min(fr, nfrag - 1) * Frag<W>::kBytes +
                                            (size_t)lane * 16 * LV + 16 * v);
            if constexpr (W == MOE_INT4_G128)
                sc[c][m] = bf16_to_f32(*(const uint16_t*)(mats[m] + (size_t)nfrag * 1024 +
                                                           ((size_t)r16 * nfrag + min(fr, nfrag - 1)) * 2));
        }
    }

    const uint8_t* in_base = (MODE == kGateUp) ? (const uint8_t*)a.x : (const uint8_t*)a.h;
    const size_t row_bytes = (size_t)K * ESZ;

    {
        // ---- stage the group's activation rows in LDS (16-byte vectors) ----------------------
        {
            // source row of each token: its activation row (gate/up) or its h row (down)
            int* s_row = (int*)(s_red + (size_t)KS * NTG * NM * 16);
            if ((int)threadIdx.x < nt) {
                const int i = threadIdx.x;
                s_row[i] = (MODE == kGateUp) ? (shared ? (i0 + i) : (a.perm[p0 + i0 + i] / a.k)) : (p0 + i0 + i);
            }
            __syncthreads();
            const int vec_per_row = (int)(row_bytes / 16);
            for (int v = threadIdx.x; v < nt * vec_per_row; v += blockDim.x) {
                const int i = v / vec_per_row, c = v - i * vec_per_row;
                ((uint4*)(s_x + (size_t)i * row_bytes))[c] =
                    ((const uint4*)(in_base + (size_t)s_row[i] * row_bytes))[c];
            }
        }
        __syncthreads();

        float acc[NTG][NM];
        gemv_group<W, kBf16Act, FPW, NTG, NM>(wreg, sc, s_x, row_bytes, f0, nmine, nt, q, acc);

        // ---- join the four input quarters, then the waves -----------------------------------
#pragma unroll
        for (int i = 0; i < NTG; ++i) {
            if (i < nt) {
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    const float v = quarter_sum_low(acc[i][m]);
                    if (lane < 16) s_red[((wv * NTG + i) * NM + m) * 16 + lane] = v;
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
                for (int w2 = 0; w2 < KS; ++w2) s += s_red[((w2 * NTG + i) * NM + m) * 16 + r];
                v[m] = s;
            }
            const size_t row = (size_t)(p0 + i0 + i);
            if constexpr (MODE == kGateUp) {
                const float h = silu_mul(v[0], v[NM - 1]);
                if (kBf16Act) ((uint16_t*)a.h)[row * a.f + rb * 16 + r] = f32_to_bf16(h);
                else ((float*)a.h)[row * a.f + rb * 16 + r] = h;
            } else {
                a.y_perm[row * a.d + rb * 16 + r] = v[0];
            }
        }
    }
}

struct Plan {
    int fpw, ks, ntg;
    size_t lds;
};

// fragments per wave: the smallest of 4/8/16 that needs at most 8 waves
Plan plan_for(int K, int kin, int esz, int T) {
    const int nfrag = K / kin;
    Plan p{4, 1, 1, 0};
    for (int f : {4, 8, 16}) {
        p.fpw = f;
        p.ks = (nfrag + f - 1) / f;
        if (p.ks <= 8) break;
    }
    // tokens per LDS group: up to 16, with activations + partial sums within 64 KB
    auto lds = [&](int g) { return (size_t)g * K * esz + (size_t)p.ks * g * 2 * 16 * 4; };
    int ntg = 1;
    while (ntg < 16 && ntg < T && lds(2 * ntg) <= 65536) ntg <<= 1;
    p.ntg = ntg;
    p.lds = lds(ntg) + 16 * sizeof(int);  // + source-row table
    return p;
}

template <int MODE, int W, bool kBf16Act, int FPW>
moe_status launch_ntg(const FfnArgs& a, const Plan& p, dim3 grid, hipStream_t st, const char* name) {
    dim3 block(64 * p.ks);
    ProfScope ps(name, st);
    switch (p.ntg) {
        case 1: ffn_gemv_kernel<MODE, W, kBf16Act, FPW, 1><<<grid, block, p.lds, st>>>(a); break;
        case 2: ffn_gemv_kernel<MODE, W, kBf16Act, FPW, 2><<<grid, block, p.lds, st>>>(a); break;
        case 4: ffn_gemv_kernel<MODE, W, kBf16Act, FPW, 4><<<grid, block, p.lds, st>>>(a); break;
        case 8: ffn_gemv_kernel<MODE, W, kBf16Act, FPW, 8><<<grid, block, p.lds, st>>>(a); break;
        default: ffn_gemv_kernel<MODE, W, kBf16Act, FPW, 16><<<grid, block, p.lds, st>>>(a); break;
    }
    return check_launch(name);
}

template <int MODE, int W, bool kBf16Act>
moe_status launch(const FfnArgs& a, hipStream_t st, const char* name) {
    const int K = (MODE == kGateUp) ? a.d : a.f;
    const Plan p = plan_for(K, Frag<W>::kIn, kBf16Act ? 2 : 4, a.T);
    // work items: sum over experts of ceil(n_e / ntg) <= T*k/ntg + min(E, T*k), plus the shared chunks
    const int64_t tk = (int64_t)a.T * a.k;
    const int64_t items = (tk + p.ntg - 1) / p.ntg + std::min<int64_t>(a.E, tk) +
                          (a.shared_w ? (a.T + p.ntg - 1) / p.ntg : 0);
    if (items > 65535) return set_error(MOE_ESHAPE, "%s: %lld work items exceed one launch", name, (long long)items);
    dim3 grid((unsigned)((MODE == kGateUp ? a.f : a.d) / 16), (unsigned)items);
    if constexpr (W == MOE_INT4_G128) {  // dequantised fragments are 4x larger: at most 8 per wave
        if (p.fpw == 4) return launch_ntg<MODE, W, kBf16Act, 4>(a, p, grid, st, name);
        Plan q = p;
        q.fpw = 8;
        q.ks = (K / 128 + 7) / 8;
        q.lds = (size_t)q.ntg * K * 2 + (size_t)q.ks * q.ntg * 2 * 16 * 4 + 16 * sizeof(int);
        if (q.ks > 8 || q.lds > 65536) return set_error(MOE_ESHAPE, "%s: K=%d too large for int4 weights", name, K);
        return launch_ntg<MODE, W, kBf16Act, 8>(a, q, grid, st, name);
    } else {
        switch (p.fpw) {
            case 4: return launch_ntg<MODE, W, kBf16Act, 4>(a, p, grid, st, name);
            case 8: return launch_ntg<MODE, W, kBf16Act, 8>(a, p, grid, st, name);
            default: return launch_ntg<MODE, W, kBf16Act, 16>(a, p, grid, st, name);
        }
    }
}

}  // namespace

moe_status ffn_gemv(const FfnArgs& a, moe_dtype act, moe_dtype w, hipStream_t st) {
    moe_status r;
    if (w == MOE_BF16 && act == MOE_BF16) {
        r = launch<kGateUp, MOE_BF16, true>(a, st, "ffn_gemv_gateup_bf16");
        if (r == MOE_OK) r = launch<kDown, MOE_BF16, true>(a, st, "ffn_gemv_down_bf16");
    } else if (w == MOE_INT4_G128 && act == MOE_BF16) {
        r = launch<kGateUp, MOE_INT4_G128, true>(a, st, "ffn_gemv_gateup_int4");
        if (r == MOE_OK) r = launch<kDown, MOE_INT4_G128, true>(a, st, "ffn_gemv_down_int4");
    } else if (w == MOE_F32 && act == MOE_F32) {
        r = launch<kGateUp, MOE_F32, false>(a, st, "ffn_gemv_gateup_f32");
        if (r == MOE_OK) r = launch<kDown, MOE_F32, false>(a, st, "ffn_gemv_down_f32");
    } else {
        return set_error(MOE_EDTYPE, "moe_expert_ffn_grouped: unsupported act/weight dtypes (%d,%d)", (int)act, (int)w);
    }
    return r;
}

}  // namespace moe
