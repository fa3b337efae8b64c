// Grouped SwiGLU experts for few tokens per expert (decode): streaming GEMV over expert slots on
// the vector ALUs, and the dispatch between the decode kernels.  Each projection goes to the
// K-streaming matrix-core kernel (ffn_gemv_ks.hip) where its launch plan applies, else for bf16
// to the split-input matrix-core kernel (ffn_gemv_mfma.hip), else to the kernel below, which
// serves binary32 weights, int4 weights for single tokens, and shapes the others do not cover.
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

// LDS layout: [NTG][K] activations, then [waves][NTG][NM][16] partial sums.
// A workgroup owns RB consecutive 16-row blocks (RB > 1 only where one block is small: the down
// projection's rows hold only f inputs); its waves are RB groups of KSW waves, each group splitting
// its row block's inputs.
// Largest workgroup of a launch shape (bounds the registers the compiler may give each lane).
constexpr int max_threads(int mode, int w) { return (mode == kDown && w != MOE_INT4_G128) ? 1024 : 512; }

template <int MODE, int W, bool kBf16Act, int FPW, int NTG, int RB>
__global__ __launch_bounds__(max_threads(MODE, W)) void ffn_gemv_kernel(FfnArgs a) {
    constexpr int NM = (MODE == kGateUp) ? 2 : 1;
    constexpr int LV = Frag<W>::kLaneVec;
    constexpr int ESZ = kBf16Act ? 2 : 4;
    extern __shared__ __align__(16) uint8_t smem[];

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int KS = blockDim.x >> 6;   // waves in the workgroup
    const int KSW = KS / RB;          // waves per row block
    const int q = lane >> 4, r16 = lane & 15;
    const int rbi = wv / KSW;         // this wave's row block within the workgroup
    const int rb = blockIdx.x * RB + rbi;
    const int K = (MODE == kGateUp) ? a.d : a.f;
    const int nfrag = K / Frag<W>::kIn;
    uint8_t* s_x = smem;
    float* s_red = (float*)(smem + (size_t)NTG * K * ESZ);

    int e, chunk;
    if (!find_work(a.counts, a.E, a.T, NTG, a.shared_w != nullptr, blockIdx.y, e, chunk, a.n_lo, a.n_hi)) return;
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
        if (slot == MOE_SLOT_ELSEWHERE) return;  // rows produced elsewhere: leave them
        if (slot < 0 || slot >= a.n_slots) {
            // absent or invalid slot: flag it and give the expert's rows zeros; nothing is read
            if (threadIdx.x == 0) *a.status = 1;
            for (int i = threadIdx.x; i < nt * 16 * RB; i += blockDim.x) {
                const size_t row = (size_t)(p0 + i0 + i / (16 * RB));
                const int c = blockIdx.x * RB * 16 + i % (16 * RB);
                if (MODE == kGateUp) {
                    if (kBf16Act) ((uint16_t*)a.h)[row * a.f + c] = 0;
                    else ((float*)a.h)[row * a.f + c] = 0.f;
                } else {
                    store_y(a, row, c, 0.f);
                }
            }
            return;
        }
        base = a.pool + (size_t)slot * a.stride;
    }

    // ---- the group's activation rows: issue their loads first ---------------------------------
    // Loads complete in issue order, so activation loads issued after the weight loads could only
    // be used once every weight had arrived.  Lane i < nt of each wave reads token i's source row
    // (its activation row, or its h row in the down projection); each thread then loads up to XV
    // 16-byte vectors of the group's rows into registers, before any weight load.
    const uint8_t* in_base = (MODE == kGateUp) ? (const uint8_t*)a.x : (const uint8_t*)a.h;
    const size_t row_bytes = (size_t)K * ESZ;
    constexpr int XV = (NTG <= 2) ? 2 : 4;  // vectors a thread loads ahead; the copy loop below takes any rest
    const int vpr = (int)(row_bytes / 16);
    const int total = nt * vpr;
    int my_row = 0;
    if (lane < nt)
        my_row = (MODE == kGateUp) ? (shared ? (i0 + lane) : (a.perm[p0 + i0 + lane] / a.k)) : (p0 + i0 + lane);
    u32x4_t xr[XV];
#pragma unroll
    for (int u = 0; u < XV; ++u) {
        // unconditional (clamped) loads: no branch, so they stay in flight together
        const int v = min((int)threadIdx.x + u * (int)blockDim.x, total - 1);
        const int i = v / vpr;
        const int row = __shfl(my_row, i, 64);
        xr[u] = *(const u32x4_t*)(in_base + (size_t)row * row_bytes + (size_t)(v - i * vpr) * 16);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep them ahead of the weight loads

    // ---- this wave's fragments: issue every load now ---------------------------------------
    const int per = (nfrag + KSW - 1) / KSW;
    const int f0 = __builtin_amdgcn_readfirstlane((wv - rbi * KSW) * per);
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

    {
        // ---- stage the group's activation rows in LDS (16-byte vectors) ----------------------
        {
#pragma unroll
            for (int u = 0; u < XV; ++u) {
                const int v = (int)threadIdx.x + u * (int)blockDim.x;
                if (v < total) ((u32x4_t*)s_x)[v] = xr[u];
            }
            // rows beyond XV vectors per thread (large K with many tokens): plain copies
            for (int v = (int)threadIdx.x + XV * (int)blockDim.x; v < total; v += blockDim.x) {
                const int i = v / vpr;
                const int row = (MODE == kGateUp) ? (shared ? (i0 + i) : (a.perm[p0 + i0 + i] / a.k)) : (p0 + i0 + i);
                ((u32x4_t*)s_x)[v] = *(const u32x4_t*)(in_base + (size_t)row * row_bytes + (size_t)(v - i * vpr) * 16);
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
        for (int idx = threadIdx.x; idx < nt * 16 * RB; idx += blockDim.x) {
            const int bi = idx / (nt * 16), rem = idx - bi * nt * 16;
            const int i = rem >> 4, r = rem & 15;
            float v[NM];
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                float s = 0.f;
                for (int w2 = bi * KSW; w2 < (bi + 1) * KSW; ++w2) s += s_red[((w2 * NTG + i) * NM + m) * 16 + r];
                v[m] = s;
            }
            const size_t row = (size_t)(p0 + i0 + i);
            const int col = (blockIdx.x * RB + bi) * 16 + r;
            if constexpr (MODE == kGateUp) {
                const float h = silu_mul(v[0], v[NM - 1]);
                if (kBf16Act) ((uint16_t*)a.h)[row * a.f + col] = f32_to_bf16(h);
                else ((float*)a.h)[row * a.f + col] = h;
            } else {
                store_y(a, row, col, v[0]);
            }
        }
    }
}

struct Plan {
    int fpw, ksw, rb, ntg;
    size_t lds;
};

// Shape of one launch.  Fragments per wave: the smallest of the allowed counts with at most 8 waves
// per workgroup (16 for the dense down projection, measured faster there).  The down projection
// groups up to 4 row blocks per workgroup when one row block is small (K = f inputs), so that a
// workgroup still streams tens of KB of weights.
Plan plan_for(int MODE, int W, int M, int K, int kin, int esz, int T) {
    const int nfrag = K / kin;
    // binary32 fragments are twice as large: at most 8 per wave, like dequantised int4 ones
    const int fpws_bf16[] = {4, 8, 12, 16}, fpws_small[] = {4, 8};
    const int* fpws = W == MOE_BF16 ? fpws_bf16 : fpws_small;
    const int nf = W == MOE_BF16 ? 4 : 2;
    Plan p{0, 0, 1, 1, 0};
    const int rbs[] = {4, 2, 1};
    for (int rb : rbs) {
        if (rb > 1 && (MODE != kDown || (M / 16) % rb != 0 || nfrag * rb > 128)) continue;
        for (int i = 0; i < nf && !p.fpw; ++i) {
            const int ksw = (nfrag + fpws[i] - 1) / fpws[i];
            const int max_waves = max_threads(MODE, W) / 64;
            if (rb * ksw <= max_waves) p = Plan{fpws[i], ksw, rb, 1, 0};
        }
        if (p.fpw) break;
    }
    // tokens per LDS group: up to 16, with activations + partial sums within 64 KB
    const int waves = p.ksw * p.rb;
    const int nm = MODE == kGateUp ? 2 : 1;
    auto lds = [&](int g) { return (size_t)g * K * esz + (size_t)waves * g * nm * 16 * 4; };
    int ntg = 1;
    while (ntg < 16 && ntg < T && lds(2 * ntg) <= 65536) ntg <<= 1;
    p.ntg = ntg;
    p.lds = lds(ntg);
    return p;
}

template <int MODE, int W, bool kBf16Act, int FPW, int RB>
moe_status launch_ntg(const FfnArgs& a, const Plan& p, dim3 grid, hipStream_t st, const char* name) {
    dim3 block(64 * p.ksw * RB);
    ProfScope ps(name, st);
    switch (p.ntg) {
        case 1: ffn_gemv_kernel<MODE, W, kBf16Act, FPW, 1, RB><<<grid, block, p.lds, st>>>(a); break;
        case 2: ffn_gemv_kernel<MODE, W, kBf16Act, FPW, 2, RB><<<grid, block, p.lds, st>>>(a); break;
        case 4: ffn_gemv_kernel<MODE, W, kBf16Act, FPW, 4, RB><<<grid, block, p.lds, st>>>(a); break;
        case 8: ffn_gemv_kernel<MODE, W, kBf16Act, FPW, 8, RB><<<grid, block, p.lds, st>>>(a); break;
        default: ffn_gemv_kernel<MODE, W, kBf16Act, FPW, 16, RB><<<grid, block, p.lds, st>>>(a); break;
    }
    return check_launch(name);
}

template <int MODE, int W, bool kBf16Act, int RB>
moe_status launch_fpw(const FfnArgs& a, const Plan& p, dim3 grid, hipStream_t st, const char* name) {
    if constexpr (W != MOE_BF16) {
        if (p.fpw == 4) return launch_ntg<MODE, W, kBf16Act, 4, RB>(a, p, grid, st, name);
        return launch_ntg<MODE, W, kBf16Act, 8, RB>(a, p, grid, st, name);
    } else {
        switch (p.fpw) {
            case 4: return launch_ntg<MODE, W, kBf16Act, 4, RB>(a, p, grid, st, name);
            case 8: return launch_ntg<MODE, W, kBf16Act, 8, RB>(a, p, grid, st, name);
            case 12: return launch_ntg<MODE, W, kBf16Act, 12, RB>(a, p, grid, st, name);
            default: return launch_ntg<MODE, W, kBf16Act, 16, RB>(a, p, grid, st, name);
        }
    }
}

template <int MODE, int W, bool kBf16Act>
moe_status launch(const FfnArgs& a, hipStream_t st, const char* name) {
    const int K = (MODE == kGateUp) ? a.d : a.f;
    const int M = (MODE == kGateUp) ? a.f : a.d;  // output rows (gate/up: pairs of rows)
    const Plan p = plan_for(MODE, W, M, K, Frag<W>::kIn, kBf16Act ? 2 : 4, a.T);
    if (!p.fpw || p.lds > 65536) return set_error(MOE_ESHAPE, "%s: K=%d too large for this kernel", name, K);
    // work items: sum over experts of ceil(n_e / ntg) <= T*k/ntg + min(E, T*k), plus the shared chunks
    const int64_t items = work_items(a, p.ntg);
    if (items > 65535) return set_error(MOE_ESHAPE, "%s: %lld work items exceed one launch", name, (long long)items);
    dim3 grid((unsigned)(M / 16 / p.rb), (unsigned)items);
    if constexpr (MODE == kDown) {
        if (p.rb == 4) return launch_fpw<MODE, W, kBf16Act, 4>(a, p, grid, st, name);
        if (p.rb == 2) return launch_fpw<MODE, W, kBf16Act, 2>(a, p, grid, st, name);
    }
    return launch_fpw<MODE, W, kBf16Act, 1>(a, p, grid, st, name);
}

}  // namespace

// One projection (mode kGateUp or kDown) of the decode kernels: the deep-issue kernel where it
// applies, else the K-streaming kernel, else the split-input matrix-core kernel (bf16), else the
// vector-ALU kernel.
moe_status ffn_gemv_proj(const FfnArgs& a, moe_dtype act, moe_dtype w, int mode, hipStream_t st) {
    moe_status r;
    if (w == MOE_BF16 && act == MOE_BF16) {
        r = ffn_gemv_deep(a, mode, MOE_BF16, st);
        if (r == MOE_EDTYPE) r = ffn_gemv_ks(a, mode, MOE_BF16, st);
        if (r == MOE_EDTYPE) r = ffn_gemv_mfma(a, mode, st);
        if (r == MOE_EDTYPE)
            r = mode == kGateUp ? launch<kGateUp, MOE_BF16, true>(a, st, "ffn_gemv_gateup_bf16")
                                : launch<kDown, MOE_BF16, true>(a, st, "ffn_gemv_down_bf16");
        return r;
    }
    if (w == MOE_INT4_G128 && act == MOE_BF16) {
        r = ffn_gemv_deep(a, mode, MOE_INT4_G128, st);
        if (r == MOE_EDTYPE) r = ffn_gemv_ks(a, mode, MOE_INT4_G128, st);
        if (r == MOE_EDTYPE)
            r = mode == kGateUp ? launch<kGateUp, MOE_INT4_G128, true>(a, st, "ffn_gemv_gateup_int4")
                                : launch<kDown, MOE_INT4_G128, true>(a, st, "ffn_gemv_down_int4");
        return r;
    }
    if (w == MOE_F32 && act == MOE_F32)
        return mode == kGateUp ? launch<kGateUp, MOE_F32, false>(a, st, "ffn_gemv_gateup_f32")
                               : launch<kDown, MOE_F32, false>(a, st, "ffn_gemv_down_f32");
    return set_error(MOE_EDTYPE, "moe_expert_ffn_grouped: unsupported act/weight dtypes (%d,%d)", (int)act, (int)w);
}

moe_status ffn_gemv(const FfnArgs& a, moe_dtype act, moe_dtype w, hipStream_t st) {
    moe_status r = ffn_gemv_proj(a, act, w, kGateUp, st);
    if (r != MOE_OK) return r;
    return ffn_gemv_proj(a, act, w, kDown, st);
}

}  // namespace moe
