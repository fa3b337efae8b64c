// Grouped SwiGLU experts for few tokens per expert (decode), bf16 weights and activations, on
// the matrix cores.
//
// Expert weights are reached through the slot table (FreeToken GGUF page, "MoE backends",
// offload backend: GPU expert slots; FreeToken linux guide, memory tier table).  The expert
// form (SwiGLU, no biases) is the plain reading; the pages do not give it.
//
// Work decomposition (weights stationary):
//   * a workgroup owns one 16-row block of one expert -- the gate and up blocks of the same 16
//     outputs, or RB blocks of W_d -- and its waves split the inputs K;
//   * the slot layout stores a block as fragments of 16 rows x 32 inputs in the lane order of the
//     A operand of v_mfma_f32_16x16x32_bf16 (lane l: row l%16, inputs 8(l/16)..+7), so a wave
//     loads its fragments with one 16-byte load per lane each and feeds them to the MFMA as is;
//   * the tokens are the N dimension: lane l loads token l%16's inputs 8(l/16)..+7 of each of its
//     fragments straight from the activation row (or h row) in global memory -- a B operand --
//     with no staging in LDS;
//   * a workgroup takes up to G groups of 16 tokens one after another with its weights held in
//     registers, so at decode batch sizes the gate/up weights of an expert are read once per row
//     block (workgroups that split one expert's tokens would each read them);
//   * the C tile (lane l: token l%16, rows 4(l/16)..+3) of every wave goes to LDS, and the waves
//     of a row block are summed there in wave order, then SiLU(g)*u (bf16) or the down output.
//
// Arithmetic: bf16 products, binary32 accumulation inside the MFMA and across fragments and
// waves; h is rounded to bf16 like the other paths.
#include <hip/hip_runtime.h>

#include "ffn.h"
#include "ffn_common.h"
#include "slot_layout.h"

#include <algorithm>

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
}

// Largest workgroup of a launch shape: 8 waves for gate/up (two matrices a wave), 16 for down.
constexpr int mfma_max_threads(int mode) { return mode == kDown ? 1024 : 512; }

// LDS: two buffers of [waves][NM][64 lanes x 4] partial sums (one when G == 1).
template <int MODE, int FPW, int G, int RB>
__global__ __launch_bounds__(mfma_max_threads(MODE)) void ffn_gemv_mfma_kernel(FfnArgs a) {
    constexpr int NM = (MODE == kGateUp) ? 2 : 1;
    constexpr int NTG = 16 * G;
    extern __shared__ __align__(16) uint8_t smem[];
    float* s_red = (float*)smem;

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int KS = blockDim.x >> 6;  // waves in the workgroup
    const int KSW = KS / RB;         // waves per row block
    const int q = lane >> 4, r16 = lane & 15;
    const int rbi = wv / KSW;
    const int rb = blockIdx.x * RB + rbi;
    const int K = (MODE == kGateUp) ? a.d : a.f;
    const int nfrag = K / 32;

    int e, chunk;
    if (!find_work(a.counts, a.E, a.T, NTG, a.shared_w != nullptr, blockIdx.y, e, chunk, a.n_lo, a.n_hi)) return;
    const bool shared = (e == -1);
    const int n_all = __builtin_amdgcn_readfirstlane(shared ? a.T : a.counts[e]);
    const int i0 = chunk * NTG;  // this workgroup's tokens: i0 .. i0 + nt - 1
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
                if (MODE == kGateUp) ((uint16_t*)a.h)[row * a.f + c] = 0;
                else store_y(a, row, c, 0.f);
            }
            return;
        }
        base = a.pool + (size_t)slot * a.stride;
    }

    // this lane's source row in token group g (token 16 g + l%16, clamped to the chunk; the
    // clamped columns of the product are computed and dropped), at input quarter l/16
    const uint8_t* in_base = (MODE == kGateUp) ? (const uint8_t*)a.x : (const uint8_t*)a.h;
    const size_t row_bytes = (size_t)K * 2;
    auto xrow = [&](int g) {
        const int i = min(16 * g + r16, nt - 1);
        const int row = (MODE == kGateUp) ? (shared ? (i0 + i) : (a.perm[p0 + i0 + i] / a.k)) : (p0 + i0 + i);
        return in_base + (size_t)row * row_bytes + q * 16;
    };

    const int per = (nfrag + KSW - 1) / KSW;
    const int f0 = __builtin_amdgcn_readfirstlane((wv - rbi * KSW) * per);
    const int nmine = __builtin_amdgcn_readfirstlane(max(0, min(per, nfrag - f0)));
    const uint8_t* mats[NM];
    if constexpr (MODE == kGateUp) {
        mats[0] = base + gu_block_offset(rb, 0, a.d, MOE_BF16);
        mats[NM - 1] = base + gu_block_offset(rb, 1, a.d, MOE_BF16);
    } else {
        mats[0] = base + down_block_offset(rb, a.d, a.f, MOE_BF16);
    }
    // clamped fragment index: the loads of a short share stay inside the block
    auto frag = [&](int c) { return min(f0 + min(c, max(nmine - 1, 0)), nfrag - 1); };

    // group 0's activations first (loads complete in issue order), then every weight fragment
    u32x4_t xb[FPW], wreg[FPW][NM];
    {
        const uint8_t* xr = xrow(0);
#pragma unroll
        for (int c = 0; c < FPW; ++c) xb[c] = *(const u32x4_t*)(xr + (size_t)frag(c) * 64);
    }
#pragma unroll
    for (int c = 0; c < FPW; ++c)
#pragma unroll
        for (int m = 0; m < NM; ++m)
            wreg[c][m] = __builtin_nontemporal_load((const u32x4_t*)(mats[m] + (size_t)frag(c) * 1024 + lane * 16));

    const int ngroups = (G == 1) ? 1 : (nt + 15) >> 4;
    const size_t buf = (size_t)KS * NM * 256;
    auto group = [&](int g) {
        f32x4_t acc[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < FPW; ++c)
            if (c < nmine)
#pragma unroll
                for (int m = 0; m < NM; ++m) acc[m] = mfma_bf16(wreg[c][m], xb[c], acc[m]);
        float* red = s_red + (g & 1) * buf;
#pragma unroll
        for (int m = 0; m < NM; ++m) *(f32x4_t*)(red + ((size_t)wv * NM + m) * 256 + lane * 4) = acc[m];
        if (g + 1 < ngroups) {
            // the next group's activations load during the join below
            const uint8_t* xr = xrow(g + 1);
#pragma unroll
            for (int c = 0; c < FPW; ++c) xb[c] = *(const u32x4_t*)(xr + (size_t)frag(c) * 64);
        }
        __syncthreads();
        // C element (row r, token column c) of a wave sits at lane 16 (r / 4) + c, component r % 4
        const int ng = min(16, nt - 16 * g);
        for (int idx = threadIdx.x; idx < RB * ng * 16; idx += blockDim.x) {
            const int bi = idx / (ng * 16), rem = idx - bi * ng * 16;
            const int c = rem >> 4, r = rem & 15;
            const int off = (16 * (r >> 2) + c) * 4 + (r & 3);
            float v[NM];
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                float s = 0.f;
                for (int w2 = bi * KSW; w2 < (bi + 1) * KSW; ++w2) s += red[((size_t)w2 * NM + m) * 256 + off];
                v[m] = s;
            }
            const size_t row = (size_t)(p0 + i0 + 16 * g + c);
            const int col = (blockIdx.x * RB + bi) * 16 + r;
            if constexpr (MODE == kGateUp) {
                ((uint16_t*)a.h)[row * a.f + col] = f32_to_bf16(silu_mul(v[0], v[NM - 1]));
            } else {
                store_y(a, row, col, v[0]);
            }
        }
    };
    group(0);  // straight-line, so its products start as the loads land
    for (int g = 1; g < ngroups; ++g) group(g);
}

struct MPlan {
    int fpw, ksw, rb, g;
    size_t lds;
};

// Shape of one launch.  Fragments per wave: 4 or 8, the fewest with at most 8 waves (gate/up) or
// 16 waves (down) per workgroup; the down projection groups up to 4 row blocks per workgroup
// (its blocks hold only f inputs).  Token groups per workgroup: gate/up takes up to 4 (64 tokens)
// so its weights are read once per expert at decode sizes; down takes one (16 tokens), which
// keeps it at two workgroups per compute unit (measured faster than fewer weight reads).
MPlan mplan_for(int MODE, int M, int K, int T) {
    const int nfrag = K / 32;
    const int nm = MODE == kGateUp ? 2 : 1;
    int g = 1;
    if (MODE == kGateUp)
        while (g < 4 && 16 * g < T) g <<= 1;
    MPlan p{0, 0, 1, g, 0};
    const int max_waves = mfma_max_threads(MODE) / 64;
    const int rbs[] = {4, 2, 1};
    const int fpws[] = {4, 8};
    for (int rb : rbs) {
        if (rb > 1 && (MODE != kDown || (M / 16) % rb != 0 || nfrag * rb > 128)) continue;
        for (int fpw : fpws) {
            const int ksw = (nfrag + fpw - 1) / fpw;
            if (rb * ksw <= max_waves) {
                p = MPlan{fpw, ksw, rb, g, 0};
                break;
            }
        }
        if (p.fpw) break;
    }
    p.lds = (size_t)p.ksw * p.rb * (g > 1 ? 2 : 1) * nm * 1024;
    return p;
}

template <int MODE, int FPW, int RB>
moe_status launch_g(const FfnArgs& a, const MPlan& p, dim3 grid, hipStream_t st, const char* name) {
    dim3 block(64 * p.ksw * RB);
    ProfScope ps(name, st);
    if constexpr (MODE == kGateUp) {
        switch (p.g) {
            case 1: ffn_gemv_mfma_kernel<MODE, FPW, 1, RB><<<grid, block, p.lds, st>>>(a); break;
            case 2: ffn_gemv_mfma_kernel<MODE, FPW, 2, RB><<<grid, block, p.lds, st>>>(a); break;
            default: ffn_gemv_mfma_kernel<MODE, FPW, 4, RB><<<grid, block, p.lds, st>>>(a); break;
        }
    } else {
        ffn_gemv_mfma_kernel<MODE, FPW, 1, RB><<<grid, block, p.lds, st>>>(a);
    }
    return check_launch(name);
}

template <int MODE, int RB>
moe_status launch_fpw(const FfnArgs& a, const MPlan& p, dim3 grid, hipStream_t st, const char* name) {
    if (p.fpw == 4) return launch_g<MODE, 4, RB>(a, p, grid, st, name);
    return launch_g<MODE, 8, RB>(a, p, grid, st, name);
}

template <int MODE>
moe_status launch(const FfnArgs& a, hipStream_t st, const char* name) {
    const int K = (MODE == kGateUp) ? a.d : a.f;
    const int M = (MODE == kGateUp) ? a.f : a.d;  // output rows (gate/up: pairs of rows)
    const MPlan p = mplan_for(MODE, M, K, a.T);
    if (!p.fpw) return set_error(MOE_ESHAPE, "%s: K=%d too large for this kernel", name, K);
    // work items: sum over experts of ceil(n_e / ntg) <= T*k/ntg + min(E, T*k), plus the shared chunks
    const int ntg = 16 * p.g;
    const int64_t items = work_items(a, ntg);
    if (items > 65535) return set_error(MOE_ESHAPE, "%s: %lld work items exceed one launch", name, (long long)items);
    dim3 grid((unsigned)(M / 16 / p.rb), (unsigned)items);
    if constexpr (MODE == kDown) {
        if (p.rb == 4) return launch_fpw<MODE, 4>(a, p, grid, st, name);
        if (p.rb == 2) return launch_fpw<MODE, 2>(a, p, grid, st, name);
    }
    return launch_fpw<MODE, 1>(a, p, grid, st, name);
}

}  // namespace

moe_status ffn_gemv_mfma(const FfnArgs& a, int mode, hipStream_t st) {
    // shapes beyond 8 fragments a wave (gate/up K > 2048 inputs, down K > 4096) are not covered
    if (mode == kGateUp) {
        if (!mplan_for(kGateUp, a.f, a.d, a.T).fpw) return MOE_EDTYPE;
        return launch<kGateUp>(a, st, "ffn_gemv_gateup_bf16");
    }
    if (!mplan_for(kDown, a.d, a.f, a.T).fpw) return MOE_EDTYPE;
    return launch<kDown>(a, st, "ffn_gemv_down_bf16");
}

}  // namespace moe
