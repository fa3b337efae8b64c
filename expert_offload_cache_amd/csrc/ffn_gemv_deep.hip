// Grouped SwiGLU experts for a handful of tokens per call (batch decode), every weight load of a
// wave in flight at once.
//
// Expert weights are reached through the slot table (FreeToken GGUF page, "MoE backends", offload
// backend: GPU expert slots; FreeToken linux guide, memory tier table).  The expert form (SwiGLU,
// no biases) is the plain reading; the pages do not give it.
//
// With at most kDeepTok tokens in the call an expert holds at most that many, so one work item is
// one expert (or the shared expert) and its weights are read exactly once.  The launch is bound by
// how many bytes are in flight: a wave that streams its share of an expert a stage at a time waits
// one memory round trip per stage or two.  Here a wave instead issues all of its loads before it
// multiplies anything:
//   - its input share of the item's activation rows, straight into LDS (direct-to-LDS loads; the
//     S waves that split the inputs take contiguous shares, and the GR row groups of a workgroup
//     share the rows: wave (si, gi) loads the rows gi, gi + GR, ... of share si);
//   - int4: the group scales of its rows for its stages (one 16- or 8-byte load per row block);
//   - its weight fragments, stage by stage (NS stages x RA row blocks, one 16-byte non-temporal
//     load per lane each: 16-32 KB a wave);
// then waits for the activation loads only, meets the workgroup once, and multiplies stage by stage
// as the weight loads land (vector loads return in issue order).  For gate/up with several tokens
// the activation rows' addresses need the permutation entries: those are loaded first, and the
// scales and the first half of the weight stages go out before the activation rows, so the
// weights do not wait for that round trip.  The S partial sums of a row block
// are joined through LDS in share order; SiLU(g)*u (rounded to bf16) or the down output is written
// from registers.
//
// Operands of v_mfma_f32_16x16x32_bf16 as in the K-streaming kernel: bf16 weights are the A operand
// (C: token l%16, rows 4(l/16)..+3); int4 weights are widened to bf16 (128 + u) and are the B
// operand (C: row l%16, tokens 4(l/16)..+3), with a product against an all-ones operand giving the
// sum of the activations for the offset.  Arithmetic: bf16 products, binary32 sums.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "ffn.h"
#include "ffn_common.h"
#include "slot_layout.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;

constexpr int kDeepTok = 8;  // most tokens a call may hold

__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
}

template <int W>
struct DeepFrag;
template <>
struct DeepFrag<MOE_BF16> {
    static constexpr int kIn = 32, kXv = 1;  // inputs per stage; 16-byte activation vectors per lane a stage
};
template <>
struct DeepFrag<MOE_INT4_G128> {
    static constexpr int kIn = 128, kXv = 4;
};

// vmcnt(N) only (expcnt, lgkmcnt left alone)
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int MODE, int W, int RA, int S, int NS, int GR>
__global__ __launch_bounds__(64 * S * GR) void ffn_gemv_deep_kernel(FfnArgs a) {
    static_assert(MODE == kDown || RA % 2 == 0, "gate/up rows come in gate/up pairs");
    constexpr bool kInt4 = (W == MOE_INT4_G128);
    constexpr int KIN = DeepFrag<W>::kIn, XV = DeepFrag<W>::kXv;
    constexpr int NOUT = (MODE == kGateUp ? RA / 2 : RA) * 16;  // output rows of a wave
    constexpr int SHARE = NS * KIN * 2;                          // bytes of one activation row's share
    constexpr int SCV = kInt4 ? (NS % 8 == 0 ? 16 : 8) : 0;      // bytes per scale load
    constexpr int NSC = kInt4 ? NS * 2 / SCV : 0;                // scale loads per row block
    constexpr int NLATER = NSC * RA + NS * RA;                   // loads issued after the activations
    static_assert(!kInt4 || NS % 4 == 0, "int4 scales are loaded 4 or 8 stages at a time");
    static_assert(SHARE % 16 == 0 && NLATER < 64, "load counts");
    extern __shared__ __align__(16) uint8_t smem[];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int si = wv % S, gi = wv / S;
    const int q = lane >> 4, r16 = lane & 15;
    const int K = (MODE == kGateUp) ? a.d : a.f;
    const int nst = K / KIN;  // = S * NS (checked on the host)
    const int ks_base = si * NS;

    int e, chunk, slot, nt, p0;  // nt: 1 .. kDeepTok
    if (!find_item(a, 16, blockIdx.y, e, chunk, slot, nt, p0)) return;
    const bool shared = (e == -1);
    const int orow0 = (blockIdx.x * GR + gi) * NOUT;
    const uint8_t* base;
    if (shared) {
        base = a.shared_w;
    } else {
        if (slot == MOE_SLOT_ELSEWHERE) return;  // rows produced elsewhere: leave them (whole workgroup)
        if (slot < 0 || slot >= a.n_slots) {
            // absent or invalid slot: flag it and give the expert's rows zeros; nothing is read
            if (si == 0) {
                if (lane == 0) *a.status = 1;
                for (int i = lane; i < nt * NOUT; i += 64) {
                    const size_t row = (size_t)(p0 + i / NOUT);
                    const int c = orow0 + i % NOUT;
                    if (MODE == kGateUp) ((uint16_t*)a.h)[row * a.f + c] = 0;
                    else store_y(a, row, c, 0.f);
                }
            }
            return;
        }
        base = a.pool + (size_t)slot * a.stride;
    }

    // Issue order.  Gate/up with several tokens: the permutation entries first, then the group
    // scales and the first half of the weight stages, then the activation rows (their addresses
    // need the entries), then the second half; the multiply starts once the activations (and so
    // the first half) have landed.  Otherwise (one token, or down: no entry to wait for): the
    // activation rows, the scales, then every weight stage.
    const bool split = MODE == kGateUp && a.T > 1;
    const int H = split ? NS / 2 : 0;  // weight stages issued before the activation rows
    int pe = 0;
    if (MODE == kGateUp && split && !shared) pe = a.perm[p0 + min(lane, nt - 1)];
    asm volatile("" ::: "memory");

    const uint8_t* wp[RA];
#pragma unroll
    for (int u = 0; u < RA; ++u) {
        if constexpr (MODE == kGateUp)
            wp[u] = base + gu_block_offset(orow0 / 16 + u / 2, u & 1, a.d, (moe_dtype)W);
        else
            wp[u] = base + down_block_offset(orow0 / 16 + u, a.d, a.f, (moe_dtype)W);
    }
    u32x4_t sc[RA][kInt4 ? NSC : 1];
    auto issue_scales = [&]() __attribute__((always_inline)) {
        if constexpr (kInt4) {
#pragma unroll
            for (int u = 0; u < RA; ++u)
#pragma unroll
                for (int c = 0; c < NSC; ++c) {
                    const uint8_t* p = wp[u] + (size_t)nst * 1024 + ((size_t)r16 * nst + ks_base) * 2 + c * SCV;
                    if constexpr (SCV == 16) {
                        sc[u][c] = *(const u32x4_t*)p;
                    } else {
                        const uint2 v = *(const uint2*)p;
                        sc[u][c] = u32x4_t{v.x, v.y, 0u, 0u};
                    }
                }
        }
    };
    u32x4_t w[NS][RA];
    auto issue_stages = [&](int s0, int s1) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < NS; ++s)
            if (s >= s0 && s < s1)
#pragma unroll
                for (int u = 0; u < RA; ++u)
                    w[s][u] =
                        __builtin_nontemporal_load((const u32x4_t*)(wp[u] + (size_t)(ks_base + s) * 1024 + lane * 16));
        asm volatile("" ::: "memory");
    };
    if (split) {
        issue_scales();
        issue_stages(0, H);
    }

    // ---- activation rows of share si -> LDS [nt][SHARE], contiguous rows -------------------------
    const uint8_t* in_base = (MODE == kGateUp) ? (const uint8_t*)a.x : (const uint8_t*)a.h;
    // share si's region: nt rows, rounded up to whole 1 KB load blocks (the last block's overrun)
    uint8_t* xs = smem + (size_t)si * ((nt * SHARE + 1023) / 1024 * 1024);
    {
        // lane i: token row i (clamped) of the item, as a source row index
        const int i = min(lane, nt - 1);
        int src_row;
        if (MODE == kGateUp) src_row = shared ? i : (split ? pe / a.k : 0);
        else src_row = p0 + i;
        const int nvec = nt * (SHARE / 16);  // 16-byte vectors of the share
        // wave gi takes the 64-vector blocks gi, gi + GR, ... (each lands contiguously in LDS)
        for (int b = gi; b * 64 < nvec; b += GR) {
            const int v = min(b * 64 + lane, nvec - 1);  // past the end: reload the last vector (never read)
            const int r = v / (SHARE / 16), c = v - r * (SHARE / 16);
            const int gr = __shfl(src_row, r, 64);
            const uint8_t* src = in_base + (size_t)gr * K * 2 + (size_t)ks_base * KIN * 2 + (size_t)c * 16;
            __builtin_amdgcn_global_load_lds((gbl_ptr_t)src, (lds_ptr_t)(xs + b * 1024), 16, 0, 0);
        }
    }
    asm volatile("" ::: "memory");
    if (!split) issue_scales();
    issue_stages(H, NS);
    // the activation loads (issued before the scales or the remaining weight stages) have landed,
    // in every wave
    if (split) wait_vm<(NS - NS / 2) * RA>();
    else wait_vm<NLATER>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    // ---- multiply, stage by stage as the weights land ------------------------------------------
    const uint8_t* xrow = xs + (size_t)min(r16, nt - 1) * SHARE + q * 16;  // this lane's token row
    f32x4_t acc[RA];
#pragma unroll
    for (int u = 0; u < RA; ++u) acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const u32x4_t ones = {kOnes, kOnes, kOnes, kOnes};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        u32x4_t xv[XV];
#pragma unroll
        for (int v = 0; v < XV; ++v) xv[v] = *(const u32x4_t*)(xrow + s * (XV * 64) + v * 64);
        if constexpr (!kInt4) {
#pragma unroll
            for (int u = 0; u < RA; ++u) acc[u] = mfma16(w[s][u], xv[0], acc[u]);
        } else {
            f32x4_t px = {0.f, 0.f, 0.f, 0.f}, pm[RA];
#pragma unroll
            for (int u = 0; u < RA; ++u) pm[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 4; ++st) {
#pragma unroll
                for (int u = 0; u < RA; ++u) {
                    const uint32_t wd = st == 0 ? w[s][u].x : st == 1 ? w[s][u].y : st == 2 ? w[s][u].z : w[s][u].w;
                    uint32_t wb[4];
                    int4_word_to_bf16(wd, wb);
                    const u32x4_t bw = {wb[0], wb[1], wb[2], wb[3]};
                    pm[u] = mfma16(xv[st], bw, pm[u]);
                }
                px = mfma16(xv[st], ones, px);
            }
            // group scale of this lane's row at stage s: element s of the preloaded scales
            constexpr int SPL = SCV / 2;  // scales per load
#pragma unroll
            for (int u = 0; u < RA; ++u) {
                const u32x4_t sv = sc[u][s / SPL];
                const int el = s % SPL;
                const uint32_t word = (el / 2) == 0 ? sv.x : (el / 2) == 1 ? sv.y : (el / 2) == 2 ? sv.z : sv.w;
                const float scl = as_f32((el & 1) ? (word & 0xFFFF0000u) : (word << 16));
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[u][i] = __builtin_fmaf(scl, __builtin_fmaf(-136.0f, px[i], pm[u][i]), acc[u][i]);
            }
        }
    }

    // ---- join the S input shares in share order -------------------------------------------------
    if constexpr (S > 1) {
        __syncthreads();  // every wave is done with its activation rows (the join reuses the LDS)
        f32x4_t* red = (f32x4_t*)smem;
#pragma unroll
        for (int u = 0; u < RA; ++u) red[(wv * RA + u) * 64 + lane] = acc[u];
        __syncthreads();
        if (si != 0) return;
#pragma unroll
        for (int w2 = 1; w2 < S; ++w2)
#pragma unroll
            for (int u = 0; u < RA; ++u) acc[u] += red[((wv + w2) * RA + u) * 64 + lane];
    }

    // ---- outputs from the accumulators ---------------------------------------------------------
    with_y_type<MODE>(a, [&](auto yt) __attribute__((always_inline)) {
        constexpr bool YB = decltype(yt)::value;
        if constexpr (!kInt4) {
            // lane l: token l%16, rows 4(l/16) .. +3 of each row block
            const int tok = r16;
            if (tok < nt) {
                const size_t row = (size_t)(p0 + tok);
                if constexpr (MODE == kGateUp) {
#pragma unroll
                    for (int p = 0; p < RA / 2; ++p) {
                        const f32x4_t g = acc[2 * p], u = acc[2 * p + 1];
                        uint2 o;
                        o.x = (uint32_t)f32_to_bf16(silu_mul(g[0], u[0])) | ((uint32_t)f32_to_bf16(silu_mul(g[1], u[1])) << 16);
                        o.y = (uint32_t)f32_to_bf16(silu_mul(g[2], u[2])) | ((uint32_t)f32_to_bf16(silu_mul(g[3], u[3])) << 16);
                        *(uint2*)((uint16_t*)a.h + row * a.f + orow0 + p * 16 + q * 4) = o;
                    }
                } else {
#pragma unroll
                    for (int u = 0; u < RA; ++u)
                        store_y4_as<YB>(a, row, orow0 + u * 16 + q * 4, acc[u][0], acc[u][1], acc[u][2], acc[u][3]);
                }
            }
        } else {
            // lane l: row l%16 of each row block, tokens 4(l/16) .. +3
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = 4 * q + i;
                if (tok >= nt) continue;
                const size_t row = (size_t)(p0 + tok);
                if constexpr (MODE == kGateUp) {
#pragma unroll
                    for (int p = 0; p < RA / 2; ++p)
                        ((uint16_t*)a.h)[row * a.f + orow0 + p * 16 + r16] =
                            f32_to_bf16(silu_mul(acc[2 * p][i], acc[2 * p + 1][i]));
                } else {
#pragma unroll
                    for (int u = 0; u < RA; ++u) store_y_as<YB>(a, row, orow0 + u * 16 + r16, acc[u][i]);
                }
            }
        }
    });
}

// One launch shape: RA row blocks a wave, inputs split over S waves of NS stages each, GR row
// groups a workgroup.  A shape that does not fit returns MOE_EDTYPE with nothing launched.
template <int MODE, int W, int RA, int S, int NS, int GR>
moe_status launch_deep(const FfnArgs& a, hipStream_t st, const char* name) {
    constexpr int KIN = DeepFrag<W>::kIn;
    const int M = (MODE == kGateUp) ? a.f : a.d;
    const int K = (MODE == kGateUp) ? a.d : a.f;
    const int per_wave = (MODE == kGateUp) ? RA / 2 : RA;
    if (a.T > kDeepTok || K % KIN != 0 || K / KIN != S * NS || (M / 16) % (per_wave * GR) != 0) return MOE_EDTYPE;
    const int64_t items = work_items(a, 16);
    const size_t xbytes = (size_t)S * (((size_t)std::min(a.T, kDeepTok) * NS * KIN * 2 + 1023) / 1024 * 1024);
    const size_t jbytes = S > 1 ? (size_t)S * GR * RA * 1024 : 0;
    const size_t lds = std::max(xbytes, jbytes);
    if (lds > 160 * 1024) return MOE_EDTYPE;
    auto kern = ffn_gemv_deep_kernel<MODE, W, RA, S, NS, GR>;
    if (lds > 64 * 1024)
        MOE_HIP(hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
    dim3 grid((unsigned)(M / 16 / (per_wave * GR)), (unsigned)items), block(64 * S * GR);
    ProfScope ps(name, st);
    kern<<<grid, block, lds, st>>>(a);
    return check_launch(name);
}

}  // namespace

#ifndef MOE_DEEP_GU4_SMALL
#define MOE_DEEP_GU4_SMALL 2, 4, 8, 1
#endif
#ifndef MOE_DEEP_GU4
#define MOE_DEEP_GU4 2, 2, 16, 2
#endif
#ifndef MOE_DEEP_DN4
#define MOE_DEEP_DN4 4, 4, 4, 1
#endif

// int4 weights, at most kDeepTok tokens (MOE_EDTYPE otherwise, or where the plan does not divide the
// shapes).  Plans by measurement on MI355X over the DeepSeek-V4-Flash shaped int4 layer (d 4096,
// d_ff 2048) at 1, 2 and 8 tokens, against the K-streaming kernel's 21.3 / 28.4 / 65.5 us (gate/up)
// and 14.5 / 18.3 / 33.8 us (down), per-launch HIP events:
//   gate/up: one gate/up pair a wave, four waves splitting the inputs (8 stages, 16 KB a wave) up to
//     2 tokens (19.2 / 26.9 us); above, two waves splitting them (16 stages, 32 KB a wave) in
//     workgroups of two row groups (53.8 us at 8 tokens);
//   down: four row blocks a wave, four waves splitting the inputs (4 stages, 16 KB a wave):
//     12.9 / 16.2 / 28.9 us.
// bf16 weights stay on the K-streaming kernel: this one measured within 1 us of it at 1 token and
// slower at 4 and 8.
moe_status ffn_gemv_deep(const FfnArgs& a, int mode, moe_dtype w, hipStream_t st) {
    if (w != MOE_INT4_G128 || a.T > kDeepTok) return MOE_EDTYPE;
    if (mode == kGateUp) {
        if (a.T <= 2) return launch_deep<kGateUp, MOE_INT4_G128, MOE_DEEP_GU4_SMALL>(a, st, "ffn_gemv_gateup_int4");
        return launch_deep<kGateUp, MOE_INT4_G128, MOE_DEEP_GU4>(a, st, "ffn_gemv_gateup_int4");
    }
    return launch_deep<kDown, MOE_INT4_G128, MOE_DEEP_DN4>(a, st, "ffn_gemv_down_int4");
}

}  // namespace moe
