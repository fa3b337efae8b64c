// Grouped SwiGLU experts for few tokens per expert (decode), K-streaming on the matrix cores.
//
// Expert weights are reached through the slot table (FreeToken GGUF page, "MoE backends",
// offload backend: GPU expert slots; FreeToken linux guide, memory tier table).  The expert
// form (SwiGLU, no biases) is the plain reading; the pages do not give it.
//
// Work decomposition (weights streamed through each wave; at most one join per workgroup):
//   * a wave owns RA row blocks (16 rows each) of one expert -- in the gate/up launch RA/2 pairs
//     of a gate block and the up block of the same 16 outputs -- for all tokens of its chunk (up
//     to G groups of 16), over the whole input range K or, when S waves split it, a 1/S share
//     (contiguous, or interleaved: wave s takes the stages s, s+S, ...);
//   * its inputs are streamed in stages of one slot fragment (32 inputs bf16, 128 int4): stage
//     ks + R - 1's weight fragments (one 16-byte load per lane and row block) and activation
//     slices (the same inputs of each token) are issued together while stage ks is multiplied,
//     so the loads of a wave complete in the order they are used and each wave keeps R - 1
//     stages in flight from start to end;
//   * the partial sums never leave the wave: SiLU(g)*u (bf16) or the down output is formed in
//     registers and stored directly.  LDS is used only where the inputs are split over S waves
//     (one join at the end) and by the staged-rows variant (XL): items of at most 4 tokens copy
//     their activation rows to LDS once, so only weight loads go through the in-order load
//     queue.
// The waves of a workgroup take consecutive row-block ranges of the same (expert, chunk) item.
//
// Operands of v_mfma_f32_16x16x32_bf16 (lane l: row or token l%16, inputs 8(l/16)..+7 of the 32):
//   bf16 weights are the A operand, so C holds token l%16, rows 4(l/16)..+3 in lane l;
//   int4 weights are the B operand (after widening), so C holds row l%16, tokens 4(l/16)..+3 and
//   each lane applies its own row's group scale.  An int4 nibble u becomes the bf16 value
//   128 + u with one AND-OR per pair; a second product against an all-ones operand gives sum x
//   over the same 128 inputs, and acc += s * (sum (136 + q) x - 136 sum x) = sum (q s) x.
// Arithmetic: bf16 products, binary32 sums; h is rounded to bf16 like the other paths.
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

constexpr int kKsWaves = 4;  // waves per workgroup

template <int W>
struct KsFrag;
template <>
struct KsFrag<MOE_BF16> {
    static constexpr int kIn = 32, kXv = 1;  // inputs per stage; 16-byte activation vectors per token block
};
template <>
struct KsFrag<MOE_INT4_G128> {
    static constexpr int kIn = 128, kXv = 4;
};

constexpr int kXlTok = 4;  // most tokens an item may hold when its activation rows are staged in LDS

template <int MODE, int W, int RA, int G, int R, int S, bool XL, bool IL, bool CW>
__global__ __launch_bounds__(64 * kKsWaves) void ffn_gemv_ks_kernel(FfnArgs a) {
    static_assert(MODE == kDown || RA % 2 == 0, "gate/up rows come in gate/up pairs");
    static_assert(kKsWaves % S == 0, "input split");
    static_assert(!XL || G == 1, "staged activation rows: one token group");
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int XV = KsFrag<W>::kXv;
    constexpr int NTG = 16 * G;
    constexpr bool kInt4 = (W == MOE_INT4_G128);
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int q = lane >> 4, r16 = lane & 15;
    const int K = (MODE == kGateUp) ? a.d : a.f;
    const int nst = K / KsFrag<W>::kIn;  // stages of the whole input range
    // CW: weight loads through the cache instead of non-temporal (see launch_ks's caller)
    constexpr bool kCachedW = CW;
    const int nsw = nst / S;             // stages of this wave's share
    const int si = wv % S;               // this wave's share of the inputs
    // share si: stages si*nsw .. +nsw-1, or with IL the stages si, si+S, si+2S, ... (the S waves of
    // a row-block group then read adjacent 1 KB fragments at the same time)
    const int ks_base = IL ? si : si * nsw;
    constexpr int kStep = IL ? S : 1;

    int e, chunk, slot, n_all, p0;
    if (!find_item(a, NTG, blockIdx.y, e, chunk, slot, n_all, p0)) return;
    const bool shared = (e == -1);
    const int i0 = chunk * NTG;  // this item's tokens: i0 .. i0 + nt - 1
    const int nt = __builtin_amdgcn_readfirstlane(min(NTG, n_all - i0));
    // first output row (16 per row block, or per gate/up pair) of this wave
    const int orow0 = (blockIdx.x * (kKsWaves / S) + wv / S) * (MODE == kGateUp ? RA / 2 : RA) * 16;
    constexpr int NOUT = (MODE == kGateUp ? RA / 2 : RA) * 16;
    const uint8_t* base;
    if (shared) {
        base = a.shared_w;
    } else {
        if (slot == MOE_SLOT_ELSEWHERE) return;  // rows produced elsewhere: leave them
        if (slot < 0 || slot >= a.n_slots) {
            // absent or invalid slot: flag it and give the expert's rows zeros; nothing is read
            if (lane == 0) *a.status = 1;
            for (int i = lane; i < nt * NOUT; i += 64) {
                const size_t row = (size_t)(p0 + i0 + i / NOUT);
                const int c = orow0 + i % NOUT;
                if (MODE == kGateUp) ((uint16_t*)a.h)[row * a.f + c] = 0;
                else store_y(a, row, c, 0.f);
            }
            return;
        }
        base = a.pool + (size_t)slot * a.stride;
    }

    const uint8_t* wp[RA];
#pragma unroll
    for (int u = 0; u < RA; ++u) {
        if constexpr (MODE == kGateUp)
            wp[u] = base + gu_block_offset(orow0 / 16 + u / 2, u & 1, a.d, (moe_dtype)W);
        else
            wp[u] = base + down_block_offset(orow0 / 16 + u, a.d, a.f, (moe_dtype)W);
    }
    // token group j: this lane's token 16 j + l%16 (clamped to the chunk; the clamped columns
    // are computed and dropped), input quarter l/16
    const uint8_t* in_base = (MODE == kGateUp) ? (const uint8_t*)a.x : (const uint8_t*)a.h;
    // gate/up: the token groups' permutation entries, loaded together and used only after the
    // first stages' weight loads are issued below (the shared expert loads entries it ignores)
    int pe[G];
    if constexpr (MODE == kGateUp && !XL) {
        const int32_t* pb = a.perm + (shared ? 0 : p0 + i0);
#pragma unroll
        for (int j = 0; j < G; ++j) pe[j] = pb[min(16 * j + r16, nt - 1)];
        asm volatile("" ::: "memory");  // keep these loads ahead of the weight loads
    }
    const uint8_t* xp[G];
    auto set_rows = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const int i = min(16 * j + r16, nt - 1);
            int row;
            if constexpr (MODE == kGateUp && !XL) row = shared ? (i0 + i) : pe[j] / a.k;
            else row = (MODE == kGateUp) ? (shared ? (i0 + i) : (a.perm[p0 + i0 + i] / a.k)) : (p0 + i0 + i);
            xp[j] = in_base + (size_t)row * K * 2 + q * 16;
        }
    };
    if constexpr (XL) set_rows();

    // XL: the item's activation rows (at most kXlTok) are staged in LDS once, so only weight
    // loads go through the in-order load queue and the stages read their activations from LDS
    if constexpr (XL) {
        const int vpr = K * 2 / 16;  // 16-byte vectors a row
        const int total = nt * vpr;
        for (int v0 = 0; v0 < total; v0 += 8 * 64 * kKsWaves) {
            u32x4_t t[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int v = min(v0 + u * 64 * kKsWaves + (int)threadIdx.x, total - 1);
                const int i = v / vpr;
                const int row = (MODE == kGateUp) ? (shared ? (i0 + i) : (a.perm[p0 + i0 + i] / a.k)) : (p0 + i0 + i);
                t[u] = *(const u32x4_t*)(in_base + (size_t)row * K * 2 + (size_t)(v - i * vpr) * 16);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int v = v0 + u * 64 * kKsWaves + (int)threadIdx.x;
                if (v < total) ((u32x4_t*)smem)[v] = t[u];
            }
        }
        __syncthreads();
    }
    const uint8_t* s_xrow = smem + (size_t)min(r16, nt - 1) * K * 2 + q * 16;  // XL: this lane's row

    u32x4_t wst[R][RA], xst[R][G][XV];
    uint32_t sst[R][kInt4 ? RA : 1];
    // local stage ks into register set (w, x, s); past the end of the share its last stage is
    // repeated (never used)
    auto issue_x = [&](int ks, u32x4_t (&x)[G][XV]) __attribute__((always_inline)) {
        ks = ks_base + kStep * min(ks, nsw - 1);
#pragma unroll
        for (int j = 0; j < G; ++j)
            if (!XL && (j == 0 || 16 * j < nt))  // token groups the item does not fill are not loaded
#pragma unroll
                for (int v = 0; v < XV; ++v) x[j][v] = *(const u32x4_t*)(xp[j] + (size_t)ks * (XV * 64) + v * 64);
    };
    auto issue_w = [&](int ks, u32x4_t (&w)[RA], uint32_t (&s)[kInt4 ? RA : 1]) __attribute__((always_inline)) {
        ks = ks_base + kStep * min(ks, nsw - 1);
        if constexpr (kInt4) {
#pragma unroll
            for (int u = 0; u < RA; ++u)
                s[u] = *(const uint16_t*)(wp[u] + (size_t)nst * 1024 + ((size_t)r16 * nst + ks) * 2);
        }
#pragma unroll
        for (int u = 0; u < RA; ++u) {
            const u32x4_t* src = (const u32x4_t*)(wp[u] + (size_t)ks * 1024 + lane * 16);
            if constexpr (kCachedW) w[u] = *src;
            else w[u] = __builtin_nontemporal_load(src);
        }
    };
    auto issue = [&](int ks, u32x4_t (&w)[RA], u32x4_t (&x)[G][XV], uint32_t (&s)[kInt4 ? RA : 1])
        __attribute__((always_inline)) {
        issue_x(ks, x);
        issue_w(ks, w, s);
    };

    f32x4_t acc[RA][G];
#pragma unroll
    for (int u = 0; u < RA; ++u)
#pragma unroll
        for (int j = 0; j < G; ++j) acc[u][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const u32x4_t ones = {kOnes, kOnes, kOnes, kOnes};

    auto compute = [&](int ks, const u32x4_t (&w)[RA], u32x4_t (&x)[G][XV], const uint32_t (&s)[kInt4 ? RA : 1])
        __attribute__((always_inline)) {
        if constexpr (XL) {
#pragma unroll
            for (int v = 0; v < XV; ++v)
                x[0][v] = *(const u32x4_t*)(s_xrow + (size_t)(ks_base + kStep * ks) * (XV * 64) + v * 64);
        }
        if constexpr (!kInt4) {
#pragma unroll
            for (int j = 0; j < G; ++j)
                if (j == 0 || 16 * j < nt)
#pragma unroll
                    for (int u = 0; u < RA; ++u) acc[u][j] = mfma_bf16(w[u], x[j][0], acc[u][j]);
        } else {
            f32x4_t px[G], pm[RA][G];
#pragma unroll
            for (int j = 0; j < G; ++j) {
                px[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int u = 0; u < RA; ++u) pm[u][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int st = 0; st < 4; ++st) {
#pragma unroll
                for (int u = 0; u < RA; ++u) {
                    const uint32_t wd = st == 0 ? w[u].x : st == 1 ? w[u].y : st == 2 ? w[u].z : w[u].w;
                    uint32_t wb[4];
                    int4_word_to_bf16(wd, wb);
                    const u32x4_t bw = {wb[0], wb[1], wb[2], wb[3]};
#pragma unroll
                    for (int j = 0; j < G; ++j)
                        if (j == 0 || 16 * j < nt) pm[u][j] = mfma_bf16(x[j][st], bw, pm[u][j]);
                }
#pragma unroll
                for (int j = 0; j < G; ++j)
                    if (j == 0 || 16 * j < nt) px[j] = mfma_bf16(x[j][st], ones, px[j]);
            }
#pragma unroll
            for (int u = 0; u < RA; ++u) {
                const float sc = as_f32(s[u] << 16);
#pragma unroll
                for (int j = 0; j < G; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[u][j][i] = __builtin_fmaf(sc, __builtin_fmaf(-136.0f, px[j][i], pm[u][j][i]), acc[u][j][i]);
            }
        }
    };

    // the first stages' weights go out before the activation rows' addresses are known
#pragma unroll
    for (int s = 0; s < R - 1; ++s) issue_w(s, wst[s], sst[s]);
    if constexpr (!XL) set_rows();
#pragma unroll
    for (int s = 0; s < R - 1; ++s) issue_x(s, xst[s]);
    for (int ks0 = 0; ks0 < nsw; ks0 += R) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            issue(ks0 + r + R - 1, wst[(r + R - 1) % R], xst[(r + R - 1) % R], sst[(r + R - 1) % R]);
            if (ks0 + r < nsw) compute(ks0 + r, wst[r], xst[r], sst[r]);
        }
    }
    if constexpr (S > 1) {
        // join the S shares in LDS in share order; the first wave of each group stores
        uint8_t* jb = smem + (XL ? (size_t)min(a.T, kXlTok) * K * 2 : 0);
        f32x4_t* red = (f32x4_t*)jb + (size_t)wv * RA * G * 64;
#pragma unroll
        for (int u = 0; u < RA; ++u)
#pragma unroll
            for (int j = 0; j < G; ++j) red[(u * G + j) * 64 + lane] = acc[u][j];
        __syncthreads();
        if (si != 0) return;
#pragma unroll
        for (int w2 = 1; w2 < S; ++w2) {
            const f32x4_t* o = (const f32x4_t*)jb + (size_t)(wv + w2) * RA * G * 64;
#pragma unroll
            for (int u = 0; u < RA; ++u)
#pragma unroll
                for (int j = 0; j < G; ++j) acc[u][j] += o[(u * G + j) * 64 + lane];
        }
    }

    // ---- outputs straight from the accumulators ------------------------------------------------
    with_y_type<MODE>(a, [&](auto yt) __attribute__((always_inline)) {
        constexpr bool YB = decltype(yt)::value;
        if constexpr (!kInt4) {
            // lane l: token 16 j + l%16, rows 4(l/16) .. +3 of each row block
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const int tok = 16 * j + r16;
                if (tok >= nt) continue;
                const size_t row = (size_t)(p0 + i0 + tok);
                if constexpr (MODE == kGateUp) {
#pragma unroll
                    for (int p = 0; p < RA / 2; ++p) {
                        const f32x4_t g = acc[2 * p][j], u = acc[2 * p + 1][j];
                        uint2 o;
                        o.x = (uint32_t)f32_to_bf16(silu_mul(g[0], u[0])) | ((uint32_t)f32_to_bf16(silu_mul(g[1], u[1])) << 16);
                        o.y = (uint32_t)f32_to_bf16(silu_mul(g[2], u[2])) | ((uint32_t)f32_to_bf16(silu_mul(g[3], u[3])) << 16);
                        *(uint2*)((uint16_t*)a.h + row * a.f + orow0 + p * 16 + q * 4) = o;
                    }
                } else {
#pragma unroll
                    for (int u = 0; u < RA; ++u)
                        store_y4_as<YB>(a, row, orow0 + u * 16 + q * 4, acc[u][j][0], acc[u][j][1], acc[u][j][2], acc[u][j][3]);
                }
            }
        } else {
            // lane l: row l%16 of each row block, tokens 16 j + 4(l/16) .. +3
#pragma unroll
            for (int j = 0; j < G; ++j) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tok = 16 * j + 4 * q + i;
                    if (tok >= nt) continue;
                    const size_t row = (size_t)(p0 + i0 + tok);
                    if constexpr (MODE == kGateUp) {
#pragma unroll
                        for (int p = 0; p < RA / 2; ++p)
                            ((uint16_t*)a.h)[row * a.f + orow0 + p * 16 + r16] =
                                f32_to_bf16(silu_mul(acc[2 * p][j][i], acc[2 * p + 1][j][i]));
                    } else {
#pragma unroll
                        for (int u = 0; u < RA; ++u) store_y_as<YB>(a, row, orow0 + u * 16 + r16, acc[u][j][i]);
                    }
                }
            }
        }
    });
}

}  // namespace

// One launch shape: RA row blocks a wave, G token groups an item, R stages in flight, inputs split
// over S waves.  An unsupported shape returns MOE_EDTYPE with nothing launched.
template <int MODE, int W, int RA, int G, int R, int S, bool XL = false, bool IL = false, bool CW = false>
static moe_status launch_ks(const FfnArgs& a, hipStream_t st, const char* name) {
    const int M = (MODE == kGateUp) ? a.f : a.d;            // output rows
    const int K = (MODE == kGateUp) ? a.d : a.f;
    const int per_wave = (MODE == kGateUp) ? RA / 2 : RA;    // output row blocks a wave
    const int groups = kKsWaves / S;                         // row-block groups a workgroup
    if ((M / 16) % (per_wave * groups) != 0 || (K / KsFrag<W>::kIn) % S != 0) return MOE_EDTYPE;
    if (XL && (a.T > kXlTok || (size_t)kXlTok * K * 2 > 65536)) return MOE_EDTYPE;
    const int ntg = 16 * G;
    const int64_t items = work_items(a, ntg);
    if (items > 65535) return set_error(MOE_ESHAPE, "%s: %lld work items exceed one launch", name, (long long)items);
    dim3 grid((unsigned)(M / 16 / (per_wave * groups)), (unsigned)items), block(64 * kKsWaves);
    // staged rows: as many as an item can hold (min(T, kXlTok)); then the S-way join buffer
    const size_t lds = (XL ? (size_t)std::min(a.T, kXlTok) * K * 2 : 0) + (S > 1 ? (size_t)kKsWaves * RA * G * 1024 : 0);
    ProfScope ps(name, st);
    ffn_gemv_ks_kernel<MODE, W, RA, G, R, S, XL, IL, CW><<<grid, block, lds, st>>>(a);
    return check_launch(name);
}

// Launch shape by projection, weight type and batch (-1: leave the launch to the other decode
// kernels).  Chosen by measurement on MI355X over the decode workloads (Qwen3-30B-A3B-like bf16
// and DeepSeek-V4-Flash-like int4 layers, 1 to 64 tokens):
//   bf16 gate/up: four waves split the inputs of a wave's row blocks, interleaved (wave s takes
//     stages s, s+4, ...: the group reads adjacent fragments at a time, measured 1-2 us faster
//     than contiguous shares); one gate/up pair a wave over 16-token items up to 16 tokens, two
//     pairs a wave over 16-token items with cached weight loads up to 64 (the dispatch below
//     gives the figures), two pairs a wave over 32-token items above;
//   bf16 down: one row block a wave with 5 stages in flight for up to 4 tokens, four row blocks
//     a wave with one stage ahead up to 16 tokens (19.7 against 21.0 us at 16), two row blocks
//     a wave over 32-token items with two waves splitting their inputs, interleaved, up to 32
//     tokens (24.2 against 25.4 us at 24 tokens and 26.1 against 28.2 at 32; equal at 48 and
//     35.4 against 33.1 at 64), else the same without the split;
//   int4 gate/up: below 8 tokens four waves split the inputs of two gate/up pairs, interleaved
//     (21.9 against 22.5 us for the vector-ALU kernel at one token, 29.0 against 31.9 for two
//     waves splitting one pair at two); from 8 tokens one wave takes two pairs over all inputs
//     with two stages in flight (65.6 against 67.9 us at 8 tokens);
//   int4 down: up to 4 tokens, four waves split the inputs of four row blocks a wave,
//     interleaved (14.7 against 15.0 us at one token), else one row block a wave with 7 stages in
//     flight and the item's h rows staged in LDS; above 4 tokens four row blocks a wave with one
//     stage in flight ahead (33.8 against 41.7 us at 8 tokens for two waves splitting the inputs
//     of two row blocks).
static int ks_plan(int mode, moe_dtype w, int T) {
    if (w == MOE_BF16) {
        if (mode == kGateUp) return T <= 16 ? 0 : 1;
        return T <= 4 ? 0 : T <= 16 ? 2 : T <= 32 ? 3 : 1;
    }
    if (w == MOE_INT4_G128) {
        if (mode == kGateUp) return T >= 8 ? 1 : 2;
        return T <= kXlTok ? 1 : 0;
    }
    return -1;
}

moe_status ffn_gemv_ks(const FfnArgs& a, int mode, moe_dtype w, hipStream_t st) {
    const int plan = ks_plan(mode, w, a.T);
    if (plan < 0) return MOE_EDTYPE;
    if (w == MOE_BF16 && mode == kGateUp) {
        if (plan == 0) return launch_ks<kGateUp, MOE_BF16, 2, 1, 4, 4, false, true>(a, st, "ffn_gemv_gateup_bf16");
        // Decode calls (17 to 64 tokens) take 16-token items and read the weights through the cache:
        // an expert holding more than 16 tokens has several items, which stream the same weights,
        // and the later ones (the next blockIdx.y with the same blockIdx.x, on the same XCD a few
        // dispatches later) find them in L2, so the smaller items buy more workgroups for little
        // HBM traffic.  Measured against 32-token items with non-temporal loads: 58.3 -> 56.3 us at
        // 64 tokens (323.5 MB a launch before), 47.5 -> 44.5 us at 32 (with cached loads alone:
        // 56.8 and 47.5).  The next step's router logits, whose weights the cached expert weights
        // displace, take about 0.4 us longer.  The light experts of a bf16 prefill call (single
        // items, nothing read twice) ran 3-5 % slower with cached weight loads, and up to 16 tokens
        // the cached 16-token plan with two pairs a wave is slower than plan 0, so both stay as
        // they were.
        if (a.T <= 64) return launch_ks<kGateUp, MOE_BF16, 4, 1, 4, 4, false, true, true>(a, st, "ffn_gemv_gateup_bf16");
        return launch_ks<kGateUp, MOE_BF16, 4, 2, 4, 4, false, true>(a, st, "ffn_gemv_gateup_bf16");
    }
    if (w == MOE_BF16) {
        if (plan == 0) return launch_ks<kDown, MOE_BF16, 1, 1, 6, 1>(a, st, "ffn_gemv_down_bf16");
        if (plan == 2) {
            const moe_status r = launch_ks<kDown, MOE_BF16, 4, 2, 2, 1>(a, st, "ffn_gemv_down_bf16");
            if (r != MOE_EDTYPE) return r;
        }
        if (plan == 3) {
            const moe_status r = launch_ks<kDown, MOE_BF16, 2, 2, 4, 2, false, true>(a, st, "ffn_gemv_down_bf16");
            if (r != MOE_EDTYPE) return r;
        }
        return launch_ks<kDown, MOE_BF16, 2, 2, 4, 1>(a, st, "ffn_gemv_down_bf16");
    }
    // a plan whose row blocks do not divide the matrix returns EDTYPE before launching: the next
    if (mode == kGateUp) {
        moe_status r = plan == 1 ? launch_ks<kGateUp, MOE_INT4_G128, 4, 1, 3, 1>(a, st, "ffn_gemv_gateup_int4")
                                 : launch_ks<kGateUp, MOE_INT4_G128, 4, 1, 2, 4, false, true>(a, st, "ffn_gemv_gateup_int4");
        if (r != MOE_EDTYPE) return r;
        if (a.T < 2) return MOE_EDTYPE;  // one token: the vector-ALU kernel is as fast as the plan below
        return launch_ks<kGateUp, MOE_INT4_G128, 2, 1, 4, 2>(a, st, "ffn_gemv_gateup_int4");
    }
    if (plan == 1) {
        moe_status r = launch_ks<kDown, MOE_INT4_G128, 4, 1, 2, 4, false, true>(a, st, "ffn_gemv_down_int4");
        if (r != MOE_EDTYPE) return r;
        r = launch_ks<kDown, MOE_INT4_G128, 1, 1, 8, 1, true>(a, st, "ffn_gemv_down_int4");
        if (r != MOE_EDTYPE) return r;  // rows too long to stage: the plan below
    } else {
        const moe_status r = launch_ks<kDown, MOE_INT4_G128, 4, 1, 2, 1>(a, st, "ffn_gemv_down_int4");
        if (r != MOE_EDTYPE) return r;
    }
    return launch_ks<kDown, MOE_INT4_G128, 2, 1, 3, 2>(a, st, "ffn_gemv_down_int4");
}

}  // namespace moe
