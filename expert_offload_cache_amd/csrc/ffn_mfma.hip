// Grouped SwiGLU experts for many tokens per expert (prefill): bf16 MFMA grouped GEMM.
//
// Expert weights are reached through the slot table (FreeToken GGUF page, "MoE backends",
// offload backend); the expert form (SwiGLU, no biases) is the plain reading.  With hundreds
// of tokens per expert the contraction is dense and runs on the matrix cores:
// v_mfma_f32_16x16x32_bf16 takes A = 16 weight rows x 32 inputs with lane l holding row l%16,
// inputs 8(l/16)..+7 -- exactly one 16-byte lane share of the slot layout's fragments -- and
// B = 32 inputs x 16 tokens with the same input split; C (binary32) holds, in lane l, token
// l%16 and weight rows 4(l/16)..+3.
//
// Tiling: a workgroup of 8 waves (4 along weight rows x 2 along tokens) computes 256 weight
// rows x NT tokens of one expert (NT = 128 or 256); each wave owns 64 rows x NT/2 tokens.  In the
// gate/up launch a wave's 64 rows are 32 gate rows and the same 32 up rows, so SwiGLU is
// applied in registers before one bf16 store of h.  Inputs advance 64 at a time through a
// double-buffered LDS stage: weights are copied fragment for fragment (the global layout is the
// LDS layout), token rows are gathered through the permutation into a padded [token][input]
// tile.  Global loads run two stages ahead of the MFMAs in registers.
// Workgroup (m, n) follows (m, n-1) sixteen blocks later in dispatch order, i.e. on the same
// XCD (blocks go round-robin over 8), so an expert's weight tile is reused from that XCD's L2
// across its token tiles.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "ffn.h"
#include "ffn_common.h"
#include "slot_layout.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMT = 256;             // weight rows per workgroup
constexpr int kKT = 64;              // inputs per LDS stage (two fragments)
constexpr int kBRow = kKT * 2 + 16;  // padded LDS row of one token (bytes)
constexpr int kAStage = kMT * kKT * 2;  // 32 KB

template <int NT>
struct Tile {
    static constexpr int kNTW = NT / 32;           // 16-token blocks per wave
    static constexpr int kBV = NT * 8 / 512;       // B vectors per thread per stage
    static constexpr int kBStage = NT * kBRow;
    static constexpr int kStage = kAStage + kBStage;
    static constexpr int kLds = 2 * kStage;        // 100 KB (NT 128) or 136 KB (NT 256)
};

__device__ __forceinline__ f32x4_t mfma(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
}

template <int MODE, int NT>
__global__ __launch_bounds__(512) void ffn_mfma_kernel(FfnArgs a) {
    using TL = Tile<NT>;
    constexpr int NTW = TL::kNTW, BV = TL::kBV;
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv & 3, wn = wv >> 2;  // wave position: 4 along rows, 2 along tokens
    const int K = (MODE == kGateUp) ? a.d : a.f;
    const int nks = K / kKT;  // stages (even)

    int e, chunk;
    if (!find_work(a.counts, a.E, a.T, NT, a.shared_w != nullptr, blockIdx.y, e, chunk)) return;
    const bool shared = e == -1;
    const int n_all = __builtin_amdgcn_readfirstlane(shared ? a.T : a.counts[e]);
    const int t0 = chunk * NT;
    const int nt = __builtin_amdgcn_readfirstlane(min(NT, n_all - t0));
    const int p0 = __builtin_amdgcn_readfirstlane(shared ? a.T * a.k : a.offsets[e]);
    const uint8_t* base;
    if (shared) {
        base = a.shared_w;
    } else {
        const int slot = __builtin_amdgcn_readfirstlane(a.slot_of_expert[e]);
        if (slot < 0 || slot >= a.n_slots) {
            if (tid == 0) *a.status = 1;
            // zeros for this tile's outputs; nothing is read from the pool
            const int rows0 = (MODE == kGateUp) ? blockIdx.x * (kMT / 2) : blockIdx.x * kMT;
            const int nr = (MODE == kGateUp) ? kMT / 2 : kMT;
            for (int i = tid; i < nt * nr; i += blockDim.x) {
                const size_t row = (size_t)(p0 + t0 + i / nr);
                const int col = rows0 + i % nr;
                if (MODE == kGateUp) ((uint16_t*)a.h)[row * a.f + col] = 0;
                else a.y_perm[row * a.d + col] = 0.f;
            }
            return;
        }
        base = a.pool + (size_t)slot * a.stride;
    }

    // A source of this thread: 16 row blocks x 2 fragments per stage = 2048 vectors, 4 per
    // thread; vector v = tid + 512u is row block (tid>>7) + 4u (gate/up: g0,u0,g1,u1,...; down:
    // d blocks), bytes 16*(tid&127) of its two fragments.  In both launches the row block's byte
    // offset is linear in the block index, so the four sources are one pointer and a stride.
    const size_t rbb = rowblock_bytes(K, MOE_BF16);
    const uint8_t* a_src;
    {
        const int j = tid >> 7;
        if constexpr (MODE == kGateUp) a_src = base + gu_block_offset(blockIdx.x * 8 + (j >> 1), j & 1, a.d, MOE_BF16);
        else a_src = base + down_block_offset(blockIdx.x * 16 + j, a.d, a.f, MOE_BF16);
        a_src += (size_t)(tid & 127) * 16;
    }
    // B source: 8 threads cover one token's 64 inputs of a stage (128 contiguous bytes); thread
    // tid stages inputs 8*(tid&7)..+7 of tokens (tid>>3) + 64u.  Tokens past the tile's end read
    // the tile's first row instead: MFMA columns are independent and those columns are never
    // stored.  Row offsets fit 32 bits (activation and h buffers are far below 4 GiB).
    const int seg = tid & 7;
    const uint8_t* b_base = (MODE == kGateUp) ? (const uint8_t*)a.x : (const uint8_t*)a.h;
    uint32_t b_off[BV];
#pragma unroll
    for (int u = 0; u < BV; ++u) {
        int tok = (tid >> 3) + u * 64;
        tok = tok < nt ? tok : 0;
        int src;
        if (MODE == kGateUp) src = shared ? (t0 + tok) : (a.perm[p0 + t0 + tok] / a.k);
        else src = p0 + t0 + tok;
        b_off[u] = (uint32_t)src * (uint32_t)(K * 2) + (uint32_t)seg * 16;
    }
    const uint32_t s_off = (uint32_t)(tid >> 3) * kBRow + seg * 16;  // LDS B slot of u = 0

    f32x4_t acc[4][NTW];  // [row block of the wave][token block of the wave]
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j) acc[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

    u32x4_t pa[4], pb[BV], qa[4], qb[BV];  // native vectors: registers, never memory
#define MFMA_GLOAD(KS, RA, RB)                                                                         \
    do {                                                                                               \
        const int ks_ = (KS);                                                                          \
        _Pragma("unroll") for (int u = 0; u < 4; ++u) RA[u] =                                          \
            *(const u32x4_t*)(a_src + (size_t)u * 4 * rbb + (size_t)ks_ * 2048);                         \
        _Pragma("unroll") for (int u = 0; u < BV; ++u) RB[u] =                                         \
            *(const u32x4_t*)(b_base + b_off[u] + (size_t)ks_ * (kKT * 2));                              \
        __builtin_amdgcn_sched_barrier(0); /* issue here, ahead of the MFMAs */                        \
    } while (0)
#define MFMA_SSTORE(BUF, RA, RB)                                                                       \
    do {                                                                                               \
        uint8_t* sa_ = smem + (BUF) * TL::kStage;                                                      \
        _Pragma("unroll") for (int u = 0; u < 4; ++u) *(u32x4_t*)(sa_ + (size_t)(tid + u * 512) * 16) = RA[u]; \
        _Pragma("unroll") for (int u = 0; u < BV; ++u) *(u32x4_t*)(sa_ + kAStage + s_off + u * 64 * kBRow) = RB[u]; \
    } while (0)
#define MFMA_COMPUTE(BUF)                                                                              \
    do {                                                                                               \
        const uint8_t* sa_ = smem + (BUF) * TL::kStage;                                                \
        const uint8_t* sb_ = sa_ + kAStage;                                                            \
        _Pragma("unroll") for (int kk = 0; kk < 2; ++kk) {                                             \
            u32x4_t av[4];                                                                               \
            _Pragma("unroll") for (int i = 0; i < 4; ++i) av[i] =                                      \
                *(const u32x4_t*)(sa_ + ((wm * 4 + i) * 2 + kk) * 1024 + lane * 16);                     \
            _Pragma("unroll") for (int j = 0; j < NTW; ++j) {                                          \
                const int tok = (wn * NTW + j) * 16 + (lane & 15);                                     \
                const u32x4_t bv = *(const u32x4_t*)(sb_ + tok * kBRow + (kk * 32 + 8 * (lane >> 4)) * 2); \
                _Pragma("unroll") for (int i = 0; i < 4; ++i) acc[i][j] = mfma(av[i], bv, acc[i][j]);  \
            }                                                                                          \
        }                                                                                              \
    } while (0)

    // stages ks and ks+1 per trip; the last two stages are peeled so that the loop body has no
    // branch (a conditional store there makes the back edge wait for every load in flight)
    MFMA_GLOAD(0, pa, pb);
    MFMA_GLOAD(1, qa, qb);
    MFMA_SSTORE(0, pa, pb);
    __syncthreads();
    for (int ks = 0; ks < nks - 2; ks += 2) {
        MFMA_GLOAD(ks + 2, pa, pb);
        MFMA_COMPUTE(0);
        MFMA_SSTORE(1, qa, qb);
        __syncthreads();
        MFMA_GLOAD(ks + 3, qa, qb);
        MFMA_COMPUTE(1);
        MFMA_SSTORE(0, pa, pb);
        __syncthreads();
    }
    MFMA_COMPUTE(0);
    MFMA_SSTORE(1, qa, qb);
    __syncthreads();
    MFMA_COMPUTE(1);
#undef MFMA_GLOAD
#undef MFMA_SSTORE
#undef MFMA_COMPUTE

    // ---- epilogue --------------------------------------------------------------------------
    const int quad = lane >> 4;  // C rows 4*quad .. +3 of each 16-row tile
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
        const int tok = (wn * NTW + j) * 16 + (lane & 15);
        if (tok >= nt) continue;
        const size_t row = (size_t)(p0 + t0 + tok);
        if constexpr (MODE == kGateUp) {
#pragma unroll
            for (int i2 = 0; i2 < 2; ++i2) {  // wave row blocks (g, u) pairs: (i2*2, i2*2+1)
                const f32x4_t g = acc[2 * i2][j], u = acc[2 * i2 + 1][j];
                const int col = (blockIdx.x * 8 + wm * 2 + i2) * 16 + quad * 4;
                uint2 o;
                o.x = (uint32_t)f32_to_bf16(silu_mul(g[0], u[0])) | ((uint32_t)f32_to_bf16(silu_mul(g[1], u[1])) << 16);
                o.y = (uint32_t)f32_to_bf16(silu_mul(g[2], u[2])) | ((uint32_t)f32_to_bf16(silu_mul(g[3], u[3])) << 16);
                *(uint2*)((uint16_t*)a.h + row * a.f + col) = o;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int col = (blockIdx.x * 16 + wm * 4 + i) * 16 + quad * 4;
                *(float4*)(a.y_perm + row * a.d + col) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
            }
        }
    }
}

template <int MODE, int NT>
moe_status launch(const FfnArgs& a, hipStream_t st, const char* name) {
    const int M = (MODE == kGateUp) ? 2 * a.f : a.d;  // weight rows (gate and up together)
    const int64_t tk = (int64_t)a.T * a.k;
    const int64_t items = (tk + NT - 1) / NT + std::min<int64_t>(a.E, tk) + (a.shared_w ? (a.T + NT - 1) / NT : 0);
    if (items > 65535) return set_error(MOE_ESHAPE, "%s: %lld token tiles exceed one launch", name, (long long)items);
    auto kern = ffn_mfma_kernel<MODE, NT>;
    MOE_HIP(hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, Tile<NT>::kLds));
    dim3 grid((unsigned)(M / kMT), (unsigned)items);
    ProfScope p(name, st);
    kern<<<grid, 512, Tile<NT>::kLds, st>>>(a);
    return check_launch(name);
}

}  // namespace

// Many tokens per expert and bf16: the MFMA path.  Other cases report MOE_EDTYPE ("not mine").
moe_status ffn_mfma(const FfnArgs& a, moe_dtype act, moe_dtype w, hipStream_t st) {
    if (act != MOE_BF16 || w != MOE_BF16 || a.T <= 64) return MOE_EDTYPE;
    if ((2 * a.f) % kMT || a.d % kMT || a.d % (2 * kKT) || a.f % (2 * kKT)) return MOE_EDTYPE;
    moe_status r = launch<kGateUp, 128>(a, st, "ffn_mfma_gateup_bf16");
    if (r != MOE_OK) return r;
    return launch<kDown, 128>(a, st, "ffn_mfma_down_bf16");
}

}  // namespace moe
