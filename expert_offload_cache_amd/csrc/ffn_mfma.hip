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
// rows x 128 tokens of one expert; each wave owns 64 rows x 64 tokens = 16 MFMA tiles.  In the
// gate/up launch a wave's 64 rows are 32 gate rows and the same 32 up rows, so SwiGLU is
// applied in registers before one bf16 store of h.  Inputs advance 64 at a time through a
// double-buffered LDS stage: weights are copied fragment for fragment (the global layout is the
// LDS layout), token rows are gathered through the permutation into a padded [token][input]
// tile.  Workgroup (m, n) follows (m, n-1) sixteen blocks later in dispatch order, i.e. on the
// same XCD (blocks go round-robin over 8), so an expert's weight tile is reused from that XCD's
// L2 across its token tiles.
#include <hip/hip_runtime.h>

#include "ffn.h"
#include "ffn_common.h"
#include "slot_layout.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMT = 256;           // weight rows per workgroup
constexpr int kNT = 128;           // tokens per workgroup
constexpr int kKT = 64;            // inputs per LDS stage (two fragments)
constexpr int kBRow = kKT * 2 + 16;  // padded LDS row of one token (bytes)
constexpr int kAStage = kMT * kKT * 2;       // 32 KB
constexpr int kBStage = kNT * kBRow;         // 18 KB
constexpr int kStage = kAStage + kBStage;
constexpr int kLds = 2 * kStage;             // 100 KB

__device__ __forceinline__ f32x4_t mfma(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
}

// Token tile n of expert item a -> same scheme as the GEMV work items (kNT tokens per chunk).
template <int MODE>
__global__ __launch_bounds__(512) void ffn_mfma_kernel(FfnArgs a) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv & 3, wn = wv >> 2;  // wave position: 4 along rows, 2 along tokens
    const int K = (MODE == kGateUp) ? a.d : a.f;
    const int nkb = K / 32;  // fragments along the inputs

    int e, chunk;
    if (!find_work(a.counts, a.E, a.T, kNT, a.shared_w != nullptr, blockIdx.y, e, chunk)) return;
    const bool shared = e == -1;
    const int n_all = __builtin_amdgcn_readfirstlane(shared ? a.T : a.counts[e]);
    const int t0 = chunk * kNT;
    const int nt = __builtin_amdgcn_readfirstlane(min(kNT, n_all - t0));
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

    // 16 row blocks of this workgroup: gate/up -> f blocks mb*8 .. +7, gate and up interleaved
    // as (g0, u0, g1, u1, ...); down -> d blocks mb*16 .. +15
    auto rowblock_src = [&](int j) -> const uint8_t* {
        if constexpr (MODE == kGateUp) {
            const int fb = blockIdx.x * 8 + (j >> 1);
            return base + gu_block_offset(fb, j & 1, a.d, MOE_BF16);
        } else {
            return base + down_block_offset(blockIdx.x * 16 + j, a.d, a.f, MOE_BF16);
        }
    };

    // token rows staged by this thread: 8 threads cover one token's 64 inputs (128 contiguous
    // bytes), so thread tid stages inputs 8*(tid&7)..+7 of tokens (tid>>3) and 64+(tid>>3)
    const int seg = tid & 7;
    const uint8_t* tok_row[2];
    bool tok_ok[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int tok = (tid >> 3) + u * 64;
        tok_ok[u] = tok < nt;
        int src = 0;
        if (tok_ok[u]) {
            if (MODE == kGateUp) src = shared ? (t0 + tok) : (a.perm[p0 + t0 + tok] / a.k);
            else src = p0 + t0 + tok;
        }
        tok_row[u] = ((MODE == kGateUp) ? (const uint8_t*)a.x : (const uint8_t*)a.h) + (size_t)src * K * 2 +
                     (size_t)seg * 16;
    }

    // global -> registers for one stage: A = 16 row blocks x 2 fragments (32 KB, 4 vectors per
    // thread, the same byte order in LDS as in the slot); B = 128 tokens x 64 inputs (2 vectors)
    uint4 ra[4], rbv[2];
    auto gload = [&](int ks) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int v = tid + u * 512;              // 16-byte vector index in the A stage
            const int j = v >> 7, within = v & 127;   // row block, vector inside its 2 KB
            ra[u] = *(const uint4*)(rowblock_src(j) + (size_t)ks * 2048 + (size_t)within * 16);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
            rbv[u] = tok_ok[u] ? *(const uint4*)(tok_row[u] + (size_t)ks * kKT * 2) : make_uint4(0, 0, 0, 0);
    };
    auto sstore = [&](int buf) {
        uint8_t* sa = smem + buf * kStage;
        uint8_t* sb = sa + kAStage;
#pragma unroll
        for (int u = 0; u < 4; ++u) *(uint4*)(sa + (size_t)(tid + u * 512) * 16) = ra[u];
#pragma unroll
        for (int u = 0; u < 2; ++u) *(uint4*)(sb + ((tid >> 3) + u * 64) * kBRow + seg * 16) = rbv[u];
    };

    f32x4_t acc[4][4];  // [row block of the wave][token block of the wave]
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

    const int nks = nkb / 2;  // stages
    gload(0);
    sstore(0);
    __syncthreads();
    for (int ks = 0; ks < nks; ++ks) {
        const int buf = ks & 1;
        if (ks + 1 < nks) gload(ks + 1);  // next stage in flight during the MFMAs
        const uint8_t* sa = smem + buf * kStage;
        const uint8_t* sb = sa + kAStage;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {  // two 32-input steps per stage
            uint4 av[4], bv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)  // wave's row blocks: wm*4 + i
                av[i] = *(const uint4*)(sa + ((size_t)(wm * 4 + i) * 2 + kk) * 1024 + lane * 16);
#pragma unroll
            for (int j = 0; j < 4; ++j) {  // wave's token blocks: wn*4 + j
                const int tok = (wn * 4 + j) * 16 + (lane & 15);
                bv[j] = *(const uint4*)(sb + tok * kBRow + (kk * 32 + 8 * (lane >> 4)) * 2);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma(av[i], bv[j], acc[i][j]);
        }
        if (ks + 1 < nks) {
            sstore(buf ^ 1);
            __syncthreads();
        }
    }

    // ---- epilogue --------------------------------------------------------------------------
    const int quad = lane >> 4;  // C rows 4*quad .. +3 of each 16-row tile
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int tok = (wn * 4 + j) * 16 + (lane & 15);
        if (tok >= nt) continue;
        const size_t row = (size_t)(p0 + t0 + tok);
        if constexpr (MODE == kGateUp) {
#pragma unroll
            for (int i2 = 0; i2 < 2; ++i2) {  // wave row blocks (g, u) pairs: (i2*2, i2*2+1)
                const f32x4_t g = acc[2 * i2][j], u = acc[2 * i2 + 1][j];
                const int fb = blockIdx.x * 8 + (wm * 4 + 2 * i2) / 2;
                const int col = fb * 16 + quad * 4;
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

template <int MODE>
moe_status launch(const FfnArgs& a, hipStream_t st, const char* name) {
    const int M = (MODE == kGateUp) ? 2 * a.f : a.d;  // weight rows (gate and up together)
    const int64_t tk = (int64_t)a.T * a.k;
    const int64_t items = (tk + kNT - 1) / kNT + std::min<int64_t>(a.E, tk) + (a.shared_w ? (a.T + kNT - 1) / kNT : 0);
    if (items > 65535) return set_error(MOE_ESHAPE, "%s: %lld token tiles exceed one launch", name, (long long)items);
    auto kern = ffn_mfma_kernel<MODE>;
    MOE_HIP(hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, kLds));
    dim3 grid((unsigned)(M / kMT), (unsigned)items);
    ProfScope p(name, st);
    kern<<<grid, 512, kLds, st>>>(a);
    return check_launch(name);
}

}  // namespace

// Many tokens per expert and bf16: the MFMA path.  Other cases report MOE_EDTYPE ("not mine").
moe_status ffn_mfma(const FfnArgs& a, moe_dtype act, moe_dtype w, hipStream_t st) {
    if (act != MOE_BF16 || w != MOE_BF16 || a.T <= 64) return MOE_EDTYPE;
    if ((2 * a.f) % kMT || a.d % kMT || a.d % kKT || a.f % kKT) return MOE_EDTYPE;
    moe_status r = launch<kGateUp>(a, st, "ffn_mfma_gateup_bf16");
    if (r != MOE_OK) return r;
    return launch<kDown>(a, st, "ffn_mfma_down_bf16");
}

}  // namespace moe
