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
// Tiling (bf16 weights): a workgroup of 8 waves computes MT = 512 weight rows x NT = 128 tokens of
// one expert; each wave owns 64 rows x 128 tokens.  In the gate/up launch a wave's 64 rows are 32
// gate rows and the same 32 up rows, so SwiGLU is applied in registers before one bf16 store of h.
// Inputs advance 32 at a time.  Each wave loads its own weight fragments (4 x 1 KB a stage, one
// 16-byte load per lane each, already in A-operand order) straight into registers, R stages
// ahead; the token rows are gathered through the permutation straight into B fragments in a ring
// of R LDS stages filled by direct-to-LDS loads (global_load_lds_dwordx4), shared by the 8 waves.
// So the LDS carries only the token fragments (written once, read by every wave as conflict-free
// 16-byte lane reads) -- measured against staging the weights in LDS too, this lifts the dense
// contraction from 0.43 to 0.46 of the MFMA peak and moves the same bits.  Measured and dropped:
// 3 to 6 stages of lead (no gain beyond 3), two 4-wave workgroups per CU with 256-row tiles (0.47
// -> 0.32 dense), 256 x 256 tiles (0.39).
// int4 weights use a 256-row variant that dequantises in registers (below).
// Workgroup (m, n) follows (m, n-1) M/MT blocks later in dispatch order; blocks go round-robin
// over the 8 XCDs, so where M/MT is a multiple of 8 (the large shapes) an expert's weight tile
// stays on one XCD and is reused from its L2 across the token tiles.
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

constexpr int kKT = 32;  // inputs per stage (one fragment)

__device__ __forceinline__ f32x4_t mfma(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
}

// Wait until at most N of this wave's direct-to-LDS loads are in flight and its LDS reads are
// done, then meet the other waves.  After it, the stage whose loads were issued before the last
// N has landed for the whole workgroup, and no wave still reads the buffer the next loads fill.
// The empty asm statements keep the compiler from moving LDS accesses across the barrier.
template <int N>
__device__ __forceinline__ void stage_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));  // vmcnt(N) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ void load_to_lds(const uint8_t* src, uint8_t* lds_wave_base) {
    // 16 bytes per lane; lane i's bytes land at lds_wave_base + 16 i whatever its source address
    __builtin_amdgcn_global_load_lds((gbl_ptr_t)src, (lds_ptr_t)lds_wave_base, 16, 0, 0);
}

// int4 weights.  A fragment of the slot layout holds 16 rows x 128 inputs (1 KB); lane l's word s
// carries inputs 32 s + 8(l/16) + 0..7 of row l%16, i.e. the A operand of the MFMA's s-th 32-input
// step, 4 bits an input.  Each wave loads its own fragments straight into registers (non-temporal,
// one 128-input group ahead) and dequantises one word per step into bf16(q s) -- the weight of the
// int4 format, rounded once to bf16 -- with the row's group scale; the token rows go through the
// same direct-to-LDS ring as in the bf16 kernel, 32 inputs a stage.
template <int MT, int NT, int WM, int R, int NW>
struct Tile4 {
    static constexpr int kWN = NW / WM;
    static constexpr int kRA = MT / 16 / WM;   // row blocks per wave
    static constexpr int kRB = NT / 16 / kWN;  // token blocks per wave
    static constexpr int kLB = NT / 16 / NW;   // token fragments each wave loads per stage
    static constexpr int kStage = NT * kKT * 2;
    static constexpr int kLds = R * kStage;
    static constexpr int kLoads = kLB;
    static_assert(kRA % 2 == 0 && kRA * WM * 16 == MT && kRB * kWN * 16 == NT && kLB * NW * 16 == NT && R >= 3,
                  "tile shape");
};

// word w of an int4 fragment (input pairs at bits 4p and 16+4p, nibble u -> q = u - 8) times the
// scale s -> the 8 bf16 A-operand values (round to nearest even; q s itself is exact in binary32).
// The nibbles are first spread one to a byte (even nibbles in lo4, odd ones in hi4), so that each
// becomes a float with one byte conversion (v_cvt_f32_ubyte0..3): byte b of lo4 holds bits 8b..8b+3
// of w, byte b of hi4 bits 8b+4..8b+7.  The empty asm statements hide the masks from the optimizer,
// which would otherwise fold them back into one bit-field extract per nibble (28 instead of 23
// vector instructions a word).
__device__ __forceinline__ u32x4_t dequant_word(uint32_t w, float s) {
    typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
    typedef float f32x2v __attribute__((ext_vector_type(2)));
    const float m8 = -8.f * s;
    uint32_t lo4 = w & 0x0F0F0F0Fu, hi4 = (w >> 4) & 0x0F0F0F0Fu;
    asm("" : "+v"(lo4));
    asm("" : "+v"(hi4));
    // pair p = (bits 4p, bits 16+4p): p=0 lo4 bytes 0,2; p=1 hi4 bytes 0,2; p=2 lo4 bytes 1,3; p=3 hi4 bytes 1,3
    const uint32_t src[4] = {lo4, hi4, lo4 >> 8, hi4 >> 8};
    uint32_t r[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const float lo = __builtin_fmaf((float)(src[p] & 0xffu), s, m8);
        const float hi = __builtin_fmaf((float)((src[p] >> 16) & 0xffu), s, m8);
        r[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){lo, hi}, bf16x2v));
    }
    return u32x4_t{r[0], r[1], r[2], r[3]};
}

template <int MODE, int MT, int NT, int WM, int R, int NW>
__global__ __launch_bounds__(NW * 64, 2) void ffn_mfma_int4_kernel(FfnArgs a) {
    using TL = Tile4<MT, NT, WM, R, NW>;
    constexpr int RA = TL::kRA, RB = TL::kRB, LB = TL::kLB;
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv % WM, wn = wv / WM;
    const int K = (MODE == kGateUp) ? a.d : a.f;
    const int nks = K / kKT;   // 32-input stages
    const int ng = K / 128;    // int4 groups (fragments per row block)

    int e, chunk;
    if (!find_work(a.counts, a.E, a.T, NT, a.shared_w != nullptr, blockIdx.y, e, chunk, a.n_lo, a.n_hi)) return;
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
        if (slot == MOE_SLOT_ELSEWHERE) return;  // rows produced elsewhere: leave them
        if (slot < 0 || slot >= a.n_slots) {
            if (tid == 0) *a.status = 1;
            const int rows0 = (MODE == kGateUp) ? blockIdx.x * (MT / 2) : blockIdx.x * MT;
            const int nr = (MODE == kGateUp) ? MT / 2 : MT;
            for (int i = tid; i < nt * nr; i += blockDim.x) {
                const size_t row = (size_t)(p0 + t0 + i / nr);
                const int col = rows0 + i % nr;
                if (MODE == kGateUp) ((uint16_t*)a.h)[row * a.f + col] = 0;
                else store_y(a, row, col, 0.f);
            }
            return;
        }
        base = a.pool + (size_t)slot * a.stride;
    }

    // this wave's row blocks (gate/up: pairs g, u of the same 16 outputs) and their scales
    const uint8_t* a_blk[RA];
#pragma unroll
    for (int u = 0; u < RA; ++u) {
        const int j = wm * RA + u;
        if constexpr (MODE == kGateUp)
            a_blk[u] = base + gu_block_offset(blockIdx.x * (MT / 32) + (j >> 1), j & 1, a.d, MOE_INT4_G128);
        else
            a_blk[u] = base + down_block_offset(blockIdx.x * (MT / 16) + j, a.d, a.f, MOE_INT4_G128);
    }
    const int r16 = lane & 15;
    u32x4_t aw[RA], an[RA];  // raw fragments of the current and the next group
    uint32_t sc[RA], sn[RA];  // their bf16 scales, converted where used (not across the loop edge)
    auto load_group = [&](int g, u32x4_t (&w)[RA], uint32_t (&scl)[RA]) __attribute__((always_inline)) {
        g = min(g, ng - 1);  // past the end: reload the last group (never used)
#pragma unroll
        for (int u = 0; u < RA; ++u) {
            w[u] = __builtin_nontemporal_load((const u32x4_t*)(a_blk[u] + (size_t)g * 1024 + lane * 16));
            scl[u] = *(const uint16_t*)(a_blk[u] + (size_t)ng * 1024 + ((size_t)r16 * ng + g) * 2);
        }
    };

    // B fragment lane l: token 16 tb + l%16, inputs 8(l/16)..+7 of the stage.  Tokens past the
    // tile's end read the tile's first row: MFMA columns are independent and are never stored.
    const uint8_t* b_src[LB];
    {
        const uint8_t* b_base = (MODE == kGateUp) ? (const uint8_t*)a.x : (const uint8_t*)a.h;
#pragma unroll
        for (int u = 0; u < LB; ++u) {
            int tok = (LB * wv + u) * 16 + (lane & 15);
            tok = tok < nt ? tok : 0;
            int src;
            if (MODE == kGateUp) src = shared ? (t0 + tok) : (a.perm[p0 + t0 + tok] / a.k);
            else src = p0 + t0 + tok;
            b_src[u] = b_base + (size_t)src * K * 2 + (lane >> 4) * 16;
        }
    }
    auto issue = [&](int ks) __attribute__((always_inline)) {
        ks = min(ks, nks - 1);  // past the end: reload the last stage into a buffer nobody reads
        uint8_t* buf = smem + (ks % R) * TL::kStage;
#pragma unroll
        for (int u = 0; u < LB; ++u) load_to_lds(b_src[u] + (size_t)ks * (kKT * 2), buf + (LB * wv + u) * 1024);
    };

    f32x4_t acc[RA][RB];
#pragma unroll
    for (int i = 0; i < RA; ++i)
#pragma unroll
        for (int j = 0; j < RB; ++j) acc[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

    // The next group's fragments and scales (2 RA loads) are issued in step 0 of a group, after that
    // step's ring load; the barrier of step s counts them among the loads younger than stage ks
    // while they are (steps 1 .. R-1 of the group), so the ring keeps its R-1 stages of lead.
    // Two register sets take turns (group g in set g % 2), so a fragment is used in the registers
    // its load wrote and no copy makes the compiler wait for loads in flight.
    static_assert(R <= 4, "one group start at most among the R-1 younger ring loads");
    auto run_group = [&](int g, const u32x4_t (&cw)[RA], const uint32_t (&cs)[RA], u32x4_t (&nw)[RA],
                         uint32_t (&ns)[RA]) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int ks = 4 * g + s;
            if (s == 0) stage_barrier<(R - 2) * TL::kLoads>();
            else if (s <= R - 1) stage_barrier<(R - 2) * TL::kLoads + 2 * RA>();
            else stage_barrier<(R - 2) * TL::kLoads>();
            issue(ks + R - 1);
            if (s == 0) load_group(g + 1, nw, ns);
            const uint8_t* sb = smem + (ks % R) * TL::kStage;
            u32x4_t av[RA], bv[RB];
#pragma unroll
            for (int i = 0; i < RA; ++i) av[i] = dequant_word(cw[i][s], bf16_to_f32((uint16_t)cs[i]));
#pragma unroll
            for (int j = 0; j < RB; ++j) bv[j] = *(const u32x4_t*)(sb + (wn * RB + j) * 1024 + lane * 16);
#pragma unroll
            for (int j = 0; j < RB; ++j)
#pragma unroll
                for (int i = 0; i < RA; ++i) acc[i][j] = mfma(av[i], bv[j], acc[i][j]);
        }
    };
    load_group(0, aw, sc);
#pragma unroll
    for (int s = 0; s < R - 1; ++s) issue(s);
    for (int g = 0; g < ng; g += 2) {
        run_group(g, aw, sc, an, sn);
        if (g + 1 < ng) run_group(g + 1, an, sn, aw, sc);
    }
    __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));  // drain the tail reloads (vmcnt(0))

    // ---- epilogue (as in the bf16 kernel) ---------------------------------------------------------
    const int quad = lane >> 4;
#pragma unroll
    for (int j = 0; j < RB; ++j) {
        const int tok = (wn * RB + j) * 16 + (lane & 15);
        if (tok >= nt) continue;
        const size_t row = (size_t)(p0 + t0 + tok);
        if constexpr (MODE == kGateUp) {
#pragma unroll
            for (int i2 = 0; i2 < RA / 2; ++i2) {
                const f32x4_t g = acc[2 * i2][j], u = acc[2 * i2 + 1][j];
                const int col = (blockIdx.x * (MT / 32) + (wm * RA) / 2 + i2) * 16 + quad * 4;
                uint2 o;
                o.x = (uint32_t)f32_to_bf16(silu_mul(g[0], u[0])) | ((uint32_t)f32_to_bf16(silu_mul(g[1], u[1])) << 16);
                o.y = (uint32_t)f32_to_bf16(silu_mul(g[2], u[2])) | ((uint32_t)f32_to_bf16(silu_mul(g[3], u[3])) << 16);
                *(uint2*)((uint16_t*)a.h + row * a.f + col) = o;
            }
        } else {
#pragma unroll
            for (int i = 0; i < RA; ++i) {
                const int col = (blockIdx.x * (MT / 16) + wm * RA + i) * 16 + quad * 4;
                store_y4(a, row, col, acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
            }
        }
    }
}

// bf16 weights with the A operands in registers: each wave loads its own weight fragments
// (RA row blocks x 1 KB a stage) straight into one of R register sets, R stages ahead like the
// token ring; only the token rows go through LDS, so the LDS carries B reads and DMA writes only.
// The weight loads are ordinary (cached) loads: the 32 workgroups of an XCD that share a weight
// tile find it in their L2 (non-temporal loads were 8 % slower on the routed 8192-token layer).
// Step ks multiplies its first half of token blocks, meets the other waves (stage ks+1 landed),
// refills stage ks's LDS buffer, reads stage ks+1's token fragments around its second half of
// MFMAs and then refills its weight registers, so a step begins with its operands in registers.
template <int MODE, int MT, int NT, int WM, int R, int NW>
__global__ __launch_bounds__(NW * 64, 2) void ffn_mfma_areg_kernel(FfnArgs a) {
    using TL = Tile4<MT, NT, WM, R, NW>;
    constexpr int RA = TL::kRA, RB = TL::kRB, LB = TL::kLB;
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv % WM, wn = wv / WM;
    const int K = (MODE == kGateUp) ? a.d : a.f;
    const int nks = K / kKT;

    int e, chunk;
    if (!find_work(a.counts, a.E, a.T, NT, a.shared_w != nullptr, blockIdx.y, e, chunk, a.n_lo, a.n_hi)) return;
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
        if (slot == MOE_SLOT_ELSEWHERE) return;
        if (slot < 0 || slot >= a.n_slots) {
            if (tid == 0) *a.status = 1;
            const int rows0 = (MODE == kGateUp) ? blockIdx.x * (MT / 2) : blockIdx.x * MT;
            const int nr = (MODE == kGateUp) ? MT / 2 : MT;
            for (int i = tid; i < nt * nr; i += blockDim.x) {
                const size_t row = (size_t)(p0 + t0 + i / nr);
                const int col = rows0 + i % nr;
                if (MODE == kGateUp) ((uint16_t*)a.h)[row * a.f + col] = 0;
                else store_y(a, row, col, 0.f);
            }
            return;
        }
        base = a.pool + (size_t)slot * a.stride;
    }
    const uint8_t* a_blk[RA];
#pragma unroll
    for (int u = 0; u < RA; ++u) {
        const int j = wm * RA + u;
        if constexpr (MODE == kGateUp)
            a_blk[u] = base + gu_block_offset(blockIdx.x * (MT / 32) + (j >> 1), j & 1, a.d, MOE_BF16) + lane * 16;
        else
            a_blk[u] = base + down_block_offset(blockIdx.x * (MT / 16) + j, a.d, a.f, MOE_BF16) + lane * 16;
    }
    const uint8_t* b_src[LB];
    {
        const uint8_t* b_base = (MODE == kGateUp) ? (const uint8_t*)a.x : (const uint8_t*)a.h;
#pragma unroll
        for (int u = 0; u < LB; ++u) {
            int tok = (LB * wv + u) * 16 + (lane & 15);
            tok = tok < nt ? tok : 0;
            int src;
            if (MODE == kGateUp) src = shared ? (t0 + tok) : (a.perm[p0 + t0 + tok] / a.k);
            else src = p0 + t0 + tok;
            b_src[u] = b_base + (size_t)src * K * 2 + (lane >> 4) * 16;
        }
    }
    u32x4_t areg[R][RA];
    f32x4_t acc[RA][RB];
#pragma unroll
    for (int i = 0; i < RA; ++i)
#pragma unroll
        for (int j = 0; j < RB; ++j) acc[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

    // stage ks: the token fragments to LDS buffer ks % R, this wave's weight fragments to register
    // set ks % R; past the end both repeat the last stage (never used)
    auto issue_lds = [&](int ks) __attribute__((always_inline)) {
        ks = min(ks, nks - 1);
        uint8_t* buf = smem + (ks % R) * TL::kStage;
#pragma unroll
        for (int u = 0; u < LB; ++u) load_to_lds(b_src[u] + (size_t)ks * (kKT * 2), buf + (LB * wv + u) * 1024);
    };
    auto issue_a = [&](int ks, u32x4_t (&set)[RA]) __attribute__((always_inline)) {
        ks = min(ks, nks - 1);
#pragma unroll
        for (int u = 0; u < RA; ++u) set[u] = *(const u32x4_t*)(a_blk[u] + (size_t)ks * 1024);
    };
    constexpr int H = RB / 2;
    // token blocks past the tile's last token are neither read from LDS nor multiplied (a tile of
    // an expert with few tokens then costs its weight stream, not a full tile of MFMAs); their
    // rows are still loaded into the ring so every wave's load count per stage stays fixed.
    // Measured on the routed 8192-token DeepSeek-shaped layer: FFN 3,864 -> 3,779 us, bitwise the
    // same rows.  The int4 GEMM keeps every token block: the same skip there made its 8192-token
    // FFN 2 % slower (its tail tiles spend their time widening weights, not in the MFMAs).
    const int nb = __builtin_amdgcn_readfirstlane((nt + 15) / 16 - wn * RB);
    u32x4_t bv[RB];
    auto read_b = [&](int ks, int j0) __attribute__((always_inline)) {
        const uint8_t* sb = smem + (ks % R) * TL::kStage;
#pragma unroll
        for (int j = j0; j < j0 + H; ++j)
            if (j < nb) bv[j] = *(const u32x4_t*)(sb + (wn * RB + j) * 1024 + lane * 16);
    };
    auto step = [&](int ks, u32x4_t (&cur)[RA]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < H; ++j)
            if (j < nb)
#pragma unroll
                for (int i = 0; i < RA; ++i) acc[i][j] = mfma(cur[i], bv[j], acc[i][j]);
        // stage ks+1 landed (younger: stages ks+2 .. ks+R-1); every wave's reads of stage ks are done
        stage_barrier<(R - 2) * (LB + RA)>();
        issue_lds(ks + R);  // into stage ks's buffer
        const bool more = ks + 1 < nks;
        if (more) read_b(ks + 1, 0);
#pragma unroll
        for (int j = H; j < RB; ++j)
            if (j < nb)
#pragma unroll
                for (int i = 0; i < RA; ++i) acc[i][j] = mfma(cur[i], bv[j], acc[i][j]);
        if (more) read_b(ks + 1, H);
        issue_a(ks + R, cur);  // set ks % R: its last use was just above
    };
#pragma unroll
    for (int r = 0; r < R; ++r) {
        issue_lds(r);
        issue_a(r, areg[r]);
    }
    stage_barrier<(R - 1) * (LB + RA)>();
    read_b(0, 0);
    read_b(0, H);
    int ks = 0;
    for (; ks + R <= nks; ks += R) {
#pragma unroll
        for (int r = 0; r < R; ++r) step(ks + r, areg[r]);
    }
#pragma unroll
    for (int r = 0; r < R - 1; ++r)
        if (ks + r < nks) step(ks + r, areg[r]);
    __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));

    const int quad = lane >> 4;
#pragma unroll
    for (int j = 0; j < RB; ++j) {
        const int tok = (wn * RB + j) * 16 + (lane & 15);
        if (tok >= nt) continue;
        const size_t row = (size_t)(p0 + t0 + tok);
        if constexpr (MODE == kGateUp) {
#pragma unroll
            for (int i2 = 0; i2 < RA / 2; ++i2) {
                const f32x4_t g = acc[2 * i2][j], u = acc[2 * i2 + 1][j];
                const int col = (blockIdx.x * (MT / 32) + (wm * RA) / 2 + i2) * 16 + quad * 4;
                uint2 o;
                o.x = (uint32_t)f32_to_bf16(silu_mul(g[0], u[0])) | ((uint32_t)f32_to_bf16(silu_mul(g[1], u[1])) << 16);
                o.y = (uint32_t)f32_to_bf16(silu_mul(g[2], u[2])) | ((uint32_t)f32_to_bf16(silu_mul(g[3], u[3])) << 16);
                *(uint2*)((uint16_t*)a.h + row * a.f + col) = o;
            }
        } else {
#pragma unroll
            for (int i = 0; i < RA; ++i) {
                const int col = (blockIdx.x * (MT / 16) + wm * RA + i) * 16 + quad * 4;
                store_y4(a, row, col, acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
            }
        }
    }
}

template <int MODE, int MT, int NT, int WM, int R, int NW>
moe_status launch_areg(const FfnArgs& a, hipStream_t st, const char* name) {
    using TL = Tile4<MT, NT, WM, R, NW>;
    const int M = (MODE == kGateUp) ? 2 * a.f : a.d;
    const int64_t items = work_items(a, NT);
    if (items > 65535) return set_error(MOE_ESHAPE, "%s: %lld token tiles exceed one launch", name, (long long)items);
    auto kern = ffn_mfma_areg_kernel<MODE, MT, NT, WM, R, NW>;
    MOE_HIP(hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, TL::kLds));
    dim3 grid((unsigned)(M / MT), (unsigned)items);
    ProfScope p(name, st);
    kern<<<grid, NW * 64, TL::kLds, st>>>(a);
    return check_launch(name);
}

template <int MODE, int MT, int NT, int WM, int R, int NW>
moe_status launch_int4(const FfnArgs& a, hipStream_t st, const char* name) {
    using TL = Tile4<MT, NT, WM, R, NW>;
    const int M = (MODE == kGateUp) ? 2 * a.f : a.d;
    const int64_t items = work_items(a, NT);
    if (items > 65535) return set_error(MOE_ESHAPE, "%s: %lld token tiles exceed one launch", name, (long long)items);
    auto kern = ffn_mfma_int4_kernel<MODE, MT, NT, WM, R, NW>;
    MOE_HIP(hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, TL::kLds));
    dim3 grid((unsigned)(M / MT), (unsigned)items);
    ProfScope p(name, st);
    kern<<<grid, NW * 64, TL::kLds, st>>>(a);
    return check_launch(name);
}

}  // namespace

#ifndef MOE_MFMA_MT
#define MOE_MFMA_MT 512
#endif
#ifndef MOE_MFMA_NT
#define MOE_MFMA_NT 128
#endif
#ifndef MOE_MFMA_WM
#define MOE_MFMA_WM 8
#endif
#ifndef MOE_MFMA_R
#define MOE_MFMA_R 3
#endif
#ifndef MOE_MFMA_NW
#define MOE_MFMA_NW 8
#endif
#ifndef MOE_MFMA4_MT
#define MOE_MFMA4_MT 256
#endif
#ifndef MOE_MFMA4_R
#define MOE_MFMA4_R 4
#endif
#ifndef MOE_MFMA4_NW
#define MOE_MFMA4_NW 8
#endif
#ifndef MOE_MFMA4_WM
#define MOE_MFMA4_WM 8
#endif

// Many tokens per expert, bf16 activations, bf16 or int4 weights: the MFMA path, one projection
// (mode kGateUp or kDown).  Other cases report MOE_EDTYPE ("not mine").
moe_status ffn_mfma_proj(const FfnArgs& a, moe_dtype act, moe_dtype w, int mode, hipStream_t st) {
    constexpr int MT = MOE_MFMA_MT, NT = MOE_MFMA_NT, WM = MOE_MFMA_WM, R = MOE_MFMA_R, NW = MOE_MFMA_NW;
    if (act != MOE_BF16 || a.T <= 64) return MOE_EDTYPE;
    if (w == MOE_INT4_G128) {
        // 256 weight rows a workgroup: 2 row blocks x 8 token blocks a wave keep the accumulators,
        // the raw fragments of two groups and the dequantised operands within 256 registers
        constexpr int MT4 = MOE_MFMA4_MT, R4 = MOE_MFMA4_R, NW4 = MOE_MFMA4_NW, WM4 = MOE_MFMA4_WM;
        if ((2 * a.f) % MT4 || a.d % MT4) return MOE_EDTYPE;
        if (mode == kGateUp) return launch_int4<kGateUp, MT4, NT, WM4, R4, NW4>(a, st, "ffn_mfma_gateup_int4");
        return launch_int4<kDown, MT4, NT, WM4, R4, NW4>(a, st, "ffn_mfma_down_int4");
    }
    if (w != MOE_BF16) return MOE_EDTYPE;
    if ((2 * a.f) % MT || a.d % MT) return MOE_EDTYPE;
    if (mode == kGateUp) return launch_areg<kGateUp, MT, NT, WM, R, NW>(a, st, "ffn_mfma_gateup_bf16");
    return launch_areg<kDown, MT, NT, WM, R, NW>(a, st, "ffn_mfma_down_bf16");
}

moe_status ffn_mfma(const FfnArgs& a, moe_dtype act, moe_dtype w, hipStream_t st) {
    moe_status r = ffn_mfma_proj(a, act, w, kGateUp, st);
    if (r != MOE_OK) return r;
    return ffn_mfma_proj(a, act, w, kDown, st);
}

}  // namespace moe
