// moe_route: router logits in one fixed binary32 order, top-k selection, renormalised gates.
//
// The pages (FreeToken linux guide, "MoE memory handling") state only that a router activates
// a few experts per token.  The summation order is this library's reading, chosen so that the
// selected ids are reproducible bit for bit: 64 contiguous segments of d/64 elements, each
// summed from +0 in ascending index, joined pairwise neighbours first, bias added last.
//
// Two logits paths implement that one order:
//   * few tokens (decode): one wave per (token, expert); lane j owns segment j, and the pairwise
//     join is a butterfly with strides 1, 2, 4, ..., 32 done in VALU (DPP and permlane swaps;
//     a + b == b + a, so both lanes of a pair hold the same bits);
//   * many tokens (prefill), bf16 with d a multiple of 2048: 32 tokens x 32 experts per block;
//     each of the four waves owns one quarter of the inputs, i.e. 16 consecutive segments = one
//     depth-4 subtree of the join, which it runs segment after segment with a binary-counter
//     stack; the four subtree roots are then joined (0+1)+(2+3) through LDS;
//   * other prefill shapes: an LDS-tiled VALU product, each thread owning 4 tokens x 4
//     experts, running all 64 segments with a 6-level binary-counter stack.
// A second kernel selects and gates, one block per token.
// Selection is by rank: expert e is chosen iff fewer than k experts beat it (larger logit, or
// equal logit and lower id), and that count is its output position.
// moe_route_permute runs the same logits kernels; for one token a single block then selects,
// gates and sorts (moe_permute's counting sort), which saves a launch.
#include <hip/hip_runtime.h>

#include "moe_common.h"
#include "select_permute.h"

#include <algorithm>

namespace moe {
namespace {

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
    const int tb = blockIdx.x * kTT, eb = blockIdx.y * kTE;
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
                const int n = seg_idx++;
                bool carry = true;  // still joining upwards
#pragma unroll
                for (int lv = 0; lv < 6; ++lv) {
                    if (carry) {
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
                            carry = false;
                        }
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

// ---- prefill logits, bf16, d % 2048 == 0: four waves split the inputs by subtree -----------------
// Block (bx, by): tokens 32*bx .. +31, experts 32*by .. +31.  Lane (tx = l&7, ty = l>>3) owns
// tokens ty + 8a and experts tx + 8b (a, b < 4).  Inputs move in chunks of 32 per wave: global
// 16-byte loads (the next chunk's are issued before the current chunk is multiplied), widened to
// binary32 once while staged, then read back as float4 so one LDS read serves four steps.
constexpr int kSplitRow = 36;  // padded LDS row (floats): the 8 rows one read touches hit distinct banks

// Orders a wave's own LDS writes and reads (its lanes read rows other lanes of the wave staged); the
// waves of a block stage into separate areas, so they need not meet there (a block barrier per
// chunk instead measured 6-9 % slower, same bits).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ void widen_store(float* dst, u32x4_t v) {
    float4 lo = make_float4(as_f32(v.x << 16), as_f32(v.x & 0xFFFF0000u), as_f32(v.y << 16), as_f32(v.y & 0xFFFF0000u));
    float4 hi = make_float4(as_f32(v.z << 16), as_f32(v.z & 0xFFFF0000u), as_f32(v.w << 16), as_f32(v.w & 0xFFFF0000u));
    *(float4*)dst = lo;
    *(float4*)(dst + 4) = hi;
}

__global__ __launch_bounds__(256) void route_logits_split(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ w,
                                                          const float* __restrict__ bias, int T, int d,
                                                          int E, float* __restrict__ logits) {
    __shared__ __align__(16) float lds[4][2][32][kSplitRow];  // per wave: x rows, w rows
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tx = lane & 7, ty = lane >> 3;
    const int t0 = blockIdx.x * 32, e0 = blockIdx.y * 32;
    const int quarter = d / 4, nch = quarter / 32, cps = d / 64 / 32;  // chunks; chunks per segment

    // staging: vectors v = lane + 64u (u < 2) -> row v>>2, inputs 8*(v&3)..+7 of the chunk
    const uint16_t* xsrc[2];
    const uint16_t* wsrc[2];
    int srow[2], spart[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int v = lane + 64 * u;
        srow[u] = v >> 2;
        spart[u] = v & 3;
        const int t = min(t0 + srow[u], T - 1), e = min(e0 + srow[u], E - 1);  // tails: any valid row
        xsrc[u] = x + (size_t)t * d + wv * quarter + spart[u] * 8;
        wsrc[u] = w + (size_t)e * d + wv * quarter + spart[u] * 8;
    }
    float(*xs)[kSplitRow] = lds[wv][0];
    float(*ws)[kSplitRow] = lds[wv][1];

    u32x4_t gx[2], gw[2];
    auto gload = [&](int ch) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            gx[u] = *(const u32x4_t*)(xsrc[u] + ch * 32);
            gw[u] = *(const u32x4_t*)(wsrc[u] + ch * 32);
        }
    };
    auto sstore = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            widen_store(&xs[srow[u]][spart[u] * 8], gx[u]);
            widen_store(&ws[srow[u]][spart[u] * 8], gw[u]);
        }
    };

    float acc[4][4], stk[4][4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = 0.f;

    gload(0);
    sstore();
    wave_lds_sync();
    for (int ch = 0; ch < nch; ++ch) {
        gload(min(ch + 1, nch - 1));
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            float4 xv[4], wq[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) xv[a] = *(const float4*)&xs[ty + 8 * a][4 * g];
#pragma unroll
            for (int b = 0; b < 4; ++b) wq[b] = *(const float4*)&ws[tx + 8 * b][4 * g];
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    float s = acc[a][b];
                    s = madd<true>(s, xv[a].x, wq[b].x);
                    s = madd<true>(s, xv[a].y, wq[b].y);
                    s = madd<true>(s, xv[a].z, wq[b].z);
                    s = madd<true>(s, xv[a].w, wq[b].w);
                    acc[a][b] = s;
                }
        }
        if ((ch + 1) % cps == 0) {
            // close local segment n (0..15): binary-counter join, left sibling + right
            const int n = (ch + 1) / cps - 1;
            bool carry = true;
#pragma unroll
            for (int lv = 0; lv < 4; ++lv) {
                if (carry) {
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
                        carry = false;
                    }
                }
            }
            if (n != 15) {
#pragma unroll
                for (int a = 0; a < 4; ++a)
#pragma unroll
                    for (int b = 0; b < 4; ++b) acc[a][b] = 0.f;
            }
        }
        wave_lds_sync();
        sstore();
        wave_lds_sync();
    }
    __syncthreads();  // the join below reuses every wave's staging area
    // acc = this wave's subtree root.  Join the four: (q0 + q1) + (q2 + q3), then the bias.
    float* part = &lds[0][0][0][0];  // [4 waves][32 tokens][32 experts], staging no longer needed
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) part[(wv * 32 + ty + 8 * a) * 32 + tx + 8 * b] = acc[a][b];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int o = tid + 256 * i, tl = o >> 5, el = o & 31;
        const int t = t0 + tl, e = e0 + el;
        const float l = (part[o] + part[1024 + o]) + (part[2048 + o] + part[3072 + o]);
        if (t < T && e < E) logits[(size_t)t * E + e] = bias ? l + bias[e] : l;
    }
}

// ---- top-k and gates: rank selection on one token's logits held in LDS ------------------------
// rank(e) = number of experts that beat e (larger logit, or equal logit and lower id); the
// selected experts are those with rank < k and rank is their output position, so every thread
// finds its own answer without a chain of cross-lane reductions.
__device__ void select_and_gate(const float* s_logit, int E, int k, const int32_t* forced_row, int* s_sel,
                                float* s_val, int32_t* idx_out, float* w_out) {
    const int tid = threadIdx.x, nth = blockDim.x;
    if (forced_row) {
        for (int j = tid; j < k; j += nth) {
            const int id = forced_row[j];
            s_sel[j] = id;
            s_val[j] = s_logit[min(max(id, 0), E - 1)];
        }
    } else {
        // P adjacent lanes share an expert, each counting the experts i = p (mod P) that beat it;
        // the partial counts are summed over the P lanes
        const int P = nth >= 4 * E ? 4 : nth >= 2 * E ? 2 : 1;
        // with E a multiple of 4P each lane takes a contiguous quarter (or half, or all) of the
        // experts and reads them four at a time: a quarter of the LDS reads, which bound this loop
        // (s_logit is 16-byte aligned)
        const bool vec = E % (4 * P) == 0;
        const int span = E / P;
        for (int b = tid; b < E * P; b += nth) {
            const int e = b / P, p = b - e * P;
            const float v = s_logit[e];
            int r = 0;
            // unrolled so that the LDS reads issue back to back (an integer count: order-free)
            if (vec) {
                const float4* s4 = (const float4*)(s_logit + p * span);
#pragma unroll 4
                for (int c = 0; c < span / 4; ++c) {
                    const float4 q = s4[c];
                    const int i = p * span + 4 * c;
                    r += better(q.x, i, v, e) + better(q.y, i + 1, v, e) + better(q.z, i + 2, v, e) +
                         better(q.w, i + 3, v, e);
                }
            } else {
#pragma unroll 8
                for (int i = p; i < E; i += P) r += better(s_logit[i], i, v, e);
            }
            if (P >= 2) r += __shfl_xor(r, 1, 64);
            if (P >= 4) r += __shfl_xor(r, 2, 64);
            if (p == 0 && r < k) {
                s_sel[r] = e;
                s_val[r] = v;
            }
        }
    }
    __syncthreads();
    // gates: softmax over the selected logits in binary64, rounded once.  Thread j forms its own
    // term exp(v_j - max) once; every thread then sums the k terms in ascending order.
    __shared__ double s_term[1024];
    double m = -INFINITY;
#pragma unroll 8
    for (int i = 0; i < k; ++i) m = fmax(m, (double)s_val[i]);
    for (int j = tid; j < k; j += nth) s_term[j] = exp((double)s_val[j] - m);
    __syncthreads();
    for (int j = tid; j < k; j += nth) {
        double den = 0.0;
#pragma unroll 8
        for (int i = 0; i < k; ++i) den += s_term[i];
        idx_out[j] = s_sel[j];
        w_out[j] = (float)(s_term[j] / den);
    }
}

// one block per token, logits already in global memory
// above this many tokens the wave-per-token selection (route_topk_wave) runs instead
constexpr int kWaveTopkMinT = 64;

__global__ __launch_bounds__(1024) void route_topk(const float* __restrict__ logits, int T, int E, int k,
                                                  const int32_t* __restrict__ forced,
                                                  int32_t* __restrict__ topk_idx,
                                                  float* __restrict__ topk_w) {
    __shared__ __align__(16) float s_logit[1024];
    __shared__ int s_sel[1024];
    __shared__ float s_val[1024];
    const int t = blockIdx.x;
    for (int e = threadIdx.x; e < E; e += blockDim.x) s_logit[e] = logits[(size_t)t * E + e];
    __syncthreads();
    select_and_gate(s_logit, E, k, forced ? forced + (size_t)t * k : nullptr, s_sel, s_val,
                    topk_idx + (size_t)t * k, topk_w + (size_t)t * k);
}

// Many tokens (prefill): one wave per token, four tokens a workgroup.  The wave holds the token's
// logits, EPL a lane (lane l: experts l, l + 64, ...), and takes the k best in k rounds: each lane
// proposes its best expert not yet taken, a butterfly over the 64 lanes keeps the better of each
// pair (larger logit, equal logits -> lower id: `better`, a strict total order, so every lane ends
// with the same winner), lane r keeps round r's winner and its owner marks it taken.  Round r's
// winner is the expert ranked r, so the ids are route_topk's.  Gates as select_and_gate: lane j forms
// exp(v_j - max) in binary64, every lane sums the k terms in ascending j, one rounding.  Needs
// k <= 64.  A block per token keeps its barriers and a thousand threads busy for one selection;
// here one wave does it without LDS or barriers, which is what a batch of thousands of tokens needs.
template <int EPL>
__global__ __launch_bounds__(256) void route_topk_wave(const float* __restrict__ logits, int T, int E, int k,
                                                       const int32_t* __restrict__ forced,
                                                       int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;  // the whole wave
    const float* row = logits + (size_t)t * E;
    int sel_id = 0;
    float sel_v = 0.f;
    if (forced) {
        if (lane < k) {
            sel_id = forced[(size_t)t * k + lane];
            sel_v = row[min(max(sel_id, 0), E - 1)];
        }
    } else {
        float v[EPL];
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + 64 * i;
            v[i] = e < E ? row[e] : 0.f;
        }
        uint32_t taken = 0;
        for (int r = 0; r < k; ++r) {
            float bv = 0.f;
            int bi = -1;  // -1: no candidate
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                const int e = lane + 64 * i;
                if (e < E && !((taken >> i) & 1u) && (bi < 0 || better(v[i], e, bv, bi))) {
                    bv = v[i];
                    bi = e;
                }
            }
#pragma unroll
            for (int sh = 1; sh < 64; sh <<= 1) {
                const float ov = __shfl_xor(bv, sh, 64);
                const int oi = __shfl_xor(bi, sh, 64);
                if (oi >= 0 && (bi < 0 || better(ov, oi, bv, bi))) {
                    bv = ov;
                    bi = oi;
                }
            }
            if (lane == r) {
                sel_id = bi;
                sel_v = bv;
            }
            if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
        }
    }
    double m = -INFINITY;
    for (int i = 0; i < k; ++i) m = fmax(m, (double)__shfl(sel_v, i, 64));
    const double term = lane < k ? exp((double)sel_v - m) : 0.0;
    double den = 0.0;
    for (int i = 0; i < k; ++i) den += __shfl(term, i, 64);
    if (lane < k) {
        topk_idx[(size_t)t * k + lane] = sel_id;
        topk_w[(size_t)t * k + lane] = (float)(term / den);
    }
}

// For one token (batch-1 decode) one block selects and gates (select_and_gate, as route_topk) and
// then places the token's k pairs by expert straight from the selected ids: expert e's count is the
// number of pairs with id e, its offset the number of pairs with a smaller id, and pair j's sorted
// position the number of pairs before it in (id, j) order -- the stable counting sort's result for
// one token, without its passes.  One launch instead of two.  (A sort by the last of route_topk's
// blocks would need a device-scope release and acquire, which write back and invalidate an XCD's
// L2.)  Ids are clamped into [0, E) for the placement, as in moe_permute.
//
// `publish` (or NULL): coherent host memory that also receives the k ids, stored with system scope
// so that a host thread polling it sees them without a copy (the native decode steps' read-back).
__global__ __launch_bounds__(1024) void route_topk_permute1(const float* __restrict__ logits, int E, int k,
                                                           const int32_t* __restrict__ forced,
                                                           int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                                                           int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm,
                                                           int32_t* __restrict__ publish) {
    __shared__ __align__(16) float s_logit[1024];
    __shared__ int s_sel[1024];
    __shared__ float s_val[1024];
    const int tid = threadIdx.x, nth = blockDim.x;
    for (int e = tid; e < E; e += nth) s_logit[e] = logits[e];
    __syncthreads();
    // s_sel is complete after the barrier inside (nothing writes it afterwards)
    select_and_gate(s_logit, E, k, forced, s_sel, s_val, topk_idx, topk_w);
    if (publish)
        for (int j = tid; j < k; j += nth) __hip_atomic_store(publish + j, s_sel[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    for (int e = tid; e < E; e += nth) {
        int c = 0, o = 0;
        for (int j = 0; j < k; ++j) {
            const int id = min(max(s_sel[j], 0), E - 1);
            c += id == e;
            o += id < e;
        }
        counts[e] = c;
        offsets[e] = o;
    }
    if (tid == 0) offsets[E] = k;
    for (int j = tid; j < k; j += nth) {
        const int idj = min(max(s_sel[j], 0), E - 1);
        int pos = 0;
        for (int i = 0; i < k; ++i) {
            const int idi = min(max(s_sel[i], 0), E - 1);
            pos += idi < idj || (idi == idj && i < j);
        }
        perm[pos] = j;
        inv_perm[j] = pos;
    }
}

// decode: one wave per (token, expert); lane j owns segment j of the row, issues all of its
// loads first, sums its segment in ascending index, and the wave joins the 64 segment sums with
// the neighbours-first butterfly.
template <bool kBf16>
__global__ __launch_bounds__(256) void route_logits_wave(const void* __restrict__ x, const void* __restrict__ w,
                                                         const float* __restrict__ bias, int T, int d, int E,
                                                         float* __restrict__ logits) {
    const int lane = threadIdx.x & 63;
    const long g = (long)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (g >= (long)T * E) return;
    const int t = (int)(g / E), e = (int)(g - (long)t * E);
    const int S = d / 64;
    const size_t seg = (size_t)lane * S;
    float acc = 0.f;
    if (kBf16 && S % 8 == 0 && S <= 128) {
        const uint4* xr = (const uint4*)((const uint16_t*)x + (size_t)t * d + seg);
        const uint4* wr = (const uint4*)((const uint16_t*)w + (size_t)e * d + seg);
        const int nv = S / 8;
        uint4 xv[16], wv[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            xv[c] = (c < nv) ? xr[c] : make_uint4(0, 0, 0, 0);
            wv[c] = (c < nv) ? wr[c] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            if (c < nv) {
                const uint32_t xs[4] = {xv[c].x, xv[c].y, xv[c].z, xv[c].w};
                const uint32_t ws[4] = {wv[c].x, wv[c].y, wv[c].z, wv[c].w};
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    acc = madd<true>(acc, bf16_lo(xs[h]), bf16_lo(ws[h]));
                    acc = madd<true>(acc, bf16_hi(xs[h]), bf16_hi(ws[h]));
                }
            }
        }
    } else {
        for (int i = 0; i < S; ++i)
            acc = madd<kBf16>(acc, load_elem<kBf16>(x, (size_t)t * d + seg + i),
                              load_elem<kBf16>(w, (size_t)e * d + seg + i));
    }
    acc = wave_tree_sum(acc);
    if (lane == 0) logits[(size_t)t * E + e] = bias ? acc + bias[e] : acc;
}

// decode, bf16: one wave per tile of TB tokens x EB experts.  Lane j owns segment j of every
// row of the tile, so each activation and router row is read once per tile instead of once per
// (token, expert) pair; every logit still sums its segment in ascending index and joins the 64
// segment sums with the neighbours-first butterfly, the order of route_logits_wave.
template <int TB, int EB, int CG>
__global__ __launch_bounds__(256) void route_logits_wave_tile(const uint16_t* __restrict__ x,
                                                              const uint16_t* __restrict__ w,
                                                              const float* __restrict__ bias, int T, int d, int E,
                                                              float* __restrict__ logits) {
    const int lane = threadIdx.x & 63;
    const int ntt = (T + TB - 1) / TB, nte = (E + EB - 1) / EB;
    const long g = (long)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (g >= (long)ntt * nte) return;
    const int t0 = (int)(g / nte) * TB, e0 = (int)(g % nte) * EB;
    const int S = d / 64;  // segment length, a multiple of 8 (checked by the caller)
    const int nv = S / 8;
    const size_t seg = (size_t)lane * S;
    const uint4* xr[TB];
    const uint4* wr[EB];
#pragma unroll
    for (int i = 0; i < TB; ++i) xr[i] = (const uint4*)(x + (size_t)min(t0 + i, T - 1) * d + seg);
#pragma unroll
    for (int j = 0; j < EB; ++j) wr[j] = (const uint4*)(w + (size_t)min(e0 + j, E - 1) * d + seg);
    float acc[TB][EB];
#pragma unroll
    for (int i = 0; i < TB; ++i)
#pragma unroll
        for (int j = 0; j < EB; ++j) acc[i][j] = 0.f;
    // chunks of 8 inputs, CG at a time: issue the group's loads, then the products in index order
    for (int c0 = 0; c0 < nv; c0 += CG) {
        uint4 xv[CG][TB], wv[CG][EB];
#pragma unroll
        for (int c = 0; c < CG; ++c) {
            const int cc = min(c0 + c, nv - 1);
#pragma unroll
            for (int i = 0; i < TB; ++i) xv[c][i] = xr[i][cc];
#pragma unroll
            for (int j = 0; j < EB; ++j) wv[c][j] = wr[j][cc];
        }
#pragma unroll
        for (int c = 0; c < CG; ++c) {
            if (c0 + c < nv) {
#pragma unroll
                for (int h = 0; h < 4; ++h) {
#pragma unroll
                    for (int i = 0; i < TB; ++i) {
                        const uint32_t xs = h == 0 ? xv[c][i].x : h == 1 ? xv[c][i].y : h == 2 ? xv[c][i].z : xv[c][i].w;
#pragma unroll
                        for (int j = 0; j < EB; ++j) {
                            const uint32_t ws = h == 0 ? wv[c][j].x : h == 1 ? wv[c][j].y : h == 2 ? wv[c][j].z : wv[c][j].w;
                            acc[i][j] = madd<true>(acc[i][j], bf16_lo(xs), bf16_lo(ws));
                            acc[i][j] = madd<true>(acc[i][j], bf16_hi(xs), bf16_hi(ws));
                        }
                    }
                }
            }
        }
    }
    // join each logit's 64 segment sums; lane i * EB + j writes logit (t0 + i, e0 + j)
    float out = 0.f;
#pragma unroll
    for (int i = 0; i < TB; ++i)
#pragma unroll
        for (int j = 0; j < EB; ++j) {
            const float v = wave_tree_sum(acc[i][j]);
            if (lane == i * EB + j) out = v;
        }
    const int i = lane / EB, j = lane % EB;
    if (lane < TB * EB && t0 + i < T && e0 + j < E) {
        const int e = e0 + j;
        logits[(size_t)(t0 + i) * E + e] = bias ? out + bias[e] : out;
    }
}

moe_status check_route_args(const char* fn, const void* x, moe_dtype act, int T, int d, const void* w_router,
                             int E, int k, const void* topk_idx, const void* topk_w, const void* logits) {
    MOE_CHECK(act == MOE_F32 || act == MOE_BF16, MOE_EDTYPE, "%s: activations must be F32 or BF16", fn);
    MOE_CHECK(E >= 1 && E <= 1024 && k >= 1 && k <= E, MOE_ESHAPE, "%s: need 1 <= k <= E <= 1024 (k=%d E=%d)", fn,
              k, E);
    MOE_CHECK(d >= 64 && d <= 16384 && d % 64 == 0, MOE_ESHAPE, "%s: d=%d must be a multiple of 64 in [64,16384]",
              fn, d);
    MOE_CHECK(x && w_router && topk_idx && topk_w && logits, MOE_EINVAL, "%s: NULL pointer", fn);
    MOE_CHECK(T <= (1 << 24), MOE_ESHAPE, "%s: T=%d too large", fn, T);
    return MOE_OK;
}

moe_status launch_route_logits(const void* x, bool bf, int T, int d, const void* w_router, const float* bias,
                               int E, float* logits, hipStream_t st) {
    if (T >= 32 && T <= 64 && bf && d <= 2048 && (d / 64) % 8 == 0 && E >= 4) {
        // 4 tokens x 2 experts a wave (measured faster than one wave a pair and than 4 x 4 tiles
        // at 64 tokens and d <= 2048; slower at 4-16 tokens or wider rows, where the pair-per-wave
        // kernel has more waves)
        const long tiles = (long)((T + 3) / 4) * ((E + 1) / 2);
        ProfScope p("route_logits_wave", st);
        route_logits_wave_tile<4, 2, 4><<<(unsigned)((tiles + 3) / 4), 256, 0, st>>>(
            (const uint16_t*)x, (const uint16_t*)w_router, bias, T, d, E, logits);
    } else if (T <= 64) {
        const long waves = (long)T * E;
        ProfScope p("route_logits_wave", st);
        if (bf) route_logits_wave<true><<<(unsigned)((waves + 3) / 4), 256, 0, st>>>(x, w_router, bias, T, d, E, logits);
        else route_logits_wave<false><<<(unsigned)((waves + 3) / 4), 256, 0, st>>>(x, w_router, bias, T, d, E, logits);
    } else if (bf && d % 2048 == 0 && (((uintptr_t)x | (uintptr_t)w_router) & 15) == 0) {
        dim3 grid((unsigned)((T + 31) / 32), (unsigned)((E + 31) / 32));
        ProfScope p("route_logits_split", st);
        route_logits_split<<<grid, 256, 0, st>>>((const uint16_t*)x, (const uint16_t*)w_router, bias, T, d, E, logits);
    } else {
        dim3 grid((unsigned)((T + kTT - 1) / kTT), (unsigned)((E + kTE - 1) / kTE));
        ProfScope p("route_logits_tiled", st);
        if (bf) route_logits_tiled<true><<<grid, 256, 0, st>>>(x, w_router, bias, T, d, E, logits);
        else route_logits_tiled<false><<<grid, 256, 0, st>>>(x, w_router, bias, T, d, E, logits);
    }
    return check_launch("route_logits");
}

moe_status launch_route_topk(const float* logits, int T, int E, int k, const int32_t* forced_idx,
                             int32_t* topk_idx, float* topk_w, hipStream_t st) {
    ProfScope p("route_topk", st);
    if (T > kWaveTopkMinT && k <= 64) {
        // many tokens: a wave per token (E <= 1024 holds 16 logits a lane at most)
        const unsigned blocks = (unsigned)((T + 3) / 4);
#define RTW(N) route_topk_wave<N><<<blocks, 256, 0, st>>>(logits, T, E, k, forced_idx, topk_idx, topk_w)
        if (E <= 64) RTW(1);
        else if (E <= 128) RTW(2);
        else if (E <= 256) RTW(4);
        else if (E <= 512) RTW(8);
        else RTW(16);
#undef RTW
        return check_launch("route_topk");
    }
    // up to 4 threads per expert share its comparisons
    const int nth = std::min(1024, std::max(64, (E * 4 + 63) / 64 * 64));
    route_topk<<<T, nth, 0, st>>>(logits, T, E, k, forced_idx, topk_idx, topk_w);
    return check_launch("route_topk");
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_route(const void* x, moe_dtype act, int T, int d, const void* w_router,
                                const float* bias, int E, int k, const int32_t* forced_idx,
                                int32_t* topk_idx, float* topk_w, float* logits, moe_stream s) {
    MOE_CHECK(T >= 0, MOE_ESHAPE, "moe_route: T=%d < 0", T);
    if (T == 0) return MOE_OK;
    moe_status r = check_route_args("moe_route", x, act, T, d, w_router, E, k, topk_idx, topk_w, logits);
    if (r != MOE_OK) return r;
    hipStream_t st = (hipStream_t)s;
    r = launch_route_logits(x, act == MOE_BF16, T, d, w_router, bias, E, logits, st);
    if (r != MOE_OK) return r;
    return launch_route_topk(logits, T, E, k, forced_idx, topk_idx, topk_w, st);
}

namespace moe {
// moe_route_permute; at T = 1 the ids also go to `publish` (coherent host memory, or NULL)
moe_status route_permute_publish(const void* x, moe_dtype act, int T, int d, const void* w_router, const float* bias,
                                 int E, int k, const int32_t* forced_idx, int32_t* topk_idx, float* topk_w,
                                 float* logits, int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                                 void* ws, size_t ws_bytes, int32_t* publish, moe_stream s) {
    MOE_CHECK(T >= 0, MOE_ESHAPE, "moe_route_permute: T=%d < 0", T);
    if (T == 0) return moe_permute(nullptr, 0, k, E, counts, offsets, perm, inv_perm, nullptr, 0, s);
    moe_status r = check_route_args("moe_route_permute", x, act, T, d, w_router, E, k, topk_idx, topk_w, logits);
    if (r != MOE_OK) return r;
    MOE_CHECK((int64_t)T * k <= (1 << 24), MOE_ESHAPE, "moe_route_permute: T*k too large");
    MOE_CHECK(counts && offsets && perm && inv_perm, MOE_EINVAL, "moe_route_permute: NULL pointer");
    hipStream_t st = (hipStream_t)s;
    r = launch_route_logits(x, act == MOE_BF16, T, d, w_router, bias, E, logits, st);
    if (r != MOE_OK) return r;
    if (T > 1) {
        r = launch_route_topk(logits, T, E, k, forced_idx, topk_idx, topk_w, st);
        if (r != MOE_OK) return r;
        return moe_permute(topk_idx, T, k, E, counts, offsets, perm, inv_perm, ws, ws_bytes, s);
    }
    // one token: the top-k block's threads, a power of two with 4 threads an expert (as route_topk)
    int nth = 64;
    while (nth < 1024 && nth < 4 * E) nth *= 2;
    ProfScope p("route_topk_permute", st);
    route_topk_permute1<<<1, nth, 0, st>>>(logits, E, k, forced_idx, topk_idx, topk_w, counts, offsets, perm,
                                           inv_perm, publish);
    return check_launch("route_topk_permute");
}
}  // namespace moe

extern "C" moe_status moe_route_permute(const void* x, moe_dtype act, int T, int d, const void* w_router,
                                        const float* bias, int E, int k, const int32_t* forced_idx,
                                        int32_t* topk_idx, float* topk_w, float* logits, int32_t* counts,
                                        int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* ws,
                                        size_t ws_bytes, moe_stream s) {
    return route_permute_publish(x, act, T, d, w_router, bias, E, k, forced_idx, topk_idx, topk_w, logits, counts,
                                 offsets, perm, inv_perm, ws, ws_bytes, nullptr, s);
}
