/*
 * ORACLE (test infrastructure only; never linked into or called by the product library).
 *
 * Router logits l[t,e] = x[t,:] . W_r[e,:] + b[e] in binary32, summed in one fixed
 * order so that the top-k selection that follows is reproducible bit for bit.
 * The pages name a router that picks a few of many experts per token (FreeToken
 * linux guide, "MoE memory handling" section) but not how its scores are summed;
 * the order below is this project's reading, and the GPU router follows it too.
 *
 * Order, for a row of length d (a multiple of 64):
 *   the row is cut into 64 contiguous segments of S = d/64 elements;
 *   segment j's sum starts at +0 and adds fl(x_i * w_i) for i = jS .. jS+S-1 in
 *   ascending order, each product and each sum rounded to nearest even (this file
 *   is built with -ffp-contract=off, so no fused multiply-add);
 *   the 64 segment sums are joined pairwise, neighbours first:
 *       level 0 = segment sums, level m+1 [i] = level m [2i] + level m [2i+1],
 *   six levels down to one value;
 *   with a bias, the logit is fl(sum + b_e).
 */
#include <stdint.h>
#include <string.h>

static inline float bf16_bits_to_f32(uint16_t h) {
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static float dot_canonical(const float* xr, const float* wr, int d) {
    int S = d / 64;
    float lvl[64];
    for (int j = 0; j < 64; ++j) {
        float a = 0.0f;
        for (int i = j * S; i < (j + 1) * S; ++i) {
            float p = xr[i] * wr[i];
            a = a + p;
        }
        lvl[j] = a;
    }
    for (int n = 32; n >= 1; n >>= 1)
        for (int i = 0; i < n; ++i) lvl[i] = lvl[2 * i] + lvl[2 * i + 1];
    return lvl[0];
}

/*
 * x: [T, d], w: [E, d], both binary32 (is_bf16 = 0) or bfloat16 bit patterns
 * (is_bf16 = 1); bias: [E] binary32 or NULL; out: [T, E] binary32.
 * Returns 0, or -1 if d is not a multiple of 64 or exceeds 16384.
 */
int oracle_router_logits(const void* x, const void* w, int is_bf16, const float* bias, int T, int d,
                         int E, float* out) {
    if (d % 64 != 0 || d > 16384 || d <= 0) return -1;
#pragma omp parallel
    {
        float xr[16384];
        float wrow[16384];
#pragma omp for schedule(static)
        for (int64_t te = 0; te < (int64_t)T * E; ++te) {
            int t = (int)(te / E), e = (int)(te % E);
            for (int i = 0; i < d; ++i) {
                if (is_bf16) {
                    xr[i] = bf16_bits_to_f32(((const uint16_t*)x)[(int64_t)t * d + i]);
                    wrow[i] = bf16_bits_to_f32(((const uint16_t*)w)[(int64_t)e * d + i]);
                } else {
                    xr[i] = ((const float*)x)[(int64_t)t * d + i];
                    wrow[i] = ((const float*)w)[(int64_t)e * d + i];
                }
            }
            float s = dot_canonical(xr, wrow, d);
            out[te] = bias ? s + bias[e] : s;
        }
    }
    return 0;
}
