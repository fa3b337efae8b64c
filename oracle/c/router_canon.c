/*
 * ORACLE (test infrastructure only; never linked into or called by the product library).
 *
 * Router logits l[t,e] = x[t,:] . W_r[e,:] + b[e] in binary32, summed in one fixed
 * order so that the top-k selection that follows is reproducible bit for bit.
 * The pages name a router that picks a few of many experts per token (FreeToken
 * linux guide, "MoE memory handling" section) but not how its scores are summed;
 * the order below is this project's reading, and the GPU router follows it too.
 *
 * Order, for a row of length d:
 *   chunk width V = 16 / sizeof(element) if d % (64 V) == 0, otherwise V = 1;
 *   element i belongs to partial sum j = (i / V) mod 64;
 *   each partial starts at +0 and adds fl(x_i * w_i) for its elements in
 *   ascending i, each product and sum rounded to nearest even (no fused
 *   multiply-add: this file is built with -ffp-contract=off);
 *   the 64 partials are combined by the butterfly a_j <- a_j + a_{j xor s}
 *   for s = 32, 16, 8, 4, 2, 1 (all j at once), and the sum is a_0;
 *   with a bias, the logit is fl(a_0 + b_e).
 */
#include <stdint.h>
#include <string.h>

static inline float bf16_bits_to_f32(uint16_t h) {
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static float dot_canonical(const float* xr, const float* wr, int d, int V) {
    float a[64];
    for (int j = 0; j < 64; ++j) a[j] = 0.0f;
    for (int i = 0; i < d; ++i) {
        int j = (i / V) % 64;
        float p = xr[i] * wr[i];
        a[j] = a[j] + p;
    }
    for (int s = 32; s >= 1; s >>= 1) {
        float b[64];
        for (int j = 0; j < 64; ++j) b[j] = a[j] + a[j ^ s];
        memcpy(a, b, sizeof(a));
    }
    return a[0];
}

/*
 * x: [T, d], w: [E, d], both binary32 (is_bf16 = 0) or bfloat16 bit patterns
 * (is_bf16 = 1); bias: [E] binary32 or NULL; out: [T, E] binary32.
 */
void oracle_router_logits(const void* x, const void* w, int is_bf16, const float* bias, int T, int d,
                          int E, float* out) {
    int esize = is_bf16 ? 2 : 4;
    int V = 16 / esize;
    if (d % (64 * V) != 0) V = 1;
    if (d > 16384) return; /* rows are staged on the stack */
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
            float s = dot_canonical(xr, wrow, d, V);
            out[te] = bias ? s + bias[e] : s;
        }
    }
}
