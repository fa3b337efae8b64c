/*
 * Seeded synthetic-input generator (inputs only: no step of the MoE layer is
 * computed here).
 *
 * Every tensor is a pure function of (seed, stream, element index), so any
 * expert of any layer can be regenerated on its own and in any order.
 *
 * Uniform source: the SplitMix64 sequence (Steele, Lea, Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014).  A stream starts
 * at state0 = mix(seed ^ mix(stream + STREAM_SALT)); output c of the stream is
 * mix(state0 + (c + 1) * GOLDEN).
 *
 * Gaussian shape: the Irwin-Hall construction (sum of twelve uniforms minus
 * six).  Element i uses outputs 3i, 3i+1, 3i+2; each 64-bit output is split
 * into four 16-bit integers u, S = sum of the twelve, and
 *     z = (S - 393210) / 65536            (exact in float and double)
 * which has mean 0 and variance 1 - 2^-32, supported on [-6, 6].  The value
 * handed out is w = fl32(z * fl32(sigma)), optionally rounded to bfloat16 with
 * round-to-nearest-even.  All steps are integer or exactly-rounded IEEE
 * operations, so the bits do not depend on the compiler or the libm.
 *
 * int4 weights: per output row, groups of 128 consecutive inputs,
 *     s = bf16_rne(max|w| / 7),  q = clamp(round_half_even(w / s), -7, 7),
 * stored offset-binary (q + 8) with element 2i in the low nibble of byte i and
 * element 2i+1 in the high nibble; scales are bfloat16 bit patterns.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL
#define STREAM_SALT 0x632BE59BD9B4E019ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t stream_state(uint64_t seed, uint64_t stream) {
    return mix64(seed ^ mix64(stream + STREAM_SALT));
}

static inline uint64_t stream_out(uint64_t state0, uint64_t c) {
    return mix64(state0 + (c + 1) * GOLDEN);
}

static inline float irwin_hall(uint64_t state0, uint64_t i) {
    uint64_t s = 0;
    for (int j = 0; j < 3; ++j) {
        uint64_t r = stream_out(state0, 3 * i + (uint64_t)j);
        s += (r & 0xFFFF) + ((r >> 16) & 0xFFFF) + ((r >> 32) & 0xFFFF) + (r >> 48);
    }
    /* s <= 786420 < 2^24: the subtraction and the power-of-two division are exact */
    return ((float)((int64_t)s - 393210)) / 65536.0f;
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40); /* quiet NaN */
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

static inline float bf16_to_f32(uint16_t h) {
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* out[i] = fl32(z_{start+i} * sigma) */
void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t start, int64_t n, float sigma,
                      float* out) {
    uint64_t st = stream_state(seed, stream);
#pragma omp parallel for schedule(static) if (n > 65536)
    for (int64_t i = 0; i < n; ++i) out[i] = irwin_hall(st, start + (uint64_t)i) * sigma;
}

/* out[i] = bf16_rne(fl32(z_{start+i} * sigma)) as raw bits */
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t start, int64_t n, float sigma,
                       uint16_t* out) {
    uint64_t st = stream_state(seed, stream);
#pragma omp parallel for schedule(static) if (n > 65536)
    for (int64_t i = 0; i < n; ++i)
        out[i] = f32_to_bf16_rne(irwin_hall(st, start + (uint64_t)i) * sigma);
}

/* Raw 64-bit outputs c = start .. start+n-1 of a stream (for tests of the definition). */
void synth_raw_u64(uint64_t seed, uint64_t stream, uint64_t start, int64_t n, uint64_t* out) {
    uint64_t st = stream_state(seed, stream);
    for (int64_t i = 0; i < n; ++i) out[i] = stream_out(st, start + (uint64_t)i);
}

/* round half to even of a float to an integer-valued float */
static inline float rint_even(float v) { return nearbyintf(v); /* default FE_TONEAREST */ }

/*
 * Quantise one [rows, K] matrix (K % 128 == 0) to symmetric int4 with bf16
 * group scales.  w may be NULL, in which case the matrix is generated from
 * (seed, stream) with the given sigma and never stored in full.
 * packed: [rows][K/2] bytes; scales: [rows][K/128] bf16 bits.
 */
void synth_quant_int4(const float* w, uint64_t seed, uint64_t stream, float sigma, int64_t rows,
                      int64_t K, uint8_t* packed, uint16_t* scales) {
    uint64_t st = stream_state(seed, stream);
    int64_t G = K / 128;
#pragma omp parallel for schedule(static) if (rows * K > 65536)
    for (int64_t r = 0; r < rows; ++r) {
        float buf[128];
        for (int64_t g = 0; g < G; ++g) {
            float amax = 0.0f;
            for (int j = 0; j < 128; ++j) {
                int64_t idx = r * K + g * 128 + j;
                float v = w ? w[idx] : irwin_hall(st, (uint64_t)idx) * sigma;
                buf[j] = v;
                float a = fabsf(v);
                if (a > amax) amax = a;
            }
            uint16_t sb = f32_to_bf16_rne(amax / 7.0f);
            float s = bf16_to_f32(sb);
            scales[r * G + g] = sb;
            for (int j = 0; j < 128; j += 2) {
                int q[2];
                for (int h = 0; h < 2; ++h) {
                    float qq = (s == 0.0f) ? 0.0f : rint_even(buf[j + h] / s);
                    if (qq > 7.0f) qq = 7.0f;
                    if (qq < -7.0f) qq = -7.0f;
                    q[h] = (int)qq + 8;
                }
                packed[r * (K / 2) + (g * 128 + j) / 2] = (uint8_t)(q[0] | (q[1] << 4));
            }
        }
    }
}
