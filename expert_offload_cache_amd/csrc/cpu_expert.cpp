// Host execution of a routed expert straight from its packed slot image: the CPU side of the
// hybrid miss path (FreeToken RTX 5090 page, miss split: a miss is streamed to the GPU or run on
// the CPU, the split set by measured host and PCIe bandwidths; stork.ai article, miss policy).
//
// The image is read in the slot layout the GPU uses (16-row blocks of fragments, int4 nibbles in
// lane order, bf16 scales after the fragments), so a miss run here needs no repacking.  Arithmetic:
// binary32 accumulation; h = silu(g) * u rounded to bf16 like the GPU path, then the down rows.
// int4: per 128-input group, sum (u - 8) x over the group's nibbles u, times the group's scale.
//
// Work is split over a persistent pool of host threads (row blocks of each projection).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <condition_variable>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

#include <immintrin.h>

#include "moe_common.h"
#include "slot_layout.h"

using namespace moe;

namespace {

// ---- a persistent pool: parallel_for(n, fn) runs fn(i) for i < n on up to `threads` threads ----
class Pool {
public:
    explicit Pool(int n) {
        for (int i = 0; i < n; ++i) workers_.emplace_back([this] { loop(); });
    }
    ~Pool() {
        {
            std::lock_guard<std::mutex> g(m_);
            stop_ = true;
        }
        cv_.notify_all();
        for (auto& t : workers_) t.join();
    }
    int size() const { return (int)workers_.size() + 1; }
    void parallel_for(int n, int threads, const std::function<void(int)>& fn) {
        std::lock_guard<std::mutex> one(call_);  // one job at a time
        const int helpers = std::max(0, std::min(threads, size()) - 1);
        {
            std::lock_guard<std::mutex> g(m_);
            fn_ = &fn;
            n_ = n;
            next_.store(0);
            active_ = helpers;
            want_ = helpers;
            ++gen_;
        }
        cv_.notify_all();
        run();
        std::unique_lock<std::mutex> g(m_);
        done_cv_.wait(g, [&] { return active_ == 0; });
        fn_ = nullptr;
    }

private:
    void run() {
        for (int i; (i = next_.fetch_add(1)) < n_;) (*fn_)(i);
    }
    void loop() {
        uint64_t seen = 0;
        for (;;) {
            std::unique_lock<std::mutex> g(m_);
            cv_.wait(g, [&] { return stop_ || (gen_ != seen && want_ > 0); });
            if (stop_) return;
            seen = gen_;
            --want_;
            g.unlock();
            run();
            g.lock();
            if (--active_ == 0) done_cv_.notify_all();
        }
    }
    std::vector<std::thread> workers_;
    std::mutex m_, call_;
    std::condition_variable cv_, done_cv_;
    const std::function<void(int)>* fn_ = nullptr;
    int n_ = 0, active_ = 0, want_ = 0;
    uint64_t gen_ = 0;
    bool stop_ = false;
    std::atomic<int> next_{0};
};

Pool& pool() {
    static Pool p([] {
        const char* env = std::getenv("MOE_CPU_THREADS");
        int n = env ? std::atoi(env) : (int)std::thread::hardware_concurrency();
        return std::max(0, std::min(n, 64) - 1);
    }());
    return p;
}

inline float bf16f(uint16_t h) { return as_f32((uint32_t)h << 16); }
inline float round_bf16(float v) { return bf16f(f32_to_bf16(v)); }

// Inputs of one 128-input int4 group in the nibble order of the slot layout: lane quarter q,
// word s, nibble k (bits 4k) holds input 32 s + 8 q + (k < 4 ? 2 k : 2 (k - 4) + 1).
struct Int4Inputs {
    std::vector<float> xp;    // [groups][4 q][4 s][8 k]
    std::vector<float> gsum;  // [groups]: sum of the group's 128 inputs
    void build(const float* x, int K) {
        const int G = K / 128;
        xp.resize((size_t)G * 128);
        gsum.assign(G, 0.f);
        for (int g = 0; g < G; ++g) {
            float s_all = 0.f;
            for (int q = 0; q < 4; ++q)
                for (int s = 0; s < 4; ++s)
                    for (int k = 0; k < 8; ++k) {
                        const int j = k < 4 ? 2 * k : 2 * (k - 4) + 1;
                        const float v = x[g * 128 + 32 * s + 8 * q + j];
                        xp[(size_t)g * 128 + (q * 4 + s) * 8 + k] = v;
                        s_all += v;
                    }
            gsum[g] = s_all;
        }
    }
};

// rows 16 of one int4 block against n tokens' permuted inputs -> out[t][16]
__attribute__((target("avx2,fma"))) void int4_block_avx2(const uint8_t* blk, int K, const Int4Inputs* xin, int n,
                                                         float (*out)[16]) {
    const int G = K / 128;
    const uint16_t* scales = (const uint16_t*)(blk + (size_t)G * 1024);
    const __m256i shifts = _mm256_setr_epi32(0, 4, 8, 12, 16, 20, 24, 28);
    const __m256i mask = _mm256_set1_epi32(0xF);
    for (int t = 0; t < n; ++t) {
        __m256 tot[16];
        float corr[16];
        for (int r = 0; r < 16; ++r) {
            tot[r] = _mm256_setzero_ps();
            corr[r] = 0.f;
        }
        for (int g = 0; g < G; ++g) {
            const uint32_t* frag = (const uint32_t*)(blk + (size_t)g * 1024);
            const float* xg = xin[t].xp.data() + (size_t)g * 128;
            for (int r = 0; r < 16; ++r) {
                __m256 acc = _mm256_setzero_ps();
                for (int q = 0; q < 4; ++q) {
                    const uint32_t* w = frag + (q * 16 + r) * 4;  // lane q*16 + r: 4 words
                    for (int s = 0; s < 4; ++s) {
                        __m256i v = _mm256_and_si256(_mm256_srlv_epi32(_mm256_set1_epi32((int)w[s]), shifts), mask);
                        acc = _mm256_fmadd_ps(_mm256_cvtepi32_ps(v), _mm256_loadu_ps(xg + (q * 4 + s) * 8), acc);
                    }
                }
                const float sc = bf16f(scales[r * G + g]);
                tot[r] = _mm256_fmadd_ps(acc, _mm256_set1_ps(sc), tot[r]);
                corr[r] += sc * xin[t].gsum[g];
            }
        }
        for (int r = 0; r < 16; ++r) {
            alignas(32) float v[8];
            _mm256_store_ps(v, tot[r]);
            out[t][r] = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7])) - 8.f * corr[r];
        }
    }
}

void int4_block_scalar(const uint8_t* blk, int K, const Int4Inputs* xin, int n, float (*out)[16]) {
    const int G = K / 128;
    const uint16_t* scales = (const uint16_t*)(blk + (size_t)G * 1024);
    for (int t = 0; t < n; ++t)
        for (int r = 0; r < 16; ++r) {
            float tot = 0.f;
            for (int g = 0; g < G; ++g) {
                const uint32_t* frag = (const uint32_t*)(blk + (size_t)g * 1024);
                const float* xg = xin[t].xp.data() + (size_t)g * 128;
                float acc = 0.f;
                for (int q = 0; q < 4; ++q)
                    for (int s = 0; s < 4; ++s) {
                        const uint32_t w = frag[(q * 16 + r) * 4 + s];
                        for (int k = 0; k < 8; ++k) acc += (float)((w >> (4 * k)) & 0xF) * xg[(q * 4 + s) * 8 + k];
                    }
                const float sc = bf16f(scales[r * G + g]);
                tot += sc * (acc - 8.f * xin[t].gsum[g]);
            }
            out[t][r] = tot;
        }
}

// rows 16 of one bf16 block (fragments 16 x 32, lane l: row l%16, inputs 8(l/16)..+7)
void bf16_block(const uint8_t* blk, int K, const float* x, int n, float (*out)[16]) {
    const int nf = K / 32;
    for (int t = 0; t < n; ++t)
        for (int r = 0; r < 16; ++r) {
            float acc = 0.f;
            for (int fr = 0; fr < nf; ++fr)
                for (int q = 0; q < 4; ++q) {
                    const uint16_t* w = (const uint16_t*)(blk + (size_t)fr * 1024) + (q * 16 + r) * 8;
                    const float* xv = x + (size_t)t * K + fr * 32 + 8 * q;
                    for (int j = 0; j < 8; ++j) acc += bf16f(w[j]) * xv[j];
                }
            out[t][r] = acc;
        }
}

}  // namespace

extern "C" moe_status moe_cpu_expert_ffn(const void* slot_image, moe_dtype w, int d, int f, const void* x, int n,
                                         float* y, int threads) {
    MOE_CHECK(w == MOE_BF16 || w == MOE_INT4_G128, MOE_EDTYPE, "moe_cpu_expert_ffn: weights must be bf16 or int4");
    MOE_CHECK(slot_shape_ok(d, f, w), MOE_ESHAPE, "moe_cpu_expert_ffn: unsupported shape d=%d f=%d", d, f);
    MOE_CHECK(n >= 1 && n <= 256, MOE_ESHAPE, "moe_cpu_expert_ffn: n=%d tokens out of [1,256]", n);
    MOE_CHECK(slot_image && x && y, MOE_EINVAL, "moe_cpu_expert_ffn: NULL pointer");
    const uint8_t* img = (const uint8_t*)slot_image;
    const bool i4 = w == MOE_INT4_G128;
    const bool avx2 = __builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma");
    Pool& P = pool();
    const int nthr = threads > 0 ? threads : P.size();

    std::vector<float> xf((size_t)n * d), h((size_t)n * f);
    for (size_t i = 0; i < xf.size(); ++i) xf[i] = bf16f(((const uint16_t*)x)[i]);
    std::vector<Int4Inputs> xin(i4 ? n : 0), hin(i4 ? n : 0);
    for (int t = 0; t < (i4 ? n : 0); ++t) xin[t].build(xf.data() + (size_t)t * d, d);

    auto block = [&](const uint8_t* blk, int K, const std::vector<Int4Inputs>& in, const float* dense, float(*out)[16]) {
        if (!i4) bf16_block(blk, K, dense, n, out);
        else if (avx2) int4_block_avx2(blk, K, in.data(), n, out);
        else int4_block_scalar(blk, K, in.data(), n, out);
    };
    // gate/up: f/16 pairs of row blocks -> h (bf16-rounded, as on the GPU)
    P.parallel_for(f / 16, nthr, [&](int b) {
        std::vector<float> g16((size_t)n * 16), u16((size_t)n * 16);
        block(img + gu_block_offset(b, 0, d, w), d, xin, xf.data(), (float(*)[16])g16.data());
        block(img + gu_block_offset(b, 1, d, w), d, xin, xf.data(), (float(*)[16])u16.data());
        for (int t = 0; t < n; ++t)
            for (int r = 0; r < 16; ++r) {
                const float gv = g16[t * 16 + r], uv = u16[t * 16 + r];
                h[(size_t)t * f + b * 16 + r] = round_bf16(gv / (1.0f + std::exp(-gv)) * uv);
            }
    });
    for (int t = 0; t < (i4 ? n : 0); ++t) hin[t].build(h.data() + (size_t)t * f, f);
    // down: d/16 row blocks -> y
    P.parallel_for(d / 16, nthr, [&](int b) {
        std::vector<float> o((size_t)n * 16);
        block(img + down_block_offset(b, d, f, w), f, hin, h.data(), (float(*)[16])o.data());
        for (int t = 0; t < n; ++t)
            for (int r = 0; r < 16; ++r) y[(size_t)t * d + b * 16 + r] = o[t * 16 + r];
    });
    return MOE_OK;
}
