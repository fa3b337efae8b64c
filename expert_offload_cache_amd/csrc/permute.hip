// moe_permute: stable counting sort of the T*k (token, choice) pairs by expert id.
//
// The pages do not describe this step; the plain reading is a counting sort of the flat pair
// ids t*k + j, stable within an expert, done by one workgroup without atomics on positions
// (permute_block in select_permute.h), so the result is deterministic.
#include <hip/hip_runtime.h>

#include "moe_common.h"
#include "select_permute.h"

namespace moe {
namespace {

constexpr int kMaxE = kPermMaxE;

template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void permute_kernel(const int32_t* __restrict__ ids, int N, int E,
                                                             int nbits, int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ perm,
                                                             int32_t* __restrict__ inv_perm) {
    __shared__ int32_t run[WAVES * kMaxE];
    __shared__ int32_t s_wave[WAVES];
    permute_block<WAVES>(ids, N, E, nbits, counts, offsets, perm, inv_perm, run, s_wave);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_permute(const int32_t* topk_idx, int T, int k, int E, int32_t* counts,
                                  int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* ws,
                                  size_t ws_bytes, moe_stream s) {
    (void)ws;
    (void)ws_bytes;
    MOE_CHECK(T >= 0 && k >= 1 && E >= 1 && E <= kMaxE && k <= E, MOE_ESHAPE,
              "moe_permute: need T >= 0, 1 <= k <= E <= %d (T=%d k=%d E=%d)", kMaxE, T, k, E);
    MOE_CHECK((int64_t)T * k <= (1 << 24), MOE_ESHAPE, "moe_permute: T*k too large");
    MOE_CHECK(counts && offsets && (T == 0 || (topk_idx && perm && inv_perm)), MOE_EINVAL,
              "moe_permute: NULL pointer");
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    hipStream_t st = (hipStream_t)s;
    ProfScope p("permute", st);
    const int N = T * k;
    // 8 waves up to 4096 pairs (4.1 us at 512 pairs against 4.5 with 4 waves, 6.8 with 2), 16 above
    if (N <= 4096) permute_kernel<8><<<1, 512, 0, st>>>(topk_idx, N, E, nbits, counts, offsets, perm, inv_perm);
    else permute_kernel<16><<<1, 1024, 0, st>>>(topk_idx, N, E, nbits, counts, offsets, perm, inv_perm);
    return check_launch("permute");
}
