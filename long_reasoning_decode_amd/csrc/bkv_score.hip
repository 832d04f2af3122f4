// bkv_score.hip -- scoring kernel: one 8-wave workgroup per unit (the work
// is in bkv_score_impl.hpp), scores written as exp2 of the per-key codes.
#include "bkv_score_impl.hpp"

namespace bkv {

namespace {

template <int D, int KS, bool MEAN>
__global__ __launch_bounds__(score::kThreads) void score_kernel(ScoreArgs a) {
    using L = score::Layout<D>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    uint32_t* codes = reinterpret_cast<uint32_t*>(smem + L::fixed_bytes(MEAN));
    const int u = blockIdx.x;
    if (u >= a.units) return;
    score::unit_codes<D, KS, MEAN>(a, u, smem, codes);
    float* out = a.scores + (size_t)u * a.n_len;
    for (int j = threadIdx.x; j < a.n_len; j += score::kThreads) out[j] = score::score_of<MEAN>(codes[j]);
}

template <int D, int KS, bool MEAN>
hipError_t launch_one(const ScoreArgs& a, hipStream_t st) {
    const size_t smem = score::Layout<D>::fixed_bytes(MEAN) + (size_t)a.n_len * 4;
    hipLaunchKernelGGL((score_kernel<D, KS, MEAN>), dim3(a.units), dim3(score::kThreads), smem, st, a);
    return hipGetLastError();
}

template <int D, bool MEAN>
hipError_t launch_dm(const ScoreArgs& a, hipStream_t st) {
    // query heads per workgroup: the smallest power of two >= G; key split KS = waves / heads
    constexpr int W = score::kWaves;
    if (a.G <= 1) return launch_one<D, W, MEAN>(a, st);
    if (a.G <= 2) return launch_one<D, W / 2, MEAN>(a, st);
    if (a.G <= 4) return launch_one<D, W / 4, MEAN>(a, st);
    return launch_one<D, 1, MEAN>(a, st);
}

template <int D>
hipError_t launch_d(const ScoreArgs& a, hipStream_t st) {
    return a.pool_mean ? launch_dm<D, true>(a, st) : launch_dm<D, false>(a, st);
}

}  // namespace

hipError_t launch_score(const ScoreArgs& a, int d, hipStream_t st) {
    if (a.units <= 0 || a.n_len <= 0) return hipSuccess;
    return d == 64 ? launch_d<64>(a, st) : launch_d<128>(a, st);
}

}  // namespace bkv
