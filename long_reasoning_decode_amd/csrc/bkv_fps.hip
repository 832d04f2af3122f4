// bkv_fps.hip -- kernels of the continual FPS buffer update and of the
// end-of-cycle merge (Notes §2.2, Eq. 9 and App. Alg. 1-2).  Four independent
// wavefronts per workgroup, one query buffer each; the per-buffer work is in
// bkv_fps_impl.hpp.
#include "bkv_fps_impl.hpp"

namespace bkv {

namespace {

constexpr int kWavesPerBlock = 4;

template <int D, bool MERGE>
__global__ __launch_bounds__(64 * kWavesPerBlock) void fps_kernel(FpsArgs a) {
    __shared__ fps::Smem s[kWavesPerBlock];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int b = blockIdx.x * kWavesPerBlock + wave;
    if (b >= a.nbuf) return;
    if (MERGE) fps::merge_one<D>(a, b, s[wave], lane);
    else fps::update_one<D>(a, b, s[wave], lane);
}

}  // namespace

hipError_t launch_fps(const FpsArgs& a, int d, bool merge, hipStream_t st) {
    if (a.nbuf <= 0) return hipSuccess;
    dim3 grid((a.nbuf + kWavesPerBlock - 1) / kWavesPerBlock), block(64 * kWavesPerBlock);
    if (d == 64) {
        if (merge) hipLaunchKernelGGL((fps_kernel<64, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((fps_kernel<64, false>), grid, block, 0, st, a);
    } else {
        if (merge) hipLaunchKernelGGL((fps_kernel<128, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((fps_kernel<128, false>), grid, block, 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace bkv
