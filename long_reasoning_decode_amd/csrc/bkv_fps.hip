// bkv_fps.hip -- kernels of the continual FPS buffer update and of the
// end-of-cycle merge (Notes §2.2, Eq. 9 and App. Alg. 1-2): four independent
// wavefronts per workgroup (the per-buffer work is in bkv_fps_impl.hpp).  The
// update appends each buffer's query and samples the buffers that filled up,
// a run of buffers per wave when there are many; the merge takes two buffers
// per wave.
#include <atomic>

#include "bkv_fps_impl.hpp"

namespace bkv {

namespace {

constexpr int kWavesPerBlock = 4;

// MODE kMerge: two buffers per wave.  kUpdate, kCompress: wave w of W takes the
// contiguous buffers [w nbuf / W, (w + 1) nbuf / W), kMaxBuffersPerWave at a
// time, so every wave has the same share (to one buffer) when all of them sample.
constexpr int kUpdate = 0, kMerge = 1, kCompress = 2;

template <int D, int MODE>
__global__ __launch_bounds__(64 * kWavesPerBlock) void fps_kernel(FpsArgs a) {
    __shared__ fps::Smem s[kWavesPerBlock];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    if constexpr (MODE == kMerge) {
        if (2 * w >= a.nbuf) return;
        fps::merge_pair<D>(a, (int)(2 * w), s[wave], lane);
    } else {
        const int64_t n_waves = (int64_t)gridDim.x * kWavesPerBlock;
        const int64_t lo = w * a.nbuf / n_waves, hi = (w + 1) * a.nbuf / n_waves;
        for (int64_t b0 = lo; b0 < hi; b0 += fps::kMaxBuffersPerWave) {
            const int nw = (int)(hi - b0 < fps::kMaxBuffersPerWave ? hi - b0 : fps::kMaxBuffersPerWave);
            fps::update_wave<D, MODE == kCompress>(a, (int)b0, nw, s[wave], lane);
        }
    }
}

}  // namespace

// Workgroups of the update kernel resident on the current device at once.  The
// figure is queried once per device and head size and kept in a process-wide
// memo (the library's only global state, written with relaxed atomics: every
// writer stores the same value).
hipError_t fps_grid_limit(int d, int64_t* out) {
    constexpr int kMaxDev = 64;
    static std::atomic<int64_t> cache[2][kMaxDev] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const int di = d == 64 ? 0 : 1;
    if (dev >= 0 && dev < kMaxDev && cache[di][dev].load(std::memory_order_relaxed) > 0) {
        *out = cache[di][dev].load(std::memory_order_relaxed);
        return hipSuccess;
    }
    int cus = 0, per_cu = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = d == 64 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fps_kernel<64, kUpdate>,
                                                                   64 * kWavesPerBlock, 0)
                    : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fps_kernel<128, kUpdate>,
                                                                   64 * kWavesPerBlock, 0);
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)(cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1);
    if (dev >= 0 && dev < kMaxDev) cache[di][dev].store(n, std::memory_order_relaxed);
    *out = n;
    return hipSuccess;
}

hipError_t launch_fps(const FpsArgs& a, int d, bool merge, hipStream_t st) {
    if (a.nbuf <= 0) return hipSuccess;
    if (a.src == kSrcNaive)   // the beacons come from the history at each eviction: fps_sel only receives -1s
        return launch_offer_merge(a, d, st);
    if (a.src != kSrcFps && !a.compress) return merge ? launch_offer_merge(a, d, st) : launch_offer(a, d, st);
    // merge: two buffers per wave; update: at most one buffer per wave
    int64_t blocks = ((merge ? (a.nbuf + 1) / 2 : a.nbuf) + kWavesPerBlock - 1) / kWavesPerBlock;
    if (!merge) {   // the update: at most the workgroups the chip holds at once
        int64_t fit = 0;
        const hipError_t e = fps_grid_limit(d, &fit);
        if (e != hipSuccess) return e;
        if (blocks > fit) blocks = fit;
    }
    dim3 grid((unsigned)blocks), block(64 * kWavesPerBlock);
    if (d == 64) {
        if (merge) hipLaunchKernelGGL((fps_kernel<64, kMerge>), grid, block, 0, st, a);
        else if (a.compress) hipLaunchKernelGGL((fps_kernel<64, kCompress>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((fps_kernel<64, kUpdate>), grid, block, 0, st, a);
    } else {
        if (merge) hipLaunchKernelGGL((fps_kernel<128, kMerge>), grid, block, 0, st, a);
        else if (a.compress) hipLaunchKernelGGL((fps_kernel<128, kCompress>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((fps_kernel<128, kUpdate>), grid, block, 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace bkv
