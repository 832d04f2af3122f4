// bkv_fps.hip -- kernels of the continual FPS buffer update and of the
// end-of-cycle merge (Notes §2.2, Eq. 9 and App. Alg. 1-2), independent
// wavefronts in both.  The update (and the compression at the freeze point)
// appends each buffer's query and samples the buffers that filled up, four
// per wave at a time, a run of buffers per wave (bkv_fps_impl.hpp; 13 KB of
// LDS and at most 168 VGPRs per wave, three waves per SIMD).  In a decode
// step the update also appends the step's key and value rows, so that the
// step is one launch.  The merge samples beacons ++ recents, two buffers per
// wave and four waves per SIMD (bkv_fps_pair.hpp).
#include <atomic>

#include "bkv_append_impl.hpp"
#include "bkv_fps_pair.hpp"
#include "bkv_step.hpp"

namespace bkv {

namespace {

constexpr int kWavesPerBlock = 2;        // update and compression
constexpr int kMergeWavesPerBlock = 2;   // merge

// Wave w of W takes the contiguous buffers [w nbuf / W, (w + 1) nbuf / W),
// kMaxBuffersPerWave at a time, so every wave has the same share (to one
// buffer) when all of them sample.
template <int D, bool COMPRESS>
__global__ __launch_bounds__(64 * kWavesPerBlock, 3) void fps_kernel(FpsArgs a, AppendArgs app) {
    __shared__ fps::Smem s[kWavesPerBlock];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    const int64_t n_waves = (int64_t)gridDim.x * kWavesPerBlock;
    if (!COMPRESS && app.units > 0) {   // the step's key and value rows: wave w takes a contiguous share of pieces
        constexpr int T = D / 8;
        const int64_t n = (int64_t)app.units * T;
        const int64_t p1 = (w + 1) * n / n_waves;
        for (int64_t p = w * n / n_waves + lane; p < p1; p += 64) append_piece<D>(app, p / T, (int)(p % T));
    }
    const int64_t lo = w * a.nbuf / n_waves, hi = (w + 1) * a.nbuf / n_waves;
    for (int64_t b0 = lo; b0 < hi; b0 += fps::kMaxBuffersPerWave) {
        const int nw = (int)(hi - b0 < fps::kMaxBuffersPerWave ? hi - b0 : fps::kMaxBuffersPerWave);
        fps::update_wave<D, COMPRESS>(a, (int)b0, nw, s[wave], lane);
    }
}

// Two buffers per wave.
template <int D>
__global__ __launch_bounds__(64 * kMergeWavesPerBlock, 4) void merge_kernel(FpsArgs a) {
    __shared__ fps::PairSmem s[kMergeWavesPerBlock];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * kMergeWavesPerBlock + wave;
    if (2 * w >= a.nbuf) return;
    fps::merge_pair<D>(a, (int)(2 * w), s[wave], lane);
}

template <int D>
hipError_t blocks_per_cu(int* out) {
    int u = 0, c = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&u, fps_kernel<D, false>, 64 * kWavesPerBlock, 0);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&c, fps_kernel<D, true>, 64 * kWavesPerBlock, 0);
    *out = u < c ? u : c;
    return e;
}

}  // namespace

// Workgroups of the update kernels resident on the current device at once
// (the lesser of the update and the compression).  The figure is queried once
// per device and head size and kept in a process-wide memo (the library's
// only global state, written with relaxed atomics: every writer stores the
// same value).
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
    if (e == hipSuccess) e = d == 64 ? blocks_per_cu<64>(&per_cu) : blocks_per_cu<128>(&per_cu);
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)(cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1);
    if (dev >= 0 && dev < kMaxDev) cache[di][dev].store(n, std::memory_order_relaxed);
    *out = n;
    return hipSuccess;
}

namespace {

// The update or the compression kernel over every buffer (with app.units > 0, the update also appends
// app's key and value rows).
hipError_t launch_update(const FpsArgs& a, const AppendArgs& app, int d, hipStream_t st) {
    // at most one buffer per wave, and at most the workgroups the chip holds at once
    int64_t blocks = (a.nbuf + kWavesPerBlock - 1) / kWavesPerBlock;
    int64_t fit = 0;
    const hipError_t e = fps_grid_limit(d, &fit);
    if (e != hipSuccess) return e;
    if (blocks > fit) blocks = fit;
    dim3 grid((unsigned)blocks), block(64 * kWavesPerBlock);
    if (d == 64) {
        if (a.compress) hipLaunchKernelGGL((fps_kernel<64, true>), grid, block, 0, st, a, app);
        else hipLaunchKernelGGL((fps_kernel<64, false>), grid, block, 0, st, a, app);
    } else {
        if (a.compress) hipLaunchKernelGGL((fps_kernel<128, true>), grid, block, 0, st, a, app);
        else hipLaunchKernelGGL((fps_kernel<128, false>), grid, block, 0, st, a, app);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fps_step(const FpsArgs& a, const AppendArgs& app, int d, hipStream_t st) {
    if (a.nbuf <= 0) return hipSuccess;
    return launch_update(a, app, d, st);
}

hipError_t launch_fps(const FpsArgs& a, int d, bool merge, hipStream_t st) {
    if (a.nbuf <= 0) return hipSuccess;
    if (a.src == kSrcNaive)   // the beacons come from the history at each eviction: fps_sel only receives -1s
        return launch_offer_merge(a, d, st);
    if (a.src != kSrcFps && !a.compress) return merge ? launch_offer_merge(a, d, st) : launch_offer(a, d, st);
    if (merge) {
        const int64_t blocks = ((a.nbuf + 1) / 2 + kMergeWavesPerBlock - 1) / kMergeWavesPerBlock;
        dim3 grid((unsigned)blocks), block(64 * kMergeWavesPerBlock);
        if (d == 64) hipLaunchKernelGGL((merge_kernel<64>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((merge_kernel<128>), grid, block, 0, st, a);
        return hipGetLastError();
    }
    AppendArgs none{};
    none.units = 0;
    return launch_update(a, none, d, st);
}

}  // namespace bkv
