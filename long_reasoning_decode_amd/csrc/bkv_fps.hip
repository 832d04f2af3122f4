// bkv_fps.hip -- kernels of the continual FPS buffer update and of the
// end-of-cycle merge (Notes §2.2, Eq. 9 and App. Alg. 1-2).  The update is an
// append kernel (16 bytes per lane) followed by the sampling round, which only
// the buffers that filled up do; the sampling rounds and the merge run four
// independent wavefronts per workgroup, one query buffer each (the per-buffer
// work is in bkv_fps_impl.hpp).
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
    else fps::compress_one<D>(a, b, s[wave], lane);
}

// First half of the buffer update: append each buffer's new query at slot
// qcount (clamped to [0, B_Q^max - 1]) and count it.  16 lanes per buffer
// for d = 128 (8 for d = 64), each copying 16 bytes; a buffer's lanes sit in
// one wave, so all of them read the count before any of them writes it.
template <int D>
__global__ __launch_bounds__(256) void append_q_kernel(FpsArgs a) {
    constexpr int kPieces = D / 8;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t b = t / kPieces;
    const int piece = (int)(t % kPieces);
    if (b >= a.nbuf) return;
    const int bqmax = a.n_beacon + a.n_recent_q;
    const int c = clampi(a.qcount[b], 0, bqmax - 1);
    const u32x4_t v = reinterpret_cast<const u32x4_t*>(a.q_new + b * D)[piece];
    reinterpret_cast<u32x4_t*>(a.qbuf + (b * a.qcap + c) * D)[piece] = v;
    if (piece == 0) a.qcount[b] = c + 1;
}

}  // namespace

hipError_t launch_fps(const FpsArgs& a, int d, bool merge, hipStream_t st) {
    if (a.nbuf <= 0) return hipSuccess;
    if (a.src != kSrcFps) return merge ? launch_offer_merge(a, d, st) : launch_offer(a, d, st);
    if (!merge) {
        const int64_t threads = (int64_t)a.nbuf * (d / 8);
        dim3 g((unsigned)((threads + 255) / 256)), blk(256);
        if (d == 64) hipLaunchKernelGGL(append_q_kernel<64>, g, blk, 0, st, a);
        else hipLaunchKernelGGL(append_q_kernel<128>, g, blk, 0, st, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
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
