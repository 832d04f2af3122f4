// bkv_stream.hip -- per-decode-step kernels of the eviction cycle (Notes §2.2,
// App. Alg. 2; Summary, pseudocode): every unit appends the step's key,
// rotated to its position, and its value at row L of the cache; in the last
// n_recent_q steps before the cache is full, every query buffer's new query
// goes to the recent ring (earlier in the cycle it goes through the FPS
// buffer update instead, see bkv_fps.hip).
#include "bkv_append_impl.hpp"

namespace bkv {

namespace {

constexpr int kAppendThreads = 256;

// D / 8 threads per unit, thread j taking piece j of its unit's rows.
template <int D>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a) {
    constexpr int T = D / 8;
    const int64_t t = (int64_t)blockIdx.x * kAppendThreads + threadIdx.x;
    const int64_t unit = t / T;
    if (unit >= a.units) return;
    append_piece<D>(a, unit, (int)(t % T));
}

// Thread per 16-byte piece of a query row: q_recent[uq][slot] = q_new[uq];
// the first `batch` threads also record the positions.
template <int D>
__global__ __launch_bounds__(256) void ring_kernel(RingArgs a) {
    constexpr int kPieces = D / 8;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t < a.batch) a.pos_recent[t * a.n_recent_q + a.slot] = a.pos[t];
    if (t >= (int64_t)a.qbufs * kPieces) return;
    const int64_t uq = t / kPieces;
    const int piece = (int)(t % kPieces);
    const u32x4_t v = reinterpret_cast<const u32x4_t*>(a.q_new + uq * D)[piece];
    reinterpret_cast<u32x4_t*>(a.q_recent + (uq * a.n_recent_q + a.slot) * D)[piece] = v;
}

// Full-history beacons (the naive FPS of Notes §3.2 Fig. 7): thread per
// 16-byte piece, hist[uq][hcount[uq]] = q_new[uq] and the count grows by one
// while it is below hcap (a full history takes no more rows).  The pieces of
// one buffer sit in one wavefront, whose count load completes before its
// count store, so every piece sees the count from before the call.
template <int D>
__global__ __launch_bounds__(256) void history_kernel(HistArgs a) {
    constexpr int kPieces = D / 8;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (int64_t)a.qbufs * kPieces) return;
    const int64_t uq = t / kPieces;
    const int piece = (int)(t % kPieces);
    const int n = a.hcount[uq] > 0 ? a.hcount[uq] : 0;
    if (n >= a.hcap) return;
    const u32x4_t v = reinterpret_cast<const u32x4_t*>(a.q_new + uq * D)[piece];
    reinterpret_cast<u32x4_t*>(a.hist + (uq * a.hcap + n) * D)[piece] = v;
    if (piece == 0) a.hcount[uq] = n + 1;
}

}  // namespace

hipError_t launch_history_append(const HistArgs& a, int d, hipStream_t st) {
    const int64_t threads = (int64_t)a.qbufs * (d / 8);
    if (threads <= 0) return hipSuccess;
    dim3 grid((unsigned)((threads + 255) / 256)), block(256);
    if (d == 64) hipLaunchKernelGGL(history_kernel<64>, grid, block, 0, st, a);
    else hipLaunchKernelGGL(history_kernel<128>, grid, block, 0, st, a);
    return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, int d, hipStream_t st) {
    if (a.units <= 0) return hipSuccess;
    const int64_t threads = (int64_t)a.units * (d / 8);
    dim3 grid((unsigned)((threads + kAppendThreads - 1) / kAppendThreads)), block(kAppendThreads);
    if (d == 64) hipLaunchKernelGGL(append_kernel<64>, grid, block, 0, st, a);
    else hipLaunchKernelGGL(append_kernel<128>, grid, block, 0, st, a);
    return hipGetLastError();
}

hipError_t launch_ring(const RingArgs& a, int d, hipStream_t st) {
    const int64_t n = (int64_t)a.qbufs * (d / 8);
    const int64_t threads = n > a.batch ? n : a.batch;
    if (threads <= 0) return hipSuccess;
    dim3 grid((unsigned)((threads + 255) / 256)), block(256);
    if (d == 64) hipLaunchKernelGGL(ring_kernel<64>, grid, block, 0, st, a);
    else hipLaunchKernelGGL(ring_kernel<128>, grid, block, 0, st, a);
    return hipGetLastError();
}

}  // namespace bkv
