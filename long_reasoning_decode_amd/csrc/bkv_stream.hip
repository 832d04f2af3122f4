// bkv_stream.hip -- per-decode-step kernels of the eviction cycle (Notes §2.2,
// App. Alg. 2; Summary, pseudocode): every unit appends the step's key,
// rotated to its position, and its value at row L of the cache; in the last
// n_recent_q steps before the cache is full, every query buffer's new query
// goes to the recent ring (earlier in the cycle it goes through the FPS
// buffer update instead, see bkv_fps.hip).
#include "bkv_device.hpp"
#include "bkv_internal.hpp"

namespace bkv {

namespace {

constexpr int kAppendThreads = 256;

// D / 8 threads per unit.  Thread j rotates the pairs (i, i + D/2) for
// i = 4j .. 4j + 3 of the new key in fp32, each product and sum rounded on
// its own, then rounds to bf16 -- the same rotation as the observation rows
// of the scoring kernel -- and copies 16 bytes of the value row.
template <int D>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a) {
    constexpr int T = D / 8;
    const int64_t t = (int64_t)blockIdx.x * kAppendThreads + threadIdx.x;
    const int64_t unit = t / T;
    const int j = (int)(t % T);
    if (unit >= a.units) return;
    const int b = (int)((unit / a.hkv) % a.batch);
    const int p = clampi(a.pos[b], 0, a.rope_rows - 1);
    const size_t dst = ((size_t)unit * a.cap + a.L) * D;
    const bkv_bf16* k = a.k_new + (size_t)unit * D;
    const uint2 lo = *reinterpret_cast<const uint2*>(k + 4 * j);            // x_i,       i = 4j .. 4j + 3
    const uint2 hi = *reinterpret_cast<const uint2*>(k + 4 * j + D / 2);    // x_{i+D/2}
    const f32x4_t* cs = reinterpret_cast<const f32x4_t*>(a.rope_cs + ((size_t)p * (D / 2) + 4 * j) * 2);
    const f32x4_t cs01 = cs[0], cs23 = cs[1];                               // (c, s) of pairs i, i+1 | i+2, i+3
    const float c[4] = {cs01[0], cs01[2], cs23[0], cs23[2]};
    const float sn[4] = {cs01[1], cs01[3], cs23[1], cs23[3]};
    const uint32_t xw0[2] = {lo.x, lo.y}, xw1[2] = {hi.x, hi.y};
    uint32_t y0w[2], y1w[2];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        uint32_t o0 = 0, o1 = 0;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int q = 2 * w + e;
            const float x0 = bf16_bits_to_f32((xw0[w] >> (16 * e)) & 0xFFFFu);
            const float x1 = bf16_bits_to_f32((xw1[w] >> (16 * e)) & 0xFFFFu);
            const float y0 = x0 * c[q] - x1 * sn[q];
            const float y1 = x1 * c[q] + x0 * sn[q];
            o0 |= f32_to_bf16_bits(y0) << (16 * e);
            o1 |= f32_to_bf16_bits(y1) << (16 * e);
        }
        y0w[w] = o0;
        y1w[w] = o1;
    }
    *reinterpret_cast<uint2*>(a.K + dst + 4 * j) = make_uint2(y0w[0], y0w[1]);
    *reinterpret_cast<uint2*>(a.K + dst + 4 * j + D / 2) = make_uint2(y1w[0], y1w[1]);
    reinterpret_cast<u32x4_t*>(a.V + dst)[j] = reinterpret_cast<const u32x4_t*>(a.v_new + (size_t)unit * D)[j];
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
