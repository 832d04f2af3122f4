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

constexpr int kUnitsPerBlock = 4;   // one wave per unit

// Wave per unit.  Lane i < D/2 rotates the pair (i, i + D/2) of the new key
// in fp32, each product and sum rounded on its own, then rounds to bf16 --
// the same rotation as the observation rows of the scoring kernel.  The value
// row is copied four bytes per lane.
template <int D>
__global__ __launch_bounds__(64 * kUnitsPerBlock) void append_kernel(AppendArgs a) {
    const int unit = blockIdx.x * kUnitsPerBlock + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (unit >= a.units) return;
    const int b = (unit / a.hkv) % a.batch;
    const int p = clampi(a.pos[b], 0, a.rope_rows - 1);
    const size_t dst = ((size_t)unit * a.cap + a.L) * D;
    const bkv_bf16* k = a.k_new + (size_t)unit * D;
    if (lane < D / 2) {
        const float c = a.rope_cs[((size_t)p * (D / 2) + lane) * 2];
        const float s = a.rope_cs[((size_t)p * (D / 2) + lane) * 2 + 1];
        const float x0 = bf16_bits_to_f32(k[lane]);
        const float x1 = bf16_bits_to_f32(k[lane + D / 2]);
        const float y0 = x0 * c - x1 * s;
        const float y1 = x1 * c + x0 * s;
        a.K[dst + lane] = (bkv_bf16)f32_to_bf16_bits(y0);
        a.K[dst + lane + D / 2] = (bkv_bf16)f32_to_bf16_bits(y1);
    }
    if (lane < D / 2) {
        const uint32_t* v = reinterpret_cast<const uint32_t*>(a.v_new + (size_t)unit * D);
        reinterpret_cast<uint32_t*>(a.V + dst)[lane] = v[lane];
    }
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

}  // namespace

hipError_t launch_append(const AppendArgs& a, int d, hipStream_t st) {
    if (a.units <= 0) return hipSuccess;
    dim3 grid((a.units + kUnitsPerBlock - 1) / kUnitsPerBlock), block(64 * kUnitsPerBlock);
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
