// bkv_compact.hip -- in-place compaction kernel: two wavefronts per unit, one
// moves the kept K rows and one the kept V rows (bkv_compact_impl.hpp).
#include "bkv_compact_impl.hpp"
#include "bkv_internal.hpp"

namespace bkv {

namespace {

constexpr int kCompactWaves = 4;   // two units per workgroup

template <int D>
__global__ __launch_bounds__(64 * kCompactWaves) void compact_kernel(CompactArgs a) {
    extern __shared__ uint16_t src_all[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int gw = blockIdx.x * kCompactWaves + wave;
    const int u = gw >> 1;
    if (u >= a.units) return;
    const int N = a.n_len, B = a.budget;
    if (N <= B) return;  // nothing evicted: idx is the identity
    uint16_t* src = src_all + wave * ((B + 7) & ~7);
    const int32_t* idx = a.idx + (size_t)u * B;
    for (int r = lane; r < B; r += 64) src[r] = (uint16_t)clampi(idx[r], 0, N - 1);
    compact::wave_barrier_lds();
    bkv_bf16* X = ((gw & 1) ? a.V : a.K) + (size_t)u * a.cap * D;
    compact::move_rows<D>(X, src, compact::first_moved(src, B, lane), B, lane);
}

}  // namespace

hipError_t launch_compact(const CompactArgs& a, int d, hipStream_t st) {
    if (a.units <= 0 || a.n_len <= a.budget) return hipSuccess;
    const long waves = 2l * a.units;
    dim3 grid((unsigned)((waves + kCompactWaves - 1) / kCompactWaves)), block(64 * kCompactWaves);
    const size_t smem = (size_t)kCompactWaves * ((a.budget + 7) & ~7) * sizeof(uint16_t);
    if (d == 64) hipLaunchKernelGGL(compact_kernel<64>, grid, block, smem, st, a);
    else hipLaunchKernelGGL(compact_kernel<128>, grid, block, smem, st, a);
    return hipGetLastError();
}

}  // namespace bkv
