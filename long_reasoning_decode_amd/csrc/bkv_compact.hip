// bkv_compact.hip -- in-place gather of the kept K/V rows (Notes §2.3, Eq. 8:
// K^ = K[:, I_final, :], V^ = V[:, I_final, :]).
//
// One wavefront per unit.  idx is strictly ascending, so idx[r] >= r: every
// row's source sits at or after its destination.  The wave skips the leading
// run with idx[r] == r (nothing to move), then walks destination chunks in
// ascending order; for each chunk it issues all 16-byte loads (K and V) before
// any store.  Vector memory operations of one wave complete in issue order,
// so when a store to row x is issued every earlier load -- including any that
// reads row x as a source -- has returned; and a load of a later chunk reads
// rows at or after that chunk's first destination, beyond every row stored
// so far.  No other wave touches the unit, so no barrier is needed.
#include "bkv_device.hpp"
#include "bkv_internal.hpp"

namespace bkv {

namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kChunkRows = 16;

template <int D>
__global__ __launch_bounds__(64 * kWavesPerBlock) void compact_kernel(CompactArgs a) {
    constexpr int kPieces = D / 8;                          // 16-byte pieces per row
    constexpr int kPer = kChunkRows * kPieces / 64;         // pieces per lane per tensor
    const int lane = threadIdx.x & 63;
    const int u = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    if (u >= a.units) return;
    const int N = a.n_len, B = a.budget;
    if (N <= B) return;  // nothing evicted: idx is the identity
    const int32_t* idx = a.idx + (size_t)u * B;
    bkv_bf16* K = a.K + (size_t)u * a.cap * D;
    bkv_bf16* V = a.V + (size_t)u * a.cap * D;

    // first destination that moves
    int first = B;
    for (int base = 0; base < B; base += 64) {
        const int r = base + lane;
        const bool moved = r < B && idx[r] != r;
        const uint64_t m = __ballot(moved);
        if (m) {
            first = base + __ffsll((unsigned long long)m) - 1;
            break;
        }
    }
    for (int r0 = first; r0 < B; r0 += kChunkRows) {
        u32x4_t kv[kPer], vv[kPer];
        int dst[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int p = lane + 64 * j;
            const int row = r0 + p / kPieces;
            const int col = p % kPieces;
            dst[j] = row < B ? row : -1;
            if (row < B) {
                const int src = clampi(idx[row], 0, N - 1);
                kv[j] = *reinterpret_cast<const u32x4_t*>(K + (size_t)src * D + col * 8);
                vv[j] = *reinterpret_cast<const u32x4_t*>(V + (size_t)src * D + col * 8);
            }
        }
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            if (dst[j] >= 0) {
                const int col = (lane + 64 * j) % kPieces;
                *reinterpret_cast<u32x4_t*>(K + (size_t)dst[j] * D + col * 8) = kv[j];
                *reinterpret_cast<u32x4_t*>(V + (size_t)dst[j] * D + col * 8) = vv[j];
            }
        }
    }
}

}  // namespace

hipError_t launch_compact(const CompactArgs& a, int d, hipStream_t st) {
    if (a.units <= 0 || a.n_len <= a.budget) return hipSuccess;
    dim3 grid((a.units + kWavesPerBlock - 1) / kWavesPerBlock), block(64 * kWavesPerBlock);
    if (d == 64) hipLaunchKernelGGL(compact_kernel<64>, grid, block, 0, st, a);
    else hipLaunchKernelGGL(compact_kernel<128>, grid, block, 0, st, a);
    return hipGetLastError();
}

}  // namespace bkv
