// bkv_compact.hip -- in-place gather of the kept K/V rows (Notes §2.3, Eq. 8:
// K^ = K[:, I_final, :], V^ = V[:, I_final, :]).
//
// One wavefront per unit.  idx is strictly ascending, so idx[r] >= r: every
// row's source sits at or after its destination.  The wave skips the leading
// run with idx[r] == r (nothing to move), then walks destination chunks of
// kChunkRows rows in ascending order, software-pipelined: the loads of chunk
// c+1 are issued before the stores of chunk c.  This is safe because
//   * chunk c+1 reads rows >= its first destination, which lies beyond every
//     row that chunk c (or any earlier chunk) stores;
//   * a store of chunk c needs its own loads' data, and a wave's vector
//     memory operations complete in issue order, so every load issued before
//     it -- all loads of chunks <= c, including any that read the row it
//     overwrites -- has returned by then.
// No other wave touches the unit, so no barrier is needed.  The unit's kept
// indices are staged in LDS once, so the gather addresses cost no extra
// global round trip inside the loop (as uint16: n_len <= 8192).
#include "bkv_device.hpp"
#include "bkv_internal.hpp"

namespace bkv {

namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kChunkRows = 16;
constexpr int kMaxBudget = 8192;   // staged as uint16 (n_len <= 8192)

template <int D>
struct Chunk {
    static constexpr int kPieces = D / 8;                     // 16-byte pieces per row
    static constexpr int kPer = kChunkRows * kPieces / 64;    // pieces per lane per tensor
    u32x4_t k[kPer], v[kPer];
};

template <int D>
__device__ __forceinline__ void load_chunk(Chunk<D>& c, const bkv_bf16* K, const bkv_bf16* V,
                                           const uint16_t* sidx, int r0, int B, int N, int lane) {
#pragma unroll
    for (int j = 0; j < Chunk<D>::kPer; ++j) {
        const int p = lane + 64 * j;
        const int row = r0 + p / Chunk<D>::kPieces;
        const int col = p % Chunk<D>::kPieces;
        if (row < B) {
            const int src = sidx[row];
            c.k[j] = *reinterpret_cast<const u32x4_t*>(K + (size_t)src * D + col * 8);
            c.v[j] = *reinterpret_cast<const u32x4_t*>(V + (size_t)src * D + col * 8);
        }
    }
}

template <int D>
__device__ __forceinline__ void store_chunk(const Chunk<D>& c, bkv_bf16* K, bkv_bf16* V, int r0, int B, int lane) {
#pragma unroll
    for (int j = 0; j < Chunk<D>::kPer; ++j) {
        const int p = lane + 64 * j;
        const int row = r0 + p / Chunk<D>::kPieces;
        const int col = p % Chunk<D>::kPieces;
        if (row < B) {
            *reinterpret_cast<u32x4_t*>(K + (size_t)row * D + col * 8) = c.k[j];
            *reinterpret_cast<u32x4_t*>(V + (size_t)row * D + col * 8) = c.v[j];
        }
    }
}

template <int D>
__global__ __launch_bounds__(64 * kWavesPerBlock) void compact_kernel(CompactArgs a) {
    extern __shared__ uint16_t sidx_all[];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int u = blockIdx.x * kWavesPerBlock + wave;
    if (u >= a.units) return;
    const int N = a.n_len, B = a.budget;
    if (N <= B) return;  // nothing evicted: idx is the identity
    uint16_t* sidx = sidx_all + wave * ((B + 7) & ~7);
    const int32_t* idx = a.idx + (size_t)u * B;
    bkv_bf16* K = a.K + (size_t)u * a.cap * D;
    bkv_bf16* V = a.V + (size_t)u * a.cap * D;

    // stage the kept indices; find the first destination that moves
    int first = B;
    for (int base = 0; base < B; base += 64) {
        const int r = base + lane;
        const int s = r < B ? clampi(idx[r], 0, N - 1) : r;
        if (r < B) sidx[r] = (uint16_t)s;
        const uint64_t m = __ballot(s != r);
        if (m && first == B) first = base + __ffsll((unsigned long long)m) - 1;
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    if (first >= B) return;

    Chunk<D> c0, c1;
    int r0 = first;
    load_chunk<D>(c0, K, V, sidx, r0, B, N, lane);
    while (true) {
        const int r1 = r0 + kChunkRows;
        if (r1 < B) load_chunk<D>(c1, K, V, sidx, r1, B, N, lane);
        store_chunk<D>(c0, K, V, r0, B, lane);
        if (r1 >= B) break;
        const int r2 = r1 + kChunkRows;
        if (r2 < B) load_chunk<D>(c0, K, V, sidx, r2, B, N, lane);
        store_chunk<D>(c1, K, V, r1, B, lane);
        if (r2 >= B) break;
        r0 = r2;
    }
}

}  // namespace

hipError_t launch_compact(const CompactArgs& a, int d, hipStream_t st) {
    if (a.units <= 0 || a.n_len <= a.budget) return hipSuccess;
    if (a.budget > kMaxBudget) return hipErrorInvalidValue;
    dim3 grid((a.units + kWavesPerBlock - 1) / kWavesPerBlock), block(64 * kWavesPerBlock);
    const size_t smem = (size_t)kWavesPerBlock * ((a.budget + 7) & ~7) * sizeof(uint16_t);
    if (d == 64) hipLaunchKernelGGL(compact_kernel<64>, grid, block, smem, st, a);
    else hipLaunchKernelGGL(compact_kernel<128>, grid, block, smem, st, a);
    return hipGetLastError();
}

}  // namespace bkv
