// bkv_compact_impl.hpp -- in-place gather of one tensor's kept rows by one
// wavefront (Notes §2.3, Eq. 8: K^ = K[:, I_final, :], V^ likewise).
//
// The kept slots of the unit are staged in LDS (uint16: n_len <= 8192) and
// strictly ascending, so src[r] >= r: every row's source sits at or after its
// destination.  The wave skips the leading run with src[r] == r, then walks
// destination chunks of kChunkRows rows in ascending order, software-
// pipelined: the loads of chunk c+1 are issued before the stores of chunk c.
// This is safe because
//   * chunk c+1 reads rows >= its first destination, which lies beyond every
//     row that chunk c (or any earlier chunk) stores;
//   * a store of chunk c needs its own loads' data, and a wave's vector
//     memory operations complete in issue order, so every load issued before
//     it -- all loads of chunks <= c, including any that read the row it
//     overwrites -- has returned by then.
// K and V are independent, so one wave may move K while another moves V.
// Loads and stores are non-temporal: the moved rows are not reused soon.
#pragma once

#include "bkv_device.hpp"

namespace bkv {
namespace compact {

constexpr int kChunkRows = 32;

template <int D>
struct Chunk {
    static constexpr int kPieces = D / 8;                     // 16-byte pieces per row
    static constexpr int kPer = kChunkRows * kPieces / 64;    // pieces per lane
    u32x4_t v[kPer];
};

template <int D>
__device__ __forceinline__ void load_chunk(Chunk<D>& c, const bkv_bf16* X, const uint16_t* src, int r0, int B,
                                           int lane) {
#pragma unroll
    for (int j = 0; j < Chunk<D>::kPer; ++j) {
        const int p = lane + 64 * j;
        const int row = r0 + p / Chunk<D>::kPieces;
        const int col = p % Chunk<D>::kPieces;
        if (row < B)
            c.v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(X + (size_t)src[row] * D + col * 8));
    }
}

template <int D>
__device__ __forceinline__ void store_chunk(const Chunk<D>& c, bkv_bf16* X, int r0, int B, int lane) {
#pragma unroll
    for (int j = 0; j < Chunk<D>::kPer; ++j) {
        const int p = lane + 64 * j;
        const int row = r0 + p / Chunk<D>::kPieces;
        const int col = p % Chunk<D>::kPieces;
        if (row < B) __builtin_nontemporal_store(c.v[j], reinterpret_cast<u32x4_t*>(X + (size_t)row * D + col * 8));
    }
}

// The wave's LDS writes are complete and visible to its other lanes; the
// compiler does not move LDS accesses across this point.
__device__ __forceinline__ void wave_barrier_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// First destination row whose source differs from itself (B if none).
__device__ __forceinline__ int first_moved(const uint16_t* src, int B, int lane) {
    for (int base = 0; base < B; base += 64) {
        const int r = base + lane;
        const uint64_t m = __ballot(r < B && src[r] != r);
        if (m) return base + __ffsll((unsigned long long)m) - 1;
    }
    return B;
}

// Move rows [first, B) of X: X[r] <- X[src[r]].  One wavefront.
template <int D>
__device__ void move_rows(bkv_bf16* X, const uint16_t* src, int first, int B, int lane) {
    if (first >= B) return;
    Chunk<D> c0, c1;
    int r0 = first;
    load_chunk<D>(c0, X, src, r0, B, lane);
    while (true) {
        const int r1 = r0 + kChunkRows;
        if (r1 < B) load_chunk<D>(c1, X, src, r1, B, lane);
        store_chunk<D>(c0, X, r0, B, lane);
        if (r1 >= B) break;
        const int r2 = r1 + kChunkRows;
        if (r2 < B) load_chunk<D>(c0, X, src, r2, B, lane);
        store_chunk<D>(c1, X, r1, B, lane);
        if (r2 >= B) break;
        r0 = r2;
    }
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | 0x0F70 | ((N >> 4) << 14));
}

__device__ __forceinline__ void wg_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// load_chunk with every row past B replaced by row B - 1, so that all kPer
// load instructions issue (the wait counts below rely on it); the extra rows
// are never stored.
template <int D>
__device__ __forceinline__ void load_chunk_all(Chunk<D>& c, const bkv_bf16* X, const uint16_t* src, int r0, int B,
                                               int lane) {
#pragma unroll
    for (int j = 0; j < Chunk<D>::kPer; ++j) {
        const int p = lane + 64 * j;
        const int row = min(r0 + p / Chunk<D>::kPieces, B - 1);
        const int col = p % Chunk<D>::kPieces;
        c.v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(X + (size_t)src[row] * D + col * 8));
    }
}

// One window: window a's loads are done in every wave.  Issue the loads of
// window a + 2 kWin into `nxt`, store window a from `cur`, then wait until
// this wave's loads of window a + kWin (issued one step earlier) are done
// and meet at the barrier.  Returns false when window a was the last.
template <int D, int NW>
__device__ __forceinline__ bool window_step(Chunk<D>& cur, Chunk<D>& nxt, bkv_bf16* X, const uint16_t* src, int a,
                                            int B, int w, int lane) {
    constexpr int kWin = NW * kChunkRows;
    constexpr int kPer = Chunk<D>::kPer;
    const bool ahead = a + 2 * kWin < B;
    if (ahead) load_chunk_all<D>(nxt, X, src, a + 2 * kWin + w * kChunkRows, B, lane);
    store_chunk<D>(cur, X, a + w * kChunkRows, B, lane);
    if (a + kWin >= B) return false;
    // issued after window a + kWin's loads: at least window a's kPer stores (all its rows are below B),
    // and kPer loads of window a + 2 kWin when ahead
    if (ahead) wait_vm<2 * kPer>();
    else wait_vm<kPer>();
    wg_barrier();
    return true;
}

// Move rows [first, B) of X by NW waves of one workgroup (w = this wave's
// index among them), in windows of NW chunks: wave w moves chunk w of each
// window.  Every wave's loads of a window complete before any of the window's
// stores (a wait and a barrier), so no source row is overwritten before it
// is read.  A window's stores and the loads of any later window touch
// disjoint rows -- a later window's sources lie at or after its destinations,
// which follow this window's -- so each wave keeps two windows of loads in
// flight: the loads of window n + 2 are issued before the stores of window n
// (three chunks of registers in rotation).  All NW waves, and any other waves
// of the workgroup, must call it with the same first and B (they meet the
// same barriers).
template <int D, int NW>
__device__ void move_rows_wg(bkv_bf16* X, const uint16_t* src, int first, int B, int w, int lane) {
    if (first >= B) return;
    constexpr int kWin = NW * kChunkRows;
    Chunk<D> c0, c1, c2;
    int a = first;
    load_chunk<D>(c0, X, src, a + w * kChunkRows, B, lane);
    wait_vm<0>();
    wg_barrier();
    if (a + kWin < B) load_chunk<D>(c1, X, src, a + kWin + w * kChunkRows, B, lane);
    while (true) {
        if (!window_step<D, NW>(c0, c2, X, src, a, B, w, lane)) break;
        a += kWin;
        if (!window_step<D, NW>(c1, c0, X, src, a, B, w, lane)) break;
        a += kWin;
        if (!window_step<D, NW>(c2, c1, X, src, a, B, w, lane)) break;
        a += kWin;
    }
}

}  // namespace compact
}  // namespace bkv
