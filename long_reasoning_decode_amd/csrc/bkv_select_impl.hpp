// bkv_select_impl.hpp -- keep set of one unit by one workgroup: the forced
// prefix and recent window, plus the top-k of the other keys by score, ties
// to the lower index (Notes §2.3, Eq. 8).
//
// The unit's scores sit in LDS as order-preserving uint32 codes; an MSB-first
// radix select (4 passes of 8 bits over 256-bin LDS histograms) finds the
// k-th largest candidate code T and how many candidates equal to T still
// fit.  Ties at T go to the lowest indices, found with a block-wide prefix
// count; a second prefix count over the keep flags writes the kept slots in
// ascending order.  Integer work only: the result is exact for the given
// fp32 scores.
#pragma once

#include "bkv_device.hpp"

namespace bkv {
namespace sel {

struct Scratch {
    uint32_t* keys;   // [n_len] (LDS)
    uint32_t* hist;   // [256]   (LDS)
    int* wsum;        // [waves] (LDS)
    uint32_t* bin;    // [2]     (LDS)
};

// Exclusive block-wide prefix sum of v; also returns the total.
template <int BLOCK>
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum, int& total) {
    constexpr int kWaves = BLOCK / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const int s = wsum[w];
        if (w < wave) base += s;
        tot += s;
    }
    __syncthreads();
    total = tot;
    return base + x - v;
}

// Kept slots of one unit from its score codes w.keys[0..N) (f32_order of the
// scores, already in LDS and visible to the workgroup): idx (global, [B], -1
// padded; may be null) and src (LDS, [min(N, B)] as uint16; may be null).
// All BLOCK threads call it.
template <int BLOCK>
__device__ void select_staged(int N, int B, int n_prefix, int n_recent_kv, int32_t* idx, uint16_t* src,
                              const Scratch& w) {
    const int tid = threadIdx.x;
    if (N <= B) {
        for (int r = tid; r < B; r += BLOCK) {
            if (idx) idx[r] = r < N ? r : -1;
            if (src && r < N) src[r] = (uint16_t)r;
        }
        __syncthreads();
        return;
    }
    const int np = n_prefix < N ? n_prefix : N;
    const int rs = N - n_recent_kv > 0 ? N - n_recent_kv : 0;
    const int k_sel = B - np - (N - rs);   // >= 0: checked on the host

    // ---- radix select of the k_sel-th largest candidate code
    uint32_t prefix = 0, pmask = 0;
    int remaining = k_sel;
    if (k_sel > 0) {
        for (int shift = 24; shift >= 0; shift -= 8) {
            for (int i = tid; i < 256; i += BLOCK) w.hist[i] = 0;
            __syncthreads();
            for (int j = np + tid; j < rs; j += BLOCK) {
                const uint32_t k = w.keys[j];
                if ((k & pmask) == prefix) atomicAdd(&w.hist[(k >> shift) & 255u], 1u);
            }
            __syncthreads();
            if (tid < 64) {
                // lane l owns bins 4l..4l+3; inclusive suffix sums over lanes
                const int l = tid;
                const uint32_t h0 = w.hist[4 * l], h1 = w.hist[4 * l + 1], h2 = w.hist[4 * l + 2],
                               h3 = w.hist[4 * l + 3];
                const uint32_t own = h0 + h1 + h2 + h3;
                uint32_t suf = own;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const uint32_t y = __shfl_down(suf, off, 64);
                    if (l + off < 64) suf += y;
                }
                const uint32_t above = suf - own;   // codes in bins > 4l+3
                const uint32_t rem = (uint32_t)remaining;
                if (above < rem && rem <= suf) {
                    uint32_t acc = above;
                    const uint32_t hh[4] = {h0, h1, h2, h3};
                    int bin = 4 * l;
                    for (int q = 3; q >= 0; --q) {
                        if (acc + hh[q] >= rem) {
                            bin = 4 * l + q;
                            break;
                        }
                        acc += hh[q];
                    }
                    w.bin[0] = (uint32_t)bin;
                    w.bin[1] = acc;
                }
            }
            __syncthreads();
            prefix |= w.bin[0] << shift;
            pmask |= 255u << shift;
            remaining -= (int)w.bin[1];
            __syncthreads();
        }
    }
    // k_sel == 0: take nothing (T above every code, no equal takes)
    const uint32_t T = k_sel > 0 ? prefix : 0xFFFFFFFFu;
    const int need_eq = k_sel > 0 ? remaining : 0;

    // ---- keep flags; ties at T to the lowest indices
    const int seg = (N + BLOCK - 1) / BLOCK;
    const int j0 = tid * seg < N ? tid * seg : N;
    const int j1 = j0 + seg < N ? j0 + seg : N;
    int n_eq = 0;
    for (int j = j0; j < j1; ++j) n_eq += (j >= np && j < rs && w.keys[j] == T) ? 1 : 0;
    int tot;
    int eq_rank = block_exclusive_scan<BLOCK>(n_eq, w.wsum, tot);
    int n_keep = 0;
    for (int j = j0; j < j1; ++j) {
        bool keep;
        if (j < np || j >= rs) keep = true;
        else {
            const uint32_t k = w.keys[j];
            if (k > T) keep = k_sel > 0;
            else if (k == T) keep = eq_rank++ < need_eq;
            else keep = false;
        }
        n_keep += keep ? 1 : 0;
    }
    int pos = block_exclusive_scan<BLOCK>(n_keep, w.wsum, tot);
    eq_rank = block_exclusive_scan<BLOCK>(n_eq, w.wsum, tot);
    for (int j = j0; j < j1; ++j) {
        bool keep;
        if (j < np || j >= rs) keep = true;
        else {
            const uint32_t k = w.keys[j];
            if (k > T) keep = k_sel > 0;
            else if (k == T) keep = eq_rank++ < need_eq;
            else keep = false;
        }
        if (keep) {
            if (pos < B) {
                if (idx) idx[pos] = j;
                if (src) src[pos] = (uint16_t)j;
            }
            ++pos;
        }
    }
    __syncthreads();
}

// As select_staged, with the scores read from global memory first.
template <int BLOCK>
__device__ void select_unit(const float* sc, int N, int B, int n_prefix, int n_recent_kv, int32_t* idx,
                            uint16_t* src, const Scratch& w) {
    if (N > B) {
        for (int j = threadIdx.x; j < N; j += BLOCK) w.keys[j] = f32_order(sc[j]);
        __syncthreads();
    }
    select_staged<BLOCK>(N, B, n_prefix, n_recent_kv, idx, src, w);
}

}  // namespace sel
}  // namespace bkv
