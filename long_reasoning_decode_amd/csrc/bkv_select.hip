// bkv_select.hip -- keep set of each unit: forced prefix and recent window,
// plus the top-k of the other keys by score (Notes §2.3, Eq. 8).
//
// One workgroup per unit.  The unit's scores live in LDS as order-preserving
// uint32 codes; an MSB-first radix select (4 passes of 8 bits, 256-bin LDS
// histograms) finds the k-th largest candidate code T and how many candidates
// equal to T still fit.  Ties at T go to the lowest indices, found with a
// block-wide prefix count; a second prefix count over the keep flags writes
// the kept slots in ascending order.  Integer work only: the result is exact
// for the given fp32 scores.
#include "bkv_device.hpp"
#include "bkv_internal.hpp"

namespace bkv {

namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;

// Exclusive block-wide prefix sum of v; also returns the total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum, int& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int y = __shfl_up(x, off, 64);
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

__global__ __launch_bounds__(kBlock) void select_kernel(SelectArgs a) {
    extern __shared__ uint32_t keys[];
    __shared__ uint32_t hist[256];
    __shared__ int wsum[kWaves];
    __shared__ uint32_t s_bin, s_above;

    const int u = blockIdx.x;
    if (u >= a.units) return;
    const int tid = threadIdx.x;
    const int N = a.n_len, B = a.budget;
    int32_t* out = a.idx + (size_t)u * B;
    if (N <= B) {
        for (int r = tid; r < B; r += kBlock) out[r] = r < N ? r : -1;
        return;
    }
    const float* sc = a.scores + (size_t)u * N;
    const int np = a.n_prefix < N ? a.n_prefix : N;
    const int rs = N - a.n_recent_kv > 0 ? N - a.n_recent_kv : 0;
    const int k_sel = B - np - (N - rs);   // >= 0: checked on the host
    for (int j = tid; j < N; j += kBlock) keys[j] = f32_order(sc[j]);
    __syncthreads();

    // ---- radix select of the k_sel-th largest candidate code
    uint32_t prefix = 0, pmask = 0;
    int remaining = k_sel;
    if (k_sel > 0) {
        for (int shift = 24; shift >= 0; shift -= 8) {
            for (int i = tid; i < 256; i += kBlock) hist[i] = 0;
            __syncthreads();
            for (int j = np + tid; j < rs; j += kBlock) {
                const uint32_t k = keys[j];
                if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
            }
            __syncthreads();
            if (tid < 64) {
                // lane l owns bins 4l..4l+3; inclusive suffix sums over lanes
                const int l = tid;
                const uint32_t h0 = hist[4 * l], h1 = hist[4 * l + 1], h2 = hist[4 * l + 2], h3 = hist[4 * l + 3];
                const uint32_t own = h0 + h1 + h2 + h3;
                uint32_t suf = own;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    uint32_t y = __shfl_down(suf, off, 64);
                    if (l + off < 64) suf += y;
                }
                const uint32_t above = suf - own;   // codes in bins > 4l+3
                const uint32_t rem = (uint32_t)remaining;
                if (above < rem && rem <= suf) {
                    uint32_t acc = above;
                    const uint32_t hh[4] = {h0, h1, h2, h3};
                    int bin = 4 * l;
                    for (int q = 3; q >= 0; --q) {
                        if (acc + hh[q] >= rem) { bin = 4 * l + q; break; }
                        acc += hh[q];
                    }
                    s_bin = (uint32_t)bin;
                    s_above = acc;
                }
            }
            __syncthreads();
            prefix |= s_bin << shift;
            pmask |= 255u << shift;
            remaining -= (int)s_above;
            __syncthreads();
        }
    }
    // k_sel == 0: take nothing (T above every code, no equal takes)
    const uint32_t T = k_sel > 0 ? prefix : 0xFFFFFFFFu;
    const int need_eq = k_sel > 0 ? remaining : 0;

    // ---- keep flags; ties at T to the lowest indices
    const int seg = (N + kBlock - 1) / kBlock;
    const int j0 = tid * seg < N ? tid * seg : N;
    const int j1 = j0 + seg < N ? j0 + seg : N;
    int n_eq = 0;
    for (int j = j0; j < j1; ++j) n_eq += (j >= np && j < rs && keys[j] == T) ? 1 : 0;
    int tot;
    int eq_rank = block_exclusive_scan(n_eq, wsum, tot);
    int n_keep = 0;
    for (int j = j0; j < j1; ++j) {
        bool keep;
        if (j < np || j >= rs) keep = true;
        else {
            const uint32_t k = keys[j];
            if (k > T) keep = k_sel > 0;
            else if (k == T) keep = eq_rank++ < need_eq;
            else keep = false;
        }
        n_keep += keep ? 1 : 0;
    }
    int pos = block_exclusive_scan(n_keep, wsum, tot);
    eq_rank = block_exclusive_scan(n_eq, wsum, tot);
    for (int j = j0; j < j1; ++j) {
        bool keep;
        if (j < np || j >= rs) keep = true;
        else {
            const uint32_t k = keys[j];
            if (k > T) keep = k_sel > 0;
            else if (k == T) keep = eq_rank++ < need_eq;
            else keep = false;
        }
        if (keep) {
            if (pos < B) out[pos] = j;
            ++pos;
        }
    }
}

}  // namespace

hipError_t launch_select(const SelectArgs& a, hipStream_t st) {
    if (a.units <= 0 || a.budget <= 0) return hipSuccess;
    const size_t smem = (size_t)(a.n_len > a.budget ? a.n_len : 1) * 4;
    hipLaunchKernelGGL(select_kernel, dim3(a.units), dim3(kBlock), smem, st, a);
    return hipGetLastError();
}

}  // namespace bkv
