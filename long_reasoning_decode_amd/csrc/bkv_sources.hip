// bkv_sources.hip -- the other sources of beacons that the reading notes
// ablate, with the buffer, count and cycle of continual FPS unchanged:
//   initial (Initial+Recent, Notes §3.4 Table 3): the first n_beacon queries a
//            buffer is offered; later ones are ignored, the merge keeps it;
//   random  (random history, Notes §3.2 Fig. 6): a uniform random sample of
//            n_beacon of all queries offered so far, kept by reservoir
//            sampling (Vitter's Algorithm R).  The count is the number of
//            offers; offer n (0-based) takes slot n while n < n_beacon, else
//            slot floor(r (n + 1) / 2^32) if that is below n_beacon, r being
//            the first word of Philox4x32-10 (Salmon, Moraes, Dror, Shaw,
//            "Parallel random numbers: as easy as 1, 2, 3", SC 2011) at
//            counter (n, buffer, 0, 0) and key (seed, 0).  Collection-phase
//            queries are offered as they come, the cycle's recents at the
//            merge, in ring order, so the beacons stay frozen while the
//            recents are collected.
#include "bkv_device.hpp"
#include "bkv_internal.hpp"

namespace bkv {

namespace {

// Philox4x32-10: per round the counter (c0, c1, c2, c3) becomes
// (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)); the key
// then advances by the Weyl constants.
__device__ __forceinline__ uint32_t philox_first(uint32_t c0, uint32_t c1, uint32_t k0) {
    constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u, kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;
    uint32_t c2 = 0u, c3 = 0u, k1 = 0u;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint32_t hi0 = __umulhi(kM0, c0), lo0 = kM0 * c0;
        const uint32_t hi1 = __umulhi(kM1, c2), lo1 = kM1 * c2;
        const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
        k0 += kW0;
        k1 += kW1;
    }
    return c0;
}

// Slot that offer n of buffer b goes to, or -1 if it is dropped.
__device__ __forceinline__ int reservoir_slot(uint32_t seed, int64_t b, int n, int nb) {
    if (n < nb) return n;
    const uint32_t r = philox_first((uint32_t)n, (uint32_t)b, seed);
    const uint32_t j = (uint32_t)(((uint64_t)r * (uint64_t)((uint32_t)n + 1u)) >> 32);
    return j < (uint32_t)nb ? (int)j : -1;
}

// One offer per buffer: thread per 16-byte piece of the new query.  All
// pieces of a buffer lie in one wave, so every lane reads the count before
// the piece-0 lane writes it.
template <int D>
__global__ __launch_bounds__(256) void offer_kernel(FpsArgs a) {
    constexpr int kPieces = D / 8;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t b = t / kPieces;
    const int piece = (int)(t % kPieces);
    if (b >= a.nbuf) return;
    const int nb = a.n_beacon;
    const int n = a.qcount[b] > 0 ? a.qcount[b] : 0;
    int slot;
    if (a.src == kSrcInitial) slot = n < nb ? n : -1;
    else slot = reservoir_slot(a.seed, b, n, nb);
    if (slot >= 0)
        reinterpret_cast<u32x4_t*>(a.qbuf + (b * a.qcap + slot) * D)[piece] =
            reinterpret_cast<const u32x4_t*>(a.q_new + b * D)[piece];
    if (a.fps_sel)
        for (int i = piece; i < nb; i += kPieces) a.fps_sel[b * nb + i] = -1;
    if (piece == 0 && (a.src == kSrcRandom || slot >= 0)) a.qcount[b] = n + 1;
}

// The random source's merge: the n_recent_q recents offered in ring order, one
// wave per buffer.  Lane i decides recent i's slot; a slot keeps the last
// recent that lands in it.
template <int D>
__global__ __launch_bounds__(256) void offer_merge_kernel(FpsArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t b = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (b >= a.nbuf) return;
    const int nb = a.n_beacon, nrq = a.n_recent_q;
    const int n0 = a.qcount[b] > 0 ? a.qcount[b] : 0;
    const int slot = lane < nrq ? reservoir_slot(a.seed, b, n0 + lane, nb) : -1;
    bool last = slot >= 0;
    for (int k = 0; k < nrq; ++k) {
        const int sk = __shfl(slot, k, 64);
        if (k > lane && sk == slot) last = false;
    }
    if (last) {
        const u32x4_t* src = reinterpret_cast<const u32x4_t*>(a.q_recent + (b * nrq + lane) * D);
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(a.qbuf + (b * a.qcap + slot) * D);
#pragma unroll
        for (int p = 0; p < D / 8; ++p) dst[p] = src[p];
    }
    if (a.fps_sel)
        for (int i = lane; i < nb; i += 64) a.fps_sel[b * nb + i] = -1;
    if (lane == 0 && nrq > 0) a.qcount[b] = n0 + nrq;   // no recents: nothing offered, the count stays
}

// fps_sel of the initial source's merge (nothing else changes).
__global__ __launch_bounds__(256) void fill_sel_kernel(int32_t* sel, int64_t n) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t < n) sel[t] = -1;
}

// Prefill under the initial or random source: one 256-thread workgroup per
// buffer.  initial: the first min(P, n_beacon) prompt rows; random: every
// prompt row offered in order, each slot keeping the last offer that lands
// in it (an LDS max over the offers), count P.
template <int D>
__global__ __launch_bounds__(256) void prefill_src_kernel(PrefillArgs a) {
    constexpr int kPieces = D / 8;
    __shared__ int last[32];
    const int b = blockIdx.x, tid = threadIdx.x;
    if (b >= a.nbuf) return;
    const int nb = a.n_beacon, P = a.P;
    const bkv_bf16* Q = a.q + (size_t)b * a.q_stride;
    bkv_bf16* buf = a.qbuf + (size_t)b * a.qcap * D;
    if (tid < 32) last[tid] = -1;
    __syncthreads();
    if (a.src == kSrcInitial) {
        for (int s = tid; s < nb && s < P; s += 256) last[s] = s;
    } else {
        for (int n = tid; n < P; n += 256) {
            const int j = reservoir_slot(a.seed, b, n, nb);
            if (j >= 0) atomicMax(&last[j], n);
        }
    }
    __syncthreads();
    for (int e = tid; e < nb * kPieces; e += 256) {
        const int s = e / kPieces, p = e % kPieces;
        if (last[s] >= 0)
            reinterpret_cast<u32x4_t*>(buf + (size_t)s * D)[p] =
                reinterpret_cast<const u32x4_t*>(Q + (size_t)last[s] * D)[p];
    }
    if (a.fps_sel)
        for (int i = tid; i < nb; i += 256) a.fps_sel[(size_t)b * nb + i] = last[i];
    if (tid == 0) a.qcount[b] = a.src == kSrcInitial ? (P < nb ? P : nb) : P;
}

}  // namespace

hipError_t launch_offer(const FpsArgs& a, int d, hipStream_t st) {
    if (a.nbuf <= 0) return hipSuccess;
    const int64_t threads = (int64_t)a.nbuf * (d / 8);
    dim3 g((unsigned)((threads + 255) / 256)), blk(256);
    if (d == 64) hipLaunchKernelGGL(offer_kernel<64>, g, blk, 0, st, a);
    else hipLaunchKernelGGL(offer_kernel<128>, g, blk, 0, st, a);
    return hipGetLastError();
}

hipError_t launch_offer_merge(const FpsArgs& a, int d, hipStream_t st) {
    if (a.nbuf <= 0) return hipSuccess;
    if (a.src == kSrcInitial || a.src == kSrcNaive) {   // the buffer stays as it is
        if (!a.fps_sel || a.n_beacon == 0) return hipSuccess;
        const int64_t n = (int64_t)a.nbuf * a.n_beacon;
        hipLaunchKernelGGL(fill_sel_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a.fps_sel, n);
        return hipGetLastError();
    }
    dim3 g((unsigned)((a.nbuf + 3) / 4)), blk(256);
    if (d == 64) hipLaunchKernelGGL(offer_merge_kernel<64>, g, blk, 0, st, a);
    else hipLaunchKernelGGL(offer_merge_kernel<128>, g, blk, 0, st, a);
    return hipGetLastError();
}

hipError_t launch_prefill_src(const PrefillArgs& a, int d, hipStream_t st) {
    if (a.nbuf <= 0) return hipSuccess;
    if (d == 64) hipLaunchKernelGGL(prefill_src_kernel<64>, dim3(a.nbuf), dim3(256), 0, st, a);
    else hipLaunchKernelGGL(prefill_src_kernel<128>, dim3(a.nbuf), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace bkv
