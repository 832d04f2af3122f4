// bkv_evict.hip -- the eviction of one unit by one 8-wave workgroup (Notes
// §2.3, Eq. 7-8): its scores (bkv_score_impl.hpp), its keep set by an LDS
// radix select over them (bkv_select_impl.hpp), and the in-place compaction
// of its K and V rows (bkv_compact_impl.hpp), with nothing but the optional
// outputs leaving the chip in between.  Doing all three in one workgroup
// keeps the unit's keys in the MALL from the first scoring pass to the
// compaction, so only the first pass and the value rows are read from HBM.
// The merge of the query buffers runs as its own launch afterwards.
#include "bkv_compact_impl.hpp"
#include "bkv_score_impl.hpp"
#include "bkv_select_impl.hpp"

namespace bkv {

namespace {

// Select scratch and kept slots, placed in the key ring once scoring is done.
constexpr int kHistOff = 0;        // uint32 [256]
constexpr int kWsumOff = 1024;     // int [waves]
constexpr int kBinOff = 1280;      // uint32 [2]
constexpr int kFirstOff = 1296;    // int
constexpr int kSrcOff = 2048;      // uint16 [budget]

template <int D, int KS, bool MEAN>
__global__ __launch_bounds__(score::kThreads) void evict_kernel(EvictArgs a) {
    using L = score::Layout<D>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    uint32_t* codes = reinterpret_cast<uint32_t*>(smem + L::fixed_bytes(MEAN));
    const int u = blockIdx.x;
    if (u >= a.sc.units) return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int N = a.sc.n_len;

    // scores, then the order codes of the fp32 scores, which the select ranks
    score::unit_codes<D, KS, MEAN>(a.sc, u, smem, codes);
    float* sc_out = a.sc.scores ? a.sc.scores + (size_t)u * N : nullptr;
    for (int j = tid; j < N; j += score::kThreads) {
        const float s = score::score_of<MEAN>(codes[j]);
        if (sc_out) sc_out[j] = s;
        codes[j] = f32_order(s);
    }
    __syncthreads();

    // keep set (kept slots ascending in LDS, and optionally in global memory)
    const int B = a.budget;
    uint16_t* src = reinterpret_cast<uint16_t*>(smem + kSrcOff);
    sel::Scratch w{codes, reinterpret_cast<uint32_t*>(smem + kHistOff), reinterpret_cast<int*>(smem + kWsumOff),
                   reinterpret_cast<uint32_t*>(smem + kBinOff)};
    sel::select_staged<score::kThreads>(N, B, a.n_prefix, a.n_recent_kv, a.idx ? a.idx + (size_t)u * B : nullptr,
                                        src, w);

    // in-place compaction: the first half of the waves move K rows, the second half V rows
    const int Bv = N < B ? N : B;
    int* first_sh = reinterpret_cast<int*>(smem + kFirstOff);
    if (wave == 0) {
        const int f = compact::first_moved(src, Bv, lane);
        if (lane == 0) *first_sh = f;
    }
    __syncthreads();
    const int first = *first_sh;
    constexpr int kHalf = score::kWaves / 2;
    bkv_bf16* X = (wave < kHalf ? a.K : a.V) + (size_t)u * a.sc.cap * D;
    compact::move_rows_wg<D, kHalf>(X, src, first, Bv, wave % kHalf, lane);
}

template <int D, int KS, bool MEAN>
hipError_t launch_one(const EvictArgs& a, hipStream_t st) {
    using L = score::Layout<D>;
    static_assert(kSrcOff + 2 * 8192 <= L::kRingBytes, "select scratch fits in the key ring");
    const size_t smem = L::fixed_bytes(MEAN) + (size_t)a.sc.n_len * 4;
    hipLaunchKernelGGL((evict_kernel<D, KS, MEAN>), dim3(a.sc.units), dim3(score::kThreads), smem, st, a);
    return hipGetLastError();
}

template <int D, bool MEAN>
hipError_t launch_dm(const EvictArgs& a, hipStream_t st) {
    // query heads per workgroup: the smallest power of two >= G; key split KS = waves / heads
    constexpr int W = score::kWaves;
    if (a.sc.G <= 1) return launch_one<D, W, MEAN>(a, st);
    if (a.sc.G <= 2) return launch_one<D, W / 2, MEAN>(a, st);
    if (a.sc.G <= 4) return launch_one<D, W / 4, MEAN>(a, st);
    return launch_one<D, 1, MEAN>(a, st);
}

template <int D>
hipError_t launch_d(const EvictArgs& a, hipStream_t st) {
    return a.sc.pool_mean ? launch_dm<D, true>(a, st) : launch_dm<D, false>(a, st);
}

}  // namespace

hipError_t launch_evict(const EvictArgs& a, int d, hipStream_t st) {
    if (a.sc.units <= 0 || a.sc.n_len <= 0) return hipSuccess;
    return d == 64 ? launch_d<64>(a, st) : launch_d<128>(a, st);
}

}  // namespace bkv
