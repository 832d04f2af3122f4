// bkv_select.hip -- keep-set kernel: one workgroup per unit (the work is in
// bkv_select_impl.hpp).
#include "bkv_internal.hpp"
#include "bkv_select_impl.hpp"

namespace bkv {

namespace {

constexpr int kSelBlock = 256;

__global__ __launch_bounds__(kSelBlock) void select_kernel(SelectArgs a) {
    extern __shared__ uint32_t keys[];
    __shared__ uint32_t hist[256];
    __shared__ int wsum[kSelBlock / 64];
    __shared__ uint32_t bin[2];
    const int u = blockIdx.x;
    if (u >= a.units) return;
    sel::Scratch w{keys, hist, wsum, bin};
    sel::select_unit<kSelBlock>(a.scores + (size_t)u * a.n_len, a.n_len, a.budget, a.n_prefix, a.n_recent_kv,
                                a.idx + (size_t)u * a.budget, nullptr, w);
}

}  // namespace

hipError_t launch_select(const SelectArgs& a, hipStream_t st) {
    if (a.units <= 0 || a.budget <= 0) return hipSuccess;
    const size_t smem = (size_t)(a.n_len > a.budget ? a.n_len : 1) * 4;
    hipLaunchKernelGGL(select_kernel, dim3(a.units), dim3(kSelBlock), smem, st, a);
    return hipGetLastError();
}

}  // namespace bkv
