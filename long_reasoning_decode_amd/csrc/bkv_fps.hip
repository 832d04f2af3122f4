// bkv_fps.hip -- continual farthest point sampling of pre-RoPE queries.
//
// One wavefront owns one query buffer (at most 32 candidate rows).  The
// candidates are staged in LDS as fp32, transposed ([k][row]) so that a lane
// can fetch four rows' k-th elements with one 16-byte read; the 32 x 32 Gram
// matrix is register-blocked 4 x 4 per lane (64 lanes cover 1024 entries).
//
// The arithmetic follows one fixed fp32 order so that the selected indices
// are reproducible bit for bit (Notes §2.2, App. Alg. 1):
//   dot_ij = fma chain over k = 0..d-1 from +0 (bf16 products are exact),
//   nrm_i  = sqrt(dot_ii) (correctly rounded), cos_ij = dot_ij / (nrm_i*nrm_j),
//   0 when a norm is 0, a_i = (left-to-right sum of cos_ij over j) / n,
// then argmin a (seed), and n_beacon - 1 greedy steps r = argmin over the
// untaken rows of S, S_j = max(S_j, cos_jr).  Ties go to the lower index.
#include "bkv_device.hpp"
#include "bkv_internal.hpp"

namespace bkv {

namespace {

constexpr int kMaxRows = 32;
constexpr int kXStride = kMaxRows + 4;   // floats per k-row of the transposed stage (16-B aligned)
constexpr int kCStride = kMaxRows + 1;   // floats per row of the cosine matrix

template <int D>
struct FpsSmem {
    float x[D][kXStride];            // x[k][row]
    float c[kMaxRows][kCStride];     // Gram, then cosines
    float nrm[kMaxRows];
    int sel[kMaxRows];
};

// Stage rows [0, n) into s.x: row r < n0 comes from src0 + r*stride0, rows
// n0 <= r < n from src1 + (r - n0)*stride1.  Rows n..31 are zero.
template <int D>
__device__ void stage_rows(FpsSmem<D>& s, const bkv_bf16* src0, int n0, size_t stride0,
                           const bkv_bf16* src1, int n, size_t stride1, int lane) {
    constexpr int kChunks = D / 8;  // 16-byte chunks per row
    for (int ci = lane; ci < kMaxRows * kChunks; ci += kWave) {
        int r = ci % kMaxRows;
        int kc = ci / kMaxRows;
        u32x4_t w = {0u, 0u, 0u, 0u};
        if (r < n) {
            const bkv_bf16* p = r < n0 ? src0 + (size_t)r * stride0 : src1 + (size_t)(r - n0) * stride1;
            w = *reinterpret_cast<const u32x4_t*>(p + kc * 8);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            s.x[kc * 8 + 2 * e][r] = __uint_as_float(w[e] << 16);
            s.x[kc * 8 + 2 * e + 1][r] = __uint_as_float(w[e] & 0xFFFF0000u);
        }
    }
}

// FPS over the n staged rows (n > m >= 1).  Leaves the selection order in
// s.sel[0..m) and returns, in every lane, the 32-bit mask of taken rows.
template <int D>
__device__ uint32_t fps_select(FpsSmem<D>& s, int n, int m, int lane) {
    // Gram matrix, 4 x 4 block per lane.
    const int bi = lane >> 3, bj = lane & 7;
    float acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = 0.0f;
    for (int k = 0; k < D; ++k) {
        f32x4_t xa = *reinterpret_cast<const f32x4_t*>(&s.x[k][4 * bi]);
        f32x4_t xb = *reinterpret_cast<const f32x4_t*>(&s.x[k][4 * bj]);
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[a][b] = __builtin_fmaf(xa[a], xb[b], acc[a][b]);
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) s.c[4 * bi + a][4 * bj + b] = acc[a][b];
    __syncthreads();
    if (lane < kMaxRows) s.nrm[lane] = __builtin_sqrtf(s.c[lane][lane]);
    __syncthreads();
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        float ni = s.nrm[4 * bi + a];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            float nj = s.nrm[4 * bj + b];
            float den = ni * nj;
            acc[a][b] = (ni == 0.0f || nj == 0.0f) ? 0.0f : acc[a][b] / den;
        }
    }
    __syncthreads();
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) s.c[4 * bi + a][4 * bj + b] = acc[a][b];
    __syncthreads();

    // Seed: lowest mean cosine.
    float v = __builtin_inff();
    int vi = kWave + lane;
    if (lane < n) {
        float sum = 0.0f;
        for (int j = 0; j < n; ++j) sum = sum + s.c[lane][j];
        v = sum / (float)n;
        vi = lane;
    }
    wave_argmin(v, vi);
    const int p = vi;
    float S = (lane < n) ? s.c[lane][p] : 0.0f;
    bool taken = (lane == p);
    if (lane == 0) s.sel[0] = p;
    for (int it = 1; it < m; ++it) {
        float cv = (lane < n && !taken) ? S : __builtin_inff();
        int ci = (lane < n && !taken) ? lane : kWave + lane;
        wave_argmin(cv, ci);
        const int r = ci;
        if (lane == r) taken = true;
        if (lane == 0) s.sel[it] = r;
        if (lane < n) {
            float c = s.c[lane][r];
            S = (c > S) ? c : S;
        }
    }
    __syncthreads();
    return (uint32_t)__ballot(taken);
}

// Write the taken rows, ascending, to dst[0..), converting back to bf16
// (exact: the staged values came from bf16).
template <int D>
__device__ void write_rows(const FpsSmem<D>& s, uint32_t mask, bkv_bf16* dst, int lane) {
    constexpr int kChunks = D / 8;
    const int cnt = __popc(mask);
    for (int ci = lane; ci < cnt * kChunks; ci += kWave) {
        int w = ci / kChunks, kc = ci % kChunks;
        // row = position of the w-th set bit
        uint32_t mm = mask;
        for (int q = 0; q < w; ++q) mm &= mm - 1;
        int r = __ffs(mm) - 1;
        u32x4_t o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            uint32_t lo = __float_as_uint(s.x[kc * 8 + 2 * e][r]) >> 16;
            uint32_t hi = __float_as_uint(s.x[kc * 8 + 2 * e + 1][r]) & 0xFFFF0000u;
            o[e] = lo | hi;
        }
        *reinterpret_cast<u32x4_t*>(dst + (size_t)w * D + kc * 8) = o;
    }
}

// Rows copied as they are (no sampling): src rows of the staged set [0, n).
template <int D>
__device__ void write_all(const FpsSmem<D>& s, int n, bkv_bf16* dst, int lane) {
    write_rows<D>(s, n >= 32 ? 0xFFFFFFFFu : ((1u << n) - 1u), dst, lane);
}

template <int D>
__global__ __launch_bounds__(kWave) void fps_update_kernel(FpsArgs a) {
    __shared__ FpsSmem<D> s;
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    if (b >= a.nbuf) return;
    const int bqmax = a.n_beacon + a.n_recent_q;
    bkv_bf16* buf = a.qbuf + (size_t)b * a.qcap * D;
    const bkv_bf16* qn = a.q_new + (size_t)b * D;
    const int c = clampi(a.qcount[b], 0, bqmax - 1);
    const int n = c + 1;
    if (n < bqmax) {
        // append only
        for (int kc = lane; kc < D / 8; kc += kWave)
            *reinterpret_cast<u32x4_t*>(buf + (size_t)c * D + kc * 8) =
                *reinterpret_cast<const u32x4_t*>(qn + kc * 8);
        if (lane == 0) a.qcount[b] = n;
        if (a.fps_sel)
            for (int i = lane; i < a.n_beacon; i += kWave) a.fps_sel[(size_t)b * a.n_beacon + i] = -1;
        return;
    }
    stage_rows<D>(s, buf, c, D, qn, n, D, lane);
    __syncthreads();
    const int m = a.n_beacon;
    if (n <= m) {
        write_all<D>(s, n, buf, lane);
        if (lane == 0) a.qcount[b] = n;
        if (a.fps_sel)
            for (int i = lane; i < m; i += kWave) a.fps_sel[(size_t)b * m + i] = i < n ? i : -1;
        return;
    }
    uint32_t mask = m > 0 ? fps_select<D>(s, n, m, lane) : 0u;
    write_rows<D>(s, mask, buf, lane);
    if (lane == 0) a.qcount[b] = m;
    if (a.fps_sel)
        for (int i = lane; i < m; i += kWave) a.fps_sel[(size_t)b * m + i] = s.sel[i];
}

template <int D>
__global__ __launch_bounds__(kWave) void fps_merge_kernel(FpsArgs a) {
    __shared__ FpsSmem<D> s;
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    if (b >= a.nbuf) return;
    const int m = a.n_beacon;
    bkv_bf16* buf = a.qbuf + (size_t)b * a.qcap * D;
    const bkv_bf16* rec = a.q_recent + (size_t)b * a.n_recent_q * D;
    const int nb = clampi(a.qcount[b], 0, m);
    const int n = nb + a.n_recent_q;
    if (m <= 0) {  // nothing is kept
        if (lane == 0) a.qcount[b] = 0;
        return;
    }
    stage_rows<D>(s, buf, nb, D, rec, n, D, lane);
    __syncthreads();
    if (n <= m) {
        write_all<D>(s, n, buf, lane);
        if (lane == 0) a.qcount[b] = n;
        if (a.fps_sel)
            for (int i = lane; i < m; i += kWave) a.fps_sel[(size_t)b * m + i] = i < n ? i : -1;
        return;
    }
    uint32_t mask = fps_select<D>(s, n, m, lane);
    write_rows<D>(s, mask, buf, lane);
    if (lane == 0) a.qcount[b] = m;
    if (a.fps_sel)
        for (int i = lane; i < m; i += kWave) a.fps_sel[(size_t)b * m + i] = s.sel[i];
}

}  // namespace

hipError_t launch_fps(const FpsArgs& a, int d, bool merge, hipStream_t st) {
    if (a.nbuf <= 0) return hipSuccess;
    dim3 grid(a.nbuf), block(kWave);
    if (d == 64) {
        if (merge) hipLaunchKernelGGL(fps_merge_kernel<64>, grid, block, 0, st, a);
        else hipLaunchKernelGGL(fps_update_kernel<64>, grid, block, 0, st, a);
    } else {
        if (merge) hipLaunchKernelGGL(fps_merge_kernel<128>, grid, block, 0, st, a);
        else hipLaunchKernelGGL(fps_update_kernel<128>, grid, block, 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace bkv
