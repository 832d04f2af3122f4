// bkv_fps_impl.hpp -- continual farthest point sampling of pre-RoPE queries,
// one wavefront per query buffer (device functions of the buffer-update and
// merge kernels).
//
// The Gram matrix of the (at most 32) candidates is register-blocked 4 x 4
// per lane (64 lanes cover the 32 x 32 entries); the rows stream through LDS
// in stages of 32 columns, transposed ([k][row]) so one 16-byte read gives
// four rows' k-th elements.
//
// The arithmetic follows one fixed fp32 order so that the selected indices
// are reproducible bit for bit (Notes §2.2, App. Alg. 1):
//   dot_ij = fma chain over k = 0..d-1 from +0 (bf16 products are exact),
//   nrm_i  = sqrt(dot_ii) (correctly rounded), cos_ij = dot_ij / (nrm_i*nrm_j),
//   0 when a norm is 0, a_i = (left-to-right sum of cos_ij over j) / n,
// then argmin a (seed), and n_beacon - 1 greedy steps r = argmin over the
// untaken rows of S, S_j = max(S_j, cos_jr).  Ties go to the lower index.
// The argmins are DPP reductions inside each 16-lane row plus one scalar
// comparison of the two rows that hold candidates.  Each wave uses only its
// own LDS area, so waves of one workgroup never wait for each other.
#pragma once

#include "bkv_device.hpp"
#include "bkv_internal.hpp"

namespace bkv {
namespace fps {

constexpr int kMaxRows = 32;
constexpr int kStageK = 32;              // Gram columns staged per round
constexpr int kXStride = kMaxRows + 4;   // floats per k-row of the stage (16-B aligned)
constexpr int kCStride = kMaxRows + 1;   // floats per row of the cosine matrix

struct Smem {
    float x[kStageK][kXStride];      // x[k - k0][row]
    float c[kMaxRows][kCStride];     // Gram, then cosines
    float nrm[kMaxRows];
    int sel[kMaxRows];
};

// The wave's LDS writes are complete and visible to its other lanes; the
// compiler does not move LDS accesses across this point.
__device__ __forceinline__ void wave_lds_sync() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Source row r of the candidate set: rows r < n0 from src0, the rest from src1.
__device__ __forceinline__ const bkv_bf16* cand_row(const bkv_bf16* src0, int n0, const bkv_bf16* src1,
                                                    int r, int D) {
    return r < n0 ? src0 + (size_t)r * D : src1 + (size_t)(r - n0) * D;
}

template <int CTRL>
__device__ __forceinline__ void dpp_argmin_step(float& v, int& i) {
    const float v2 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
    const int i2 = __builtin_amdgcn_update_dpp(0, i, CTRL, 0xF, 0xF, false);
    const bool take = (v2 < v) || (v2 == v && i2 < i);
    v = take ? v2 : v;
    i = take ? i2 : i;
}

// Argmin of (v, i) over lanes 0..31 (lanes 32..63 must hold +inf); every lane
// receives the winning index.  Smallest v, then smallest i.
__device__ __forceinline__ int argmin32(float v, int i) {
    dpp_argmin_step<0xB1>(v, i);    // quad_perm [1,0,3,2]
    dpp_argmin_step<0x4E>(v, i);    // quad_perm [2,3,0,1]
    dpp_argmin_step<0x141>(v, i);   // row_half_mirror
    dpp_argmin_step<0x140>(v, i);   // row_mirror: every lane of a row holds the row's argmin
    const float v0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const int i0 = __builtin_amdgcn_readlane(i, 0);
    const float v1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const int i1 = __builtin_amdgcn_readlane(i, 16);
    return ((v1 < v0) || (v1 == v0 && i1 < i0)) ? i1 : i0;
}

// FPS over candidate rows [0, n) (n > m >= 1); leaves the selection order in
// s.sel[0..m) and returns the 32-bit mask of taken rows.
template <int D>
__device__ uint32_t select(Smem& s, const bkv_bf16* src0, int n0, const bkv_bf16* src1, int n, int m, int lane) {
    const int bi = lane >> 3, bj = lane & 7;
    float acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = 0.0f;
    // each lane stages two 16-byte pieces (row r, 8 consecutive k) per round
    const int r_a = lane & 31, kc_a = lane >> 5;
    for (int k0 = 0; k0 < D; k0 += kStageK) {
        u32x4_t w[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int kc = kc_a + 2 * q;                    // 0..3: 8-column piece within the stage
            w[q] = u32x4_t{0u, 0u, 0u, 0u};
            if (r_a < n) w[q] = *reinterpret_cast<const u32x4_t*>(cand_row(src0, n0, src1, r_a, D) + k0 + kc * 8);
        }
        wave_lds_sync();  // the previous round's reads of s.x are done
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int kc = kc_a + 2 * q;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s.x[kc * 8 + 2 * e][r_a] = __uint_as_float(w[q][e] << 16);
                s.x[kc * 8 + 2 * e + 1][r_a] = __uint_as_float(w[q][e] & 0xFFFF0000u);
            }
        }
        wave_lds_sync();
#pragma unroll 8
        for (int k = 0; k < kStageK; ++k) {
            const f32x4_t xa = *reinterpret_cast<const f32x4_t*>(&s.x[k][4 * bi]);
            const f32x4_t xb = *reinterpret_cast<const f32x4_t*>(&s.x[k][4 * bj]);
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) acc[a][b] = __builtin_fmaf(xa[a], xb[b], acc[a][b]);
        }
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) s.c[4 * bi + a][4 * bj + b] = acc[a][b];
    wave_lds_sync();
    if (lane < kMaxRows) s.nrm[lane] = __builtin_sqrtf(s.c[lane][lane]);
    wave_lds_sync();
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const float ni = s.nrm[4 * bi + a];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float nj = s.nrm[4 * bj + b];
            const float den = ni * nj;
            acc[a][b] = (ni == 0.0f || nj == 0.0f) ? 0.0f : acc[a][b] / den;
        }
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) s.c[4 * bi + a][4 * bj + b] = acc[a][b];
    wave_lds_sync();

    // seed: lowest mean cosine
    float v = __builtin_inff();
    if (lane < n) {
        float sum = 0.0f;
        for (int j = 0; j < n; ++j) sum = sum + s.c[lane][j];
        v = sum / (float)n;
    }
    const int p = argmin32(v, lane);
    float S = (lane < n) ? s.c[lane][p] : 0.0f;
    bool taken = (lane == p);
    if (lane == 0) s.sel[0] = p;
    for (int it = 1; it < m; ++it) {
        const float cv = (lane < n && !taken) ? S : __builtin_inff();
        const int r = argmin32(cv, lane);
        taken = taken || (lane == r);
        if (lane == 0) s.sel[it] = r;
        if (lane < n) {
            const float c = s.c[lane][r];
            S = (c > S) ? c : S;
        }
    }
    wave_lds_sync();
    return (uint32_t)__ballot(taken);
}

// Copy the rows in `mask` (ascending) to dst[0..).  dst may be src0 itself:
// a kept row's source slot is never below its destination, and every load is
// issued (and, by in-order completion, returned) before the first store.
template <int D>
__device__ void write_rows(uint32_t mask, const bkv_bf16* src0, int n0, const bkv_bf16* src1, bkv_bf16* dst,
                           int lane) {
    constexpr int kChunks = D / 8;                          // 16-byte pieces per row
    constexpr int kPer = kMaxRows * kChunks / 64;           // pieces per lane, at most
    const int cnt = __popc(mask);
    u32x4_t buf[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int ci = lane + 64 * j;
        const int w = ci / kChunks, kc = ci % kChunks;
        if (w < cnt) {
            uint32_t mm = mask;
            for (int q = 0; q < w; ++q) mm &= mm - 1;
            const int r = __ffs(mm) - 1;
            buf[j] = *reinterpret_cast<const u32x4_t*>(cand_row(src0, n0, src1, r, D) + kc * 8);
        }
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int ci = lane + 64 * j;
        const int w = ci / kChunks, kc = ci % kChunks;
        if (w < cnt) *reinterpret_cast<u32x4_t*>(dst + (size_t)w * D + kc * 8) = buf[j];
    }
}

// Sampling round of the continual FPS buffer update for buffer b (Notes §2.2,
// Eq. 9), after the step's query has been appended: a buffer whose count has
// reached B_Q^max becomes FPS(buffer, n_beacon), survivors in ascending slot
// order, count n_beacon; other buffers are left as they are.
template <int D>
__device__ void compress_one(const FpsArgs& a, int b, Smem& s, int lane) {
    const int bqmax = a.n_beacon + a.n_recent_q;
    const int m = a.n_beacon;
    bkv_bf16* buf = a.qbuf + (size_t)b * a.qcap * D;
    const int n = a.qcount[b];
    if (n != bqmax) {
        if (a.fps_sel)
            for (int i = lane; i < m; i += kWave) a.fps_sel[(size_t)b * m + i] = -1;
        return;
    }
    if (n <= m) {  // no sampling: keep all rows (only when n_recent_q == 0)
        if (a.fps_sel)
            for (int i = lane; i < m; i += kWave) a.fps_sel[(size_t)b * m + i] = i < n ? i : -1;
        return;
    }
    const uint32_t mask = select<D>(s, buf, n, buf, n, m, lane);
    write_rows<D>(mask, buf, n, buf, buf, lane);
    if (lane == 0) a.qcount[b] = m;
    if (a.fps_sel)
        for (int i = lane; i < m; i += kWave) a.fps_sel[(size_t)b * m + i] = s.sel[i];
}

// End-of-cycle merge of buffer b: FPS over beacons ++ recents (Notes §2.2, App. Alg. 2).
template <int D>
__device__ void merge_one(const FpsArgs& a, int b, Smem& s, int lane) {
    const int m = a.n_beacon;
    bkv_bf16* buf = a.qbuf + (size_t)b * a.qcap * D;
    const bkv_bf16* rec = a.q_recent + (size_t)b * a.n_recent_q * D;
    const int nb = clampi(a.qcount[b], 0, m);
    const int n = nb + a.n_recent_q;
    if (m <= 0) {  // nothing is kept
        if (lane == 0) a.qcount[b] = 0;
        return;
    }
    if (n <= m) {
        write_rows<D>(n >= 32 ? 0xFFFFFFFFu : ((1u << n) - 1u), buf, nb, rec, buf, lane);
        if (lane == 0) a.qcount[b] = n;
        if (a.fps_sel)
            for (int i = lane; i < m; i += kWave) a.fps_sel[(size_t)b * m + i] = i < n ? i : -1;
        return;
    }
    const uint32_t mask = select<D>(s, buf, nb, rec, n, m, lane);
    write_rows<D>(mask, buf, nb, rec, buf, lane);
    if (lane == 0) a.qcount[b] = m;
    if (a.fps_sel)
        for (int i = lane; i < m; i += kWave) a.fps_sel[(size_t)b * m + i] = s.sel[i];
}

}  // namespace fps
}  // namespace bkv
