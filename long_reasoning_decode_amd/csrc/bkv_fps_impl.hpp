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
// An argmin is a DPP minimum over the 32 candidate lanes followed by the
// lowest lane whose value equals it (a ballot and a find-first-set), which is
// the lowest index among equal values.  Each wave uses only its own LDS area,
// so waves of one workgroup never wait for each other.
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
    union {
        float x[kStageK][kXStride];  // x[k - k0][row], while the Gram accumulates
        float c[kMaxRows][kCStride]; // then the Gram, then the cosines
    };
    float nrm[kMaxRows];
    int sel[kMaxRows];
    int row_of[kMaxRows];            // source row of each destination row of a compaction
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

// Integer key ordered as the float v with -0 taken as +0 (v not NaN).
__device__ __forceinline__ int order_key(float v) {
    const int b = __float_as_int(v + 0.0f);
    return b ^ ((b >> 31) & 0x7FFFFFFF);
}

// Disabled rows (ROW_MASK) read INT_MAX, the identity of the minimum.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_min_step(int k) {
    return min(k, __builtin_amdgcn_update_dpp(0x7FFFFFFF, k, CTRL, ROW_MASK, 0xF, false));
}

// Lowest lane among 0..31 holding the smallest v (lanes 32..63 must hold
// +inf, and no lane NaN); the same in every lane.  Equal values (+0 and -0
// included) go to the lower lane, as in a scan that keeps the first minimum.
__device__ __forceinline__ int argmin32(float v) {
    const int k = order_key(v);
    int m = dpp_min_step<0xB1>(k);        // quad_perm [1,0,3,2]
    m = dpp_min_step<0x4E>(m);            // quad_perm [2,3,0,1]
    m = dpp_min_step<0x141>(m);           // row_half_mirror
    m = dpp_min_step<0x140>(m);           // row_mirror: every lane of a row holds the row's minimum
    m = dpp_min_step<0x142, 0xA>(m);      // row_bcast15: rows 1 and 3 also take the previous row's
    return __builtin_ctzll(__ballot(k == __builtin_amdgcn_readlane(m, 31)));
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
    wave_lds_sync();   // the last reads of x are done before c overwrites it
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
            const float q = acc[a][b] / den;
            acc[a][b] = ((ni == 0.0f) | (nj == 0.0f)) ? 0.0f : q;
        }
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) s.c[4 * bi + a][4 * bj + b] = acc[a][b];
    wave_lds_sync();

    // seed: lowest mean cosine (row sums read down the columns: the matrix is symmetric bit for bit)
    float v = __builtin_inff();
    {
        const int c0 = lane & (kMaxRows - 1);
        float sum = 0.0f;
#pragma unroll 8
        for (int j = 0; j < n; ++j) sum = sum + s.c[j][c0];
        if (lane < n) v = sum / (float)n;
    }
    const int p = argmin32(v);
    // lane j < n: S_j (cosines are read along row r, equal to column r); lane i < m: the i-th pick
    const int col = lane & (kMaxRows - 1);
    float S = s.c[p][col];
    bool taken = lane == p;
    int pick = p;
    for (int it = 1; it < m; ++it) {
        const float cv = ((lane < n) & !taken) ? S : __builtin_inff();
        const int r = argmin32(cv);
        taken = taken | (lane == r);
        pick = lane == it ? r : pick;
        const float c = s.c[r][col];
        S = (c > S) ? c : S;
    }
    if (lane < m) s.sel[lane] = pick;
    wave_lds_sync();
    return (uint32_t)__ballot(taken);
}

// Copy the rows in `mask` (ascending) to dst[0..), dst == src0 (in place;
// rows r < n0 come from src0, the rest from src1).  Rows already in place
// are skipped.  The rows go in groups of 8
// destinations, each group's loads issued (and, by in-order completion,
// returned) before its stores; a kept row's source slot is never below its
// destination, so no group reads a slot an earlier group wrote.
template <int D>
__device__ void write_rows(Smem& s, uint32_t mask, bkv_bf16* src0, int n0, const bkv_bf16* src1, int lane) {
    constexpr int kChunks = D / 8;                          // 16-byte pieces per row
    constexpr int kGroup = 8;                               // destination rows per group
    constexpr int kPer = kGroup * kChunks / 64;             // pieces per lane per group
    if (lane < kMaxRows && ((mask >> lane) & 1u)) s.row_of[__popc(mask & ((1u << lane) - 1u))] = lane;
    wave_lds_sync();
    const int cnt = __popc(mask);
    // destinations below the first dropped row that also come from src0 are already in place
    const int dropped = mask == 0xFFFFFFFFu ? kMaxRows : __builtin_ctz(~mask);
    const int first = dropped < n0 ? dropped : n0;
    for (int g0 = first & ~(kGroup - 1); g0 < cnt; g0 += kGroup) {
        u32x4_t buf[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int ci = lane + 64 * j;
            const int w = g0 + ci / kChunks, kc = ci % kChunks;
            if ((w >= first) & (w < cnt)) {
                const int r = s.row_of[w];
                buf[j] = *reinterpret_cast<const u32x4_t*>(cand_row(src0, n0, src1, r, D) + kc * 8);
            }
        }
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int ci = lane + 64 * j;
            const int w = g0 + ci / kChunks, kc = ci % kChunks;
            if ((w >= first) & (w < cnt)) *reinterpret_cast<u32x4_t*>(src0 + (size_t)w * D + kc * 8) = buf[j];
        }
    }
    wave_lds_sync();   // row_of reads done before the next use of the area
}

constexpr int kMaxBuffersPerWave = 16;

// The continual FPS buffer update (Notes §2.2, Eq. 9) of the nw buffers
// b0 .. b0 + nw - 1 (nw <= kMaxBuffersPerWave) by one wave: append each buffer's new query at
// slot c = qcount (clamped to [0, B_Q^max - 1]); a buffer whose count reaches
// B_Q^max becomes FPS(buffer, n_beacon), survivors in ascending slot order,
// count n_beacon.  All counts and query pieces are loaded at once (one memory
// latency per wave), and the sampling reads each new row from q_new, so
// nothing it reads depends on the appends' stores.
template <int D>
__device__ void update_wave(const FpsArgs& a, int b0, int nw, Smem& s, int lane) {
    constexpr int kPieces = D / 8;                 // 16-byte pieces per row
    constexpr int kPerPass = kWave / kPieces;      // buffers per pass of the wave
    const int bqmax = a.n_beacon + a.n_recent_q;
    const int m = a.n_beacon;
    const int c_l = lane < nw ? clampi(a.qcount[b0 + lane], 0, bqmax - 1) : 0;   // count of buffer b0 + lane
    constexpr int kMaxPass = (kMaxBuffersPerWave + kPerPass - 1) / kPerPass;
    u32x4_t piece[kMaxPass];
#pragma unroll
    for (int p = 0; p < kMaxPass; ++p) {
        const int bi = p * kPerPass + lane / kPieces;
        if (p * kPerPass < nw && bi < nw)
            piece[p] = reinterpret_cast<const u32x4_t*>(a.q_new + (size_t)(b0 + bi) * D)[lane % kPieces];
    }
#pragma unroll
    for (int p = 0; p < kMaxPass; ++p) {
        const int bi = p * kPerPass + lane / kPieces;
        const int c = __shfl(c_l, bi < kWave ? bi : 0, kWave);
        if (p * kPerPass < nw && bi < nw)
            reinterpret_cast<u32x4_t*>(a.qbuf + ((size_t)(b0 + bi) * a.qcap + c) * D)[lane % kPieces] = piece[p];
    }
    const int n_l = c_l + 1;
    const bool full = lane < nw && n_l >= bqmax && n_l > m;
    if (lane < nw && !full) {
        a.qcount[b0 + lane] = n_l;
    }
    if (a.fps_sel && m > 0) {   // buffers that do not sample: -1s (all kept when n_recent_q == 0)
        const int passes = (nw * m + kWave - 1) / kWave;
        for (int p = 0; p < passes; ++p) {   // uniform loop: every lane takes part in the shuffles
            const int e = p * kWave + lane;
            const int bi = e < nw * m ? e / m : 0, i = e % m;
            const int n = __shfl(n_l, bi, kWave);
            const bool f = __shfl((int)full, bi, kWave) != 0;
            if (e < nw * m && !f) a.fps_sel[(size_t)(b0 + bi) * m + i] = (n >= bqmax && i < n) ? i : -1;
        }
    }
    uint64_t todo = __ballot(full);
    while (todo) {
        const int bi = __builtin_ctzll(todo);
        todo &= todo - 1;
        const int b = b0 + bi;
        const int c = __builtin_amdgcn_readlane(c_l, bi);   // uniform: the select's loops stay scalar
        bkv_bf16* buf = a.qbuf + (size_t)b * a.qcap * D;
        const bkv_bf16* qn = a.q_new + (size_t)b * D;
        const uint32_t mask = select<D>(s, buf, c, qn, c + 1, m, lane);
        write_rows<D>(s, mask, buf, c, qn, lane);
        if (lane == 0) a.qcount[b] = m;
        if (a.fps_sel)
            for (int i = lane; i < m; i += kWave) a.fps_sel[(size_t)b * m + i] = s.sel[i];
    }
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
        write_rows<D>(s, n >= 32 ? 0xFFFFFFFFu : ((1u << n) - 1u), buf, nb, rec, lane);
        if (lane == 0) a.qcount[b] = n;
        if (a.fps_sel)
            for (int i = lane; i < m; i += kWave) a.fps_sel[(size_t)b * m + i] = i < n ? i : -1;
        return;
    }
    const uint32_t mask = select<D>(s, buf, nb, rec, n, m, lane);
    write_rows<D>(s, mask, buf, nb, rec, lane);
    if (lane == 0) a.qcount[b] = m;
    if (a.fps_sel)
        for (int i = lane; i < m; i += kWave) a.fps_sel[(size_t)b * m + i] = s.sel[i];
}

}  // namespace fps
}  // namespace bkv
