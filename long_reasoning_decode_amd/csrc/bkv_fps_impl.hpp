// bkv_fps_impl.hpp -- continual farthest point sampling of pre-RoPE queries
// (device functions of the buffer-update and merge kernels).  One wavefront
// samples two buffers at a time, one per half-wave (lanes 0-31 and 32-63):
// lane i of a half holds candidate row i.
//
// The Gram matrices come from the matrix cores: 128 (or 64) fp32 MFMA
// 32x32x1 rank-1 updates, two blocks per instruction (one per buffer), each
// lane feeding the k-th element of its row as both operands.  Each update
// rounds once per element, so the chain is the same sequence of fused
// multiply-adds as a scalar loop over k.
//
// The arithmetic follows one fixed fp32 order so that the selected indices
// are reproducible bit for bit (Notes §2.2, App. Alg. 1):
//   dot_ij = fma chain over k = 0..d-1 from +0 (bf16 products are exact),
//   nrm_i  = sqrt(dot_ii) (correctly rounded), cos_ij = dot_ij / (nrm_i*nrm_j),
//   0 when a norm is 0, a_i = (left-to-right sum of cos_ij over j) / n,
// then argmin a (seed), and n_beacon - 1 greedy steps r = argmin over the
// untaken rows of S, S_j = max(S_j, cos_jr).  Ties go to the lower index.
// An argmin is a DPP minimum over each half's 32 lanes followed by the
// lowest lane whose value equals it (a ballot and a find-first-set), which is
// the lowest index among equal values.  Each wave uses only its own LDS area,
// so waves of one workgroup never wait for each other.
#pragma once

#include "bkv_device.hpp"
#include "bkv_internal.hpp"

namespace bkv {
namespace fps {

constexpr int kMaxRows = 32;
constexpr int kCStride = kMaxRows + 1;   // floats per row of a cosine matrix

typedef float f32x32_t __attribute__((ext_vector_type(32)));

struct Smem {
    float c[2][kMaxRows][kCStride];  // per half: the Gram, then the cosines
    float nrm[2][kMaxRows];
    int sel[2][kMaxRows];
    int row_of[kMaxRows];            // source row of each destination row of a compaction
};

// The wave's LDS writes are complete and visible to its other lanes; the
// compiler does not move LDS accesses across this point.
__device__ __forceinline__ void wave_lds_sync() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Source row r of a candidate set: rows r < n0 from src0, the rest from src1.
__device__ __forceinline__ const bkv_bf16* cand_row(const bkv_bf16* src0, int n0, const bkv_bf16* src1,
                                                    int r, int D) {
    return r < n0 ? src0 + (size_t)r * D : src1 + (size_t)(r - n0) * D;
}

// The candidates of one buffer: n rows, [0, n0) from src0 and [n0, n) from
// src1 (n = 0: no buffer in this half).
struct Cand {
    const bkv_bf16* src0;
    int n0;
    const bkv_bf16* src1;
    int n;
};

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

// Per half-wave: the lowest lane of the half holding the half's smallest
// key, as an index 0..31, in every lane of the half.
__device__ __forceinline__ int argmin_keys_halves(int k, int lane) {
    int m = dpp_min_step<0xB1>(k);        // quad_perm [1,0,3,2]
    m = dpp_min_step<0x4E>(m);            // quad_perm [2,3,0,1]
    m = dpp_min_step<0x141>(m);           // row_half_mirror
    m = dpp_min_step<0x140>(m);           // row_mirror: every lane of a row holds the row's minimum
    m = dpp_min_step<0x142, 0xA>(m);      // row_bcast15: rows 1 and 3 also take the previous row's
    const int m0 = __builtin_amdgcn_readlane(m, 31), m1 = __builtin_amdgcn_readlane(m, 63);
    const uint32_t e0 = (uint32_t)__ballot(k == m0);           // lanes 0..31 holding half 0's minimum
    const uint32_t e1 = (uint32_t)(__ballot(k == m1) >> 32);   // lanes 32..63 holding half 1's
    const int r0 = __builtin_ctz(e0), r1 = __builtin_ctz(e1);
    return lane < 32 ? r0 : r1;
}

// The same for float values (no lane NaN): equal values, +0 and -0
// included, go to the lower lane, as in a scan that keeps the first minimum.
__device__ __forceinline__ int argmin_halves(float v, int lane) { return argmin_keys_halves(order_key(v), lane); }

// Gram entries acc (as laid out by the rank-1 updates) into s.c, the norms
// into s.nrm, then the cosines over the Gram entries in s.c.  The matrices
// are symmetric bit for bit (the products are exact and both triangles
// accumulate them in the same order, and nrm_i nrm_j = nrm_j nrm_i), so
// each cosine is computed once and written to both of its entries: lane i
// of half h takes the pairs (i, (i + k) mod 32), k = 0 .. 16, of set h -- 17
// divisions instead of 32.  An entry (i, i + k) is read as a Gram entry
// only by lane i at step k (and its mirror (i + k, i) only by lane i + k at
// step 32 - k, which exists for k = 16 alone); each step's reads precede its
// writes, so no lane reads an entry another lane has already turned into a
// cosine.
__device__ __forceinline__ void cosines2(Smem& s, const f32x32_t& acc, int h, int i) {
#pragma unroll
    for (int r = 0; r < 32; ++r) s.c[r / 16][8 * ((r % 16) / 4) + 4 * h + (r % 4)][i] = acc[r];
    wave_lds_sync();
    const float ni = __builtin_sqrtf(s.c[h][i][i]);
    s.nrm[h][i] = ni;
    wave_lds_sync();
#pragma unroll 2
    for (int k = 0; k <= kMaxRows / 2; ++k) {
        const int j = (i + k) & (kMaxRows - 1);
        const float g = s.c[h][i][j];
        const float nj = s.nrm[h][j];
        const float cq = g / (ni * nj);
        const float v = ((ni == 0.0f) | (nj == 0.0f)) ? 0.0f : cq;
        s.c[h][i][j] = v;
        s.c[h][j][i] = v;
    }
    wave_lds_sync();
}

// Cosine matrices of both halves' sets into s.c (and the norms into s.nrm).
// Lane i of half h loads row i of set h (lanes past n load a copy of row
// n - 1, or row 0 of src0 in an empty half: their dot products are computed
// but never read) in groups of four 16-byte pieces, issued two groups ahead
// of the group whose 32 rank-1 updates run, so only the first group's latency
// is exposed and at most three groups' registers are held.
template <int D>
__device__ void gram2(Smem& s, const Cand& c0, const Cand& c1, int lane) {
    constexpr int kGroups = D / 32;
    const int h = lane >> 5, i = lane & 31;
    const int n = h ? c1.n : c0.n;
    const bkv_bf16* src0 = h ? c1.src0 : c0.src0;
    const bkv_bf16* src1 = h ? c1.src1 : c0.src1;
    const int n0 = h ? c1.n0 : c0.n0;
    const int ic = i < n ? i : (n > 0 ? n - 1 : 0);
    const bkv_bf16* p = n > 0 ? cand_row(src0, n0, src1, ic, D) : src0;
    constexpr int kAhead = 2;   // groups in flight ahead of the one in use
    u32x4_t g[kAhead + 1][4];
#pragma unroll
    for (int gi = 0; gi < kAhead && gi < kGroups; ++gi)
#pragma unroll
        for (int q = 0; q < 4; ++q) g[gi][q] = *reinterpret_cast<const u32x4_t*>(p + gi * 32 + q * 8);
    f32x32_t acc = f32x32_t{};
#pragma unroll
    for (int gi = 0; gi < kGroups; ++gi) {
        u32x4_t (&cur)[4] = g[gi % (kAhead + 1)];
        if (gi + kAhead < kGroups) {
            u32x4_t (&nxt)[4] = g[(gi + kAhead) % (kAhead + 1)];
#pragma unroll
            for (int q = 0; q < 4; ++q) nxt[q] = *reinterpret_cast<const u32x4_t*>(p + (gi + kAhead) * 32 + q * 8);
        }
        asm volatile("" : "+v"(cur[0]), "+v"(cur[1]), "+v"(cur[2]), "+v"(cur[3]));
#pragma unroll
        for (int k = 0; k < 32; ++k) {
            const uint32_t w = cur[k / 8][(k % 8) / 2];
            const float v = __uint_as_float((k & 1) ? (w & 0xFFFF0000u) : (w << 16));
            acc = __builtin_amdgcn_mfma_f32_32x32x1f32(v, v, acc, 0, 0, 0);
        }
    }
    cosines2(s, acc, h, i);
}

// FPS over the cosine matrices in s.c of the two halves' sets (n0 and n1
// rows, each n > m, or 0 for an empty half; with m = 0 only the seed is
// marked taken, and the caller keeps no rows).  Leaves the selection
// orders in s.sel[h][0..m) and returns the taken rows, half h in bits
// 32h .. 32h + 31.
__device__ uint64_t fps2(Smem& s, int n0, int n1, int m, int lane) {
    const int h = lane >> 5, i = lane & 31;
    const int n = h ? n1 : n0;
    // seed: lowest mean cosine (row sums read down the columns: the matrices are symmetric bit for bit)
    const int nmax = n0 > n1 ? n0 : n1;
    float sum = 0.0f;
    if (n0 == kMaxRows && n1 == kMaxRows) {   // both sets full (every sampling round of a stream)
#pragma unroll 8
        for (int j = 0; j < kMaxRows; ++j) sum = sum + s.c[h][j][i];
    } else {
        for (int j = 0; j < nmax; ++j) {
            const float cj = s.c[h][j][i];
            sum = j < n ? sum + cj : sum;
        }
    }
    const float v = i < n ? sum / (float)n : __builtin_inff();
    const int p = argmin_halves(v, lane);
    // lane i < n: the order key of S_i (the largest cosine to the rows taken; cosines read along row r,
    // equal to column r), kOut once taken; lane i < m: the i-th pick.  Taking the maximum of keys is
    // taking the maximum of the cosines, and keys compare as the cosines do.
    constexpr int kOut = 0x7FFFFFFF;   // above every finite value's key
    int Sk = ((i < n) & (i != p)) ? order_key(s.c[h][p][i]) : kOut;
    int pick = p;
    for (int it = 1; it < m; ++it) {
        const int r = argmin_keys_halves(Sk, lane);
        pick = i == it ? r : pick;
        const int ck = order_key(s.c[h][r][i]);
        Sk = i == r ? kOut : max(Sk, ck);
    }
    if (i < m) s.sel[h][i] = pick;
    wave_lds_sync();
    return __ballot((Sk == kOut) & (i < n));
}

// Copy the rows in `mask` (ascending) to dst[0..), dst == src0 (in place;
// rows r < n0 come from src0, the rest from src1).  Rows already in place
// are skipped.  The rows go in groups of 8 destinations, each group's loads
// issued (and, by in-order completion, returned) before its stores; a kept
// row's source slot is never below its destination, so no group reads a slot
// an earlier group wrote.
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
// COMPRESS: no query is appended; a buffer holding more than n_beacon rows
// (count clamped as above) becomes FPS(buffer, n_beacon) the same way, and
// the other buffers are left as they are.
template <int D, bool COMPRESS>
__device__ void update_wave(const FpsArgs& a, int b0, int nw, Smem& s, int lane_in) {
    const int lane = lane_in;
    constexpr int kPieces = D / 8;                 // 16-byte pieces per row
    constexpr int kPerPass = kWave / kPieces;      // buffers per pass of the wave
    const int bqmax = a.n_beacon + a.n_recent_q;
    const int m = a.n_beacon;
    constexpr bool compress = COMPRESS;
    const int c_l = lane < nw ? clampi(a.qcount[b0 + lane], 0, bqmax - 1) : 0;   // count of buffer b0 + lane
    if constexpr (!compress) {
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
    }
    const int n_l = compress ? c_l : c_l + 1;
    const bool full = lane < nw && (compress ? n_l > m : n_l >= bqmax && n_l > m);
    if (compress && m == 0) {   // nothing is kept
        if (lane < nw && n_l > 0) a.qcount[b0 + lane] = 0;
        return;
    }
    if (lane < nw && !full && !compress) {
        a.qcount[b0 + lane] = n_l;
    }
    if (a.fps_sel && m > 0) {   // buffers that do not sample: -1s (all kept when n_recent_q == 0)
        const int passes = (nw * m + kWave - 1) / kWave;
        for (int p = 0; p < passes; ++p) {   // uniform loop: every lane takes part in the shuffles
            const int e = p * kWave + lane;
            const int bi = e < nw * m ? e / m : 0, i = e % m;
            const int n = __shfl(n_l, bi, kWave);
            const bool f = __shfl((int)full, bi, kWave) != 0;
            if (e < nw * m && !f)
                a.fps_sel[(size_t)(b0 + bi) * m + i] = (!compress && n >= bqmax && i < n) ? i : -1;
        }
    }
    uint64_t todo = __ballot(full);
    while (todo) {   // two buffers per round
        int lane_r = lane_in;   // opaque per round: lane-derived addresses are not held across rounds
        asm volatile("" : "+v"(lane_r));
        const int bi0 = __builtin_ctzll(todo);
        todo &= todo - 1;
        const bool two = todo != 0;
        const int bi1 = two ? __builtin_ctzll(todo) : bi0;
        todo &= todo - 1;
        const int c0 = __builtin_amdgcn_readlane(c_l, bi0), c1 = __builtin_amdgcn_readlane(c_l, bi1);
        bkv_bf16* buf0 = a.qbuf + (size_t)(b0 + bi0) * a.qcap * D;
        bkv_bf16* buf1 = a.qbuf + (size_t)(b0 + bi1) * a.qcap * D;
        // candidates: the buffer's rows, then (update) the new query
        const bkv_bf16* qn0 = compress ? buf0 : a.q_new + (size_t)(b0 + bi0) * D;
        const bkv_bf16* qn1 = compress ? buf1 : a.q_new + (size_t)(b0 + bi1) * D;
        constexpr int add = compress ? 0 : 1;
        const Cand A{buf0, c0, qn0, c0 + add}, B{buf1, c1, qn1, two ? c1 + add : 0};
        gram2<D>(s, A, B, lane_r);
        const uint64_t mask = fps2(s, A.n, B.n, m, lane_r);
        write_rows<D>(s, (uint32_t)mask, buf0, c0, qn0, lane_r);
        if (lane_r == 0) a.qcount[b0 + bi0] = m;
        if (a.fps_sel)
            for (int i = lane_r; i < m; i += kWave) a.fps_sel[(size_t)(b0 + bi0) * m + i] = s.sel[0][i];
        if (two) {
            write_rows<D>(s, (uint32_t)(mask >> 32), buf1, c1, qn1, lane_r);
            if (lane_r == 0) a.qcount[b0 + bi1] = m;
            if (a.fps_sel)
                for (int i = lane_r; i < m; i += kWave) a.fps_sel[(size_t)(b0 + bi1) * m + i] = s.sel[1][i];
        }
    }
}

// End-of-cycle merge of buffers b and b + 1 (when below nbuf): FPS over
// beacons ++ recents (Notes §2.2, App. Alg. 2).
template <int D>
__device__ void merge_pair(const FpsArgs& a, int b, Smem& s, int lane) {
    const int m = a.n_beacon;
    const int nbuf_here = a.nbuf - b < 2 ? a.nbuf - b : 2;
    Cand c[2];
    bkv_bf16* bufs[2] = {a.qbuf, a.qbuf};
    bool samples[2] = {false, false};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        c[h] = Cand{a.qbuf, 0, a.qbuf, 0};
        if (h >= nbuf_here) continue;
        bkv_bf16* buf = a.qbuf + (size_t)(b + h) * a.qcap * D;
        const bkv_bf16* rec = a.q_recent + (size_t)(b + h) * a.n_recent_q * D;
        const int nb = clampi(a.qcount[b + h], 0, m);
        const int n = nb + a.n_recent_q;
        if (m <= 0) {  // nothing is kept
            if (lane == 0) a.qcount[b + h] = 0;
        } else if (n <= m) {
            write_rows<D>(s, n >= 32 ? 0xFFFFFFFFu : ((1u << n) - 1u), buf, nb, rec, lane);
            if (lane == 0) a.qcount[b + h] = n;
            if (a.fps_sel)
                for (int i = lane; i < m; i += kWave) a.fps_sel[(size_t)(b + h) * m + i] = i < n ? i : -1;
        } else {
            c[h] = Cand{buf, nb, rec, n};
            bufs[h] = buf;
            samples[h] = true;
        }
    }
    if (!samples[0] && !samples[1]) return;
    gram2<D>(s, c[0], c[1], lane);
    const uint64_t mask = fps2(s, c[0].n, c[1].n, m, lane);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (!samples[h]) continue;
        write_rows<D>(s, (uint32_t)(mask >> (32 * h)), bufs[h], c[h].n0, c[h].src1, lane);
        if (lane == 0) a.qcount[b + h] = m;
        if (a.fps_sel)
            for (int i = lane; i < m; i += kWave) a.fps_sel[(size_t)(b + h) * m + i] = s.sel[h][i];
    }
}

}  // namespace fps
}  // namespace bkv
