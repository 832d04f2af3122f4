// bkv_fps_pair.hpp -- the end-of-cycle merge of the query buffers (Notes §2.2,
// App. Alg. 2): FPS over beacons ++ recents, two candidate sets per wavefront,
// one per half-wave (lanes 0-31 and 32-63), lane i of a half holding row i.
//
// The merge runs once per eviction over every buffer of the batch, a few
// sets per wave, so it is bound by how much latency the SIMDs can hide
// rather than by its arithmetic: half-wave sets keep the LDS area at 9 KB
// and the registers at 128 per wave, and four waves share a SIMD, where the
// four-set code of the buffer update (bkv_fps_impl.hpp) fits two.
//
// The Gram matrices: 128 (or 64) fp32 MFMA 32x32x1 rank-1 updates, two
// blocks per instruction (one per set), each lane feeding the k-th element of
// its row as both operands; each update rounds once per element, so every
// entry is the same chain of fused multiply-adds as a scalar loop over k.  The
// arithmetic is the fixed fp32 order of bkv_fps_impl.hpp, so the two paths
// select the same rows bit for bit.
#pragma once

#include "bkv_fps_impl.hpp"

namespace bkv {
namespace fps {

typedef float f32x32_t __attribute__((ext_vector_type(32)));

struct PairSmem {
    alignas(16) float c[2][kMaxRows][kCStride];   // per half: the Gram, then the cosines; then the moves
    float nrm[2][kMaxRows];
    int row_of[kMaxRows];                         // source row of each destination row of a copy
};

// The candidates of one buffer: n rows, [0, n0) from src0 and [n0, n) from
// src1 (n = 0: no buffer in this half).
struct Cand {
    bkv_bf16* src0;
    int n0;
    const bkv_bf16* src1;
    int n;
};

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_min_masked(int k) {
    return min(k, __builtin_amdgcn_update_dpp(0x7FFFFFFF, k, CTRL, ROW_MASK, 0xF, false));
}

// Per half-wave: the lowest lane of the half holding the half's smallest key,
// as an index 0..31, in every lane of the half.
__device__ __forceinline__ int argmin_halves(int k, int lane) {
    int m = row_min(k);                   // every lane of a 16-lane row holds the row's minimum
    m = dpp_min_masked<0x142, 0xA>(m);    // row_bcast15: rows 1 and 3 also take the previous row's
    const int m0 = __builtin_amdgcn_readlane(m, 31), m1 = __builtin_amdgcn_readlane(m, 63);
    const uint32_t e0 = (uint32_t)__ballot(k == m0);           // lanes 0..31 holding half 0's minimum
    const uint32_t e1 = (uint32_t)(__ballot(k == m1) >> 32);   // lanes 32..63 holding half 1's
    return lane < 32 ? __builtin_ctz(e0) : __builtin_ctz(e1);
}

// Gram entries acc (as laid out by the rank-1 updates) into s.c, the norms
// into s.nrm, then the cosines.  Each cosine is computed once and written to
// both of its entries: lane i of half h takes the pairs (i, (i + k) mod 32),
// k = 0 .. 16, of set h (the pair (i, i + 16) by both of its lanes, which
// write the same value).  Every lane reads all its Gram entries and norms
// before any lane writes a cosine.
__device__ __forceinline__ void cosines_pair(PairSmem& s, const f32x32_t& acc, int h, int i) {
#pragma unroll
    for (int r = 0; r < 32; ++r) s.c[r / 16][8 * ((r % 16) / 4) + 4 * h + (r % 4)][i] = acc[r];
    wave_lds_sync();
    const float ni = __builtin_sqrtf(s.c[h][i][i]);
    s.nrm[h][i] = ni;
    wave_lds_sync();
    float gv[kHalf + 1], nv[kHalf + 1];
#pragma unroll
    for (int k = 0; k <= kHalf; ++k) {
        const int j = (i + k) & (kMaxRows - 1);
        gv[k] = s.c[h][i][j];
        nv[k] = s.nrm[h][j];
    }
    wave_lds_sync();   // every lane's reads are done before the first cosine overwrites a Gram entry
#pragma unroll
    for (int k = 0; k <= kHalf; ++k) gv[k] = cosine(gv[k], ni, nv[k]);
#pragma unroll
    for (int k = 0; k <= kHalf; ++k) {
        const int j = (i + k) & (kMaxRows - 1);
        s.c[h][i][j] = gv[k];
        s.c[h][j][i] = gv[k];
    }
    wave_lds_sync();
}

// Cosine matrices of both halves' sets into s.c (and the norms into s.nrm).
// Lane i of half h loads row i of set h (lanes past n load a copy of row
// n - 1, or row 0 of src0 in an empty half: their dot products are computed
// but never read) in groups of four 16-byte pieces, issued two groups ahead
// of the group whose 32 rank-1 updates run.
template <int D>
__device__ __forceinline__ void gram_pair(PairSmem& s, const Cand& c0, const Cand& c1, int lane) {
    constexpr int kGroups = D / 32;
    const int h = lane >> 5, i = lane & 31;
    const int n = h ? c1.n : c0.n, n0 = h ? c1.n0 : c0.n0;
    const bkv_bf16* src0 = h ? c1.src0 : c0.src0;
    const bkv_bf16* src1 = h ? c1.src1 : c0.src1;
    const int ic = i < n ? i : (n > 0 ? n - 1 : 0);
    const bkv_bf16* p = n > 0 ? cand_row(src0, n0, src1, ic, D) : src0;
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
    cosines_pair(s, acc, h, i);
}

// FPS over the cosine matrices in s.c of the two halves' sets (n0 and n1
// rows, each n > m >= 1, or 0 for an empty half).  Returns the taken rows,
// half h in bits 32 h .. 32 h + 31, and in `pick` lane i's pick number i.
__device__ __forceinline__ uint64_t fps_pair(PairSmem& s, int n0, int n1, int m, int lane, int& pick) {
    const int h = lane >> 5, i = lane & 31;
    const int n = h ? n1 : n0;
    // seed: lowest mean cosine (row sums read down the columns: the matrices are symmetric bit for bit)
    float sum = 0.0f;
    if (n0 == kMaxRows && n1 == kMaxRows) {   // both sets full (every merge of a stream)
#pragma unroll 8
        for (int j = 0; j < kMaxRows; ++j) sum = sum + s.c[h][j][i];
    } else {
        const int nmax = n0 > n1 ? n0 : n1;
        for (int j = 0; j < nmax; ++j) {
            const float cj = s.c[h][j][i];
            sum = j < n ? sum + cj : sum;
        }
    }
    const float v = i < n ? sum / (float)n : __builtin_inff();
    const int p = argmin_halves(order_key(v), lane);
    // lane i < n: the order key of S_i (the largest cosine to the rows taken), kOut once taken
    constexpr int kOut = 0x7FFFFFFF;   // above every finite value's key
    int Sk = ((i < n) & (i != p)) ? order_key(s.c[h][p][i]) : kOut;
    pick = p;
    for (int it = 1; it < m; ++it) {
        const int r = argmin_halves(Sk, lane);
        pick = i == it ? r : pick;
        const int ck = order_key(s.c[h][r][i]);
        Sk = i == r ? kOut : max(Sk, ck);
    }
    return __ballot((Sk == kOut) & (i < n));
}

// The compactions of both halves' sets (as compact4, with lane i of half h
// owning row i of set h): the moves are listed in LDS by half, then by
// ascending destination, and copied 64 rows at a time.
template <int D>
__device__ __forceinline__ void compact_pair(PairSmem& s, uint32_t mask, bkv_bf16* dst, int n0, const bkv_bf16* src1,
                                             int lane) {
    constexpr int kPieces = D / 8;
    constexpr int kRowsPerPass = kWave / kPieces;
    constexpr int kPasses = 16;
    constexpr int kChunk = kRowsPerPass * kPasses;
    const int h = lane >> 5, i = lane & 31;
    const int w = __popc(mask & ((1u << i) - 1u));
    const bool mv_i = ((mask >> i) & 1u) && !(i < n0 && w == i);
    const uint64_t bm = __ballot(mv_i);
    const int c0 = __popcll(bm & 0xFFFFFFFFull), total = __popcll(bm);
    const uint64_t lt = (1ull << lane) - 1ull;
    Move* mv = reinterpret_cast<Move*>(&s.c[0][0][0]);
    wave_lds_sync();   // the matrices' last reads are done before the list overwrites them
    if (mv_i) mv[(h ? c0 : 0) + __popcll(bm & lt & (h ? 0xFFFFFFFF00000000ull : 0xFFFFFFFFull))] =
        Move{cand_row(dst, n0, src1, i, D), dst + (size_t)w * D};
    wave_lds_sync();
    const int row = lane / kPieces, piece = lane % kPieces;
    for (int e0 = 0; e0 < total; e0 += kChunk) {
        u32x4_t buf[kPasses];
#pragma unroll
        for (int j = 0; j < kPasses; ++j) {
            const int e = e0 + j * kRowsPerPass + row;
            if (e < total) buf[j] = reinterpret_cast<const u32x4_t*>(mv[e].src)[piece];
        }
#pragma unroll
        for (int j = 0; j < kPasses; ++j) {
            const int e = e0 + j * kRowsPerPass + row;
            if (e < total) reinterpret_cast<u32x4_t*>(mv[e].dst)[piece] = buf[j];
        }
    }
    wave_lds_sync();   // the list's reads are done before the next use of the area
}

// Copy of one buffer's rows in `mask` (ascending) to dst[0..) (in place; rows
// r < n0 from dst, the rest from src1), for a buffer that keeps every
// candidate.  Rows already in place are skipped; the rows go in groups of 8
// destinations, each group's loads before its stores (a kept row's source slot
// is never below its destination).
template <int D>
__device__ __forceinline__ void copy_rows(PairSmem& s, uint32_t mask, bkv_bf16* dst, int n0, const bkv_bf16* src1,
                                          int lane) {
    constexpr int kChunks = D / 8;
    constexpr int kGroup = 8;
    constexpr int kPer = kGroup * kChunks / 64;
    if (lane < kMaxRows && ((mask >> lane) & 1u)) s.row_of[__popc(mask & ((1u << lane) - 1u))] = lane;
    wave_lds_sync();
    const int cnt = __popc(mask);
    const int dropped = mask == 0xFFFFFFFFu ? kMaxRows : __builtin_ctz(~mask);
    const int first = dropped < n0 ? dropped : n0;
    for (int g0 = first & ~(kGroup - 1); g0 < cnt; g0 += kGroup) {
        u32x4_t buf[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int ci = lane + 64 * j;
            const int w = g0 + ci / kChunks, kc = ci % kChunks;
            if ((w >= first) & (w < cnt))
                buf[j] = *reinterpret_cast<const u32x4_t*>(cand_row(dst, n0, src1, s.row_of[w], D) + kc * 8);
        }
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int ci = lane + 64 * j;
            const int w = g0 + ci / kChunks, kc = ci % kChunks;
            if ((w >= first) & (w < cnt)) *reinterpret_cast<u32x4_t*>(dst + (size_t)w * D + kc * 8) = buf[j];
        }
    }
    wave_lds_sync();
}

// End-of-cycle merge of buffers b and b + 1 (when below nbuf).  A buffer with
// at most n_beacon candidates keeps them all; the others are sampled.
template <int D>
__device__ __forceinline__ void merge_pair(const FpsArgs& a, int b, PairSmem& s, int lane) {
    const int m = a.n_beacon;
    const int here = a.nbuf - b < 2 ? a.nbuf - b : 2;
    Cand c[2] = {Cand{a.qbuf, 0, a.qbuf, 0}, Cand{a.qbuf, 0, a.qbuf, 0}};
    bool samples[2] = {false, false};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (h >= here) continue;
        bkv_bf16* buf = a.qbuf + (size_t)(b + h) * a.qcap * D;
        const bkv_bf16* rec = a.q_recent + (size_t)(b + h) * a.n_recent_q * D;
        const int nb = clampi(a.qcount[b + h], 0, m > 0 ? m : 0);
        const int n = nb + a.n_recent_q;
        if (m <= 0) {  // nothing is kept
            if (lane == 0) a.qcount[b + h] = 0;
        } else if (n <= m) {   // every candidate is kept
            copy_rows<D>(s, n >= 32 ? 0xFFFFFFFFu : ((1u << n) - 1u), buf, nb, rec, lane);
            if (lane == 0) a.qcount[b + h] = n;
            if (a.fps_sel)
                for (int k = lane; k < m; k += kWave) a.fps_sel[(size_t)(b + h) * m + k] = k < n ? k : -1;
        } else {
            c[h] = Cand{buf, nb, rec, n};
            samples[h] = true;
        }
    }
    if (!samples[0] && !samples[1]) return;
    gram_pair<D>(s, c[0], c[1], lane);
    int pick;
    const uint64_t taken = fps_pair(s, c[0].n, c[1].n, m, lane, pick);
    const int h = lane >> 5, i = lane & 31;
    const int n = h ? c[1].n : c[0].n, n0 = h ? c[1].n0 : c[0].n0;
    bkv_bf16* src0 = h ? c[1].src0 : c[0].src0;
    const bkv_bf16* src1 = h ? c[1].src1 : c[0].src1;
    compact_pair<D>(s, n > 0 ? (uint32_t)(taken >> (32 * h)) : 0u, src0, n0, src1, lane);
    if (n > 0) {
        if (i == 0) a.qcount[b + h] = m;
        if (a.fps_sel && i < m) a.fps_sel[(size_t)(b + h) * m + i] = pick;
    }
}

}  // namespace fps
}  // namespace bkv
