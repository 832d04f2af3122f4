// bkv_fps_impl.hpp -- continual farthest point sampling of pre-RoPE queries
// (device functions of the buffer-update kernel, and the arithmetic the merge
// in bkv_fps_pair.hpp shares).  One wavefront samples four candidate sets
// (buffers) at a time, one per 16-lane row of the wave: lane t of row g holds
// candidate rows t and t + 16 of set g.
//
// The Gram matrices come from the matrix cores.  For each k, three fp32 MFMA
// 16x16x1 rank-1 updates with four blocks (one block per set) build the two
// diagonal tiles, rows 0-15 x 0-15 and 16-31 x 16-31, and the off-diagonal
// tile rows 0-15 x 16-31; the fourth tile is the transpose of the third, so
// three quarters of the products of the full matrix are issued.  Each update
// rounds once per element, so every entry is the same sequence of fused
// multiply-adds as a scalar loop over k.
//
// The arithmetic follows one fixed fp32 order so that the selected indices
// are reproducible bit for bit (Notes §2.2, App. Alg. 1):
//   dot_ij = fma chain over k = 0..d-1 from +0 (bf16 products are exact),
//   nrm_i  = sqrt(dot_ii) (correctly rounded), cos_ij = dot_ij / (nrm_i*nrm_j),
//   0 when a norm is 0, a_i = (left-to-right sum of cos_ij over j) / n,
// then argmin a (seed), and n_beacon - 1 greedy steps r = argmin over the
// untaken rows of S, S_j = max(S_j, cos_jr).  Ties go to the lower index.
// An argmin takes the minimum over the 16 lanes of a row by DPP, then the
// minimum of the indices of the rows holding it, which is the lowest index
// among equal values.  Each wave uses only its own LDS area, so waves of one
// workgroup never wait for each other.
#pragma once

#include "bkv_device.hpp"
#include "bkv_internal.hpp"

namespace bkv {
namespace fps {

constexpr int kMaxRows = 32;
constexpr int kHalf = kMaxRows / 2;   // rows per lane of a set: t and t + kHalf
constexpr int kSets = 4;              // candidate sets per wave, one per 16-lane row
constexpr int kCStride = kMaxRows + 1;   // floats per row of a half-wave set's cosine matrix (bkv_fps_pair.hpp)
// A set's symmetric 32 x 32 matrix is kept as three 16 x 16 tiles: rows 0-15 x 0-15 (D0), rows 16-31 x
// 16-31 (D1), both in full, and rows 0-15 x 16-31 (O, rows padded to 17 floats so that reading a column
// of it is conflict-free); rows 16-31 x 0-15 are read from O transposed.
constexpr int kTile = kHalf * kHalf;
constexpr int kOStride = kHalf + 1;
constexpr int kSetStride = 2 * kTile + kHalf * kOStride;   // 784 floats per set

typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kAhead = 2;   // row groups in flight ahead of the one the Gram is using (half-wave sets)
constexpr int kAhead4 = 1;  // the same for the four-set Gram, whose two rows per lane double the registers

struct Smem {
    alignas(16) float c[kSets * kSetStride];   // per set: the Gram, then the cosines; then the compaction's moves
    float nrm[kSets][kMaxRows];
};

// Tiles of set g: D0[i][j] = entry (i, j), D1[i][j] = (16 + i, 16 + j), O[i][j] = (i, 16 + j), i, j < 16.
__device__ __forceinline__ float* d0_of(Smem& s, int g) { return s.c + g * kSetStride; }
__device__ __forceinline__ float* d1_of(Smem& s, int g) { return s.c + g * kSetStride + kTile; }
__device__ __forceinline__ float* o_of(Smem& s, int g) { return s.c + g * kSetStride + 2 * kTile; }

// Entries (r, t) and (r, 16 + t) of set g, for a row r < 32 and t < 16:
// (r, t) is D0[r][t] or O[t][r - 16], (r, 16 + t) is O[r][t] or D1[r - 16][t],
// each at a lane base plus a multiple of r (16-lane reads stay on distinct
// banks: consecutive t, or rows of stride 17).
struct RowPair {
    const float* a_lo;   // D0 + t
    const float* a_hi;   // O + 17 t - 16
    const float* b_lo;   // O + t
    const float* b_hi;   // D1 + t - 256
    __device__ __forceinline__ RowPair(Smem& s, int g, int t)
        : a_lo(d0_of(s, g) + t), a_hi(o_of(s, g) + t * kOStride - kHalf), b_lo(o_of(s, g) + t),
          b_hi(d1_of(s, g) + t - kHalf * kHalf) {}
    __device__ __forceinline__ void read(int r, float& a, float& b) const {
        const bool lo = r < kHalf;
        a = lo ? a_lo[r * kHalf] : a_hi[r];
        b = lo ? b_lo[r * kOStride] : b_hi[r * kHalf];
    }
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

// Integer key ordered as the float v with -0 taken as +0 (v not NaN).
__device__ __forceinline__ int order_key(float v) {
    const int b = __float_as_int(v + 0.0f);
    return b ^ ((b >> 31) & 0x7FFFFFFF);
}

template <int CTRL>
__device__ __forceinline__ int dpp_min_step(int k) {
    return min(k, __builtin_amdgcn_update_dpp(0x7FFFFFFF, k, CTRL, 0xF, 0xF, false));
}

// The minimum of k over the lane's 16-lane row, in every lane of the row.
__device__ __forceinline__ int row_min(int k) {
    k = dpp_min_step<0xB1>(k);    // quad_perm [1,0,3,2]
    k = dpp_min_step<0x4E>(k);    // quad_perm [2,3,0,1]: the quad's minimum
    k = dpp_min_step<0x141>(k);   // row_half_mirror: the 8 lanes' minimum
    k = dpp_min_step<0x140>(k);   // row_mirror: the row's minimum
    return k;
}

// Argmin over a set's 32 rows, lane t holding the keys of rows t (ka) and
// t + 16 (kb): the lowest row index holding the smallest key, in every lane
// of the row.
__device__ __forceinline__ int argmin_set(int ka, int kb, int t) {
    const int m = row_min(min(ka, kb));
    return row_min(ka == m ? t : (kb == m ? t + kHalf : kMaxRows));
}

template <int D>
__device__ __forceinline__ void gram4(Smem& s, const bkv_bf16* pa, const bkv_bf16* pb, int lane) {
    constexpr int kGroups = D / 32;
    u32x4_t ga[kAhead4 + 1][4], gb[kAhead4 + 1][4];
#pragma unroll
    for (int gi = 0; gi < kAhead4 && gi < kGroups; ++gi)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            ga[gi][q] = *reinterpret_cast<const u32x4_t*>(pa + gi * 32 + q * 8);
            gb[gi][q] = *reinterpret_cast<const u32x4_t*>(pb + gi * 32 + q * 8);
        }
    f32x16_t d0 = f32x16_t{}, d1 = f32x16_t{}, o = f32x16_t{};
#pragma unroll
    for (int gi = 0; gi < kGroups; ++gi) {
        u32x4_t (&ca)[4] = ga[gi % (kAhead4 + 1)];
        u32x4_t (&cb)[4] = gb[gi % (kAhead4 + 1)];
        if (gi + kAhead4 < kGroups) {
            u32x4_t (&na)[4] = ga[(gi + kAhead4) % (kAhead4 + 1)];
            u32x4_t (&nb)[4] = gb[(gi + kAhead4) % (kAhead4 + 1)];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                na[q] = *reinterpret_cast<const u32x4_t*>(pa + (gi + kAhead4) * 32 + q * 8);
                nb[q] = *reinterpret_cast<const u32x4_t*>(pb + (gi + kAhead4) * 32 + q * 8);
            }
        }
        asm volatile("" : "+v"(ca[0]), "+v"(ca[1]), "+v"(ca[2]), "+v"(ca[3]));
        asm volatile("" : "+v"(cb[0]), "+v"(cb[1]), "+v"(cb[2]), "+v"(cb[3]));
#pragma unroll
        for (int k = 0; k < 32; ++k) {
            const uint32_t wa = ca[k / 8][(k % 8) / 2], wb = cb[k / 8][(k % 8) / 2];
            const float u = __uint_as_float((k & 1) ? (wa & 0xFFFF0000u) : (wa << 16));
            const float v = __uint_as_float((k & 1) ? (wb & 0xFFFF0000u) : (wb << 16));
            d0 = __builtin_amdgcn_mfma_f32_16x16x1f32(u, u, d0, 0, 0, 0);
            d1 = __builtin_amdgcn_mfma_f32_16x16x1f32(v, v, d1, 0, 0, 0);
            o = __builtin_amdgcn_mfma_f32_16x16x1f32(u, v, o, 0, 0, 0);
        }
    }
    const int q = lane >> 4, j = lane & 15;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int g = r >> 2, i = 4 * q + (r & 3);
        d0_of(s, g)[i * kHalf + j] = d0[r];
        d1_of(s, g)[i * kHalf + j] = d1[r];
        o_of(s, g)[i * kOStride + j] = o[r];
    }
    wave_lds_sync();
}

__device__ __forceinline__ float cosine(float g, float ni, float nj) {
    const float cq = g / (ni * nj);
    return ((ni == 0.0f) | (nj == 0.0f)) ? 0.0f : cq;
}

// The Gram entries in s.c become cosines, the norms go to s.nrm.  The
// matrices are symmetric bit for bit (the products are exact, both triangles
// accumulate them in the same order, and nrm_i nrm_j = nrm_j nrm_i), so each
// cosine is computed once and written to the entries that hold it.  Lane t
// of set g takes, in D0, the pairs (t, (t + k) mod 16), k = 0..8, writing
// both (t, c) and (c, t) (the pair (t, t + 8) by both of its lanes, which
// write the same value); the same in D1; and row t of O, all 16 of its
// entries.  Every lane reads the Gram entries of a tile before any lane
// writes a cosine into it.
__device__ __forceinline__ void cosines4(Smem& s, int lane) {
    const int g = lane >> 4, t = lane & 15;
    float* D0 = d0_of(s, g);
    float* D1 = d1_of(s, g);
    float* O = o_of(s, g);
    const float na = __builtin_sqrtf(D0[t * kHalf + t]);
    const float nb = __builtin_sqrtf(D1[t * kHalf + t]);
    s.nrm[g][t] = na;
    s.nrm[g][kHalf + t] = nb;
    wave_lds_sync();
    constexpr int kDiag = kHalf / 2 + 1;   // 9 pairs per lane in each diagonal tile
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
        float* T = tile ? D1 : D0;
        const float ni = tile ? nb : na;
        const float* nr = s.nrm[g] + tile * kHalf;
        float gv[kDiag], nv[kDiag];
#pragma unroll
        for (int k = 0; k < kDiag; ++k) {
            const int c = (t + k) & (kHalf - 1);
            gv[k] = T[t * kHalf + c];
            nv[k] = nr[c];
        }
        wave_lds_sync();   // every lane's reads of the tile are done before the first cosine overwrites it
#pragma unroll
        for (int k = 0; k < kDiag; ++k) gv[k] = cosine(gv[k], ni, nv[k]);
#pragma unroll
        for (int k = 0; k < kDiag; ++k) {
            const int c = (t + k) & (kHalf - 1);
            T[t * kHalf + c] = gv[k];
            T[c * kHalf + t] = gv[k];
        }
    }
    {
        float gv[kHalf], nv[kHalf];
#pragma unroll
        for (int j = 0; j < kHalf; ++j) {
            gv[j] = O[t * kOStride + j];
            nv[j] = s.nrm[g][kHalf + j];
        }
#pragma unroll
        for (int j = 0; j < kHalf; ++j) O[t * kOStride + j] = cosine(gv[j], na, nv[j]);
    }
    wave_lds_sync();
}

// Taken rows of the four sets (bit t + 16 h of set g's mask: row t + 16 h).
struct Picks {
    uint64_t ta, tb;   // ballots of the taken rows t (ta) and t + 16 (tb), lane 16 g + t
    int pa, pb;        // the lane's picks number t and t + 16
    __device__ __forceinline__ uint32_t mask(int g) const {
        return (uint32_t)((ta >> (16 * g)) & 0xFFFFu) | ((uint32_t)((tb >> (16 * g)) & 0xFFFFu) << 16);
    }
};

// FPS over the cosine matrices in s.c of the four sets (n: the lane's set
// size, each n > m or 0 for an unused set; m >= 1).  Returns the taken rows
// and, per lane, the picks number t and t + 16 in selection order.
__device__ __forceinline__ Picks fps4(Smem& s, int n, int m, int lane) {
    const int g = lane >> 4, t = lane & 15;
    // seed: lowest mean cosine (row sums read down the columns: the matrices are symmetric bit for bit)
    // Rows j < 16 hold (j, t) in D0 and (j, 16 + t) in O; rows 16 + j hold (16 + j, t) = O[t][j] and
    // (16 + j, 16 + t) in D1: one loop per half, so that every address is a fixed offset.
    const float* D0 = d0_of(s, g);
    const float* D1 = d1_of(s, g);
    const float* O = o_of(s, g);
    float sa = 0.0f, sb = 0.0f;
    if (__ballot((n != kMaxRows) & (n != 0)) == 0) {   // every set full (every sampling round of a stream)
#pragma unroll
        for (int j = 0; j < kHalf; ++j) {
            sa = sa + D0[j * kHalf + t];
            sb = sb + O[j * kOStride + t];
        }
#pragma unroll
        for (int j = 0; j < kHalf; ++j) {
            sa = sa + O[t * kOStride + j];
            sb = sb + D1[j * kHalf + t];
        }
    } else {   // the reads are made unconditional (opaque), so that they are not turned into branches
#pragma unroll
        for (int j = 0; j < kHalf; ++j) {
            float ca = D0[j * kHalf + t], cb = O[j * kOStride + t];
            asm volatile("" : "+v"(ca), "+v"(cb));
            sa = j < n ? sa + ca : sa;
            sb = j < n ? sb + cb : sb;
        }
#pragma unroll
        for (int j = 0; j < kHalf; ++j) {
            float ca = O[t * kOStride + j], cb = D1[j * kHalf + t];
            asm volatile("" : "+v"(ca), "+v"(cb));
            sa = kHalf + j < n ? sa + ca : sa;
            sb = kHalf + j < n ? sb + cb : sb;
        }
    }
    const float va = t < n ? sa / (float)n : __builtin_inff();
    const float vb = kHalf + t < n ? sb / (float)n : __builtin_inff();
    const int p = argmin_set(order_key(va), order_key(vb), t);
    // S of rows t and t + 16 as order keys (the largest cosine to the rows taken; cosines read along row
    // r, equal to column r), kOut once taken or past n.  The maximum of two keys is the key of the larger
    // cosine, and keys compare as the cosines do.
    constexpr int kOut = 0x7FFFFFFF;   // above every finite value's key
    const RowPair rows(s, g, t);
    float pa_, pb_;
    rows.read(p, pa_, pb_);
    int ka = ((t < n) & (t != p)) ? order_key(pa_) : kOut;
    int kb = ((kHalf + t < n) & (kHalf + t != p)) ? order_key(pb_) : kOut;
    Picks pk;
    pk.pa = p;
    pk.pb = p;
    for (int it = 1; it < m; ++it) {
        const int r = argmin_set(ka, kb, t);
        pk.pa = t == it ? r : pk.pa;
        pk.pb = kHalf + t == it ? r : pk.pb;
        float ra_, rb_;
        rows.read(r, ra_, rb_);
        const int ca = order_key(ra_), cb = order_key(rb_);
        ka = t == r ? kOut : max(ka, ca);
        kb = kHalf + t == r ? kOut : max(kb, cb);
    }
    pk.ta = __ballot((ka == kOut) & (t < n));
    pk.tb = __ballot((kb == kOut) & (kHalf + t < n));
    return pk;
}

// One move of a compaction: a source row and its destination slot.
struct Move {
    const bkv_bf16* src;
    bkv_bf16* dst;
};

// The compactions of the four sets, after fps4 (the matrices are no longer
// needed, so their LDS holds the list of moves).  Lane t of set g owns rows t
// and t + 16: a kept row i goes to slot popcount(mask below i) of dst (the
// set's buffer); rows r < n0 come from dst itself, the others from src1 (the
// new query or the recent queries).  A row whose slot does not change is not
// moved.  The moves are listed by set, then by ascending destination, and
// copied 64 rows at a time (16-byte pieces, 16 lanes per row), each piece's
// load issued before its store.  Within a set a row's source slot is never
// below its destination and the destinations ascend, so no load reads a slot
// that an earlier store of the same set wrote, and a store waits for its own
// load and hence (loads complete in order) for every earlier one.
template <int D>
__device__ __forceinline__ void compact4(Smem& s, uint32_t mask, bkv_bf16* dst, int n0, const bkv_bf16* src1,
                                         int lane) {
    constexpr int kPieces = D / 8;                 // 16-byte pieces per row
    constexpr int kRowsPerPass = kWave / kPieces;  // rows one wave instruction covers
    constexpr int kPasses = 16;                    // pieces per lane per chunk
    constexpr int kChunk = kRowsPerPass * kPasses; // rows per chunk
    const int g = lane >> 4, t = lane & 15;
    const int ia = t, ib = kHalf + t;
    const int wa = __popc(mask & ((1u << ia) - 1u)), wb = __popc(mask & ((1u << ib) - 1u));
    const bool ma = ((mask >> ia) & 1u) && !(ia < n0 && wa == ia);
    const bool mb = ((mask >> ib) & 1u) && !(ib < n0 && wb == ib);
    const uint64_t ba = __ballot(ma), bb = __ballot(mb);
    const uint64_t lt = (1ull << lane) - 1ull;
    int off = 0, total = 0, ca_g = 0;
#pragma unroll
    for (int h = 0; h < kSets; ++h) {
        const uint64_t set = 0xFFFFull << (16 * h);
        const int ca = __popcll(ba & set), cb = __popcll(bb & set);
        off = h < g ? off + ca + cb : off;
        ca_g = h == g ? ca : ca_g;
        total += ca + cb;
    }
    const uint64_t mine = 0xFFFFull << (16 * g);
    Move* mv = reinterpret_cast<Move*>(s.c);
    wave_lds_sync();   // the matrices' last reads are done before the list overwrites them
    if (ma) mv[off + __popcll(ba & mine & lt)] = Move{cand_row(dst, n0, src1, ia, D), dst + (size_t)wa * D};
    if (mb) mv[off + ca_g + __popcll(bb & mine & lt)] = Move{cand_row(dst, n0, src1, ib, D), dst + (size_t)wb * D};
    wave_lds_sync();
    const int row = lane / kPieces, piece = lane % kPieces;
    for (int e0 = 0; e0 < total; e0 += kChunk) {
        u32x4_t buf[kPasses];
        Move m[kPasses];
#pragma unroll
        for (int j = 0; j < kPasses; ++j) {
            const int e = e0 + j * kRowsPerPass + row;
            if (e < total) {
                m[j] = mv[e];
                buf[j] = reinterpret_cast<const u32x4_t*>(m[j].src)[piece];
            }
        }
#pragma unroll
        for (int j = 0; j < kPasses; ++j) {
            const int e = e0 + j * kRowsPerPass + row;
            if (e < total) reinterpret_cast<u32x4_t*>(m[j].dst)[piece] = buf[j];
        }
    }
    wave_lds_sync();   // the list's reads are done before the next use of the area
}

constexpr int kMaxBuffersPerWave = 32;

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
__device__ __forceinline__ void update_wave(const FpsArgs& a, int b0, int nw, Smem& s, int lane_in) {
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
    while (todo) {   // four buffers per round, one per 16-lane row
        int lane_r = lane_in;   // opaque per round: lane-derived addresses are not held across rounds
        asm volatile("" : "+v"(lane_r));
        const int g = lane_r >> 4, t = lane_r & 15;
        int bi[kSets], cs[kSets];
        bool have[kSets];
#pragma unroll
        for (int h = 0; h < kSets; ++h) {
            have[h] = todo != 0;
            bi[h] = have[h] ? __builtin_ctzll(todo) : 0;
            todo &= todo - 1;
            cs[h] = __builtin_amdgcn_readlane(c_l, bi[h]);
        }
        constexpr int add = compress ? 0 : 1;
        // the lane's set: the buffer's rows, then (update) the new query
        const int my_bi = g == 0 ? bi[0] : g == 1 ? bi[1] : g == 2 ? bi[2] : bi[3];
        const int my_c = g == 0 ? cs[0] : g == 1 ? cs[1] : g == 2 ? cs[2] : cs[3];
        const bool my_have = g == 0 ? have[0] : g == 1 ? have[1] : g == 2 ? have[2] : have[3];
        const int n = my_have ? my_c + add : 0;
        const bkv_bf16* buf = a.qbuf + (size_t)(b0 + my_bi) * a.qcap * D;
        const bkv_bf16* qn = compress ? buf : a.q_new + (size_t)(b0 + my_bi) * D;
        const int ra = t < n ? t : (n > 0 ? n - 1 : 0), rb = kHalf + t < n ? kHalf + t : (n > 0 ? n - 1 : 0);
        gram4<D>(s, cand_row(buf, my_c, qn, ra, D), cand_row(buf, my_c, qn, rb, D), lane_r);
        cosines4(s, lane_r);
        const Picks pk = fps4(s, n, m, lane_r);
        bkv_bf16* dst = a.qbuf + (size_t)(b0 + my_bi) * a.qcap * D;
        compact4<D>(s, my_have ? pk.mask(g) : 0u, dst, my_c, qn, lane_r);
        if (my_have) {
            if (t == 0) a.qcount[b0 + my_bi] = m;
            if (a.fps_sel) {
                int32_t* sel = a.fps_sel + (size_t)(b0 + my_bi) * m;
                if (t < m) sel[t] = pk.pa;
                if (kHalf + t < m) sel[kHalf + t] = pk.pb;
            }
        }
    }
}

}  // namespace fps
}  // namespace bkv
