// bkv_prefill.hip -- prefill initialisation of the query buffers: farthest
// point sampling of each query head's prompt queries down to n_beacon rows
// (Notes §2.2: at prefill the first representatives are sampled from the
// prompt's queries; the steps are those of App. Alg. 1).
//
// One 512-thread workgroup per buffer (one per CU: eight waves of up to 256
// VGPRs); thread tid owns rows j = c * 512 + tid (chunk c).  The rows of the
// first 256 / d chunks stay in registers as packed bf16 (128 VGPRs); the next
// ones stay in LDS (bf16, swizzled so that a wave's row reads are
// conflict-free), up to the 160 KB a CU has; rows beyond that (prompts of
// several thousand queries) are re-read from global memory on every pass.
// Prompts whose rows past the first 128 / d chunks fit in LDS at one per
// thread take the fp32 path instead (those chunks in registers in fp32).
// The norms and S values of rows outside the registers live in LDS.
//
// Arithmetic, in one fixed fp32 order (bit-identical selections):
//   nrm_j = sqrt(fma chain of x_j . x_j over k ascending, from +0);
//   inv_j = 1 / nrm_j (0 if nrm_j is 0), u_j[k] = x_j[k] * inv_j;
//   s[k]  = pairwise sum of u_j[k] over j: a balanced binary tree over the
//           row index, padded with zero rows to a power of two.  Lanes form
//           the low six levels (an LDS transpose, then DPP), waves the next
//           three (LDS), chunks the rest;
//   a_j   = (fma chain of u_j[k] * s[k]) / P, the mean cosine of row j to all
//           rows (cos is the dot product of unit rows), seed p = argmin a;
//   then n_beacon - 1 steps: S_j = max(S_j, cos(x_j, x_r)) for the last pick
//   r with cos = (fma chain of x_j . x_r) / (nrm_j * nrm_r) (0 if a norm is
//   0), next pick = argmin of S over the rows not taken.
// Every argmin takes the lowest row index among equal values.  The
// survivors are written to the buffer in ascending prompt order.
#include "bkv_device.hpp"
#include "bkv_internal.hpp"

namespace bkv {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxChunks = BKV_PREFILL_MAX / kThreads;
constexpr int kLdsBytes = 160 * 1024;   // LDS of one CU (the most a workgroup is given)

template <int D, bool F32 = true>
struct Pre {
    // chunks of rows in registers: 128 VGPRs of them, in fp32 (F32) or packed bf16
    static constexpr int kRegChunks = (F32 ? 128 : 256) / D;
    static constexpr int kRegRows = kRegChunks * kThreads;
    // LDS layout (bytes)
    static constexpr int kXrOff = 0;                                 // float [2][D]   picked row
    static constexpr int kXnOff = kXrOff + 2 * D * 4;                // float [2]      its norm
    static constexpr int kWvOff = kXnOff + 16;                       // int [2][waves] wave minima (keys)
    static constexpr int kWiOff = kWvOff + 2 * kWaves * 4;           // int   [2][waves]
    static constexpr int kPartOff = kWiOff + 2 * kWaves * 4;         // float [waves][D] wave column sums
    static constexpr int kSlabOff = kPartOff + kWaves * D * 4;       // float [waves][4][64] column transposes
    static constexpr int kCsumOff = kSlabOff + kWaves * 256 * 4;     // float [chunks][D]
    static constexpr int kSsumOff = kCsumOff + kMaxChunks * D * 4;   // float [D]
    static constexpr int kSelOff = kSsumOff + D * 4;                 // int [32]
    static constexpr int kOtherOff = kSelOff + 32 * 4;               // float nrm[n_other], S[n_other]; then rows
    static constexpr int kRowBytes = 2 * D;
    // rows outside the registers, and how many of them fit in LDS
    __host__ __device__ static int n_other(int P) { return P > kRegRows ? P - kRegRows : 0; }
    __host__ __device__ static int rows_off(int P) { return (kOtherOff + n_other(P) * 8 + 15) & ~15; }
    __host__ __device__ static int n_lds_rows(int P, int lds_bytes) {
        const int room = (lds_bytes - rows_off(P)) / kRowBytes;
        return room < 0 ? 0 : (n_other(P) < room ? n_other(P) : room);
    }
    __host__ __device__ static size_t bytes(int P, int lds_bytes) {
        return (size_t)rows_off(P) + (size_t)n_lds_rows(P, lds_bytes) * kRowBytes;
    }
};

// Ends the work on one 8-element piece of a row: the accumulator must be
// final here and no memory access moves across, so the compiler neither reads
// the next pieces' fp32 operands early nor sinks the multiply-adds past the
// loop (either keeps a whole fp32 row live and spills the resident rows).
__device__ __forceinline__ void piece_fence(float& acc) { asm volatile("" : "+v"(acc)::"memory"); }

// bf16 halves of a packed word.  The shift and the mask are made opaque
// (fresh() at the top of every pass), so the compiler can neither hoist the
// unpacking of the resident rows out of the loop over the greedy steps nor
// share it between passes: either would keep a second, fp32 copy of the rows
// in registers and spill.
struct Bf {
    uint32_t sh, mk;
    static __device__ __forceinline__ Bf fresh() {
        Bf u;
        asm volatile("s_mov_b32 %0, 16" : "=s"(u.sh));
        asm volatile("s_mov_b32 %0, 0xffff0000" : "=s"(u.mk));
        return u;
    }
    __device__ __forceinline__ float lo(uint32_t w) const { return __uint_as_float(w << sh); }
    __device__ __forceinline__ float hi(uint32_t w) const { return __uint_as_float(w & mk); }
};

template <int D>
__device__ __forceinline__ void load_row(const bkv_bf16* Q, int P, int j, u32x4_t (&x)[D / 8]) {
    if (j < P) {
        const u32x4_t* src = reinterpret_cast<const u32x4_t*>(Q + (size_t)j * D);
#pragma unroll
        for (int p = 0; p < D / 8; ++p) x[p] = src[p];
    } else {
#pragma unroll
        for (int p = 0; p < D / 8; ++p) x[p] = u32x4_t{0u, 0u, 0u, 0u};
    }
}

// For R rows at once: acc[r] = fma chain over k ascending (from +0) of
// x_r[k] * y[k], or of (x_r[k] * inv[r]) * y[k] with SCALE, y fp32 in LDS
// (the same address for every lane: broadcast reads).  The next piece of y is
// read while the current one is used, and each piece of y serves every row.
template <int D, int R, bool SCALE>
__device__ __forceinline__ void fma_rows(const u32x4_t (&x)[R][D / 8], const float* y, const float* inv,
                                         float (&acc)[R]) {
    const Bf u = Bf::fresh();
    constexpr int NP = D / 8;
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0f;
    f32x4_t ya = *reinterpret_cast<const f32x4_t*>(y);
    f32x4_t yb = *reinterpret_cast<const f32x4_t*>(y + 4);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        f32x4_t na = ya, nb = yb;
        if (p + 1 < NP) {
            na = *reinterpret_cast<const f32x4_t*>(y + 8 * (p + 1));
            nb = *reinterpret_cast<const f32x4_t*>(y + 8 * (p + 1) + 4);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const u32x4_t w = x[r][p];
            float e[8] = {u.lo(w[0]), u.hi(w[0]), u.lo(w[1]), u.hi(w[1]),
                          u.lo(w[2]), u.hi(w[2]), u.lo(w[3]), u.hi(w[3])};
            if constexpr (SCALE) {
#pragma unroll
                for (int k = 0; k < 8; ++k) e[k] = e[k] * inv[r];
            }
            float a = acc[r];
            a = __builtin_fmaf(e[0], ya[0], a);
            a = __builtin_fmaf(e[1], ya[1], a);
            a = __builtin_fmaf(e[2], ya[2], a);
            a = __builtin_fmaf(e[3], ya[3], a);
            a = __builtin_fmaf(e[4], yb[0], a);
            a = __builtin_fmaf(e[5], yb[1], a);
            a = __builtin_fmaf(e[6], yb[2], a);
            a = __builtin_fmaf(e[7], yb[3], a);
            piece_fence(a);
            acc[r] = a;
        }
        ya = na;
        yb = nb;
    }
}

template <int D>
__device__ __forceinline__ const u32x4_t (&one_row(const u32x4_t (&x)[D / 8]))[1][D / 8] {
    return *reinterpret_cast<const u32x4_t(*)[1][D / 8]>(&x);
}

template <int D>
__device__ __forceinline__ float norm_of(const u32x4_t (&x)[D / 8]) {
    const Bf u = Bf::fresh();
    float acc = 0.0f;
#pragma unroll
    for (int p = 0; p < D / 8; ++p) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float a = u.lo(x[p][e]), b = u.hi(x[p][e]);
            acc = __builtin_fmaf(a, a, acc);
            acc = __builtin_fmaf(b, b, acc);
        }
    }
    return __builtin_sqrtf(acc);
}

template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_add(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xF, false));
}

// Sums of four columns over the wave's 64 rows (row = lane; v0..v3 are the
// lane's entries of the four columns), as a pairwise tree over the lane
// index: the values pass through the wave's own 1 KB of LDS (column k at
// words 64 k .. 64 k + 63, so that the writes and the reads are
// conflict-free); lane 16 c + m adds rows 4m .. 4m + 3 of column c in pairs,
// then the 16 lanes of its DPP row finish the tree over m: pairs of lanes,
// blocks of 4, halves (mirrored lanes hold the same block sums), the whole
// row.  Lane 16 c writes column c's sum to dst[c].  A wave's LDS accesses
// complete in order, so the reads see this call's writes and the next call's
// writes follow these reads.
__device__ __forceinline__ void col4_sum(float v0, float v1, float v2, float v3, float* slab, float* dst,
                                         int lane) {
    slab[lane] = v0;
    slab[64 + lane] = v1;
    slab[128 + lane] = v2;
    slab[192 + lane] = v3;
    const int c = lane >> 4, m = lane & 15;
    const f32x4_t r = *reinterpret_cast<const f32x4_t*>(slab + 64 * c + 4 * m);
    float v = (r[0] + r[1]) + (r[2] + r[3]);
    v = dpp_add<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]: blocks of 8 rows
    v = dpp_add<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]: 16 rows
    v = dpp_add<0x141, 0xF>(v);   // row_half_mirror: 32 rows
    v = dpp_add<0x140, 0xF>(v);   // row_mirror: all 64
    if (m == 0) dst[c] = v;
}

constexpr int kNoKey = 0x7FFFFFFF;   // above every candidate's key

// Integer key ordered as the float v, with -0 taken as +0 (v not NaN); a
// thread with no candidate (i == kNone) gives kNoKey.
__device__ __forceinline__ int key_of(float v, int i) {
    const int b = __float_as_int(v + 0.0f);
    return i == 0x7FFFFFFF ? kNoKey : b ^ ((b >> 31) & 0x7FFFFFFF);
}

template <int CTRL>
__device__ __forceinline__ int dpp_min(int k) {
    return min(k, __builtin_amdgcn_update_dpp(kNoKey, k, CTRL, 0xF, 0xF, false));
}

// The minimum of k over the wave, uniform: DPP inside each 16-lane row, then
// the four rows' minima.
__device__ __forceinline__ int wave_min(int k) {
    k = dpp_min<0xB1>(k);    // quad_perm [1,0,3,2]
    k = dpp_min<0x4E>(k);    // quad_perm [2,3,0,1]
    k = dpp_min<0x141>(k);   // row_half_mirror
    k = dpp_min<0x140>(k);   // row_mirror: every lane of a row holds the row's minimum
    const int a = __builtin_amdgcn_readlane(k, 0), b = __builtin_amdgcn_readlane(k, 16);
    const int c = __builtin_amdgcn_readlane(k, 32), d = __builtin_amdgcn_readlane(k, 48);
    return min(min(a, b), min(c, d));
}

// Workgroup argmin of (v, i), each thread holding its own best row i (kNone:
// none) and its value v: the lowest row index among the smallest values, in
// every thread.  Values compare through their order keys, so equal values
// (+0 and -0 included) go to the lower index.
__device__ __forceinline__ int block_argmin(float v, int i, int* wk, int* wi, int wave, int lane) {
    const int k = key_of(v, i);
    const int m = wave_min(k);
    const int idx = wave_min(k == m ? i : kNoKey);
    if (lane == 0) {
        wk[wave] = m;
        wi[wave] = idx;
    }
    __syncthreads();
    int kv[kWaves], iv[kWaves];   // every wave's pair read at once, then reduced in registers
#pragma unroll
    for (int w = 0; w < kWaves; w += 4) {
        const int4 a = *reinterpret_cast<const int4*>(wk + w), b = *reinterpret_cast<const int4*>(wi + w);
        kv[w] = a.x, kv[w + 1] = a.y, kv[w + 2] = a.z, kv[w + 3] = a.w;
        iv[w] = b.x, iv[w + 1] = b.y, iv[w + 2] = b.z, iv[w + 3] = b.w;
    }
    int gm = kv[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) gm = min(gm, kv[w]);
    int gi = kNoKey;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) gi = min(gi, kv[w] == gm ? iv[w] : kNoKey);
    return gi;
}

// Column sums of one chunk's unit rows u = x * inv into csum[c][0 .. D):
// pairwise over the lanes (col4_sum), then over the waves.  All threads call
// it.
template <int D>
__device__ __forceinline__ void chunk_colsum(const u32x4_t (&x)[D / 8], float inv, int c, float* part, float* slab,
                                             float* csum, int wave, int lane, int tid) {
    const Bf u = Bf::fresh();
    float* sl = slab + wave * 256;
#pragma unroll
    for (int p = 0; p < D / 8; ++p) {
        const u32x4_t w = x[p];
        col4_sum(u.lo(w[0]) * inv, u.hi(w[0]) * inv, u.lo(w[1]) * inv, u.hi(w[1]) * inv, sl, part + wave * D + 8 * p,
                 lane);
        col4_sum(u.lo(w[2]) * inv, u.hi(w[2]) * inv, u.lo(w[3]) * inv, u.hi(w[3]) * inv, sl,
                 part + wave * D + 8 * p + 4, lane);
    }
    __syncthreads();
    if (tid < D) {
        const float* q = part + tid;
        const float s01 = q[0 * D] + q[1 * D], s23 = q[2 * D] + q[3 * D];
        const float s45 = q[4 * D] + q[5 * D], s67 = q[6 * D] + q[7 * D];
        csum[c * D + tid] = (s01 + s23) + (s45 + s67);
    }
    __syncthreads();
}

// Mean cosine of a row to all rows: (fma chain of u[k] * s[k]) / P.
template <int D>
__device__ __forceinline__ float mean_cos(const u32x4_t (&x)[D / 8], float inv, const float* ssum, float fP) {
    float acc[1];
    const float iv[1] = {inv};
    fma_rows<D, 1, true>(one_row<D>(x), ssum, iv, acc);
    return acc[0] / fP;
}

// cos(x, y) with y fp32 in LDS: dot / (|x| |y|), 0 if a norm is 0.
template <int D>
__device__ __forceinline__ float cos_to(const u32x4_t (&x)[D / 8], float nx, const float* y, float ny) {
    float dt[1];
    fma_rows<D, 1, false>(one_row<D>(x), y, nullptr, dt);
    return (nx == 0.0f || ny == 0.0f) ? 0.0f : dt[0] / (nx * ny);
}

template <int D>
__device__ __forceinline__ void store_row_f32(const u32x4_t (&x)[D / 8], float* dst) {
    const Bf u = Bf::fresh();
#pragma unroll
    for (int p = 0; p < D / 8; ++p) {
        const u32x4_t w = x[p];
        *reinterpret_cast<f32x4_t*>(dst + 8 * p) = f32x4_t{u.lo(w[0]), u.hi(w[0]), u.lo(w[1]), u.hi(w[1])};
        *reinterpret_cast<f32x4_t*>(dst + 8 * p + 4) = f32x4_t{u.lo(w[2]), u.hi(w[2]), u.lo(w[3]), u.hi(w[3])};
    }
}

__device__ __forceinline__ float inv_of(float nr) { return nr == 0.0f ? 0.0f : 1.0f / nr; }

// A zero the compiler cannot see through.  Added to an LDS index inside a
// loop over rows, it keeps the reads of a whole fp32 row (128 VGPRs) from
// being hoisted out of the loop, while the pointer keeps its LDS provenance.
__device__ __forceinline__ int opaque_zero() {
    int z = 0;
    asm volatile("" : "+s"(z));
    return z;
}

constexpr int kNone = 0x7FFFFFFF;

// 16-byte slot of piece p of LDS row s: the piece index is XORed with bits
// of the row so that the 64 lanes of a wave, reading one piece of 64
// consecutive rows, hit every bank once per 256 bytes.
template <int D>
__device__ __forceinline__ int lds_slot(int s, int p) {
    constexpr int kPer256 = 256 / (2 * D);   // rows per 256 bytes: 1 (d = 128) or 2 (d = 64)
    return s * (D / 8) + (p ^ ((s / kPer256) & (D / 8 - 1)));
}

// With every row past the registers in LDS and at most one per thread (the
// fp32 path), rows are stored piece-major: piece p of row s at slot
// p * 512 + s.  A wave's 64 lanes read 64 consecutive slots (conflict-free),
// and the pieces of a row sit at fixed offsets from its first, so no address
// is computed per piece.
template <int D, bool F32>
__device__ __forceinline__ int slot(int s, int p) {
    return F32 ? p * kThreads + s : lds_slot<D>(s, p);
}

// Row j = RC * 512 + s outside the registers: from LDS when s < n_lds, else
// from global memory.  Rows past the prompt are zero.
template <int D>
__device__ __forceinline__ void fetch_row(const bkv_bf16* Q, int P, int j, int s, int n_lds, const u32x4_t* lrows,
                                          u32x4_t (&x)[D / 8]) {
    if (j < P && s < n_lds) {
#pragma unroll
        for (int p = 0; p < D / 8; ++p) x[p] = lrows[lds_slot<D>(s, p)];
    } else {
        load_row<D>(Q, P, j, x);
    }
}

// ---- register rows in fp32 (when every other row fits in LDS): no unpacking
// of the register-resident rows on any pass.

template <int D, int R, bool F32>
struct RegRows {
    using type = u32x4_t[R][D / 8];   // packed bf16
};
template <int D, int R>
struct RegRows<D, R, true> {
    using type = float[R][D];
};

template <int D>
__device__ __forceinline__ void to_reg(const u32x4_t (&w)[D / 8], u32x4_t (&x)[D / 8]) {
#pragma unroll
    for (int p = 0; p < D / 8; ++p) x[p] = w[p];
}
template <int D>
__device__ __forceinline__ void to_reg(const u32x4_t (&w)[D / 8], float (&x)[D]) {
#pragma unroll
    for (int p = 0; p < D / 8; ++p)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[8 * p + 2 * e] = __uint_as_float(w[p][e] << 16);
            x[8 * p + 2 * e + 1] = __uint_as_float(w[p][e] & 0xFFFF0000u);
        }
}

template <int D>
__device__ __forceinline__ float norm_of(const float (&x)[D]) {
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < D; ++k) acc = __builtin_fmaf(x[k], x[k], acc);
    return __builtin_sqrtf(acc);
}

// fma_rows for fp32 rows: the same chains, with the same piece pacing of y.
// The scale factors pass through an opaque copy, so the products x * inv are
// not shared with the column sums' (keeping them from one pass to the next
// would hold a second fp32 row).
template <int D, int R, bool SCALE>
__device__ __forceinline__ void fma_rows(const float (&x)[R][D], const float* y, const float* inv_in,
                                         float (&acc)[R]) {
    constexpr int NP = D / 8;
    float inv[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        inv[r] = SCALE ? inv_in[r] : 0.0f;
        asm volatile("" : "+v"(inv[r]));
    }
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0f;
    f32x4_t ya = *reinterpret_cast<const f32x4_t*>(y);
    f32x4_t yb = *reinterpret_cast<const f32x4_t*>(y + 4);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        f32x4_t na = ya, nb = yb;
        if (p + 1 < NP) {
            na = *reinterpret_cast<const f32x4_t*>(y + 8 * (p + 1));
            nb = *reinterpret_cast<const f32x4_t*>(y + 8 * (p + 1) + 4);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float e[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) e[k] = SCALE ? x[r][8 * p + k] * inv[r] : x[r][8 * p + k];
            float a = acc[r];
            a = __builtin_fmaf(e[0], ya[0], a);
            a = __builtin_fmaf(e[1], ya[1], a);
            a = __builtin_fmaf(e[2], ya[2], a);
            a = __builtin_fmaf(e[3], ya[3], a);
            a = __builtin_fmaf(e[4], yb[0], a);
            a = __builtin_fmaf(e[5], yb[1], a);
            a = __builtin_fmaf(e[6], yb[2], a);
            a = __builtin_fmaf(e[7], yb[3], a);
            piece_fence(a);
            acc[r] = a;
        }
        ya = na;
        yb = nb;
    }
}

template <int D>
__device__ __forceinline__ void chunk_colsum(const float (&x)[D], float inv, int c, float* part, float* slab,
                                             float* csum, int wave, int lane, int tid) {
    float* sl = slab + wave * 256;
#pragma unroll
    for (int k = 0; k < D; k += 4)
        col4_sum(x[k] * inv, x[k + 1] * inv, x[k + 2] * inv, x[k + 3] * inv, sl, part + wave * D + k, lane);
    __syncthreads();
    if (tid < D) {
        const float* q = part + tid;
        const float s01 = q[0 * D] + q[1 * D], s23 = q[2 * D] + q[3 * D];
        const float s45 = q[4 * D] + q[5 * D], s67 = q[6 * D] + q[7 * D];
        csum[c * D + tid] = (s01 + s23) + (s45 + s67);
    }
    __syncthreads();
}

template <int D>
__device__ __forceinline__ void store_row_f32(const float (&x)[D], float* dst) {
#pragma unroll
    for (int k = 0; k < D; k += 4) *reinterpret_cast<f32x4_t*>(dst + k) = f32x4_t{x[k], x[k + 1], x[k + 2], x[k + 3]};
}

// The fma chain of LDS row s (scaled by inv with SCALE) against y, its pieces
// read one ahead instead of the whole row at once.
template <int D, bool SCALE>
__device__ __forceinline__ float fma_lds_row(const u32x4_t* lrows, int s, const float* y, float inv) {
    const Bf u = Bf::fresh();
    constexpr int NP = D / 8;
    float acc = 0.0f;
    u32x4_t w = lrows[slot<D, true>(s, 0)];
    f32x4_t ya = *reinterpret_cast<const f32x4_t*>(y);
    f32x4_t yb = *reinterpret_cast<const f32x4_t*>(y + 4);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        u32x4_t nw = w;
        f32x4_t na = ya, nb = yb;
        if (p + 1 < NP) {
            nw = lrows[slot<D, true>(s, p + 1)];
            na = *reinterpret_cast<const f32x4_t*>(y + 8 * (p + 1));
            nb = *reinterpret_cast<const f32x4_t*>(y + 8 * (p + 1) + 4);
        }
        float e[8] = {u.lo(w[0]), u.hi(w[0]), u.lo(w[1]), u.hi(w[1]),
                      u.lo(w[2]), u.hi(w[2]), u.lo(w[3]), u.hi(w[3])};
        if constexpr (SCALE) {
#pragma unroll
            for (int k = 0; k < 8; ++k) e[k] = e[k] * inv;
        }
        acc = __builtin_fmaf(e[0], ya[0], acc);
        acc = __builtin_fmaf(e[1], ya[1], acc);
        acc = __builtin_fmaf(e[2], ya[2], acc);
        acc = __builtin_fmaf(e[3], ya[3], acc);
        acc = __builtin_fmaf(e[4], yb[0], acc);
        acc = __builtin_fmaf(e[5], yb[1], acc);
        acc = __builtin_fmaf(e[6], yb[2], acc);
        acc = __builtin_fmaf(e[7], yb[3], acc);
        piece_fence(acc);
        w = nw;
        ya = na;
        yb = nb;
    }
    return acc;
}

// A greedy step's chains on the fp32 path: the register rows and this
// thread's LDS row (slot s) against y in one loop over pieces, so that each
// piece of y is read once for all of them and the chains interleave.  Each
// chain is the same as fma_rows' and fma_lds_row's.
template <int D, int R>
__device__ __forceinline__ void fma_rows_lds(const float (&x)[R][D], const u32x4_t* lrows, int s, const float* y,
                                             float (&acc)[R], float& acc_l) {
    const Bf u = Bf::fresh();
    constexpr int NP = D / 8;
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0f;
    float al = 0.0f;
    u32x4_t w = lrows[slot<D, true>(s, 0)];
    f32x4_t ya = *reinterpret_cast<const f32x4_t*>(y);
    f32x4_t yb = *reinterpret_cast<const f32x4_t*>(y + 4);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        u32x4_t nw = w;
        f32x4_t na = ya, nb = yb;
        if (p + 1 < NP) {
            nw = lrows[slot<D, true>(s, p + 1)];
            na = *reinterpret_cast<const f32x4_t*>(y + 8 * (p + 1));
            nb = *reinterpret_cast<const f32x4_t*>(y + 8 * (p + 1) + 4);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float a = acc[r];
            a = __builtin_fmaf(x[r][8 * p + 0], ya[0], a);
            a = __builtin_fmaf(x[r][8 * p + 1], ya[1], a);
            a = __builtin_fmaf(x[r][8 * p + 2], ya[2], a);
            a = __builtin_fmaf(x[r][8 * p + 3], ya[3], a);
            a = __builtin_fmaf(x[r][8 * p + 4], yb[0], a);
            a = __builtin_fmaf(x[r][8 * p + 5], yb[1], a);
            a = __builtin_fmaf(x[r][8 * p + 6], yb[2], a);
            a = __builtin_fmaf(x[r][8 * p + 7], yb[3], a);
            piece_fence(a);
            acc[r] = a;
        }
        al = __builtin_fmaf(u.lo(w[0]), ya[0], al);
        al = __builtin_fmaf(u.hi(w[0]), ya[1], al);
        al = __builtin_fmaf(u.lo(w[1]), ya[2], al);
        al = __builtin_fmaf(u.hi(w[1]), ya[3], al);
        al = __builtin_fmaf(u.lo(w[2]), yb[0], al);
        al = __builtin_fmaf(u.hi(w[2]), yb[1], al);
        al = __builtin_fmaf(u.lo(w[3]), yb[2], al);
        al = __builtin_fmaf(u.hi(w[3]), yb[3], al);
        piece_fence(al);
        w = nw;
        ya = na;
        yb = nb;
    }
    acc_l = al;
}

// Publishes pick r (uniform): its norm at xn[par] and its row in fp32 at
// xr[par] for the greedy step, and marks it taken.  A row held in bf16 (in
// LDS, in memory, or, on the packed path, in its lane's registers, staged
// through xr[1 - par], which no thread reads in this step) is converted by
// the first D / 8 lanes of its owner's wave, one 16-byte piece each, rather
// than by the owner alone; an fp32 register row is stored by its lane.
template <int D, bool F32, int RC, typename Rows>
__device__ __forceinline__ void publish(int r, int par, float* xr, float* xn, const Rows& xv, const float (&nrm)[RC],
                                        uint32_t& taken, const float* nst, float* Sst, const u32x4_t* lrows, int n_lds,
                                        const bkv_bf16* Q, int wave, int lane, int tid) {
    constexpr int RR = RC * kThreads;
    const int owner = r & (kThreads - 1), c_r = r / kThreads;
    float* dst = xr + par * D;
    if (F32 && c_r < RC) {   // an fp32 register row
        if (tid == owner) {
#pragma unroll
            for (int cc = 0; cc < RC; ++cc)
                if (cc == c_r) {
                    taken |= 1u << cc;
                    xn[par] = nrm[cc];
                    store_row_f32<D>(xv[cc], dst);
                }
        }
        return;
    }
    if (wave != owner / kWave) return;
    const bool me = lane == (owner & (kWave - 1));
    u32x4_t w = u32x4_t{0u, 0u, 0u, 0u};
    if (c_r < RC) {   // packed register row (the packed path only)
        if constexpr (!F32) {
            u32x4_t* stage = reinterpret_cast<u32x4_t*>(xr + (1 - par) * D);
            if (me) {
#pragma unroll
                for (int cc = 0; cc < RC; ++cc)
                    if (cc == c_r) {
                        taken |= 1u << cc;
                        xn[par] = nrm[cc];
#pragma unroll
                        for (int p = 0; p < D / 8; ++p) stage[p] = xv[cc][p];
                    }
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the stage is written before its pieces are read
            if (lane < D / 8) w = stage[lane];
        }
    } else {
        const int s = r - RR;
        if (me) {
            xn[par] = nst[s];
            Sst[s] = __builtin_nanf("");
        }
        if (lane < D / 8) {
            if constexpr (F32)   // every row past the registers is in LDS
                w = lrows[slot<D, true>(s, lane)];
            else
                w = s < n_lds ? lrows[slot<D, false>(s, lane)] : reinterpret_cast<const u32x4_t*>(Q + (size_t)r * D)[lane];
        }
    }
    if (lane < D / 8) {
        float* dp = dst + 8 * lane;
        *reinterpret_cast<f32x4_t*>(dp) = f32x4_t{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xFFFF0000u),
                                                  __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xFFFF0000u)};
        *reinterpret_cast<f32x4_t*>(dp + 4) = f32x4_t{__uint_as_float(w[2] << 16), __uint_as_float(w[2] & 0xFFFF0000u),
                                                      __uint_as_float(w[3] << 16), __uint_as_float(w[3] & 0xFFFF0000u)};
    }
}

// F32: the register-resident rows are kept in fp32 and the LDS rows (at most
// one per thread, piece-major) are streamed piece by piece; only when every
// row outside the registers is in LDS (no global tier), where the registers
// allow it.
template <int D, bool F32>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillArgs a) {
    using L = Pre<D, F32>;
    constexpr int RC = L::kRegChunks;
    constexpr int RR = L::kRegRows;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    float* xr = reinterpret_cast<float*>(smem + L::kXrOff);
    float* xn = reinterpret_cast<float*>(smem + L::kXnOff);
    int* wk = reinterpret_cast<int*>(smem + L::kWvOff);
    int* wi = reinterpret_cast<int*>(smem + L::kWiOff);
    float* part = reinterpret_cast<float*>(smem + L::kPartOff);
    float* slab = reinterpret_cast<float*>(smem + L::kSlabOff);
    float* csum = reinterpret_cast<float*>(smem + L::kCsumOff);
    float* ssum = reinterpret_cast<float*>(smem + L::kSsumOff);
    int* sel = reinterpret_cast<int*>(smem + L::kSelOff);

    const int b = blockIdx.x;
    if (b >= a.nbuf) return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int P = a.P, m = a.n_beacon;
    const bkv_bf16* Q = a.q + (size_t)b * a.q_stride;
    bkv_bf16* buf = a.qbuf + (size_t)b * a.qcap * D;

    if (m <= 0) {   // no representatives kept
        if (tid == 0) a.qcount[b] = 0;
        return;
    }
    if (P <= m) {   // nothing to sample: the prompt's rows are the representatives
        for (int e = tid; e < P * (D / 8); e += kThreads)
            reinterpret_cast<u32x4_t*>(buf)[e] = reinterpret_cast<const u32x4_t*>(Q)[e];
        if (a.fps_sel)
            for (int i = tid; i < m; i += kThreads) a.fps_sel[(size_t)b * m + i] = i < P ? i : -1;
        if (tid == 0) a.qcount[b] = P;
        return;
    }

    const int C = (P + kThreads - 1) / kThreads;   // chunks of rows (uniform over the workgroup)
    const int n_other = L::n_other(P);
    const int n_lds = L::n_lds_rows(P, a.lds_bytes);
    float* nst = reinterpret_cast<float*>(smem + L::kOtherOff);   // norms of the rows outside the registers
    float* Sst = nst + n_other;                                   // their S (NaN once taken)
    u32x4_t* lrows = reinterpret_cast<u32x4_t*>(smem + L::rows_off(P));

    // ---- norms and column sums of the unit rows, chunk by chunk (each chunk's
    // sums go to its own slot, so the order of the chunks does not matter).
    // The rows past the registers come first, copied into LDS on the way while
    // there is room; then the register rows are loaded.
#pragma unroll 1
    for (int c = RC; c < C; ++c) {
        const int j = c * kThreads + tid, s = j - RR;
        u32x4_t tmp[D / 8];
        load_row<D>(Q, P, j, tmp);
        const float nr = norm_of<D>(tmp);
        if (j < P) {
            nst[s] = nr;
            if (s < n_lds) {
#pragma unroll
                for (int p = 0; p < D / 8; ++p) lrows[slot<D, F32>(s, p)] = tmp[p];
            }
        }
        chunk_colsum<D>(tmp, inv_of(nr), c, part, slab, csum, wave, lane, tid);
    }
    typename RegRows<D, RC, F32>::type xv;
    float nrm[RC];
#pragma unroll
    for (int c = 0; c < RC; ++c) {
        u32x4_t w[D / 8];
        load_row<D>(Q, P, c * kThreads + tid, w);
        to_reg<D>(w, xv[c]);
    }
#pragma unroll
    for (int c = 0; c < RC; ++c) nrm[c] = norm_of<D>(xv[c]);
#pragma unroll
    for (int c = 0; c < RC; ++c)
        if (c < C) chunk_colsum<D>(xv[c], inv_of(nrm[c]), c, part, slab, csum, wave, lane, tid);
    // pairwise over the chunks, bottom-up in place; chunks past the last are zero
    if (tid < D) {
        int Cp = 1;
        while (Cp < C) Cp *= 2;
        for (int w = 1; w < Cp; w *= 2)
            for (int c = 0; c < C; c += 2 * w)
                csum[c * D + tid] = csum[c * D + tid] + (c + w < C ? csum[(c + w) * D + tid] : 0.0f);
        ssum[tid] = csum[tid];
    }
    __syncthreads();

    // ---- seed: the lowest mean cosine.  Selections are branch-free so that
    // the compiler cannot sink a row's arithmetic past the loop over pieces.
    const float fP = (float)P;
    float bv = __builtin_inff();
    int bi = kNone;
    {
        float inv[RC], av[RC];
#pragma unroll
        for (int c = 0; c < RC; ++c) inv[c] = inv_of(nrm[c]);
        fma_rows<D, RC, true>(xv, ssum, inv, av);
#pragma unroll
        for (int c = 0; c < RC; ++c) av[c] = av[c] / fP;
#pragma unroll
        for (int c = 0; c < RC; ++c) {
            const int j = c * kThreads + tid;
            const bool take = (j < P) & ((bi == kNone) | (av[c] < bv));
            bv = take ? av[c] : bv;
            bi = take ? j : bi;
        }
    }
#pragma unroll 1
    for (int c = RC; c < C; ++c) {
        const int j = c * kThreads + tid, s = j - RR;
        if (j >= P) break;
        float av;
        if constexpr (F32) {
            av = fma_lds_row<D, true>(lrows, s, ssum + opaque_zero(), inv_of(nst[s])) / fP;
        } else {
            u32x4_t tmp[D / 8];
            fetch_row<D>(Q, P, j, s, n_lds, lrows, tmp);
            av = mean_cos<D>(tmp, inv_of(nst[s]), ssum + opaque_zero(), fP);
        }
        if (bi == kNone || av < bv) {
            bv = av;
            bi = j;
        }
    }
    int r = block_argmin(bv, bi, wk, wi, wave, lane);

    // ---- greedy steps
    float S[RC];
    uint32_t taken = 0u;
#pragma unroll
    for (int c = 0; c < RC; ++c) S[c] = -__builtin_inff();
    for (int s = tid; s < n_other; s += kThreads) Sst[s] = -__builtin_inff();
    for (int t = 0;; ++t) {
        const int par = t & 1;
        // publish pick t: the selection order, its row and norm for the update
        if (tid == 0) sel[t] = r;
        publish<D, F32>(r, par, xr, xn, xv, nrm, taken, nst, Sst, lrows, n_lds, Q, wave, lane, tid);
        __syncthreads();
        if (t + 1 == m) break;
        const float* y = xr + par * D;
        const float ny = xn[par];
        bv = __builtin_inff();
        bi = kNone;
        // fp32 path with a row in LDS per thread (C = RC + 1): that row's chain runs with the register rows'
        float dl = 0.0f;
        {
            float dt[RC];
            if constexpr (F32) {
                if (C > RC) fma_rows_lds<D, RC>(xv, lrows, tid, y, dt, dl);
                else fma_rows<D, RC, false>(xv, y, nullptr, dt);
            } else {
                fma_rows<D, RC, false>(xv, y, nullptr, dt);
            }
#pragma unroll
            for (int c = 0; c < RC; ++c) {
                const int j = c * kThreads + tid;
                const bool live = (j < P) & !(taken & (1u << c));
                const float cs = (nrm[c] == 0.0f || ny == 0.0f) ? 0.0f : dt[c] / (nrm[c] * ny);
                const float sv = (live & (cs > S[c])) ? cs : S[c];
                S[c] = sv;
                const bool take = live & ((bi == kNone) | (sv < bv));
                bv = take ? sv : bv;
                bi = take ? j : bi;
            }
        }
#pragma unroll 1
    for (int c = RC; c < C; ++c) {
            const int j = c * kThreads + tid, s = j - RR;
            if (j >= P) break;
            float sv = Sst[s];
            if (sv != sv) continue;   // taken
            float cs;
            if constexpr (F32) {   // s == tid: the row's chain ran above
                const float nx = nst[s];
                cs = (nx == 0.0f || ny == 0.0f) ? 0.0f : dl / (nx * ny);
            } else {
                u32x4_t tmp[D / 8];
                fetch_row<D>(Q, P, j, s, n_lds, lrows, tmp);
                cs = cos_to<D>(tmp, nst[s], y + opaque_zero(), ny);
            }
            if (cs > sv) sv = cs;
            Sst[s] = sv;
            if (bi == kNone || sv < bv) {
                bv = sv;
                bi = j;
            }
        }
        const int q = (t + 1) & 1;
        r = block_argmin(bv, bi, wk + q * kWaves, wi + q * kWaves, wave, lane);
    }

    // ---- survivors in ascending prompt order, the selection order, the count
    if (a.fps_sel)
        for (int i = tid; i < m; i += kThreads) a.fps_sel[(size_t)b * m + i] = sel[i];
    for (int e = tid; e < m * (D / 8); e += kThreads) {
        const int i = e / (D / 8), p = e % (D / 8);
        const int ji = sel[i];
        int rank = 0;
        for (int k = 0; k < m; ++k) rank += sel[k] < ji ? 1 : 0;
        reinterpret_cast<u32x4_t*>(buf + (size_t)rank * D)[p] =
            reinterpret_cast<const u32x4_t*>(Q + (size_t)ji * D)[p];
    }
    if (tid == 0) a.qcount[b] = m;
}

template <int D>
hipError_t launch_d(PrefillArgs a, hipStream_t st) {
    // LDS for the rows past the registers: what one workgroup may take, at most a CU's 160 KB
    int dev = 0, lim = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&lim, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess) return e;
    a.lds_bytes = lim < kLdsBytes ? lim : kLdsBytes;
    // fp32 path: every row past the registers in LDS, at most one per thread, in a piece-major area sized
    // for one row per thread (its slots are p * 512 + s whatever the row count)
    using F = Pre<D, true>;
    using B = Pre<D, false>;
    const size_t f32_lds = (size_t)F::rows_off(a.P) + (size_t)kThreads * F::kRowBytes;
    if (F::n_other(a.P) <= kThreads && f32_lds <= (size_t)a.lds_bytes) {
        hipLaunchKernelGGL((prefill_kernel<D, true>), dim3(a.nbuf), dim3(kThreads), f32_lds, st, a);
    } else {
        if ((int)B::rows_off(a.P) > a.lds_bytes) return hipErrorInvalidValue;
        hipLaunchKernelGGL((prefill_kernel<D, false>), dim3(a.nbuf), dim3(kThreads), B::bytes(a.P, a.lds_bytes), st, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int d, hipStream_t st) {
    if (a.nbuf <= 0) return hipSuccess;
    return d == 64 ? launch_d<64>(a, st) : launch_d<128>(a, st);
}

}  // namespace bkv
