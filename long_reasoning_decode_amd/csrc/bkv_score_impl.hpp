// bkv_score_impl.hpp -- scores of one unit's keys by one 8-wave workgroup
// (device functions of the scoring kernel and of the fused eviction kernel).
//
// Scores (Notes §2.1 Eq. 4-5, §2.3 Eq. 7):
//   Score_j = max over the observation rows r of the unit's G query heads of
//             exp(z_rj - c_r),   c_r = logsumexp over the keys row r sees,
// computed in base 2 (z scaled by log2(e)/sqrt(d)).  Each query head gives 32
// rows: its beacons (buffer rows 0 .. min(qcount, n_beacon)) rotated to the
// current step t, then its recent queries rotated to their own positions
// (Notes §2.3, realignment); other row slots are inactive.
//
// Waves: head = wave / KS owns one query head's 32 rows (inactive when
// head >= G), ks = wave % KS takes the key tiles j = ks (mod KS).  The unit's
// keys stream twice through a 3-stage LDS ring of 2-tile (64-key) stages,
// filled by the gfx950 LDS-DMA load (global_load_lds_dwordx4) two stages ahead,
// in an XOR-swizzled layout: each DMA instruction reads whole key rows
// (coalesced) and the MFMA operand reads hit distinct banks.
//   pass 1: D[key][row] = K Q^T on bf16 MFMA 32x32x16 (fp32 accumulate); each
//           lane keeps an online (max, sum) of one row; the KS partials of a
//           row are merged in LDS into c_r;
//   pass 2: D[row][key] = Q K^T; max over the wave's rows of z - c per key,
//           then over the heads with LDS atomics.  It walks the stages last
//           to first: its first three stages are still in the ring from
//           pass 1, and the keys it reads last are the first ones the
//           compaction of the fused eviction kernel moves (more of them are
//           still in the caches then).
// Mean pooling (Notes §2.1 Eq. 6, pooled over queries and heads as in the
// Max/Mean ablation of Notes §3.3 Table 2) replaces pass 2's max by the sum of
// exp2(z - c) over the wave's rows; the heads' partial sums of a stage go to
// LDS and are added in head order by one wave during the next stage, so the
// result does not depend on wave timing.  The divisor counts every
// observation row of the group, sum_h min(qcount_h, n_beacon) + n_recent_q.
// One unit per 8-wave workgroup and two workgroups per CU keep about 512
// units in flight (about 285 MB at 2176 keys of d = 128), so a unit's keys
// are still in the MALL when the second pass (and the compaction of the
// fused eviction kernel) reads them again.
//
// Because the DMA bypasses registers, the compiler does not track it: the
// loops wait on vmcnt explicitly (this wave's DMA for the current stage) and
// use a bare s_barrier (so all waves' DMA for it is done) fenced against
// compiler reordering.
//
// Observation rows are rotated straight into the MFMA operand registers: with
// the 32x32x16 operand layout a lane holds, for its row, k = s*16 + half*8 + e
// (s < d/16, e < 8), so the RoPE partner k + d/2 sits in chunk s + d/32 of
// the same lane.  Rotation: fp32, every product and sum rounded on its own,
// then round to nearest even bf16.
#pragma once

#include "bkv_device.hpp"
#include "bkv_internal.hpp"

namespace bkv {
namespace score {

constexpr int kTileKeys = 32;
constexpr int kStageTiles = 2;                  // tiles per ring stage
constexpr int kStages = 3;                      // two stages in flight while one is consumed
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

template <int D>
struct Layout {
    static constexpr int kCpr = D / 8;                                // 16-byte chunks per key row
    static constexpr int kTileBytes = kTileKeys * D * 2;              // 8 KB (d = 128)
    static constexpr int kDmaPerTile = kTileBytes / 1024;             // 64 lanes x 16 B per DMA instruction
    static constexpr int kStageBytes = kStageTiles * kTileBytes;
    static constexpr int kDmaPerWave = kStageTiles * kDmaPerTile / kWaves;
    static constexpr int kRingBytes = kStages * kStageBytes;
    static constexpr int kCrowOff = kRingBytes;                       // float [8 heads][32 rows]
    static constexpr int kPartOff = kCrowOff + 8 * 32 * 4;            // float2 [waves][32 rows]
    static constexpr int kPsumOff = kPartOff + kWaves * 32 * 8;       // mean: float [2][8 heads][64 keys]
    static constexpr int kPsumBytes = 2 * 8 * kStageTiles * kTileKeys * 4;
    // then uint32 per-key codes [n_len]
    static constexpr int fixed_bytes(bool mean) { return mean ? kPsumOff + kPsumBytes : kPsumOff; }
    static_assert((kStageTiles * kDmaPerTile) % kWaves == 0, "stage DMA split");
};

// Score of a key from its code: max pooling keeps f32_order(max log2 weight),
// mean pooling the fp32 bits of the mean weight.
template <bool MEAN>
__device__ __forceinline__ float score_of(uint32_t code) {
    if constexpr (MEAN) return __uint_as_float(code);
    else return __builtin_amdgcn_exp2f(f32_unorder(code));
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // s_waitcnt immediate (gfx9): vmcnt[3:0] | expcnt[6:4]=7 | lgkmcnt[11:8]=15 | vmcnt[5:4]<<14
    __builtin_amdgcn_s_waitcnt((N & 15) | 0x0F70 | ((N >> 4) << 14));
}

// Workgroup barrier without the memory fence __syncthreads() carries (which
// would drain every in-flight DMA); the empty asm statements stop the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS accesses are done
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

struct RowInfo {
    int pos;
    int vis;     // last visible key slot
    bool valid;
};

__device__ __forceinline__ RowInfo row_info(const ScoreArgs& a, int uq, int b, int r) {
    RowInfo ri{0, -1, false};
    if (r < a.n_beacon) {
        const int nb_eff = clampi(a.qcount[uq], 0, a.n_beacon);
        if (r < nb_eff) {
            ri.pos = a.t[b];
            ri.vis = a.n_len - 1;
            ri.valid = true;
        }
    } else if (r < a.n_beacon + a.n_recent_q) {
        const int i = r - a.n_beacon;
        ri.pos = a.pos_recent[(size_t)b * a.n_recent_q + i];
        ri.vis = a.causal ? a.n_len - a.n_recent_q + i : a.n_len - 1;
        ri.valid = ri.vis >= 0;
    }
    ri.pos = clampi(ri.pos, 0, a.rope_rows - 1);
    return ri;
}

// Last key slot that observation row `row` sees (rows of inactive slots are
// treated as seeing everything; their c is +inf so they never contribute).
__device__ __forceinline__ int row_vis(const ScoreArgs& a, int row) {
    if (a.causal && row >= a.n_beacon && row < a.n_beacon + a.n_recent_q)
        return a.n_len - a.n_recent_q + (row - a.n_beacon);
    return a.n_len - 1;
}

template <int D>
__device__ __forceinline__ const bkv_bf16* row_src(const ScoreArgs& a, int uq, int r) {
    if (r < a.n_beacon) return a.qbuf + ((size_t)uq * a.qcap + r) * D;
    return a.q_recent + ((size_t)uq * a.n_recent_q + (r - a.n_beacon)) * D;
}

// Rotate this lane's half of one observation row into MFMA operand chunks.
template <int D>
__device__ __forceinline__ void rope_operand(const bkv_bf16* src, const float* cs_row, int half,
                                             bf16x8_t* op) {
    constexpr int kS = D / 16;   // operand chunks per lane
    constexpr int kH = D / 32;   // chunks in the first half of d
    u32x4_t raw[kS];
#pragma unroll
    for (int s = 0; s < kS; ++s)
        raw[s] = *reinterpret_cast<const u32x4_t*>(src + s * 16 + half * 8);
#pragma unroll
    for (int s = 0; s < kH; ++s) {
        const float* cs = cs_row + (size_t)(s * 16 + half * 8) * 2;
        f32x4_t t4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) t4[q] = *reinterpret_cast<const f32x4_t*>(cs + 4 * q);
        u32x4_t lo, hi;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
            uint32_t olo = 0, ohi = 0;
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int e = 2 * e2 + p;
                const float c = t4[e >> 1][(e & 1) * 2];
                const float sn = t4[e >> 1][(e & 1) * 2 + 1];
                const uint32_t w0 = raw[s][e2], w1 = raw[s + kH][e2];
                const float x0 = p ? __uint_as_float(w0 & 0xFFFF0000u) : __uint_as_float(w0 << 16);
                const float x1 = p ? __uint_as_float(w1 & 0xFFFF0000u) : __uint_as_float(w1 << 16);
                const float ac = x0 * c, bs = x1 * sn, bc = x1 * c, as = x0 * sn;
                const float y0 = ac - bs;
                const float y1 = bc + as;
                olo |= f32_to_bf16_bits(y0) << (16 * p);
                ohi |= f32_to_bf16_bits(y1) << (16 * p);
            }
            lo[e2] = olo;
            hi[e2] = ohi;
        }
        op[s] = __builtin_bit_cast(bf16x8_t, lo);
        op[s + kH] = __builtin_bit_cast(bf16x8_t, hi);
    }
}

// LDS 16-byte slot of (key row within the tile, 16-byte chunk of d).
template <int D>
__device__ __forceinline__ int slot_of(int row, int chunk) {
    constexpr int kCpr = D / 8;
    return row * kCpr + (chunk ^ (row & (kCpr - 1)));
}

template <int D>
__device__ __forceinline__ bf16x8_t k_operand(const bkv_bf16* tile, int row, int s, int half) {
    return __builtin_bit_cast(bf16x8_t,
                              *reinterpret_cast<const u32x4_t*>(tile + slot_of<D>(row, 2 * s + half) * 8));
}

// This wave's share of the DMA that fills one ring stage with the keys of
// stage `st` (tiles 4 st .. 4 st + 3).  Keys beyond the cache end load the
// last row; they are masked or skipped later.
template <int D>
__device__ __forceinline__ void dma_stage(const bkv_bf16* Ku, int st, int n_len, bkv_bf16* stage, int wave,
                                          int lane) {
    using L = Layout<D>;
#pragma unroll
    for (int k = 0; k < L::kDmaPerWave; ++k) {
        const int ins = wave * L::kDmaPerWave + k;
        const int tile = ins / L::kDmaPerTile, piece = ins % L::kDmaPerTile;
        const int slot = piece * 64 + lane;
        const int row = slot / L::kCpr;
        const int chunk = (slot % L::kCpr) ^ (row & (L::kCpr - 1));
        const int key = min((st * kStageTiles + tile) * kTileKeys + row, n_len - 1);
        __builtin_amdgcn_global_load_lds(
            Ku + (size_t)key * D + chunk * 8,
            (__attribute__((address_space(3))) void*)(stage + tile * (L::kTileBytes / 2) + piece * 64 * 8), 16, 0,
            0);
    }
}

// Per-key codes of unit u into codes[0 .. n_len) in LDS (see score_of).  All
// waves call it; on return the codes are complete and visible to the
// workgroup, and this wave has no memory operation in flight.
template <int D, int KS, bool MEAN>
__device__ void unit_codes(const ScoreArgs& a, int u, unsigned char* smem, uint32_t* codes) {
    using L = Layout<D>;
    constexpr int kS = D / 16;
    bkv_bf16* ring = reinterpret_cast<bkv_bf16*>(smem);
    float* crow = reinterpret_cast<float*>(smem + L::kCrowOff);
    float2* part = reinterpret_cast<float2*>(smem + L::kPartOff);

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int r = lane & 31, half = lane >> 5;
    const int head = wave / KS, ks = wave % KS;
    const bool active = head < a.G;
    const int b = (u / a.hkv) % a.batch;
    const int n_len = a.n_len;
    const bkv_bf16* Ku = a.K + (size_t)u * a.cap * D;
    const float sc2 = 1.4426950408889634f / __builtin_sqrtf((float)D);
    const int n_tiles = (n_len + kTileKeys - 1) / kTileKeys;
    const int n_st = (n_tiles + kStageTiles - 1) / kStageTiles;
    auto stage = [&](int i) { return ring + (i % kStages) * (L::kStageBytes / 2); };

    // first two stages in flight while the rows are rotated
    dma_stage<D>(Ku, 0, n_len, stage(0), wave, lane);
    if (n_st > 1) dma_stage<D>(Ku, 1, n_len, stage(1), wave, lane);
    asm volatile("" ::: "memory");
    bf16x8_t qop[kS];
    RowInfo ri{0, -1, false};
    if (active) ri = row_info(a, u * a.G + head, b, r);
    if (ri.valid) {
        rope_operand<D>(row_src<D>(a, u * a.G + head, r), a.rope_cs + (size_t)ri.pos * (D / 2) * 2, half, qop);
    } else {
#pragma unroll
        for (int s = 0; s < kS; ++s) qop[s] = __builtin_bit_cast(bf16x8_t, u32x4_t{0u, 0u, 0u, 0u});
    }
    const int vis = ri.valid ? ri.vis : -1;
    // every valid row sees keys [0, vis_floor]; rows that are not valid get c = +inf
    const int vis_floor = (a.causal && a.n_recent_q > 0) ? n_len - a.n_recent_q : n_len - 1;
    for (int j = tid; j < n_len; j += kThreads) codes[j] = f32_order(-__builtin_inff());

    // ---- pass 1: per-row online (max, sum), base 2
    float m_run = -__builtin_inff(), l_run = 0.0f;
    for (int st = 0; st < n_st; ++st) {
        if (st + 1 < n_st) wait_vm<L::kDmaPerWave>();
        else wait_vm<0>();
        lds_barrier();
        if (st + 2 < n_st) dma_stage<D>(Ku, st + 2, n_len, stage(st + 2), wave, lane);
        if (!active) continue;
#pragma unroll
        for (int i = 0; i < kStageTiles; ++i) {
            const int j = st * kStageTiles + i;
            if (j >= n_tiles || j % KS != ks) continue;
            const bkv_bf16* tl = stage(st) + i * (L::kTileBytes / 2);
            const int key0 = j * kTileKeys;
            f32x16_t acc = f32x16_t{};
#pragma unroll
            for (int s = 0; s < kS; ++s)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_operand<D>(tl, r, s, half), qop[s], acc, 0, 0, 0);
            float z[16];
            if (key0 + kTileKeys - 1 > vis_floor) {   // tile reaches a causal limit or the cache end
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int key = key0 + 8 * (q >> 2) + 4 * half + (q & 3);
                    z[q] = (key > vis || key >= n_len) ? -__builtin_inff() : acc[q];
                }
            } else {
#pragma unroll
                for (int q = 0; q < 16; ++q) z[q] = acc[q];
            }
            // common case: every term relative to the running max stays below 2^32
            float sum = 0.0f;
#pragma unroll
            for (int q = 0; q < 16; ++q) sum += __builtin_amdgcn_exp2f(__builtin_fmaf(z[q], sc2, -m_run));
            if (sum <= 4294967296.0f) {
                l_run += sum;
            } else {  // first keys of the row, or a much larger logit: rescale
                float tmax = -__builtin_inff();
#pragma unroll
                for (int q = 0; q < 16; ++q) tmax = __builtin_fmaxf(tmax, z[q]);
                const float mnew = __builtin_fmaxf(m_run, tmax * sc2);
                if (mnew != -__builtin_inff()) {
                    float s2 = 0.0f;
#pragma unroll
                    for (int q = 0; q < 16; ++q) s2 += __builtin_amdgcn_exp2f(__builtin_fmaf(z[q], sc2, -mnew));
                    l_run = l_run * __builtin_amdgcn_exp2f(m_run - mnew) + s2;
                    m_run = mnew;
                }
            }
        }
    }
    // merge the two key halves of each row; then the KS waves of each head
    {
        const float m2 = __shfl_xor(m_run, 32, 64);
        const float l2 = __shfl_xor(l_run, 32, 64);
        const float M = __builtin_fmaxf(m_run, m2);
        float Ls = 0.0f;
        if (M != -__builtin_inff())
            Ls = l_run * __builtin_amdgcn_exp2f(m_run - M) + l2 * __builtin_amdgcn_exp2f(m2 - M);
        if (half == 0) part[wave * 32 + r] = float2{M, Ls};
    }
    lds_barrier();   // every wave is done with the ring and has published its partials
    // Pass 2 takes the stages last to first.  Stage i sits in ring slot i % kStages in both passes, so
    // the last kStages stages of pass 1, its first ones, are still in the ring and need no load.
    auto rev = [&](int i) { return n_st - 1 - i; };
    if (active && ks == 0 && half == 0) {
        float M = -__builtin_inff(), Ls = 0.0f;
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            const float2 p = part[(head * KS + k) * 32 + r];
            const float Mn = __builtin_fmaxf(M, p.x);
            if (Mn != -__builtin_inff())
                Ls = Ls * __builtin_amdgcn_exp2f(M - Mn) + p.y * __builtin_amdgcn_exp2f(p.x - Mn);
            M = Mn;
        }
        float c = __builtin_inff();
        if (ri.valid && M != -__builtin_inff() && Ls > 0.0f) c = M + __builtin_log2f(Ls);
        crow[head * 32 + r] = c;
    }
    lds_barrier();   // c_r published

    // ---- pass 2: max (or sum) over rows of z - c, per key
    float cq[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) cq[q] = active ? crow[head * 32 + 8 * (q >> 2) + 4 * half + (q & 3)] : 0.0f;
    constexpr int kStageKeys = kStageTiles * kTileKeys;
    float* psum = reinterpret_cast<float*>(smem + L::kPsumOff);
    float inv_rows = 0.0f;
    if constexpr (MEAN) {
        int rows = 0;
        for (int h = 0; h < a.G; ++h) rows += clampi(a.qcount[u * a.G + h], 0, a.n_beacon) + a.n_recent_q;
        inv_rows = rows > 0 ? 1.0f / (float)rows : 0.0f;
    }
    // mean: one wave adds the heads' partial sums of stage rs, in head order
    auto reduce_stage = [&](int rs) {
        if (wave != rs % kWaves) return;
        const float* ps = psum + (rs & 1) * (8 * kStageKeys);
        const int key = rev(rs) * kStageKeys + lane;
        float sum = 0.0f;
        for (int h = 0; h < a.G; ++h) sum += ps[h * kStageKeys + lane];
        if (key < n_len) codes[key] = __float_as_uint(sum * inv_rows);
    };
    for (int st = 0; st < n_st; ++st) {
        if (st + 1 < n_st) wait_vm<L::kDmaPerWave>();
        else wait_vm<0>();
        lds_barrier();
        if (st + 2 < n_st && st + 2 >= kStages) dma_stage<D>(Ku, rev(st + 2), n_len, stage(rev(st + 2)), wave, lane);
        if constexpr (MEAN) {
            if (st > 0) reduce_stage(st - 1);
        }
        if (!active) continue;
#pragma unroll
        for (int i = 0; i < kStageTiles; ++i) {
            const int j = rev(st) * kStageTiles + i;
            if (j >= n_tiles || j % KS != ks) continue;
            const bkv_bf16* tl = stage(rev(st)) + i * (L::kTileBytes / 2);
            const int key = j * kTileKeys + r;
            f32x16_t acc = f32x16_t{};
#pragma unroll
            for (int s = 0; s < kS; ++s)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qop[s], k_operand<D>(tl, r, s, half), acc, 0, 0, 0);
            const bool edge = j * kTileKeys + kTileKeys - 1 > vis_floor;
            if constexpr (MEAN) {
                float sm = 0.0f;
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    float e = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[q], sc2, -cq[q]));
                    if (edge && key > row_vis(a, 8 * (q >> 2) + 4 * half + (q & 3))) e = 0.0f;
                    sm += e;
                }
                sm += __shfl_xor(sm, 32, 64);
                if (half == 0) psum[(st & 1) * (8 * kStageKeys) + head * kStageKeys + i * kTileKeys + r] = sm;
            } else {
                float cm = -__builtin_inff();
                if (edge) {
#pragma unroll
                    for (int q = 0; q < 16; ++q) {
                        float tv = __builtin_fmaf(acc[q], sc2, -cq[q]);
                        if (key > row_vis(a, 8 * (q >> 2) + 4 * half + (q & 3))) tv = -__builtin_inff();
                        cm = __builtin_fmaxf(cm, tv);
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < 16; ++q) cm = __builtin_fmaxf(cm, __builtin_fmaf(acc[q], sc2, -cq[q]));
                }
                cm = __builtin_fmaxf(cm, __shfl_xor(cm, 32, 64));
                if (half == 0 && key < n_len) atomicMax(&codes[key], f32_order(cm));
            }
        }
    }
    if constexpr (MEAN) {
        lds_barrier();   // the last stage's partial sums are in LDS
        reduce_stage(n_st - 1);
    }
    __syncthreads();
}

}  // namespace score
}  // namespace bkv
