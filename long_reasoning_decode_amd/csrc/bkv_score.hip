// bkv_score.hip -- beacon/recent attention scores of every cached key.
//
// Scores (Notes §2.1 Eq. 4-5, §2.3 Eq. 7):
//   Score_j = max over the observation rows r of the unit's G query heads of
//             exp(z_rj - c_r),   c_r = logsumexp over the keys row r sees,
// computed in base 2 (z scaled by log2(e)/sqrt(d)).  Each query head gives one
// tile of 32 rows: its beacons (buffer rows 0 .. min(qcount, n_beacon))
// rotated to the current step t, then its recent queries rotated to their own
// positions (Notes §2.3, realignment); other row slots are inactive.
//
// One workgroup owns one unit (layer, batch element, KV head).  Each wave owns
// one query head (two when G > 4 or G = 2) and keeps its rotated rows in MFMA
// operand registers for the whole unit.  The unit's keys stream twice:
//   pass 1: D[key][row] = K Q^T on bf16 MFMA 32x32x16 (fp32 accumulate); each
//           lane keeps an online (max, sum) of one row -> c_r;
//   pass 2: D[row][key] = Q K^T; each lane keeps max over rows of z - c for
//           one key; exp2 once per key at the end.
// K streams through a 3-stage LDS ring of 32-key tiles filled by the gfx950
// LDS-DMA load (global_load_lds_dwordx4), two tiles ahead of the MFMAs, in an
// XOR-swizzled layout: each DMA instruction reads whole key rows (coalesced)
// and the MFMA operand reads hit distinct banks.  Because the DMA bypasses
// registers, the compiler does not track it: the loop waits on vmcnt
// explicitly (this wave's DMA for the current tile) and uses a bare s_barrier
// (so all waves' DMA for it is done) fenced against compiler reordering.
//
// Observation rows are rotated in the prologue straight into the MFMA operand
// registers: with the 32x32x16 operand layout a lane holds, for its row,
// k = s*16 + half*8 + e (s < d/16, e < 8), so the RoPE partner k + d/2 sits in
// chunk s + d/32 of the same lane.  Rotation: fp32, every product and sum
// rounded on its own, then round to nearest even bf16.
#include "bkv_device.hpp"
#include "bkv_internal.hpp"

namespace bkv {

namespace {

constexpr int kTileKeys = 32;
constexpr int kStages = 3;
constexpr int kMaxTiles = 8;  // query heads per unit

template <int D>
struct ScoreLayout {
    static constexpr int kCpr = D / 8;                            // 16-byte chunks per key row
    static constexpr int kTileBytes = kTileKeys * D * 2;          // 8 KB (d = 128)
    static constexpr int kDmaPerTile = kTileBytes / 1024;         // 64 lanes x 16 B per DMA instruction
    static constexpr int kRingBytes = kStages * kTileBytes;
    static constexpr int kCrowBytes = kMaxTiles * 32 * 4;
    static constexpr int kFixed = kRingBytes + kCrowBytes;        // + n_len * 4 for the per-key max
};

// Wait until at most n of this wave's vector memory operations are in flight.
__device__ __forceinline__ void wait_vm(int n) {
    // s_waitcnt immediate (gfx9): vmcnt[3:0] | expcnt[6:4]=7 | lgkmcnt[11:8]=15 | vmcnt[5:4]<<14
    switch (n) {
        case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
        case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
        case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
        case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
        default: __builtin_amdgcn_s_waitcnt(0x0F78); break;  // 8
    }
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
    const int nb_eff = clampi(a.qcount[uq], 0, a.n_beacon);
    if (r < a.n_beacon) {
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

// This wave's share of the DMA that fills one ring stage with keys [key0, key0 + 32).
template <int D, int W>
__device__ __forceinline__ void dma_tile(const bkv_bf16* Ku, int key0, int n_len, bkv_bf16* stage, int wave,
                                         int lane) {
    using L = ScoreLayout<D>;
#pragma unroll
    for (int j = 0; j < L::kDmaPerTile / W; ++j) {
        const int ins = wave * (L::kDmaPerTile / W) + j;
        const int slot = ins * 64 + lane;
        const int row = slot / L::kCpr;
        const int chunk = (slot % L::kCpr) ^ (row & (L::kCpr - 1));
        const int key = min(key0 + row, n_len - 1);
        __builtin_amdgcn_global_load_lds(Ku + (size_t)key * D + chunk * 8,
                                         (__attribute__((address_space(3))) void*)(stage + ins * 64 * 8), 16, 0, 0);
    }
}

template <int D, int W, int TPW>
__global__ __launch_bounds__(64 * W) void score_kernel(ScoreArgs a) {
    using L = ScoreLayout<D>;
    constexpr int kS = D / 16;
    constexpr int kDmaMine = L::kDmaPerTile / W;   // DMA instructions per tile per wave
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    bkv_bf16* ring = reinterpret_cast<bkv_bf16*>(smem);
    float* crow = reinterpret_cast<float*>(smem + L::kRingBytes);
    uint32_t* colmax = reinterpret_cast<uint32_t*>(smem + L::kFixed);

    const int u = blockIdx.x;
    if (u >= a.units) return;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int r = lane & 31, half = lane >> 5;
    const int b = (u / a.hkv) % a.batch;
    const int n_len = a.n_len;
    const bkv_bf16* Ku = a.K + (size_t)u * a.cap * D;
    const float sc2 = 1.4426950408889634f / __builtin_sqrtf((float)D);
    const int n_tiles = (n_len + kTileKeys - 1) / kTileKeys;
    const int vis_floor = (a.causal && a.n_recent_q > 0) ? n_len - a.n_recent_q : n_len - 1;
    auto stage = [&](int i) { return ring + (i % kStages) * (L::kTileBytes / 2); };

    // ---- prologue: observation rows -> operand registers
    bf16x8_t qop[TPW][kS];
    bool valid_r[TPW];
    int vis_r[TPW];
#pragma unroll
    for (int ti = 0; ti < TPW; ++ti) {
        const int tile = wave * TPW + ti;
        RowInfo ri{0, -1, false};
        if (tile < a.G) ri = row_info(a, u * a.G + tile, b, r);
        valid_r[ti] = ri.valid;
        vis_r[ti] = ri.valid ? ri.vis : n_len - 1;
        if (ri.valid) {
            rope_operand<D>(row_src<D>(a, u * a.G + tile, r), a.rope_cs + (size_t)ri.pos * (D / 2) * 2, half,
                            qop[ti]);
        } else {
#pragma unroll
            for (int s = 0; s < kS; ++s) qop[ti][s] = __builtin_bit_cast(bf16x8_t, u32x4_t{0u, 0u, 0u, 0u});
        }
    }
    for (int j = tid; j < n_len; j += 64 * W) colmax[j] = f32_order(-__builtin_inff());
    __builtin_amdgcn_s_waitcnt(0);  // prologue loads done: from here vmcnt counts only the DMA

    // ---- pass 1: per-row log-sum-exp (base 2)
    float m_run[TPW], l_run[TPW];
#pragma unroll
    for (int ti = 0; ti < TPW; ++ti) {
        m_run[ti] = -__builtin_inff();
        l_run[ti] = 0.0f;
    }
    dma_tile<D, W>(Ku, 0, n_len, stage(0), wave, lane);
    if (n_tiles > 1) dma_tile<D, W>(Ku, kTileKeys, n_len, stage(1), wave, lane);
    for (int i = 0; i < n_tiles; ++i) {
        wait_vm(i + 1 < n_tiles ? kDmaMine : 0);
        lds_barrier();
        if (i + 2 < n_tiles) dma_tile<D, W>(Ku, (i + 2) * kTileKeys, n_len, stage(i + 2), wave, lane);
        const bkv_bf16* tl = stage(i);
        const int key0 = i * kTileKeys;
        f32x16_t acc[TPW];
#pragma unroll
        for (int ti = 0; ti < TPW; ++ti) acc[ti] = f32x16_t{};
#pragma unroll
        for (int s = 0; s < kS; ++s) {
            const bf16x8_t kop = k_operand<D>(tl, r, s, half);
#pragma unroll
            for (int ti = 0; ti < TPW; ++ti)
                acc[ti] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[ti][s], acc[ti], 0, 0, 0);
        }
        const bool need_mask = key0 + kTileKeys - 1 > vis_floor;
#pragma unroll
        for (int ti = 0; ti < TPW; ++ti) {
            float z[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                z[q] = acc[ti][q];
                if (need_mask) {
                    const int key = key0 + 8 * (q >> 2) + 4 * half + (q & 3);
                    if (key >= n_len || key > vis_r[ti]) z[q] = -__builtin_inff();
                }
            }
            // common case: every term relative to the running max stays below 2^32
            float sum = 0.0f;
#pragma unroll
            for (int q = 0; q < 16; ++q) sum += __builtin_amdgcn_exp2f(__builtin_fmaf(z[q], sc2, -m_run[ti]));
            if (sum <= 4294967296.0f) {
                l_run[ti] += sum;
            } else {  // first keys of the row, or a much larger logit: rescale
                float tmax = -__builtin_inff();
#pragma unroll
                for (int q = 0; q < 16; ++q) tmax = __builtin_fmaxf(tmax, z[q]);
                const float mnew = __builtin_fmaxf(m_run[ti], tmax * sc2);
                if (mnew != -__builtin_inff()) {
                    float s2 = 0.0f;
#pragma unroll
                    for (int q = 0; q < 16; ++q) s2 += __builtin_amdgcn_exp2f(__builtin_fmaf(z[q], sc2, -mnew));
                    l_run[ti] = l_run[ti] * __builtin_amdgcn_exp2f(m_run[ti] - mnew) + s2;
                    m_run[ti] = mnew;
                }
            }
        }
    }
    // merge the two key halves of each row; publish c_r
#pragma unroll
    for (int ti = 0; ti < TPW; ++ti) {
        const float m2 = __shfl_xor(m_run[ti], 32, 64);
        const float l2 = __shfl_xor(l_run[ti], 32, 64);
        const float M = __builtin_fmaxf(m_run[ti], m2);
        float c = __builtin_inff();
        if (valid_r[ti] && M != -__builtin_inff()) {
            const float Ls = l_run[ti] * __builtin_amdgcn_exp2f(m_run[ti] - M) + l2 * __builtin_amdgcn_exp2f(m2 - M);
            c = M + __builtin_log2f(Ls);
        }
        if (half == 0) crow[(wave * TPW + ti) * 32 + r] = c;
    }
    // start pass 2's stream; the barrier also publishes c_r
    lds_barrier();  // every wave is done with the ring
    dma_tile<D, W>(Ku, 0, n_len, stage(0), wave, lane);
    if (n_tiles > 1) dma_tile<D, W>(Ku, kTileKeys, n_len, stage(1), wave, lane);

    // ---- pass 2: running max over rows of z - c, per key
    float cq[TPW][16];
#pragma unroll
    for (int ti = 0; ti < TPW; ++ti)
#pragma unroll
        for (int q = 0; q < 16; ++q) cq[ti][q] = crow[(wave * TPW + ti) * 32 + 8 * (q >> 2) + 4 * half + (q & 3)];
    for (int i = 0; i < n_tiles; ++i) {
        wait_vm(i + 1 < n_tiles ? kDmaMine : 0);
        lds_barrier();
        if (i + 2 < n_tiles) dma_tile<D, W>(Ku, (i + 2) * kTileKeys, n_len, stage(i + 2), wave, lane);
        const bkv_bf16* tl = stage(i);
        const int key0 = i * kTileKeys;
        f32x16_t acc[TPW];
#pragma unroll
        for (int ti = 0; ti < TPW; ++ti) acc[ti] = f32x16_t{};
#pragma unroll
        for (int s = 0; s < kS; ++s) {
            const bf16x8_t kop = k_operand<D>(tl, r, s, half);
#pragma unroll
            for (int ti = 0; ti < TPW; ++ti)
                acc[ti] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qop[ti][s], kop, acc[ti], 0, 0, 0);
        }
        const int key = key0 + r;
        const bool need_mask = key0 + kTileKeys - 1 > vis_floor;
        float cm = -__builtin_inff();
#pragma unroll
        for (int ti = 0; ti < TPW; ++ti)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                float tv = __builtin_fmaf(acc[ti][q], sc2, -cq[ti][q]);
                if (need_mask && key > row_vis(a, 8 * (q >> 2) + 4 * half + (q & 3))) tv = -__builtin_inff();
                cm = __builtin_fmaxf(cm, tv);
            }
        cm = __builtin_fmaxf(cm, __shfl_xor(cm, 32, 64));
        if (half == 0 && key < n_len) atomicMax(&colmax[key], f32_order(cm));
    }
    __syncthreads();
    float* out = a.scores + (size_t)u * n_len;
    for (int j = tid; j < n_len; j += 64 * W) out[j] = __builtin_amdgcn_exp2f(f32_unorder(colmax[j]));
}

template <int D, int W, int TPW>
hipError_t launch_one(const ScoreArgs& a, hipStream_t st) {
    const size_t smem = ScoreLayout<D>::kFixed + (size_t)a.n_len * 4;
    hipLaunchKernelGGL((score_kernel<D, W, TPW>), dim3(a.units), dim3(64 * W), smem, st, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const ScoreArgs& a, hipStream_t st) {
    switch (a.G) {
        case 1: return launch_one<D, 1, 1>(a, st);
        case 2: return launch_one<D, 1, 2>(a, st);
        case 3:
        case 4: return launch_one<D, 4, 1>(a, st);
        default: return launch_one<D, 4, 2>(a, st);
    }
}

}  // namespace

hipError_t launch_score(const ScoreArgs& a, int d, hipStream_t st) {
    if (a.units <= 0 || a.n_len <= 0) return hipSuccess;
    return d == 64 ? launch_d<64>(a, st) : launch_d<128>(a, st);
}

}  // namespace bkv
