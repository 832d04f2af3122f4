// bkv_score.hip -- beacon/recent attention scores of every cached key.
//
// One workgroup owns one unit (layer, batch element, KV head) and its G query
// heads; each query head contributes one tile of 32 observation rows: its
// beacons (buffer rows 0 .. min(qcount, n_beacon)) rotated to the current
// step t, and its recent queries rotated to their own positions (Notes §2.3,
// realignment).  Row slots beyond those are inactive.
//
// Scores (Notes §2.1 Eq. 4-5, §2.3 Eq. 7):
//   Score_j = max over rows r of exp(z_rj - c_r),  c_r = logsumexp_j z_rj,
// computed in base 2 (z scaled by log2(e)/sqrt(d)).  Two streaming passes over
// the unit's keys, both on bf16 MFMA 32x32x16 with fp32 accumulation:
//   pass 1: D[key][row] tiles, per-lane online (max, sum) of one row -> c_r;
//   pass 2: D[row][key] tiles, per-lane running max over rows of z - c for
//           one key; exp2 once per key at the end.
// The unit's K rows stream through a double-buffered LDS tile (32 keys x d),
// loaded with coalesced 16-byte global reads; the second pass re-reads a
// unit that the same workgroup has just streamed, so it is served mostly
// from the L2 / infinity cache rather than HBM.
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

template <int D>
struct ScoreLayout {
    static constexpr int kRow = D + 8;                         // bf16 per LDS key row (16 B pad)
    static constexpr int kTileBytes = kTileKeys * kRow * 2;
    static constexpr int kKBytes = 2 * kTileBytes;             // double buffer
    static constexpr int kCrowBytes = 8 * 32 * 4;              // c_r of up to 8 tiles
    static constexpr int kFixed = kKBytes + kCrowBytes;
};

// Row role of observation slot r of query buffer uq.
struct RowInfo {
    int pos;
    int vis;     // last visible key slot
    bool valid;
};

__device__ __forceinline__ RowInfo row_info(const ScoreArgs& a, int uq, int b, int r) {
    RowInfo ri;
    ri.pos = 0;
    ri.vis = -1;
    ri.valid = false;
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

template <int D, int W>
__device__ __forceinline__ void load_tile_regs(const bkv_bf16* Ku, int key0, int n_len,
                                               u32x4_t* regs, int tid) {
    constexpr int kChunks = kTileKeys * D / 8;
    constexpr int kPer = (kChunks + 64 * W - 1) / (64 * W);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int ci = tid + j * 64 * W;
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (ci < kChunks) {
            const int row = ci / (D / 8), col = ci % (D / 8);
            if (key0 + row < n_len)
                v = *reinterpret_cast<const u32x4_t*>(Ku + (size_t)(key0 + row) * D + col * 8);
        }
        regs[j] = v;
    }
}

template <int D, int W>
__device__ __forceinline__ void store_tile_lds(bkv_bf16* lds, const u32x4_t* regs, int tid) {
    constexpr int kChunks = kTileKeys * D / 8;
    constexpr int kPer = (kChunks + 64 * W - 1) / (64 * W);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int ci = tid + j * 64 * W;
        if (ci < kChunks) {
            const int row = ci / (D / 8), col = ci % (D / 8);
            *reinterpret_cast<u32x4_t*>(lds + row * ScoreLayout<D>::kRow + col * 8) = regs[j];
        }
    }
}

template <int D, int W, int TPW>
__global__ __launch_bounds__(64 * W) void score_kernel(ScoreArgs a) {
    using L = ScoreLayout<D>;
    constexpr int kS = D / 16;
    constexpr int kChunks = kTileKeys * D / 8;
    constexpr int kPer = (kChunks + 64 * W - 1) / (64 * W);
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    bkv_bf16* kt = reinterpret_cast<bkv_bf16*>(smem);
    float* crow = reinterpret_cast<float*>(smem + L::kKBytes);
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

    // ---- prologue: observation rows -> operand registers
    bf16x8_t qop[TPW][kS];
    int vis_r[TPW];
    bool valid_r[TPW];
#pragma unroll
    for (int ti = 0; ti < TPW; ++ti) {
        const int tile = wave * TPW + ti;
        const bool tile_ok = tile < a.G;
        RowInfo ri;
        ri.valid = false;
        ri.vis = -1;
        if (tile_ok) ri = row_info(a, u * a.G + tile, b, r);
        valid_r[ti] = ri.valid;
        vis_r[ti] = ri.valid ? ri.vis : n_len - 1;
        if (ri.valid) {
            rope_operand<D>(row_src<D>(a, u * a.G + tile, r),
                            a.rope_cs + (size_t)ri.pos * (D / 2) * 2, half, qop[ti]);
        } else {
#pragma unroll
            for (int s = 0; s < kS; ++s) qop[ti][s] = __builtin_bit_cast(bf16x8_t, u32x4_t{0u, 0u, 0u, 0u});
        }
    }
    for (int j = tid; j < n_len; j += 64 * W) colmax[j] = f32_order(-__builtin_inff());

    const int n_tiles = (n_len + kTileKeys - 1) / kTileKeys;
    const int vis_floor = (a.causal && a.n_recent_q > 0) ? n_len - a.n_recent_q : n_len - 1;

    // ---- pass 1: per-row log-sum-exp (base 2)
    float m_run[TPW], l_run[TPW];
#pragma unroll
    for (int ti = 0; ti < TPW; ++ti) {
        m_run[ti] = -__builtin_inff();
        l_run[ti] = 0.0f;
    }
    u32x4_t pre[kPer];
    load_tile_regs<D, W>(Ku, 0, n_len, pre, tid);
    for (int kt_i = 0; kt_i < n_tiles; ++kt_i) {
        bkv_bf16* buf = kt + (kt_i & 1) * (L::kTileBytes / 2);
        store_tile_lds<D, W>(buf, pre, tid);
        __syncthreads();
        const int key0 = kt_i * kTileKeys;
        if (kt_i + 1 < n_tiles) load_tile_regs<D, W>(Ku, key0 + kTileKeys, n_len, pre, tid);
        f32x16_t acc[TPW];
#pragma unroll
        for (int ti = 0; ti < TPW; ++ti) acc[ti] = f32x16_t{};
#pragma unroll
        for (int s = 0; s < kS; ++s) {
            const bf16x8_t kop = __builtin_bit_cast(
                bf16x8_t, *reinterpret_cast<const u32x4_t*>(buf + r * L::kRow + s * 16 + half * 8));
#pragma unroll
            for (int ti = 0; ti < TPW; ++ti)
                acc[ti] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[ti][s], acc[ti], 0, 0, 0);
        }
        const bool need_mask = key0 + kTileKeys - 1 > vis_floor;
#pragma unroll
        for (int ti = 0; ti < TPW; ++ti) {
            float z[16];
            float tmax = -__builtin_inff();
            if (!need_mask) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    z[i] = acc[ti][i];
                    tmax = __builtin_fmaxf(tmax, z[i]);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = key0 + 8 * (i >> 2) + 4 * half + (i & 3);
                    const bool ok = key < n_len && key <= vis_r[ti];
                    z[i] = ok ? acc[ti][i] : -__builtin_inff();
                    tmax = __builtin_fmaxf(tmax, z[i]);
                }
            }
            const float mnew = __builtin_fmaxf(m_run[ti], tmax * sc2);
            if (mnew != -__builtin_inff()) {
                float sum = 0.0f;
#pragma unroll
                for (int i = 0; i < 16; ++i) sum += __builtin_amdgcn_exp2f(__builtin_fmaf(z[i], sc2, -mnew));
                l_run[ti] = l_run[ti] * __builtin_amdgcn_exp2f(m_run[ti] - mnew) + sum;
                m_run[ti] = mnew;
            }
        }
    }
    // combine the two key halves of each row; publish c_r
#pragma unroll
    for (int ti = 0; ti < TPW; ++ti) {
        const float m2 = __shfl_xor(m_run[ti], 32, 64);
        const float l2 = __shfl_xor(l_run[ti], 32, 64);
        const float M = __builtin_fmaxf(m_run[ti], m2);
        float c = __builtin_inff();
        if (valid_r[ti] && M != -__builtin_inff()) {
            const float Lsum = l_run[ti] * __builtin_amdgcn_exp2f(m_run[ti] - M) + l2 * __builtin_amdgcn_exp2f(m2 - M);
            c = M + __builtin_log2f(Lsum);
        }
        if (half == 0) crow[(wave * TPW + ti) * 32 + r] = c;
    }
    __syncthreads();

    // ---- pass 2: running max over rows of z - c, per key
    float cq[TPW][16];
    int visq[TPW][16];
#pragma unroll
    for (int ti = 0; ti < TPW; ++ti)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int row = 8 * (i >> 2) + 4 * half + (i & 3);
            cq[ti][i] = crow[(wave * TPW + ti) * 32 + row];
            const int tile = wave * TPW + ti;
            int v = n_len - 1;
            if (tile < a.G && row >= a.n_beacon && row < a.n_beacon + a.n_recent_q && a.causal)
                v = n_len - a.n_recent_q + (row - a.n_beacon);
            visq[ti][i] = v;
        }
    load_tile_regs<D, W>(Ku, 0, n_len, pre, tid);
    for (int kt_i = 0; kt_i < n_tiles; ++kt_i) {
        bkv_bf16* buf = kt + (kt_i & 1) * (L::kTileBytes / 2);
        store_tile_lds<D, W>(buf, pre, tid);
        __syncthreads();
        const int key0 = kt_i * kTileKeys;
        if (kt_i + 1 < n_tiles) load_tile_regs<D, W>(Ku, key0 + kTileKeys, n_len, pre, tid);
        f32x16_t acc[TPW];
#pragma unroll
        for (int ti = 0; ti < TPW; ++ti) acc[ti] = f32x16_t{};
#pragma unroll
        for (int s = 0; s < kS; ++s) {
            const bf16x8_t kop = __builtin_bit_cast(
                bf16x8_t, *reinterpret_cast<const u32x4_t*>(buf + r * L::kRow + s * 16 + half * 8));
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
            for (int i = 0; i < 16; ++i) {
                float tv = __builtin_fmaf(acc[ti][i], sc2, -cq[ti][i]);
                if (need_mask && key > visq[ti][i]) tv = -__builtin_inff();
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
        case 2: return launch_one<D, 2, 1>(a, st);
        case 3: return launch_one<D, 3, 1>(a, st);
        case 4: return launch_one<D, 4, 1>(a, st);
        case 5:
        case 6: return launch_one<D, 3, 2>(a, st);
        default: return launch_one<D, 4, 2>(a, st);
    }
}

}  // namespace

size_t score_smem_bytes(int d, int n_len) {
    return (d == 64 ? ScoreLayout<64>::kFixed : ScoreLayout<128>::kFixed) + (size_t)n_len * 4;
}

hipError_t launch_score(const ScoreArgs& a, int d, hipStream_t st) {
    if (a.units <= 0 || a.n_len <= 0) return hipSuccess;
    return d == 64 ? launch_d<64>(a, st) : launch_d<128>(a, st);
}

}  // namespace bkv
