// bkv_attention.hip -- one decode step's attention over the (compressed)
// cache (Notes §2.1, the second formula: the new token's query attends over
// the cached keys, new one included, and takes the softmax-weighted sum of
// the values), and the append of the new key and value it follows.
//
// One 4-wave workgroup per unit (layer, batch element, KV head); its G query
// heads are the rows of one MFMA operand (rows G..31 are zero).  Each wave
// takes a contiguous quarter of the cache in tiles of 32 keys and keeps a
// flash-attention state per row (running max and sum in base 2, fp32 output
// accumulator); the four states are merged through LDS at the end.
//   * logits: bf16 MFMA 32x32x16, keys as the A operand read straight from
//     HBM into registers (the next tile's loads are issued before the current
//     tile is used), the rotated queries as the B operand (RoPE as in the
//     scoring kernel);
//   * weights: exp2 of the scaled logits minus the running max, handed to the
//     value pass through a wave-private LDS tile;
//   * values: fp32 multiply-adds on the VALU, each lane owning a slice of one
//     row's output, value rows read from HBM.
// The work is bound by reading K and V once: 4 * d bytes per cached row.
#include "bkv_device.hpp"
#include "bkv_internal.hpp"
#include "bkv_score_impl.hpp"

namespace bkv {

namespace {

constexpr int kAttnWaves = 4;
constexpr int kTile = 32;

template <int D>
__device__ __forceinline__ void load_k_operand(const bkv_bf16* Ku, int key, int half, bf16x8_t (&op)[D / 16]) {
    const bkv_bf16* row = Ku + (size_t)key * D + half * 8;
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
        op[s] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(row + s * 16));
}

// GP: query rows padded to a power of two (lanes per output row = 64 / GP).
template <int D, int GP>
__global__ __launch_bounds__(64 * kAttnWaves) void attn_kernel(AttnArgs a) {
    constexpr int kS = D / 16;
    constexpr int LPR = (64 / GP < D / 2) ? 64 / GP : D / 2;   // lanes per output row
    constexpr int CPL = D / LPR;                              // output columns per lane (even)
    __shared__ float p_lds[kAttnWaves][GP][kTile];
    __shared__ float alpha_lds[kAttnWaves][GP];
    __shared__ float m_lds[kAttnWaves][GP], l_lds[kAttnWaves][GP];
    __shared__ __attribute__((aligned(16))) float o_lds[kAttnWaves][GP][D];

    const int u = blockIdx.x;
    if (u >= a.units) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 31, half = lane >> 5;
    const int G = a.G, L = a.n_len;
    const int b = (u / a.hkv) % a.batch;
    const bkv_bf16* Ku = a.K + (size_t)u * a.cap * D;
    const bkv_bf16* Vu = a.V + (size_t)u * a.cap * D;
    const float sc2 = 1.4426950408889634f / __builtin_sqrtf((float)D);

    // query rows rotated into the B operand (rows past G are zero)
    bf16x8_t qop[kS];
    if (r < G) {
        const int p = clampi(a.pos[b], 0, a.rope_rows - 1);
        score::rope_operand<D>(a.q + ((size_t)u * G + r) * D, a.rope_cs + (size_t)p * (D / 2) * 2, half, qop);
    } else {
#pragma unroll
        for (int s = 0; s < kS; ++s) qop[s] = __builtin_bit_cast(bf16x8_t, u32x4_t{0u, 0u, 0u, 0u});
    }

    // this wave's tiles
    const int n_tiles = (L + kTile - 1) / kTile;
    const int t0 = wave * n_tiles / kAttnWaves, t1 = (wave + 1) * n_tiles / kAttnWaves;
    const int rr = lane / LPR, c0 = (lane % LPR) * CPL;   // output row and first column of this lane
    const bool owns = rr < GP;                             // lanes past GP * LPR hold no output
    float m_run = -__builtin_inff(), l_run = 0.0f;          // per query row r (lanes r, r + 32 agree)
    float o[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) o[c] = 0.0f;

    bf16x8_t kop[kS];
    if (t0 < t1) load_k_operand<D>(Ku, min(t0 * kTile + r, L - 1), half, kop);
    for (int t = t0; t < t1; ++t) {
        const int k0 = t * kTile;
        f32x16_t acc = f32x16_t{};
#pragma unroll
        for (int s = 0; s < kS; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[s], qop[s], acc, 0, 0, 0);
        if (t + 1 < t1) load_k_operand<D>(Ku, min((t + 1) * kTile + r, L - 1), half, kop);
        // acc[q] = logit of key k0 + 8 (q >> 2) + 4 half + (q & 3) for query row r
        float z[16];
        float tmax = -__builtin_inff();
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int key = k0 + 8 * (q >> 2) + 4 * half + (q & 3);
            z[q] = key < L ? acc[q] * sc2 : -__builtin_inff();
            tmax = __builtin_fmaxf(tmax, z[q]);
        }
        tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float m_new = __builtin_fmaxf(m_run, tmax);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        float lsum = 0.0f;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const float pv = __builtin_amdgcn_exp2f(z[q] - m_new);
            lsum += pv;
            if (r < GP) p_lds[wave][r][8 * (q >> 2) + 4 * half + (q & 3)] = pv;
        }
        lsum += __shfl_xor(lsum, 32, 64);
        l_run = l_run * alpha + lsum;
        m_run = m_new;
        if (r < GP && half == 0) alpha_lds[wave][r] = alpha;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's P tile is in LDS
        // values: o[rr][c0 .. c0 + CPL) = alpha o + sum_k P[rr][k] V[k0 + k][c0 ..]
        const float al = owns ? alpha_lds[wave][rr] : 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) o[c] *= al;
#pragma unroll 4
        for (int k = 0; k < kTile && owns; ++k) {
            const float pk = p_lds[wave][rr][k];
            const int key = min(k0 + k, L - 1);
            const bkv_bf16* vrow = Vu + (size_t)key * D + c0;
            uint32_t w[CPL / 2];
#pragma unroll
            for (int e = 0; e < CPL / 2; ++e) w[e] = reinterpret_cast<const uint32_t*>(vrow)[e];
#pragma unroll
            for (int e = 0; e < CPL / 2; ++e) {
                o[2 * e] = __builtin_fmaf(pk, __uint_as_float(w[e] << 16), o[2 * e]);
                o[2 * e + 1] = __builtin_fmaf(pk, __uint_as_float(w[e] & 0xFFFF0000u), o[2 * e + 1]);
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // P reads done before the next tile's writes
    }

    // merge the four waves' states
    if (r < GP && half == 0) {
        m_lds[wave][r] = m_run;
        l_lds[wave][r] = l_run;
    }
    if (owns) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) o_lds[wave][rr][c0 + c] = o[c];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < G * D; e += 64 * kAttnWaves) {
        const int row = e / D, col = e % D;
        float M = -__builtin_inff();
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w) M = __builtin_fmaxf(M, m_lds[w][row]);
        float num = 0.0f, den = 0.0f;
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w) {
            const float f = __builtin_amdgcn_exp2f(m_lds[w][row] - M);
            num = __builtin_fmaf(o_lds[w][row][col], f, num);
            den = __builtin_fmaf(l_lds[w][row], f, den);
        }
        a.out[((size_t)u * G + row) * D + col] = num / den;
    }
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t st) {
    dim3 g(a.units), blk(64 * kAttnWaves);
    if (a.G <= 1) hipLaunchKernelGGL((attn_kernel<D, 1>), g, blk, 0, st, a);
    else if (a.G <= 2) hipLaunchKernelGGL((attn_kernel<D, 2>), g, blk, 0, st, a);
    else if (a.G <= 4) hipLaunchKernelGGL((attn_kernel<D, 4>), g, blk, 0, st, a);
    else hipLaunchKernelGGL((attn_kernel<D, 8>), g, blk, 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, int d, hipStream_t st) {
    if (a.units <= 0 || a.n_len <= 0) return hipSuccess;
    return d == 64 ? launch_d<64>(a, st) : launch_d<128>(a, st);
}

}  // namespace bkv
