// bkv_append_impl.hpp -- one step's key and value rows into the cache (Notes
// §2.2, App. Alg. 2): the key rotated to its position, as the observation
// rows of the scoring are, and the value copied.  Shared by the append kernel
// and the buffer update that runs it in the same launch.
#pragma once

#include "bkv_device.hpp"
#include "bkv_internal.hpp"

namespace bkv {

// Piece j < D / 8 of unit `unit`'s new rows: the pairs (i, i + D/2) for
// i = 4j .. 4j + 3 of the new key rotated in fp32, each product and sum
// rounded on its own, then rounded to bf16, and 16 bytes of the value row.
template <int D>
__device__ __forceinline__ void append_piece(const AppendArgs& a, int64_t unit, int j) {
    const int b = (int)((unit / a.hkv) % a.batch);
    const int p = clampi(a.pos[b], 0, a.rope_rows - 1);
    const size_t dst = ((size_t)unit * a.cap + a.L) * D;
    const bkv_bf16* k = a.k_new + (size_t)unit * D;
    const uint2 lo = *reinterpret_cast<const uint2*>(k + 4 * j);            // x_i,       i = 4j .. 4j + 3
    const uint2 hi = *reinterpret_cast<const uint2*>(k + 4 * j + D / 2);    // x_{i+D/2}
    const f32x4_t* cs = reinterpret_cast<const f32x4_t*>(a.rope_cs + ((size_t)p * (D / 2) + 4 * j) * 2);
    const f32x4_t cs01 = cs[0], cs23 = cs[1];                               // (c, s) of pairs i, i+1 | i+2, i+3
    const float c[4] = {cs01[0], cs01[2], cs23[0], cs23[2]};
    const float sn[4] = {cs01[1], cs01[3], cs23[1], cs23[3]};
    const uint32_t xw0[2] = {lo.x, lo.y}, xw1[2] = {hi.x, hi.y};
    uint32_t y0w[2], y1w[2];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        uint32_t o0 = 0, o1 = 0;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int q = 2 * w + e;
            const float x0 = bf16_bits_to_f32((xw0[w] >> (16 * e)) & 0xFFFFu);
            const float x1 = bf16_bits_to_f32((xw1[w] >> (16 * e)) & 0xFFFFu);
            const float y0 = x0 * c[q] - x1 * sn[q];
            const float y1 = x1 * c[q] + x0 * sn[q];
            o0 |= f32_to_bf16_bits(y0) << (16 * e);
            o1 |= f32_to_bf16_bits(y1) << (16 * e);
        }
        y0w[w] = o0;
        y1w[w] = o1;
    }
    *reinterpret_cast<uint2*>(a.K + dst + 4 * j) = make_uint2(y0w[0], y0w[1]);
    *reinterpret_cast<uint2*>(a.K + dst + 4 * j + D / 2) = make_uint2(y1w[0], y1w[1]);
    reinterpret_cast<u32x4_t*>(a.V + dst)[j] = reinterpret_cast<const u32x4_t*>(a.v_new + (size_t)unit * D)[j];
}

}  // namespace bkv
