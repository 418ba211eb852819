// The Q4_K dot product of one quant chunk for a lane-per-row wavefront, shared
// by the kernels that stream Q4_K tiles (the GEMV engines and the layer-chain
// launch).
//
// Format: "用 Python 重写 picoLM" page, dequantize_q4_K listing. A 144-byte
// super-block holds fp16 d (bytes 0-1), fp16 dmin (2-3), twelve bytes of packed
// 6-bit scales/mins (4-15) and 128 quant bytes (16-143). Quant chunk c (bytes
// 16+32c .. +31) gives weights 64c+t from its low nibbles (sub-block 2c) and
// 64c+32+t from its high nibbles (sub-block 2c+1). Weight = d*sc_j*q - dmin*mn_j.
#pragma once

#include "qwg_device.h"

namespace qwg {

// Scale and min of sub-blocks 2G and 2G+1 from the packed bytes p[0..11]
// (h.y = p[0..3], h.z = p[4..7], h.w = p[8..11]). For j < 4 the six bits sit in
// byte j (scale) / byte j+4 (min); for j >= 4 the low nibble comes from byte
// j+4 and the top two bits from bits 6-7 of byte j-4 (scale) / byte j (min).
template <int G>
__device__ __forceinline__ void q4k_scales(const uint4 &h, uint32_t &sc0, uint32_t &sc1,
                                           uint32_t &mn0, uint32_t &mn1) {
    if constexpr (G < 2) {
        constexpr int s0 = 16 * G, s1 = 16 * G + 8;
        sc0 = (h.y >> s0) & 63u;
        sc1 = (h.y >> s1) & 63u;
        mn0 = (h.z >> s0) & 63u;
        mn1 = (h.z >> s1) & 63u;
    } else {
        constexpr int s0 = 16 * (G - 2), s1 = s0 + 8;
        sc0 = ((h.w >> s0) & 15u) | (((h.y >> (s0 + 6)) & 3u) << 4);
        sc1 = ((h.w >> s1) & 15u) | (((h.y >> (s1 + 6)) & 3u) << 4);
        mn0 = ((h.w >> (s0 + 4)) & 15u) | (((h.z >> (s0 + 6)) & 3u) << 4);
        mn1 = ((h.w >> (s1 + 4)) & 15u) | (((h.z >> (s1 + 6)) & 3u) << 4);
    }
}

// Wavefront G's share of one super-block for this lane's row: quant chunk G.
// xat(bt, i) is activation 256*b + 64*G + i of batch element bt (uniform
// across the wave).
template <int G, int NB, typename XAt>
__device__ __forceinline__ void q4k_chunk_at(const uint8_t *rowp, XAt xat,
                                             const float (&sx0)[NB], const float (&sx1)[NB],
                                             uint32_t mlo, uint32_t mhi, float (&acc)[NB]) {
    const uint4 h = *(const uint4 *)rowp;
    const uint4 qa = *(const uint4 *)(rowp + 16 + 32 * G);
    const uint4 qb = *(const uint4 *)(rowp + 32 + 32 * G);
    uint32_t sc0, sc1, mn0, mn1;
    q4k_scales<G>(h, sc0, sc1, mn0, mn1);
    const float d = h2f_lo(h.x);
    const float dmin = h2f_hi(h.x);
    // Low nibbles enter as q*2^-24 and high nibbles as q*2^-20; fold 2^24 / 2^20
    // into the (exact) products d*sc.
    const float dsc0 = d * (float)(sc0 << 24);
    const float dsc1 = d * (float)(sc1 << 20);
    const float dmn0 = dmin * (float)mn0;
    const float dmn1 = dmin * (float)mn1;
    const uint32_t q[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
#pragma unroll
    for (int bt = 0; bt < NB; ++bt) {
        float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const uint32_t e = q[m] & mlo;            // bytes 0, 2: low nibbles
            const uint32_t o = (q[m] >> 8) & mlo;     // bytes 1, 3: low nibbles
            const uint32_t eh = q[m] & mhi;           // bytes 0, 2: high nibbles << 4
            const uint32_t oh = (q[m] >> 8) & mhi;    // bytes 1, 3: high nibbles << 4
            s0 = __builtin_fmaf(h2f_lo(e), xat(bt, 4 * m + 0), s0);
            s0 = __builtin_fmaf(h2f_lo(o), xat(bt, 4 * m + 1), s0);
            s0 = __builtin_fmaf(h2f_hi(e), xat(bt, 4 * m + 2), s0);
            s0 = __builtin_fmaf(h2f_hi(o), xat(bt, 4 * m + 3), s0);
            s1 = __builtin_fmaf(h2f_lo(eh), xat(bt, 32 + 4 * m + 0), s1);
            s1 = __builtin_fmaf(h2f_lo(oh), xat(bt, 32 + 4 * m + 1), s1);
            s1 = __builtin_fmaf(h2f_hi(eh), xat(bt, 32 + 4 * m + 2), s1);
            s1 = __builtin_fmaf(h2f_hi(oh), xat(bt, 32 + 4 * m + 3), s1);
        }
        float a = acc[bt];
        a = __builtin_fmaf(dsc0, s0, a);
        a = __builtin_fmaf(dsc1, s1, a);
        a = __builtin_fmaf(-dmn0, sx0[bt], a);
        a = __builtin_fmaf(-dmn1, sx1[bt], a);
        acc[bt] = a;
    }
}

// q4k_chunk_at for batch 1 with each sub-block's products summed in two
// interleaved chains (even and odd dwords of quants), added at the end: half
// the dependent FMA latency, for wavefronts that run with few others on their
// SIMD (the layer-chain launch). Same operations otherwise; the fp32 sums
// round in another order.
template <int G, typename XAt>
__device__ __forceinline__ void q4k_chunk_2chains(const uint8_t *rowp, XAt xat, float sx0,
                                                  float sx1, uint32_t mlo, uint32_t mhi,
                                                  float &acc) {
    const uint4 h = *(const uint4 *)rowp;
    const uint4 qa = *(const uint4 *)(rowp + 16 + 32 * G);
    const uint4 qb = *(const uint4 *)(rowp + 32 + 32 * G);
    uint32_t sc0, sc1, mn0, mn1;
    q4k_scales<G>(h, sc0, sc1, mn0, mn1);
    const float d = h2f_lo(h.x);
    const float dmin = h2f_hi(h.x);
    const float dsc0 = d * (float)(sc0 << 24);
    const float dsc1 = d * (float)(sc1 << 20);
    const float dmn0 = dmin * (float)mn0;
    const float dmn1 = dmin * (float)mn1;
    const uint32_t q[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
    float s0[2] = {0.0f, 0.0f}, s1[2] = {0.0f, 0.0f};
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int c = m & 1;
        const uint32_t e = q[m] & mlo;
        const uint32_t o = (q[m] >> 8) & mlo;
        const uint32_t eh = q[m] & mhi;
        const uint32_t oh = (q[m] >> 8) & mhi;
        s0[c] = __builtin_fmaf(h2f_lo(e), xat(4 * m + 0), s0[c]);
        s0[c] = __builtin_fmaf(h2f_lo(o), xat(4 * m + 1), s0[c]);
        s0[c] = __builtin_fmaf(h2f_hi(e), xat(4 * m + 2), s0[c]);
        s0[c] = __builtin_fmaf(h2f_hi(o), xat(4 * m + 3), s0[c]);
        s1[c] = __builtin_fmaf(h2f_lo(eh), xat(32 + 4 * m + 0), s1[c]);
        s1[c] = __builtin_fmaf(h2f_lo(oh), xat(32 + 4 * m + 1), s1[c]);
        s1[c] = __builtin_fmaf(h2f_hi(eh), xat(32 + 4 * m + 2), s1[c]);
        s1[c] = __builtin_fmaf(h2f_hi(oh), xat(32 + 4 * m + 3), s1[c]);
    }
    float a = acc;
    a = __builtin_fmaf(dsc0, s0[0] + s0[1], a);
    a = __builtin_fmaf(dsc1, s1[0] + s1[1], a);
    a = __builtin_fmaf(-dmn0, sx0, a);
    a = __builtin_fmaf(-dmn1, sx1, a);
    acc = a;
}

// The same with xg pointing at x[256*b + 64*G] of batch element 0, rows n_in
// apart.
template <int G, int NB>
__device__ __forceinline__ void q4k_chunk(const uint8_t *rowp, cfloat_p xg, int n_in,
                                          const float (&sx0)[NB], const float (&sx1)[NB],
                                          uint32_t mlo, uint32_t mhi, float (&acc)[NB]) {
    q4k_chunk_at<G, NB>(
        rowp, [&](int bt, int i) { return xg[(int64_t)bt * n_in + i]; }, sx0, sx1, mlo, mhi, acc);
}

// Sum of v over lanes 0..31, left in lanes 16..31, and over lanes 32..63, left
// in lanes 48..63. The butterfly gives every lane of a 16-lane row its row's
// sum (bitwise the same in each lane); a row broadcast then adds row 0's sum
// into row 1 and row 2's into row 3. Measured against a 16-lane xor shuffle
// (a bpermute through LDS and its address arithmetic): Q4_K stream 91.8 ->
// 90.2 us on one box.
__device__ __forceinline__ float half_wave_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
    // row_bcast:15 into rows 1 and 3 only
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false));
    return v;
}

}  // namespace qwg
