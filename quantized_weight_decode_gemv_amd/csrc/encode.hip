// Encoder for the 98-byte IQ3 container (the iq3_pack.py page's encode()):
// fp32 weights -> blocks, every rounding as float32 numpy evaluates that
// function, so the bytes are identical to the CPU reference's:
//  1. signs (x < 0) and magnitudes; in each group of eight whose signs
//     multiply to -1 the sign of the first smallest magnitude is flipped;
//  2. d = sqrt(mean(mag^2)) / 20 + 1e-12, the mean's sum in numpy's pairwise
//     order (two halves of 128, eight running sums each, combined as a tree),
//     stored as fp16 (round to nearest even), its value used from then on;
//  3. per 32-weight sub-block and code 0..15: db = d*(0.5+code)*0.5; each
//     group of four magnitudes divided by max(db, 1e-20) takes the first grid
//     row of least g2 - 2*(q.g) (q.g summed left to right, no fused
//     multiply-add; g2 the row's sum of squares); the code's error is the
//     pairwise sum of (row*db - mag)^2 over the 32 weights; the first code of
//     least error is kept;
//  4. index bytes, words (four 7-bit sign groups, code in bits 28-31), d.
// One 256-thread workgroup per super-block: thread t owns weight t for steps
// 1-2, then four (sub-block, code, group) searches over the grid in LDS.
#include "qwg_device.h"

namespace qwg {

namespace {

__global__ __launch_bounds__(256) void iq3_encode_kernel(const float *__restrict__ x,
                                                         const float *__restrict__ grid,
                                                         uint8_t *__restrict__ dst,
                                                         int64_t nblocks) {
    __shared__ float4 sgrid[256];
    __shared__ float sg2[256];
    __shared__ float smag[256];
    __shared__ float ssq[256];
    __shared__ float sterm[8][16][32];    // [sub-block][code][weight] squared errors
    __shared__ uint8_t sidx[8][16][8];    // [sub-block][code][group] chosen rows
    __shared__ uint32_t sneg[8];          // sign bits of each sub-block's 32 weights
    __shared__ float serr[8][16];
    __shared__ float spart[16];
    __shared__ float sdv;

    const int t = threadIdx.x;
    const int lane = t & 63;
    {
        const float4 g = *(const float4 *)(grid + 4 * t);
        sgrid[t] = g;
        // numpy's order for four terms: one running sum from zero
        float r = 0.0f;
        r = __fadd_rn(r, __fmul_rn(g.x, g.x));
        r = __fadd_rn(r, __fmul_rn(g.y, g.y));
        r = __fadd_rn(r, __fmul_rn(g.z, g.z));
        r = __fadd_rn(r, __fmul_rn(g.w, g.w));
        sg2[t] = r;
    }

    for (int64_t blk = blockIdx.x; blk < nblocks; blk += gridDim.x) {
        const float v = x[blk * kQK + t];
        const float mag = fabsf(v);
        bool neg = v < 0.0f;
        smag[t] = mag;
        ssq[t] = __fmul_rn(mag, mag);
        __syncthreads();

        // 1. parity fix within the eight lanes of this weight's group
        const uint64_t nm = __ballot(neg);
        const uint32_t gbits = (uint32_t)(nm >> (lane & ~7)) & 0xFFu;
        if (__builtin_popcount(gbits) & 1) {
            const int g0 = t & ~7;
            int am = 0;
            for (int j = 1; j < 8; ++j)
                if (smag[g0 + j] < smag[g0 + am]) am = j;
            if ((t & 7) == am) neg = !neg;
        }
        const uint64_t fixed = __ballot(neg);
        if ((lane & 31) == 0) sneg[t >> 5] = (uint32_t)(fixed >> (lane & 32));

        // 2. d: eight running sums over each half of 128, then the trees
        if (t < 16) {
            const int h = t >> 3, j = t & 7;
            float r = ssq[128 * h + j];
            for (int i = 1; i < 16; ++i) r = __fadd_rn(r, ssq[128 * h + 8 * i + j]);
            spart[t] = r;
        }
        __syncthreads();
        if (t == 0) {
            float half[2];
            for (int h = 0; h < 2; ++h) {
                const float *r = spart + 8 * h;
                half[h] = __fadd_rn(__fadd_rn(__fadd_rn(r[0], r[1]), __fadd_rn(r[2], r[3])),
                                    __fadd_rn(__fadd_rn(r[4], r[5]), __fadd_rn(r[6], r[7])));
            }
            const float mean = __fdiv_rn(__fadd_rn(half[0], half[1]), 256.0f);
            const float d = __fadd_rn(__fdiv_rn(__fsqrt_rn(mean), 20.0f), 1e-12f);
            const _Float16 dh = (_Float16)d;
            const uint16_t bits = __builtin_bit_cast(uint16_t, dh);
            dst[blk * kIq3Bytes + 96] = (uint8_t)(bits & 0xFF);
            dst[blk * kIq3Bytes + 97] = (uint8_t)(bits >> 8);
            sdv = (float)dh;
        }
        __syncthreads();

        // 3. the searches: task = (sub-block ib, code, group g)
        const float dv = sdv;
#pragma unroll 1
        for (int k = 0; k < 4; ++k) {
            const int task = t + 256 * k;
            const int ib = task >> 7, code = (task >> 3) & 15, g = task & 7;
            const float db = __fmul_rn(__fmul_rn(dv, 0.5f + (float)code), 0.5f);
            const float den = db > 1e-20f ? db : 1e-20f;
            const float *m = smag + 32 * ib + 4 * g;
            const float q0 = __fdiv_rn(m[0], den), q1 = __fdiv_rn(m[1], den);
            const float q2 = __fdiv_rn(m[2], den), q3 = __fdiv_rn(m[3], den);
            int bi = 0;
            float bs = 0.0f;
            for (int e = 0; e < 256; ++e) {
                const float4 ge = sgrid[e];
                float dot = __fmul_rn(q0, ge.x);
                dot = __fadd_rn(dot, __fmul_rn(q1, ge.y));
                dot = __fadd_rn(dot, __fmul_rn(q2, ge.z));
                dot = __fadd_rn(dot, __fmul_rn(q3, ge.w));
                const float sc = __fsub_rn(sg2[e], __fmul_rn(2.0f, dot));
                if (e == 0 || sc < bs) {
                    bs = sc;
                    bi = e;
                }
            }
            sidx[ib][code][g] = (uint8_t)bi;
            const float4 gb = sgrid[bi];
            const float gv[4] = {gb.x, gb.y, gb.z, gb.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float df = __fsub_rn(__fmul_rn(gv[c], db), m[c]);
                sterm[ib][code][4 * g + c] = __fmul_rn(df, df);
            }
        }
        __syncthreads();

        // the codes' errors: numpy's pairwise order for 32 terms
        if (t < 128) {
            const int ib = t >> 4, code = t & 15;
            const float *T = sterm[ib][code];
            float r[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                r[j] = __fadd_rn(__fadd_rn(__fadd_rn(T[j], T[j + 8]), T[j + 16]), T[j + 24]);
            serr[ib][code] = __fadd_rn(__fadd_rn(__fadd_rn(r[0], r[1]), __fadd_rn(r[2], r[3])),
                                       __fadd_rn(__fadd_rn(r[4], r[5]), __fadd_rn(r[6], r[7])));
        }
        __syncthreads();

        // 4. the first code of least error, then the block's bytes
        if (t < 8) {
            const int ib = t;
            int best = 0;
            float be = serr[ib][0];
            for (int code = 1; code < 16; ++code)
                if (serr[ib][code] < be) {
                    be = serr[ib][code];
                    best = code;
                }
            uint8_t *out = dst + blk * kIq3Bytes;
            for (int g = 0; g < 8; ++g) out[8 * ib + g] = sidx[ib][best][g];
            const uint32_t sb = sneg[ib];
            uint32_t word = (uint32_t)best << 28;
            for (int l = 0; l < 4; ++l) word |= ((sb >> (8 * l)) & 0x7Fu) << (7 * l);
            for (int k = 0; k < 4; ++k) out[64 + 4 * ib + k] = (uint8_t)(word >> (8 * k));
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_iq3_encode(const float *x, const float *grid, uint8_t *dst, int64_t nblocks,
                             hipStream_t s) {
    int64_t groups = nblocks;
    if (groups > 65536) groups = 65536;
    hipLaunchKernelGGL(iq3_encode_kernel, dim3((unsigned)groups), dim3(256), 0, s, x, grid, dst,
                       nblocks);
    return hipGetLastError();
}

}  // namespace qwg
