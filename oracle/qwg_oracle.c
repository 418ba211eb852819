/*
 * qwg oracle: plain, slow CPU reference. TEST INFRASTRUCTURE ONLY (see
 * qwg_oracle.h): only tests/, __graft_entry__.smoke() and bench.py's
 * cpu_baseline leg use it; the HIP library never does.
 *
 * Built with -O2 -ffp-contract=off and no fast-math, so every fp32 operation
 * below is one IEEE round-to-nearest-even operation in the order written.
 *
 * Citations name the page and the listing or passage on it:
 *   [picoLM]  "用 Python 重写 picoLM", dequantize_q4_K listing
 *   [iq3pack] iq3_pack.py page: module docstring (byte layout) and decode()
 *   [codebook] codebook.py page: the format table of its module docstring,
 *             get_d, get_s, eff_np and dequant (llama.cpp's IQ3_XXS blocks)
 */
#include "qwg_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ fp16 */

/*
 * IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * e == 0: subnormal, value = m * 2^-24.  e == 31: infinity or NaN.
 * Otherwise (1024 + m) * 2^(e - 25). Evaluated in double, where every binary16
 * value is exact, then narrowed to float, where it is exact as well.
 * [picoLM] reads d and dmin as fp16 fields; [iq3pack] reads d as fp16.
 */
float orc_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return (float)(sign ? -v : v);
}

/*
 * binary32 -> binary16, round to nearest even (IEEE 754): magnitudes from
 * 65520 up become infinity, those below 2^-14 are multiples of 2^-24, the
 * rest have 11 significant bits. Evaluated in double, where every step is
 * exact except rint's rounding, which is the mode's (nearest even).
 * [iq3pack] stores d as fp16 (astype(np.float16)).
 */
uint16_t orc_f32_to_f16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if (isnan(f))
        return sign | 0x7E00;
    double a = fabs((double)f);
    if (a >= 65520.0)
        return sign | 0x7C00;
    if (a < ldexp(1.0, -14))
        return sign | (uint16_t)rint(ldexp(a, 24));   /* 1024 is the smallest normal */
    int e;
    frexp(a, &e);
    int E = e - 1;                                      /* 2^E <= a < 2^(E+1) */
    double n = rint(ldexp(a, 10 - E));                  /* 1024 .. 2048 */
    if (n >= 2048.0) {
        n = 1024.0;
        E += 1;
    }
    if (E > 15)
        return sign | 0x7C00;
    return sign | (uint16_t)((E + 15) << 10) | (uint16_t)(n - 1024.0);
}

/* ------------------------------------------------------------------ Q4_K */

/*
 * [picoLM] scale unpack: for sub-block j < 4 the scale is the low six bits of
 * packed byte j and the min the low six bits of byte j+4. For j >= 4 the
 * six-bit fields straddle bytes: the low four bits come from byte j+4 (low
 * nibble for the scale, high nibble for the min) and the top two bits from bits
 * 6..7 of byte j-4 (scale) or byte j (min).
 */
void orc_q4k_unpack_scales(const uint8_t p[12], uint8_t sc[8], uint8_t mn[8])
{
    for (int j = 0; j < 8; ++j) {
        if (j < 4) {
            sc[j] = p[j] & 63;
            mn[j] = p[j + 4] & 63;
        } else {
            sc[j] = (uint8_t)((p[j + 4] & 0xF) | ((p[j - 4] >> 6) << 4));
            mn[j] = (uint8_t)((p[j + 4] >> 4) | ((p[j] >> 6) << 4));
        }
    }
}

/*
 * The inverse of the unpack above (the page prints only the unpack). Each of
 * the 96 bits of p is written by exactly one field bit, so this is the unique
 * preimage: bytes 0..3 carry sc[0..3] plus the top two bits of sc[4..7], bytes
 * 4..7 carry mn[0..3] plus the top two bits of mn[4..7], bytes 8..11 carry the
 * low nibbles of sc[4..7] (low half) and mn[4..7] (high half).
 */
void orc_q4k_pack_scales(const uint8_t sc[8], const uint8_t mn[8], uint8_t p[12])
{
    for (int j = 0; j < 4; ++j) {
        p[j] = (uint8_t)((sc[j] & 63) | ((sc[j + 4] >> 4) << 6));
        p[j + 4] = (uint8_t)((mn[j] & 63) | ((mn[j + 4] >> 4) << 6));
        p[j + 8] = (uint8_t)((sc[j + 4] & 15) | ((mn[j + 4] & 15) << 4));
    }
}

/*
 * [picoLM] one block: d = fp16 at bytes 0..1, dmin = fp16 at bytes 2..3, the
 * packed scales at bytes 4..15, 128 quant bytes at 16..143. The quants form four
 * 32-byte chunks; chunk c holds weights 64c..64c+31 in its low nibbles (sub-block
 * 2c) and weights 64c+32..64c+63 in its high nibbles (sub-block 2c+1).
 * Weight value, in fp32 and in this order: (d * sc_j) * q - dmin * mn_j.
 */
static void q4k_block(const uint8_t *b, float *out)
{
    float d = orc_f16_to_f32((uint16_t)(b[0] | (b[1] << 8)));
    float dmin = orc_f16_to_f32((uint16_t)(b[2] | (b[3] << 8)));
    uint8_t sc[8], mn[8];
    orc_q4k_unpack_scales(b + 4, sc, mn);
    const uint8_t *qs = b + 16;
    for (int i = 0; i < ORC_QK; ++i) {
        int j = i / 32;         /* sub-block */
        int c = i / 64;         /* 32-byte chunk */
        uint8_t byte = qs[32 * c + i % 32];
        int q = (j % 2 == 0) ? (byte & 0xF) : (byte >> 4);
        float t = (d * (float)sc[j]) * (float)q;
        float u = dmin * (float)mn[j];
        out[i] = t - u;
    }
}

int orc_dequant_q4k(const uint8_t *src, int64_t n, float *dst)
{
    if (!src || !dst)
        return 1;
    if (n < 0 || n % ORC_QK)
        return 2;
    for (int64_t ib = 0; ib < n / ORC_QK; ++ib)
        q4k_block(src + ORC_Q4K_BYTES * ib, dst + ORC_QK * ib);
    return 0;
}

/* ------------------------------------------------------------------ IQ3 */

/*
 * 1 if weight t (0..31) of a sub-block is negative, from the sub-block's
 * uint32: weight t belongs to group t/8, whose seven stored sign bits sit at
 * bits 7*(t/8) .. 7*(t/8)+6; position j = t%8 < 7 reads bit j of them, and the
 * eighth position carries their parity, so that every group of eight has an
 * even number of negatives.
 */
static int container_weight_negative(uint32_t word, int t)
{
    uint32_t stored = (word >> (7 * (t >> 3))) & 0x7Fu;
    int j = t & 7;
    if (j < 7)
        return (int)((stored >> j) & 1u);
    return __builtin_popcount(stored) & 1;
}

/*
 * [iq3pack] one block: bytes 0..63 are grid indices (one per 4 weights), bytes
 * 64..95 eight little-endian uint32 words (one per 32-weight sub-block), bytes
 * 96..97 the fp16 super-scale d. In word ib, bits 7l..7l+6 (l = 0..3) are the
 * signs of weights 8l..8l+6 of the sub-block (bit set = negative), the sign of
 * weight 8l+7 is the XOR of those seven bits, and bits 28..31 are the sub-scale
 * code. Sub-block scale db = d * (0.5 + code) * 0.5, and weight t of sub-block ib
 * is grid[idx[8ib + t/4]][t % 4] * sign_t * db, with the grid in weight units.
 * decode() forms db in double (0.5 + an integer promotes), signs the
 * magnitude in fp32 and stores the double product as fp32; this does the same.
 */
static void iq3_block(const uint8_t *b, const float *grid, float *out)
{
    double d = orc_f16_to_f32((uint16_t)(b[96] | (b[97] << 8)));
    for (int ib = 0; ib < 8; ++ib) {
        const uint8_t *wp = b + 64 + 4 * ib;
        uint32_t word = (uint32_t)wp[0] | ((uint32_t)wp[1] << 8) | ((uint32_t)wp[2] << 16) |
                        ((uint32_t)wp[3] << 24);
        uint32_t code = (word >> 28) & 0xF;
        double db = d * (0.5 + (double)code) * 0.5;
        for (int t = 0; t < 32; ++t) {
            float mag = grid[4 * b[8 * ib + t / 4] + t % 4];
            /* the signed magnitude is exact in fp32; the product with db is
             * formed in double and stored as fp32 */
            float signed_mag = container_weight_negative(word, t) ? -mag : mag;
            out[32 * ib + t] = (float)((double)signed_mag * db);
        }
    }
}

int orc_dequant_iq3(const uint8_t *src, const float *grid, int64_t n, float *dst)
{
    if (!src || !grid || !dst)
        return 1;
    if (n < 0 || n % ORC_QK)
        return 2;
    for (int64_t ib = 0; ib < n / ORC_QK; ++ib)
        iq3_block(src + ORC_IQ3_BYTES * ib, grid, dst + ORC_QK * ib);
    return 0;
}

/*
 * [codebook] IQ3_XXS in llama.cpp's own byte order, 98 bytes per 256 weights:
 * the fp16 d at bytes 0..1 (get_d), the sub-scale s of 32-weight sub-block ib
 * in the top four bits of the little-endian uint32 at bytes 66+4ib (get_s),
 * and the codes in the remaining bytes. The effective sub-block scale is
 * eff = d * (0.5 + s) * 0.5, formed in fp32 in that order (eff_np), and each
 * weight is its integer value v (a codebook entry times its sign) times eff,
 * one fp32 product (dequant).
 *
 * The page leaves the code bytes to llama.cpp; the reading taken here is the
 * same field structure as the 98-byte container of the iq3_pack.py page with
 * the page's positions: the 64 grid indices at bytes 2..65 (index 8ib + t/4
 * for weight t of sub-block ib), and the signs in the low 28 bits of each
 * uint32, seven per group of eight weights (bit 7l+j negates weight 8l+j),
 * the eighth chosen so that a group has an even number of negatives (the
 * page's free-code section states that rule). The grid is the codebook as the
 * caller passes it (for llama.cpp's table, its integer entries 4..62).
 */
static void iq3_xxs_block(const uint8_t *b, const float *grid, float *out)
{
    float d = orc_f16_to_f32((uint16_t)(b[0] | (b[1] << 8)));
    for (int ib = 0; ib < 8; ++ib) {
        const uint8_t *wp = b + 66 + 4 * ib;
        uint32_t word = (uint32_t)wp[0] | ((uint32_t)wp[1] << 8) | ((uint32_t)wp[2] << 16) |
                        ((uint32_t)wp[3] << 24);
        uint32_t s = word >> 28;
        float eff = d * (0.5f + (float)s);
        eff = eff * 0.5f;
        for (int t = 0; t < 32; ++t) {
            float entry = grid[4 * b[2 + 8 * ib + t / 4] + t % 4];
            float v = container_weight_negative(word, t) ? -entry : entry;
            out[32 * ib + t] = v * eff;
        }
    }
}

int orc_dequant_iq3_xxs(const uint8_t *src, const float *grid, int64_t n, float *dst)
{
    if (!src || !grid || !dst)
        return 1;
    if (n < 0 || n % ORC_QK)
        return 2;
    for (int64_t ib = 0; ib < n / ORC_QK; ++ib)
        iq3_xxs_block(src + ORC_IQ3_BYTES * ib, grid, dst + ORC_QK * ib);
    return 0;
}

/*
 * [codebook] IQ3_S, 110 bytes per 256 weights: fp16 d at bytes 0..1 (get_d);
 * the 64 grid indices are 9 bits, their low eight bits at bytes 2..65 (index
 * k at byte 2+k) and their ninth bits packed little-endian at bytes 66..73
 * (bit k%8 of byte 66+k/8); one sign bit per weight packed little-endian at
 * bytes 74..105 (bit t%8 of byte 74+t/8 set = weight t negative); the 4-bit
 * sub-scales of the eight 32-weight sub-blocks as nibbles at bytes 106..109,
 * low nibble first (get_s). All positions as the page's encode writes them.
 * eff = d * (1 + 2s) in fp32 (eff_np); weight t = v * eff with v = grid entry
 * (index t/4, component t%4) times its sign (dequant). The grid has 512 rows.
 */
static void iq3s_block(const uint8_t *b, const float *grid, float *out)
{
    float d = orc_f16_to_f32((uint16_t)(b[0] | (b[1] << 8)));
    for (int ib = 0; ib < 8; ++ib) {
        int s = (b[106 + ib / 2] >> (4 * (ib % 2))) & 15;
        float eff = d * (1.0f + 2.0f * (float)s);
        for (int j = 0; j < 32; ++j) {
            int t = 32 * ib + j;
            int k = t / 4;
            int idx = b[2 + k] | (((b[66 + k / 8] >> (k % 8)) & 1) << 8);
            int neg = (b[74 + t / 8] >> (t % 8)) & 1;
            float entry = grid[4 * idx + t % 4];
            float v = neg ? -entry : entry;
            out[t] = v * eff;
        }
    }
}

/*
 * [codebook] IQ4_XS, 136 bytes per 256 weights: fp16 d at bytes 0..1; the
 * 6-bit sub-scale s of sub-block ib has its low four bits in nibble ib of
 * bytes 4..7 (low nibble first) and its top two bits at bits 2ib..2ib+1 of
 * the little-endian uint16 at bytes 2..3 (get_s). eff = d * (s - 32) in fp32
 * (eff_np); weight = v * eff, v = table[q] for the weight's 4-bit code q
 * (dequant; the 16-value table as the caller passes it). The page leaves the
 * code bytes to llama.cpp; the reading taken here: bytes 8..135, sixteen per
 * sub-block in the nibble order the page's encode writes for IQ4_NL: byte
 * 8+16ib+j holds weight j of sub-block ib in its low nibble and weight j+16
 * in its high nibble (j < 16).
 */
static void iq4xs_block(const uint8_t *b, const float *table, float *out)
{
    float d = orc_f16_to_f32((uint16_t)(b[0] | (b[1] << 8)));
    unsigned hi = (unsigned)(b[2] | (b[3] << 8));
    for (int ib = 0; ib < 8; ++ib) {
        int lo = (b[4 + ib / 2] >> (4 * (ib % 2))) & 15;
        int s = lo | (((hi >> (2 * ib)) & 3) << 4);
        float eff = d * ((float)s - 32.0f);
        for (int j = 0; j < 32; ++j) {
            uint8_t byte = b[8 + 16 * ib + j % 16];
            int q = j < 16 ? (byte & 15) : (byte >> 4);
            out[32 * ib + j] = table[q] * eff;
        }
    }
}

int orc_dequant_iq3s(const uint8_t *src, const float *grid, int64_t n, float *dst)
{
    if (!src || !grid || !dst)
        return 1;
    if (n < 0 || n % ORC_QK)
        return 2;
    for (int64_t ib = 0; ib < n / ORC_QK; ++ib)
        iq3s_block(src + ORC_IQ3S_BYTES * ib, grid, dst + ORC_QK * ib);
    return 0;
}

int orc_dequant_iq4xs(const uint8_t *src, const float *table, int64_t n, float *dst)
{
    if (!src || !table || !dst)
        return 1;
    if (n < 0 || n % ORC_QK)
        return 2;
    for (int64_t ib = 0; ib < n / ORC_QK; ++ib)
        iq4xs_block(src + ORC_IQ4XS_BYTES * ib, table, dst + ORC_QK * ib);
    return 0;
}

/* ------------------------------------------------------------------ IQ3 encoder */

/*
 * A float32 sum in numpy's pairwise order (its add.reduce over a contiguous
 * axis): below 8 terms, one running sum from 0; up to 128 terms, eight running
 * sums r[j] over elements j, j+8, j+16, ..., combined as
 * ((r0+r1)+(r2+r3))+((r4+r5)+(r6+r7)), then any remainder added in order;
 * longer runs split at n/2 rounded down to a multiple of 8, halves summed this
 * way and added.
 */
static float np_pairwise(const float *a, int n)
{
    if (n < 8) {
        float r = 0.0f;
        for (int i = 0; i < n; ++i)
            r += a[i];
        return r;
    }
    if (n <= 128) {
        float r[8];
        for (int j = 0; j < 8; ++j)
            r[j] = a[j];
        int i;
        for (i = 8; i < n - (n % 8); i += 8)
            for (int j = 0; j < 8; ++j)
                r[j] += a[i + j];
        float res = ((r[0] + r[1]) + (r[2] + r[3])) + ((r[4] + r[5]) + (r[6] + r[7]));
        for (; i < n; ++i)
            res += a[i];
        return res;
    }
    int n2 = n / 2;
    n2 -= n2 % 8;
    return np_pairwise(a, n2) + np_pairwise(a + n2, n - n2);
}

/*
 * [iq3pack] encode(), one 256-weight super-block, in float32 as the page's
 * numpy evaluates it:
 *  1. signs (negative when x < 0) and magnitudes; in every group of eight
 *     whose signs multiply to -1, the sign of the first smallest magnitude is
 *     flipped, so the stored seven signs and their parity describe the group;
 *  2. d = sqrt(mean(mag^2)) / 20 + 1e-12 (mean: pairwise sum / 256), stored
 *     as fp16, and the stored value is used from here on;
 *  3. per 32-weight sub-block, for every code 0..15: db = d*(0.5+code)*0.5,
 *     each group of four magnitudes divided by max(db, 1e-20) goes to the grid
 *     row of least g2 - 2*(q.g) (g2 = the row's sum of squares; the first such
 *     row), and the code's error is the pairwise sum of (grid*db - mag)^2 over
 *     the 32 weights; the first code of least error is kept;
 *  4. index bytes, the four 7-bit sign groups and the code form the word.
 * The page leaves the matrix product's order to its BLAS; here q.g is summed
 * left to right, product by product, without fused multiply-adds.
 */
static void iq3_encode_block(const float *x, const float *grid, const float *g2, uint8_t *out)
{
    float sign[256], mag[256], sq[256];
    for (int t = 0; t < 256; ++t) {
        sign[t] = x[t] < 0.0f ? -1.0f : 1.0f;
        mag[t] = fabsf(x[t]);
    }
    for (int b = 0; b < 32; ++b) {
        int neg = 0;
        for (int j = 0; j < 8; ++j)
            neg += sign[8 * b + j] < 0.0f;
        if (neg & 1) {
            int am = 0;
            for (int j = 1; j < 8; ++j)
                if (mag[8 * b + j] < mag[8 * b + am])
                    am = j;
            sign[8 * b + am] = -sign[8 * b + am];
        }
    }
    for (int t = 0; t < 256; ++t)
        sq[t] = mag[t] * mag[t];
    float mean = np_pairwise(sq, 256) / 256.0f;
    float d = sqrtf(mean) / 20.0f + 1e-12f;
    uint16_t dh = orc_f32_to_f16(d);
    out[96] = (uint8_t)(dh & 0xFF);
    out[97] = (uint8_t)(dh >> 8);
    float dv = orc_f16_to_f32(dh);
    for (int ib = 0; ib < 8; ++ib) {
        const float *m = mag + 32 * ib;
        float best_err = 0.0f;
        int best_code = 0;
        uint8_t best_idx[8] = {0};
        for (int code = 0; code < 16; ++code) {
            float db = dv * (0.5f + (float)code);
            db = db * 0.5f;
            float den = db > 1e-20f ? db : 1e-20f;
            uint8_t idx[8];
            float terms[32];
            for (int g = 0; g < 8; ++g) {
                float q[4];
                for (int c = 0; c < 4; ++c)
                    q[c] = m[4 * g + c] / den;
                int bi = 0;
                float bs = 0.0f;
                for (int e = 0; e < 256; ++e) {
                    const float *ge = grid + 4 * e;
                    float dot = q[0] * ge[0];
                    dot = dot + q[1] * ge[1];
                    dot = dot + q[2] * ge[2];
                    dot = dot + q[3] * ge[3];
                    float sc = g2[e] - 2.0f * dot;
                    if (e == 0 || sc < bs) {
                        bs = sc;
                        bi = e;
                    }
                }
                idx[g] = (uint8_t)bi;
                for (int c = 0; c < 4; ++c) {
                    float rec = grid[4 * bi + c] * db;
                    float df = rec - m[4 * g + c];
                    terms[4 * g + c] = df * df;
                }
            }
            float err = np_pairwise(terms, 32);
            if (code == 0 || err < best_err) {
                best_err = err;
                best_code = code;
                memcpy(best_idx, idx, 8);
            }
        }
        uint32_t word = (uint32_t)best_code << 28;
        for (int l = 0; l < 4; ++l) {
            uint32_t seven = 0;
            for (int j = 0; j < 7; ++j)
                seven |= (uint32_t)(sign[32 * ib + 8 * l + j] < 0.0f) << j;
            word |= seven << (7 * l);
        }
        memcpy(out + 8 * ib, best_idx, 8);
        for (int k = 0; k < 4; ++k)
            out[64 + 4 * ib + k] = (uint8_t)(word >> (8 * k));
    }
}

int orc_encode_iq3(const float *x, const float *grid, int64_t n_rows, int64_t n_in, uint8_t *dst)
{
    if (!x || !grid || !dst)
        return 1;
    if (n_rows < 1 || n_in <= 0 || n_in % ORC_QK)
        return 2;
    float g2[256];
    for (int e = 0; e < 256; ++e) {
        float r = 0.0f;   /* numpy's order for four terms: one running sum from 0 */
        for (int c = 0; c < 4; ++c)
            r += grid[4 * e + c] * grid[4 * e + c];
        g2[e] = r;
    }
    const int64_t nb = n_in / ORC_QK;
    int nth = orc_get_threads();
#pragma omp parallel for num_threads(nth) schedule(static)
    for (int64_t k = 0; k < n_rows * nb; ++k)
        iq3_encode_block(x + k * ORC_QK, grid, g2, dst + k * ORC_IQ3_BYTES);
    return 0;
}

/* ------------------------------------------------------------------ GEMV / GEMM */

static int g_threads = 0;

void orc_set_threads(int n) { g_threads = n; }

int orc_get_threads(void)
{
#ifdef _OPENMP
    return g_threads > 0 ? g_threads : omp_get_max_threads();
#else
    return 1;
#endif
}

/* One row: dequantize all of it to fp32, then fp64 dot products against each of
 * `batch` activation rows, k ascending. */
static void row_dot(const float *wrow, const float *x, int64_t n_in, int batch, int64_t n_out,
                    int64_t row, double *y, double *s)
{
    for (int bt = 0; bt < batch; ++bt) {
        const float *xb = x + (int64_t)bt * n_in;
        double acc = 0.0, abs_acc = 0.0;
        for (int64_t k = 0; k < n_in; ++k) {
            double p = (double)wrow[k] * (double)xb[k];
            acc += p;
            abs_acc += fabs(p);
        }
        y[(int64_t)bt * n_out + row] = acc;
        if (s)
            s[(int64_t)bt * n_out + row] = abs_acc;
    }
}

typedef void (*block_fn)(const uint8_t *, const float *, float *);

static void q4k_block_g(const uint8_t *b, const float *grid, float *out)
{
    (void)grid;
    q4k_block(b, out);
}

/* rows == NULL: all n_out rows, outputs indexed by row. Otherwise output i is
 * row rows[i]. */
static int gemm_generic(block_fn fn, int nbytes, const uint8_t *w, const float *grid,
                        const float *x, int64_t n_in, int64_t n_out, int batch,
                        const int64_t *rows, int64_t nrows, double *y, double *s)
{
    if (!w || !x || !y)
        return 1;
    if (n_in <= 0 || n_in % ORC_QK || n_out < 1 || batch < 1 || batch > 8)
        return 2;
    const int64_t nb = n_in / ORC_QK;
    const int64_t row_bytes = nb * nbytes;
    const int64_t count = rows ? nrows : n_out;
    const int64_t out_stride = rows ? nrows : n_out;
    int nth = orc_get_threads();
    int err = 0;
#pragma omp parallel num_threads(nth)
    {
        float *buf = (float *)malloc(sizeof(float) * (size_t)n_in);
        if (!buf) {
#pragma omp atomic write
            err = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t i = 0; i < count; ++i) {
                int64_t r = rows ? rows[i] : i;
                const uint8_t *wr = w + r * row_bytes;
                for (int64_t ib = 0; ib < nb; ++ib)
                    fn(wr + ib * nbytes, grid, buf + ib * ORC_QK);
                row_dot(buf, x, n_in, batch, out_stride, i, y, s);
            }
            free(buf);
        }
    }
    return err ? 3 : 0;
}

int orc_gemv_q4k(const uint8_t *w, const float *x, int64_t n_in, int64_t n_out, double *y,
                 double *s)
{
    return gemm_generic(q4k_block_g, ORC_Q4K_BYTES, w, NULL, x, n_in, n_out, 1, NULL, 0, y, s);
}

int orc_gemv_iq3(const uint8_t *w, const float *grid, const float *x, int64_t n_in,
                 int64_t n_out, double *y, double *s)
{
    if (!grid)
        return 1;
    return gemm_generic(iq3_block, ORC_IQ3_BYTES, w, grid, x, n_in, n_out, 1, NULL, 0, y, s);
}

int orc_gemm_q4k(const uint8_t *w, const float *x, int64_t n_in, int64_t n_out, int batch,
                 double *y, double *s)
{
    return gemm_generic(q4k_block_g, ORC_Q4K_BYTES, w, NULL, x, n_in, n_out, batch, NULL, 0, y,
                        s);
}

int orc_gemv_q4k_rows(const uint8_t *w, const float *x, int64_t n_in, const int64_t *rows,
                      int64_t nrows, double *y, double *s)
{
    if (!rows)
        return 1;
    if (nrows < 1)
        return 2;
    /* n_out only bounds the batch stride here; rows are trusted to be in range. */
    return gemm_generic(q4k_block_g, ORC_Q4K_BYTES, w, NULL, x, n_in, 1, 1, rows, nrows, y, s);
}

int orc_gemv_iq3_rows(const uint8_t *w, const float *grid, const float *x, int64_t n_in,
                      const int64_t *rows, int64_t nrows, double *y, double *s)
{
    if (!rows || !grid)
        return 1;
    if (nrows < 1)
        return 2;
    return gemm_generic(iq3_block, ORC_IQ3_BYTES, w, grid, x, n_in, 1, 1, rows, nrows, y, s);
}

int orc_gemv_iq3_xxs(const uint8_t *w, const float *grid, const float *x, int64_t n_in,
                     int64_t n_out, double *y, double *s)
{
    if (!grid)
        return 1;
    return gemm_generic(iq3_xxs_block, ORC_IQ3_BYTES, w, grid, x, n_in, n_out, 1, NULL, 0, y,
                        s);
}

int orc_gemv_iq3_xxs_rows(const uint8_t *w, const float *grid, const float *x, int64_t n_in,
                          const int64_t *rows, int64_t nrows, double *y, double *s)
{
    if (!rows || !grid)
        return 1;
    if (nrows < 1)
        return 2;
    return gemm_generic(iq3_xxs_block, ORC_IQ3_BYTES, w, grid, x, n_in, 1, 1, rows, nrows, y,
                        s);
}

int orc_gemv_iq3s(const uint8_t *w, const float *grid, const float *x, int64_t n_in,
                  int64_t n_out, double *y, double *s)
{
    if (!grid)
        return 1;
    return gemm_generic(iq3s_block, ORC_IQ3S_BYTES, w, grid, x, n_in, n_out, 1, NULL, 0, y, s);
}

int orc_gemv_iq4xs(const uint8_t *w, const float *table, const float *x, int64_t n_in,
                   int64_t n_out, double *y, double *s)
{
    if (!table)
        return 1;
    return gemm_generic(iq4xs_block, ORC_IQ4XS_BYTES, w, table, x, n_in, n_out, 1, NULL, 0, y, s);
}

int orc_gemv_iq3s_rows(const uint8_t *w, const float *grid, const float *x, int64_t n_in,
                       const int64_t *rows, int64_t nrows, double *y, double *s)
{
    if (!rows || !grid)
        return 1;
    if (nrows < 1)
        return 2;
    return gemm_generic(iq3s_block, ORC_IQ3S_BYTES, w, grid, x, n_in, 1, 1, rows, nrows, y, s);
}

int orc_gemv_iq4xs_rows(const uint8_t *w, const float *table, const float *x, int64_t n_in,
                        const int64_t *rows, int64_t nrows, double *y, double *s)
{
    if (!rows || !table)
        return 1;
    if (nrows < 1)
        return 2;
    return gemm_generic(iq4xs_block, ORC_IQ4XS_BYTES, w, table, x, n_in, 1, 1, rows, nrows, y, s);
}
