/*
 * iq_oracle.c -- plain CPU reference of the importance-weighted IQ codebook
 * encode (IQ1_S, IQ2_XS), its decode, the top-C candidate emission and the
 * local-Hessian choice search.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  The product path never calls it and
 * shares no code, header, table or constant with it.
 *
 * Sources (NVIDIA Model-Optimizer pull-request pages):
 *  - "Add IQ tests and release notes" (#2450), the code review: the IQ1_S
 *    50-byte block layout (fp16 d, 32 low index bytes, 8 uint16 qh words with
 *    3 high index bits per group, a 3-bit local scale in bits 12-14 and the
 *    delta sign in bit 15), the IQ2_XS 74-byte layout (32 uint16 codes = 9-bit
 *    grid index + 7-bit sign mask, then 16 four-bit local scales), the scale
 *    predictor d = (amax / 16.875) * 0.61 rounded to fp16, the 16-way choice
 *    (8 local scales x 2 delta signs) and the rule that the lowest index wins
 *    on equal error, and the worked decode example (d = 2, local scale 3 gives
 *    14, bit 15 set gives delta = -1/8).
 *  - "Weight the IQ1 encoders by the square root of GPTQ's Hessian diagonal"
 *    (#2723), summary: each 8-value group is s*(q + delta) with q a ternary
 *    grid entry and delta = +-1/8; the codes minimise sum w*(x - s*(q+delta))^2;
 *    the local scale and delta are shared by the 4 groups of a 32-value
 *    sub-block.
 *  - "Register each GGML IQ format once" (#2525), IQ2_S commit body, section
 *    "What's distinctive about it": IQ2_XS stores a 7-bit parity-coded sign
 *    index and flips the weakest element to fix parity.
 *  - "Register each GGML IQ format once" (#2525), IQ1_M commit bodies (#2513
 *    "What's distinctive about it", "A scale-anchor correction"; #2595 "The
 *    kernel"): IQ1_M has no leading scale field, its fp16 d is reassembled
 *    from the top nibbles of four 16-bit scale words; a local scale per two
 *    groups and a delta shift per group, both searched with the IQ1_S grid;
 *    ties prefer the lower shift, then the lower entry; the anchor is
 *    clamp(0.58 + 0.035 * peak_to_rms, 0.65, 0.95) instead of 0.61.
 *  - "[4/4] Run the local-Hessian choice search as one CUDA kernel" (#3218)
 *    and the embedded "[1/4] ... local_hessian" body (#3158), steps 1-3: encode
 *    under every choice, give each group its best choice under its own H_gg,
 *    then revisit the groups twice, each taking the choice that most lowers the
 *    block's dw^T H dw with the others held.
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes of the repository):
 *  - choice index c = k + 8*deltabit; lowest c wins, lowest entry wins;
 *  - d is computed in fp32 (IEEE divide, then multiply, no contraction) and
 *    rounded to fp16 to nearest-even; fp16 d == 0 gives the all-zero block;
 *  - IQ2_XS local scale s = d*(2k+1), k = 0..15, one per 16 values; its
 *    predictor is d = fp16((amax / 155) * 0.61) (155 = 31 * 5, the top local
 *    multiplier times the largest grid magnitude);
 *  - the "weakest" element of an IQ2_XS group is the one with the smallest
 *    w*x*x, evaluated in fp32 as (w*x)*x, lowest index on ties; the flip is
 *    applied before the magnitude search; mask bit j (j < 7) = element j
 *    negative; element 7 negative iff the mask has odd popcount;
 *  - IQ2_XS scale nibble of scale group m: low half of byte 66 + m/2 for even
 *    m, high half for odd m;
 *  - choice search: ties go to the lowest candidate index; a sweep changes a
 *    group only on a strict improvement; groups are visited in ascending order;
 *  - IQ1_M: 56 bytes = 32 low index bytes, 16 bytes holding one nibble per
 *    group (3 high index bits, then the shift bit: set = -1/8; even group in
 *    the low nibble), then four little-endian 16-bit scale words; word w holds
 *    the 3-bit local scales k of scale groups 4w..4w+3 at bits 0, 3, 6, 9 and
 *    nibble w of d's fp16 bits at bits 12-15; s = d*(2k+1), k = 0..7; the
 *    predictor divisor is 16.875 as for IQ1_S; peak_to_rms = amax / sqrt(mean
 *    of squares) in fp32, the squares summed in a fixed order (64 partial sums
 *    of 4 consecutive squares, then pairwise at distances 1, 2, 4, ..., 32),
 *    the anchor 0.58 + 0.035 * ratio (multiply, then add) clamped to
 *    [0.65, 0.95]; an all-zero block has d = 0.
 *
 * All search arithmetic is float64 in the direct form sum_j w_j (x_j - xhat_j)^2.
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR_NONFINITE 1
#define ORC_ERR_IMPORTANCE 2
#define ORC_ERR_SCALE_RANGE 3
#define ORC_ERR_ARG 4
#define ORC_ERR_CODE 5

/* ---------------------------------------------------------------------- */
/* fp16 helpers, written from the IEEE 754 binary16 definition.            */
/* ---------------------------------------------------------------------- */

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* float32 -> binary16 bits, round to nearest, ties to even. */
uint16_t orc_f32_to_f16(float f)
{
    uint32_t x = f32_bits(f);
    uint32_t sign = (x >> 16) & 0x8000u;
    uint32_t a = x & 0x7fffffffu;
    if (a >= 0x7f800000u)                      /* inf or nan */
        return (uint16_t)(sign | 0x7c00u | (a > 0x7f800000u ? 0x200u : 0u));
    if (a >= 0x477ff000u)                      /* >= 65520 rounds to inf */
        return (uint16_t)(sign | 0x7c00u);
    if (a < 0x38800000u) {                     /* below 2^-14: subnormal half */
        /* value * 2^24 is the subnormal mantissa; exact in double. */
        double m = (double)fabsf(f) * 16777216.0;
        double r = nearbyint(m);               /* default mode: ties to even */
        return (uint16_t)(sign | (uint32_t)r);
    }
    uint32_t e = (a >> 23) - 127u + 15u;
    uint32_t mant = a & 0x7fffffu;
    uint32_t h = (e << 10) | (mant >> 13);
    uint32_t rem = mant & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u)))
        h += 1u;                               /* carry may move into the exponent */
    return (uint16_t)(sign | h);
}

double orc_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m | 0x400), e - 25);
    return sign ? -v : v;
}

/* ---------------------------------------------------------------------- */
/* Super-block scale predictor (review of #2450: d = (amax/16.875)*0.61).  */
/* ---------------------------------------------------------------------- */

static float block_amax(const float* x, int n)
{
    float m = 0.0f;
    for (int j = 0; j < n; ++j) {
        float a = fabsf(x[j]);
        if (a > m) m = a;
    }
    return m;
}

/* fp32 divide, then fp32 multiply (the library is built without contraction),
 * then fp16 round-to-nearest-even. */
uint16_t orc_predict_scale(float amax, float divisor, float anchor)
{
    volatile float t = amax / divisor;
    volatile float u = t * anchor;
    return orc_f32_to_f16(u);
}

#define IQ1S_DIVISOR 16.875f
#define IQ2XS_DIVISOR 155.0f
#define SCALE_ANCHOR 0.61f

static int check_block_inputs(const float* x, const float* w, int n)
{
    for (int j = 0; j < n; ++j)
        if (!isfinite(x[j])) return ORC_ERR_NONFINITE;
    if (w)
        for (int j = 0; j < n; ++j)
            if (!isfinite(w[j]) || w[j] < 0.0f) return ORC_ERR_IMPORTANCE;
    return ORC_OK;
}

/* Scale of one block: predicted, or the pinned fp16 value.  Returns an error
 * code; *dh receives the fp16 bits. */
static int block_scale(const float* x, float divisor, const uint16_t* pinned, uint16_t* dh)
{
    uint16_t h;
    if (pinned) {
        h = *pinned;
    } else {
        h = orc_predict_scale(block_amax(x, 256), divisor, SCALE_ANCHOR);
    }
    if ((h & 0x7c00u) == 0x7c00u) return ORC_ERR_SCALE_RANGE;   /* inf / nan */
    if ((h & 0x8000u) && (h & 0x7fffu)) return ORC_ERR_SCALE_RANGE; /* negative */
    *dh = (uint16_t)(h & 0x7fffu);                               /* -0 -> +0 */
    return ORC_OK;
}

/* ---------------------------------------------------------------------- */
/* IQ1_S                                                                   */
/* ---------------------------------------------------------------------- */

/* Weighted squared error of one group of 8 against s*(q + delta). */
static double iq1s_group_error(const float* x, const float* w, const float* q,
                               double s, double delta)
{
    double e = 0.0;
    for (int j = 0; j < 8; ++j) {
        double r = (double)x[j] - s * ((double)q[j] + delta);
        e += (w ? (double)w[j] : 1.0) * r * r;
    }
    return e;
}

/* Best grid entry of one group for a fixed (s, delta): lowest index among the
 * minima.  Returns the index, writes the error. */
static int iq1s_best_entry(const float* x, const float* w, const float* grid, int n,
                           double s, double delta, double* err)
{
    int best = 0;
    double be = INFINITY;
    for (int e = 0; e < n; ++e) {
        double v = iq1s_group_error(x, w, grid + 8 * e, s, delta);
        if (v < be) { be = v; best = e; }
    }
    *err = be;
    return best;
}

static void iq1s_pack_subblock(uint8_t* blk, int i, const int ent[4], int k, int dbit)
{
    uint32_t qh = 0;
    for (int l = 0; l < 4; ++l) {
        blk[2 + 4 * i + l] = (uint8_t)(ent[l] & 0xff);
        qh |= (uint32_t)((ent[l] >> 8) & 7) << (3 * l);
    }
    qh |= (uint32_t)k << 12;
    qh |= (uint32_t)dbit << 15;
    blk[34 + 2 * i] = (uint8_t)(qh & 0xff);
    blk[35 + 2 * i] = (uint8_t)(qh >> 8);
}

/* Encode one 256-value block.  choices: NULL, or 8 forced choice indices
 * (c = k + 8*deltabit) for the 8 sub-blocks. */
static int iq1s_encode_block(const float* x, const float* w, const float* grid, int n,
                             const uint16_t* pinned, const int32_t* choices, uint8_t* blk)
{
    memset(blk, 0, 50);
    int st = check_block_inputs(x, w, 256);
    if (st) return st;
    uint16_t dh;
    st = block_scale(x, IQ1S_DIVISOR, pinned, &dh);
    if (st) return st;
    if (dh == 0) return ORC_OK;                  /* canonical zero block */
    double d = orc_f16_to_f64(dh);
    blk[0] = (uint8_t)(dh & 0xff);
    blk[1] = (uint8_t)(dh >> 8);

    for (int i = 0; i < 8; ++i) {
        int c_lo = 0, c_hi = 16;
        if (choices) { c_lo = choices[i]; c_hi = c_lo + 1; }
        double best_cost = INFINITY;
        int best_c = c_lo, best_ent[4] = {0, 0, 0, 0};
        for (int c = c_lo; c < c_hi; ++c) {
            int k = c & 7, dbit = c >> 3;
            double s = d * (double)(2 * k + 1);
            double delta = dbit ? -0.125 : 0.125;
            double cost = 0.0;
            int ent[4];
            for (int l = 0; l < 4; ++l) {
                int off = 32 * i + 8 * l;
                double ge;
                ent[l] = iq1s_best_entry(x + off, w ? w + off : NULL, grid, n, s, delta, &ge);
                cost += ge;
            }
            if (cost < best_cost) {
                best_cost = cost;
                best_c = c;
                memcpy(best_ent, ent, sizeof(ent));
            }
        }
        iq1s_pack_subblock(blk, i, best_ent, best_c & 7, best_c >> 3);
    }
    return ORC_OK;
}

/* Returns ORC_ERR_CODE if an index is beyond the grid; that group decodes to 0. */
static int iq1s_decode_block(const uint8_t* blk, const float* grid, int n, double* out)
{
    int st = ORC_OK;
    uint16_t dh = (uint16_t)(blk[0] | (blk[1] << 8));
    double d = orc_f16_to_f64(dh);
    for (int i = 0; i < 8; ++i) {
        uint32_t qh = (uint32_t)blk[34 + 2 * i] | ((uint32_t)blk[35 + 2 * i] << 8);
        int k = (qh >> 12) & 7;
        double delta = (qh >> 15) ? -0.125 : 0.125;
        double s = d * (double)(2 * k + 1);
        for (int l = 0; l < 4; ++l) {
            int e = blk[2 + 4 * i + l] | (((qh >> (3 * l)) & 7) << 8);
            if (e >= n) {
                st = ORC_ERR_CODE;
                for (int j = 0; j < 8; ++j) out[32 * i + 8 * l + j] = 0.0;
                continue;
            }
            const float* q = grid + 8 * e;
            for (int j = 0; j < 8; ++j)
                out[32 * i + 8 * l + j] = s * ((double)q[j] + delta);
        }
    }
    return st;
}

/* ---------------------------------------------------------------------- */
/* IQ1_M                                                                   */
/* ---------------------------------------------------------------------- */

#define IQ1M_DIVISOR 16.875f

/* The peak-to-RMS anchor of one block, in fp32 with the fixed summation order
 * (every operation rounded to fp32: volatile, and no contraction). */
float orc_iq1m_anchor(const float* x, float amax)
{
    volatile float p[64], q[64];
    for (int l = 0; l < 64; ++l) {
        volatile float a0 = x[4 * l] * x[4 * l];
        volatile float a1 = x[4 * l + 1] * x[4 * l + 1];
        volatile float a2 = x[4 * l + 2] * x[4 * l + 2];
        volatile float a3 = x[4 * l + 3] * x[4 * l + 3];
        volatile float s = a0 + a1;
        s = s + a2;
        s = s + a3;
        p[l] = s;
    }
    for (int o = 1; o < 64; o <<= 1) {
        for (int l = 0; l < 64; ++l) q[l] = p[l] + p[l ^ o];
        for (int l = 0; l < 64; ++l) p[l] = q[l];
    }
    volatile float mean = p[0] / 256.0f;
    volatile float rms = sqrtf(mean);
    volatile float ratio = amax / rms;
    volatile float t = 0.035f * ratio;
    volatile float a = 0.58f + t;
    if (a < 0.65f) a = 0.65f;
    if (a > 0.95f) a = 0.95f;
    return a;
}

static int iq1m_block_scale(const float* x, const uint16_t* pinned, uint16_t* dh)
{
    uint16_t h;
    if (pinned) {
        h = *pinned;
    } else {
        float amax = block_amax(x, 256);
        h = amax > 0.0f ? orc_predict_scale(amax, IQ1M_DIVISOR, orc_iq1m_anchor(x, amax)) : 0;
    }
    if ((h & 0x7c00u) == 0x7c00u) return ORC_ERR_SCALE_RANGE;
    if ((h & 0x8000u) && (h & 0x7fffu)) return ORC_ERR_SCALE_RANGE;
    *dh = (uint16_t)(h & 0x7fffu);
    return ORC_OK;
}

/* Best (shift, entry) of one group for local scale s: the least error, then
 * the lower shift (delta = +1/8 first), then the lower entry. */
static void iq1m_best_group(const float* x, const float* w, const float* grid, int n, double s,
                            int* dbit, int* ent, double* err)
{
    double be = INFINITY;
    int bd = 0, bi = 0;
    for (int sh = 0; sh < 2; ++sh) {
        double delta = sh ? -0.125 : 0.125;
        double ge;
        int e = iq1s_best_entry(x, w, grid, n, s, delta, &ge);
        if (ge < be) { be = ge; bd = sh; bi = e; }
    }
    *dbit = bd;
    *ent = bi;
    *err = be;
}

static void iq1m_pack_group(uint8_t* blk, int g, int ent, int dbit)
{
    blk[g] = (uint8_t)(ent & 0xff);
    uint32_t nib = (uint32_t)((ent >> 8) & 7) | ((uint32_t)dbit << 3);
    blk[32 + g / 2] |= (uint8_t)(nib << (4 * (g & 1)));
}

static void iq1m_pack_scales(uint8_t* blk, const int k[16], uint16_t dh)
{
    for (int wd = 0; wd < 4; ++wd) {
        uint32_t v = 0;
        for (int t = 0; t < 4; ++t) v |= (uint32_t)(k[4 * wd + t] & 7) << (3 * t);
        v |= (uint32_t)((dh >> (4 * wd)) & 0xf) << 12;
        blk[48 + 2 * wd] = (uint8_t)(v & 0xff);
        blk[49 + 2 * wd] = (uint8_t)(v >> 8);
    }
}

/* choices: NULL or 16 forced local scales k in 0..7 (one per scale group). */
static int iq1m_encode_block(const float* x, const float* w, const float* grid, int n,
                             const uint16_t* pinned, const int32_t* choices, uint8_t* blk)
{
    memset(blk, 0, 56);
    int st = check_block_inputs(x, w, 256);
    if (st) return st;
    uint16_t dh;
    st = iq1m_block_scale(x, pinned, &dh);
    if (st) return st;
    if (dh == 0) return ORC_OK;
    double d = orc_f16_to_f64(dh);
    int kk[16];
    for (int m = 0; m < 16; ++m) {
        int k_lo = 0, k_hi = 8;
        if (choices) { k_lo = choices[m]; k_hi = k_lo + 1; }
        double best_cost = INFINITY;
        int best_k = k_lo, best_d[2] = {0, 0}, best_e[2] = {0, 0};
        for (int k = k_lo; k < k_hi; ++k) {
            double s = d * (double)(2 * k + 1);
            double cost = 0.0;
            int db[2], en[2];
            for (int h = 0; h < 2; ++h) {
                int off = 16 * m + 8 * h;
                double ge;
                iq1m_best_group(x + off, w ? w + off : NULL, grid, n, s, &db[h], &en[h], &ge);
                cost += ge;
            }
            if (cost < best_cost) {
                best_cost = cost;
                best_k = k;
                best_d[0] = db[0]; best_d[1] = db[1];
                best_e[0] = en[0]; best_e[1] = en[1];
            }
        }
        kk[m] = best_k;
        for (int h = 0; h < 2; ++h) iq1m_pack_group(blk, 2 * m + h, best_e[h], best_d[h]);
    }
    iq1m_pack_scales(blk, kk, dh);
    return ORC_OK;
}

static int iq1m_decode_block(const uint8_t* blk, const float* grid, int n, double* out)
{
    int st = ORC_OK;
    uint32_t sc[4];
    for (int wd = 0; wd < 4; ++wd) sc[wd] = (uint32_t)blk[48 + 2 * wd] | ((uint32_t)blk[49 + 2 * wd] << 8);
    /* d's fp16 bits: nibble wd (bits 4wd..4wd+3) is the top nibble of scale
       word wd (IQ1_M codec body, the four scale words) */
    uint16_t dh = 0;
    for (int wd = 0; wd < 4; ++wd) dh = (uint16_t)(dh | ((sc[wd] >> 12) << (4 * wd)));
    double d = orc_f16_to_f64(dh);
    for (int g = 0; g < 32; ++g) {
        int m = g / 2;
        int k = (int)((sc[m / 4] >> (3 * (m % 4))) & 7u);
        uint32_t nib = (blk[32 + g / 2] >> (4 * (g & 1))) & 0xfu;
        int e = blk[g] | (int)((nib & 7u) << 8);
        double delta = (nib & 8u) ? -0.125 : 0.125;
        double s = d * (double)(2 * k + 1);
        if (e >= n) {
            st = ORC_ERR_CODE;
            for (int j = 0; j < 8; ++j) out[8 * g + j] = 0.0;
            continue;
        }
        for (int j = 0; j < 8; ++j) out[8 * g + j] = s * ((double)grid[8 * e + j] + delta);
    }
    return st;
}

/* Top-C local scales of every scale group of one IQ1_M block, ordered by
 * (cost, k); each with its two codes (entry | shift << 11) and its error
 * vector xhat - x over the 16 columns.  A zero scale orders k = 0, 1, ... with
 * entry 0 and shift +1/8. */
static int iq1m_candidates_block(const float* x, const float* w, const float* grid, int n,
                                 int top_c, float* cand_err, int32_t* cand_choice,
                                 uint16_t* cand_codes)
{
    int st = check_block_inputs(x, w, 256);
    if (st) return st;
    uint16_t dh;
    st = iq1m_block_scale(x, NULL, &dh);
    if (st) return st;
    double d = orc_f16_to_f64(dh);
    for (int m = 0; m < 16; ++m) {
        double cost[8];
        int db[8][2], en[8][2];
        for (int k = 0; k < 8; ++k) {
            double s = d * (double)(2 * k + 1);
            cost[k] = 0.0;
            for (int h = 0; h < 2; ++h) {
                int off = 16 * m + 8 * h;
                double ge;
                iq1m_best_group(x + off, w ? w + off : NULL, grid, n, s, &db[k][h], &en[k][h], &ge);
                cost[k] += ge;
            }
            if (dh == 0) {
                cost[k] = 0.0;
                db[k][0] = db[k][1] = en[k][0] = en[k][1] = 0;
            }
        }
        int used[8] = {0};
        for (int r = 0; r < top_c; ++r) {
            int kb = -1;
            for (int k = 0; k < 8; ++k) {
                if (used[k]) continue;
                if (kb < 0 || cost[k] < cost[kb]) kb = k;
            }
            used[kb] = 1;
            cand_choice[m * top_c + r] = kb;
            double s = d * (double)(2 * kb + 1);
            for (int h = 0; h < 2; ++h) {
                const float* q = grid + 8 * en[kb][h];
                double delta = db[kb][h] ? -0.125 : 0.125;
                if (cand_codes)
                    cand_codes[(m * top_c + r) * 2 + h] = (uint16_t)(en[kb][h] | (db[kb][h] << 11));
                for (int j = 0; j < 8; ++j) {
                    int col = 16 * m + 8 * h + j;
                    double xhat = s * ((double)q[j] + delta);
                    cand_err[(m * top_c + r) * 16 + 8 * h + j] = (float)(xhat - (double)x[col]);
                }
            }
        }
    }
    return ORC_OK;
}

/* ---------------------------------------------------------------------- */
/* IQ2_XS                                                                  */
/* ---------------------------------------------------------------------- */

/* Signs of one group: input signs, with the weakest element flipped when the
 * count of negatives is odd.  Returns the 7-bit mask, fills sigma. */
static int iq2xs_group_signs(const float* x, const float* w, double* sigma)
{
    int neg[8], cnt = 0;
    for (int j = 0; j < 8; ++j) { neg[j] = x[j] < 0.0f; cnt += neg[j]; }
    if (cnt & 1) {
        int jw = 0;
        float best = INFINITY;
        for (int j = 0; j < 8; ++j) {
            volatile float wx = (w ? w[j] : 1.0f) * x[j];
            volatile float weak = wx * x[j];
            if (weak < best) { best = weak; jw = j; }
        }
        neg[jw] = !neg[jw];
    }
    int mask = 0;
    for (int j = 0; j < 8; ++j) {
        sigma[j] = neg[j] ? -1.0 : 1.0;
        if (j < 7 && neg[j]) mask |= 1 << j;
    }
    return mask;
}

static double iq2xs_group_error(const float* x, const float* w, const double* sigma,
                                const float* q, double s)
{
    double e = 0.0;
    for (int j = 0; j < 8; ++j) {
        double r = (double)x[j] - s * sigma[j] * (double)q[j];
        e += (w ? (double)w[j] : 1.0) * r * r;
    }
    return e;
}

static int iq2xs_best_entry(const float* x, const float* w, const double* sigma,
                            const float* grid, int n, double s, double* err)
{
    int best = 0;
    double be = INFINITY;
    for (int e = 0; e < n; ++e) {
        double v = iq2xs_group_error(x, w, sigma, grid + 8 * e, s);
        if (v < be) { be = v; best = e; }
    }
    *err = be;
    return best;
}

/* Per-scale-group costs of all 16 local scales with their winning entries. */
static void iq2xs_scale_group_costs(const float* x, const float* w, const float* grid, int n,
                                    double d, int m, double sig[2][8],
                                    double cost[16], int ent[16][2])
{
    for (int k = 0; k < 16; ++k) {
        double s = d * (double)(2 * k + 1);
        cost[k] = 0.0;
        for (int h = 0; h < 2; ++h) {
            int off = 16 * m + 8 * h;
            double ge;
            ent[k][h] = iq2xs_best_entry(x + off, w ? w + off : NULL, sig[h], grid, n, s, &ge);
            cost[k] += ge;
        }
    }
}

/* choices: NULL or 16 forced local scales (one per scale group). */
static int iq2xs_encode_block(const float* x, const float* w, const float* grid, int n,
                              const uint16_t* pinned, const int32_t* choices, uint8_t* blk)
{
    memset(blk, 0, 74);
    int st = check_block_inputs(x, w, 256);
    if (st) return st;
    uint16_t dh;
    st = block_scale(x, IQ2XS_DIVISOR, pinned, &dh);
    if (st) return st;
    if (dh == 0) return ORC_OK;
    double d = orc_f16_to_f64(dh);
    blk[0] = (uint8_t)(dh & 0xff);
    blk[1] = (uint8_t)(dh >> 8);

    for (int m = 0; m < 16; ++m) {
        double sig[2][8];
        int mask[2];
        for (int h = 0; h < 2; ++h) {
            int off = 16 * m + 8 * h;
            mask[h] = iq2xs_group_signs(x + off, w ? w + off : NULL, sig[h]);
        }
        double cost[16];
        int ent[16][2];
        iq2xs_scale_group_costs(x, w, grid, n, d, m, sig, cost, ent);
        int kb;
        if (choices) {
            kb = choices[m];
        } else {
            kb = 0;
            for (int k = 1; k < 16; ++k)
                if (cost[k] < cost[kb]) kb = k;
        }
        for (int h = 0; h < 2; ++h) {
            int g = 2 * m + h;
            uint32_t code = (uint32_t)ent[kb][h] | ((uint32_t)mask[h] << 9);
            blk[2 + 2 * g] = (uint8_t)(code & 0xff);
            blk[3 + 2 * g] = (uint8_t)(code >> 8);
        }
        if (m & 1) blk[66 + m / 2] |= (uint8_t)(kb << 4);
        else       blk[66 + m / 2] |= (uint8_t)kb;
    }
    return ORC_OK;
}

static int iq2xs_decode_block(const uint8_t* blk, const float* grid, int n, double* out)
{
    int st = ORC_OK;
    uint16_t dh = (uint16_t)(blk[0] | (blk[1] << 8));
    double d = orc_f16_to_f64(dh);
    for (int g = 0; g < 32; ++g) {
        uint32_t code = (uint32_t)blk[2 + 2 * g] | ((uint32_t)blk[3 + 2 * g] << 8);
        int e = code & 0x1ff;
        int mask = code >> 9;
        int m = g / 2;
        int k = (m & 1) ? (blk[66 + m / 2] >> 4) : (blk[66 + m / 2] & 15);
        double s = d * (double)(2 * k + 1);
        int pc = 0;
        for (int j = 0; j < 7; ++j) pc += (mask >> j) & 1;
        if (e >= n) {
            st = ORC_ERR_CODE;
            for (int j = 0; j < 8; ++j) out[8 * g + j] = 0.0;
            continue;
        }
        for (int j = 0; j < 8; ++j) {
            int neg = j < 7 ? (mask >> j) & 1 : (pc & 1);
            out[8 * g + j] = s * (neg ? -1.0 : 1.0) * (double)grid[8 * e + j];
        }
    }
    return st;
}

/* Top-C candidates of every scale group of one IQ2_XS block: the C lowest
 * (cost, k) local scales, their codes and their error vectors xhat - x. */
static int iq2xs_candidates_block(const float* x, const float* w, const float* grid, int n,
                                  int top_c, float* cand_err, int32_t* cand_choice,
                                  uint16_t* cand_codes)
{
    int st = check_block_inputs(x, w, 256);
    if (st) return st;
    uint16_t dh;
    st = block_scale(x, IQ2XS_DIVISOR, NULL, &dh);
    if (st) return st;
    double d = orc_f16_to_f64(dh);
    for (int m = 0; m < 16; ++m) {
        double sig[2][8];
        int mask[2];
        for (int h = 0; h < 2; ++h) {
            int off = 16 * m + 8 * h;
            mask[h] = iq2xs_group_signs(x + off, w ? w + off : NULL, sig[h]);
        }
        double cost[16];
        int ent[16][2];
        iq2xs_scale_group_costs(x, w, grid, n, d, m, sig, cost, ent);
        if (dh == 0) {
            /* zero block: every choice decodes to zero with entry 0 and no signs */
            for (int k = 0; k < 16; ++k) { cost[k] = 0.0; ent[k][0] = ent[k][1] = 0; }
            mask[0] = mask[1] = 0;
            for (int h = 0; h < 2; ++h) for (int j = 0; j < 8; ++j) sig[h][j] = 1.0;
        }
        int used[16] = {0};
        for (int r = 0; r < top_c; ++r) {
            int kb = -1;
            for (int k = 0; k < 16; ++k) {
                if (used[k]) continue;
                if (kb < 0 || cost[k] < cost[kb]) kb = k;
            }
            used[kb] = 1;
            cand_choice[m * top_c + r] = kb;
            double s = d * (double)(2 * kb + 1);
            for (int h = 0; h < 2; ++h) {
                const float* q = grid + 8 * ent[kb][h];
                if (cand_codes)
                    cand_codes[(m * top_c + r) * 2 + h] =
                        (uint16_t)(ent[kb][h] | (mask[h] << 9));
                for (int j = 0; j < 8; ++j) {
                    int col = 16 * m + 8 * h + j;
                    double xhat = s * sig[h][j] * (double)q[j];
                    cand_err[(m * top_c + r) * 16 + 8 * h + j] = (float)(xhat - (double)x[col]);
                }
            }
        }
    }
    return ORC_OK;
}

/* Top-C candidates of every sub-block of one IQ1_S block (#3158 step 1 with
 * IQ1_S's choice c = k + 8*deltabit, #3159): the C lowest (cost, c) choices of
 * each 32-value sub-block, their four entries and their error vectors
 * xhat - x over the 32 columns.  A zero scale makes every choice decode to
 * zero, so the order is c = 0, 1, ... with entries 0. */
static int iq1s_candidates_block(const float* x, const float* w, const float* grid, int n,
                                 int top_c, float* cand_err, int32_t* cand_choice,
                                 uint16_t* cand_codes)
{
    int st = check_block_inputs(x, w, 256);
    if (st) return st;
    uint16_t dh;
    st = block_scale(x, IQ1S_DIVISOR, NULL, &dh);
    if (st) return st;
    double d = orc_f16_to_f64(dh);
    for (int i = 0; i < 8; ++i) {
        double cost[16];
        int ent[16][4];
        for (int c = 0; c < 16; ++c) {
            int k = c & 7, dbit = c >> 3;
            double s = d * (double)(2 * k + 1);
            double delta = dbit ? -0.125 : 0.125;
            cost[c] = 0.0;
            for (int l = 0; l < 4; ++l) {
                int off = 32 * i + 8 * l;
                double ge;
                ent[c][l] = iq1s_best_entry(x + off, w ? w + off : NULL, grid, n, s, delta, &ge);
                cost[c] += ge;
            }
            if (dh == 0) {
                cost[c] = 0.0;
                for (int l = 0; l < 4; ++l) ent[c][l] = 0;
            }
        }
        int used[16] = {0};
        for (int r = 0; r < top_c; ++r) {
            int cb = -1;
            for (int c = 0; c < 16; ++c) {
                if (used[c]) continue;
                if (cb < 0 || cost[c] < cost[cb]) cb = c;
            }
            used[cb] = 1;
            cand_choice[i * top_c + r] = cb;
            double s = d * (double)(2 * (cb & 7) + 1);
            double delta = (cb >> 3) ? -0.125 : 0.125;
            for (int l = 0; l < 4; ++l) {
                const float* q = grid + 8 * ent[cb][l];
                if (cand_codes) cand_codes[(i * top_c + r) * 4 + l] = (uint16_t)ent[cb][l];
                for (int j = 0; j < 8; ++j) {
                    int col = 32 * i + 8 * l + j;
                    double xhat = s * ((double)q[j] + delta);
                    cand_err[(i * top_c + r) * 32 + 8 * l + j] = (float)(xhat - (double)x[col]);
                }
            }
        }
    }
    return ORC_OK;
}

/* ---------------------------------------------------------------------- */
/* Batched entry points (OpenMP over blocks).                              */
/* x: [nblk][256]; imp: NULL or [nblk][256]; scales: NULL or [nblk];       */
/* choices: NULL or [nblk][8] (IQ1_S) / [nblk][16] (IQ2_XS).               */
/* The return value is the first error code in block order, 0 if none.    */
/* ---------------------------------------------------------------------- */

static int first_error(const int* st, int64_t n)
{
    for (int64_t b = 0; b < n; ++b)
        if (st[b]) return st[b];
    return ORC_OK;
}

int orc_iq1s_encode(const float* x, const float* imp, int64_t nblk, const float* grid,
                    int32_t n, const uint16_t* scales, const int32_t* choices, uint8_t* out)
{
    if (n <= 0 || n > 2048) return ORC_ERR_ARG;
    int* st = (int*)calloc((size_t)(nblk > 0 ? nblk : 1), sizeof(int));
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < nblk; ++b)
        st[b] = iq1s_encode_block(x + 256 * b, imp ? imp + 256 * b : NULL, grid, n,
                                  scales ? scales + b : NULL, choices ? choices + 8 * b : NULL,
                                  out + 50 * b);
    int r = first_error(st, nblk);
    free(st);
    return r;
}

int orc_iq2xs_encode(const float* x, const float* imp, int64_t nblk, const float* grid,
                     int32_t n, const uint16_t* scales, const int32_t* choices, uint8_t* out)
{
    if (n <= 0 || n > 512) return ORC_ERR_ARG;
    int* st = (int*)calloc((size_t)(nblk > 0 ? nblk : 1), sizeof(int));
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < nblk; ++b)
        st[b] = iq2xs_encode_block(x + 256 * b, imp ? imp + 256 * b : NULL, grid, n,
                                   scales ? scales + b : NULL, choices ? choices + 16 * b : NULL,
                                   out + 74 * b);
    int r = first_error(st, nblk);
    free(st);
    return r;
}

int orc_iq1m_encode(const float* x, const float* imp, int64_t nblk, const float* grid,
                    int32_t n, const uint16_t* scales, const int32_t* choices, uint8_t* out)
{
    if (n <= 0 || n > 2048) return ORC_ERR_ARG;
    int* st = (int*)calloc((size_t)(nblk > 0 ? nblk : 1), sizeof(int));
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < nblk; ++b)
        st[b] = iq1m_encode_block(x + 256 * b, imp ? imp + 256 * b : NULL, grid, n,
                                  scales ? scales + b : NULL, choices ? choices + 16 * b : NULL,
                                  out + 56 * b);
    int r = first_error(st, nblk);
    free(st);
    return r;
}

int orc_iq1m_decode(const uint8_t* packed, int64_t nblk, const float* grid, int32_t n, double* out)
{
    int* st = (int*)calloc((size_t)(nblk > 0 ? nblk : 1), sizeof(int));
    #pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nblk; ++b)
        st[b] = iq1m_decode_block(packed + 56 * b, grid, n, out + 256 * b);
    int r = first_error(st, nblk);
    free(st);
    return r;
}

/* cand_err: [nblk][16][top_c][16] float; cand_choice: [nblk][16][top_c];
 * cand_codes: NULL or [nblk][16][top_c][2] (entry | shift << 11). */
int orc_iq1m_candidates(const float* x, const float* imp, int64_t nblk, const float* grid,
                        int32_t n, int32_t top_c, float* cand_err, int32_t* cand_choice,
                        uint16_t* cand_codes)
{
    if (n <= 0 || n > 2048 || top_c < 1 || top_c > 8) return ORC_ERR_ARG;
    int* st = (int*)calloc((size_t)(nblk > 0 ? nblk : 1), sizeof(int));
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < nblk; ++b)
        st[b] = iq1m_candidates_block(x + 256 * b, imp ? imp + 256 * b : NULL, grid, n, top_c,
                                      cand_err + (size_t)b * 16 * top_c * 16,
                                      cand_choice + (size_t)b * 16 * top_c,
                                      cand_codes ? cand_codes + (size_t)b * 16 * top_c * 2 : NULL);
    int r = first_error(st, nblk);
    free(st);
    return r;
}

/* fp16 bits of the predicted IQ1_M scale of each block (0 for amax = 0). */
void orc_iq1m_predict(const float* x, int64_t nblk, uint16_t* out)
{
    for (int64_t b = 0; b < nblk; ++b) {
        const float* xb = x + 256 * b;
        float amax = block_amax(xb, 256);
        out[b] = amax > 0.0f ? orc_predict_scale(amax, IQ1M_DIVISOR, orc_iq1m_anchor(xb, amax)) : 0;
    }
}

int orc_iq1s_decode(const uint8_t* packed, int64_t nblk, const float* grid, int32_t n, double* out)
{
    int* st = (int*)calloc((size_t)(nblk > 0 ? nblk : 1), sizeof(int));
    #pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nblk; ++b)
        st[b] = iq1s_decode_block(packed + 50 * b, grid, n, out + 256 * b);
    int r = first_error(st, nblk);
    free(st);
    return r;
}

int orc_iq2xs_decode(const uint8_t* packed, int64_t nblk, const float* grid, int32_t n, double* out)
{
    int* st = (int*)calloc((size_t)(nblk > 0 ? nblk : 1), sizeof(int));
    #pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nblk; ++b)
        st[b] = iq2xs_decode_block(packed + 74 * b, grid, n, out + 256 * b);
    int r = first_error(st, nblk);
    free(st);
    return r;
}

/* cand_err: [nblk][16][top_c][16] float; cand_choice: [nblk][16][top_c];
 * cand_codes: NULL or [nblk][16][top_c][2]. */
int orc_iq2xs_candidates(const float* x, const float* imp, int64_t nblk, const float* grid,
                         int32_t n, int32_t top_c, float* cand_err, int32_t* cand_choice,
                         uint16_t* cand_codes)
{
    if (n <= 0 || n > 512 || top_c < 1 || top_c > 16) return ORC_ERR_ARG;
    int* st = (int*)calloc((size_t)(nblk > 0 ? nblk : 1), sizeof(int));
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < nblk; ++b)
        st[b] = iq2xs_candidates_block(x + 256 * b, imp ? imp + 256 * b : NULL, grid, n, top_c,
                                       cand_err + (size_t)b * 16 * top_c * 16,
                                       cand_choice + (size_t)b * 16 * top_c,
                                       cand_codes ? cand_codes + (size_t)b * 16 * top_c * 2 : NULL);
    int r = first_error(st, nblk);
    free(st);
    return r;
}

/* cand_err: [nblk][8][top_c][32] float; cand_choice: [nblk][8][top_c];
 * cand_codes: NULL or [nblk][8][top_c][4] (the four grid entries). */
int orc_iq1s_candidates(const float* x, const float* imp, int64_t nblk, const float* grid,
                        int32_t n, int32_t top_c, float* cand_err, int32_t* cand_choice,
                        uint16_t* cand_codes)
{
    if (n <= 0 || n > 2048 || top_c < 1 || top_c > 16) return ORC_ERR_ARG;
    int* st = (int*)calloc((size_t)(nblk > 0 ? nblk : 1), sizeof(int));
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < nblk; ++b)
        st[b] = iq1s_candidates_block(x + 256 * b, imp ? imp + 256 * b : NULL, grid, n, top_c,
                                      cand_err + (size_t)b * 8 * top_c * 32,
                                      cand_choice + (size_t)b * 8 * top_c,
                                      cand_codes ? cand_codes + (size_t)b * 8 * top_c * 4 : NULL);
    int r = first_error(st, nblk);
    free(st);
    return r;
}

/* ---------------------------------------------------------------------- */
/* Local-Hessian choice search (#3158 steps 2-3; #3218), float64.          */
/* H: [256][256]; cand: [rows][G][C][L], L = 256/G.                        */
/* picks: [rows][G]; trace: NULL or [sweeps+1][rows][G].                   */
/* ---------------------------------------------------------------------- */

static double quad_form_block(const float* H, int g, int L, const float* a, const float* b)
{
    /* a^T H_gg b */
    double s = 0.0;
    for (int i = 0; i < L; ++i) {
        double t = 0.0;
        for (int j = 0; j < L; ++j)
            t += (double)H[(size_t)(g * L + i) * 256 + g * L + j] * (double)b[j];
        s += (double)a[i] * t;
    }
    return s;
}

static void choice_search_row(const float* H, const float* cand, int G, int C, int sweeps,
                              int32_t* picks, int32_t* trace, int64_t rows, int64_t row)
{
    int L = 256 / G;
    double* Q = (double*)malloc(sizeof(double) * G * C);
    double* r = (double*)malloc(sizeof(double) * 256);
    double* e = (double*)malloc(sizeof(double) * 256);
    double* rest = (double*)malloc(sizeof(double) * L);
    double* score = (double*)malloc(sizeof(double) * C);
    int* p = (int*)malloc(sizeof(int) * G);
#define CAND(g, c) (cand + ((size_t)(g) * C + (c)) * L)
    /* Step 2: each group's best choice under its own diagonal block. */
    for (int g = 0; g < G; ++g) {
        int best = 0;
        for (int c = 0; c < C; ++c) {
            Q[g * C + c] = quad_form_block(H, g, L, CAND(g, c), CAND(g, c));
            if (Q[g * C + c] < Q[g * C + best]) best = c;
        }
        p[g] = best;
        for (int i = 0; i < L; ++i) e[g * L + i] = (double)CAND(g, best)[i];
    }
    if (trace)
        for (int g = 0; g < G; ++g) trace[(size_t)row * G + g] = p[g];
    /* r = H e */
    for (int i = 0; i < 256; ++i) {
        double t = 0.0;
        for (int j = 0; j < 256; ++j) t += (double)H[(size_t)i * 256 + j] * e[j];
        r[i] = t;
    }
    /* Step 3: sweeps in ascending group order, strict improvement only. */
    for (int sw = 0; sw < sweeps; ++sw) {
        for (int g = 0; g < G; ++g) {
            for (int i = 0; i < L; ++i) {
                double t = 0.0;
                for (int j = 0; j < L; ++j)
                    t += (double)H[(size_t)(g * L + i) * 256 + g * L + j] * e[g * L + j];
                rest[i] = r[g * L + i] - t;
            }
            int best = 0;
            for (int c = 0; c < C; ++c) {
                double dot = 0.0;
                for (int i = 0; i < L; ++i) dot += (double)CAND(g, c)[i] * rest[i];
                score[c] = Q[g * C + c] + 2.0 * dot;
                if (score[c] < score[best]) best = c;
            }
            if (score[best] < score[p[g]]) {
                for (int i = 0; i < L; ++i) {
                    double de = (double)CAND(g, best)[i] - e[g * L + i];
                    if (de == 0.0) continue;
                    for (int u = 0; u < 256; ++u)
                        r[u] += (double)H[(size_t)u * 256 + g * L + i] * de;
                    e[g * L + i] = (double)CAND(g, best)[i];
                }
                p[g] = best;
            }
        }
        if (trace)
            for (int g = 0; g < G; ++g)
                trace[((size_t)(sw + 1) * rows + row) * G + g] = p[g];
    }
#undef CAND
    for (int g = 0; g < G; ++g) picks[(size_t)row * G + g] = p[g];
    free(Q); free(r); free(e); free(rest); free(score); free(p);
}

int orc_choice_search(const float* H, const float* cand, int64_t rows, int32_t G, int32_t C,
                      int32_t sweeps, int32_t* picks, int32_t* trace)
{
    if ((G != 8 && G != 16) || C < 1 || C > 16 || sweeps < 0) return ORC_ERR_ARG;
    int L = 256 / G;
    #pragma omp parallel for schedule(dynamic, 4)
    for (int64_t row = 0; row < rows; ++row)
        choice_search_row(H, cand + (size_t)row * G * C * L, G, C, sweeps, picks, trace, rows, row);
    return ORC_OK;
}

/* J = e^T H e of a row for given picks (float64). */
double orc_choice_objective(const float* H, const float* cand_row, int32_t G, int32_t C,
                            const int32_t* picks_row)
{
    int L = 256 / G;
    double e[256];
    for (int g = 0; g < G; ++g)
        for (int i = 0; i < L; ++i)
            e[g * L + i] = (double)cand_row[((size_t)g * C + picks_row[g]) * L + i];
    double J = 0.0;
    for (int i = 0; i < 256; ++i) {
        double t = 0.0;
        for (int j = 0; j < 256; ++j) t += (double)H[(size_t)i * 256 + j] * e[j];
        J += e[i] * t;
    }
    return J;
}

/* Replay check of another implementation's decision trace on one row.
 * trace_row: [(sweeps+1)][G] picks after step 2 and after each sweep.
 * Every decision must be optimal within tol * J (J of the row's state at that
 * point, float64): step 2 picks within tol of each group's minimum; at each
 * sweep visit, a switch must not raise the row's J and must reach the minimum
 * within tol, and a keep must leave no choice better by more than tol.
 * Returns 0 if every decision passes, else 1 + the index of the first failing
 * decision (stage*G + g); *worst receives the largest violation / J seen. */
int orc_choice_replay(const float* H, const float* cand_row, int32_t G, int32_t C,
                      int32_t sweeps, const int32_t* trace_row, double tol, double* worst)
{
    if ((G != 8 && G != 16) || C < 1 || C > 16) { *worst = INFINITY; return -1; }
    int L = 256 / G;
    double e[256], r[256], rest[32], score[16];   /* L is 16 or 32 */
    int p[16];
    double wv = 0.0;
    int fail = 0;
#define CANDR(g, c) (cand_row + ((size_t)(g) * C + (c)) * L)
    for (int g = 0; g < G; ++g) {
        p[g] = trace_row[g];
        if (p[g] < 0 || p[g] >= C) { *worst = INFINITY; return 1 + g; }
        for (int i = 0; i < L; ++i) e[g * L + i] = (double)CANDR(g, p[g])[i];
    }
    double J = orc_choice_objective(H, cand_row, G, C, p);
    double scale = fabs(J) > 0 ? fabs(J) : 1.0;
    for (int g = 0; g < G; ++g) {
        double qmin = INFINITY;
        for (int c = 0; c < C; ++c) {
            double q = quad_form_block(H, g, L, CANDR(g, c), CANDR(g, c));
            if (q < qmin) qmin = q;
        }
        double qp = quad_form_block(H, g, L, CANDR(g, p[g]), CANDR(g, p[g]));
        double v = (qp - qmin) / scale;
        if (v > wv) wv = v;
        if (v > tol && !fail) fail = 1 + g;
    }
    for (int i = 0; i < 256; ++i) {
        double t = 0.0;
        for (int j = 0; j < 256; ++j) t += (double)H[(size_t)i * 256 + j] * e[j];
        r[i] = t;
    }
    for (int sw = 0; sw < sweeps; ++sw) {
        const int32_t* next = trace_row + (size_t)(sw + 1) * G;
        for (int g = 0; g < G; ++g) {
            J = 0.0;
            for (int i = 0; i < 256; ++i) J += e[i] * r[i];
            scale = fabs(J) > 0 ? fabs(J) : 1.0;
            for (int i = 0; i < L; ++i) {
                double t = 0.0;
                for (int j = 0; j < L; ++j)
                    t += (double)H[(size_t)(g * L + i) * 256 + g * L + j] * e[g * L + j];
                rest[i] = r[g * L + i] - t;
            }
            double smin = INFINITY;
            for (int c = 0; c < C; ++c) {
                double dot = 0.0;
                for (int i = 0; i < L; ++i) dot += (double)CANDR(g, c)[i] * rest[i];
                score[c] = quad_form_block(H, g, L, CANDR(g, c), CANDR(g, c)) + 2.0 * dot;
                if (score[c] < smin) smin = score[c];
            }
            int d = next[g];
            if (d < 0 || d >= C) { *worst = INFINITY; return 1 + (sw + 1) * G + g; }
            double v;
            if (d != p[g]) {
                double up = (score[d] - score[p[g]]) / scale;   /* must be <= 0 */
                double gap = (score[d] - smin) / scale;
                v = up > gap ? up : gap;
            } else {
                v = (score[p[g]] - smin) / scale;
            }
            if (v > wv) wv = v;
            if (v > tol && !fail) fail = 1 + (sw + 1) * G + g;
            if (d != p[g]) {
                for (int i = 0; i < L; ++i) {
                    double de = (double)CANDR(g, d)[i] - e[g * L + i];
                    if (de == 0.0) continue;
                    for (int u = 0; u < 256; ++u)
                        r[u] += (double)H[(size_t)u * 256 + g * L + i] * de;
                    e[g * L + i] = (double)CANDR(g, d)[i];
                }
                p[g] = d;
            }
        }
    }
#undef CANDR
    *worst = wv;
    return fail;
}

/* Threads an OpenMP parallel region of this library uses. */
int orc_num_threads(void)
{
    return omp_get_max_threads();
}
