/*
 * focus_oracle.c -- scalar CPU oracle for the FOCUS NVFP4 quantizer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this file's library.  The
 * product path (the HIP library and its Python binding) never calls it, and
 * it shares no code, header, table or constant generator with the HIP path.
 *
 * What it computes, and where that is defined:
 *   "FOCUS NVFP4 scales for Llama-3.2-1B-Instruct (our reproduction)",
 *   section "What this is":
 *     - field table, row s2: the tensor scale is the largest magnitude of
 *       the weight divided by 6*448;
 *     - field table, rows m and q: one block factor m per 16 consecutive
 *       elements along in_features, two logits q per block (one per
 *       8-element sub-block), all FP32, row-major over [out, in];
 *     - equation S_b: block scale = E4M3 of the block maximum times m_b
 *       over (6*s2), clamped to [2^-6, 448];
 *     - equation c_i: element code = E2M1 of w_i over
 *       (S_b * sigmoid(q_k) * s2), clamped to [-6, 6];
 *     - equation w'_i: dequantized weight = c_i * S_b * s2;
 *     - the paragraph after the equations: E2M1 rounds to the nearest
 *       value with ties to even, and a block whose scaled maximum is zero
 *       takes scale 1 before the clamp.
 *   The same page, same section, says activations carry one scale per
 *   token; the per-token path below is that scale with m = 1 and no
 *   relaxation (sigmoid = 1).
 *
 * Precision.  The page stores m, q and s2 in FP32, so every operation of the
 * formulas is one IEEE binary32 operation with round-to-nearest-even, in the
 * order the formulas are printed (left to right, the parenthesised
 * denominator as one product).  Build with -ffp-contract=off, no fast-math.
 * The only function evaluated beyond binary32 operations is exp: expf is
 * taken as the correctly rounded binary32 exponential, computed here as the
 * x87 extended-precision expl rounded once to binary32.
 *
 * Format definitions (OCP Microscaling formats, used by NVFP4):
 *   E2M1: sign + 2 exponent bits (bias 1) + 1 mantissa bit; magnitudes
 *         0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes 0..7.
 *   E4M3 (E4M3FN): sign + 4 exponent bits (bias 7) + 3 mantissa bits, no
 *         infinities, 0x7F/0xFF are NaN, largest finite 448 (0x7E).
 *   BF16: the top 16 bits of an IEEE binary32.
 * Rounding to each format is written out from its definition: pick the
 * nearest representable value, ties to the code whose last mantissa bit is
 * 0.  This is slow and meant to be obviously right, not fast.
 *
 * Later sections, each citing its own source: FourOverSix (block scale for
 * maximum 6 or 4), FOCUS on MXFP4 (32-blocks, E8M0 scale), FlipQuant MixFP4
 * (per-tile E0M3 / E2M1), and the NVFP4 linear layer that consumes the
 * stored format (Y = X' W'^T in binary64).
 *
 * Readings where the pages are silent (each one is tested):
 *   - the sign of a zero code follows the sign of the quotient, so a
 *     negative element that rounds to zero is stored as code 0x8;
 *   - two codes per byte, element 2j in the low nibble;
 *   - sub-block k of block b uses q[r, 2b+k], k = 0 for elements 0..7;
 *   - "scaled maximum is 0" is tested on the computed quotient t;
 *   - s2 == 0 (all-zero tensor or token): every block takes scale 1 and
 *     every code is a signed zero.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stddef.h>

#define ORACLE_ABI 1

int oracle_abi_version(void) { return ORACLE_ABI; }

/* ---------- binary32 <-> bits, BF16 decode ------------------------------ */

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* BF16 is the upper half of a binary32: decoding is exact. */
float oracle_bf16_value(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/* ---------- E2M1 ------------------------------------------------------- */

static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

float oracle_e2m1_value(unsigned code)
{
    double v = E2M1_MAG[code & 7u];
    return (float)((code & 8u) ? -v : v);
}

/* Nearest E2M1 value to x, ties to the even code (mantissa bit 0).  The
 * sign bit of the code is the sign bit of x, zero included.  |x| - v is
 * exact in double for any binary32 x with |x| <= 6, so the comparison is
 * exact; larger |x| all map to 6, the nearest value. */
unsigned oracle_e2m1_round(float x)
{
    unsigned sign = (bits_from_f32(x) >> 31) & 1u;
    double a = fabs((double)x);
    /* the clamp to [-6, 6] of equation c_i: beyond 6 the nearest value is
     * 6, and for huge magnitudes the binary64 distances below could no
     * longer tell 4 from 6 */
    if (a > 6.0) a = 6.0;
    unsigned best = 0;
    double best_d = INFINITY;
    for (unsigned k = 0; k < 8; ++k) {
        double d = fabs(a - E2M1_MAG[k]);
        if (d < best_d || (d == best_d && (k & 1u) == 0u)) {
            best_d = d;
            best = k;
        }
    }
    return (sign << 3) | best;
}

/* ---------- E4M3 (E4M3FN) ---------------------------------------------- */

/* Decode from the field definition: exponent field 0 is subnormal
 * (m/8 * 2^-6), otherwise (1 + m/8) * 2^(e-7).  0x7F / 0xFF are NaN. */
float oracle_e4m3_value(unsigned byte)
{
    unsigned s = (byte >> 7) & 1u, e = (byte >> 3) & 15u, m = byte & 7u;
    double v;
    if (e == 15u && m == 7u) return NAN;
    if (e == 0u) v = ldexp((double)m / 8.0, -6);
    else v = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return (float)(s ? -v : v);
}

/* Nearest non-negative finite E4M3 value to t >= 0, ties to the even
 * byte (mantissa LSB 0), by search over all 127 finite codes 0x00..0x7E.
 * The quantizer only calls this with t in [2^-6, 448]. */
unsigned oracle_e4m3_round(float t)
{
    unsigned best = 0;
    double best_d = INFINITY;
    for (unsigned b = 0; b <= 0x7Eu; ++b) {
        double d = fabs((double)t - (double)oracle_e4m3_value(b));
        if (d < best_d || (d == best_d && (b & 1u) == 0u)) {
            best_d = d;
            best = b;
        }
    }
    return best;
}

/* ---------- BF16 rounding ---------------------------------------------- */

/* Nearest BF16 to x, ties to even.  Candidates are x truncated to 16 bits
 * (toward zero) and the next BF16 away from zero; the infinity pattern
 * counts as 2^128 so that IEEE overflow rounding falls out.  NaN maps to
 * the canonical quiet NaN. */
uint16_t oracle_bf16_round(float x)
{
    uint32_t u = bits_from_f32(x);
    if (isnan(x)) return (uint16_t)(((u >> 16) & 0x8000u) | 0x7FC0u);
    if (isinf(x)) return (uint16_t)(u >> 16);
    uint16_t lo = (uint16_t)(u >> 16);
    uint16_t hi = (uint16_t)(lo + 1u);
    double ax = fabs((double)x);
    double vlo = fabs((double)oracle_bf16_value(lo));
    double vhi = ((hi & 0x7FFFu) == 0x7F80u) ? ldexp(1.0, 128)
                                             : fabs((double)oracle_bf16_value(hi));
    double dlo = ax - vlo, dhi = vhi - ax;
    if (dlo < dhi) return lo;
    if (dhi < dlo) return hi;
    return (lo & 1u) ? hi : lo;
}

/* ---------- sigmoid ---------------------------------------------------- */

/* sigmoid(q) = 1 / (1 + expf(-q)), three binary32 roundings: expf, the
 * sum, the quotient.  expf is correctly rounded (see the header). */
float oracle_expf(float x) { return (float)expl((long double)x); }

float oracle_sigmoid(float q)
{
    float e = oracle_expf(-q);
    float s = 1.0f + e;
    return 1.0f / s;
}

/* ---------- tensor scale ----------------------------------------------- */

/* s2 = amax(|W|) / (6 * 448).  6*448 = 2688 is exact in binary32.  The
 * maximum of an empty tensor is taken as 0. */
float oracle_tensor_scale(const uint16_t* w, int64_t n, float* amax_out)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(oracle_bf16_value(w[i]));
        if (a > amax) amax = a;
    }
    if (amax_out) *amax_out = amax;
    return amax / 2688.0f;
}

/* ---------- one block -------------------------------------------------- */

/* Block scale byte for block maximum a, factor mb, tensor scale s2:
 * t = (a * mb) / (6 * s2); t == 0 -> 1; clamp to [2^-6, 448]; E4M3. */
unsigned oracle_block_scale(float a, float mb, float s2)
{
    float t;
    if (s2 == 0.0f) {
        t = 1.0f;
    } else {
        float num = a * mb;
        float den = 6.0f * s2;
        t = num / den;
        if (t == 0.0f) t = 1.0f;
    }
    t = fminf(fmaxf(t, 0x1p-6f), 448.0f);
    return oracle_e4m3_round(t);
}

/* Code of one element: x = w / ((S * sig) * s2), clamp [-6, 6], E2M1. */
unsigned oracle_element_code(uint16_t w, float S, float sig, float s2)
{
    float wf = oracle_bf16_value(w);
    if (s2 == 0.0f) return ((uint32_t)w >> 15) << 3;
    float d = (S * sig) * s2;
    float x = wf / d;
    x = fminf(fmaxf(x, -6.0f), 6.0f);
    return oracle_e2m1_round(x);
}

/* w' = (c * S) * s2, rounded to BF16. */
uint16_t oracle_dequant_value(unsigned code, float S, float s2)
{
    float c = oracle_e2m1_value(code);
    float v = (c * S) * s2;
    return oracle_bf16_round(v);
}

/* Codes of n elements of one sub-block under a given sigmoid value; used
 * by the tests to check whether a code difference is explained by a
 * different rounding of sigmoid. */
void oracle_subblock_codes(const uint16_t* w, int n, float S, float sig, float s2,
                           uint8_t* codes_out)
{
    for (int i = 0; i < n; ++i) codes_out[i] = (uint8_t)oracle_element_code(w[i], S, sig, s2);
}

/* ---------- the quantizer ---------------------------------------------- */

/* W [rows, cols] BF16 row-major (cols % 16 == 0); m [rows, cols/16] or NULL
 * (m = 1); q [rows, cols/8] or NULL (sigmoid = 1); s2 per tensor.
 * Outputs: codes [rows, cols/2] (element 2j low nibble), scales
 * [rows, cols/16] E4M3 bytes, wdeq [rows, cols] BF16 or NULL. */
void oracle_quantize(const uint16_t* w, int64_t rows, int64_t cols,
                     const float* m, const float* q, float s2,
                     uint8_t* codes, uint8_t* scales, uint16_t* wdeq)
{
    int64_t nb = cols / 16;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const uint16_t* wb = w + r * cols + b * 16;
            float a = 0.0f;
            for (int i = 0; i < 16; ++i) {
                float v = fabsf(oracle_bf16_value(wb[i]));
                if (v > a) a = v;
            }
            float mb = m ? m[r * nb + b] : 1.0f;
            unsigned sb = oracle_block_scale(a, mb, s2);
            float S = oracle_e4m3_value(sb);
            scales[r * nb + b] = (uint8_t)sb;
            unsigned c[16];
            for (int k = 0; k < 2; ++k) {
                float sig = q ? oracle_sigmoid(q[r * (2 * nb) + 2 * b + k]) : 1.0f;
                for (int i = 0; i < 8; ++i)
                    c[8 * k + i] = oracle_element_code(wb[8 * k + i], S, sig, s2);
            }
            for (int j = 0; j < 8; ++j)
                codes[r * (cols / 2) + b * 8 + j] = (uint8_t)(c[2 * j] | (c[2 * j + 1] << 4));
            if (wdeq)
                for (int i = 0; i < 16; ++i)
                    wdeq[r * cols + b * 16 + i] = oracle_dequant_value(c[i], S, s2);
        }
    }
}

/* Dequantize stored codes and scale bytes: s2_per_row = 0 uses s2[0] for
 * every row, 1 uses s2[r]. */
void oracle_dequantize(const uint8_t* codes, const uint8_t* scales, const float* s2,
                       int s2_per_row, int64_t rows, int64_t cols, uint16_t* out)
{
    int64_t nb = cols / 16;
    for (int64_t r = 0; r < rows; ++r) {
        float s = s2_per_row ? s2[r] : s2[0];
        for (int64_t i = 0; i < cols; ++i) {
            uint8_t byte = codes[r * (cols / 2) + i / 2];
            unsigned code = (i & 1) ? (byte >> 4) : (byte & 15u);
            float S = oracle_e4m3_value(scales[r * nb + i / 16]);
            out[r * cols + i] = oracle_dequant_value(code, S, s);
        }
    }
}

/* Per-token activations: each row t gets s2_t = amax|x_t| / 2688 and is
 * quantized with m = 1 and sigmoid = 1. */
void oracle_quantize_act_per_token(const uint16_t* x, int64_t tokens, int64_t hidden,
                                   uint8_t* codes, uint8_t* scales, float* s2_out,
                                   uint16_t* xdeq)
{
    for (int64_t t = 0; t < tokens; ++t) {
        float s2 = oracle_tensor_scale(x + t * hidden, hidden, NULL);
        s2_out[t] = s2;
        oracle_quantize(x + t * hidden, 1, hidden, NULL, NULL, s2,
                        codes + t * (hidden / 2), scales + t * (hidden / 16),
                        xdeq ? xdeq + t * hidden : NULL);
    }
}

/* ---------- array forms of the rounding helpers (for the tests) -------- */

void oracle_e2m1_round_n(const float* x, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)oracle_e2m1_round(x[i]);
}

void oracle_e4m3_round_n(const float* t, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)oracle_e4m3_round(t[i]);
}

void oracle_bf16_round_n(const float* x, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_round(x[i]);
}

void oracle_sigmoid_n(const float* q, int64_t n, float* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_sigmoid(q[i]);
}

void oracle_expf_n(const float* x, int64_t n, float* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_expf(x[i]);
}

/* ---------- FourOverSix (RTN weights, per-token activations) ----------- */

/* FourOverSix, as the FOCUS page describes its evaluation activations
 * ("FOCUS NVFP4 scales for Llama-3.2-1B-Instruct (our reproduction)",
 * section "Calibration", the differences from the paper) and its
 * FourOverSix baseline rows (section "Perplexity"): plain NVFP4 (m = 1, no
 * relaxation) in which each 16-element block's scale maps the block maximum
 * either to 6 or to 4, whichever quantizes the block with the lower error.
 * Readings where the page is silent:
 *   - candidate k in {6, 4}: t_k = a / (k * s2) (one binary32 division of
 *     the block maximum by the rounded product k*s2), zero -> 1, clamp to
 *     [2^-6, 448], E4M3; codes E2M1(clamp(w / (S_k * s2), -6, 6));
 *   - error of a candidate: sum over the 16 elements, in element order, of
 *     e*e with e = w - (c*S_k)*s2, every operation binary32;
 *   - the 4-candidate is taken only when its error is strictly lower
 *     (ties keep 6); s2 = amax / (6*448) as for NVFP4;
 *   - s2 == 0: every block is a zero block (scale byte 0x38, signed zeros). */

static void fo6_candidate(const uint16_t* wb, float a, float k, float s2,
                          unsigned* sb_out, unsigned c[16], float* err_out)
{
    float t = a / (k * s2);
    if (t == 0.0f) t = 1.0f;
    t = fminf(fmaxf(t, 0x1p-6f), 448.0f);
    unsigned sb = oracle_e4m3_round(t);
    float S = oracle_e4m3_value(sb);
    float err = 0.0f;
    for (int i = 0; i < 16; ++i) {
        c[i] = oracle_element_code(wb[i], S, 1.0f, s2);
        float v = (oracle_e2m1_value(c[i]) * S) * s2;
        float e = oracle_bf16_value(wb[i]) - v;
        err = err + e * e;
    }
    *sb_out = sb;
    *err_out = err;
}

/* One block: returns the scale byte, fills the 16 codes. */
unsigned oracle_fo6_block(const uint16_t* wb, float s2, uint8_t* codes16)
{
    unsigned c6[16], c4[16], sb6, sb4;
    float e6, e4;
    if (s2 == 0.0f) {
        for (int i = 0; i < 16; ++i) codes16[i] = (uint8_t)(((uint32_t)wb[i] >> 15) << 3);
        return 0x38;
    }
    float a = 0.0f;
    for (int i = 0; i < 16; ++i) {
        float v = fabsf(oracle_bf16_value(wb[i]));
        if (v > a) a = v;
    }
    fo6_candidate(wb, a, 6.0f, s2, &sb6, c6, &e6);
    fo6_candidate(wb, a, 4.0f, s2, &sb4, c4, &e4);
    const int four = e4 < e6;
    for (int i = 0; i < 16; ++i) codes16[i] = (uint8_t)(four ? c4[i] : c6[i]);
    return four ? sb4 : sb6;
}

/* W [rows, cols] with one s2 for the tensor (weights) or, when s2_per_row,
 * s2[r] for row r (activations).  Outputs as oracle_quantize. */
void oracle_fo6_quantize(const uint16_t* w, int64_t rows, int64_t cols, const float* s2,
                         int s2_per_row, uint8_t* codes, uint8_t* scales, uint16_t* wdeq)
{
    int64_t nb = cols / 16;
    for (int64_t r = 0; r < rows; ++r) {
        float s = s2_per_row ? s2[r] : s2[0];
        for (int64_t b = 0; b < nb; ++b) {
            const uint16_t* wb = w + r * cols + b * 16;
            uint8_t c[16];
            unsigned sb = oracle_fo6_block(wb, s, c);
            float S = oracle_e4m3_value(sb);
            scales[r * nb + b] = (uint8_t)sb;
            for (int j = 0; j < 8; ++j)
                codes[r * (cols / 2) + b * 8 + j] = (uint8_t)(c[2 * j] | (c[2 * j + 1] << 4));
            if (wdeq)
                for (int i = 0; i < 16; ++i)
                    wdeq[r * cols + b * 16 + i] = oracle_dequant_value(c[i], S, s);
        }
    }
}

/* Per-token FourOverSix activations: s2_t = amax|x_t| / 2688 per row. */
void oracle_fo6_quantize_act_per_token(const uint16_t* x, int64_t tokens, int64_t hidden,
                                       uint8_t* codes, uint8_t* scales, float* s2_out,
                                       uint16_t* xdeq)
{
    for (int64_t t = 0; t < tokens; ++t)
        s2_out[t] = oracle_tensor_scale(x + t * hidden, hidden, NULL);
    oracle_fo6_quantize(x, tokens, hidden, s2_out, 1, codes, scales, xdeq);
}

/* ---------- FOCUS on MXFP4 ---------------------------------------------- */

/* The technical summary of the FOCUS paper ("Technische Samenvatting:
 * FOCUS ...", section "Methodologie", Coupled-Relaxation and Dual-Granularity
 * Scaling) applies the method to MXFP4 as well: 32-element hardware blocks
 * with a power-of-two (E8M0) dequantization scale, each block split into
 * sub-blocks of 8 that are quantized with their own relaxation coefficient,
 * the stored scale shared by the whole block.  Readings where the pages are
 * silent (the same shape as the NVFP4 formulas of the FOCUS page):
 *   - block scale: the OCP Microscaling conversion applied to the scaled
 *     block maximum t = max|w_b| * m_b (binary32 product): S_b =
 *     2^(floor(log2 t) - 2) (2 = the exponent of E2M1's largest value 6),
 *     exponent clamped to [-127, 127] (the E8M0 range); t == 0 -> scale 1;
 *     byte = exponent + 127;
 *   - no tensor scale;
 *   - sub-block k (0..3, elements 8k..8k+7) of block b of row r uses
 *     q[r, 4b+k]; m is [rows, cols/32];
 *   - c_i = E2M1(clamp(w_i / (S_b * sigmoid(q_k)), -6, 6)); w' = BF16(c*S_b). */

/* E8M0 value of a byte (0xFF is NaN). */
float oracle_e8m0_value(unsigned byte)
{
    if ((byte & 0xFFu) == 0xFFu) return NAN;
    return ldexpf(1.0f, (int)(byte & 0xFFu) - 127);
}

unsigned oracle_mx_block_scale(float a, float mb)
{
    float t = a * mb;
    if (t == 0.0f) return 127u;
    int e2;
    (void)frexpf(t, &e2);          /* t = f * 2^e2, f in [0.5, 1) */
    int e = (e2 - 1) - 2;          /* floor(log2 t) - emax(E2M1) */
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return (unsigned)(e + 127);
}

/* W [rows, cols] (cols % 32 == 0); m [rows, cols/32] or NULL; q [rows,
 * cols/8] or NULL.  codes [rows, cols/2] (element 2j low nibble), scales
 * [rows, cols/32] E8M0 bytes, wdeq [rows, cols] BF16 or NULL. */
void oracle_mx_quantize(const uint16_t* w, int64_t rows, int64_t cols, const float* m,
                        const float* q, uint8_t* codes, uint8_t* scales, uint16_t* wdeq)
{
    int64_t nb = cols / 32;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const uint16_t* wb = w + r * cols + b * 32;
            float a = 0.0f;
            for (int i = 0; i < 32; ++i) {
                float v = fabsf(oracle_bf16_value(wb[i]));
                if (v > a) a = v;
            }
            float mb = m ? m[r * nb + b] : 1.0f;
            unsigned sb = oracle_mx_block_scale(a, mb);
            float S = oracle_e8m0_value(sb);
            scales[r * nb + b] = (uint8_t)sb;
            unsigned c[32];
            for (int k = 0; k < 4; ++k) {
                float sig = q ? oracle_sigmoid(q[r * (4 * nb) + 4 * b + k]) : 1.0f;
                for (int i = 0; i < 8; ++i)
                    c[8 * k + i] = oracle_element_code(wb[8 * k + i], S, sig, 1.0f);
            }
            for (int j = 0; j < 16; ++j)
                codes[r * (cols / 2) + b * 16 + j] = (uint8_t)(c[2 * j] | (c[2 * j + 1] << 4));
            if (wdeq)
                for (int i = 0; i < 32; ++i)
                    wdeq[r * cols + b * 32 + i] = oracle_dequant_value(c[i], S, 1.0f);
        }
    }
}

void oracle_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                          uint16_t* out)
{
    int64_t nb = cols / 32;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t i = 0; i < cols; ++i) {
            uint8_t byte = codes[r * (cols / 2) + i / 2];
            unsigned code = (i & 1) ? (byte >> 4) : (byte & 15u);
            float S = oracle_e8m0_value(scales[r * nb + i / 32]);
            out[r * cols + i] = oracle_dequant_value(code, S, 1.0f);
        }
}

/* ---------- FlipQuant MixFP4 tile maps ---------------------------------- */

/* "Llama-3.1-8B-Instruct FlipQuant MixFP4 maps", section "What this is": a
 * map holds one bit per weight tile (8x64, 16x64 or 256x64, rows x input
 * columns); a set bit stores the tile's 4-bit elements as E0M3 (uniform
 * levels 0..7), a clear bit as E2M1 with FourOverSix; everything else is
 * NVFP4 (16-element blocks, E4M3 block scale, FP32 tensor scale).  Readings
 * where the page is silent:
 *   - an E0M3 block's scale maps the block maximum to 7: t = a / (7*s2),
 *     zero -> 1, clamp [2^-6, 448], E4M3;
 *   - E0M3 code = sign bit (bit 3) | nearest integer 0..7 to |x| (ties to
 *     the even integer), x = clamp(w / (S*s2), -7, 7);
 *   - w' = BF16((c*S)*s2) with c the signed integer level;
 *   - the map is row-major [rows/tile_rows, cols/tile_cols], one byte per
 *     tile (nonzero = E0M3). */

unsigned oracle_e0m3_round(float x)
{
    unsigned sign = (bits_from_f32(x) >> 31) & 1u;
    double a = fabs((double)x);
    unsigned best = 0;
    double best_d = INFINITY;
    for (unsigned k = 0; k < 8; ++k) {
        double d = fabs(a - (double)k);
        if (d < best_d || (d == best_d && (k & 1u) == 0u)) {
            best_d = d;
            best = k;
        }
    }
    return (sign << 3) | best;
}

float oracle_e0m3_value(unsigned code)
{
    float v = (float)(code & 7u);
    return (code & 8u) ? -v : v;
}

/* One E0M3 block: scale byte, 16 codes. */
unsigned oracle_e0m3_block(const uint16_t* wb, float s2, uint8_t* codes16)
{
    if (s2 == 0.0f) {
        for (int i = 0; i < 16; ++i) codes16[i] = (uint8_t)(((uint32_t)wb[i] >> 15) << 3);
        return 0x38;
    }
    float a = 0.0f;
    for (int i = 0; i < 16; ++i) {
        float v = fabsf(oracle_bf16_value(wb[i]));
        if (v > a) a = v;
    }
    float t = a / (7.0f * s2);
    if (t == 0.0f) t = 1.0f;
    t = fminf(fmaxf(t, 0x1p-6f), 448.0f);
    unsigned sb = oracle_e4m3_round(t);
    float S = oracle_e4m3_value(sb);
    float d = S * s2;
    for (int i = 0; i < 16; ++i) {
        float x = oracle_bf16_value(wb[i]) / d;
        x = fminf(fmaxf(x, -7.0f), 7.0f);
        codes16[i] = (uint8_t)oracle_e0m3_round(x);
    }
    return sb;
}

void oracle_mixfp4_quantize(const uint16_t* w, int64_t rows, int64_t cols, float s2,
                            const uint8_t* map, int64_t tile_rows, int64_t tile_cols,
                            uint8_t* codes, uint8_t* scales, uint16_t* wdeq)
{
    int64_t nb = cols / 16, tiles_per_row = cols / tile_cols;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const uint16_t* wb = w + r * cols + b * 16;
            int e0m3 = map[(r / tile_rows) * tiles_per_row + (b * 16) / tile_cols] != 0;
            uint8_t c[16];
            unsigned sb = e0m3 ? oracle_e0m3_block(wb, s2, c) : oracle_fo6_block(wb, s2, c);
            float S = oracle_e4m3_value(sb);
            scales[r * nb + b] = (uint8_t)sb;
            for (int j = 0; j < 8; ++j)
                codes[r * (cols / 2) + b * 8 + j] = (uint8_t)(c[2 * j] | (c[2 * j + 1] << 4));
            if (wdeq)
                for (int i = 0; i < 16; ++i) {
                    float cv = e0m3 ? oracle_e0m3_value(c[i]) : oracle_e2m1_value(c[i]);
                    wdeq[r * cols + b * 16 + i] = oracle_bf16_round((cv * S) * s2);
                }
        }
    }
}

/* ---------- the NVFP4 linear layer (consumer of the stored format) ------ */

/* "FOCUS NVFP4 scales for Llama-3.2-1B-Instruct (our reproduction)": section
 * "What this is" (the deployed model is plain NVFP4 and runs on standard
 * NVFP4 kernels) and section "Perplexity" (weights in NVFP4 with one FP32
 * scale per tensor, activations in NVFP4 with one scale per token).  The
 * layer computes Y = X' W'^T with the dequantized operands taken as real
 * numbers: X'[t,k] = c*S*s2x[t], W'[o,k] = c*S*s2w (no BF16 rounding of the
 * operands).  Written out: for every (t, o) the sum over k, in k order, of
 * the products (c_x*S_x)*(c_w*S_w) -- each exact in binary64 (at most
 * 10 significant bits) -- accumulated in binary64, then multiplied by
 * s2x[t] and s2w.  yabs receives the same sum of |products| times
 * |s2x[t]*s2w|, the scale of any rounding error in another summation order.
 * Layouts: codes [rows, K/2] (element 2j in the low nibble), scale bytes
 * [rows, K/16], Y [M, N] row-major; xs2 has M entries when xs2_per_row, else 1. */
static double nvfp4_element(const uint8_t* codes, const uint8_t* scales, int64_t row, int64_t K,
                            int64_t k)
{
    uint8_t byte = codes[row * (K / 2) + k / 2];
    unsigned c = (k & 1) ? (byte >> 4) : (byte & 15u);
    return (double)oracle_e2m1_value(c) * (double)oracle_e4m3_value(scales[row * (K / 16) + k / 16]);
}

void oracle_nvfp4_linear(const uint8_t* xc, const uint8_t* xs, const float* xs2, int xs2_per_row,
                         int64_t M, const uint8_t* wc, const uint8_t* ws, const float* ws2,
                         int64_t N, int64_t K, double* y, double* yabs)
{
    for (int64_t t = 0; t < M; ++t) {
        double sx = (double)xs2[xs2_per_row ? t : 0];
        for (int64_t o = 0; o < N; ++o) {
            double acc = 0.0, aabs = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = nvfp4_element(xc, xs, t, K, k) * nvfp4_element(wc, ws, o, K, k);
                acc += p;
                aabs += fabs(p);
            }
            double s = sx * (double)ws2[0];
            y[t * N + o] = acc * s;
            if (yabs) yabs[t * N + o] = aabs * fabs(s);
        }
    }
}

/* Dequantize stored MixFP4 ("Llama-3.1-8B-Instruct FlipQuant MixFP4 maps",
 * section "What this is"): the tile's map entry says how the block's codes
 * read (E0M3 level or E2M1 value); w' = BF16((c*S)*s2) as in the quantizer. */
void oracle_mixfp4_dequantize(const uint8_t* codes, const uint8_t* scales, float s2, const uint8_t* map,
                              int64_t rows, int64_t cols, int64_t tile_rows, int64_t tile_cols,
                              uint16_t* out)
{
    int64_t nb = cols / 16, tiles_per_row = cols / tile_cols;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            int e0m3 = map[(r / tile_rows) * tiles_per_row + (b * 16) / tile_cols] != 0;
            float S = oracle_e4m3_value(scales[r * nb + b]);
            for (int i = 0; i < 16; ++i) {
                uint8_t byte = codes[r * (cols / 2) + b * 8 + i / 2];
                unsigned c = (i & 1) ? (byte >> 4) : (byte & 15u);
                float cv = e0m3 ? oracle_e0m3_value(c) : oracle_e2m1_value(c);
                out[r * cols + b * 16 + i] = oracle_bf16_round((cv * S) * s2);
            }
        }
    }
}
