// focus_numerics.h -- device arithmetic of the FOCUS NVFP4 quantizer
// (binary32 block scale, sigmoid, element quotient, E2M1 / E4M3 / BF16
// conversions), shared by the kernels and by the test-only helper library
// that re-checks these helpers exhaustively on the GPU.  Every helper
// reproduces one step of the binary32 contract bit for bit; the argument for
// each is stated at the helper.  Method: "FOCUS NVFP4 scales for
// Llama-3.2-1B-Instruct (our reproduction)", section "What this is",
// equations S_b, c_i and w'_i.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace focus {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// element helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// E4M3FN byte of t, t a binary32 in [2^-6, 448]: round the mantissa to 3
// bits (nearest, ties to even) and rebias the exponent from 127 to 7.
__device__ __forceinline__ uint32_t e4m3_byte_normal(float t) {
    uint32_t u = __float_as_uint(t);
    u += 0x7FFFFu + ((u >> 20) & 1u);
    return (u >> 20) - (120u << 3);
}

// Value of a normal E4M3FN byte (0x08..0x7E).
__device__ __forceinline__ float e4m3_normal_value(uint32_t b) {
    return __uint_as_float((b + (120u << 3)) << 20);
}

// Value of any E4M3FN byte (subnormals, sign, NaN for 0x7F / 0xFF).
__device__ __forceinline__ float e4m3_any_value(uint32_t b) {
    uint32_t e = (b >> 3) & 15u, mm = b & 7u;
    float v = e ? __uint_as_float(((e + 120u) << 23) | (mm << 20)) : (float)mm * 0x1p-9f;
    if ((b & 0x7Fu) == 0x7Fu) v = __builtin_nanf("");
    return (b & 0x80u) ? -v : v;
}

// Block quotient t of equation S_b, zero-block rule, clamp.  The binary32
// quotient (a*m)/den is formed as RN32(RN64(num * RN64(1/den))), which is
// the IEEE binary32 quotient for any binary32 num and den: the binary64
// value is within 2^-52 of num/den, while num/den is never within 2^-49 of
// a binary32 midpoint (see the element quotient).  rden = RN64(1/den) is
// computed once per tensor.
__device__ __forceinline__ float block_t(float a, float mb, double rden) {
    const float num = a * mb;
    float t = (float)((double)num * rden);
    t = (t == 0.0f) ? 1.0f : t;
    return fminf(fmaxf(t, 0x1p-6f), 448.0f);
}

// 2^(j/64), j = 0..63, each rounded to binary64 (computed with 80-digit
// decimal arithmetic).
__device__ const double kExp2Frac64[64] = {
    0x1.0000000000000p+0, 0x1.02c9a3e778061p+0, 0x1.059b0d3158574p+0, 0x1.0874518759bc8p+0,
    0x1.0b5586cf9890fp+0, 0x1.0e3ec32d3d1a2p+0, 0x1.11301d0125b51p+0, 0x1.1429aaea92de0p+0,
    0x1.172b83c7d517bp+0, 0x1.1a35beb6fcb75p+0, 0x1.1d4873168b9aap+0, 0x1.2063b88628cd6p+0,
    0x1.2387a6e756238p+0, 0x1.26b4565e27cddp+0, 0x1.29e9df51fdee1p+0, 0x1.2d285a6e4030bp+0,
    0x1.306fe0a31b715p+0, 0x1.33c08b26416ffp+0, 0x1.371a7373aa9cbp+0, 0x1.3a7db34e59ff7p+0,
    0x1.3dea64c123422p+0, 0x1.4160a21f72e2ap+0, 0x1.44e086061892dp+0, 0x1.486a2b5c13cd0p+0,
    0x1.4bfdad5362a27p+0, 0x1.4f9b2769d2ca7p+0, 0x1.5342b569d4f82p+0, 0x1.56f4736b527dap+0,
    0x1.5ab07dd485429p+0, 0x1.5e76f15ad2148p+0, 0x1.6247eb03a5585p+0, 0x1.6623882552225p+0,
    0x1.6a09e667f3bcdp+0, 0x1.6dfb23c651a2fp+0, 0x1.71f75e8ec5f74p+0, 0x1.75feb564267c9p+0,
    0x1.7a11473eb0187p+0, 0x1.7e2f336cf4e62p+0, 0x1.82589994cce13p+0, 0x1.868d99b4492edp+0,
    0x1.8ace5422aa0dbp+0, 0x1.8f1ae99157736p+0, 0x1.93737b0cdc5e5p+0, 0x1.97d829fde4e50p+0,
    0x1.9c49182a3f090p+0, 0x1.a0c667b5de565p+0, 0x1.a5503b23e255dp+0, 0x1.a9e6b5579fdbfp+0,
    0x1.ae89f995ad3adp+0, 0x1.b33a2b84f15fbp+0, 0x1.b7f76f2fb5e47p+0, 0x1.bcc1e904bc1d2p+0,
    0x1.c199bdd85529cp+0, 0x1.c67f12e57d14bp+0, 0x1.cb720dcef9069p+0, 0x1.d072d4a07897cp+0,
    0x1.d5818dcfba487p+0, 0x1.da9e603db3285p+0, 0x1.dfc97337b9b5fp+0, 0x1.e502ee78b3ff6p+0,
    0x1.ea4afa2a490dap+0, 0x1.efa1bee615a27p+0, 0x1.f50765b6e4540p+0, 0x1.fa7c1819e90d8p+0};

// exp(x) in binary64 to about 2^-52 relative, for rounding once to
// binary32: x = (k/64) ln2 + r with |r| <= ln2/128 (Cody-Waite split of
// ln2/64 into a 32-bit head and a tail, so k*head is exact), exp(r) - 1 by
// its Taylor polynomial of degree 5 (truncation below 2^-54), and 2^(k/64)
// = 2^(k>>6) * table[k & 63].  x is first clamped to [-105, 89], outside of
// which the binary32 result is 0 or +inf anyway.  Rounded to binary32 it
// agreed with the correctly rounded exponential on every binary32 input in
// [-105, 89] that was checked against the platform's binary64 exp (all of
// them) and against an extended-precision reference (a 23 M sample).
__device__ __forceinline__ double exp_f64(double x, const double* tab) {
    x = fmin(fmax(x, -105.0), 89.0);
    const double kd = __builtin_rint(x * 0x1.71547652b82fep+6);  // x * 64/ln2
    const int k = (int)kd;
    double r = __builtin_fma(kd, -0x1.62e42fee00000p-7, x);
    r = __builtin_fma(kd, -0x1.a39ef35793c76p-39, r);
    double p = __builtin_fma(0x1.1111111111111p-7, r, 0x1.5555555555555p-5);  // 1/120, 1/24
    p = __builtin_fma(p, r, 0x1.5555555555555p-3);                             // 1/6
    p = __builtin_fma(p, r, 0.5);
    p = __builtin_fma(p, r, 1.0);
    p = p * r;
    const double t = tab[k & 63];
    return __builtin_ldexp(__builtin_fma(t, p, t), k >> 6);
}

// Which exp the sigmoid uses: 1 = exp_f64 with the 2^(j/64) table staged in
// LDS once per workgroup; 0 = the platform binary64 exp (no table).
constexpr int kExpImpl = 1;

// The workgroup's copy of kExp2Frac64 (64 doubles, 512 B of LDS), filled
// before the first use; every thread of the workgroup must call this.
__device__ __forceinline__ void stage_exp_table(double* lds_tab) {
    if (kExpImpl == 1) {
        if (threadIdx.x < 64) lds_tab[threadIdx.x] = kExp2Frac64[threadIdx.x];
        __syncthreads();
    }
}

// 1/s rounded to nearest binary32 for s >= 1: hardware reciprocal plus one
// fused correction step, which equals the IEEE quotient for every binary32
// s in [1, 2^126) (checked exhaustively); larger s (q < -87) take the IEEE
// division.
__device__ __forceinline__ float recip_rn_ge1(float s) {
    if (s < 0x1p126f) {
        const float y = __builtin_amdgcn_rcpf(s);
        const float e = __builtin_fmaf(-s, y, 1.0f);
        return __builtin_fmaf(e, y, y);
    }
    return 1.0f / s;
}

// 1/d in binary64 with relative error at most 2^-53 for every positive
// binary32 d (hardware reciprocal, about 2^-24, then two Newton steps;
// checked exhaustively).
__device__ __forceinline__ double recip_f64(double d) {
    double r = __builtin_amdgcn_rcp(d);
    double e = __builtin_fma(-d, r, 1.0);
    r = __builtin_fma(r, e, r);
    e = __builtin_fma(-d, r, 1.0);
    return __builtin_fma(r, e, r);
}

// sigmoid(q) = 1 / (1 + expf(-q)): three binary32 roundings (expf
// correctly rounded, the sum, the quotient).
__device__ __forceinline__ float sigmoid_cr(float q, const double* tab) {
    const float e = kExpImpl == 1 ? (float)exp_f64(-(double)q, tab) : (float)exp(-(double)q);
    const float s = 1.0f + e;
    return recip_rn_ge1(s);
}

// Eight binary32 values -> eight E2M1 codes in one dword, element 2j in the
// low nibble of byte j.  The instruction saturates beyond +-6, which is the
// clamp of equation c_i.
__device__ __forceinline__ uint32_t pack8(const float* x) {
    uint32_t v = 0;
    v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, x[0], x[1], 1.0f, 0);
    v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, x[2], x[3], 1.0f, 1);
    v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, x[4], x[5], 1.0f, 2);
    v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, x[6], x[7], 1.0f, 3);
    return v;
}

__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
    f32x2 f = {a, b};
    bf16x2 h = __builtin_convertvector(f, bf16x2);
    return __builtin_bit_cast(uint32_t, h);
}

// w' of two codes (byte `sel` of `codes`): BF16((c*S)*s2).
template <int SEL>
__device__ __forceinline__ uint32_t dequant_pair(uint32_t codes, float S, float s2) {
    f32x2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, SEL);
    float v0 = (c[0] * S) * s2;
    float v1 = (c[1] * S) * s2;
    return bf16_pair(v0, v1);
}

__device__ __forceinline__ uint4 dequant8(uint32_t codes, float S, float s2) {
    uint4 o;
    o.x = dequant_pair<0>(codes, S, s2);
    o.y = dequant_pair<1>(codes, S, s2);
    o.z = dequant_pair<2>(codes, S, s2);
    o.w = dequant_pair<3>(codes, S, s2);
    return o;
}

// Block maximum of 16 BF16 values as a binary32: integer maximum of the
// magnitude bits (exact, and cheaper than a float max that must quiet NaNs).
__device__ __forceinline__ float block_amax_bits(uint4 a, uint4 b) {
    const uint32_t mask = 0x7FFF7FFFu;
    u16x2 m0 = __builtin_bit_cast(u16x2, a.x & mask);
    u16x2 m1 = __builtin_bit_cast(u16x2, a.y & mask);
    u16x2 m2 = __builtin_bit_cast(u16x2, a.z & mask);
    u16x2 m3 = __builtin_bit_cast(u16x2, a.w & mask);
    u16x2 m4 = __builtin_bit_cast(u16x2, b.x & mask);
    u16x2 m5 = __builtin_bit_cast(u16x2, b.y & mask);
    u16x2 m6 = __builtin_bit_cast(u16x2, b.z & mask);
    u16x2 m7 = __builtin_bit_cast(u16x2, b.w & mask);
    m0 = __builtin_elementwise_max(__builtin_elementwise_max(m0, m1), __builtin_elementwise_max(m2, m3));
    m4 = __builtin_elementwise_max(__builtin_elementwise_max(m4, m5), __builtin_elementwise_max(m6, m7));
    m0 = __builtin_elementwise_max(m0, m4);
    const uint32_t mx = max((uint32_t)m0[0], (uint32_t)m0[1]);
    return __uint_as_float(mx << 16);
}

// Codes of 8 elements f[0..7] for the denominator d of their sub-block.
__device__ __forceinline__ uint32_t encode8(const float* f, float d) {
    float x[8];
    if (d != 0.0f) {
        const double r = recip_f64((double)d);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (float)((double)f[i] * r);
    } else {
        // Literal equation c_i when the denominator underflowed to 0.
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = fminf(fmaxf(f[i] / d, -6.0f), 6.0f);
    }
    return pack8(x);
}

// Sign-only codes (s2 == 0): code 8 for a negative zero, 0 otherwise.
__device__ __forceinline__ uint32_t sign_codes8(uint4 v) {
    uint32_t out = 0;
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t lo = (d[i] >> 15) & 1u, hi = (d[i] >> 31) & 1u;
        out |= ((lo << 3) | (hi << 7)) << (8 * i);
    }
    return out;
}

// ---------------------------------------------------------------------------
// MXFP4 (FOCUS on 32-element blocks with an E8M0 scale)
// ---------------------------------------------------------------------------

// E8M0 byte of the scaled block maximum t = max|w_b| * m_b: the OCP
// Microscaling rule 2^(floor(log2 t) - 2), exponent clamped to [-127, 127];
// t == 0 -> 1 (byte 127).  The hardware frexp exponent gives floor(log2 t) + 1
// for every finite t, subnormals included.
__device__ __forceinline__ uint32_t mx_scale_byte(float t) {
    if (t == 0.0f) return 127u;
    int e = __builtin_amdgcn_frexp_expf(t) - 1 - 2;
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
    return (uint32_t)(e + 127);
}

// Value of an E8M0 byte 0..254 (2^(b-127); 2^-127 is a binary32 subnormal).
__device__ __forceinline__ float e8m0_value(uint32_t b) {
    return b ? __uint_as_float(b << 23) : __uint_as_float(0x00400000u);
}

// ---------------------------------------------------------------------------
// FourOverSix: the block scale maps the block maximum to 6 or to 4, whichever
// quantizes the block with the lower binary32 squared error (summed in element
// order; the 4-candidate only when strictly lower).  m = 1, no relaxation.
// ---------------------------------------------------------------------------

// The exact error of one candidate: binary32 sum, in element order, of
// (w - (c*S)*s2)^2 over the 16 elements, from its packed codes c0 (elements
// 0-7) and c1 (8-15).
__device__ __forceinline__ float fo6_sq_err(const float* f, uint32_t c0, uint32_t c1, float S, float s2) {
    float e = 0.0f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t c = h ? c1 : c0;
#pragma unroll
        for (int sel = 0; sel < 4; ++sel) {
            f32x2 cv;
            if (sel == 0) cv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);
            else if (sel == 1) cv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1);
            else if (sel == 2) cv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 2);
            else cv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 3);
            const float v0 = (cv[0] * S) * s2;
            const float v1 = (cv[1] * S) * s2;
            const float e0 = f[8 * h + 2 * sel] - v0;
            const float e1 = f[8 * h + 2 * sel + 1] - v1;
            e = e + e0 * e0;
            e = e + e1 * e1;
        }
    }
    return e;
}

// Two elements of a FourOverSix candidate: their exact quotients x = RN(f/d)
// (r = recip_f64(d), as in encode8) go into byte SEL of `codes`, and the
// squares of x - c (c the decoded code value; the difference is exact by
// Sterbenz's lemma, since c/2 <= |x| <= 2c whenever c != 0) are added to
// `acc` with fused multiply-adds.
template <int SEL>
__device__ __forceinline__ void fo6_pair_est(float f0, float f1, double r, uint32_t& codes, float& acc) {
    const float x0 = (float)((double)f0 * r);
    const float x1 = (float)((double)f1 * r);
    codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, x0, x1, 1.0f, SEL);
    const f32x2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, SEL);
    const float u0 = x0 - c[0], u1 = x1 - c[1];
    acc = __builtin_fmaf(u0, u0, acc);
    acc = __builtin_fmaf(u1, u1, acc);
}

// Codes of 8 elements for the candidate whose binary64 reciprocal is r, plus
// the running estimate sum (x - c)^2.
__device__ __forceinline__ uint32_t fo6_encode8_est(const float* f, double r, float& acc) {
    uint32_t v = 0;
    fo6_pair_est<0>(f[0], f[1], r, v, acc);
    fo6_pair_est<1>(f[2], f[3], r, v, acc);
    fo6_pair_est<2>(f[4], f[5], r, v, acc);
    fo6_pair_est<3>(f[6], f[7], r, v, acc);
    return v;
}

// Range of s2 in which the estimate below is proven to decide exactly:
// every d = S*s2 lies in [2^-60, 2^57], so d^2 is normal, underflow costs at
// most 2^-30 in units of d^2, and no error sum overflows.
constexpr float kFo6S2Lo = 0x1p-54f;
constexpr float kFo6S2Hi = 0x1p48f;

// The FourOverSix decision (true: the 4-candidate).  The rule compares the
// two exact binary32 error sums E4 < E6.  Both candidates' codes are exact
// (exact quotients); their errors are first estimated in units of d^2:
// Ê = fused sum of (x - c)^2.  For s2 in [kFo6S2Lo, kFo6S2Hi] the exact sum
// satisfies |E/d^2 - Ê| <= 2^-24 (41.3 + 193.3 Ê) (the derivation uses
// |x| <= 6.376 and |x - c| <= 1, rounding of d, the quotient, c*S*s2, the
// difference, the square and 15 additions, and underflow bounded by 2^-150
// per operation).  With rho = d4/d6, E4/d6^2 is rho^2 E4/d4^2, so with the
// margins M = 2^-24 (80 + 400 Ê) (which also cover the rounding of rho^2 and
// of the comparisons) rho^2 (Ê4 + M4) < Ê6 - M6 proves E4 < E6 and
// rho^2 (Ê4 - M4) > Ê6 + M6 proves E4 > E6.  Anything in between (ties
// included) is decided by the exact sums.
__device__ __forceinline__ bool fo6_choose_four(const float* f, float s2, float S6, float d6, uint32_t c60,
                                                uint32_t c61, float e6, float S4, float d4, uint32_t c40,
                                                uint32_t c41, float e4) {
    const float rho = d4 * __builtin_amdgcn_rcpf(d6);
    const float rho2 = rho * rho;
    const float p4 = rho2 * e4;
    const float m4 = rho2 * __builtin_fmaf(400.0f * 0x1p-24f, e4, 80.0f * 0x1p-24f);
    const float m6 = __builtin_fmaf(400.0f * 0x1p-24f, e6, 80.0f * 0x1p-24f);
    if (p4 + m4 < e6 - m6) return true;
    if (p4 - m4 > e6 + m6) return false;
    return fo6_sq_err(f, c40, c41, S4, s2) < fo6_sq_err(f, c60, c61, S6, s2);
}

// ---------------------------------------------------------------------------
// FlipQuant MixFP4 E0M3 elements: uniform levels 0..7 with a sign bit (bit
// 3); the block scale maps the block maximum to 7.
// ---------------------------------------------------------------------------

// Code of a binary32 x in [-7, 7]: |x| + 2^23 is rounded to an integer by
// the binary32 addition (the spacing of binary32 in [2^23, 2^24) is 1), to
// nearest with ties to the even integer, and that integer is the low three
// bits.  The sign bit of x (also of -0) becomes bit 3.
__device__ __forceinline__ uint32_t e0m3_code(float x) {
    const uint32_t mag = __float_as_uint(__builtin_fabsf(x) + 0x1p23f) & 7u;
    return ((__float_as_uint(x) >> 28) & 8u) | mag;
}

// E0M3 codes of f[0..7] for the denominator d = S*s2, element 2j in the low
// nibble of byte j; the quotient is formed exactly as in encode8.
__device__ __forceinline__ uint32_t encode8_e0m3(const float* f, float d) {
    uint32_t v = 0;
    if (d != 0.0f) {
        const double r = recip_f64((double)d);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float x = fminf(fmaxf((float)((double)f[i] * r), -7.0f), 7.0f);
            v |= e0m3_code(x) << (4 * i);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v |= e0m3_code(fminf(fmaxf(f[i] / d, -7.0f), 7.0f)) << (4 * i);
    }
    return v;
}

// Signed level of an E0M3 code (-0 for code 8).
__device__ __forceinline__ float e0m3_level(uint32_t c) {
    return __uint_as_float(__float_as_uint((float)(c & 7u)) | ((c & 8u) << 28));
}

// w' of eight E0M3 codes: BF16((c*S)*s2).
__device__ __forceinline__ uint4 dequant8_e0m3(uint32_t codes, float S, float s2) {
    uint32_t o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const float v0 = (e0m3_level(codes >> (8 * p)) * S) * s2;
        const float v1 = (e0m3_level(codes >> (8 * p + 4)) * S) * s2;
        o[p] = bf16_pair(v0, v1);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// n / d for n < 2^31 and 1 <= d < 2^31 with a precomputed multiplier:
// M = ceil(2^(31+l) / d), l = ceil(log2 d), so M in [2^31, 2^32) and
// M*d - 2^(31+l) < d; then floor(n*M / 2^(31+l)) = floor(n/d), because the
// excess n*(M*d - 2^(31+l)) / (d*2^(31+l)) is below 2^-l <= 1/d and the
// fractional part of n/d is at most (d-1)/d.
__device__ __forceinline__ uint32_t div_magic(uint32_t n, uint32_t M, uint32_t sh) {
    return (uint32_t)(((uint64_t)n * M) >> sh);
}

}  // namespace focus
