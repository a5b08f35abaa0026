// focus_kernels.hip -- gfx950 kernels of the FOCUS NVFP4 quantizer.
//
// The method ("FOCUS NVFP4 scales for Llama-3.2-1B-Instruct (our
// reproduction)", section "What this is", equations S_b, c_i, w'_i and the
// paragraph after them):
//   s2  = amax|W| / (6*448)                                  (field table, s2)
//   t   = (max|w_b| * m_b) / (6*s2);  t == 0 -> 1;  clamp [2^-6, 448]
//   S_b = E4M3(t)                                             (equation S_b)
//   c_i = E2M1(clamp(w_i / ((S_b * sigmoid(q_k)) * s2), -6, 6)) (equation c_i)
//   w'_i = BF16((c_i * S_b) * s2)                             (equation w'_i)
// Every operation is one binary32 operation, round to nearest even; E2M1
// rounds to nearest, ties to even; sigmoid(q) = 1/(1 + expf(-q)) with expf
// correctly rounded.
//
// How each step maps onto CDNA4 (wave64) while staying bit-exact:
//  * One lane owns one 16-element block: two 16-byte loads of W, so a
//    wavefront streams 2 KB of contiguous weights; m (4 B/lane) and q
//    (8 B/lane) are read coalesced beside it; codes leave as 8 B/lane and
//    w' as two 16-byte stores.  No LDS is needed: nothing is shared.
//  * Block maximum: integer maximum of the BF16 magnitude bits (exact; the
//    bit patterns of non-negative floats order like their values).
//  * t = (a*m)/(6*s2) uses one binary64 reciprocal of the denominator per
//    tensor (exact, by the argument below); sigmoid uses a table-driven
//    binary64 exp rounded once to binary32 (the correctly rounded expf on
//    every input checked) and a corrected hardware reciprocal that equals
//    the IEEE binary32 quotient (checked exhaustively).
//  * Element quotient x = RN32(w/d) without a binary32 division per
//    element: r ~ 1/d once per sub-block (hardware reciprocal and two Newton
//    steps, relative error <= 2^-53 for every binary32 d, checked
//    exhaustively), then x = RN32(RN64(w*r)).  The binary64 value is within
//    2^-52 (relative) of w/d.  A binary32 midpoint is M*2^g with M odd and
//    2^24 < M < 2^25; with w = W*2^a and d = D*2^b (W, D odd, D < 2^24) the
//    difference w/d - M*2^g has numerator W*2^a - M*D*2^(b+g), a nonzero
//    multiple of the smaller power of two (M*D > 2^24 exceeds any binary32
//    significand W), so |w/d - mid| / (w/d) >= 1/(M*D) > 2^-49 whenever the
//    two are close.  Hence rounding the binary64 value once gives exactly the
//    IEEE binary32 quotient.  If d == 0 the sub-block falls back to the
//    literal binary32 division and clamp.
//  * E2M1 rounding and packing: v_cvt_scalef32_pk_fp4_f32 with scale 1.0
//    (RNE, saturating to +-6, sign-preserving for zeros; checked against the
//    E2M1 definition for every non-NaN binary32 input, both nibble slots).
//    Element 2j lands in the low nibble.
//  * w': v_cvt_scalef32_pk_f32_fp4 with scale 1.0 decodes two codes (exact),
//    then (c*S)*s2 in binary32 and v_cvt_pk_bf16_f32 (RNE; checked for every
//    non-NaN binary32 input).
//  * E4M3 rounding of t in [2^-6, 448] is integer RNE on the binary32 bits
//    (normal range only, so no subnormal or overflow case exists).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "focus_internal.h"

namespace focus {

constexpr int kThreads = 256;
constexpr int64_t kMaxGrid = 1 << 20;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Streaming memory access.  Weights, factors and logits are read exactly
// once and the outputs are not read back by the kernel, so loads and stores
// may bypass cache retention (nontemporal); the choice is set here.
constexpr bool kNtLoad = false;
constexpr bool kNtStore = true;
// Weights read as contiguous 1 KB per load instruction and regrouped per
// block through LDS, or read per block as two 16-byte loads at a 32-byte
// lane stride.  Measured on the 8B set: the regrouping pays when w' is also
// written (75 % vs 73 % of peak) and costs when only codes are (68 % vs
// 72 %), so it follows the w' flag.
template <bool DEQ>
struct LdsLoadW { static constexpr bool value = DEQ; };

// A value every lane of the workgroup reads and nobody writes during the
// kernel (a tensor's s2): read it through the constant address space so it
// becomes a scalar load.
__device__ __forceinline__ float ld_uniform(const float* p) {
    return *(const __attribute__((address_space(4))) float*)(uintptr_t)p;
}

__device__ __forceinline__ uint4 ld16(const uint4* p, int64_t i) {
    if (kNtLoad) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + i);
        return make_uint4(v.x, v.y, v.z, v.w);
    }
    return p[i];
}
__device__ __forceinline__ float ld4f(const float* p, int64_t i) {
    return kNtLoad ? __builtin_nontemporal_load(p + i) : p[i];
}
__device__ __forceinline__ float2 ld8f(const float2* p, int64_t i) {
    if (kNtLoad) {
        const f32x2 v = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(p) + i);
        return make_float2(v[0], v[1]);
    }
    return p[i];
}
__device__ __forceinline__ uint2 ld8u(const uint2* p, int64_t i) {
    if (kNtLoad) {
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p) + i);
        return make_uint2(v.x, v.y);
    }
    return p[i];
}
__device__ __forceinline__ void st16(uint4* p, int64_t i, uint4 v) {
    if (kNtStore) __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p) + i);
    else p[i] = v;
}
__device__ __forceinline__ void st8(uint2* p, int64_t i, uint2 v) {
    if (kNtStore) __builtin_nontemporal_store(u32x2{v.x, v.y}, reinterpret_cast<u32x2*>(p) + i);
    else p[i] = v;
}

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

// Store 32 bytes per lane for the 64 consecutive blocks of one wavefront so
// that every store instruction writes 1 KB of contiguous memory: lane l
// deposits its block in the wavefront's 2 KB of LDS, then writes half-block
// l and half-block 64 + l.  Stores of 16 bytes at a 32-byte lane stride
// leave every cache line half written by each instruction, which costs a
// third of the write bandwidth when reads and writes mix.  All 64 lanes must
// call this (uniform control flow); `valid` is the number of blocks of the
// wavefront that exist.  The LDS instructions of one wavefront execute in
// order, and the compiler keeps these may-alias accesses in program order,
// so no fence is needed (a fence would also wait for the global stores).
__device__ __forceinline__ void wave_store_blocks(uint4* dst, uint4 lo, uint4 hi, uint4* xch,
                                                  int lane, int64_t valid) {
    xch[2 * lane] = lo;
    xch[2 * lane + 1] = hi;
    __builtin_amdgcn_wave_barrier();
    const uint4 h0 = xch[lane];
    const uint4 h1 = xch[64 + lane];
    __builtin_amdgcn_wave_barrier();
    const int64_t halves = 2 * valid;
    if (lane < halves) st16(dst, lane, h0);
    if (64 + lane < halves) st16(dst, 64 + lane, h1);
}

// The inverse regrouping for loads: lane l holds half-blocks l and 64 + l of
// the wavefront's 64 consecutive blocks (two contiguous 1 KB loads) and
// receives block l (its two halves) through the wavefront's 2 KB of LDS.
__device__ __forceinline__ void wave_gather_blocks(uint4& lo, uint4& hi, uint4* xch, int lane) {
    xch[lane] = lo;
    xch[64 + lane] = hi;
    __builtin_amdgcn_wave_barrier();
    lo = xch[2 * lane];
    hi = xch[2 * lane + 1];
    __builtin_amdgcn_wave_barrier();
}

// One 16-element block: codes (two dwords) and scale byte are stored here;
// w' (32 bytes) is returned in deq0 / deq1 for the caller's wavefront-wide
// contiguous store.
template <bool HAS_SIG, bool DEQ>
__device__ __forceinline__ void quantize_block(uint4 a, uint4 b, float mb, float q0, float q1,
                                               float s2, double rden, const double* tab,
                                               uint2* codes_out, uint8_t* scale_out, uint4& deq0,
                                               uint4& deq1) {
    const uint32_t v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    float f[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        f[2 * i] = bf16_lo(v[i]);
        f[2 * i + 1] = bf16_hi(v[i]);
    }
    if (s2 == 0.0f) {
        // every block is a zero block: scale 1, signed-zero codes, w' = +-0
        *scale_out = 0x38;
        st8(codes_out, 0, make_uint2(sign_codes8(a), sign_codes8(b)));
        if (DEQ) {
            const uint32_t z = 0x80008000u;
            deq0 = make_uint4(a.x & z, a.y & z, a.z & z, a.w & z);
            deq1 = make_uint4(b.x & z, b.y & z, b.z & z, b.w & z);
        }
        return;
    }
    const float amax = block_amax_bits(a, b);
    const uint32_t sb = e4m3_byte_normal(block_t(amax, mb, rden));
    const float S = e4m3_normal_value(sb);
    float sig0 = 1.0f, sig1 = 1.0f;
    if (HAS_SIG) {
        sig0 = sigmoid_cr(q0, tab);
        sig1 = sigmoid_cr(q1, tab);
    }
    const float d0 = (S * sig0) * s2;
    const float d1 = (S * sig1) * s2;
    const uint32_t c0 = encode8(f, d0);
    const uint32_t c1 = encode8(f + 8, d1);
    st8(codes_out, 0, make_uint2(c0, c1));
    *scale_out = (uint8_t)sb;
    if (DEQ) {
        deq0 = dequant8(c0, S, s2);
        deq1 = dequant8(c1, S, s2);
    }
}

// ---------------------------------------------------------------------------
// batches: up to kBatch tensors per launch, described in the kernel argument
// segment (structure of arrays, about 2.3 KB).  Work is cut into tiles of
// kThreads * U blocks; tile_start[j] is the first tile of tensor j, so a
// workgroup finds its tensor by a binary search over scalar loads.
// ---------------------------------------------------------------------------

__device__ __forceinline__ int find_tensor(const int64_t* tile_start, int n, int64_t tile) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tile_start[mid] <= tile) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// ---------------------------------------------------------------------------
// focus_quantize(_many): one lane per 16-element block, U blocks per lane
// per tile with all loads issued before any arithmetic
// ---------------------------------------------------------------------------

constexpr int kQuantU = 2;
constexpr int64_t kQuantTile = (int64_t)kThreads * kQuantU;

template <bool HAS_M, bool HAS_Q, bool DEQ>
__global__ __launch_bounds__(kThreads) void k_quantize(QuantBatch bt, int64_t ntiles) {
    __shared__ uint4 xch[DEQ ? kThreads / 64 : 1][128];
    constexpr bool kLdsLoadW = LdsLoadW<DEQ>::value;
    __shared__ uint4 xchw[kLdsLoadW ? kThreads / 64 : 1][128];
    __shared__ double tab[HAS_Q ? 64 : 1];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    if (HAS_Q) stage_exp_table(tab);
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int j = find_tensor(bt.tile_start, bt.n, tile);
        const uint4* __restrict__ w = bt.w[j];
        const float* __restrict__ m = bt.m[j];
        const float2* __restrict__ q = bt.q[j];
        const float s2 = ld_uniform(bt.s2[j]);
        const double rden = 1.0 / (double)(6.0f * s2);
        const int64_t nblk = bt.nblk[j];
        const int64_t tile0 = (tile - bt.tile_start[j]) * kQuantTile;
        uint4 va[kQuantU], vb[kQuantU];
        float mb[kQuantU];
        float2 qq[kQuantU];
#pragma unroll
        for (int k = 0; k < kQuantU; ++k) {
            const int64_t first = tile0 + (int64_t)k * kThreads + wave * 64;  // block of lane 0
            const int64_t blk = first + lane;
            if (kLdsLoadW) {
                // half-blocks 2*first + lane and 2*first + 64 + lane
                const int64_t h = 2 * first + lane, nh = 2 * nblk;
                va[k] = h < nh ? ld16(w, h) : make_uint4(0, 0, 0, 0);
                vb[k] = h + 64 < nh ? ld16(w, h + 64) : make_uint4(0, 0, 0, 0);
            } else if (blk < nblk) {
                va[k] = ld16(w, 2 * blk);
                vb[k] = ld16(w, 2 * blk + 1);
            }
            if (blk < nblk) {
                mb[k] = HAS_M ? ld4f(m, blk) : 1.0f;
                qq[k] = HAS_Q ? ld8f(q, blk) : make_float2(0.0f, 0.0f);
            }
        }
#pragma unroll
        for (int k = 0; k < kQuantU; ++k) {
            const int64_t first = tile0 + (int64_t)k * kThreads + wave * 64;  // block of lane 0
            const int64_t blk = first + lane;
            if (kLdsLoadW && first < nblk) wave_gather_blocks(va[k], vb[k], xchw[wave], lane);
            uint4 d0 = make_uint4(0, 0, 0, 0), d1 = d0;
            if (blk < nblk)
                quantize_block<HAS_Q, DEQ>(va[k], vb[k], mb[k], qq[k].x, qq[k].y, s2, rden, tab,
                                           bt.codes[j] + blk, bt.scales[j] + blk, d0, d1);
            if (DEQ && first < nblk)
                wave_store_blocks(bt.wdeq[j] + 2 * first, d0, d1, xch[DEQ ? wave : 0], lane,
                                  nblk - first);
        }
    }
}

// ---------------------------------------------------------------------------
// focus_dequantize(_many): one lane per block
// ---------------------------------------------------------------------------

constexpr int64_t kDeqTile = (int64_t)kThreads * 2;

__global__ __launch_bounds__(kThreads) void k_dequantize(DequantBatch bt, int64_t ntiles) {
    __shared__ uint4 xch[kThreads / 64][128];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int j = find_tensor(bt.tile_start, bt.n, tile);
        const uint2* __restrict__ codes = bt.codes[j];
        const uint8_t* __restrict__ scales = bt.scales[j];
        const float* __restrict__ s2p = bt.s2[j];
        const int64_t nblk = bt.nblk[j], nb_row = bt.nb_row[j];
        const bool per_row = bt.per_row[j] != 0;
        const int64_t tile0 = (tile - bt.tile_start[j]) * kDeqTile;
        uint2 c[2];
        uint32_t sb[2];
        float s2v[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int64_t blk = tile0 + (int64_t)k * kThreads + threadIdx.x;
            if (blk < nblk) {
                c[k] = ld8u(codes, blk);
                sb[k] = scales[blk];
            }
        }
        if (per_row) {  // uniform branch: one s2 per row (activations)
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int64_t blk = tile0 + (int64_t)k * kThreads + threadIdx.x;
                if (blk < nblk) s2v[k] = s2p[blk / nb_row];
            }
        } else {
            const float s2u = ld_uniform(s2p);
            s2v[0] = s2v[1] = s2u;
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int64_t first = tile0 + (int64_t)k * kThreads + wave * 64;
            const int64_t blk = first + lane;
            uint4 d0 = make_uint4(0, 0, 0, 0), d1 = d0;
            if (blk < nblk) {
                const float S = e4m3_any_value(sb[k]);
                d0 = dequant8(c[k].x, S, s2v[k]);
                d1 = dequant8(c[k].y, S, s2v[k]);
            }
            if (first < nblk) wave_store_blocks(bt.out[j] + 2 * first, d0, d1, xch[wave], lane, nblk - first);
        }
    }
}

// ---------------------------------------------------------------------------
// focus_tensor_scale(_many): clear, reduce (max of BF16 magnitude bits),
// finalize
// ---------------------------------------------------------------------------

__global__ void k_clear_acc(ScaleBatch bt) {
    if ((int)threadIdx.x < bt.n) *reinterpret_cast<uint32_t*>(bt.s2[threadIdx.x]) = 0u;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
    return v;
}

constexpr int kAmaxVecPerThread = 8;                                  // 16-byte vectors per lane per tile
constexpr int64_t kAmaxTile = (int64_t)kThreads * kAmaxVecPerThread;  // vectors per tile (32 KB)
constexpr int64_t kAmaxGrid = 1024;                                   // workgroups per launch (at most)

__device__ __forceinline__ u16x2 max_mag2(u16x2 acc, uint32_t v) {
    return __builtin_elementwise_max(acc, __builtin_bit_cast(u16x2, v & 0x7FFF7FFFu));
}

// Combine the lanes' maxima of one tensor and fold them into its
// accumulator.  Called by every thread of the workgroup (uniform control).
__device__ __forceinline__ void amax_flush(u16x2 mx, uint32_t* acc, uint32_t* part) {
    uint32_t mm = wave_max_u32(max((uint32_t)mx[0], (uint32_t)mx[1]));
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) part[wave] = mm;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = part[0];
#pragma unroll
        for (int k = 1; k < kThreads / 64; ++k) r = max(r, part[k]);
        atomicMax(acc, r << 16);
    }
    __syncthreads();
}

// Persistent reduction: workgroup g owns the contiguous tile range
// [g*per, (g+1)*per) of the batch (tiles of all tensors laid end to end),
// keeps a running maximum in registers, and flushes it (wave reduce, LDS,
// one atomic max on the tensor's accumulator) only when its range moves on
// to the next tensor and at the end.  The accumulator is the s2 slot itself,
// holding the bits of a non-negative binary32 (the BF16 magnitude shifted
// up); an integer atomic max orders such floats exactly.  Loads are
// nontemporal: the weights are read once.
__global__ __launch_bounds__(kThreads) void k_amax(ScaleBatch bt, int64_t ntiles) {
    __shared__ uint32_t part[kThreads / 64];
    const int64_t per = (ntiles + gridDim.x - 1) / gridDim.x;
    const int64_t lo = (int64_t)blockIdx.x * per;
    const int64_t hi = lo + per < ntiles ? lo + per : ntiles;
    if (lo >= hi) return;  // whole workgroup
    int j = find_tensor(bt.tile_start, bt.n, lo);
    u16x2 mx = {0, 0};
    for (int64_t tile = lo; tile < hi; ++tile) {
        if (tile >= bt.tile_start[j + 1]) {
            amax_flush(mx, reinterpret_cast<uint32_t*>(bt.s2[j]), part);
            mx = u16x2{0, 0};
            j = find_tensor(bt.tile_start, bt.n, tile);
        }
        const uint16_t* __restrict__ w16 = bt.w[j];
        const u32x4* __restrict__ w = reinterpret_cast<const u32x4*>(w16);
        const int64_t numel = bt.numel[j];
        const int64_t nvec = numel / 8;
        const int64_t base = (tile - bt.tile_start[j]) * kAmaxTile + threadIdx.x;
        u32x4 v[kAmaxVecPerThread];
#pragma unroll
        for (int k = 0; k < kAmaxVecPerThread; ++k) {
            const int64_t i = base + (int64_t)k * kThreads;
            v[k] = i < nvec ? __builtin_nontemporal_load(w + i) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int k = 0; k < kAmaxVecPerThread; ++k)
            mx = max_mag2(max_mag2(max_mag2(max_mag2(mx, v[k].x), v[k].y), v[k].z), v[k].w);
        // the last numel % 8 elements: read one by one by the lane that would
        // have loaded vector nvec
#pragma unroll
        for (int k = 0; k < kAmaxVecPerThread; ++k) {
            if (base + (int64_t)k * kThreads == nvec) {
                for (int64_t e = nvec * 8; e < numel; ++e) mx = max_mag2(mx, (uint32_t)w16[e]);
            }
        }
    }
    amax_flush(mx, reinterpret_cast<uint32_t*>(bt.s2[j]), part);
}

__global__ void k_finalize_s2(ScaleBatch bt) {
    const int j = threadIdx.x;
    if (j >= bt.n) return;
    uint32_t* acc = reinterpret_cast<uint32_t*>(bt.s2[j]);
    const float amax = __uint_as_float(*acc);
    *bt.s2[j] = amax / 2688.0f;
    if (bt.amax[j]) *bt.amax[j] = amax;
}

// ---------------------------------------------------------------------------
// focus_quantize_act_per_token: one wavefront per token row
// ---------------------------------------------------------------------------

__device__ __forceinline__ float wave_max_f32(float v) {
    // non-negative binary32: integer order equals value order
    return __uint_as_float(wave_max_u32(__float_as_uint(v)));
}

// RB > 0: lane keeps up to RB blocks of the row in registers (rows of at most
// 64*RB blocks).  RB == 0: rows of any length, read twice (the second read
// hits the caches).
template <int RB, bool DEQ>
__global__ __launch_bounds__(kThreads) void k_act(const uint4* __restrict__ x, int64_t tokens,
                                                  int64_t nb, uint2* __restrict__ codes,
                                                  uint8_t* __restrict__ scales,
                                                  float* __restrict__ s2out,
                                                  uint4* __restrict__ xdeq) {
    __shared__ uint4 xch[DEQ ? kThreads / 64 : 1][128];
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (row >= tokens) return;  // uniform per wavefront; nothing below synchronizes the workgroup
    const int64_t base = row * nb;
    float amax = 0.0f;
    constexpr int R = RB > 0 ? RB : 1;
    uint4 va[R], vb[R];
    if (RB > 0) {
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const int64_t j = lane + 64 * k;
            if (j < nb) {
                va[k] = x[2 * (base + j)];
                vb[k] = x[2 * (base + j) + 1];
                amax = fmaxf(amax, block_amax_bits(va[k], vb[k]));
            }
        }
    } else {
        for (int64_t j = lane; j < nb; j += 64)
            amax = fmaxf(amax, block_amax_bits(x[2 * (base + j)], x[2 * (base + j) + 1]));
    }
    amax = wave_max_f32(amax);
    const float s2 = amax / 2688.0f;
    if (lane == 0) s2out[row] = s2;
    const double rden = 1.0 / (double)(6.0f * s2);
    uint4* xw = xch[DEQ ? (threadIdx.x >> 6) : 0];
    if (RB > 0) {
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const int64_t j0 = 64 * k, j = j0 + lane;
            uint4 d0 = make_uint4(0, 0, 0, 0), d1 = d0;
            if (j < nb)
                quantize_block<false, DEQ>(va[k], vb[k], 1.0f, 0.0f, 0.0f, s2, rden, nullptr, codes + base + j,
                                           scales + base + j, d0, d1);
            if (DEQ && j0 < nb) wave_store_blocks(xdeq + 2 * (base + j0), d0, d1, xw, lane, nb - j0);
        }
    } else {
        for (int64_t j0 = 0; j0 < nb; j0 += 64) {
            const int64_t j = j0 + lane;
            uint4 d0 = make_uint4(0, 0, 0, 0), d1 = d0;
            if (j < nb)
                quantize_block<false, DEQ>(x[2 * (base + j)], x[2 * (base + j) + 1], 1.0f, 0.0f, 0.0f,
                                           s2, rden, nullptr, codes + base + j, scales + base + j, d0, d1);
            if (DEQ) wave_store_blocks(xdeq + 2 * (base + j0), d0, d1, xw, lane, nb - j0);
        }
    }
}

// ---------------------------------------------------------------------------
// launchers (arguments already validated by the C ABI layer)
// ---------------------------------------------------------------------------

static inline unsigned grid_for_tiles(int64_t ntiles) {
    int64_t g = ntiles < 1 ? 1 : ntiles;
    if (g > kMaxGrid) g = kMaxGrid;
    return (unsigned)g;
}

hipError_t launch_tensor_scale(ScaleBatch& bt, hipStream_t stream) {
    int64_t t = 0;
    for (int j = 0; j < bt.n; ++j) {
        bt.tile_start[j] = t;
        const int64_t nv = (bt.numel[j] + 7) / 8;  // vectors, the last one possibly partial
        const int64_t nt = (nv + kAmaxTile - 1) / kAmaxTile;
        t += nt > 0 ? nt : 1;
    }
    bt.tile_start[bt.n] = t;
    const int64_t g = t < kAmaxGrid ? t : kAmaxGrid;
    hipLaunchKernelGGL(k_clear_acc, dim3(1), dim3(kBatch), 0, stream, bt);
    hipLaunchKernelGGL(k_amax, dim3((unsigned)g), dim3(kThreads), 0, stream, bt, t);
    hipLaunchKernelGGL(k_finalize_s2, dim3(1), dim3(kBatch), 0, stream, bt);
    return hipGetLastError();
}

hipError_t launch_quantize(QuantBatch& bt, int key, hipStream_t stream) {
    int64_t t = 0;
    for (int j = 0; j < bt.n; ++j) {
        bt.tile_start[j] = t;
        t += (bt.nblk[j] + kQuantTile - 1) / kQuantTile;
    }
    bt.tile_start[bt.n] = t;
    const dim3 grid(grid_for_tiles(t)), block(kThreads);
    switch (key) {
#define FOCUS_Q_CASE(K, HM, HQ, DQ)                                                            \
    case K:                                                                                    \
        hipLaunchKernelGGL((k_quantize<HM, HQ, DQ>), grid, block, 0, stream, bt, t);          \
        break;
        FOCUS_Q_CASE(0, false, false, false)
        FOCUS_Q_CASE(1, false, false, true)
        FOCUS_Q_CASE(2, false, true, false)
        FOCUS_Q_CASE(3, false, true, true)
        FOCUS_Q_CASE(4, true, false, false)
        FOCUS_Q_CASE(5, true, false, true)
        FOCUS_Q_CASE(6, true, true, false)
        FOCUS_Q_CASE(7, true, true, true)
#undef FOCUS_Q_CASE
    }
    return hipGetLastError();
}

hipError_t launch_dequantize(DequantBatch& bt, hipStream_t stream) {
    int64_t t = 0;
    for (int j = 0; j < bt.n; ++j) {
        bt.tile_start[j] = t;
        t += (bt.nblk[j] + kDeqTile - 1) / kDeqTile;
    }
    bt.tile_start[bt.n] = t;
    hipLaunchKernelGGL(k_dequantize, dim3(grid_for_tiles(t)), dim3(kThreads), 0, stream, bt, t);
    return hipGetLastError();
}

hipError_t launch_act_per_token(const uint16_t* x, int64_t tokens, int64_t hidden, uint8_t* codes,
                                uint8_t* scales, float* s2_out, uint16_t* xdeq,
                                hipStream_t stream) {
    const int64_t nb = hidden / 16;
    const int64_t rows_per_wg = kThreads / 64;
    const dim3 grid((unsigned)((tokens + rows_per_wg - 1) / rows_per_wg)), block(kThreads);
    auto X = reinterpret_cast<const uint4*>(x);
    auto C = reinterpret_cast<uint2*>(codes);
    auto D = reinterpret_cast<uint4*>(xdeq);
#define FOCUS_ACT(RB)                                                                          \
    do {                                                                                       \
        if (xdeq)                                                                              \
            hipLaunchKernelGGL((k_act<RB, true>), grid, block, 0, stream, X, tokens, nb, C,    \
                               scales, s2_out, D);                                             \
        else                                                                                   \
            hipLaunchKernelGGL((k_act<RB, false>), grid, block, 0, stream, X, tokens, nb, C,   \
                               scales, s2_out, D);                                             \
    } while (0)
    if (nb <= 64) FOCUS_ACT(1);
    else if (nb <= 128) FOCUS_ACT(2);
    else if (nb <= 256) FOCUS_ACT(4);
    else if (nb <= 512) FOCUS_ACT(8);
    else FOCUS_ACT(0);
#undef FOCUS_ACT
    return hipGetLastError();
}

}  // namespace focus
