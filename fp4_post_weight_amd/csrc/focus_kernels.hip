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
//  * Block maximum: binary32 max of |w| (exact).
//  * t and sigmoid use IEEE binary32 division (the compiler's correctly
//    rounded sequence).  expf is evaluated as the binary64 exp rounded once
//    to binary32, which is the correctly rounded binary32 exponential except
//    when exp lands within about 2^-52 of a binary32 midpoint.
//  * Element quotient x = RN32(w/d) without a binary32 division per
//    element: r = RN64(1/d) once per sub-block, then x = RN32(RN64(w*r)).
//    The binary64 value is within 2^-52 (relative) of w/d; w has at most 8
//    significant bits and d at most 24, so w/d is never closer than about
//    2^-49 (relative) to a binary32 midpoint (a midpoint has a 25-bit odd
//    significand M, and w = M*d*2^k is impossible with an odd significand of
//    w below 2^8 < M).  Hence rounding the binary64 value once gives exactly
//    the IEEE binary32 quotient.  If d == 0 the sub-block falls back to the
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

// Block quotient t of equation S_b, zero-block rule, clamp.
__device__ __forceinline__ float block_t(float a, float mb, float den) {
    float t = (a * mb) / den;
    t = (t == 0.0f) ? 1.0f : t;
    return fminf(fmaxf(t, 0x1p-6f), 448.0f);
}

// sigmoid(q) = 1 / (1 + expf(-q)) with expf correctly rounded (see header).
__device__ __forceinline__ float sigmoid_cr(float q) {
    float e = (float)exp(-(double)q);
    float s = 1.0f + e;
    return 1.0f / s;
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

// Codes of 8 elements f[0..7] for the denominator d of their sub-block.
__device__ __forceinline__ uint32_t encode8(const float* f, float d) {
    float x[8];
    if (d != 0.0f) {
        const double r = 1.0 / (double)d;
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

// One 16-element block: codes (two dwords), scale byte, optional w'.
template <bool HAS_SIG, bool DEQ>
__device__ __forceinline__ void quantize_block(uint4 a, uint4 b, float mb, float q0, float q1,
                                               float s2, float den, uint2* codes_out,
                                               uint8_t* scale_out, uint4* deq_out) {
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
        *codes_out = make_uint2(sign_codes8(a), sign_codes8(b));
        if (DEQ) {
            const uint32_t z = 0x80008000u;
            deq_out[0] = make_uint4(a.x & z, a.y & z, a.z & z, a.w & z);
            deq_out[1] = make_uint4(b.x & z, b.y & z, b.z & z, b.w & z);
        }
        return;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i += 2) amax = fmaxf(amax, fmaxf(fabsf(f[i]), fabsf(f[i + 1])));
    const uint32_t sb = e4m3_byte_normal(block_t(amax, mb, den));
    const float S = e4m3_normal_value(sb);
    float sig0 = 1.0f, sig1 = 1.0f;
    if (HAS_SIG) {
        sig0 = sigmoid_cr(q0);
        sig1 = sigmoid_cr(q1);
    }
    const float d0 = (S * sig0) * s2;
    const float d1 = (S * sig1) * s2;
    const uint32_t c0 = encode8(f, d0);
    const uint32_t c1 = encode8(f + 8, d1);
    *codes_out = make_uint2(c0, c1);
    *scale_out = (uint8_t)sb;
    if (DEQ) {
        deq_out[0] = dequant8(c0, S, s2);
        deq_out[1] = dequant8(c1, S, s2);
    }
}

// ---------------------------------------------------------------------------
// focus_quantize: one lane per 16-element block, grid-stride over blocks
// ---------------------------------------------------------------------------

template <bool HAS_M, bool HAS_Q, bool DEQ>
__global__ __launch_bounds__(kThreads) void k_quantize(
    const uint4* __restrict__ w, const float* __restrict__ m, const float2* __restrict__ q,
    const float* __restrict__ s2p, uint2* __restrict__ codes, uint8_t* __restrict__ scales,
    uint4* __restrict__ wdeq, int64_t nblk) {
    const float s2 = *s2p;
    const float den = 6.0f * s2;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t blk = (int64_t)blockIdx.x * kThreads + threadIdx.x; blk < nblk; blk += stride) {
        const uint4 a = w[2 * blk];
        const uint4 b = w[2 * blk + 1];
        const float mb = HAS_M ? m[blk] : 1.0f;
        float2 qq = make_float2(0.0f, 0.0f);
        if (HAS_Q) qq = q[blk];
        quantize_block<HAS_Q, DEQ>(a, b, mb, qq.x, qq.y, s2, den, codes + blk, scales + blk,
                                   DEQ ? wdeq + 2 * blk : nullptr);
    }
}

// ---------------------------------------------------------------------------
// focus_dequantize: one lane per block
// ---------------------------------------------------------------------------

template <bool PER_ROW>
__global__ __launch_bounds__(kThreads) void k_dequantize(
    const uint2* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ s2p, int64_t nblk, int64_t nb_row, uint4* __restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const float s2u = PER_ROW ? 0.0f : *s2p;
    for (int64_t blk = (int64_t)blockIdx.x * kThreads + threadIdx.x; blk < nblk; blk += stride) {
        const uint2 c = codes[blk];
        const float S = e4m3_any_value(scales[blk]);
        const float s2 = PER_ROW ? s2p[blk / nb_row] : s2u;
        out[2 * blk] = dequant8(c.x, S, s2);
        out[2 * blk + 1] = dequant8(c.y, S, s2);
    }
}

// ---------------------------------------------------------------------------
// focus_tensor_scale: clear, reduce (max of BF16 magnitude bits), finalize
// ---------------------------------------------------------------------------

__global__ void k_fill_u32(uint32_t* p, uint32_t v) { *p = v; }

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
    return v;
}

// acc: the bits of a non-negative binary32 (the BF16 magnitude shifted up),
// combined with an integer atomic max, which orders such floats exactly.
__global__ __launch_bounds__(kThreads) void k_amax(const uint4* __restrict__ w, int64_t nvec,
                                                   const uint16_t* __restrict__ tail, int ntail,
                                                   uint32_t* __restrict__ acc) {
    u16x2 mx = {0, 0};
    const uint32_t mask = 0x7FFF7FFFu;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += stride) {
        const uint4 v = w[i];
        u16x2 a = __builtin_bit_cast(u16x2, v.x & mask);
        u16x2 b = __builtin_bit_cast(u16x2, v.y & mask);
        u16x2 c = __builtin_bit_cast(u16x2, v.z & mask);
        u16x2 d = __builtin_bit_cast(u16x2, v.w & mask);
        mx = __builtin_elementwise_max(mx, __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                                                     __builtin_elementwise_max(c, d)));
    }
    uint32_t m = max((uint32_t)mx[0], (uint32_t)mx[1]);
    if (blockIdx.x == 0 && (int)threadIdx.x < ntail) m = max(m, (uint32_t)(tail[threadIdx.x] & 0x7FFFu));
    m = wave_max_u32(m);
    __shared__ uint32_t part[kThreads / 64];
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) part[wave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = part[0];
#pragma unroll
        for (int k = 1; k < kThreads / 64; ++k) r = max(r, part[k]);
        atomicMax(acc, r << 16);
    }
}

__global__ void k_finalize_s2(uint32_t* acc_s2, float* amax_out) {
    const float amax = __uint_as_float(*acc_s2);
    *reinterpret_cast<float*>(acc_s2) = amax / 2688.0f;
    if (amax_out) *amax_out = amax;
}

// ---------------------------------------------------------------------------
// focus_quantize_act_per_token: one wavefront per token row
// ---------------------------------------------------------------------------

__device__ __forceinline__ float wave_max_f32(float v) {
    // non-negative binary32: integer order equals value order
    return __uint_as_float(wave_max_u32(__float_as_uint(v)));
}

__device__ __forceinline__ float block_amax(uint4 a, uint4 b) {
    const uint32_t v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fmaxf(fabsf(bf16_lo(v[i])), fabsf(bf16_hi(v[i]))));
    return m;
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
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (row >= tokens) return;  // uniform per wavefront
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
                amax = fmaxf(amax, block_amax(va[k], vb[k]));
            }
        }
    } else {
        for (int64_t j = lane; j < nb; j += 64)
            amax = fmaxf(amax, block_amax(x[2 * (base + j)], x[2 * (base + j) + 1]));
    }
    amax = wave_max_f32(amax);
    const float s2 = amax / 2688.0f;
    if (lane == 0) s2out[row] = s2;
    const float den = 6.0f * s2;
    if (RB > 0) {
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const int64_t j = lane + 64 * k;
            if (j < nb)
                quantize_block<false, DEQ>(va[k], vb[k], 1.0f, 0.0f, 0.0f, s2, den, codes + base + j,
                                           scales + base + j, DEQ ? xdeq + 2 * (base + j) : nullptr);
        }
    } else {
        for (int64_t j = lane; j < nb; j += 64)
            quantize_block<false, DEQ>(x[2 * (base + j)], x[2 * (base + j) + 1], 1.0f, 0.0f, 0.0f, s2,
                                       den, codes + base + j, scales + base + j,
                                       DEQ ? xdeq + 2 * (base + j) : nullptr);
    }
}

// ---------------------------------------------------------------------------
// launchers (arguments already validated by the C ABI layer)
// ---------------------------------------------------------------------------

static inline unsigned grid_for(int64_t items) {
    int64_t g = (items + kThreads - 1) / kThreads;
    if (g < 1) g = 1;
    if (g > kMaxGrid) g = kMaxGrid;
    return (unsigned)g;
}

hipError_t launch_tensor_scale(const uint16_t* w, int64_t numel, float* s2_out, float* amax_out,
                               hipStream_t stream) {
    uint32_t* acc = reinterpret_cast<uint32_t*>(s2_out);
    hipLaunchKernelGGL(k_fill_u32, dim3(1), dim3(1), 0, stream, acc, 0u);
    const int64_t nvec = numel / 8;
    const int ntail = (int)(numel - nvec * 8);
    if (numel > 0) {
        int64_t g = (nvec + kThreads - 1) / kThreads;
        if (g > 2048) g = 2048;
        if (g < 1) g = 1;
        hipLaunchKernelGGL(k_amax, dim3((unsigned)g), dim3(kThreads), 0, stream,
                           reinterpret_cast<const uint4*>(w), nvec, w + nvec * 8, ntail, acc);
    }
    hipLaunchKernelGGL(k_finalize_s2, dim3(1), dim3(1), 0, stream, acc, amax_out);
    return hipGetLastError();
}

hipError_t launch_quantize(const uint16_t* w, int64_t rows, int64_t cols, const float* m,
                           const float* q, const float* s2, uint8_t* codes, uint8_t* scales,
                           uint16_t* wdeq, hipStream_t stream) {
    const int64_t nblk = rows * (cols / 16);
    const dim3 grid(grid_for(nblk)), block(kThreads);
    auto W = reinterpret_cast<const uint4*>(w);
    auto Q = reinterpret_cast<const float2*>(q);
    auto C = reinterpret_cast<uint2*>(codes);
    auto D = reinterpret_cast<uint4*>(wdeq);
    const int key = (m ? 4 : 0) | (q ? 2 : 0) | (wdeq ? 1 : 0);
    switch (key) {
#define FOCUS_Q_CASE(K, HM, HQ, DQ)                                                             \
    case K:                                                                                     \
        hipLaunchKernelGGL((k_quantize<HM, HQ, DQ>), grid, block, 0, stream, W, m, Q, s2, C,   \
                           scales, D, nblk);                                                    \
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

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* s2,
                             int s2_per_row, int64_t rows, int64_t cols, uint16_t* out,
                             hipStream_t stream) {
    const int64_t nb = cols / 16, nblk = rows * nb;
    const dim3 grid(grid_for(nblk)), block(kThreads);
    auto C = reinterpret_cast<const uint2*>(codes);
    auto O = reinterpret_cast<uint4*>(out);
    if (s2_per_row)
        hipLaunchKernelGGL(k_dequantize<true>, grid, block, 0, stream, C, scales, s2, nblk, nb, O);
    else
        hipLaunchKernelGGL(k_dequantize<false>, grid, block, 0, stream, C, scales, s2, nblk, nb, O);
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
