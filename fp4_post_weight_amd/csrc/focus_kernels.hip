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
    const float amax = block_amax_bits(a, b);
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
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int j = find_tensor(bt.tile_start, bt.n, tile);
        const uint4* __restrict__ w = bt.w[j];
        const float* __restrict__ m = bt.m[j];
        const float2* __restrict__ q = bt.q[j];
        const float s2 = *bt.s2[j];
        const float den = 6.0f * s2;
        const int64_t nblk = bt.nblk[j];
        const int64_t base = (tile - bt.tile_start[j]) * kQuantTile + threadIdx.x;
        uint4 va[kQuantU], vb[kQuantU];
        float mb[kQuantU];
        float2 qq[kQuantU];
#pragma unroll
        for (int k = 0; k < kQuantU; ++k) {
            const int64_t blk = base + (int64_t)k * kThreads;
            if (blk < nblk) {
                va[k] = w[2 * blk];
                vb[k] = w[2 * blk + 1];
                mb[k] = HAS_M ? m[blk] : 1.0f;
                qq[k] = HAS_Q ? q[blk] : make_float2(0.0f, 0.0f);
            }
        }
#pragma unroll
        for (int k = 0; k < kQuantU; ++k) {
            const int64_t blk = base + (int64_t)k * kThreads;
            if (blk < nblk)
                quantize_block<HAS_Q, DEQ>(va[k], vb[k], mb[k], qq[k].x, qq[k].y, s2, den,
                                           bt.codes[j] + blk, bt.scales[j] + blk,
                                           DEQ ? bt.wdeq[j] + 2 * blk : nullptr);
        }
    }
}

// ---------------------------------------------------------------------------
// focus_dequantize(_many): one lane per block
// ---------------------------------------------------------------------------

constexpr int64_t kDeqTile = (int64_t)kThreads * 2;

__global__ __launch_bounds__(kThreads) void k_dequantize(DequantBatch bt, int64_t ntiles) {
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int j = find_tensor(bt.tile_start, bt.n, tile);
        const uint2* __restrict__ codes = bt.codes[j];
        const uint8_t* __restrict__ scales = bt.scales[j];
        const float* __restrict__ s2p = bt.s2[j];
        const int64_t nblk = bt.nblk[j], nb_row = bt.nb_row[j];
        const bool per_row = bt.per_row[j] != 0;
        const int64_t base = (tile - bt.tile_start[j]) * kDeqTile + threadIdx.x;
        const float s2u = per_row ? 0.0f : *s2p;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int64_t blk = base + (int64_t)k * kThreads;
            if (blk < nblk) {
                const uint2 c = codes[blk];
                const float S = e4m3_any_value(scales[blk]);
                const float s2 = per_row ? s2p[blk / nb_row] : s2u;
                bt.out[j][2 * blk] = dequant8(c.x, S, s2);
                bt.out[j][2 * blk + 1] = dequant8(c.y, S, s2);
            }
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

constexpr int kAmaxVecPerThread = 8;  // 8 x 16 B per lane per tile
constexpr int64_t kAmaxTile = (int64_t)kThreads * kAmaxVecPerThread;  // in 16-byte vectors

// The accumulator is the s2 slot itself, holding the bits of a non-negative
// binary32 (the BF16 magnitude shifted up); an integer atomic max orders such
// floats exactly.  Each tile covers kAmaxTile 16-byte vectors of one tensor;
// the last partial vector of a tensor is read element by element.
__global__ __launch_bounds__(kThreads) void k_amax(ScaleBatch bt, int64_t ntiles) {
    __shared__ uint32_t part[kThreads / 64];
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int j = find_tensor(bt.tile_start, bt.n, tile);
        const uint16_t* __restrict__ w16 = bt.w[j];
        const uint4* __restrict__ w = reinterpret_cast<const uint4*>(w16);
        const int64_t numel = bt.numel[j];
        const int64_t nvec = numel / 8;
        const int64_t base = (tile - bt.tile_start[j]) * kAmaxTile + threadIdx.x;
        u16x2 mx = {0, 0};
        const uint32_t mask = 0x7FFF7FFFu;
        uint4 v[kAmaxVecPerThread];
#pragma unroll
        for (int k = 0; k < kAmaxVecPerThread; ++k) {
            const int64_t i = base + (int64_t)k * kThreads;
            v[k] = i < nvec ? w[i] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < kAmaxVecPerThread; ++k) {
            u16x2 a = __builtin_bit_cast(u16x2, v[k].x & mask);
            u16x2 b = __builtin_bit_cast(u16x2, v[k].y & mask);
            u16x2 c = __builtin_bit_cast(u16x2, v[k].z & mask);
            u16x2 d = __builtin_bit_cast(u16x2, v[k].w & mask);
            mx = __builtin_elementwise_max(mx, __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                                                         __builtin_elementwise_max(c, d)));
        }
        uint32_t mm = max((uint32_t)mx[0], (uint32_t)mx[1]);
        // the tail (numel % 8 elements) belongs to the tile holding vector nvec
        const int64_t tail_vec_tile = nvec / kAmaxTile;
        if (tile - bt.tile_start[j] == tail_vec_tile && (int)threadIdx.x < (int)(numel - nvec * 8))
            mm = max(mm, (uint32_t)(w16[nvec * 8 + threadIdx.x] & 0x7FFFu));
        mm = wave_max_u32(mm);
        const int wave = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0) part[wave] = mm;
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t r = part[0];
#pragma unroll
            for (int k = 1; k < kThreads / 64; ++k) r = max(r, part[k]);
            atomicMax(reinterpret_cast<uint32_t*>(bt.s2[j]), r << 16);
        }
        __syncthreads();
    }
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

static inline unsigned grid_for_tiles(int64_t ntiles) {
    int64_t g = ntiles < 1 ? 1 : ntiles;
    if (g > kMaxGrid) g = kMaxGrid;
    return (unsigned)g;
}

hipError_t launch_tensor_scale(ScaleBatch& bt, hipStream_t stream) {
    int64_t t = 0;
    for (int j = 0; j < bt.n; ++j) {
        bt.tile_start[j] = t;
        const int64_t nvec = bt.numel[j] / 8;
        t += nvec / kAmaxTile + 1;  // the +1 tile holds the partial vector tail
    }
    bt.tile_start[bt.n] = t;
    hipLaunchKernelGGL(k_clear_acc, dim3(1), dim3(kBatch), 0, stream, bt);
    hipLaunchKernelGGL(k_amax, dim3(grid_for_tiles(t)), dim3(kThreads), 0, stream, bt, t);
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
