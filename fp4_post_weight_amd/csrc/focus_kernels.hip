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

//
// The same streaming kernels also carry the adjacent formats, selected at
// compile time: FourOverSix (each 16-block's scale maps its maximum to 6 or 4,
// whichever gives the lower binary32 squared error; "FOCUS NVFP4 scales ...",
// sections "Calibration" and "Perplexity"), FOCUS on MXFP4 (32-blocks with an
// E8M0 scale; the technical summary's section "Methodologie"), and FlipQuant
// MixFP4 (a per-tile map choosing E0M3 levels 0..7 or FourOverSix E2M1;
// "Llama-3.1-8B-Instruct FlipQuant MixFP4 maps", section "What this is").

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "focus_internal.h"
#include "focus_launch.h"
#include "focus_numerics.h"

namespace focus {

constexpr int kThreads = 256;
constexpr int64_t kMaxGrid = 1 << 20;


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
// contiguous store.  PRE: the caller already holds the block maximum
// (block_amax_bits of a, b) and passes it in amax_pre.
template <bool HAS_SIG, bool DEQ, bool PRE = false>
__device__ __forceinline__ void quantize_block(uint4 a, uint4 b, float mb, float q0, float q1,
                                               float s2, double rden, const double* tab,
                                               uint2* codes_out, uint8_t* scale_out, uint4& deq0,
                                               uint4& deq1, float amax_pre = 0.0f) {
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
    const float amax = PRE ? amax_pre : block_amax_bits(a, b);
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

// FourOverSix for one block; same interface as quantize_block (rden6 and
// rden4 are RN64(1/RN32(6*s2)) and RN64(1/RN32(4*s2))).
template <bool DEQ, bool PRE = false>
__device__ __forceinline__ void fo6_block(uint4 a, uint4 b, float s2, double rden6, double rden4,
                                          uint2* codes_out, uint8_t* scale_out, uint4& deq0,
                                          uint4& deq1, float amax_pre = 0.0f) {
    const uint32_t v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    float f[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        f[2 * i] = bf16_lo(v[i]);
        f[2 * i + 1] = bf16_hi(v[i]);
    }
    if (s2 == 0.0f) {
        *scale_out = 0x38;
        st8(codes_out, 0, make_uint2(sign_codes8(a), sign_codes8(b)));
        if (DEQ) {
            const uint32_t z = 0x80008000u;
            deq0 = make_uint4(a.x & z, a.y & z, a.z & z, a.w & z);
            deq1 = make_uint4(b.x & z, b.y & z, b.z & z, b.w & z);
        }
        return;
    }
    const float amax = PRE ? amax_pre : block_amax_bits(a, b);
    const uint32_t sb6 = e4m3_byte_normal(block_t(amax, 1.0f, rden6));
    const uint32_t sb4 = e4m3_byte_normal(block_t(amax, 1.0f, rden4));
    const float S6 = e4m3_normal_value(sb6), S4 = e4m3_normal_value(sb4);
    const float d6 = S6 * s2, d4 = S4 * s2;
    uint32_t c0, c1;
    bool four = false;
    if (sb4 == sb6) {
        // identical candidates: equal errors, and a tie keeps 6
        c0 = encode8(f, d6);
        c1 = encode8(f + 8, d6);
    } else if (s2 >= kFo6S2Lo && s2 <= kFo6S2Hi) {
        const double r6 = recip_f64((double)d6), r4 = recip_f64((double)d4);
        float e6a = 0.0f, e6b = 0.0f, e4a = 0.0f, e4b = 0.0f;
        const uint32_t c60 = fo6_encode8_est(f, r6, e6a), c61 = fo6_encode8_est(f + 8, r6, e6b);
        const uint32_t c40 = fo6_encode8_est(f, r4, e4a), c41 = fo6_encode8_est(f + 8, r4, e4b);
        four = fo6_choose_four(f, s2, S6, d6, c60, c61, e6a + e6b, S4, d4, c40, c41, e4a + e4b);
        c0 = four ? c40 : c60;
        c1 = four ? c41 : c61;
    } else {
        // outside the estimate's proven range: both exact error sums
        const uint32_t c60 = encode8(f, d6), c61 = encode8(f + 8, d6);
        const uint32_t c40 = encode8(f, d4), c41 = encode8(f + 8, d4);
        four = fo6_sq_err(f, c40, c41, S4, s2) < fo6_sq_err(f, c60, c61, S6, s2);
        c0 = four ? c40 : c60;
        c1 = four ? c41 : c61;
    }
    const float S = four ? S4 : S6;
    st8(codes_out, 0, make_uint2(c0, c1));
    *scale_out = (uint8_t)(four ? sb4 : sb6);
    if (DEQ) {
        deq0 = dequant8(c0, S, s2);
        deq1 = dequant8(c1, S, s2);
    }
}

// FlipQuant MixFP4 E0M3 block: the scale maps the block maximum to 7
// (rden7 = RN64(1/RN32(7*s2))), codes are the signed levels 0..7; same
// interface as fo6_block.
template <bool DEQ>
__device__ __forceinline__ void e0m3_block(uint4 a, uint4 b, float s2, double rden7,
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
        *scale_out = 0x38;
        st8(codes_out, 0, make_uint2(sign_codes8(a), sign_codes8(b)));
        if (DEQ) {
            const uint32_t z = 0x80008000u;
            deq0 = make_uint4(a.x & z, a.y & z, a.z & z, a.w & z);
            deq1 = make_uint4(b.x & z, b.y & z, b.z & z, b.w & z);
        }
        return;
    }
    const uint32_t sb = e4m3_byte_normal(block_t(block_amax_bits(a, b), 1.0f, rden7));
    const float S = e4m3_normal_value(sb);
    const float d = S * s2;
    const uint32_t c0 = encode8_e0m3(f, d);
    const uint32_t c1 = encode8_e0m3(f + 8, d);
    st8(codes_out, 0, make_uint2(c0, c1));
    *scale_out = (uint8_t)sb;
    if (DEQ) {
        deq0 = dequant8_e0m3(c0, S, s2);
        deq1 = dequant8_e0m3(c1, S, s2);
    }
}

// One 16-element half of an MXFP4 32-block whose scale S (a power of two) is
// already known: the codes of its two relaxed 8-element sub-blocks (q0, q1),
// w' = BF16(c*S).  Same interface as quantize_block otherwise.
template <bool HAS_SIG, bool DEQ>
__device__ __forceinline__ void mx_half_block(uint4 a, uint4 b, float S, float q0, float q1,
                                              const double* tab, uint2* codes_out, uint4& deq0,
                                              uint4& deq1) {
    const uint32_t v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    float f[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        f[2 * i] = bf16_lo(v[i]);
        f[2 * i + 1] = bf16_hi(v[i]);
    }
    float sig0 = 1.0f, sig1 = 1.0f;
    if (HAS_SIG) {
        sig0 = sigmoid_cr(q0, tab);
        sig1 = sigmoid_cr(q1, tab);
    }
    const uint32_t c0 = encode8(f, S * sig0);
    const uint32_t c1 = encode8(f + 8, S * sig1);
    st8(codes_out, 0, make_uint2(c0, c1));
    if (DEQ) {
        deq0 = dequant8(c0, S, 1.0f);
        deq1 = dequant8(c1, S, 1.0f);
    }
}

// Maximum of two lanes' values within each lane pair (2j, 2j+1): DPP
// quad permutation [1, 0, 3, 2].
__device__ __forceinline__ uint32_t pair_max_u32(uint32_t v) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
    return max(v, o);
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

// Blocks per lane per tile (loads in flight per lane).  Measured on the 8B
// set: plain NVFP4 without w' streams best with 3 (2: 69.6 %, 3: 71.8 %,
// 4: 70.5 %, 6: 69.1 %, 8: 68.1 % of peak); MXFP4 with w' with 1 (56
// VGPRs, eight wavefronts per SIMD: 6.15 against 6.34 ms with 2 blocks and
// 6.55 with 3, medians of four interleaved runs on one box, identical
// outputs); NVFP4 with w' with 2 (1 block was 1 % faster back to back but
// not in the step, where each launch follows the tensor scale: 0.897 and
// 0.912 against 0.893 and 0.895 ms per launch, alternated runs on one box);
// MixFP4 with w' with 3 at four wavefronts per SIMD (127 VGPRs: 6.47
// against 6.60 ms with 1 block at five wavefronts, 6.75 with 2 at four and
// 6.95 with 4 at three, medians of four interleaved runs, identical
// outputs), FourOverSix
// without w' with 5 at four wavefronts per SIMD (the arithmetic of a block
// is long, so more of the next blocks' loads are in flight while it runs:
// 3.82 against 3.96 ms with 2 blocks at five wavefronts, medians of four
// interleaved runs on the same box, identical outputs; 4 blocks 3.84, 6 and
// 8 at three wavefronts 3.93 and 3.91, 1 block 50-70 % slower), every other
// variant with 2 (FourOverSix with w', MXFP4 and MixFP4 without; MXFP4
// without w' at 3 was no faster, NVFP4 without w' at 1 or 2 5 and 3 %
// slower than at 3).
template <bool DEQ, int MODE>
struct QuantU {
    static constexpr int value = DEQ ? (MODE <= 1 ? 2 : MODE == 2 ? 1 : 3) : MODE == 0 ? 3 : MODE == 1 ? 5 : 2;
};

// FlipQuant MixFP4: is block `blk` of tensor j in an E0M3 tile?  block ->
// (row, block in row) -> (tile row, tile column) with the batch's div_magic
// multipliers; every index is below 2^31 (checked on the host).
template <typename Batch>
__device__ __forceinline__ bool mix_block_is_e0m3(const Batch& bt, int j, int64_t blk, uint32_t nb_row) {
    const uint32_t ub = (uint32_t)blk, sh = bt.sh[j];
    const uint32_t r = div_magic(ub, bt.mul[j][0], sh & 255u);
    const uint32_t b = ub - r * nb_row;
    const uint32_t tr = div_magic(r, bt.mul[j][1], (sh >> 8) & 255u);
    const uint32_t tc = div_magic(b, bt.mul[j][2], sh >> 16);
    return bt.map[j][tr * bt.tiles_per_row[j] + tc] != 0;
}

// MODE 0: FOCUS NVFP4; 1: FourOverSix (m, q absent); 2: FOCUS on MXFP4 (lanes
// 2j and 2j+1 share one 32-block: m[blk/2], scale byte stored by the even
// lane, no tensor scale); 3: FlipQuant MixFP4 (Batch = MixBatch; each block
// looks up its tile's map byte: E0M3 if set, FourOverSix otherwise).
// Minimum wavefronts per SIMD the register allocation must allow (1: no
// limit).  FourOverSix codes-only with 5 blocks per lane fits 128 VGPRs
// without spilling (4 wavefronts; with 2 blocks it fit 96 VGPRs and 5
// wavefronts, which beat 4 at that block count: 1.12 against 1.15-1.18 ms on
// 64 linears of the 8B set).  MixFP4 with w' at 3 blocks per lane fits 127
// VGPRs (4 wavefronts).  With w' and two blocks per lane the FourOverSix and
// MixFP4 kernels spill at five wavefronts and were 25 % slower.
template <bool DEQ, int MODE>
struct QuantWaves {
    static constexpr int value = (MODE == 1 && !DEQ) || (MODE == 3 && DEQ) ? 4 : 1;
};

template <bool HAS_M, bool HAS_Q, bool DEQ, int MODE = 0, typename Batch = QuantBatch>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(QuantWaves<DEQ, MODE>::value)))
void k_quantize(Batch bt, int64_t ntiles) {
    constexpr bool FO6 = MODE == 1 || MODE == 3, MX = MODE == 2, MIX = MODE == 3;
    constexpr int kQuantU = QuantU<DEQ, MODE>::value;
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
        const float s2 = MX ? 1.0f : ld_uniform(bt.s2[j]);
        const double rden = MX ? 0.0 : 1.0 / (double)(6.0f * s2);
        const double rden4 = FO6 ? 1.0 / (double)(4.0f * s2) : 0.0;
        const double rden7 = MIX ? 1.0 / (double)(7.0f * s2) : 0.0;
        const int64_t nblk = bt.nblk[j];
        const int64_t tile0 = (tile - bt.tile_start[j]) * (int64_t)kThreads * kQuantU;
        uint4 va[kQuantU] = {}, vb[kQuantU] = {};
        float mb[kQuantU];
        float2 qq[kQuantU];
        bool e0[kQuantU] = {};
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
                mb[k] = HAS_M ? ld4f(m, MX ? blk >> 1 : blk) : 1.0f;
                qq[k] = HAS_Q ? ld8f(q, blk) : make_float2(0.0f, 0.0f);
                if constexpr (MIX) e0[k] = mix_block_is_e0m3(bt, j, blk, bt.nb_row[j]);
            }
        }
#pragma unroll
        for (int k = 0; k < kQuantU; ++k) {
            const int64_t first = tile0 + (int64_t)k * kThreads + wave * 64;  // block of lane 0
            const int64_t blk = first + lane;
            if (kLdsLoadW && first < nblk) wave_gather_blocks(va[k], vb[k], xchw[wave], lane);
            uint4 d0 = make_uint4(0, 0, 0, 0), d1 = d0;
            uint32_t mx_sb = 0;
            if (MX) {  // all lanes: the pair exchange needs both partners
                const uint32_t am = pair_max_u32(__float_as_uint(block_amax_bits(va[k], vb[k])));
                mx_sb = mx_scale_byte(__uint_as_float(am) * (blk < nblk ? mb[k] : 1.0f));
            }
            if (blk < nblk) {
                if (MX) {
                    mx_half_block<HAS_Q, DEQ>(va[k], vb[k], e8m0_value(mx_sb), qq[k].x, qq[k].y, tab,
                                              bt.codes[j] + blk, d0, d1);
                    if ((lane & 1) == 0) bt.scales[j][blk >> 1] = (uint8_t)mx_sb;
                } else if (MIX && e0[k])
                    e0m3_block<DEQ>(va[k], vb[k], s2, rden7, bt.codes[j] + blk, bt.scales[j] + blk,
                                    d0, d1);
                else if (FO6)
                    fo6_block<DEQ>(va[k], vb[k], s2, rden, rden4, bt.codes[j] + blk,
                                   bt.scales[j] + blk, d0, d1);
                else
                    quantize_block<HAS_Q, DEQ>(va[k], vb[k], mb[k], qq[k].x, qq[k].y, s2, rden, tab,
                                               bt.codes[j] + blk, bt.scales[j] + blk, d0, d1);
            }
            if (DEQ && first < nblk)
                wave_store_blocks(bt.wdeq[j] + 2 * first, d0, d1, xch[DEQ ? wave : 0], lane,
                                  nblk - first);
        }
    }
}

// ---------------------------------------------------------------------------
// focus_dequantize(_many): one lane per block
// ---------------------------------------------------------------------------

// Blocks per lane per tile.  Measured on the 8B set (codes and scales in,
// BF16 out): 1 block 2.82 ms, 2 blocks 2.96, 4 blocks 3.08, 8 blocks 3.28
// (medians of four interleaved runs on one box, identical outputs).
constexpr int kDeqU = 1;
constexpr int64_t kDeqTile = (int64_t)kThreads * kDeqU;

// MODE 0: NVFP4; 1: MXFP4 (E8M0 scale byte per 32 elements, i.e. per pair of
// 16-element blocks, no s2); 2: FlipQuant MixFP4 (Batch = MixDequantBatch;
// blocks of E0M3 tiles decode their codes as levels 0..7).
template <int MODE, typename Batch = DequantBatch>
__global__ __launch_bounds__(kThreads) void k_dequantize(Batch bt, int64_t ntiles) {
    constexpr bool MX = MODE == 1, MIX = MODE == 2;
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
        uint2 c[kDeqU];
        uint32_t sb[kDeqU];
        float s2v[kDeqU];
#pragma unroll
        for (int k = 0; k < kDeqU; ++k) {
            const int64_t blk = tile0 + (int64_t)k * kThreads + threadIdx.x;
            if (blk < nblk) {
                c[k] = ld8u(codes, blk);
                sb[k] = scales[MX ? blk >> 1 : blk];
            }
        }
        if (MX) {
#pragma unroll
            for (int k = 0; k < kDeqU; ++k) s2v[k] = 1.0f;
        } else if (per_row) {  // uniform branch: one s2 per row (activations)
#pragma unroll
            for (int k = 0; k < kDeqU; ++k) {
                const int64_t blk = tile0 + (int64_t)k * kThreads + threadIdx.x;
                if (blk < nblk) s2v[k] = s2p[blk / nb_row];
            }
        } else {
            const float s2u = ld_uniform(s2p);
#pragma unroll
            for (int k = 0; k < kDeqU; ++k) s2v[k] = s2u;
        }
#pragma unroll
        for (int k = 0; k < kDeqU; ++k) {
            const int64_t first = tile0 + (int64_t)k * kThreads + wave * 64;
            const int64_t blk = first + lane;
            uint4 d0 = make_uint4(0, 0, 0, 0), d1 = d0;
            if (blk < nblk) {
                const float S = MX ? e8m0_value(sb[k]) : e4m3_any_value(sb[k]);
                bool e0 = false;
                if constexpr (MIX) e0 = mix_block_is_e0m3(bt, j, blk, (uint32_t)nb_row);
                if (e0) {
                    d0 = dequant8_e0m3(c[k].x, S, s2v[k]);
                    d1 = dequant8_e0m3(c[k].y, S, s2v[k]);
                } else {
                    d0 = dequant8(c[k].x, S, s2v[k]);
                    d1 = dequant8(c[k].y, S, s2v[k]);
                }
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

constexpr int kAmaxVecPerThread = 4;                                  // 16-byte vectors per lane per tile
constexpr int64_t kAmaxTile = (int64_t)kThreads * kAmaxVecPerThread;  // vectors per tile (16 KB)
constexpr int64_t kAmaxGrid = 1024;                                   // workgroups per launch (at most)

__device__ __forceinline__ u16x2 max_mag2(u16x2 acc, uint32_t v) {
    return __builtin_elementwise_max(acc, __builtin_bit_cast(u16x2, v & 0x7FFF7FFFu));
}

// Grid-stride over the batch's 16 KB tiles laid end to end: workgroup g
// takes tiles g, g + grid, ..., so the grid sweeps one window of memory at a
// time (measured: 82 % of peak on the 8B set against 79 % for contiguous
// per-workgroup ranges) and each workgroup meets the tensors in increasing
// order (it walks the tensors in turn and computes its first tile in each,
// so no tile searches for its tensor).  A wavefront keeps its running
// maximum in registers and, leaving a tensor, reduces it and parks it in
// LDS; at the end one thread per tensor
// combines the four wavefronts and raises the tensor's accumulator -- the s2
// slot itself, holding the bits of a non-negative binary32 (the BF16
// magnitude shifted up), which an integer atomic max orders exactly.  The
// accumulator is read first: it only grows, so any value read is a lower
// bound, and the atomic is skipped when it cannot raise it (one atomic per
// tile visit would serialize on the 32 addresses).  Loads are nontemporal:
// the weights are read once.
__global__ __launch_bounds__(kThreads) void k_amax(ScaleBatch bt) {
    constexpr int U = kAmaxVecPerThread;
    constexpr int64_t kTV = kAmaxTile;
    __shared__ uint32_t part[kThreads / 64][kBatch];
    const int wave = threadIdx.x >> 6;
    for (int j = threadIdx.x; j < (kThreads / 64) * kBatch; j += kThreads) (&part[0][0])[j] = 0;
    __syncthreads();
    // Workgroup g visits tiles g, g + grid, ... in increasing order, so the
    // tile where its run in tensor j - 1 stops is its first tile in a later
    // tensor: walking the tensors in turn, no tile searches for its tensor.
    const int64_t grid = gridDim.x;
    int64_t t = blockIdx.x;
    for (int j = 0; j < bt.n; ++j) {
        const int64_t t_lo = bt.tile_start[j], t_hi = bt.tile_start[j + 1];
        if (t >= t_hi) continue;  // uniform per workgroup: no tile of tensor j here
        const uint16_t* __restrict__ w16 = bt.w[j];
        const u32x4* __restrict__ w = reinterpret_cast<const u32x4*>(w16);
        const int64_t numel = bt.numel[j];
        const int64_t nvec = numel / 8;
        u16x2 mx = {0, 0};
        for (; t < t_hi; t += grid) {
            const int64_t base = (t - t_lo) * kTV + threadIdx.x;
            u32x4 v[U];
#pragma unroll
            for (int k = 0; k < U; ++k) {
                const int64_t i = base + (int64_t)k * kThreads;
                v[k] = i < nvec ? __builtin_nontemporal_load(w + i) : u32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int k = 0; k < U; ++k)
                mx = max_mag2(max_mag2(max_mag2(max_mag2(mx, v[k].x), v[k].y), v[k].z), v[k].w);
            // the last numel % 8 elements, by the lane that would have loaded
            // vector nvec
#pragma unroll
            for (int k = 0; k < U; ++k) {
                if (base + (int64_t)k * kThreads == nvec) {
                    for (int64_t e = nvec * 8; e < numel; ++e) mx = max_mag2(mx, (uint32_t)w16[e]);
                }
            }
        }
        part[wave][j] = wave_max_u32(max((uint32_t)mx[0], (uint32_t)mx[1])) << 16;
    }
    __syncthreads();
    if (threadIdx.x < bt.n) {
        const int j = threadIdx.x;
        uint32_t m = part[0][j];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) m = max(m, part[w][j]);
        uint32_t* acc = reinterpret_cast<uint32_t*>(bt.s2[j]);
        if (m > __hip_atomic_load(acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(acc, m);
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
// focus_quantize_act_per_token: a wavefront quantizes whole token rows
// ---------------------------------------------------------------------------

constexpr int kActWaves = 4;  // wavefronts per workgroup
constexpr bool kActGather = true;

__device__ __forceinline__ float wave_max_f32(float v) {
    // non-negative binary32: integer order equals value order
    return __uint_as_float(wave_max_u32(__float_as_uint(v)));
}

// RB > 0: lane keeps up to RB blocks of the row in registers (rows of at most
// 64*RB blocks).  RB == 0: rows of any length, read twice (the second read
// hits the caches).
template <int RB, bool DEQ, bool FO6 = false>
__global__ __launch_bounds__(64 * kActWaves) void k_act(const uint4* __restrict__ x, int64_t tokens,
                                                  int64_t nb, uint2* __restrict__ codes,
                                                  uint8_t* __restrict__ scales,
                                                  float* __restrict__ s2out,
                                                  uint4* __restrict__ xdeq) {
    __shared__ uint4 xch[DEQ || kActGather ? kActWaves : 1][128];
    const int lane = threadIdx.x & 63;
    // rows strided over the grid's wavefronts (uniform per wavefront; nothing
    // below synchronizes the workgroup)
    for (int64_t row = (int64_t)blockIdx.x * kActWaves + (threadIdx.x >> 6); row < tokens;
         row += (int64_t)gridDim.x * kActWaves) {
        const int64_t base = row * nb;
        float amax = 0.0f;
        constexpr int R = RB > 0 ? RB : 1;
        uint4 va[R], vb[R];
        float bam[R];  // block maxima, kept for the quantize pass
        if (RB > 0 && kActGather && nb % 64 == 0) {
            // contiguous 1 KB per load instruction, regrouped through LDS so
            // that lane l holds block 64 k + l
            uint4* xg = xch[threadIdx.x >> 6];
#pragma unroll
            for (int k = 0; k < R; ++k) {
                if (64 * k < nb) {
                    va[k] = x[2 * (base + 64 * k) + lane];
                    vb[k] = x[2 * (base + 64 * k) + 64 + lane];
                }
            }
#pragma unroll
            for (int k = 0; k < R; ++k) {
                if (64 * k < nb) {
                    wave_gather_blocks(va[k], vb[k], xg, lane);
                    bam[k] = block_amax_bits(va[k], vb[k]);
                    amax = fmaxf(amax, bam[k]);
                }
            }
        } else if (RB > 0) {
#pragma unroll
            for (int k = 0; k < R; ++k) {
                const int64_t j = lane + 64 * k;
                if (j < nb) {
                    va[k] = x[2 * (base + j)];
                    vb[k] = x[2 * (base + j) + 1];
                    bam[k] = block_amax_bits(va[k], vb[k]);
                    amax = fmaxf(amax, bam[k]);
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
        const double rden4 = FO6 ? 1.0 / (double)(4.0f * s2) : 0.0;
        uint4* xw = xch[DEQ || kActGather ? (threadIdx.x >> 6) : 0];
        if (RB > 0) {
#pragma unroll
            for (int k = 0; k < R; ++k) {
                const int64_t j0 = 64 * k, j = j0 + lane;
                uint4 d0 = make_uint4(0, 0, 0, 0), d1 = d0;
                if (j < nb) {
                    if (FO6)
                        fo6_block<DEQ, true>(va[k], vb[k], s2, rden, rden4, codes + base + j,
                                             scales + base + j, d0, d1, bam[k]);
                    else
                        quantize_block<false, DEQ, true>(va[k], vb[k], 1.0f, 0.0f, 0.0f, s2, rden, nullptr,
                                                         codes + base + j, scales + base + j, d0, d1,
                                                         bam[k]);
                }
                if (DEQ && j0 < nb) wave_store_blocks(xdeq + 2 * (base + j0), d0, d1, xw, lane, nb - j0);
            }
        } else {
            for (int64_t j0 = 0; j0 < nb; j0 += 64) {
                const int64_t j = j0 + lane;
                uint4 d0 = make_uint4(0, 0, 0, 0), d1 = d0;
                if (j < nb) {
                    if (FO6)
                        fo6_block<DEQ>(x[2 * (base + j)], x[2 * (base + j) + 1], s2, rden, rden4,
                                       codes + base + j, scales + base + j, d0, d1);
                    else
                        quantize_block<false, DEQ>(x[2 * (base + j)], x[2 * (base + j) + 1], 1.0f, 0.0f,
                                                   0.0f, s2, rden, nullptr, codes + base + j,
                                                   scales + base + j, d0, d1);
                }
                if (DEQ) wave_store_blocks(xdeq + 2 * (base + j0), d0, d1, xw, lane, nb - j0);
            }
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
    hipError_t e = launch(k_clear_acc, dim3(1), dim3(kBatch), stream, bt);
    if (e == hipSuccess) e = launch(k_amax, dim3((unsigned)g), dim3(kThreads), stream, bt);
    if (e == hipSuccess) e = launch(k_finalize_s2, dim3(1), dim3(kBatch), stream, bt);
    return e;
}

hipError_t launch_quantize(QuantBatch& bt, int key, hipStream_t stream) {
    // keys 0-7: plain NVFP4 (bit 0: w'), 8-9: FourOverSix, 16-23: MXFP4; the
    // tile of the kernel the key selects is kThreads * QuantU blocks
    const bool dq = key & 1;
    const int mode = key < 8 ? 0 : key < 16 ? 1 : 2;
    const int u = mode == 0 ? (dq ? QuantU<true, 0>::value : QuantU<false, 0>::value)
                : mode == 1 ? (dq ? QuantU<true, 1>::value : QuantU<false, 1>::value)
                            : (dq ? QuantU<true, 2>::value : QuantU<false, 2>::value);
    const int64_t tb = (int64_t)kThreads * u;
    int64_t t = 0;
    for (int j = 0; j < bt.n; ++j) {
        bt.tile_start[j] = t;
        t += (bt.nblk[j] + tb - 1) / tb;
    }
    bt.tile_start[bt.n] = t;
    const dim3 grid(grid_for_tiles(t)), block(kThreads);
    switch (key) {
#define FOCUS_Q_CASE(K, HM, HQ, DQ) \
    case K: return launch(&k_quantize<HM, HQ, DQ>, grid, block, stream, bt, t);
        FOCUS_Q_CASE(0, false, false, false)
        FOCUS_Q_CASE(1, false, false, true)
        FOCUS_Q_CASE(2, false, true, false)
        FOCUS_Q_CASE(3, false, true, true)
        FOCUS_Q_CASE(4, true, false, false)
        FOCUS_Q_CASE(5, true, false, true)
        FOCUS_Q_CASE(6, true, true, false)
        FOCUS_Q_CASE(7, true, true, true)
#undef FOCUS_Q_CASE
        case 8: return launch(&k_quantize<false, false, false, 1>, grid, block, stream, bt, t);
        case 9: return launch(&k_quantize<false, false, true, 1>, grid, block, stream, bt, t);
#define FOCUS_MX_CASE(K, HM, HQ, DQ) \
    case 16 + K: return launch(&k_quantize<HM, HQ, DQ, 2>, grid, block, stream, bt, t);
        FOCUS_MX_CASE(0, false, false, false)
        FOCUS_MX_CASE(1, false, false, true)
        FOCUS_MX_CASE(2, false, true, false)
        FOCUS_MX_CASE(3, false, true, true)
        FOCUS_MX_CASE(4, true, false, false)
        FOCUS_MX_CASE(5, true, false, true)
        FOCUS_MX_CASE(6, true, true, false)
        FOCUS_MX_CASE(7, true, true, true)
#undef FOCUS_MX_CASE
    }
    return hipErrorInvalidValue;
}

hipError_t launch_quantize_mix(MixBatch& bt, bool deq, hipStream_t stream) {
    const int64_t tb = (int64_t)kThreads * (deq ? QuantU<true, 3>::value : QuantU<false, 3>::value);
    int64_t t = 0;
    for (int j = 0; j < bt.n; ++j) {
        bt.tile_start[j] = t;
        t += (bt.nblk[j] + tb - 1) / tb;
    }
    bt.tile_start[bt.n] = t;
    const dim3 grid(grid_for_tiles(t)), block(kThreads);
    if (deq) return launch(&k_quantize<false, false, true, 3, MixBatch>, grid, block, stream, bt, t);
    return launch(&k_quantize<false, false, false, 3, MixBatch>, grid, block, stream, bt, t);
}

hipError_t launch_dequantize(DequantBatch& bt, bool mx, hipStream_t stream) {
    int64_t t = 0;
    for (int j = 0; j < bt.n; ++j) {
        bt.tile_start[j] = t;
        t += (bt.nblk[j] + kDeqTile - 1) / kDeqTile;
    }
    bt.tile_start[bt.n] = t;
    const dim3 grid(grid_for_tiles(t)), block(kThreads);
    if (mx) return launch(&k_dequantize<1>, grid, block, stream, bt, t);
    return launch(&k_dequantize<0>, grid, block, stream, bt, t);
}

hipError_t launch_dequantize_mix(MixDequantBatch& bt, hipStream_t stream) {
    int64_t t = 0;
    for (int j = 0; j < bt.n; ++j) {
        bt.tile_start[j] = t;
        t += (bt.nblk[j] + kDeqTile - 1) / kDeqTile;
    }
    bt.tile_start[bt.n] = t;
    return launch(&k_dequantize<2, MixDequantBatch>, dim3(grid_for_tiles(t)), dim3(kThreads), stream, bt, t);
}

hipError_t launch_act_per_token(const uint16_t* x, int64_t tokens, int64_t hidden, uint8_t* codes,
                                uint8_t* scales, float* s2_out, uint16_t* xdeq, bool fo6,
                                hipStream_t stream) {
    const int64_t nb = hidden / 16;
    // Two rows per wavefront, taken in turn, but no fewer than 1024
    // workgroups while there are rows for them.  Measured on X [T, 4096]:
    // 17.2 us at T = 8192 and 125 us at 65536 against 19.1 and 129 us with
    // one row per wavefront; 16 or more rows per wavefront were slower.
    // FourOverSix likewise: 400 us at T = 131072 against 421 us with one row
    // per wavefront (31.5 against 30.9 us at T = 8192).  Issuing the second
    // row's loads before quantizing the first was slower (25 us at 8192).
    const int64_t g1 = (tokens + kActWaves - 1) / kActWaves;
    int64_t g = (tokens + 2 * kActWaves - 1) / (2 * kActWaves);
    if (g < 1024) g = g1 < 1024 ? g1 : 1024;
    const dim3 grid((unsigned)g), block(64 * kActWaves);
    auto X = reinterpret_cast<const uint4*>(x);
    auto C = reinterpret_cast<uint2*>(codes);
    auto D = reinterpret_cast<uint4*>(xdeq);
#define FOCUS_ACT_F(RB, F)                                                                          \
    return xdeq ? launch(&k_act<RB, true, F>, grid, block, stream, X, tokens, nb, C, scales, s2_out, D) \
                : launch(&k_act<RB, false, F>, grid, block, stream, X, tokens, nb, C, scales, s2_out, D)
#define FOCUS_ACT(RB)                      \
    do {                                   \
        if (fo6) FOCUS_ACT_F(RB, true);    \
        FOCUS_ACT_F(RB, false);            \
    } while (0)
    if (nb <= 64) FOCUS_ACT(1);
    if (nb <= 128) FOCUS_ACT(2);
    if (nb <= 256) FOCUS_ACT(4);
    if (nb <= 512) FOCUS_ACT(8);
    FOCUS_ACT(0);
#undef FOCUS_ACT
#undef FOCUS_ACT_F
}

}  // namespace focus
