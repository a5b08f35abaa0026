// focus_gemm.hip -- the NVFP4 linear layer on gfx950 matrix cores.
//
// What it computes ("FOCUS NVFP4 scales for Llama-3.2-1B-Instruct (our
// reproduction)": section "What this is" -- the deployed model is plain
// NVFP4 and runs on standard NVFP4 kernels -- and section "Perplexity" --
// NVFP4 weights with one FP32 scale per tensor, NVFP4 activations with one
// scale per token):
//     Y[t, o] = s2x[t] * s2w * sum_k (cx[t,k] * Sx[t, k/16]) * (cw[o,k] * Sw[o, k/16])
// with c an E2M1 value and S an E4M3 block scale.
//
// How it maps onto CDNA4:
//  * Each operand element c*S has at most 6 significant bits (a 2-bit E2M1
//    significand times a 4-bit E4M3 one) and is 0 or lies in [2^-10, 2688],
//    so it is exact in FP16, and the product of two such values (at most 12
//    bits) is exact in FP32.  The contraction therefore runs on the FP16
//    matrix cores (v_mfma_f32_32x32x16_f16) with FP32 accumulation, and
//    s2x*s2w is applied once per output.  (gfx950's FP4 matrix instructions
//    take one E8M0 scale per 32 elements; NVFP4's E4M3 scale per 16
//    elements is not expressible there.)
//  * Dequantization costs about one vector operation per element: the
//    scale bytes become FP16 two at a time (v_cvt_scalef32_pk_f16_fp8; every
//    E4M3 value is a normal FP16 number), v_cvt_scalef32_pk_f16_fp4 with
//    scale 1 turns two codes into c, and one packed FP16 multiply gives c*S.
//  * Workgroup tile 256 x 256 x 64 (4 wavefronts, each 128 x 128 = 4 x 4
//    MFMA tiles of 32 x 32, 256 FP32 accumulators per lane).  Both operand
//    tiles are dequantized once per workgroup into FP16 in LDS (rows padded
//    to 144 bytes) in two stages: while the matrix cores consume one k-step,
//    the codes of the next step (loaded into registers one step earlier)
//    are dequantized into the other stage, and the step after that is being
//    loaded.  Fragments are read two k16 slices ahead, the dequantization
//    runs in slices 0-1 interleaved with the matrix instructions, and the
//    one barrier per step sits after slice 1, so slices 2-3 cover the reads
//    of the next step's first fragments.  Measured, the matrix cores are
//    busy a little under half of the cycles, and the LDS operand traffic
//    (about 192 KB per step and CU) is the main limit: timing-only copies of
//    this kernel without the dequantization, the streaming loads and the
//    barrier were only 9 % faster, without any LDS access 30 % faster still,
//    while bare back-to-back matrix instructions of one wavefront per SIMD
//    reach about 87 % of the FP16 peak.  Taking W's fragments straight from
//    global memory into each wavefront (half the LDS traffic, twice the
//    dequantization of W) was 12 % slower.  Keeping codes in LDS and
//    dequantizing per wavefront cuts LDS traffic four-fold but doubles the
//    vector work, which lowers the clock under this load; measured, it was
//    slower.  Eight wavefronts of 128 x 64 (two per SIMD, with a prefetch
//    two steps deep) measured no faster either.
//  * The step loop runs two steps per iteration with the chunk registers
//    swapping roles: a register copy of a chunk still being loaded would
//    make every step wait for the loads it has just issued.
//  * Loads are straight-line in the common case (K % 64 == 0, aligned): a
//    row past the end of X or W reads the last row instead; it only feeds
//    outputs that are never stored.
//  * With few tokens (M <= 128) the layer is bound by streaming W, and a
//    decode kernel without shared LDS operand tiles takes over
//    (v_mfma_f32_16x16x32_f16, 1, 2, 4 or 8 tiles of 16 tokens).  When an output
//    has too few columns to fill the GPU, the sum over k is split into ranges
//    whose partials a finalize kernel adds in order.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "focus_gemm.h"
#include "focus_launch.h"
#include "focus_numerics.h"

namespace focus {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kGemmThreads = 256;
constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kWaveM = 128, kWaveN = 128;
constexpr int kTilesM = kWaveM / 32, kTilesN = kWaveN / 32;
constexpr int kLdsStride = kBK + 8;  // halves per LDS row: 144 bytes

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Codes (8 bytes per 16-element block) and scale bytes of one row's k-step:
// four blocks.  Rows beyond `nrows` and blocks beyond K read as zero.
struct RowChunk {
    u32x2 c[4];
    uint32_t s;
};

// FAST: K % 64 == 0, codes 16-byte and scales 4-byte aligned (two 16-byte
// loads and one 4-byte load per row); otherwise one 8-byte load and one byte
// per block.
template <bool FAST>
__device__ __forceinline__ RowChunk load_chunk(const uint8_t* __restrict__ codes,
                                               const uint8_t* __restrict__ scales, int64_t row,
                                               int64_t nrows, int64_t K, int64_t k0) {
    RowChunk r;
    if (FAST) {
        // Unconditional loads: a row beyond the tensor reads the last row
        // (always in bounds; nrows >= 1 here).  Such a row of X only feeds
        // output rows >= M and such a row of W only output columns >= N,
        // which are never stored, so no masking is needed -- and straight-
        // line loads let the wait counters track them exactly.
        const int64_t rr = row < nrows ? row : nrows - 1;
        const uint8_t* cp = codes + rr * (K / 2) + k0 / 2;
        const uint4 v0 = *reinterpret_cast<const uint4*>(cp);
        const uint4 v1 = *reinterpret_cast<const uint4*>(cp + 16);
        r.s = *reinterpret_cast<const uint32_t*>(scales + rr * (K / 16) + k0 / 16);
        r.c[0] = (u32x2){v0.x, v0.y};
        r.c[1] = (u32x2){v0.z, v0.w};
        r.c[2] = (u32x2){v1.x, v1.y};
        r.c[3] = (u32x2){v1.z, v1.w};
        return r;
    }
    r.s = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) r.c[b] = (u32x2){0u, 0u};
    if (row >= nrows) return r;
    const uint8_t* cp = codes + row * (K / 2) + k0 / 2;
    const uint8_t* sp = scales + row * (K / 16) + k0 / 16;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        if (k0 + 16 * b < K) {
            r.c[b] = *reinterpret_cast<const u32x2*>(cp + 8 * b);
            r.s |= (uint32_t)sp[b] << (8 * b);
        }
    }
    return r;
}

// E4M3 block scales to FP16, two per instruction: the two bytes of the low
// (HI = false) or high 16-bit half of a scale dword, lower byte first.
// Exact: every E4M3 value, subnormals included, is a normal FP16 number, and
// the NaN bytes 0x7F / 0xFF give NaN.
template <bool HI>
__device__ __forceinline__ f16x2 scale_pair(uint32_t s) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s, 1.0f, HI);
}

// c * S for the eight codes of one dword (element 2j in the low nibble of
// byte j): v_cvt_scalef32_pk_f16_fp4 with scale 1 gives c exactly, and one
// packed FP16 multiply by S gives c * S, also exact (at most 6 significant
// bits; 0 or a magnitude in [2^-10, 2688]).
__device__ __forceinline__ f16x8 codes_times(uint32_t w, _Float16 S) {
    const f16x2 s2 = {S, S};
    const f16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
    const f16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
    const f16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
    const f16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
    return (f16x8){a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
}

// Scale of block b (0-3) of a row's k-step from its two scale pairs.
__device__ __forceinline__ _Float16 block_scale(f16x2 s01, f16x2 s23, int b) {
    return b == 0 ? s01.x : b == 1 ? s01.y : b == 2 ? s23.x : s23.y;
}

// Dword kk (0-3) of a 16-byte vector.
__device__ __forceinline__ uint32_t dword_of(const uint4& v, int kk) {
    return kk == 0 ? v.x : kk == 1 ? v.y : kk == 2 ? v.z : v.w;
}

__device__ __forceinline__ void store_chunk(_Float16* lds_row, const RowChunk& r) {
    const f16x2 s01 = scale_pair<false>(r.s), s23 = scale_pair<true>(r.s);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const _Float16 S = block_scale(s01, s23, b);
        *reinterpret_cast<f16x8*>(lds_row + 16 * b) = codes_times(r.c[b].x, S);
        *reinterpret_cast<f16x8*>(lds_row + 16 * b + 8) = codes_times(r.c[b].y, S);
    }
}

// Fragments of k16-slice kk of the wavefront's 128 rows of one operand tile.
__device__ __forceinline__ void load_frags(f16x8 (&f)[4], const _Float16* tile, int row0, int kk,
                                           int frag_row, int frag_k) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
        f[i] = *reinterpret_cast<const f16x8*>(tile + (row0 + i * 32 + frag_row) * kLdsStride + kk * 16 +
                                               frag_k);
}

template <bool FAST, bool BF16_OUT>
__global__ __launch_bounds__(kGemmThreads) void k_nvfp4_linear(GemmArgs a, int64_t tiles_n) {
    // two stages of both operand tiles: the matrix cores read one while the
    // next k-step is dequantized into the other
    __shared__ _Float16 lds[2][(kBM + kBN) * kLdsStride];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t tile = blockIdx.x;
    const int64_t m0 = (tile / tiles_n) * kBM;
    const int64_t n0 = (tile % tiles_n) * kBN;
    const int frag_row = lane & 31;
    const int frag_k = (lane >> 5) * 8;
    // this workgroup's range of 64-wide k-steps [sb, se)
    const int64_t nsteps_all = (a.K + kBK - 1) / kBK;
    const int64_t sb = (int64_t)blockIdx.y * a.kchunk;
    const int64_t se = sb + a.kchunk < nsteps_all ? sb + a.kchunk : nsteps_all;

    f32x16 acc[kTilesM][kTilesN];
#pragma unroll
    for (int i = 0; i < kTilesM; ++i)
#pragma unroll
        for (int j = 0; j < kTilesN; ++j) acc[i][j] = (f32x16){};

    // thread tid stages row tid of both operand tiles (no steps: nothing to read)
    const int64_t nsteps = se > sb ? se - sb : 0;
    const int64_t mrows = nsteps > 0 ? a.M : 0, nrows = nsteps > 0 ? a.N : 0;
    RowChunk ra = load_chunk<FAST>(a.xc, a.xs, m0 + tid, mrows, a.K, sb * kBK);
    RowChunk rb = load_chunk<FAST>(a.wc, a.ws, n0 + tid, nrows, a.K, sb * kBK);
    store_chunk(lds[0] + tid * kLdsStride, ra);
    store_chunk(lds[0] + (kBM + tid) * kLdsStride, rb);
    if (nsteps > 1) {
        ra = load_chunk<FAST>(a.xc, a.xs, m0 + tid, a.M, a.K, (sb + 1) * kBK);
        rb = load_chunk<FAST>(a.wc, a.ws, n0 + tid, a.N, a.K, (sb + 1) * kBK);
    }
    __syncthreads();
    const int arow = wm * kWaveM, brow = kBM + wn * kWaveN;
    // fragments of the four k16 slices of a step, read two slices ahead
    f16x8 fa0[4], fb0[4], fa1[4], fb1[4], fa2[4], fb2[4], fa3[4], fb3[4];
    load_frags(fa0, lds[0], arow, 0, frag_row, frag_k);
    load_frags(fb0, lds[0], brow, 0, frag_row, frag_k);
    load_frags(fa1, lds[0], arow, 1, frag_row, frag_k);
    load_frags(fb1, lds[0], brow, 1, frag_row, frag_k);

    auto mfma16 = [&](const f16x8 (&fa)[4], const f16x8 (&fb)[4]) {
#pragma unroll
        for (int i = 0; i < kTilesM; ++i)
#pragma unroll
            for (int j = 0; j < kTilesN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    };
    // One k-step s: slices 0 and 1 read the fragments of slices 2 and 3 and
    // dequantize chunk s + 1 (blocks 0-1, then 2-3, both operands) into the
    // other stage; after the barrier, slices 2 and 3 read the next step's
    // slices 0 and 1 from it.  Chunk s + 2 is loaded at the start of the
    // step (clamped to the last chunk so the code stays straight-line).
    // The loop runs two steps per iteration with the chunk registers
    // swapping roles (ra/rb dequantized while na/nb load, then the reverse),
    // so no register copy waits for a load in flight.
    auto step = [&](int64_t s, const RowChunk& ra, const RowChunk& rb, RowChunk& na, RowChunk& nb) {
        const _Float16* cur = lds[s & 1];
        _Float16* nxt = lds[(s + 1) & 1];
        const int64_t kn = (sb + (s + 2 < nsteps ? s + 2 : nsteps - 1)) * kBK;
        na = load_chunk<FAST>(a.xc, a.xs, m0 + tid, a.M, a.K, kn);
        nb = load_chunk<FAST>(a.wc, a.ws, n0 + tid, a.N, a.K, kn);
        const f16x2 xa01 = scale_pair<false>(ra.s), xa23 = scale_pair<true>(ra.s);
        const f16x2 xb01 = scale_pair<false>(rb.s), xb23 = scale_pair<true>(rb.s);
        auto dequant = [&](int b) {
            const _Float16 sa = block_scale(xa01, xa23, b), sbv = block_scale(xb01, xb23, b);
            *reinterpret_cast<f16x8*>(nxt + tid * kLdsStride + 16 * b) = codes_times(ra.c[b].x, sa);
            *reinterpret_cast<f16x8*>(nxt + tid * kLdsStride + 16 * b + 8) = codes_times(ra.c[b].y, sa);
            *reinterpret_cast<f16x8*>(nxt + (kBM + tid) * kLdsStride + 16 * b) = codes_times(rb.c[b].x, sbv);
            *reinterpret_cast<f16x8*>(nxt + (kBM + tid) * kLdsStride + 16 * b + 8) = codes_times(rb.c[b].y, sbv);
        };
        // slice 0
        load_frags(fa2, cur, arow, 2, frag_row, frag_k);
        load_frags(fb2, cur, brow, 2, frag_row, frag_k);
        mfma16(fa0, fb0);
        dequant(0);
        dequant(1);
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int g = 0; g < 16; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
            if (g >= 8) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        // slice 1
        load_frags(fa3, cur, arow, 3, frag_row, frag_k);
        load_frags(fb3, cur, brow, 3, frag_row, frag_k);
        mfma16(fa1, fb1);
        dequant(2);
        dequant(3);
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int g = 0; g < 16; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
            if (g >= 8) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        // the other stage is complete and this stage's reads are done
        __syncthreads();
        // slice 2
        load_frags(fa0, nxt, arow, 0, frag_row, frag_k);
        load_frags(fb0, nxt, brow, 0, frag_row, frag_k);
        mfma16(fa2, fb2);
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
        __builtin_amdgcn_sched_barrier(0);
        // slice 3
        load_frags(fa1, nxt, arow, 1, frag_row, frag_k);
        load_frags(fb1, nxt, brow, 1, frag_row, frag_k);
        mfma16(fa3, fb3);
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    RowChunk na, nb;
    int64_t s = 0;
    for (; s + 1 < nsteps; s += 2) {
        step(s, ra, rb, na, nb);
        step(s + 1, na, nb, ra, rb);
    }
    if (s < nsteps) step(s, ra, rb, na, nb);

    // epilogue: register r of lane l in a 32 x 32 tile holds row
    // 8*(r/4) + 4*(l/32) + r%4 and column l%32; Y = acc * (s2x[row] * s2w),
    // or, with the sum split over k ranges, the unscaled partial of range
    // blockIdx.y
    if (a.ksplit > 1) {
        float* part = a.part + (int64_t)blockIdx.y * a.M * a.N;
#pragma unroll
        for (int i = 0; i < kTilesM; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm * kWaveM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row >= a.M) continue;
#pragma unroll
                for (int j = 0; j < kTilesN; ++j) {
                    const int64_t col = n0 + wn * kWaveN + j * 32 + (lane & 31);
                    if (col < a.N) part[row * a.N + col] = acc[i][j][r];
                }
            }
        return;
    }
    const float s2w = a.ws2[0];
#pragma unroll
    for (int i = 0; i < kTilesM; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t row = m0 + wm * kWaveM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (row >= a.M) continue;
            const float sc = a.xs2[a.xs2_per_row ? row : 0] * s2w;
#pragma unroll
            for (int j = 0; j < kTilesN; ++j) {
                const int64_t col = n0 + wn * kWaveN + j * 32 + (lane & 31);
                if (col >= a.N) continue;
                const float v = acc[i][j][r] * sc;
                if (BF16_OUT) {
                    const uint32_t p = bf16_pair(v, 0.0f);
                    reinterpret_cast<uint16_t*>(a.y)[row * a.N + col] = (uint16_t)(p & 0xFFFFu);
                } else {
                    reinterpret_cast<float*>(a.y)[row * a.N + col] = v;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Decode (M <= 128): v_mfma_f32_16x16x32_f16 on MT = 1, 2, 4 or 8 tiles of
// 16 tokens (every weight element feeds at most 128 outputs, so the layer is
// bound by streaming W, or by the vector work of dequantizing X, and no
// operand needs sharing between wavefronts; with aligned operands and up to
// 4 token tiles each wavefront still passes its W step through an LDS area of
// its own, so that its loads take whole cache lines).  A workgroup of WAVES
// wavefronts owns
// 16 T output columns (16 T rows of W); the 256-wide k-steps of its k range
// are dealt round-robin to its wavefronts, each accumulates MT x T partial
// 16 x 16 tiles (a dequantized W fragment feeds all MT token tiles, an X
// fragment all T column tiles), and one LDS reduction sums the WAVES partial
// tiles in wavefront order (deterministic).
//
// Within a step the sum is order-free, so lane group g = lane / 16 takes k in
// [64g, 64g + 64): 32 contiguous code bytes (blocks 4g..4g+3 of the step) and
// their 4 contiguous scale bytes, and MFMA j (k-depth 32) takes dword j of
// them in both operands.  A wavefront's two 16-byte loads per row cover the
// row's whole 128-byte step; its scale load covers the step's 16 bytes.
//
// Measured on MI355X: the launch and load latency of a few-microsecond kernel
// dominate, so the wavefronts keep one step in flight each and there are
// many of them (8 per workgroup, 16 for long rows with one token tile; 2 or 4
// steps in flight per wavefront, or 16 wavefronts per workgroup elsewhere,
// were slower), and T = 2 (T = 4 with 4 or 8 token tiles) pays only where the
// output still has most of a workgroup per CU with it (X is then read and
// dequantized half or a quarter as often).  Against 32 x 32 tiles with four steps in
// flight per wavefront (its predecessor for 16 < M <= 64), 17 to 64 tokens
// through the Llama-3.1-8B layer shapes took 36-68 us instead of 58-96 us;
// 65 to 128 tokens take about 15 % less time than the tiled kernel's
// 256-row tiles.
// ---------------------------------------------------------------------------

constexpr int kGemvK = 256;          // k per step
constexpr int64_t kGemvMaxM = 128;

struct GemvChunk {
    uint4 c0, c1;  // code bytes [32g, 32g + 32) of the row's step
    uint32_t s;    // scale bytes of blocks 4g..4g+3, lower block first
};

// FAST: K % 256 == 0, codes 16-byte and scales 4-byte aligned; rows past
// `nrows` read the last row (they feed only outputs that are never stored).
// Otherwise rows past `nrows` and blocks past K read as zero.  (Measured on
// MI355X: two 16-byte pieces 64 bytes apart per lane, which let each load
// instruction cover 64 contiguous bytes of a row, and nontemporal loads of
// W were both slower.)
template <bool FAST>
__device__ __forceinline__ GemvChunk load_gemv(const uint8_t* __restrict__ codes,
                                               const uint8_t* __restrict__ scales, int64_t row,
                                               int64_t nrows, int64_t K, int64_t k0, int g) {
    GemvChunk r;
    if (FAST) {
        const int64_t rr = row < nrows ? row : nrows - 1;
        const uint8_t* cp = codes + rr * (K / 2) + k0 / 2 + 32 * g;
        r.c0 = *reinterpret_cast<const uint4*>(cp);
        r.c1 = *reinterpret_cast<const uint4*>(cp + 16);
        r.s = *reinterpret_cast<const uint32_t*>(scales + rr * (K / 16) + k0 / 16 + 4 * g);
        return r;
    }
    r.c0 = make_uint4(0, 0, 0, 0);
    r.c1 = make_uint4(0, 0, 0, 0);
    r.s = 0;
    if (row >= nrows) return r;
    const uint8_t* cp = codes + row * (K / 2) + k0 / 2 + 32 * g;
    const uint8_t* sp = scales + row * (K / 16) + k0 / 16 + 4 * g;
    const int64_t kb = k0 + 64 * g;
    uint2 v[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        v[b] = make_uint2(0, 0);
        if (kb + 16 * b < K) {
            v[b] = *reinterpret_cast<const uint2*>(cp + 8 * b);
            r.s |= (uint32_t)sp[b] << (8 * b);
        }
    }
    r.c0 = make_uint4(v[0].x, v[0].y, v[1].x, v[1].y);
    r.c1 = make_uint4(v[2].x, v[2].y, v[3].x, v[3].y);
    return r;
}

__device__ __forceinline__ uint32_t gemv_dword(const GemvChunk& c, int j) {
    return j < 4 ? dword_of(c.c0, j) : dword_of(c.c1, j - 4);
}

// W's step through the wavefront's own LDS area (FAST loads, at most 4 token
// tiles and 2 column tiles).  In the matrix-instruction layout lanes 0-15
// hold 16 different rows, so each quad of lanes of a direct load touches 4
// cache lines; here 8 lanes load one row's whole 128-byte line (4 lanes its
// 16 scale bytes), rows are stored 144 bytes apart, so that the reads in the
// matrix layout (16 rows, 16 bytes each) hit distinct banks, and read back.
// Measured on the read pattern alone (28672 x 8192): 6.8 against 5.8 TB/s.
constexpr int kStageRow = 144;
template <int T>
struct GemvStage {
    static constexpr int bytes = 16 * T * (kStageRow + 16);  // codes, then 16 scale bytes per row
};

template <bool FAST, bool BF16_OUT, int WAVES, int T, int MT>
__global__ __launch_bounds__(64 * WAVES) void k_nvfp4_linear_gemv(GemmArgs a, GemvMembers mem) {
    constexpr bool kStaged = FAST && MT <= 4 && T <= 2;
    constexpr int kRed = WAVES * MT * T * 256 * 4;
    constexpr int kStage = kStaged ? WAVES * GemvStage<T>::bytes : 0;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kRed > kStage ? kRed : kStage];
    float(*red)[MT * T * 16 * 16] = reinterpret_cast<float(*)[MT * T * 16 * 16]>(lds);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int c16 = lane & 15, g = lane >> 4;
    // the weight (member) this workgroup's columns belong to: members share X
    // and take consecutive ranges of workgroup columns (uniform, scalar)
    int j = 0;
    while (j + 1 < mem.n && (int64_t)blockIdx.x >= mem.tile_start[j + 1]) ++j;
    const uint8_t* __restrict__ wc = mem.wc[j];
    const uint8_t* __restrict__ wsc = mem.ws[j];
    const int64_t N = mem.N[j];
    const int64_t n0 = ((int64_t)blockIdx.x - mem.tile_start[j]) * (16 * T);
    const int64_t nsteps_all = (a.K + kGemvK - 1) / kGemvK;
    const int64_t sb = (int64_t)blockIdx.y * a.kchunk;
    const int64_t se = sb + a.kchunk < nsteps_all ? sb + a.kchunk : nsteps_all;
    const int64_t nsteps = se > sb ? se - sb : 0;

    typedef float f32x4 __attribute__((ext_vector_type(4)));
    f32x4 acc[MT][T];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int t = 0; t < T; ++t) acc[m][t] = (f32x4){};

    // this wavefront's steps: wave + WAVES i for i < my, one in flight
    const int64_t my = wave < nsteps ? (nsteps - wave + WAVES - 1) / WAVES : 0;
    if (my > 0) {
        GemvChunk w[T], x[MT];
        for (int64_t i = 0; i < my; ++i) {
            const int64_t k0 = (sb + wave + (int64_t)WAVES * i) * kGemvK;
            if (kStaged) {
                uint8_t* st = lds + wave * GemvStage<T>::bytes;
                uint4 v[2 * T];
                uint32_t sv[T];
                // rows past N read the last row, as in load_gemv
#pragma unroll
                for (int r = 0; r < 2 * T; ++r) {
                    const int64_t row = n0 + 8 * r + (lane >> 3);
                    const int64_t rr = row < N ? row : N - 1;
                    v[r] = *reinterpret_cast<const uint4*>(wc + rr * (a.K / 2) + k0 / 2 + 16 * (lane & 7));
                }
#pragma unroll
                for (int r = 0; r < T; ++r) {
                    const int64_t row = n0 + 16 * r + (lane >> 2);
                    const int64_t rr = row < N ? row : N - 1;
                    sv[r] = *reinterpret_cast<const uint32_t*>(wsc + rr * (a.K / 16) + k0 / 16 + 4 * (lane & 3));
                }
#pragma unroll
                for (int r = 0; r < 2 * T; ++r)
                    *reinterpret_cast<uint4*>(st + (8 * r + (lane >> 3)) * kStageRow + 16 * (lane & 7)) = v[r];
#pragma unroll
                for (int r = 0; r < T; ++r)
                    *reinterpret_cast<uint32_t*>(st + 16 * T * kStageRow + (16 * r + (lane >> 2)) * 16 + 4 * (lane & 3)) =
                        sv[r];
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const uint8_t* rp = st + (16 * t + c16) * kStageRow + 32 * g;
                    w[t].c0 = *reinterpret_cast<const uint4*>(rp);
                    w[t].c1 = *reinterpret_cast<const uint4*>(rp + 16);
                    w[t].s = *reinterpret_cast<const uint32_t*>(st + 16 * T * kStageRow + (16 * t + c16) * 16 + 4 * g);
                }
                __builtin_amdgcn_wave_barrier();
            } else {
#pragma unroll
                for (int t = 0; t < T; ++t) w[t] = load_gemv<FAST>(wc, wsc, n0 + 16 * t + c16, N, a.K, k0, g);
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) x[m] = load_gemv<FAST>(a.xc, a.xs, 16 * m + c16, a.M, a.K, k0, g);
            f16x2 w01[T], w23[T], x01[MT], x23[MT];
#pragma unroll
            for (int t = 0; t < T; ++t) {
                w01[t] = scale_pair<false>(w[t].s);
                w23[t] = scale_pair<true>(w[t].s);
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                x01[m] = scale_pair<false>(x[m].s);
                x23[m] = scale_pair<true>(x[m].s);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                f16x8 fa[MT];
#pragma unroll
                for (int m = 0; m < MT; ++m) fa[m] = codes_times(gemv_dword(x[m], j), block_scale(x01[m], x23[m], j >> 1));
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const f16x8 fb = codes_times(gemv_dword(w[t], j), block_scale(w01[t], w23[t], j >> 1));
#pragma unroll
                    for (int m = 0; m < MT; ++m)
                        acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[m], fb, acc[m][t], 0, 0, 0);
                }
            }
        }
    }

    // register r of lane l in tile (m, t): token 16 m + 4 (l / 16) + r,
    // column 16 t + l % 16; red holds (m, t, token % 16, column % 16).  It
    // shares LDS with the staging areas, so every wavefront leaves the loop
    // first.
    if (kStaged) __syncthreads();
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][((m * T + t) * 16 + 4 * g + r) * 16 + c16] = acc[m][t][r];
    __syncthreads();
    for (int e = tid; e < MT * T * 256; e += 64 * WAVES) {
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) v += red[w][e];
        const int mt = e >> 8;
        const int64_t row = 16 * (mt / T) + ((e >> 4) & 15), col = n0 + 16 * (mt % T) + (e & 15);
        if (row < a.M && col < N) {
            if (a.ksplit > 1) {  // a single member
                a.part[((int64_t)blockIdx.y * a.M + row) * N + col] = v;
            } else {
                const float y = v * (a.xs2[a.xs2_per_row ? row : 0] * mem.ws2[j][0]);
                if (BF16_OUT) {
                    const uint32_t p = bf16_pair(y, 0.0f);
                    reinterpret_cast<uint16_t*>(mem.y[j])[row * N + col] = (uint16_t)(p & 0xFFFFu);
                } else {
                    reinterpret_cast<float*>(mem.y[j])[row * N + col] = y;
                }
            }
        }
    }
}

// Split sums: Y = (sum over the k ranges, in order, of the partials) *
// (s2x[row] * s2w).  VEC: four consecutive outputs per thread with 16-byte
// loads of each partial (M * N % 4 == 0, workspace 16-byte and Y 8- or
// 16-byte aligned); otherwise one output per thread.
template <bool BF16_OUT, bool VEC>
__global__ __launch_bounds__(256) void k_nvfp4_linear_finalize(GemmArgs a) {
    const int64_t total = a.M * a.N;
    const float s2w = a.ws2[0];
    constexpr int V = VEC ? 4 : 1;
    for (int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * V; e < total; e += (int64_t)gridDim.x * 256 * V) {
        float v[V];
        if (VEC) {
            float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            for (int64_t s = 0; s < a.ksplit; ++s) {
                const float4 p = *reinterpret_cast<const float4*>(a.part + s * total + e);
                acc.x += p.x;
                acc.y += p.y;
                acc.z += p.z;
                acc.w += p.w;
            }
            v[0] = acc.x;
            v[VEC ? 1 : 0] = acc.y;
            v[VEC ? 2 : 0] = acc.z;
            v[VEC ? 3 : 0] = acc.w;
        } else {
            float acc = 0.0f;
            for (int64_t s = 0; s < a.ksplit; ++s) acc += a.part[s * total + e];
            v[0] = acc;
        }
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const int64_t row = (e + i) / a.N;
            v[i] = v[i] * (a.xs2[a.xs2_per_row ? row : 0] * s2w);
        }
        if (BF16_OUT) {
            if (VEC) {
                const uint2 o = make_uint2(bf16_pair(v[0], v[VEC ? 1 : 0]), bf16_pair(v[VEC ? 2 : 0], v[VEC ? 3 : 0]));
                *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.y) + e) = o;
            } else {
                reinterpret_cast<uint16_t*>(a.y)[e] = (uint16_t)(bf16_pair(v[0], 0.0f) & 0xFFFFu);
            }
        } else {
            if (VEC) *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.y) + e) =
                make_float4(v[0], v[VEC ? 1 : 0], v[VEC ? 2 : 0], v[VEC ? 3 : 0]);
            else reinterpret_cast<float*>(a.y)[e] = v[0];
        }
    }
}

}  // namespace

// Splitting the sum over k.  A launch of W workgroups of the tiled kernel
// runs ceil(W / CUs) rounds (each workgroup occupies a CU).  Splitting k into
// s ranges multiplies the workgroups by s and divides each one's steps by s,
// and costs s * M * N * 8 bytes of partial traffic (FP32 written, then read
// by the finalize kernel) plus a launch.  The split count minimises
//   rounds * (steps per range * t_step + t_round) + partial bytes / bandwidth,
// with the per-step and per-round times measured on MI355X; a range keeps at
// least kMinSplitSteps steps.  The decode kernel's model is its own (in
// nvfp4_linear_splits): its workgroups are small and all resident at once.
constexpr int64_t kMinSplitSteps = 4;

// Compute units of the current device.  A failed query is returned (and
// is the caller's to report); it is never replaced by a guess.
static hipError_t device_cus(int64_t& cus) {
    int dev = 0, n = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess && n <= 0) e = hipErrorInvalidDevice;
    cus = e == hipSuccess ? n : 0;
    return e;
}

hipError_t nvfp4_linear_cus(int64_t& cus) { return device_cus(cus); }

// Decode launch configuration for an [M, N] output and `steps` 256-wide
// k-steps per k range.  16-column tiles per wavefront T: with 4 or 8 token
// tiles 4 when that still leaves a workgroup per CU (every X fragment is then
// dequantized once per 4 W fragments: 28672 x 8192 at 64 tokens 59.1 against
// 70.7 us, at 128 tokens 113 against 151), else 2 when that leaves three
// workgroups per four CUs, else 1.  With 1 or 2 token tiles, where W goes
// through the LDS staging area, 2 at most: gate and up of an 8B layer at 16
// tokens took 13.7-15.4 us against 18.1-18.9 with 4 tiles and direct loads,
// 28672 x 8192 29.2-29.7 against 32.8-33.4.  Wavefronts per workgroup: 8; 4
// for fewer than 8 steps, for eight token tiles, for four on 32 columns, where
// 8 measured slower, and for two column tiles that leave at least three
// workgroups per CU with 1 or 2 token tiles, which are then all resident at
// once (gate and up at 16 tokens 13.0-13.4 against 14.2-14.9 us, 28672 x 8192
// 25.9-26.4 against 29.5-29.6; below that 4 were slower); 16 with one token
// tile for rows of at least 32
// steps, where two wavefronts per SIMD keep too little of W in flight -- with
// one column tile when the output has a workgroup per CU (4096 x 14336 at 16
// tokens 12.5-13.1 against 13.3-13.9 us with direct loads), with two when it
// has at most one (8192 x 28672 at 1 token 23.2-23.8 against 26.8-27.1 us).
// 16-token tiles: 1, 2, 4 or 8.
struct GemvConfig {
    int t, waves, mt;
};

static GemvConfig gemv_config(int64_t M, int64_t N, int64_t steps, int64_t cus) {
    GemvConfig c;
    c.mt = M <= 16 ? 1 : M <= 32 ? 2 : M <= 64 ? 4 : 8;
    c.t = c.mt >= 4 && (N + 63) / 64 >= cus ? 4 : (N + 31) / 32 >= (3 * cus) / 4 ? 2 : 1;
    c.waves = steps >= 8 && c.mt < 8 && !(c.mt == 4 && c.t == 2) ? 8 : 4;
    if (c.mt <= 2 && c.t == 2 && (N + 31) / 32 >= 3 * cus) c.waves = 4;
    if (c.mt == 1 && c.t == 1 && steps >= 32 && (N + 15) / 16 >= cus) c.waves = 16;
    if (c.mt == 1 && c.t == 2 && steps >= 32 && (N + 31) / 32 <= cus) c.waves = 16;
    return c;
}

int64_t nvfp4_linear_splits(int64_t M, int64_t N, int64_t K, int64_t part_bytes, int64_t cus) {
    const int64_t wgs = nvfp4_linear_workgroups(M, N, cus);
    const bool gemv = M <= kGemvMaxM;
    const int64_t nsteps = gemv ? (K + kGemvK - 1) / kGemvK : (K + kBK - 1) / kBK;
    if (wgs <= 0 || nsteps == 0) return 1;
    const int64_t per = M * N * 4;
    const double t_split = 4.0e-6;  // finalize launch
    const double bw = 5.0e12;       // B/s for the partials
    if (gemv) {
        // decode: a range of c steps on a workgroup of w wavefronts takes
        // ceil(c / w) rounds of one step per wavefront, each bound by the
        // load latency, by the grid's W bytes at the streaming rate or by
        // the vector instructions per SIMD, plus a fixed cost per launch
        const double t_lat = 1.2e-6, t_fix = 2.5e-6, bw_w = 4.0e12, clock = 2.4e9;
        const GemvConfig c1 = gemv_config(M, N, nsteps, cus);
        const double wave_bytes = 16.0 * c1.t * (kGemvK / 2 + kGemvK / 16);  // W per wavefront-step
        // vector instructions per wavefront-step: about 8 per 16 x 32 operand
        // fragment (W and X) and one issue slot per MFMA, 4 cycles each
        const double wave_valu = 4.0 * (64.0 * (c1.t + c1.mt) + 8.0 * c1.t * c1.mt);
        int64_t smax = nsteps / 4;
        if (per > 0 && smax > part_bytes / per) smax = part_bytes / per;
        int64_t best = 1;
        double best_t = 0.0;
        for (int64_t s = 1; s <= smax || s == 1; ++s) {
            const int64_t chunk = (nsteps + s - 1) / s;
            const int64_t se = (nsteps + chunk - 1) / chunk;
            const int64_t w = gemv_config(M, N, chunk, cus).waves;
            double round = (double)(wgs * se * w) * wave_bytes / bw_w;
            const double valu = (double)(wgs * se * w) / (4.0 * cus) * wave_valu / clock;
            if (valu > round) round = valu;
            double t = (double)((chunk + w - 1) / w) * (round > t_lat ? round : t_lat) + t_fix;
            if (se > 1) t += (double)se * (double)M * (double)N * 8.0 / bw + t_split;
            if (s == 1 || t < best_t) {
                best_t = t;
                best = se;
            }
            if (wgs * se >= cus) break;  // more ranges only add partial traffic
        }
        return best;
    }
    if (wgs >= cus) return 1;
    const double t_step = 2.3e-6;   // s per 64-wide k-step of one workgroup
    const double t_round = 3.0e-6;  // s of fixed cost per round
    int64_t smax = nsteps / kMinSplitSteps;
    if (per > 0 && smax > part_bytes / per) smax = part_bytes / per;
    int64_t best = 1;
    double best_t = 0.0;
    for (int64_t s = 1; s <= smax || s == 1; ++s) {
        const int64_t chunk = (nsteps + s - 1) / s;
        const int64_t se = (nsteps + chunk - 1) / chunk;  // ranges actually used
        const int64_t rounds = (wgs * se + cus - 1) / cus;
        double t = (double)rounds * ((double)chunk * t_step + t_round);
        if (se > 1) t += (double)se * (double)M * (double)N * 8.0 / bw + t_split;
        if (s == 1 || t < best_t) {
            best_t = t;
            best = se;
        }
        if (s > 4 * (cus / wgs + 1)) break;  // more ranges only add rounds
    }
    return best;
}

template <bool F, bool B>
static hipError_t launch_gemv(const GemvConfig& c, dim3 grid, dim3 block, hipStream_t stream, const GemmArgs& a,
                              const GemvMembers& mem) {
#define FOCUS_GV(MT, W, T) \
    case 256 * MT + 16 * T + W: return launch(&k_nvfp4_linear_gemv<F, B, W, T, MT>, grid, block, stream, a, mem);
    switch (c.mt * 256 + c.t * 16 + c.waves) {
        FOCUS_GV(1, 8, 1) FOCUS_GV(1, 4, 1) FOCUS_GV(1, 8, 2) FOCUS_GV(1, 4, 2)
        FOCUS_GV(2, 8, 1) FOCUS_GV(2, 4, 1) FOCUS_GV(2, 8, 2) FOCUS_GV(2, 4, 2)
        FOCUS_GV(4, 8, 1) FOCUS_GV(4, 4, 1) FOCUS_GV(4, 8, 2) FOCUS_GV(4, 4, 2)
        FOCUS_GV(8, 4, 1) FOCUS_GV(8, 4, 2)
        FOCUS_GV(4, 8, 4) FOCUS_GV(4, 4, 4) FOCUS_GV(8, 4, 4)
        FOCUS_GV(1, 16, 1) FOCUS_GV(1, 16, 2)
    }
#undef FOCUS_GV
    return hipErrorInvalidValue;
}

static hipError_t launch_gemv_members(const GemmArgs& a, GemvMembers& mem, const GemvConfig& c, bool f,
                                      bool bf16_out, unsigned splits, hipStream_t stream) {
    const dim3 grid((unsigned)mem.tile_start[mem.n], splits), block(64 * c.waves);
    if (f) return bf16_out ? launch_gemv<true, true>(c, grid, block, stream, a, mem)
                           : launch_gemv<true, false>(c, grid, block, stream, a, mem);
    return bf16_out ? launch_gemv<false, true>(c, grid, block, stream, a, mem)
                    : launch_gemv<false, false>(c, grid, block, stream, a, mem);
}

hipError_t launch_nvfp4_linear_grouped(const GemmArgs& a, const GemvMembers& members, bool fast, bool bf16_out,
                                       hipStream_t stream) {
    int64_t cus = 0;
    hipError_t e = device_cus(cus);
    if (e != hipSuccess) return e;
    GemmArgs g = a;
    g.part = nullptr;
    g.part_bytes = 0;
    g.ksplit = 1;
    const int64_t nsteps = (a.K + kGemvK - 1) / kGemvK;
    g.kchunk = nsteps > 0 ? nsteps : 1;
    int64_t ntot = 0;
    for (int j = 0; j < members.n; ++j) ntot += members.N[j];
    g.N = ntot;
    const GemvConfig c = gemv_config(a.M, ntot, g.kchunk, cus);
    GemvMembers mem = members;
    mem.tile_start[0] = 0;
    for (int j = 0; j < mem.n; ++j) mem.tile_start[j + 1] = mem.tile_start[j] + (mem.N[j] + 16 * c.t - 1) / (16 * c.t);
    return launch_gemv_members(g, mem, c, fast && a.K % kGemvK == 0, bf16_out, 1, stream);
}

hipError_t launch_nvfp4_linear(const GemmArgs& args, bool fast, bool bf16_out, hipStream_t stream) {
    int64_t cus = 0;
    hipError_t e = device_cus(cus);
    if (e != hipSuccess) return e;
    GemmArgs a = args;
    const bool gemv = a.M <= kGemvMaxM;
    const int64_t nsteps = gemv ? (a.K + kGemvK - 1) / kGemvK : (a.K + kBK - 1) / kBK;
    a.ksplit = a.part ? nvfp4_linear_splits(a.M, a.N, a.K, a.part_bytes, cus) : 1;
    a.kchunk = a.ksplit > 1 ? (nsteps + a.ksplit - 1) / a.ksplit : (nsteps > 0 ? nsteps : 1);
    const unsigned splits = (unsigned)a.ksplit;
    if (gemv) {
        const bool f = fast && a.K % kGemvK == 0;
        const GemvConfig c = gemv_config(a.M, a.N, a.kchunk, cus);
        GemvMembers mem = {};
        mem.wc[0] = a.wc;
        mem.ws[0] = a.ws;
        mem.ws2[0] = a.ws2;
        mem.y[0] = a.y;
        mem.N[0] = a.N;
        mem.tile_start[0] = 0;
        mem.tile_start[1] = (a.N + 16 * c.t - 1) / (16 * c.t);
        mem.n = 1;
        e = launch_gemv_members(a, mem, c, f, bf16_out, splits, stream);
    } else {
        const int64_t tiles_m = (a.M + kBM - 1) / kBM, tiles_n = (a.N + kBN - 1) / kBN;
        const dim3 grid((unsigned)(tiles_m * tiles_n), splits), block(kGemmThreads);
        if (fast) e = bf16_out ? launch(&k_nvfp4_linear<true, true>, grid, block, stream, a, tiles_n)
                               : launch(&k_nvfp4_linear<true, false>, grid, block, stream, a, tiles_n);
        else e = bf16_out ? launch(&k_nvfp4_linear<false, true>, grid, block, stream, a, tiles_n)
                          : launch(&k_nvfp4_linear<false, false>, grid, block, stream, a, tiles_n);
    }
    if (e != hipSuccess || a.ksplit <= 1) return e;
    const int64_t total = a.M * a.N;
    const bool vec = total % 4 == 0 && ((uintptr_t)a.part & 15u) == 0 &&
                     ((uintptr_t)a.y & (bf16_out ? 7u : 15u)) == 0;
    int64_t g = (total / (vec ? 4 : 1) + 255) / 256;
    if (g > 65536) g = 65536;
    const dim3 grid((unsigned)g), block(256);
    if (vec) return bf16_out ? launch(&k_nvfp4_linear_finalize<true, true>, grid, block, stream, a)
                             : launch(&k_nvfp4_linear_finalize<false, true>, grid, block, stream, a);
    return bf16_out ? launch(&k_nvfp4_linear_finalize<true, false>, grid, block, stream, a)
                    : launch(&k_nvfp4_linear_finalize<false, false>, grid, block, stream, a);
}

int64_t nvfp4_linear_workgroups(int64_t M, int64_t N, int64_t cus) {
    if (M <= kGemvMaxM) {
        const int t = gemv_config(M, N, 1, cus).t;
        return (N + 16 * t - 1) / (16 * t);
    }
    return ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
}

// ---------------------------------------------------------------------------
// The split-k workspace of the allocation-free entry point: one file-scope
// device array per GPU (each device holds its own copy at its own address,
// from the library's load until the process ends).  Host code never passes
// the array's name to a kernel or a copy -- on the host it is only a handle
// of the symbol -- but the device address that hipGetSymbolAddress returns
// for the current device, looked up once per device and kept.
// ---------------------------------------------------------------------------

static __device__ __align__(256) float scratch[kLinearScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t nvfp4_linear_scratch(float** ptr) {
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = static_cast<float*>(p);
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace focus
