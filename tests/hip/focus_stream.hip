// focus_stream.hip -- measurement helper, not part of the quantizer: a
// kernel with the memory traffic of the quantizer with w' and none of its
// arithmetic.  Per 16-element block it reads 32 bytes of weights, 4 bytes of
// block factor and 8 bytes of logits and writes 8 bytes of codes, one scale
// byte and 32 bytes of dequantized weights, with the quantizer's layout of
// the work: 256 lanes per workgroup, two blocks per lane per tile with every
// load issued before any store, the weights read and the dequantized weights
// written as contiguous 1 KB per wavefront instruction, nontemporal stores.
// Each output is a cheap function of the inputs (so no load is dead), and
// the copy of the weights comes back unchanged.  Its rate is how fast this
// GPU moves the quantizer's traffic pattern at all: the ceiling for a
// streaming kernel of that shape.  The same for the per-token activations,
// the tensor scale (reads only) and the dequantize (mostly writes).  Loaded
// by bench.py and by its test.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kT = 256;

// U blocks per lane per tile (the quantizer with w' uses 2)
template <int U>
__global__ __launch_bounds__(kT) void k_pattern(const u32x4* __restrict__ w, const uint32_t* __restrict__ m,
                                                   const u32x2* __restrict__ q, int64_t nblk,
                                                   u32x2* __restrict__ codes, uint8_t* __restrict__ scales,
                                                   u32x4* __restrict__ wdeq, int64_t ntiles) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int64_t tile0 = tile * (int64_t)kT * U;
        u32x4 va[U], vb[U];
        uint32_t mb[U];
        u32x2 qq[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t first = tile0 + (int64_t)k * kT + wave * 64;  // block of lane 0
            const int64_t blk = first + lane, h = 2 * first + lane, nh = 2 * nblk;
            va[k] = h < nh ? w[h] : u32x4{0, 0, 0, 0};
            vb[k] = h + 64 < nh ? w[h + 64] : u32x4{0, 0, 0, 0};
            mb[k] = blk < nblk ? m[blk] : 0u;
            qq[k] = blk < nblk ? q[blk] : u32x2{0, 0};
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t first = tile0 + (int64_t)k * kT + wave * 64;
            const int64_t blk = first + lane, h = 2 * first + lane, nh = 2 * nblk;
            if (h < nh) __builtin_nontemporal_store(va[k], wdeq + h);
            if (h + 64 < nh) __builtin_nontemporal_store(vb[k], wdeq + h + 64);
            if (blk < nblk) {
                const u32x2 c = {va[k].x ^ vb[k].y ^ qq[k].x, va[k].z ^ vb[k].w ^ qq[k].y};
                __builtin_nontemporal_store(c, codes + blk);
                scales[blk] = (uint8_t)(mb[k] >> 23);
            }
        }
    }
}

// The traffic of per-token activation quantization of X [tokens, hidden]
// (hidden = 64 * RB * 16): a wavefront takes rows in turn, reads each as
// contiguous 1 KB per load instruction, and writes its codes (8 bytes per
// 16-element block), scale bytes and one float; 4 wavefronts per workgroup.
template <int RB>
__global__ __launch_bounds__(256) void k_act_pattern(const u32x4* __restrict__ x, int64_t tokens,
                                                    u32x2* __restrict__ codes, uint8_t* __restrict__ scales,
                                                    float* __restrict__ s2) {
    const int lane = threadIdx.x & 63;
    constexpr int64_t nb = 64 * RB;
    for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < tokens; row += (int64_t)gridDim.x * 4) {
        const int64_t base = row * nb;
        u32x4 va[RB], vb[RB];
#pragma unroll
        for (int k = 0; k < RB; ++k) {
            va[k] = x[2 * (base + 64 * k) + lane];
            vb[k] = x[2 * (base + 64 * k) + 64 + lane];
        }
        uint32_t acc = 0;
#pragma unroll
        for (int k = 0; k < RB; ++k) {
            const u32x2 c = {va[k].x ^ vb[k].y, va[k].z ^ vb[k].w};
            __builtin_nontemporal_store(c, codes + base + 64 * k + lane);
            scales[base + 64 * k + lane] = (uint8_t)(va[k].x ^ vb[k].z);
            acc ^= c.x;
        }
        if (lane == 0) s2[row] = __uint_as_float(acc & 0x3FFFFFFFu);
    }
}


// The traffic of the tensor scale: nvec 16-byte vectors read once, with the
// reduction kernel's layout (workgroups of 256 lanes striding over tiles of
// 256 * U vectors, U nontemporal 16-byte loads per lane per tile), each lane
// folding what it reads into one word (the maximum of the XOR of each
// vector's four words), written once at the end.
template <int U>
__global__ __launch_bounds__(256) void k_read_pattern(const u32x4* __restrict__ w, int64_t nvec,
                                                       uint32_t* __restrict__ out) {
    constexpr int64_t tv = 256 * U;
    const int64_t ntiles = (nvec + tv - 1) / tv;
    uint32_t acc = 0;
    for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const int64_t base = t * tv + threadIdx.x;
        u32x4 v[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t i = base + (int64_t)k * 256;
            v[k] = i < nvec ? __builtin_nontemporal_load(w + i) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int k = 0; k < U; ++k) acc = max(acc, v[k].x ^ v[k].y ^ v[k].z ^ v[k].w);
    }
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

// The traffic of the dequantize: per 16-element block 8 bytes of codes and
// one scale byte in, 32 bytes out, with the dequantize kernel's layout (one
// block per lane per tile of 256 blocks; each wavefront's 2 KB of output
// regrouped through LDS so that every store instruction writes 1 KB of
// contiguous memory; nontemporal stores).  Block b's output is the two
// vectors (c.x, c.y, s, c.x ^ s) and (c.y, c.x, s ^ 255, c.y ^ s), c its
// codes and s its scale byte.
__global__ __launch_bounds__(256) void k_deq_pattern(const u32x2* __restrict__ codes,
                                                     const uint8_t* __restrict__ scales, int64_t nblk,
                                                     u32x4* __restrict__ out, int64_t ntiles) {
    __shared__ u32x4 xch[4][128];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int64_t first = tile * 256 + wave * 64;  // block of lane 0
        const int64_t blk = first + lane;
        u32x2 c = {0, 0};
        uint32_t sb = 0;
        if (blk < nblk) {
            c = codes[blk];
            sb = scales[blk];
        }
        if (first < nblk) {  // uniform per wavefront
            xch[wave][2 * lane] = u32x4{c.x, c.y, sb, c.x ^ sb};
            xch[wave][2 * lane + 1] = u32x4{c.y, c.x, sb ^ 255u, c.y ^ sb};
            __builtin_amdgcn_wave_barrier();
            const u32x4 h0 = xch[wave][lane], h1 = xch[wave][64 + lane];
            __builtin_amdgcn_wave_barrier();
            const int64_t halves = 2 * (nblk - first);
            if (lane < halves) __builtin_nontemporal_store(h0, out + 2 * first + lane);
            if (64 + lane < halves) __builtin_nontemporal_store(h1, out + 2 * first + 64 + lane);
        }
    }
}

}  // namespace

extern "C" {

// w [nblk*2] 16-byte vectors, m [nblk] 4-byte words, q [nblk] 8-byte pairs
// in; codes [nblk] 8-byte pairs, scales [nblk] bytes, wdeq [nblk*2] 16-byte
// vectors out (device pointers, aligned to their element size).  wdeq
// receives a copy of w.  For block b = 64 f + l (l = b mod 64), the lane that
// owns it holds vectors A = w[128 f + l] and B = w[128 f + 64 + l] (zero past
// the end), and codes[b] = (A.x ^ B.y ^ q[b].x, A.z ^ B.w ^ q[b].y);
// scales[b] = bits 23-30 of m[b].  Returns 0 or a HIP error code.
// u: blocks per lane per tile, 1, 2 or 4 (the work layout changes, the
// outputs do not).
int focus_stream_pattern(const void* w, const void* m, const void* q, int64_t nblk, void* codes, void* scales,
                         void* wdeq, int u, void* stream) {
    if (nblk < 0 || (nblk > 0 && (!w || !m || !q || !codes || !scales || !wdeq))) return (int)hipErrorInvalidValue;
    if (u != 1 && u != 2 && u != 4) return (int)hipErrorInvalidValue;
    if (nblk == 0) return 0;
    const int64_t ntiles = (nblk + kT * u - 1) / (kT * u);
    const int64_t g = ntiles < (1 << 20) ? ntiles : (1 << 20);
    auto W = reinterpret_cast<const u32x4*>(w);
    auto M = reinterpret_cast<const uint32_t*>(m);
    auto Q = reinterpret_cast<const u32x2*>(q);
    auto C = reinterpret_cast<u32x2*>(codes);
    auto S = reinterpret_cast<uint8_t*>(scales);
    auto D = reinterpret_cast<u32x4*>(wdeq);
    int64_t n = nblk, nt = ntiles;
    void* args[] = {&W, &M, &Q, &n, &C, &S, &D, &nt};
    const void* fn = u == 1 ? reinterpret_cast<const void*>(&k_pattern<1>)
                   : u == 2 ? reinterpret_cast<const void*>(&k_pattern<2>) : reinterpret_cast<const void*>(&k_pattern<4>);
    return (int)hipLaunchKernel(fn, dim3((unsigned)g), dim3(kT), args, 0, (hipStream_t)stream);
}

// x [tokens, 1024 * rb] BF16 (16-byte aligned) in; codes [tokens, 512 * rb]
// (8-byte aligned), scales [tokens, 64 * rb], s2 [tokens] out; rb 1, 2, 4 or
// 8; grid: workgroups of 4 wavefronts.  For block b of a row (lane l =
// b mod 64, k = b / 64) the lane holds vectors A = x_row[128 k + l] and
// B = x_row[128 k + 64 + l]: codes[b] = (A.x ^ B.y, A.z ^ B.w), scales[b] =
// low byte of A.x ^ B.z, s2[row] = the bits of the XOR of the row's first
// code words with bits 30-31 cleared.  Returns 0 or a HIP error code.
int focus_stream_act_pattern(const void* x, int64_t tokens, int rb, void* codes, void* scales, void* s2, int64_t grid,
                             void* stream) {
    if (tokens < 0 || grid < 1 || (tokens > 0 && (!x || !codes || !scales || !s2))) return (int)hipErrorInvalidValue;
    if (tokens == 0) return 0;
    auto X = reinterpret_cast<const u32x4*>(x);
    auto C = reinterpret_cast<u32x2*>(codes);
    auto S = reinterpret_cast<uint8_t*>(scales);
    auto F = reinterpret_cast<float*>(s2);
    int64_t t = tokens;
    void* args[] = {&X, &t, &C, &S, &F};
    const void* fn = rb == 1 ? reinterpret_cast<const void*>(&k_act_pattern<1>)
                   : rb == 2 ? reinterpret_cast<const void*>(&k_act_pattern<2>)
                   : rb == 4 ? reinterpret_cast<const void*>(&k_act_pattern<4>)
                   : rb == 8 ? reinterpret_cast<const void*>(&k_act_pattern<8>) : nullptr;
    if (!fn) return (int)hipErrorInvalidValue;
    return (int)hipLaunchKernel(fn, dim3((unsigned)(grid < (1 << 20) ? grid : (1 << 20))), dim3(256), args, 0,
                                (hipStream_t)stream);
}


// w [nvec] 16-byte vectors in (16-byte aligned); out [grid * 256] words: word
// 256 g + t is the maximum over the vectors i with i mod 256 == t and
// (i / (256 u)) mod grid == g of the XOR of their four words (0 if none).
// u: 4 or 8 vectors per lane per tile.  Returns 0 or a HIP error code.
int focus_stream_read_pattern(const void* w, int64_t nvec, void* out, int u, int64_t grid, void* stream) {
    if (nvec < 0 || grid < 1 || grid > (1 << 20) || !out || (nvec > 0 && !w)) return (int)hipErrorInvalidValue;
    if (u != 4 && u != 8) return (int)hipErrorInvalidValue;
    auto W = reinterpret_cast<const u32x4*>(w);
    auto O = reinterpret_cast<uint32_t*>(out);
    int64_t n = nvec;
    void* args[] = {&W, &n, &O};
    const void* fn = u == 4 ? reinterpret_cast<const void*>(&k_read_pattern<4>)
                            : reinterpret_cast<const void*>(&k_read_pattern<8>);
    return (int)hipLaunchKernel(fn, dim3((unsigned)grid), dim3(256), args, 0, (hipStream_t)stream);
}

// codes [nblk] 8-byte pairs (8-byte aligned) and scales [nblk] bytes in;
// out [2 * nblk] 16-byte vectors (16-byte aligned): out[2b] = (c.x, c.y, s,
// c.x ^ s), out[2b + 1] = (c.y, c.x, s ^ 255, c.y ^ s) for c = codes[b],
// s = scales[b].  Returns 0 or a HIP error code.
int focus_stream_deq_pattern(const void* codes, const void* scales, int64_t nblk, void* out, void* stream) {
    if (nblk < 0 || (nblk > 0 && (!codes || !scales || !out))) return (int)hipErrorInvalidValue;
    if (nblk == 0) return 0;
    const int64_t ntiles = (nblk + 255) / 256;
    const int64_t g = ntiles < (1 << 20) ? ntiles : (1 << 20);
    auto C = reinterpret_cast<const u32x2*>(codes);
    auto S = reinterpret_cast<const uint8_t*>(scales);
    auto O = reinterpret_cast<u32x4*>(out);
    int64_t n = nblk, nt = ntiles;
    void* args[] = {&C, &S, &n, &O, &nt};
    return (int)hipLaunchKernel(reinterpret_cast<const void*>(&k_deq_pattern), dim3((unsigned)g), dim3(256), args, 0,
                                (hipStream_t)stream);
}

}  // extern "C"
