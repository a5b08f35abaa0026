// focus_stream.hip -- measurement helper, not part of the quantizer: one
// plain streaming kernel that reads nr and writes nw 16-byte vectors
// (nw <= nr) with no arithmetic beyond moving the bytes.  Run at the read
// and write volumes of a quantizer launch (for the 8B set with w': W, m and q
// in, codes, scales and w' out), it measures how fast this GPU moves that
// traffic mix at all, the ceiling a streaming kernel can reach.  Loaded by
// bench.py and by its test.
//
// Layout of the work: the grid strides over the read vectors in tiles of
// 256 lanes x 4 vectors, each lane's four loads issued before any store (as
// the quantizer issues its loads); read vector i is copied to write vector
// j = floor(i * nw / nr) when i is the first read vector that maps to j, so
// every write vector is written exactly once and the writes are spread
// evenly over the reads.  The vectors that are only read are folded into a
// register that reaches memory only if it equals a value no input here
// produces, so the compiler keeps the loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kT = 256;
constexpr int kU = 4;

template <bool NT_LOAD>
__global__ __launch_bounds__(kT) void k_stream(const u32x4* __restrict__ src, int64_t nr,
                                                  u32x4* __restrict__ dst, int64_t nw,
                                                  uint32_t* __restrict__ sink) {
    uint32_t acc = 0;
    const int64_t ntiles = (nr + kT * kU - 1) / (kT * kU);
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int64_t base = tile * (kT * kU) + threadIdx.x;
        u32x4 v[kU];
#pragma unroll
        for (int k = 0; k < kU; ++k) {
            const int64_t i = base + (int64_t)k * kT;
            if (i < nr) v[k] = NT_LOAD ? __builtin_nontemporal_load(src + i) : src[i];
        }
#pragma unroll
        for (int k = 0; k < kU; ++k) {
            const int64_t i = base + (int64_t)k * kT;
            if (i >= nr) continue;
            const int64_t j = (i * nw) / nr;
            const bool first = i == 0 || ((i - 1) * nw) / nr != j;
            if (first && j < nw) __builtin_nontemporal_store(v[k], dst + j);
            else acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
        }
    }
    if (acc == 0x9E3779B9u) sink[threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// src [nr] and dst [nw] 16-byte vectors (16-byte aligned device pointers),
// 0 <= nw <= nr, nr * nw < 2^63; sink: 256 uint32 of device memory; grid:
// workgroups (0: one per tile, at most 2^20).  Returns 0 or a HIP error code.
int focus_stream(const void* src, int64_t nr, void* dst, int64_t nw, void* sink, int nt_load, int64_t grid,
                 void* stream) {
    if (nr < 0 || nw < 0 || nw > nr || !src || !sink || (nw > 0 && !dst)) return (int)hipErrorInvalidValue;
    if (nr > 0 && nw > INT64_MAX / nr) return (int)hipErrorInvalidValue;
    if (nr == 0) return 0;
    const int64_t ntiles = (nr + kT * kU - 1) / (kT * kU);
    int64_t g = grid > 0 ? grid : ntiles;
    if (g > ntiles) g = ntiles;
    if (g > (1 << 20)) g = 1 << 20;
    auto s = reinterpret_cast<const u32x4*>(src);
    auto d = reinterpret_cast<u32x4*>(dst);
    auto k = reinterpret_cast<uint32_t*>(sink);
    void* args[] = {&s, &nr, &d, &nw, &k};
    const void* fn = nt_load ? reinterpret_cast<const void*>(&k_stream<true>)
                             : reinterpret_cast<const void*>(&k_stream<false>);
    return (int)hipLaunchKernel(fn, dim3((unsigned)g), dim3(kT), args, 0, (hipStream_t)stream);
}

}  // extern "C"
