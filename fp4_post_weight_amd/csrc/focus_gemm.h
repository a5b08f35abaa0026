// focus_gemm.h -- arguments and launcher of the NVFP4 linear layer kernel,
// shared by focus_gemm.hip and the C ABI.  Arguments reaching the launcher
// have been validated on the host.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace focus {

struct GemmArgs {
    const uint8_t* xc;   // activation codes [M, K/2]
    const uint8_t* xs;   // activation scale bytes [M, K/16]
    const float* xs2;    // [M] when xs2_per_row, else one value
    int xs2_per_row;
    int64_t M;
    const uint8_t* wc;   // weight codes [N, K/2]
    const uint8_t* ws;   // weight scale bytes [N, K/16]
    const float* ws2;    // one value
    int64_t N, K;
    void* y;             // [M, N] FP32 or BF16
    float* part;         // split-K partials [ksplit, M, N] FP32, or NULL
    int64_t part_bytes;  // bytes available at `part`
    int64_t ksplit;      // set by the launcher: number of k ranges
    int64_t kchunk;      // set by the launcher: 64-wide k-steps per range
};

// fast: K % 64 == 0, both code arrays 16-byte and both scale arrays 4-byte
// aligned.
hipError_t launch_nvfp4_linear(const GemmArgs& a, bool fast, bool bf16_out, hipStream_t stream);

// Workgroups one launch uses for an [M, N] output (per k range).
int64_t nvfp4_linear_workgroups(int64_t M, int64_t N);

// k ranges the launcher splits the sum into for [M, N, K] given `part_bytes`
// of workspace (1 = no split); the workspace it uses is ksplit * M * N * 4
// bytes.
int64_t nvfp4_linear_splits(int64_t M, int64_t N, int64_t K, int64_t part_bytes);

}  // namespace focus
