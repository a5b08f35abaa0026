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

// Weights that share one X, for the decode kernel (M <= 128): member j's
// output columns take workgroup columns [tile_start[j], tile_start[j + 1])
// (set by the launcher).
constexpr int kGemvMaxMembers = 8;
constexpr int64_t kLinearDecodeMaxM = 128;
struct GemvMembers {
    const uint8_t* wc[kGemvMaxMembers];
    const uint8_t* ws[kGemvMaxMembers];
    const float* ws2[kGemvMaxMembers];
    void* y[kGemvMaxMembers];
    int64_t N[kGemvMaxMembers];
    int64_t tile_start[kGemvMaxMembers + 1];
    int n;
};

// One launch of the decode kernel over every member (M <= 128, no k split;
// a's weight fields, part and split are ignored).  fast: as above, with every
// member's arrays aligned.
hipError_t launch_nvfp4_linear_grouped(const GemmArgs& a, const GemvMembers& members, bool fast, bool bf16_out,
                                       hipStream_t stream);

// Compute units of the current device (the split model depends on them).
hipError_t nvfp4_linear_cus(int64_t& cus);

// Workgroups one launch uses for an [M, N] output (per k range) on a device
// of `cus` compute units; INT64_MAX gives the largest count of any device.
int64_t nvfp4_linear_workgroups(int64_t M, int64_t N, int64_t cus);

// k ranges the launcher splits the sum into for [M, N, K] given `part_bytes`
// of workspace and `cus` compute units (1 = no split); the workspace it uses
// is ksplit * M * N * 4 bytes.
int64_t nvfp4_linear_splits(int64_t M, int64_t N, int64_t K, int64_t part_bytes, int64_t cus);

// Bytes of the per-device array that the allocation-free linear call uses as
// its split-k workspace.
constexpr int64_t kLinearScratchBytes = (int64_t)64 << 20;

// The current device's address of that array (looked up on the first call
// on each device and kept).
hipError_t nvfp4_linear_scratch(float** ptr);

}  // namespace focus
