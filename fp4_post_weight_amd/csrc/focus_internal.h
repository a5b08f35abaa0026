// focus_internal.h -- batch descriptors and launchers shared by the kernel
// file and the C ABI.  Arguments reaching these functions have been
// validated on the host.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace focus {

// Tensors per launch.  A batch travels by value in the kernel argument
// segment (structure of arrays, at most about 2.3 KB).
constexpr int kBatch = 32;

struct QuantBatch {
    const uint4* w[kBatch];
    const float* m[kBatch];
    const float2* q[kBatch];
    const float* s2[kBatch];
    uint2* codes[kBatch];
    uint8_t* scales[kBatch];
    uint4* wdeq[kBatch];
    int64_t nblk[kBatch];
    int64_t tile_start[kBatch + 1];
    int n;
};

// FlipQuant MixFP4: a QuantBatch plus, per tensor, the tile map and the three
// divisors that turn a block index into its tile (blocks per row, tile rows,
// tile columns in blocks) as div_magic multipliers; shift k of tensor j is
// byte k of sh[j].  About 3.3 KB in all.
struct MixBatch : QuantBatch {
    const uint8_t* map[kBatch];
    uint32_t nb_row[kBatch];
    uint32_t tiles_per_row[kBatch];
    uint32_t mul[kBatch][3];
    uint32_t sh[kBatch];
};

struct DequantBatch {
    const uint2* codes[kBatch];
    const uint8_t* scales[kBatch];
    const float* s2[kBatch];
    uint4* out[kBatch];
    int64_t nblk[kBatch];
    int64_t nb_row[kBatch];
    int64_t tile_start[kBatch + 1];
    int32_t per_row[kBatch];
    int n;
};

struct ScaleBatch {
    const uint16_t* w[kBatch];
    float* s2[kBatch];
    float* amax[kBatch];
    int64_t numel[kBatch];
    int64_t tile_start[kBatch + 1];
    int n;
};

// MixFP4 dequantize: a DequantBatch plus the tile map and its divisors, as in
// MixBatch (nb_row of the base batch is the first divisor).
struct MixDequantBatch : DequantBatch {
    const uint8_t* map[kBatch];
    uint32_t tiles_per_row[kBatch];
    uint32_t mul[kBatch][3];
    uint32_t sh[kBatch];
};

// key: bit 2 = m present, bit 1 = q present, bit 0 = w' written; 8 / 9 =
// FourOverSix without / with w' (m and q absent); 16 + (m, q, w' bits) =
// FOCUS on MXFP4; every tensor of one batch shares the key.
hipError_t launch_quantize(QuantBatch& bt, int key, hipStream_t stream);
hipError_t launch_quantize_mix(MixBatch& bt, bool deq, hipStream_t stream);
hipError_t launch_dequantize(DequantBatch& bt, bool mx, hipStream_t stream);
hipError_t launch_dequantize_mix(MixDequantBatch& bt, hipStream_t stream);
hipError_t launch_tensor_scale(ScaleBatch& bt, hipStream_t stream);
hipError_t launch_act_per_token(const uint16_t* x, int64_t tokens, int64_t hidden, uint8_t* codes,
                                uint8_t* scales, float* s2_out, uint16_t* xdeq, bool fo6,
                                hipStream_t stream);

}  // namespace focus
