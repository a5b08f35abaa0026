// focus_api.hip -- the extern "C" boundary of libfocus_nvfp4.
//
// Every entry point validates its arguments on the host before the first
// HIP call (so every error path runs without a GPU), then launches the
// kernels of focus_kernels.hip on the caller's stream.  Nothing is
// allocated and no state is kept.  The declarations, with the meaning,
// layout and ownership of each argument, are in include/focus_nvfp4.h.

#include "focus_nvfp4.h"
#include "focus_internal.h"

namespace {

// Sizes are bounded so that every byte offset (elements * 2) fits int64
// and every grid stays within HIP's limits.
constexpr int64_t kMaxElems = (int64_t)1 << 60;
constexpr int64_t kMaxTokens = (int64_t)1 << 31;

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

inline int shape_2d(int64_t rows, int64_t cols) {
    if (rows < 0 || cols < 0) return FOCUS_ERR_SHAPE;
    if (cols % 16 != 0) return FOCUS_ERR_SHAPE;
    if (rows != 0 && cols > kMaxElems / rows) return FOCUS_ERR_SHAPE;
    return FOCUS_OK;
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? FOCUS_OK : FOCUS_ERR_HIP; }

}  // namespace

extern "C" {

int focus_abi_version(void) { return FOCUS_NVFP4_ABI_VERSION; }

const char* focus_status_string(int status) {
    switch (status) {
        case FOCUS_OK: return "ok";
        case FOCUS_ERR_NULL: return "a required pointer is NULL";
        case FOCUS_ERR_SHAPE: return "invalid shape (negative size, cols not a multiple of 16, or too large)";
        case FOCUS_ERR_ALIGN: return "a pointer is not aligned as documented";
        case FOCUS_ERR_HIP: return "a HIP kernel launch failed";
        case FOCUS_ERR_RANGE: return "an argument is outside its documented range";
        default: return "unknown status";
    }
}

int focus_tensor_scale(const uint16_t* w_bf16, int64_t numel, float* s2_out, float* amax_out,
                       void* stream) {
    if (!s2_out || (numel > 0 && !w_bf16)) return FOCUS_ERR_NULL;
    if (numel < 0 || numel > kMaxElems) return FOCUS_ERR_SHAPE;
    if (!aligned(w_bf16, 16) || !aligned(s2_out, 4) || !aligned(amax_out, 4)) return FOCUS_ERR_ALIGN;
    return hip_status(focus::launch_tensor_scale(w_bf16, numel, s2_out, amax_out,
                                                 (hipStream_t)stream));
}

int focus_quantize(const uint16_t* w_bf16, int64_t rows, int64_t cols, const float* m,
                   const float* q, const float* s2, uint8_t* codes, uint8_t* scales,
                   uint16_t* w_deq, void* stream) {
    int st = shape_2d(rows, cols);
    if (st != FOCUS_OK) return st;
    if (rows == 0 || cols == 0) return FOCUS_OK;
    if (!w_bf16 || !s2 || !codes || !scales) return FOCUS_ERR_NULL;
    if (!aligned(w_bf16, 16) || !aligned(m, 4) || !aligned(q, 8) || !aligned(s2, 4) ||
        !aligned(codes, 8) || !aligned(w_deq, 16))
        return FOCUS_ERR_ALIGN;
    return hip_status(focus::launch_quantize(w_bf16, rows, cols, m, q, s2, codes, scales, w_deq,
                                             (hipStream_t)stream));
}

int focus_dequantize(const uint8_t* codes, const uint8_t* scales, const float* s2, int s2_per_row,
                     int64_t rows, int64_t cols, uint16_t* out, void* stream) {
    int st = shape_2d(rows, cols);
    if (st != FOCUS_OK) return st;
    if (s2_per_row != 0 && s2_per_row != 1) return FOCUS_ERR_RANGE;
    if (rows == 0 || cols == 0) return FOCUS_OK;
    if (!codes || !scales || !s2 || !out) return FOCUS_ERR_NULL;
    if (!aligned(codes, 8) || !aligned(s2, 4) || !aligned(out, 16)) return FOCUS_ERR_ALIGN;
    return hip_status(focus::launch_dequantize(codes, scales, s2, s2_per_row, rows, cols, out,
                                               (hipStream_t)stream));
}

int focus_quantize_act_per_token(const uint16_t* x_bf16, int64_t tokens, int64_t hidden,
                                 uint8_t* codes, uint8_t* scales, float* s2_out, uint16_t* x_deq,
                                 void* stream) {
    int st = shape_2d(tokens, hidden);
    if (st != FOCUS_OK) return st;
    if (tokens > kMaxTokens) return FOCUS_ERR_RANGE;
    if (tokens == 0 || hidden == 0) return FOCUS_OK;
    if (!x_bf16 || !codes || !scales || !s2_out) return FOCUS_ERR_NULL;
    if (!aligned(x_bf16, 16) || !aligned(codes, 8) || !aligned(s2_out, 4) || !aligned(x_deq, 16))
        return FOCUS_ERR_ALIGN;
    return hip_status(focus::launch_act_per_token(x_bf16, tokens, hidden, codes, scales, s2_out,
                                                  x_deq, (hipStream_t)stream));
}

}  // extern "C"
