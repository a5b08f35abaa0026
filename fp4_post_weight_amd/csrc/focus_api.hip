// focus_api.hip -- the extern "C" boundary of libfocus_nvfp4.
//
// Every entry point validates all of its arguments on the host before the
// first HIP call (so every error path runs without a GPU), then launches the
// kernels of focus_kernels.hip on the caller's stream.  Nothing is allocated
// and no state is kept.  Batched calls read their descriptor arrays during
// the call only and launch one kernel (one per phase for the tensor scale)
// per run of up to focus::kBatch tensors.  The declarations, with the
// meaning, layout and ownership of each argument, are in
// include/focus_nvfp4.h.

#include "focus_nvfp4.h"
#include "focus_gemm.h"
#include "focus_internal.h"

namespace {

// Sizes are bounded so that every byte offset (elements * 2) fits int64 and
// every grid stays within HIP's limits.
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

int check_quant(const focus_quant_desc& d) {
    int st = shape_2d(d.rows, d.cols);
    if (st != FOCUS_OK) return st;
    if (d.rows == 0 || d.cols == 0) return FOCUS_OK;
    if (!d.w_bf16 || !d.s2 || !d.codes || !d.scales) return FOCUS_ERR_NULL;
    if (!aligned(d.w_bf16, 16) || !aligned(d.m, 4) || !aligned(d.q, 8) || !aligned(d.s2, 4) ||
        !aligned(d.codes, 8) || !aligned(d.w_deq, 16))
        return FOCUS_ERR_ALIGN;
    return FOCUS_OK;
}

int check_dequant(const focus_dequant_desc& d) {
    int st = shape_2d(d.rows, d.cols);
    if (st != FOCUS_OK) return st;
    if (d.s2_per_row != 0 && d.s2_per_row != 1) return FOCUS_ERR_RANGE;
    if (d.rows == 0 || d.cols == 0) return FOCUS_OK;
    if (!d.codes || !d.scales || !d.s2 || !d.out) return FOCUS_ERR_NULL;
    if (!aligned(d.codes, 8) || !aligned(d.s2, 4) || !aligned(d.out, 16)) return FOCUS_ERR_ALIGN;
    return FOCUS_OK;
}

int check_scale(const focus_scale_desc& d) {
    if (!d.s2_out || (d.numel > 0 && !d.w_bf16)) return FOCUS_ERR_NULL;
    if (d.numel < 0 || d.numel > kMaxElems) return FOCUS_ERR_SHAPE;
    if (!aligned(d.w_bf16, 16) || !aligned(d.s2_out, 4) || !aligned(d.amax_out, 4))
        return FOCUS_ERR_ALIGN;
    return FOCUS_OK;
}

// MXFP4: cols % 32 == 0, no tensor scale (s2 is ignored and may be NULL).
int check_quant_mx(const focus_quant_desc& d) {
    int st = shape_2d(d.rows, d.cols);
    if (st != FOCUS_OK) return st;
    if (d.cols % 32 != 0) return FOCUS_ERR_SHAPE;
    if (d.rows == 0 || d.cols == 0) return FOCUS_OK;
    if (!d.w_bf16 || !d.codes || !d.scales) return FOCUS_ERR_NULL;
    if (!aligned(d.w_bf16, 16) || !aligned(d.m, 4) || !aligned(d.q, 8) || !aligned(d.codes, 8) ||
        !aligned(d.w_deq, 16))
        return FOCUS_ERR_ALIGN;
    return FOCUS_OK;
}

// MixFP4: tiles of tile_rows x tile_cols (tile_cols a multiple of 16, both
// dividing the shape); the kernel indexes blocks in 32 bits.
constexpr int64_t kMaxMixBlocks = (int64_t)1 << 31;

int check_quant_mix(const focus_mixfp4_desc& d) {
    int st = shape_2d(d.rows, d.cols);
    if (st != FOCUS_OK) return st;
    if (d.tile_rows < 1 || d.tile_cols < 16 || d.tile_cols % 16 != 0) return FOCUS_ERR_SHAPE;
    if (d.rows % d.tile_rows != 0 || d.cols % d.tile_cols != 0) return FOCUS_ERR_SHAPE;
    if (d.rows == 0 || d.cols == 0) return FOCUS_OK;
    if (d.rows * (d.cols / 16) >= kMaxMixBlocks) return FOCUS_ERR_RANGE;
    if (!d.w_bf16 || !d.s2 || !d.map || !d.codes || !d.scales) return FOCUS_ERR_NULL;
    if (!aligned(d.w_bf16, 16) || !aligned(d.s2, 4) || !aligned(d.codes, 8) || !aligned(d.w_deq, 16))
        return FOCUS_ERR_ALIGN;
    return FOCUS_OK;
}

// Multiplier and shift of focus::div_magic for a divisor 1 <= d < 2^31:
// l = ceil(log2 d), shift = 31 + l, M = ceil(2^shift / d).
void div_magic_host(uint32_t d, uint32_t& M, uint32_t& shift) {
    uint32_t l = 0;
    while (((uint64_t)1 << l) < d) ++l;
    shift = 31 + l;
    M = (uint32_t)((((uint64_t)1 << shift) + d - 1) / d);
}

int run_quantize_mix(const focus_mixfp4_desc* descs, int n, hipStream_t stream) {
    focus::MixBatch bt;
    bool deq = false;
    bt.n = 0;
    for (int i = 0; i <= n; ++i) {
        const bool end = (i == n);
        if (!end && (descs[i].rows == 0 || descs[i].cols == 0)) continue;
        const bool k = !end && descs[i].w_deq != nullptr;
        if (bt.n > 0 && (end || k != deq || bt.n == focus::kBatch)) {
            int st = hip_status(focus::launch_quantize_mix(bt, deq, stream));
            if (st != FOCUS_OK) return st;
            bt.n = 0;
        }
        if (end) break;
        const focus_mixfp4_desc& d = descs[i];
        deq = k;
        const int j = bt.n++;
        bt.w[j] = reinterpret_cast<const uint4*>(d.w_bf16);
        bt.m[j] = nullptr;
        bt.q[j] = nullptr;
        bt.s2[j] = d.s2;
        bt.codes[j] = reinterpret_cast<uint2*>(d.codes);
        bt.scales[j] = d.scales;
        bt.wdeq[j] = reinterpret_cast<uint4*>(d.w_deq);
        bt.nblk[j] = d.rows * (d.cols / 16);
        bt.map[j] = d.map;
        const uint32_t nb = (uint32_t)(d.cols / 16), tcb = (uint32_t)(d.tile_cols / 16);
        bt.nb_row[j] = nb;
        bt.tiles_per_row[j] = (uint32_t)(d.cols / d.tile_cols);
        uint32_t s0, s1, s2;
        div_magic_host(nb, bt.mul[j][0], s0);
        div_magic_host((uint32_t)d.tile_rows, bt.mul[j][1], s1);
        div_magic_host(tcb, bt.mul[j][2], s2);
        bt.sh[j] = s0 | (s1 << 8) | (s2 << 16);
    }
    return FOCUS_OK;
}

int quant_key(const focus_quant_desc& d) {
    return (d.m ? 4 : 0) | (d.q ? 2 : 0) | (d.w_deq ? 1 : 0);
}

// mode 0: FOCUS NVFP4, 1: FourOverSix, 2: FOCUS on MXFP4.
int run_quantize(const focus_quant_desc* descs, int n, hipStream_t stream, int mode = 0) {
    focus::QuantBatch bt;
    int key = -1;
    bt.n = 0;
    for (int i = 0; i <= n; ++i) {
        const bool end = (i == n);
        const bool skip = !end && (descs[i].rows == 0 || descs[i].cols == 0);
        if (skip) continue;
        const int k = end ? -1
                          : (mode == 1 ? 8 | (descs[i].w_deq ? 1 : 0)
                                       : (mode == 2 ? 16 : 0) | quant_key(descs[i]));
        if (bt.n > 0 && (end || k != key || bt.n == focus::kBatch)) {
            int st = hip_status(focus::launch_quantize(bt, key, stream));
            if (st != FOCUS_OK) return st;
            bt.n = 0;
        }
        if (end) break;
        const focus_quant_desc& d = descs[i];
        key = k;
        const int j = bt.n++;
        bt.w[j] = reinterpret_cast<const uint4*>(d.w_bf16);
        bt.m[j] = d.m;
        bt.q[j] = reinterpret_cast<const float2*>(d.q);
        bt.s2[j] = d.s2;
        bt.codes[j] = reinterpret_cast<uint2*>(d.codes);
        bt.scales[j] = d.scales;
        bt.wdeq[j] = reinterpret_cast<uint4*>(d.w_deq);
        bt.nblk[j] = d.rows * (d.cols / 16);
    }
    return FOCUS_OK;
}

int run_dequantize(const focus_dequant_desc* descs, int n, hipStream_t stream, bool mx = false) {
    focus::DequantBatch bt;
    bt.n = 0;
    for (int i = 0; i <= n; ++i) {
        const bool end = (i == n);
        if (!end && (descs[i].rows == 0 || descs[i].cols == 0)) continue;
        if (bt.n > 0 && (end || bt.n == focus::kBatch)) {
            int st = hip_status(focus::launch_dequantize(bt, mx, stream));
            if (st != FOCUS_OK) return st;
            bt.n = 0;
        }
        if (end) break;
        const focus_dequant_desc& d = descs[i];
        const int j = bt.n++;
        bt.codes[j] = reinterpret_cast<const uint2*>(d.codes);
        bt.scales[j] = d.scales;
        bt.s2[j] = d.s2;
        bt.out[j] = reinterpret_cast<uint4*>(d.out);
        bt.nb_row[j] = d.cols / 16;
        bt.nblk[j] = d.rows * (d.cols / 16);
        bt.per_row[j] = d.s2_per_row;
    }
    return FOCUS_OK;
}

int run_tensor_scale(const focus_scale_desc* descs, int n, hipStream_t stream) {
    focus::ScaleBatch bt;
    bt.n = 0;
    for (int i = 0; i <= n; ++i) {
        const bool end = (i == n);
        if (bt.n > 0 && (end || bt.n == focus::kBatch)) {
            int st = hip_status(focus::launch_tensor_scale(bt, stream));
            if (st != FOCUS_OK) return st;
            bt.n = 0;
        }
        if (end) break;
        const focus_scale_desc& d = descs[i];
        const int j = bt.n++;
        bt.w[j] = d.w_bf16;
        bt.s2[j] = d.s2_out;
        bt.amax[j] = d.amax_out;
        bt.numel[j] = d.numel;
    }
    return FOCUS_OK;
}

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
    const focus_scale_desc d = {w_bf16, numel, s2_out, amax_out};
    int st = check_scale(d);
    if (st != FOCUS_OK) return st;
    return run_tensor_scale(&d, 1, (hipStream_t)stream);
}

int focus_tensor_scale_many(const focus_scale_desc* descs, int n, void* stream) {
    if (n < 0) return FOCUS_ERR_RANGE;
    if (n > 0 && !descs) return FOCUS_ERR_NULL;
    for (int i = 0; i < n; ++i) {
        int st = check_scale(descs[i]);
        if (st != FOCUS_OK) return st;
    }
    return run_tensor_scale(descs, n, (hipStream_t)stream);
}

int focus_quantize(const uint16_t* w_bf16, int64_t rows, int64_t cols, const float* m,
                   const float* q, const float* s2, uint8_t* codes, uint8_t* scales,
                   uint16_t* w_deq, void* stream) {
    const focus_quant_desc d = {w_bf16, rows, cols, m, q, s2, codes, scales, w_deq};
    int st = check_quant(d);
    if (st != FOCUS_OK) return st;
    return run_quantize(&d, 1, (hipStream_t)stream);
}

int focus_quantize_many(const focus_quant_desc* descs, int n, void* stream) {
    if (n < 0) return FOCUS_ERR_RANGE;
    if (n > 0 && !descs) return FOCUS_ERR_NULL;
    for (int i = 0; i < n; ++i) {
        int st = check_quant(descs[i]);
        if (st != FOCUS_OK) return st;
    }
    return run_quantize(descs, n, (hipStream_t)stream);
}

int focus_dequantize(const uint8_t* codes, const uint8_t* scales, const float* s2, int s2_per_row,
                     int64_t rows, int64_t cols, uint16_t* out, void* stream) {
    const focus_dequant_desc d = {codes, scales, s2, s2_per_row, rows, cols, out};
    int st = check_dequant(d);
    if (st != FOCUS_OK) return st;
    return run_dequantize(&d, 1, (hipStream_t)stream);
}

int focus_dequantize_many(const focus_dequant_desc* descs, int n, void* stream) {
    if (n < 0) return FOCUS_ERR_RANGE;
    if (n > 0 && !descs) return FOCUS_ERR_NULL;
    for (int i = 0; i < n; ++i) {
        int st = check_dequant(descs[i]);
        if (st != FOCUS_OK) return st;
    }
    return run_dequantize(descs, n, (hipStream_t)stream);
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
                                                  x_deq, false, (hipStream_t)stream));
}

int focus_quantize_fo6(const uint16_t* w_bf16, int64_t rows, int64_t cols, const float* s2,
                       uint8_t* codes, uint8_t* scales, uint16_t* w_deq, void* stream) {
    const focus_quant_desc d = {w_bf16, rows, cols, nullptr, nullptr, s2, codes, scales, w_deq};
    int st = check_quant(d);
    if (st != FOCUS_OK) return st;
    return run_quantize(&d, 1, (hipStream_t)stream, 1);
}

int focus_quantize_fo6_many(const focus_quant_desc* descs, int n, void* stream) {
    if (n < 0) return FOCUS_ERR_RANGE;
    if (n > 0 && !descs) return FOCUS_ERR_NULL;
    for (int i = 0; i < n; ++i) {
        int st = check_quant(descs[i]);
        if (st != FOCUS_OK) return st;
        if (descs[i].m || descs[i].q) return FOCUS_ERR_RANGE;
    }
    return run_quantize(descs, n, (hipStream_t)stream, 1);
}

int focus_quantize_mx(const uint16_t* w_bf16, int64_t rows, int64_t cols, const float* m,
                      const float* q, uint8_t* codes, uint8_t* scales, uint16_t* w_deq,
                      void* stream) {
    const focus_quant_desc d = {w_bf16, rows, cols, m, q, nullptr, codes, scales, w_deq};
    int st = check_quant_mx(d);
    if (st != FOCUS_OK) return st;
    return run_quantize(&d, 1, (hipStream_t)stream, 2);
}

int focus_quantize_mx_many(const focus_quant_desc* descs, int n, void* stream) {
    if (n < 0) return FOCUS_ERR_RANGE;
    if (n > 0 && !descs) return FOCUS_ERR_NULL;
    for (int i = 0; i < n; ++i) {
        int st = check_quant_mx(descs[i]);
        if (st != FOCUS_OK) return st;
    }
    return run_quantize(descs, n, (hipStream_t)stream, 2);
}

int focus_dequantize_mx(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                        uint16_t* out, void* stream) {
    int st = shape_2d(rows, cols);
    if (st != FOCUS_OK) return st;
    if (cols % 32 != 0) return FOCUS_ERR_SHAPE;
    if (rows == 0 || cols == 0) return FOCUS_OK;
    if (!codes || !scales || !out) return FOCUS_ERR_NULL;
    if (!aligned(codes, 8) || !aligned(out, 16)) return FOCUS_ERR_ALIGN;
    const focus_dequant_desc d = {codes, scales, nullptr, 0, rows, cols, out};
    return run_dequantize(&d, 1, (hipStream_t)stream, true);
}

int focus_quantize_act_per_token_fo6(const uint16_t* x_bf16, int64_t tokens, int64_t hidden,
                                     uint8_t* codes, uint8_t* scales, float* s2_out,
                                     uint16_t* x_deq, void* stream) {
    int st = shape_2d(tokens, hidden);
    if (st != FOCUS_OK) return st;
    if (tokens > kMaxTokens) return FOCUS_ERR_RANGE;
    if (tokens == 0 || hidden == 0) return FOCUS_OK;
    if (!x_bf16 || !codes || !scales || !s2_out) return FOCUS_ERR_NULL;
    if (!aligned(x_bf16, 16) || !aligned(codes, 8) || !aligned(s2_out, 4) || !aligned(x_deq, 16))
        return FOCUS_ERR_ALIGN;
    return hip_status(focus::launch_act_per_token(x_bf16, tokens, hidden, codes, scales, s2_out,
                                                  x_deq, true, (hipStream_t)stream));
}

int focus_quantize_mixfp4(const uint16_t* w_bf16, int64_t rows, int64_t cols, const float* s2,
                          const uint8_t* map, int64_t tile_rows, int64_t tile_cols, uint8_t* codes,
                          uint8_t* scales, uint16_t* w_deq, void* stream) {
    const focus_mixfp4_desc d = {w_bf16, rows, cols, s2, map, tile_rows, tile_cols, codes, scales, w_deq};
    int st = check_quant_mix(d);
    if (st != FOCUS_OK) return st;
    return run_quantize_mix(&d, 1, (hipStream_t)stream);
}

int focus_quantize_mixfp4_many(const focus_mixfp4_desc* descs, int n, void* stream) {
    if (n < 0) return FOCUS_ERR_RANGE;
    if (n > 0 && !descs) return FOCUS_ERR_NULL;
    for (int i = 0; i < n; ++i) {
        int st = check_quant_mix(descs[i]);
        if (st != FOCUS_OK) return st;
    }
    return run_quantize_mix(descs, n, (hipStream_t)stream);
}

int focus_dequantize_mixfp4(const uint8_t* codes, const uint8_t* scales, const float* s2,
                            const uint8_t* map, int64_t rows, int64_t cols, int64_t tile_rows,
                            int64_t tile_cols, uint16_t* out, void* stream) {
    int st = shape_2d(rows, cols);
    if (st != FOCUS_OK) return st;
    if (tile_rows < 1 || tile_cols < 16 || tile_cols % 16 != 0) return FOCUS_ERR_SHAPE;
    if (rows % tile_rows != 0 || cols % tile_cols != 0) return FOCUS_ERR_SHAPE;
    if (rows == 0 || cols == 0) return FOCUS_OK;
    if (rows * (cols / 16) >= kMaxMixBlocks) return FOCUS_ERR_RANGE;
    if (!codes || !scales || !s2 || !map || !out) return FOCUS_ERR_NULL;
    if (!aligned(codes, 8) || !aligned(s2, 4) || !aligned(out, 16)) return FOCUS_ERR_ALIGN;
    focus::MixDequantBatch bt;
    bt.n = 1;
    bt.codes[0] = reinterpret_cast<const uint2*>(codes);
    bt.scales[0] = scales;
    bt.s2[0] = s2;
    bt.out[0] = reinterpret_cast<uint4*>(out);
    bt.nb_row[0] = cols / 16;
    bt.nblk[0] = rows * (cols / 16);
    bt.per_row[0] = 0;
    bt.map[0] = map;
    bt.tiles_per_row[0] = (uint32_t)(cols / tile_cols);
    uint32_t s0, s1, sh2;
    div_magic_host((uint32_t)(cols / 16), bt.mul[0][0], s0);
    div_magic_host((uint32_t)tile_rows, bt.mul[0][1], s1);
    div_magic_host((uint32_t)(tile_cols / 16), bt.mul[0][2], sh2);
    bt.sh[0] = s0 | (s1 << 8) | (sh2 << 16);
    return hip_status(focus::launch_dequantize_mix(bt, (hipStream_t)stream));
}

int64_t focus_nvfp4_linear_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0 || M > kMaxTokens || N > kMaxTokens || K > ((int64_t)1 << 40)) return 0;
    if (N > kMaxElems / M / 4) return 0;
    int64_t cus = 0;
    if (focus::nvfp4_linear_cus(cus) != hipSuccess) return -1;
    const int64_t splits = focus::nvfp4_linear_splits(M, N, K, INT64_MAX, cus);
    return splits > 1 ? splits * M * N * 4 : 0;
}

namespace {

int check_linear(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_s2, int x_s2_per_row,
                 int64_t M, const uint8_t* w_codes, const uint8_t* w_scales, const float* w_s2, int64_t N,
                 int64_t K, const void* y, int y_dtype) {
    if (M < 0 || N < 0 || K < 0 || K % 16 != 0) return FOCUS_ERR_SHAPE;
    if (M > kMaxTokens || N > kMaxTokens || K > ((int64_t)1 << 40)) return FOCUS_ERR_SHAPE;
    if ((M != 0 && K > kMaxElems / M) || (N != 0 && K > kMaxElems / N) ||
        (M != 0 && N > kMaxElems / M))
        return FOCUS_ERR_SHAPE;
    if ((x_s2_per_row != 0 && x_s2_per_row != 1) || (y_dtype != 0 && y_dtype != 1)) return FOCUS_ERR_RANGE;
    if (M == 0 || N == 0) return FOCUS_OK;
    if (focus::nvfp4_linear_workgroups(M, N, INT64_MAX) >= ((int64_t)1 << 24)) return FOCUS_ERR_RANGE;
    if (!x_s2 || !w_s2 || !y || (K > 0 && (!x_codes || !x_scales || !w_codes || !w_scales)))
        return FOCUS_ERR_NULL;
    if (!aligned(x_codes, 8) || !aligned(w_codes, 8) || !aligned(x_s2, 4) || !aligned(w_s2, 4) ||
        !aligned(y, y_dtype == 0 ? 4 : 2))
        return FOCUS_ERR_ALIGN;
    return FOCUS_OK;
}

int run_linear(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_s2, int x_s2_per_row, int64_t M,
               const uint8_t* w_codes, const uint8_t* w_scales, const float* w_s2, int64_t N, int64_t K, void* y,
               int y_dtype, float* workspace, int64_t workspace_bytes, hipStream_t stream) {
    const focus::GemmArgs a = {x_codes, x_scales, x_s2, x_s2_per_row, M,    w_codes, w_scales, w_s2,
                               N,       K,        y,    workspace,    workspace ? workspace_bytes : 0, 1, 1};
    const bool fast = K > 0 && K % 64 == 0 && aligned(x_codes, 16) && aligned(w_codes, 16) && aligned(x_scales, 4) &&
                      aligned(w_scales, 4);
    return hip_status(focus::launch_nvfp4_linear(a, fast, y_dtype == 1, stream));
}

}  // namespace

int focus_nvfp4_linear(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_s2,
                       int x_s2_per_row, int64_t M, const uint8_t* w_codes, const uint8_t* w_scales,
                       const float* w_s2, int64_t N, int64_t K, void* y, int y_dtype, float* workspace,
                       int64_t workspace_bytes, void* stream) {
    int st = check_linear(x_codes, x_scales, x_s2, x_s2_per_row, M, w_codes, w_scales, w_s2, N, K, y, y_dtype);
    if (st != FOCUS_OK) return st;
    if (workspace_bytes < 0) return FOCUS_ERR_RANGE;
    if (M == 0 || N == 0) return FOCUS_OK;
    if (!aligned(workspace, 4)) return FOCUS_ERR_ALIGN;
    return run_linear(x_codes, x_scales, x_s2, x_s2_per_row, M, w_codes, w_scales, w_s2, N, K, y, y_dtype,
                      workspace, workspace_bytes, (hipStream_t)stream);
}

int focus_nvfp4_linear_grouped(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_s2,
                               int x_s2_per_row, int64_t M, int64_t K, const focus_linear_weight* weights,
                               int n, int y_dtype, float* workspace, int64_t workspace_bytes, void* stream) {
    if (n < 0) return FOCUS_ERR_RANGE;
    if (n > 0 && !weights) return FOCUS_ERR_NULL;
    if (workspace_bytes < 0) return FOCUS_ERR_RANGE;
    for (int i = 0; i < n; ++i) {
        const focus_linear_weight& w = weights[i];
        int st = check_linear(x_codes, x_scales, x_s2, x_s2_per_row, M, w.w_codes, w.w_scales, w.w_s2, w.N, K, w.y,
                              y_dtype);
        if (st != FOCUS_OK) return st;
    }
    if (M == 0 || n == 0) return FOCUS_OK;
    if (!aligned(workspace, 4)) return FOCUS_ERR_ALIGN;
    if (M > focus::kLinearDecodeMaxM) {
        // the tiled kernel, one weight after the other (stream-ordered, so
        // they may share the workspace)
        for (int i = 0; i < n; ++i) {
            const focus_linear_weight& w = weights[i];
            if (w.N == 0) continue;
            int st = run_linear(x_codes, x_scales, x_s2, x_s2_per_row, M, w.w_codes, w.w_scales, w.w_s2, w.N, K,
                                w.y, y_dtype, workspace, workspace_bytes, (hipStream_t)stream);
            if (st != FOCUS_OK) return st;
        }
        return FOCUS_OK;
    }
    const focus::GemmArgs a = {x_codes, x_scales, x_s2, x_s2_per_row, M, nullptr, nullptr, nullptr,
                               0,       K,        nullptr, nullptr, 0, 1, 1};
    bool fast = K > 0 && K % 64 == 0 && aligned(x_codes, 16) && aligned(x_scales, 4);
    focus::GemvMembers mem = {};
    for (int i = 0; i <= n; ++i) {
        const bool end = i == n;
        if (!end && weights[i].N == 0) continue;
        if (mem.n > 0 && (end || mem.n == focus::kGemvMaxMembers)) {
            int st = hip_status(focus::launch_nvfp4_linear_grouped(a, mem, fast, y_dtype == 1, (hipStream_t)stream));
            if (st != FOCUS_OK) return st;
            mem.n = 0;
            fast = K > 0 && K % 64 == 0 && aligned(x_codes, 16) && aligned(x_scales, 4);
        }
        if (end) break;
        const focus_linear_weight& w = weights[i];
        const int j = mem.n++;
        mem.wc[j] = w.w_codes;
        mem.ws[j] = w.w_scales;
        mem.ws2[j] = w.w_s2;
        mem.y[j] = w.y;
        mem.N[j] = w.N;
        fast = fast && aligned(w.w_codes, 16) && aligned(w.w_scales, 4);
    }
    return FOCUS_OK;
}

int64_t focus_nvfp4_linear_scratch_bytes(void) { return focus::kLinearScratchBytes; }

int focus_nvfp4_linear_noalloc(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_s2,
                               int x_s2_per_row, int64_t M, const uint8_t* w_codes, const uint8_t* w_scales,
                               const float* w_s2, int64_t N, int64_t K, void* y, int y_dtype, void* stream) {
    int st = check_linear(x_codes, x_scales, x_s2, x_s2_per_row, M, w_codes, w_scales, w_s2, N, K, y, y_dtype);
    if (st != FOCUS_OK) return st;
    if (M == 0 || N == 0) return FOCUS_OK;
    float* scratch = nullptr;
    if (focus::nvfp4_linear_scratch(&scratch) != hipSuccess) return FOCUS_ERR_HIP;
    return run_linear(x_codes, x_scales, x_s2, x_s2_per_row, M, w_codes, w_scales, w_s2, N, K, y, y_dtype,
                      scratch, focus::kLinearScratchBytes, (hipStream_t)stream);
}

}  // extern "C"
