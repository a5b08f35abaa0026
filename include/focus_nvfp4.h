/*
 * focus_nvfp4.h -- C ABI of libfocus_nvfp4, the FOCUS NVFP4 quantizer for
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed.  "FOCUS NVFP4 scales for Llama-3.2-1B-Instruct (our
 * reproduction)", section "What this is", gives the method: per weight
 * tensor W [out_features, in_features] a frozen FP32 tensor scale s2 (field
 * table, row s2), per 16 consecutive elements along in_features an FP32
 * block factor m (row m), per 8-element half of a block an FP32 logit q
 * (row q), and three equations:
 *     S_b  = e4m3(clamp(max|w_b| * m_b / (6 * s2), 2^-6, 448))
 *     c_i  = E2M1(clamp(w_i / (S_b * sigmoid(q_k) * s2), -6, 6))
 *     w'_i = c_i * S_b * s2
 * with E2M1 rounded to nearest, ties to even, and a block whose scaled
 * maximum is zero taking scale 1 before the clamp.  The stored result is
 * plain NVFP4: E2M1 codes, one E4M3 scale byte per 16 elements, one FP32
 * scale per tensor (same section, paragraph after the equations).  The same
 * page quantizes activations with one scale per token.
 *
 * Arithmetic contract.  Every operation is one IEEE binary32 operation with
 * round-to-nearest-even, in the order printed above: t = (a*m)/(6*s2),
 * d = (S*sig)*s2, x = w/d, w' = bf16((c*S)*s2); sigmoid(q) = 1/(1+expf(-q))
 * with expf correctly rounded.  E4M3 is the OCP E4M3FN format (max 448).
 * Where the page is silent:
 *   - codes are packed two per byte, element 2j in the low nibble;
 *   - scale bytes are linear, row-major [rows, cols/16];
 *   - a negative element that rounds to zero keeps its sign (code 0x8);
 *   - sub-block k (0: elements 0-7, 1: elements 8-15) of block b of row r
 *     uses q[r, 2b+k];
 *   - s2 == 0 (an all-zero tensor or token) gives scale byte 0x38 (1.0) for
 *     every block and signed-zero codes.
 *
 * Conventions for every call.
 *   - All data pointers are DEVICE pointers on the current HIP device,
 *     allocated and owned by the caller; the library allocates nothing and
 *     keeps no state.  Tensors are dense and row-major.
 *   - BF16 data is passed as uint16_t bit patterns.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call is
 *     asynchronous and stream-ordered; none synchronizes.
 *   - Arguments are validated on the host before any HIP call.  A failed
 *     check returns an error status and leaves every output untouched.
 *     FOCUS_ERR_HIP reports a failed kernel launch (or a failed device
 *     query): each launch's own status is checked, so an error left by an
 *     earlier, unrelated HIP call is neither reported nor cleared.
 *   - Value preconditions are documented, not checked (a check would need a
 *     device-to-host round trip): inputs finite; s2 finite and >= 0; the
 *     denominators (S_b*sigmoid(q_k))*s2 nonzero, which holds for
 *     q > -30 and amax|W| > 2^-100.  q = +inf is allowed (sigmoid = 1).
 *   - An empty tensor (rows == 0 or cols == 0) is a no-op returning FOCUS_OK
 *     (focus_tensor_scale with numel == 0 writes s2 = 0).
 */
#ifndef FOCUS_NVFP4_H
#define FOCUS_NVFP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FOCUS_NVFP4_ABI_VERSION 1

typedef enum focus_status {
    FOCUS_OK = 0,
    FOCUS_ERR_NULL = 1,   /* a required pointer is NULL */
    FOCUS_ERR_SHAPE = 2,  /* negative size, cols % 16 != 0, or size overflow */
    FOCUS_ERR_ALIGN = 3,  /* a pointer is not aligned as documented */
    FOCUS_ERR_HIP = 4,    /* a HIP launch failed */
    FOCUS_ERR_RANGE = 5   /* an argument is outside its documented range */
} focus_status;

/* Returns FOCUS_NVFP4_ABI_VERSION of the built library. */
int focus_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* focus_status_string(int status);

/*
 * Tensor scale (field table, row s2): s2 = amax|W| / (6*448), one binary32
 * division by 2688.  The maximum is exact (an integer maximum over the BF16
 * magnitude bits).
 *   w_bf16    [numel] BF16, 16-byte aligned.
 *   numel     >= 0 elements (any count).
 *   s2_out    one float, 4-byte aligned; also the accumulator of the
 *             reduction, so it must not alias w.
 *   amax_out  one float or NULL; receives amax|W|.
 * Three kernels on `stream`: clear, reduce (atomic max), finalize.
 */
int focus_tensor_scale(const uint16_t* w_bf16, int64_t numel,
                       float* s2_out, float* amax_out, void* stream);

/*
 * The quantizer: equations S_b, c_i and (optionally) w'_i.
 *   w_bf16  [rows, cols] BF16, cols % 16 == 0, 16-byte aligned.
 *   m       [rows, cols/16] FP32, 4-byte aligned, or NULL for m = 1.
 *   q       [rows, cols/8] FP32, 8-byte aligned, or NULL for sigmoid = 1.
 *   s2      one FP32 (device pointer), e.g. written by focus_tensor_scale.
 *   codes   [rows, cols/2] bytes out, 8-byte aligned.
 *   scales  [rows, cols/16] E4M3 bytes out.
 *   w_deq   [rows, cols] BF16 out, 16-byte aligned, or NULL to skip the
 *           dequantized output.
 * One kernel launch.  Outputs must not overlap inputs.
 */
int focus_quantize(const uint16_t* w_bf16, int64_t rows, int64_t cols,
                   const float* m, const float* q, const float* s2,
                   uint8_t* codes, uint8_t* scales, uint16_t* w_deq,
                   void* stream);

/*
 * Dequantize stored NVFP4 data (equation w'_i): out = bf16((c*S)*s2).
 *   codes   [rows, cols/2] bytes, 8-byte aligned; scales [rows, cols/16].
 *   s2      s2_per_row == 0: one float used for every row (weights);
 *           s2_per_row == 1: [rows] floats, one per row (activations).
 *   out     [rows, cols] BF16, 16-byte aligned.
 * One kernel launch.  Bitwise equal to focus_quantize's w_deq.
 */
int focus_dequantize(const uint8_t* codes, const uint8_t* scales,
                     const float* s2, int s2_per_row,
                     int64_t rows, int64_t cols, uint16_t* out, void* stream);

/*
 * Per-token activation quantization (one scale per token, section "What
 * this is"): for each row t of X [tokens, hidden], s2_t = amax|x_t| / 2688,
 * then the quantizer with m = 1 and sigmoid = 1.
 *   x_bf16  [tokens, hidden] BF16, hidden % 16 == 0, 16-byte aligned.
 *   codes   [tokens, hidden/2] out, 8-byte aligned.
 *   scales  [tokens, hidden/16] out.
 *   s2_out  [tokens] FP32 out.
 *   x_deq   [tokens, hidden] BF16 out, 16-byte aligned, or NULL.
 * One kernel launch (each wavefront quantizes whole token rows).
 */
int focus_quantize_act_per_token(const uint16_t* x_bf16, int64_t tokens, int64_t hidden,
                                 uint8_t* codes, uint8_t* scales, float* s2_out,
                                 uint16_t* x_deq, void* stream);

/*
 * FourOverSix (NVFP4 with adaptive block scale), the FOCUS page's activation
 * protocol and baseline ("FOCUS NVFP4 scales for Llama-3.2-1B-Instruct (our
 * reproduction)", sections "Calibration" and "Perplexity"): plain NVFP4
 * (m = 1, no relaxation) in which each 16-element block's scale maps the
 * block maximum to 6 or to 4, whichever gives the lower error.  Readings
 * where the page is silent: error = binary32 sum, in element order, of
 * (w - (c*S)*s2)^2; the 4-candidate only when strictly lower (ties keep 6);
 * s2 = amax / (6*448) as for NVFP4.  Outputs and rules as focus_quantize /
 * focus_quantize_act_per_token (codes, E4M3 scale bytes, optional BF16 w').
 */
int focus_quantize_fo6(const uint16_t* w_bf16, int64_t rows, int64_t cols, const float* s2,
                       uint8_t* codes, uint8_t* scales, uint16_t* w_deq, void* stream);

int focus_quantize_act_per_token_fo6(const uint16_t* x_bf16, int64_t tokens, int64_t hidden,
                                     uint8_t* codes, uint8_t* scales, float* s2_out,
                                     uint16_t* x_deq, void* stream);

/*
 * FOCUS on MXFP4 (the technical summary of the FOCUS paper, section
 * "Methodologie": the method on MXFP4's 32-element blocks with an E8M0 scale
 * and relaxed sub-blocks of 8).  Readings where the pages are silent: block
 * scale = the OCP Microscaling rule applied to the scaled maximum,
 * S_b = 2^(floor(log2(max|w_b| * m_b)) - 2), exponent clamped to [-127, 127],
 * a zero scaled maximum giving 1; no tensor scale;
 * c_i = E2M1(clamp(w_i / (S_b * sigmoid(q_k)), -6, 6)); w' = BF16(c * S_b).
 *   w_bf16  [rows, cols] BF16, cols % 32 == 0, 16-byte aligned.
 *   m       [rows, cols/32] FP32 or NULL;  q [rows, cols/8] FP32 or NULL
 *           (sub-block k = 0..3 of block b: q[r, 4b + k]).
 *   codes   [rows, cols/2] (element 2j low nibble);  scales [rows, cols/32]
 *           E8M0 bytes (exponent + 127);  w_deq [rows, cols] BF16 or NULL.
 * focus_quantize_mx_many takes focus_quant_desc entries whose s2 is ignored.
 * focus_dequantize_mx: out = BF16(c * 2^(byte - 127)).
 */
int focus_quantize_mx(const uint16_t* w_bf16, int64_t rows, int64_t cols, const float* m,
                      const float* q, uint8_t* codes, uint8_t* scales, uint16_t* w_deq,
                      void* stream);

int focus_dequantize_mx(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                        uint16_t* out, void* stream);

/*
 * Batched calls.  A model holds many linears (112, 224 or 560 for the Llama
 * sets); one launch per tensor leaves the GPU idle between short kernels.
 * These calls take a HOST array of descriptors (read during the call only,
 * so it may be freed on return) and launch one kernel per run of up to 32
 * tensors (three small kernels per run for the tensor scale).  Each
 * descriptor follows the rules of the matching single call; all descriptors
 * are validated before anything is launched, and the first invalid one
 * decides the returned status.  n == 0 is a no-op.  Output buffers of
 * different descriptors must not overlap.
 */
typedef struct focus_scale_desc {
    const uint16_t* w_bf16;  /* [numel] BF16, 16-byte aligned */
    int64_t numel;
    float* s2_out;           /* one float; also the reduction accumulator */
    float* amax_out;         /* one float or NULL */
} focus_scale_desc;

int focus_tensor_scale_many(const focus_scale_desc* descs, int n, void* stream);

typedef struct focus_quant_desc {
    const uint16_t* w_bf16;  /* [rows, cols] BF16 */
    int64_t rows, cols;
    const float* m;          /* [rows, cols/16] or NULL */
    const float* q;          /* [rows, cols/8] or NULL */
    const float* s2;         /* one float */
    uint8_t* codes;          /* [rows, cols/2] */
    uint8_t* scales;         /* [rows, cols/16] */
    uint16_t* w_deq;         /* [rows, cols] or NULL */
} focus_quant_desc;

int focus_quantize_many(const focus_quant_desc* descs, int n, void* stream);

typedef struct focus_dequant_desc {
    const uint8_t* codes;    /* [rows, cols/2] */
    const uint8_t* scales;   /* [rows, cols/16] */
    const float* s2;         /* one float, or [rows] when s2_per_row == 1 */
    int s2_per_row;
    int64_t rows, cols;
    uint16_t* out;           /* [rows, cols] BF16 */
} focus_dequant_desc;

int focus_dequantize_many(const focus_dequant_desc* descs, int n, void* stream);

/* Batched FourOverSix of weights: descriptors as for focus_quantize_many with
 * m and q NULL (FOCUS_ERR_RANGE otherwise). */
int focus_quantize_fo6_many(const focus_quant_desc* descs, int n, void* stream);

/* Batched FOCUS on MXFP4 (cols % 32 == 0; s2 ignored). */
int focus_quantize_mx_many(const focus_quant_desc* descs, int n, void* stream);

/*
 * FlipQuant MixFP4 ("Llama-3.1-8B-Instruct FlipQuant MixFP4 maps", section
 * "What this is", first paragraph and the tile table): NVFP4 (16-element
 * blocks, E4M3 block scale, FP32 tensor scale s2) in which a map with one
 * entry per weight tile of tile_rows x tile_cols (output rows x input
 * columns; the page's maps use 8x64, 16x64 and 256x64) chooses the element
 * format of every block in the tile: a set entry stores E0M3 (uniform levels
 * 0..7), a clear one E2M1 with the FourOverSix scale rule (as
 * focus_quantize_fo6).  Readings where the page is silent: an E0M3 block's
 * scale maps the block maximum to 7, S = e4m3(clamp(max|w_b| / (7*s2),
 * 2^-6, 448)) with a zero maximum giving 1; its code is the sign (bit 3)
 * and the nearest integer 0..7 (ties to even) to |clamp(w / (S*s2), -7, 7)|;
 * w' = BF16((c*S)*s2) with c the signed level (E2M1 value or E0M3 level);
 * binary32 arithmetic throughout; s2 = amax / (6*448) as for NVFP4.
 *   w_bf16   [rows, cols] BF16, 16-byte aligned.
 *   s2       one float (from focus_tensor_scale).
 *   map      [rows/tile_rows, cols/tile_cols] bytes, row-major, nonzero = E0M3
 *            (device memory, like every data pointer).
 *   tile_rows >= 1, tile_cols a positive multiple of 16, dividing rows and
 *            cols (FOCUS_ERR_SHAPE otherwise); rows * cols / 16 < 2^31
 *            (FOCUS_ERR_RANGE otherwise).
 *   codes    [rows, cols/2], E2M1 or E0M3 nibbles as the tile's entry says
 *            (element 2j in the low nibble);  scales [rows, cols/16] E4M3;
 *   w_deq    [rows, cols] BF16 or NULL.
 */
int focus_quantize_mixfp4(const uint16_t* w_bf16, int64_t rows, int64_t cols, const float* s2,
                          const uint8_t* map, int64_t tile_rows, int64_t tile_cols, uint8_t* codes,
                          uint8_t* scales, uint16_t* w_deq, void* stream);

typedef struct focus_mixfp4_desc {
    const uint16_t* w_bf16;  /* [rows, cols] BF16 */
    int64_t rows, cols;
    const float* s2;         /* one float */
    const uint8_t* map;      /* [rows/tile_rows, cols/tile_cols] */
    int64_t tile_rows, tile_cols;
    uint8_t* codes;          /* [rows, cols/2] */
    uint8_t* scales;         /* [rows, cols/16] */
    uint16_t* w_deq;         /* [rows, cols] or NULL */
} focus_mixfp4_desc;

/* Batched MixFP4, with the rules of the batched calls above. */
int focus_quantize_mixfp4_many(const focus_mixfp4_desc* descs, int n, void* stream);

/* Dequantize stored MixFP4 (same page and readings): out = BF16((c*S)*s2)
 * with c the E0M3 level of a code in a tile whose map entry is nonzero and
 * its E2M1 value otherwise.  codes [rows, cols/2] (8-byte aligned), scales
 * [rows, cols/16], s2 one float, map and tiles as focus_quantize_mixfp4,
 * out [rows, cols] BF16 (16-byte aligned); the shape and range rules of
 * focus_quantize_mixfp4. */
int focus_dequantize_mixfp4(const uint8_t* codes, const uint8_t* scales, const float* s2,
                            const uint8_t* map, int64_t rows, int64_t cols, int64_t tile_rows,
                            int64_t tile_cols, uint16_t* out, void* stream);

/*
 * The NVFP4 linear layer, the consumer of the stored format ("FOCUS NVFP4
 * scales for Llama-3.2-1B-Instruct (our reproduction)": section "What this
 * is" -- the deployed model is plain NVFP4 on standard NVFP4 kernels -- and
 * section "Perplexity" -- NVFP4 weights with one FP32 scale per tensor and
 * NVFP4 activations with one scale per token):
 *     Y[t, o] = s2x[t] * s2w * sum_k (cx[t,k] * Sx[t,k/16]) * (cw[o,k] * Sw[o,k/16])
 * c the E2M1 value of a code, S the E4M3 value of a block's scale byte.
 *   x_codes  [M, K/2], x_scales [M, K/16]   activations, e.g. from
 *            focus_quantize_act_per_token(_fo6) (element 2j in the low nibble)
 *   x_s2     [M] when x_s2_per_row == 1, else one float
 *   w_codes  [N, K/2], w_scales [N, K/16], w_s2 one float: a quantized weight
 *            [out_features = N, in_features = K]
 *   y        [M, N] row-major, FP32 (y_dtype 0) or BF16 (y_dtype 1)
 *   K % 16 == 0; M, N <= 2^31; codes 8-byte aligned, y aligned to its type.
 * Arithmetic: each c*S is exact in FP16 and each product exact in FP32; the
 * sum over k is accumulated in FP32 by the matrix cores (order unspecified),
 * then multiplied by RN32(s2x[t] * s2w) and, for BF16 output, rounded once
 * to nearest even.  |Y - exact| <= (about K * 2^-24) * sum_k |products| *
 * s2x * s2w (+ half a BF16 ulp of Y).  K == 0 writes zeros.
 */
int focus_nvfp4_linear(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_s2,
                       int x_s2_per_row, int64_t M, const uint8_t* w_codes, const uint8_t* w_scales,
                       const float* w_s2, int64_t N, int64_t K, void* y, int y_dtype, float* workspace,
                       int64_t workspace_bytes, void* stream);

/* Workspace for focus_nvfp4_linear.  When an [M, N] output has too few tiles
 * to fill the GPU, the sum over k is split into ranges whose FP32 partials
 * [ranges, M, N] go to `workspace` (device memory owned by the caller,
 * 4-byte aligned), then summed in order, scaled and converted by a second
 * kernel (deterministic).  The call splits only as far as `workspace_bytes`
 * allows (NULL or 0: no split; results then differ from a split call only
 * by the FP32 summation order).  This returns the bytes for the full split
 * on the current device (0 when none helps, or when a size is out of range);
 * the split depends on the device's compute-unit count, and -1 means the
 * query of that count failed (the HIP error is left for the caller to read). */
int64_t focus_nvfp4_linear_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * Several NVFP4 weights that share one activation X (a layer's q, k and v
 * projections; gate and up), as in focus_nvfp4_linear for each of them:
 *     y_i [M, N_i] = X' W_i'^T        (same section of the same page)
 * With few tokens (M <= 128) the layer streams W, and one launch per weight
 * would cost a launch each: here every run of up to 8 weights is one launch
 * of the decode kernel, whose workgroups take the weights' output columns in
 * turn (no k split, so no workspace is used).  With more tokens the weights
 * run one after the other as focus_nvfp4_linear calls on `stream`, sharing
 * the workspace (caller-owned, as for focus_nvfp4_linear).
 *   x_codes, x_scales, x_s2, x_s2_per_row, M, K: as focus_nvfp4_linear.
 *   weights  HOST array of n descriptors (read during the call only): codes
 *            [N, K/2], scales [N, K/16], w_s2 one float, output y [M, N] of
 *            type y_dtype (shared by all); N == 0 entries are skipped.
 * Every descriptor is validated (the rules of focus_nvfp4_linear) before
 * anything is launched.  Outputs must not overlap each other or the inputs.
 */
typedef struct focus_linear_weight {
    const uint8_t* w_codes;   /* [N, K/2] */
    const uint8_t* w_scales;  /* [N, K/16] */
    const float* w_s2;        /* one float */
    int64_t N;
    void* y;                  /* [M, N] FP32 or BF16 */
} focus_linear_weight;

int focus_nvfp4_linear_grouped(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_s2,
                               int x_s2_per_row, int64_t M, int64_t K,
                               const focus_linear_weight* weights, int n, int y_dtype,
                               float* workspace, int64_t workspace_bytes, void* stream);

/*
 * focus_nvfp4_linear without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The caller passes the operands and y
 * exactly as for focus_nvfp4_linear; the split-k partials go to a scratch
 * array that the library holds in device memory, one per GPU, from the
 * library's load until the process ends, of focus_nvfp4_linear_scratch_bytes()
 * bytes (64 MiB).  The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); its first call on a device looks up that
 * device's address of the array once.
 *   Sizes: any M, N, K that focus_nvfp4_linear accepts.  The k split is
 *   limited to the ranges whose partials fit in the scratch (as when
 *   focus_nvfp4_linear is given that many workspace bytes), so no call
 *   needs more than the scratch holds and no size is rejected for it; the
 *   result equals focus_nvfp4_linear's with a workspace of
 *   min(focus_nvfp4_linear_workspace_bytes(M, N, K), scratch bytes) bit for
 *   bit.  Nothing in the scratch has to start at zero (every partial that the
 *   finalize reads is written first by the same call).
 *   Concurrency: every call on one GPU shares that GPU's scratch, which keeps
 *   the last call's contents.  Calls that may overlap on one GPU (different
 *   streams without ordering between them, several host threads) race on it
 *   and must be serialized by the caller; calls on one stream are ordered.
 *   Errors: the shape, range, NULL and alignment rules of focus_nvfp4_linear;
 *   FOCUS_ERR_HIP if the device or the array's address cannot be queried.
 */
int focus_nvfp4_linear_noalloc(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_s2,
                               int x_s2_per_row, int64_t M, const uint8_t* w_codes,
                               const uint8_t* w_scales, const float* w_s2, int64_t N, int64_t K,
                               void* y, int y_dtype, void* stream);

/* Bytes of the per-GPU scratch array of focus_nvfp4_linear_noalloc. */
int64_t focus_nvfp4_linear_scratch_bytes(void);

#ifdef __cplusplus
}
#endif

#endif /* FOCUS_NVFP4_H */
