/*
 * fp8.h -- C ABI of the 8-bit members of the library for AMD Instinct MI355X (gfx950):
 * MXFP8 and FP8 W8A8 quantization and matmul.  Shares the status codes, the output
 * dtype enum, the ownership rules and the error order of fp4.h.
 *
 * What the operations are ("vLLM per-format kernel capability matrix derived from
 * source"):
 *  - its group-size note: every MX format (MXFP4, MXFP6, MXFP8) uses 32-element blocks
 *    along K with an exponent-only (e8m0) scale per block;
 *  - MXFP8, and WHAT IS NATIVE ON AMD: MXFP8 (e4m3 elements) is the MX format with a
 *    native path on gfx95 parts;
 *  - FP8, THREE SCALING MODES: FP8 W8A8 with per-tensor scales, rowwise scales (per
 *    token for activations, per output channel for weights, computed dynamically) or
 *    block scales (1 x 128 activation blocks, 128 x 128 weight blocks).  The page's
 *    engine silently degrades rowwise to per-tensor on parts without per-token
 *    support; here each mode is asked for explicitly and runs as asked, or fails;
 *  - the same page: gfx94-class parts use the FNUZ e4m3 variant; gfx950 uses OCP
 *    e4m3fn (bias 7, max 448, no infinities, S.1111.111 = NaN), the variant here;
 *  - THE EMULATION COLUMN: the matmul's result is defined by dequantizing both
 *    operands and multiplying in high precision (here: fp32 accumulation).
 *
 * Data layout (row-major, K contiguous, no padding between rows):
 *  - codes: uint8 [rows, K], one e4m3fn code per element.
 *  - scales by mode (device memory, owned by the caller):
 *      FP8_MX          uint8 [rows, K/32]   e8m0 codes, value 2^(c-127)
 *      FP8_PER_TENSOR  none: the host fp32 tensor_scale; the scales pointer must be NULL
 *      FP8_ROWWISE     float [rows]         one per activation row / weight row
 *      FP8_BLOCK       activations float [M, K/128]; weights float [ceil(N/128), K/128]
 *                      (block (i, j) = weight rows [128 i, 128 i + 128), columns
 *                      [128 j, 128 j + 128); the last block row holds the rows that exist)
 *  - element value = e4m3(code) * scale of its block / row / tensor.
 *
 * Rounding: every encoding rounds to nearest even and saturates at 448, keeping the sign
 * of the input (a zero scale gives signed zero codes); results are bit-exact, fully
 * determined by the inputs.
 */
#ifndef FP8_H
#define FP8_H

#include "fp4.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FP8_MX = 0, FP8_PER_TENSOR = 1, FP8_ROWWISE = 2, FP8_BLOCK = 3 } fp8_scaling;

/*
 * Activation quantization, bf16 x [M, K] (row stride ldx elements, ldx >= K, ldx % 8 == 0)
 * -> codes [M, K] and scales (layout above).
 *   FP8_MX         : per 32-block E = clamp(floor(log2 amax) - 8, -127, 127) (an all-zero
 *                    block: -127), scale code E + 127, code = e4m3(x * 2^-E).
 *   FP8_PER_TENSOR : code = e4m3(fp32(x / tensor_scale)); tensor_scale is a host fp32 in
 *                    [2^-100, 2^100] (FP4_ERR_INPUT_SCALE otherwise).
 *   FP8_ROWWISE    : s[m] = fp32(amax(row m) / 448), code = e4m3(fp32(x / s[m])).
 *   FP8_BLOCK      : s[m, j] = fp32(amax(x[m, 128 j .. 128 j + 127]) / 448), likewise.
 *   Dynamic modes (MX, rowwise, block) take tensor_scale == 1.0 (FP4_ERR_FORMAT otherwise).
 * K must be a multiple of 32 (MX), 128 (block) or 8 (per-tensor, rowwise).  M == 0 is a
 * valid no-op.  Rowwise and block-weight quantization launch an amax pass first.
 */
fp4_status fp8_quantize_act(fp8_scaling mode, const void* x_bf16, int64_t M, int64_t K,
                            int64_t ldx, float tensor_scale, uint8_t* codes, void* scales,
                            void* stream);

/*
 * Weight quantization from fp32 w [N, K] (row stride ldw, ldw >= K, ldw % 4 == 0), offline
 * preparation.  Same rules as fp8_quantize_act with rows = output channels, except
 * FP8_BLOCK, which reduces amax over 128 x 128 blocks.  FP8_PER_TENSOR takes the caller's
 * tensor_scale (for instance amax(W) / 448); out-of-range: FP4_ERR_WEIGHT_SCALE.
 */
fp4_status fp8_quantize_weight(fp8_scaling mode, const float* w, int64_t N, int64_t K,
                               int64_t ldw, float tensor_scale, uint8_t* codes, void* scales,
                               void* stream);

/*
 * out[m, n] = sum_k a_hat[m, k] * w_hat[n, k], a_hat and w_hat the dequantized operands
 * (codes times their mode's scales), fp32 accumulation, written as bf16 (nearest even)
 * or fp32 with row stride ldo >= N.
 *   a_codes [M, K], w_codes [N, K] in one mode, their scales laid out as above.
 *   FP8_PER_TENSOR: a_tensor_scale and w_tensor_scale are the host scales (product
 *   fp32(a * w) applied once per output); every other mode takes 1.0 for both
 *   (FP4_ERR_FORMAT otherwise) and non-NULL scale arrays.
 *   K must be a positive multiple of 128 (the kernels advance K in 128-deep stages).
 *   M == 0 or N == 0 is a valid no-op.
 * Kernels: M <= 32 a decode kernel, 32 activation rows x 32 weight rows per workgroup
 * (64 weight rows for MX operands above 16 rows), K split over its four waves, each
 * staging its K blocks through LDS; larger M an LDS-tiled kernel, 128 x 256 outputs per
 * workgroup.  Both run on the gfx950 scaled 32x32x64 MFMA with e4m3 operands (MX: the
 * e8m0 codes are the instruction's block scales; the other modes apply their fp32 scales
 * outside it).
 * Pointers must be 16-byte aligned (FP4_ERR_ALIGN).
 */
fp4_status fp8_gemm(fp8_scaling mode, int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                    const void* a_scales, float a_tensor_scale, const uint8_t* w_codes,
                    const void* w_scales, float w_tensor_scale, void* out, int64_t ldo,
                    fp4_out out_dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8_H */
