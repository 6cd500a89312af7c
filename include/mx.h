/*
 * mx.h -- C ABI of the MX block formats of any element type for AMD Instinct MI355X
 * (gfx950): MXFP4, MXFP6 and MXFP8 quantization, and matmuls whose activations and
 * weights may use different MX element types (for instance FP4 weights with FP8
 * activations, or MXFP6 weights with MXFP4 / MXFP6 / MXFP8 activations).  Shares the
 * status codes, the output dtype enum, the ownership rules and the error order of fp4.h.
 *
 * What the operations are ("vLLM per-format kernel capability matrix derived from
 * source"):
 *  - its group-size note: MXFP4, MXFP6 and MXFP8 all use blocks of 32 elements along K
 *    with one exponent-only (e8m0) scale per block;
 *  - MXFP6: MXFP6 weights are accepted with MXFP4, MXFP6 or unquantized activations, so
 *    the two operands of a matmul need not share an element type;
 *  - MXFP8 and WHAT IS NATIVE ON AMD: MXFP8 (e4m3 elements) is native on gfx95 parts;
 *  - THE EMULATION COLUMN: the matmul's result is defined by dequantizing both operands
 *    and multiplying in high precision (here: fp32 accumulation).
 *
 * Element types (OCP MX definitions; the pages name the formats, not their bit fields):
 *   MX_E2M1  4 bits, bias 1, largest 6     (MXFP4)
 *   MX_E2M3  6 bits, bias 1, largest 7.5   (MXFP6)
 *   MX_E3M2  6 bits, bias 3, largest 28    (MXFP6)
 *   MX_E4M3  8 bits, bias 7, largest 448   (MXFP8, OCP e4m3fn)
 *
 * Data layout (row-major, K contiguous, no padding between rows):
 *  - codes: uint8 [rows, K * bits / 8]: e2m1 two per byte, element 2i in the low nibble
 *    of byte i (the MXFP4 layout of fp4.h); e2m3 / e3m2 32 elements in 24 bytes, element
 *    i of a 32-group at bits [6 i, 6 i + 6) of the group's little-endian 192 bits; e4m3
 *    one per byte.
 *  - scales: uint8 [rows, K / 32] e8m0 codes, value 2^(c - 127).
 *  - element value = element(code) * 2^(scale code - 127).
 *
 * Quantization rule (bit-exact, fully determined by the inputs): per 32-block,
 * E = clamp(floor(log2 amax) - emax, -127, 127) with emax = 2 (e2m1, e2m3), 4 (e3m2),
 * 8 (e4m3), an all-zero block E = -127; scale code E + 127; element = the nearest value
 * of x * 2^-E, ties to the even code, saturating at the largest value, the sign of x
 * kept (negative zero too).  Inputs must be finite.
 */
#ifndef MX_H
#define MX_H

#include "fp4.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MX_E2M1 = 0, MX_E2M3 = 1, MX_E3M2 = 2, MX_E4M3 = 3 } mx_elem;

/*
 * Activation quantization: bf16 x [M, K] (row stride ldx elements, ldx >= K, ldx % 8 == 0)
 * -> codes and scales of element type t.  K must be a multiple of 32; M == 0 or K == 0 is
 * a valid no-op.
 */
fp4_status mx_quantize_act(mx_elem t, const void* x_bf16, int64_t M, int64_t K, int64_t ldx,
                           uint8_t* codes, uint8_t* scales, void* stream);

/*
 * Weight quantization from fp32 w [N, K] (row stride ldw, ldw >= K, ldw % 4 == 0), offline
 * preparation; same rule.
 */
fp4_status mx_quantize_weight(mx_elem t, const float* w, int64_t N, int64_t K, int64_t ldw,
                              uint8_t* codes, uint8_t* scales, void* stream);

/*
 * out[m, n] = sum_k a_hat[m, k] * w_hat[n, k] with activations of element type a_t and
 * weights of element type w_t (any of the four each), fp32 accumulation, written as bf16
 * (nearest even) or fp32 with row stride ldo >= N.  MX formats carry no per-tensor scale.
 * K must be a positive multiple of 128 (the kernels advance K in 128-deep stages); M == 0
 * or N == 0 is a valid no-op; pointers must be 16-byte aligned (FP4_ERR_ALIGN).
 * Kernels: M <= 32 a decode kernel, 32 activation rows x 32 weight rows per workgroup
 * (64 weight rows for MX operands above 16 rows), K split over its four waves, each
 * staging its K blocks through LDS; larger M an LDS-tiled kernel, 128 x 256 outputs per
 * workgroup.  Both run on the gfx950 scaled 32x32x64 MFMA, which takes each operand's
 * element type and e8m0 block scales natively.
 */
fp4_status mx_gemm(mx_elem a_t, mx_elem w_t, int64_t M, int64_t N, int64_t K,
                   const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* w_codes,
                   const uint8_t* w_scales, void* out, int64_t ldo, fp4_out out_dtype,
                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MX_H */
