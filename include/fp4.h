/*
 * fp4.h -- C ABI of the block-scaled 4-bit (NVFP4 / MXFP4) matmul library for
 * AMD Instinct MI355X (gfx950).
 *
 * What the operations are (page titles and sections of the pages this library
 * implements):
 *  - "vLLM on the NVIDIA DGX Spark (GB10 / sm_121): A Complete Technical Guide",
 *    §6.1 NVFP4 format: e2m1 elements packed two per byte, one fp8 e4m3 block
 *    scale per 16 contiguous elements along K, and fp32 per-tensor scales folded
 *    into one alpha for the product.
 *  - same guide, §6.4 (NVFP4 vs MXFP4 table): MXFP4 = e2m1 elements, 32-element
 *    blocks, exponent-only e8m0 block scales, no per-tensor scale.
 *  - same guide, §4.3 (b12x) and §7.1 (modular fused MoE): BF16 activations are
 *    quantized to FP4 inside the expert path; the MoE is router -> quantize and
 *    dispatch -> expert GEMMs with SwiGLU between -> top-k weighted combine.
 *  - "vLLM on the DGX Spark, the Hard Way: Seven Months of GB10 Field Notes",
 *    native-FP4 conditions: a W4A4 checkpoint carries 4-bit activations; a
 *    weight-only (W4A16) one has no FP4 activations and multiplies 16-bit
 *    activations by the dequantized weights.
 *  - "GLM-5.3-Flash on vLLM, on GB10": per-expert dequant alpha is
 *    weight_scale_2 * input_scale; a weight-only checkpoint leaves input_scale at
 *    zero, which silently zeroes every routed expert.  This library refuses that
 *    case with FP4_ERR_INPUT_SCALE instead of computing with it.
 *  - "vLLM per-format kernel capability matrix derived from source", THE
 *    EMULATION COLUMN: silent fallback to another precision is the failure to
 *    avoid.  There is one kernel path per (format, mode); the only change of mode
 *    is the opt-in FP4_FLAG_ALLOW_W4A16_FALLBACK, which reports itself through
 *    FP4_OK_FELL_BACK_W4A16.
 *
 * Data layout (all row-major, K contiguous, no padding between rows):
 *  - codes  uint8 [rows, K/2]: element 2i in the low nibble of byte i, 2i+1 in the
 *    high nibble.  Nibble = sign(bit 3) | exponent(bits 2:1, bias 1) | mantissa(bit 0).
 *  - scales uint8 [rows, K/G]: NVFP4 G = 16, OCP e4m3fn codes (bias 7, max 448);
 *    MXFP4 G = 32, e8m0 codes (value 2^(c-127)).
 *  - bf16 activations: raw bfloat16 bits with a row stride in elements.
 *  - value of element k of a row = e2m1(code) * blockscale(k / G); the per-tensor
 *    scales enter only through alpha.
 *
 * Per-tensor scales are HOST fp32 values; they are dequant multipliers:
 *   NVFP4 W4A4 : alpha = weight_scale_2 * input_scale, activations are quantized with
 *                the quantize-direction multiplier 1/input_scale;
 *   NVFP4 W4A16: alpha = weight_scale_2 (input_scale is ignored and may be 0);
 *   MXFP4      : both must be exactly 1.0 (FP4_ERR_FORMAT otherwise).
 *
 * Ownership and threading: every tensor pointer is device memory owned by the
 * caller; the library allocates and frees nothing.  Calls validate on the host,
 * then enqueue kernels on the caller's stream (a hipStream_t passed as void*,
 * NULL = the null stream) and return without waiting; results are valid after the
 * stream synchronizes.  Calls are reentrant; the only process state is a per-device
 * cached architecture check and a thread-local name of the last launched kernel.
 *
 * Errors: every check runs on the host before any launch; on an error nothing is
 * launched and no output is touched.  Checks run in this order: null pointers,
 * shapes, alignment, scales, format rules, then the device (so every error but
 * FP4_ERR_DEVICE / FP4_ERR_LAUNCH can be produced without a GPU).
 */
#ifndef FP4_H
#define FP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP4_OK = 0,
  FP4_OK_FELL_BACK_W4A16 = 1, /* success, but ran weight-only as the caller allowed */
  FP4_ERR_NULL = -1,          /* a required pointer is NULL */
  FP4_ERR_SHAPE = -2,         /* negative size, K not a multiple of G, bad stride, k > E ... */
  FP4_ERR_ALIGN = -3,         /* device pointer not 16-byte aligned, or bf16 stride not a multiple of 8 */
  FP4_ERR_INPUT_SCALE = -4,   /* W4A4 input_scale not finite or outside [2^-100, 2^100] (incl. 0) */
  FP4_ERR_WEIGHT_SCALE = -5,  /* weight_scale_2 not finite or outside [2^-100, 2^100] */
  FP4_ERR_FORMAT = -6,        /* unknown enum value, or an MXFP4 per-tensor scale != 1 */
  FP4_ERR_WORKSPACE = -7,     /* workspace NULL or smaller than the reported size */
  FP4_ERR_DEVICE = -8,        /* no HIP device, or the current device is not gfx950 */
  FP4_ERR_LAUNCH = -9         /* a kernel launch reported an error */
} fp4_status;

typedef enum { FP4_NVFP4 = 0, FP4_MXFP4 = 1 } fp4_format;
typedef enum { FP4_W4A4 = 0, FP4_W4A16 = 1 } fp4_mode;
typedef enum { FP4_OUT_BF16 = 0, FP4_OUT_F32 = 1 } fp4_out;

/* Opt-in: an NVFP4 W4A4 call whose activation scale is refused runs as W4A16 and
 * returns FP4_OK_FELL_BACK_W4A16 instead of FP4_ERR_INPUT_SCALE. */
#define FP4_FLAG_ALLOW_W4A16_FALLBACK 1u
/* w_codes are in the prepared layout written by fp4_prepare_weights (see there). */
#define FP4_FLAG_PREPARED_WEIGHTS 2u

/*
 * Activation quantization (guide §6.1 / §6.4; quantize-inside-the-kernel of §4.3).
 *   x      : bf16 [M, K] with row stride ldx elements (ldx >= K, ldx % 8 == 0)
 *   codes  : out uint8 [M, K/2];   scales : out uint8 [M, K/G]
 *   NVFP4  : g = 1/input_scale (fp32); per 16-block: amax = max|x|,
 *            sf = fp32(fp32(amax*g)/6), scale = e4m3(sf) (nearest even, saturating
 *            at 448), r = fp32(g/scale), code = e2m1(x*r) (nearest even, saturating
 *            at 6; sign of x kept; all elements signed zero when scale == 0).
 *   MXFP4  : input_scale must be 1; per 32-block E = clamp(floor(log2 amax) - 2,
 *            -127, 127), scale code E+127, code = e2m1(x * 2^-E).
 * Bit-exact: the result is fully determined by the inputs.  K must be a multiple
 * of G.  M == 0 or K == 0 is a valid no-op.
 */
fp4_status fp4_quantize_act(fp4_format fmt, const void* x_bf16, int64_t M, int64_t K,
                            int64_t ldx, float input_scale, uint8_t* codes,
                            uint8_t* scales, void* stream);

/*
 * Weight quantization from fp32 (offline checkpoint preparation; same rules as
 * fp4_quantize_act with input_scale := weight_scale_2, which the caller chooses,
 * e.g. amax(W)/(6*448)).  w: fp32 [N, K], row stride ldw (ldw >= K, ldw % 4 == 0).
 */
fp4_status fp4_quantize_weight(fp4_format fmt, const float* w, int64_t N, int64_t K,
                               int64_t ldw, float weight_scale_2, uint8_t* codes,
                               uint8_t* scales, void* stream);

/*
 * Dense block-scaled matmul  out[m, n] = alpha * sum_k a_hat[m, k] * w_hat[n, k]
 * (the capability matrix's EMULATION COLUMN defines the result: dequantize, QDQ
 * the activations, multiply in high precision; here fp32 accumulation).
 *   W4A4, a_bf16 != NULL : activations quantized on the fly under input_scale
 *                          (needs workspace >= fp4_gemm_workspace_size(...));
 *   W4A4, a_bf16 == NULL : pre-quantized a_codes [M, K/2] / a_scales [M, K/G];
 *   W4A16                : a_bf16 [M, K] is used as is (a_codes ignored).
 *   w_codes [N, K/2], w_scales [N, K/G]; out [M, N] bf16 (round to nearest even)
 *   or fp32 with row stride ldo >= N.
 * Accumulation is fp32 in a fixed order: repeated calls are bitwise identical.
 */
fp4_status fp4_gemm(fp4_format fmt, fp4_mode mode, int64_t M, int64_t N, int64_t K,
                    const void* a_bf16, int64_t lda, const uint8_t* a_codes,
                    const uint8_t* a_scales, const uint8_t* w_codes,
                    const uint8_t* w_scales, float weight_scale_2, float input_scale,
                    void* out, int64_t ldo, fp4_out out_dtype, uint32_t flags,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes fp4_gemm needs for these arguments (0 unless W4A4 with a_bf16). */
size_t fp4_gemm_workspace_size(fp4_format fmt, fp4_mode mode, int64_t M, int64_t K,
                               int has_a_bf16);

/*
 * Workspace bytes with which fp4_gemm runs a W4A4 call fastest: the above, plus, for
 * prefill-sized problems (M > 64 and at least 256 output tiles of 256 x 256), room for
 * both operands' block scales re-laid in the tile kernel's stage order (a small pass
 * before the GEMM; the guide's §4.3 pre-converts scale factors to the MMA's layout).
 * fp4_gemm uses that room when workspace_bytes reaches this size, else it reads the
 * scales row by row: the results are bitwise the same either way.  0 for W4A16.
 */
size_t fp4_gemm_workspace_size_mnk(fp4_format fmt, fp4_mode mode, int64_t M, int64_t N,
                                   int64_t K, int has_a_bf16);

/* Capacity of fp4_gemm_noalloc's per-device scratch array (32 MiB). */
#define FP4_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * fp4_gemm without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, semantics and results as fp4_gemm (the same kernels);
 * the fused W4A4 activation quantization writes into a scratch array the library
 * holds in each device's memory (FP4_NOALLOC_SCRATCH_BYTES, resident until the
 * process ends).  Nothing is allocated or freed by the call.
 *   Limit: the fused case needs fp4_gemm_workspace_size(...) <= the capacity, i.e.
 *   M*K/2 + M*K/G bytes (each part rounded up to 256) -- about 59 M activation
 *   elements for NVFP4 (M = 8192 at K = 7168); larger calls return FP4_ERR_WORKSPACE
 *   before any launch.  Pre-quantized W4A4 and W4A16 calls use no scratch.
 *   Races: every call on one device shares that device's array, so calls that can
 *   overlap on one device (different streams, or threads without ordering) race on
 *   it; calls ordered on one stream do not.  The array keeps the last call's contents.
 *   The first call on a device resolves the array's device address (outside stream
 *   capture: make one call before capturing).
 */
fp4_status fp4_gemm_noalloc(fp4_format fmt, fp4_mode mode, int64_t M, int64_t N, int64_t K,
                            const void* a_bf16, int64_t lda, const uint8_t* a_codes,
                            const uint8_t* a_scales, const uint8_t* w_codes,
                            const uint8_t* w_scales, float weight_scale_2, float input_scale,
                            void* out, int64_t ldo, fp4_out out_dtype, uint32_t flags,
                            void* stream);

/*
 * Router (guide §7.1 [Router]; top-k softmax).  logits fp32 [T, E] (device);
 * topk_ids int32 [T, k]: the k largest logits, largest first, ties to the lower
 * expert index; topk_w fp32 [T, k]: softmax over all E experts at those ids,
 * divided by their sum when renormalize != 0.  1 <= k <= min(E, 32), E <= 1024.
 */
fp4_status fp4_moe_topk_softmax(const float* logits, int64_t T, int64_t E, int k,
                                int renormalize, int32_t* topk_ids, float* topk_w,
                                void* stream);

/*
 * Mixture-of-experts layer (guide §7.1 stages, §4.3 fused expert; GLM page alpha):
 *   out[t] = sum_j topk_w[t, j] * expert_{topk_ids[t, j]}(hidden[t]) (+ shared(hidden[t]))
 *   expert(x) = W2 . q2( SiLU(x_hat . W13[0:I]^T * alpha13) * (x_hat . W13[I:2I]^T * alpha13) ) * alpha2
 * W4A4: x_hat = quantized hidden (NVFP4 under a13_scale[e], MXFP4 per 32-block) and
 * q2 = quantize the fp32 intermediate (NVFP4 under a2_scale[e], MXFP4 per block).
 * W4A16: x_hat = hidden, q2 = round to bf16.  alpha13/alpha2 = w*_scale_2 (* a*_scale
 * in NVFP4 W4A4); 1 for MXFP4.
 * Pointer fields are device memory except the per-expert *_scale arrays, which are
 * HOST fp32 [E] (NVFP4; NULL for MXFP4) so they can be checked without a device
 * sync: any NVFP4 W4A4 a13/a2 scale that is zero, negative, non-finite or out of
 * range -> FP4_ERR_INPUT_SCALE (or the whole layer runs W4A16 with
 * FP4_FLAG_ALLOW_W4A16_FALLBACK).  Shared-expert pointers may all be NULL.
 * Expert ids are device data and are not checked on the host: a slot whose id lies
 * outside [0, E) (e.g. the router's output for a token with NaN logits) is dropped
 * -- it contributes nothing to out[t] -- and every kernel stays inside its buffers.
 * Launches: an NVFP4 W4A4 layer without a shared expert, with at most 4 tokens and 32
 * routed slots (H and I multiples of 128, H <= 4096, I <= 2048, E <= 192), runs in two
 * launches (gate/up with the routing and the activation quantization inside, then the
 * down projection with the weighted combine); other layers run dispatch, the two
 * expert GEMMs and the combine as separate launches.  Both write the workspace stages
 * below the same way.
 */
typedef struct {
  fp4_format fmt;
  fp4_mode mode;
  int64_t T, H, I, E;
  int k;
  uint32_t flags;
  const void* hidden_bf16;                   /* [T, H] bf16, row stride H */
  const int32_t* topk_ids;                   /* [T, k] */
  const float* topk_w;                       /* [T, k] */
  const uint8_t *w13_codes, *w13_scales;     /* [E, 2I, H/2], [E, 2I, H/G]; rows [0,I) gate, [I,2I) up */
  const uint8_t *w2_codes, *w2_scales;       /* [E, H, I/2], [E, H, I/G] */
  const float *w13_scale_2, *w2_scale_2;     /* host [E] (NVFP4) or NULL (MXFP4) */
  const float *a13_scale, *a2_scale;         /* host [E] (NVFP4 W4A4) or NULL */
  const uint8_t *sh_w13_codes, *sh_w13_scales, *sh_w2_codes, *sh_w2_scales; /* or NULL */
  float sh_w13_scale_2, sh_w2_scale_2, sh_a13_scale, sh_a2_scale;
  void* out_bf16;                            /* [T, H] bf16 */
} fp4_moe_args;

/* Byte offsets of the MoE stage outputs inside the workspace, for inspection by
 * tests; valid after the stream synchronizes following fp4_moe_grouped_gemm.
 * Rows P = T*k routed rows (+ T shared rows) in expert-sorted order. */
typedef struct {
  size_t total_bytes;
  size_t expert_offsets;  /* int32 [E+1]: first sorted row of each expert */
  size_t sorted_rows;     /* int32 [T*k]: flat index t*k+j of each sorted row; positions
                             past the routed count (see dropped ids above) hold -1 */
  size_t inverse;         /* int32 [T*k]: sorted position of flat index t*k+j */
  size_t x_codes;         /* uint8 [rows, H/2] GEMM1 input codes (W4A4) */
  size_t x_scales;        /* uint8 [rows, H/G] */
  size_t gu;              /* fp32 [gu_rows, 2I] gate/up outputs of the parts that do not
                             take the fused SwiGLU epilogue: the routed rows in sorted order
                             (unless swiglu_fused bit 0), then the shared rows (unless bit 1) */
  size_t h_codes;         /* uint8 [T*k + T, I/2] quantized intermediate (W4A4) */
  size_t h_scales;        /* uint8 [T*k + T, I/G] */
  size_t h_bf16;          /* bf16 [T*k + T, I] intermediate (W4A16) */
  size_t y;               /* fp32 [T*k + T, H] expert outputs before the combine */
  int64_t x_rows;         /* rows in x_codes: T (MXFP4) or T*k + T (NVFP4) */
  int64_t gu_rows;        /* rows in gu */
  int32_t swiglu_fused;   /* bit 0: routed rows, bit 1: shared rows have SwiGLU and the
                             requant fused into the gate/up GEMM (W4A4, H and I multiples
                             of 128; on the tiled kernel -- 128-row expert blocks, or more
                             than 64 tokens for the shared expert -- or on the streaming
                             kernel where the plain GEMM would stream too or has at most
                             16 rows, or in the two-launch small layer); their h is
                             written without gu */
} fp4_moe_layout;

size_t fp4_moe_workspace_size(const fp4_moe_args* a);
fp4_status fp4_moe_workspace_layout(const fp4_moe_args* a, fp4_moe_layout* layout);
fp4_status fp4_moe_grouped_gemm(const fp4_moe_args* a, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * One-time weight preparation ("vLLM on the NVIDIA DGX Spark (GB10 / sm_121): A Complete
 * Technical Guide", §4.3: scale factors converted to the MMA layout once, at weight
 * load; §5.3: the block scales repacked for the dequant kernel).  Repacks the codes of
 * one weight matrix into the layout the decode kernels stream, and checks its block
 * scales.
 *   w_codes [N, K/2], w_scales [N, K/G] (the layout above); N % 16 == 0, K % 128 == 0.
 *   prepared_codes: out, fp4_prepared_weight_bytes(N, K) = N * K / 2 bytes: blocks of 16
 *     rows x 128 elements, ordered by row block then K block; inside a block the 16-byte
 *     piece p = 16 q + r (q < 4, r < 16) holds bytes 16 q .. 16 q + 15 of row r's 64.
 *     The scales stay in their own layout and are passed to fp4_gemm unchanged.
 *   check: a caller-owned device int32, overwritten (the validation flag).
 * Validation: a NaN scale code (NVFP4 e4m3 S.1111.111, MXFP4 e8m0 0xFF) fails with
 * FP4_ERR_WEIGHT_SCALE.  This call synchronizes `stream` to read the flag (load-time
 * work: it is not meant for capture); prepared_codes is written either way.
 * Use: fp4_gemm / fp4_gemm_noalloc with FP4_FLAG_PREPARED_WEIGHTS and the prepared
 * codes as w_codes, for W4A4 calls with at most 64 activation rows (the decode kernels,
 * which then read each step of a wave's weights as one contiguous kilobyte); other
 * calls with the flag fail with FP4_ERR_SHAPE (M, N, K) or FP4_ERR_FORMAT (W4A16, or
 * together with FP4_FLAG_ALLOW_W4A16_FALLBACK).
 */
size_t fp4_prepared_weight_bytes(int64_t N, int64_t K);
fp4_status fp4_prepare_weights(fp4_format fmt, const uint8_t* w_codes, const uint8_t* w_scales,
                               int64_t N, int64_t K, uint8_t* prepared_codes, int32_t* check,
                               void* stream);

/* Pure predicate: 1 if the architecture name (e.g. "gfx950:sramecc+:xnack-") is one
 * this library has kernels for, else 0.  No device access.  Every call above checks
 * the current device with it and fails with FP4_ERR_DEVICE instead of launching:
 * "vLLM on the NVIDIA DGX Spark (GB10 / sm_121): A Complete Technical Guide", §2
 * and §6.3 -- an FP4 kernel built for another architecture must fail loudly rather
 * than run. */
int fp4_arch_supported(const char* gcn_arch_name);
/* Static string naming a status code (the error conventions above; the same guide's
 * §6.3 and the GLM page's refused zero activation scale are the failures they name). */
const char* fp4_status_str(fp4_status s);
/* Name of the kernel variant the calling thread launched last ("" if none), so that a
 * caller can see which kernel path ran ("vLLM on the DGX Spark, the Hard Way: Seven
 * Months of GB10 Field Notes", the five-minute model, item 2: the kernel a format
 * ends up on is chosen by a chain whose links fail silently, and the boot log's
 * record of the chosen backend is how that shows). */
const char* fp4_last_kernel(void);

#ifdef __cplusplus
}
#endif
#endif /* FP4_H */
