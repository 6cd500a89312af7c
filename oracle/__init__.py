"""CPU oracle for block-scaled 4-bit (NVFP4 / MXFP4) quantization, matmul and MoE.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The HIP library never calls it and shares no code, table or constant
generator with it.

What it computes is the plain definition the pages give for the method:

* "vLLM per-format kernel capability matrix derived from source", section
  THE EMULATION COLUMN: the emulated NVFP4/MXFP4 linear kernels dequantize the
  weights, quantize-then-dequantize the activations, and run the linear layer in
  high precision.  That is exactly what ``gemm`` does, in float64.
* "vLLM on the NVIDIA DGX Spark (GB10 / sm_121): A Complete Technical Guide",
  §6.1 (NVFP4 format) and §6.4 (NVFP4 vs MXFP4 table): element, block and
  global-scale formats.
* Same guide, §4.3 and §7.1: the fused-MoE stages (router, quantize-dispatch,
  two expert GEMMs with SwiGLU between, top-k weighted combine).
* "GLM-5.3-Flash on vLLM, on GB10", the mixture-of-experts fault: per-expert
  dequant alpha = weight_scale_2 * input_scale, and a missing activation scale
  that must be refused rather than silently zeroing the experts.

Modules
  formats  value tables and nearest-value encoders (E2M1, E4M3, E8M0), nibble packing
  quant    NVFP4 / MXFP4 quantize and dequantize (activation and weight)
  gemm     dequantize + float64 matmul, W4A4 and W4A16
  moe      top-k softmax routing, permute bookkeeping, the expert chain, combine
  fp8      MXFP8 (e4m3 elements, e8m0 scale per 32) and FP8 W8A8 with per-tensor,
           rowwise (per token / per channel) or 1x128 / 128x128 block scales
           ("vLLM per-format kernel capability matrix derived from source": the MX
           group size, MXFP8 native on gfx95, FP8's three scaling modes)
  mx       MX formats with any element type (e2m1, e2m3, e3m2, e4m3), the 6-bit packing,
           and matmuls whose two operands use different element types (same page: the
           MXFP6 section)

Pins (tests/test_oracle_*.py) tie every function to something outside itself:
closed-form value tables, torch's float8 decoders, hand-worked examples in
``tests/golden``, exact rational arithmetic on tiny GEMMs, invariants and special
cases.  The one part the pages do not fix is the fp32 operation order inside the
NVFP4 activation-scale computation (amax * g / 6, then g / scale): it is a chosen
convention, pinned only by the hand-worked examples -- parity unpinned by the
pages for that order.
"""
