// MX matmuls whose operands use any of the scaled MFMA's element types -- e2m1 (MXFP4),
// e2m3 / e3m2 (MXFP6), e4m3 (MXFP8) -- independently for activations and weights, on the
// engine of scaled_gemm.h ("vLLM per-format kernel capability matrix derived from
// source": the MX group size of 32 for all three; MXFP6 weights with MXFP4, MXFP6 or
// other activations).  The e4m3 x e4m3 pair is the FP8 entry's MX mode and is not
// instantiated here.
#include "scaled_gemm.h"

namespace fp4 {

namespace {

using namespace sg;

#define FP4_MX_CASE(FA, FW, A, W) \
  if (fa == FA && fw == FW) return launch<kF8_MX, FA, FW>(p, s, name, "mx_rows_" A "_" W, "mx_tile_" A "_" W);

}  // namespace

hipError_t launch_mx_gemm(int fa, int fw, const Fp8GemmParams& p, hipStream_t s, const char** name) {
  if (p.M == 0 || p.N == 0) return hipSuccess;
  if (p.K % 128 != 0 || p.K <= 0) return hipErrorInvalidValue;
  if (fa == kE4M3 && fw == kE4M3) return launch_fp8_gemm(kF8_MX, p, s, name);
  FP4_MX_CASE(kE2M1, kE2M1, "e2m1", "e2m1")
  FP4_MX_CASE(kE2M1, kE2M3, "e2m1", "e2m3")
  FP4_MX_CASE(kE2M1, kE3M2, "e2m1", "e3m2")
  FP4_MX_CASE(kE2M1, kE4M3, "e2m1", "e4m3")
  FP4_MX_CASE(kE2M3, kE2M1, "e2m3", "e2m1")
  FP4_MX_CASE(kE2M3, kE2M3, "e2m3", "e2m3")
  FP4_MX_CASE(kE2M3, kE3M2, "e2m3", "e3m2")
  FP4_MX_CASE(kE2M3, kE4M3, "e2m3", "e4m3")
  FP4_MX_CASE(kE3M2, kE2M1, "e3m2", "e2m1")
  FP4_MX_CASE(kE3M2, kE2M3, "e3m2", "e2m3")
  FP4_MX_CASE(kE3M2, kE3M2, "e3m2", "e3m2")
  FP4_MX_CASE(kE3M2, kE4M3, "e3m2", "e4m3")
  FP4_MX_CASE(kE4M3, kE2M1, "e4m3", "e2m1")
  FP4_MX_CASE(kE4M3, kE2M3, "e4m3", "e2m3")
  FP4_MX_CASE(kE4M3, kE3M2, "e4m3", "e3m2")
  return hipErrorInvalidValue;
}
#undef FP4_MX_CASE

}  // namespace fp4
