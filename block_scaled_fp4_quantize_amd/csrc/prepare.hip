// One-time weight preparation ("vLLM on the NVIDIA DGX Spark (GB10 / sm_121): A Complete
// Technical Guide", §4.3: scale factors converted to the MMA layout once, when the
// weights are loaded; §5.3: the block scales repacked for the dequant kernel): the
// packed e2m1 codes are repacked into the layout the decode kernels stream, and the
// block scales are checked for NaN codes.
//
// Prepared layout: blocks of 16 rows x 128 elements (64 bytes per row), block (g, s)
// holding rows 16 g .. 16 g + 15 and elements 128 s .. 128 s + 127; inside a block the
// 16-byte piece of lane l (row l % 16, bytes 16 (l / 16) of the row's 64) sits at 16 l,
// so a wave's load of one step is one contiguous kilobyte.  Blocks are ordered by g,
// then s.
#include "device.h"
#include "internal.h"

namespace fp4 {

namespace {

__global__ __launch_bounds__(256) void prepare_codes_kernel(const uint8_t* __restrict__ w, int64_t N,
                                                            int64_t K, uint8_t* __restrict__ out) {
  const int64_t S = K / 128, KB = K / 2;
  const int64_t total = (N / 16) * S * 64;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t l = i & 63, blk = i >> 6;
    const int64_t s = blk % S, g = blk / S;
    const int64_t row = g * 16 + (l & 15);
    *reinterpret_cast<uint4*>(out + i * 16) =
        *reinterpret_cast<const uint4*>(w + row * KB + s * 64 + (l >> 4) * 16);
  }
}

// *bad = 1 when any scale code is a NaN (e4m3 S.1111.111, e8m0 0xFF)
__global__ __launch_bounds__(256) void check_scales_kernel(const uint8_t* __restrict__ sc, int64_t n,
                                                           int nv, int32_t* bad) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  bool found = false;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint32_t v = sc[i];
    found |= nv ? (v & 0x7Fu) == 0x7Fu : v == 0xFFu;
  }
  if (found) *bad = 1;
}

}  // namespace

hipError_t launch_prepare(int fmt, const uint8_t* w_codes, const uint8_t* w_scales, int64_t N,
                          int64_t K, uint8_t* out, int32_t* bad, hipStream_t s) {
  const int64_t pieces = (N / 16) * (K / 128) * 64;
  const int64_t nsc = N * (K / (fmt == kNV ? 16 : 32));
  const unsigned g1 = (unsigned)((pieces + 255) / 256 < 4096 ? (pieces + 255) / 256 : 4096);
  const unsigned g2 = (unsigned)((nsc + 255) / 256 < 1024 ? (nsc + 255) / 256 : 1024);
  hipLaunchKernelGGL(check_scales_kernel, dim3(g2 ? g2 : 1), dim3(256), 0, s, w_scales, nsc,
                     fmt == kNV ? 1 : 0, bad);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(prepare_codes_kernel, dim3(g1 ? g1 : 1), dim3(256), 0, s, w_codes, N, K, out);
  return hipGetLastError();
}

}  // namespace fp4
