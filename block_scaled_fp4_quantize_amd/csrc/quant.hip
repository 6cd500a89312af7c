// Activation / weight quantization to NVFP4 or MXFP4 on gfx950.
//
// Definition: "vLLM on the NVIDIA DGX Spark (GB10 / sm_121): A Complete Technical
// Guide", §6.1 (NVFP4: e2m1 + e4m3 scale per 16 + per-tensor fp32 scale) and §6.4
// (MXFP4: e2m1 + e8m0 scale per 32); §4.3 (the fused MoE quantizes BF16
// activations to FP4 in-kernel).
//
// The pass is HBM-bound (2 B in, ~0.56 B out per bf16 element).  Each lane loads
// 8 contiguous elements with one 16-byte load, so a wave reads 1 KiB of
// contiguous input; a block's amax is reduced across the 2 (NVFP4) or 4 (MXFP4)
// lanes that hold it with lane swizzles, and every lane writes its 8 codes as one
// dword.  Scale arithmetic is fp32 with correctly rounded division, in the order
// the header documents, so codes and scales are bit-exact.
#include "device.h"
#include "internal.h"

#pragma clang fp contract(off)

namespace fp4 {

// One lane = 8 consecutive elements of one row.  FMT kNV: 2 lanes per 16-block;
// kMX: 4 lanes per 32-block.  Blocks never straddle rows (K % G == 0).
template <int FMT, typename Tin>
__global__ __launch_bounds__(256) void quant_kernel(QuantParams p) {
  constexpr int LPG = FMT == kNV ? 2 : 4;  // lanes per block
  const int64_t chunks_per_row = p.K / 8;
  const int64_t total = p.M * chunks_per_row;
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool active = c < total;
  const int64_t row = active ? c / chunks_per_row : 0;
  const int64_t kc = active ? c - row * chunks_per_row : 0;

  float v[8];
  float amax = 0.0f;
  float g = p.g;
  if (active) {
    const int64_t src = p.row_src ? (int64_t)p.row_src[row] : row;
    load8<Tin>(reinterpret_cast<const Tin*>(p.x) + src * p.ldx + kc * 8, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    if (p.row_grp) g = p.grp_g[p.row_grp[row]];
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }
  // block amax across the lanes of the block (all lanes take part)
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  if (LPG == 4) amax = fmaxf(amax, __shfl_xor(amax, 2));
  if (!active) return;

  uint32_t packed = 0;
  uint32_t sc;
  if (FMT == kNV) {
    float r;
    sc = q_nv_scale(amax, g, &r);
#pragma unroll
    for (int i = 0; i < 4; ++i) packed |= q_nv_pack2(v[2 * i], v[2 * i + 1], r) << (8 * i);
  } else {
    int E;
    sc = q_mx_scale(amax, &E);
#pragma unroll
    for (int i = 0; i < 4; ++i) packed |= q_mx_pack2(v[2 * i], v[2 * i + 1], E) << (8 * i);
  }
  *reinterpret_cast<uint32_t*>(p.codes + row * (p.K / 2) + kc * 4) = packed;
  if ((kc & (LPG - 1)) == 0) {
    constexpr int G = FMT == kNV ? 16 : 32;
    p.scales[row * (p.K / G) + kc / LPG] = (uint8_t)sc;
  }
}

hipError_t launch_quant(int fmt, const QuantParams& p, hipStream_t s, const char** name) {
  const int64_t total = p.M * (p.K / 8);
  if (total == 0) return hipSuccess;
  const dim3 block(256);
  const dim3 grid((unsigned)((total + 255) / 256));
  if (fmt == kNV) {
    if (p.in_f32) {
      *name = "quant_nvfp4_f32";
      hipLaunchKernelGGL((quant_kernel<kNV, float>), grid, block, 0, s, p);
    } else {
      *name = "quant_nvfp4_bf16";
      hipLaunchKernelGGL((quant_kernel<kNV, uint16_t>), grid, block, 0, s, p);
    }
  } else {
    if (p.in_f32) {
      *name = "quant_mxfp4_f32";
      hipLaunchKernelGGL((quant_kernel<kMX, float>), grid, block, 0, s, p);
    } else {
      *name = "quant_mxfp4_bf16";
      hipLaunchKernelGGL((quant_kernel<kMX, uint16_t>), grid, block, 0, s, p);
    }
  }
  return hipGetLastError();
}

}  // namespace fp4
