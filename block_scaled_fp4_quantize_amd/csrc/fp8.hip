// 8- and 6-bit quantization on gfx950 (MXFP8, FP8 W8A8 scales, MXFP6) and the FP8 W8A8
// matmul entry, which runs on the scaled-MFMA engine of scaled_gemm.h.
//
// What is computed ("vLLM per-format kernel capability matrix derived from source"):
//  * MXFP8 -- e4m3 elements with an e8m0 scale per 32 along K (the MX group-size note;
//    the MXFP8 section: the one MX format with a native path on gfx95);
//  * MXFP6 -- e2m3 or e3m2 elements with an e8m0 scale per 32 (the MXFP6 section);
//  * FP8 W8A8 with one of the three scaling modes of its "FP8, THREE SCALING MODES"
//    section: per-tensor; rowwise (per token for activations, per output channel for
//    weights, dynamic); block (1 x 128 activation blocks, 128 x 128 weight blocks).
// out[m, n] = sum_k a_hat[m, k] * w_hat[n, k], each operand dequantized with its own
// scales (the emulation definition of THE EMULATION COLUMN), accumulated in fp32.
// The e4m3 dot products inside the MFMA are not exact fp32 sums (the device showed up
// to 1.4e-4 of the sum of |products| per instruction), well inside the GEMM tolerance.
#include "scaled_gemm.h"

#pragma clang fp contract(off)

namespace fp4 {

namespace {

constexpr float kE4M3Max = 448.0f;

// e4m3 code of an fp32 value: nearest even, saturating at 448, the sign bit of y
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  return e4m3_code_pos(fabsf(y)) | ((__float_as_uint(y) >> 24) & 0x80u);
}

// MXFP8 block exponent (OCP MX rule, emax(e4m3) = 8): floor(log2 amax) - 8, clamped
// to [-127, 127] (read off the fp32 exponent field; zero and subnormal amax: -127)
__device__ __forceinline__ int mx8_exponent(float amax) {
  const int eb = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  return eb == 0 ? -127 : max(eb - 127 - 8, -127);
}

// ---- quantization ------------------------------------------------------------------
// One lane = 8 consecutive elements of a row.  MX: 4 lanes per 32-block; BLOCK (1 x
// 128 activations): 16 lanes per block; PER_TENSOR: no reduction.  Rowwise and 128 x
// 128 weight blocks need a whole row / block first: their scales come from
// fp8_amax_kernel and are read here.
template <int MODE, typename Tin>
__global__ __launch_bounds__(256) void fp8_quant_kernel(Fp8QuantParams p) {
  constexpr int LPB = MODE == kF8_MX ? 4 : (MODE == kF8_BLOCK ? 16 : 1);
  const int64_t cpr = p.K / 8;
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool active = c < p.M * cpr;
  const int64_t row = active ? c / cpr : 0;
  const int64_t kc = active ? c - row * cpr : 0;
  float v[8];
  float amax = 0.0f;
  if (active) {
    load8<Tin>(reinterpret_cast<const Tin*>(p.x) + row * p.ldx + kc * 8, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }
#pragma unroll
  for (int off = 1; off < LPB; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if (!active) return;
  uint32_t lo = 0, hi = 0;
  if (MODE == kF8_MX) {
    const int E = mx8_exponent(amax);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= e4m3_code(ldexpf(v[i], -E)) << (8 * i);
      hi |= e4m3_code(ldexpf(v[4 + i], -E)) << (8 * i);
    }
    if ((kc & 3) == 0) p.mx_scales[row * (p.K / 32) + kc / 4] = (uint8_t)(E + 127);
  } else {
    float s;
    if (MODE == kF8_TENSOR) {
      s = p.tensor_scale;
    } else if (MODE == kF8_BLOCK && !p.weight_blocks) {
      s = amax / kE4M3Max;
      if ((kc & 15) == 0) p.f_scales[row * (p.K / 128) + kc / 16] = s;
    } else if (MODE == kF8_BLOCK) {   // 128 x 128 weight blocks, scales already reduced
      s = p.f_scales[(row / 128) * (p.K / 128) + kc / 16];
    } else {                          // rowwise, scales already reduced
      s = p.f_scales[row];
    }
    // y = fp32(x / s); a zero scale (an all-zero row or block) gives signed zeros
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float y0 = s != 0.0f ? v[i] / s : copysignf(0.0f, v[i]);
      const float y1 = s != 0.0f ? v[4 + i] / s : copysignf(0.0f, v[4 + i]);
      lo |= e4m3_code(y0) << (8 * i);
      hi |= e4m3_code(y1) << (8 * i);
    }
  }
  *reinterpret_cast<uint2*>(p.codes + row * p.K + kc * 8) = make_uint2(lo, hi);
}

// amax / 448 of each row (rowwise), or of each 128 x 128 weight block: one workgroup
// per row or block, a fixed-order reduction (max is order-free anyway)
template <typename Tin, bool BLOCKS>
__global__ __launch_bounds__(256) void fp8_amax_kernel(Fp8QuantParams p) {
  __shared__ float red[4];
  const int tid = threadIdx.x;
  float amax = 0.0f;
  if (!BLOCKS) {
    const int64_t row = blockIdx.x;
    const Tin* x = reinterpret_cast<const Tin*>(p.x) + row * p.ldx;
    for (int64_t k = (int64_t)tid * 8; k < p.K; k += 256 * 8) {
      float v[8];
      load8<Tin>(x + k, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    }
  } else {
    const int64_t nkb = p.K / 128;
    const int64_t rb = blockIdx.x / nkb, kb = blockIdx.x - rb * nkb;
    // 128 rows x 128 columns: thread t reads columns 8 (t % 16) .. + 7 of rows t / 16 + 16 i
    for (int64_t r = rb * 128 + tid / 16; r < rb * 128 + 128 && r < p.M; r += 16) {
      float v[8];
      load8<Tin>(reinterpret_cast<const Tin*>(p.x) + r * p.ldx + kb * 128 + (tid % 16) * 8, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  if (tid == 0)
    p.f_scales[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])) / kE4M3Max;
}

// ---- MXFP6 ---------------------------------------------------------------------------
// Code of a non-negative fp32 value in a small float type without infinities (EB exponent
// bits of bias BIAS, MB mantissa bits): nearest value, ties to the even code, saturating
// at the largest value.  a is split into its binade (at least the smallest normal one)
// and rounded to MB fraction bits with rintf (round half to even); a carry into the next
// binade moves the exponent.
template <int EB, int MB, int BIAS>
__device__ __forceinline__ uint32_t small_code_pos(float a) {
  constexpr int EMIN = 1 - BIAS, EMAXE = (1 << EB) - 1 - BIAS;
  constexpr uint32_t MAXC = (((1u << EB) - 1) << MB) | ((1u << MB) - 1);
  constexpr float MAXV = (float)((2.0 - 1.0 / (1 << MB)) * (double)(1 << EMAXE));
  if (!(a < MAXV)) return MAXC;
  int ex = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;
  ex = max(ex, EMIN);
  uint32_t q = (uint32_t)rintf(ldexpf(a, MB - ex));     // exact scaling, then RNE
  int e = ex;
  if (q >= (2u << MB)) {
    q >>= 1;
    ++e;
  }
  if (q < (1u << MB)) return q;                         // subnormal: exponent field 0
  return ((uint32_t)(e + BIAS) << MB) | (q - (1u << MB));
}

template <int ELEM>
__device__ __forceinline__ uint32_t fp6_code(float y) {
  const uint32_t mag = ELEM == sg::kE2M3 ? small_code_pos<2, 3, 1>(fabsf(y))
                                         : small_code_pos<3, 2, 3>(fabsf(y));
  return mag | ((__float_as_uint(y) >> 26) & 0x20u);
}

// One lane = 8 consecutive elements (48 code bits, 6 bytes of the block's 24); 4 lanes
// per 32-block.  E = floor(log2 amax) - emax (2 for e2m3, 4 for e3m2), clamped at -127.
template <int ELEM, typename Tin>
__global__ __launch_bounds__(256) void mx6_quant_kernel(Fp8QuantParams p) {
  constexpr int EMAX = ELEM == sg::kE2M3 ? 2 : 4;
  const int64_t cpr = p.K / 8;
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool active = c < p.M * cpr;
  const int64_t row = active ? c / cpr : 0;
  const int64_t kc = active ? c - row * cpr : 0;
  float v[8];
  float amax = 0.0f;
  if (active) {
    load8<Tin>(reinterpret_cast<const Tin*>(p.x) + row * p.ldx + kc * 8, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  if (!active) return;
  const int eb = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  const int E = eb == 0 ? -127 : max(eb - 127 - EMAX, -127);
  uint64_t bits = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) bits |= (uint64_t)fp6_code<ELEM>(ldexpf(v[i], -E)) << (6 * i);
  uint16_t* d = reinterpret_cast<uint16_t*>(p.codes + row * (p.K / 32) * 24 + (kc >> 2) * 24 + (kc & 3) * 6);
  d[0] = (uint16_t)bits;
  d[1] = (uint16_t)(bits >> 16);
  d[2] = (uint16_t)(bits >> 32);
  if ((kc & 3) == 0) p.mx_scales[row * (p.K / 32) + kc / 4] = (uint8_t)(E + 127);
}

}  // namespace

hipError_t launch_fp8_quant(int mode, const Fp8QuantParams& p, hipStream_t s, const char** name) {
  const int64_t total = p.M * (p.K / 8);
  if (total == 0) return hipSuccess;
  if ((total + 255) / 256 > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 block(256), grid((unsigned)((total + 255) / 256));
  const bool f32 = p.in_f32 != 0;
  // rowwise and 128 x 128 weight blocks: the scales first (one workgroup each)
  if (mode == kF8_ROW || (mode == kF8_BLOCK && p.weight_blocks)) {
    const bool blocks = mode == kF8_BLOCK;
    const int64_t n = blocks ? ((p.M + 127) / 128) * (p.K / 128) : p.M;
    if (n > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    if (f32) {
      if (blocks) hipLaunchKernelGGL((fp8_amax_kernel<float, true>), dim3((unsigned)n), block, 0, s, p);
      else hipLaunchKernelGGL((fp8_amax_kernel<float, false>), dim3((unsigned)n), block, 0, s, p);
    } else {
      if (blocks) hipLaunchKernelGGL((fp8_amax_kernel<uint16_t, true>), dim3((unsigned)n), block, 0, s, p);
      else hipLaunchKernelGGL((fp8_amax_kernel<uint16_t, false>), dim3((unsigned)n), block, 0, s, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  static const char* names[4][2] = {{"fp8_quant_mx_bf16", "fp8_quant_mx_f32"},
                                    {"fp8_quant_tensor_bf16", "fp8_quant_tensor_f32"},
                                    {"fp8_quant_row_bf16", "fp8_quant_row_f32"},
                                    {"fp8_quant_block_bf16", "fp8_quant_block_f32"}};
  *name = names[mode][f32 ? 1 : 0];
#define FP4_F8Q(M_)                                                                        \
  if (f32) hipLaunchKernelGGL((fp8_quant_kernel<M_, float>), grid, block, 0, s, p);       \
  else hipLaunchKernelGGL((fp8_quant_kernel<M_, uint16_t>), grid, block, 0, s, p);
  switch (mode) {
    case kF8_MX: FP4_F8Q(kF8_MX) break;
    case kF8_TENSOR: FP4_F8Q(kF8_TENSOR) break;
    case kF8_ROW: FP4_F8Q(kF8_ROW) break;
    default: FP4_F8Q(kF8_BLOCK) break;
  }
#undef FP4_F8Q
  return hipGetLastError();
}

hipError_t launch_fp8_gemm(int mode, const Fp8GemmParams& p, hipStream_t s, const char** name) {
  if (p.M == 0 || p.N == 0) return hipSuccess;
  if (p.K % 128 != 0 || p.K <= 0) return hipErrorInvalidValue;
  using sg::kE4M3;
  switch (mode) {
    case kF8_MX: return sg::launch<kF8_MX, kE4M3, kE4M3>(p, s, name, "fp8_rows_mx", "fp8_tile_mx");
    case kF8_TENSOR:
      return sg::launch<kF8_TENSOR, kE4M3, kE4M3>(p, s, name, "fp8_rows_tensor", "fp8_tile_tensor");
    case kF8_ROW: return sg::launch<kF8_ROW, kE4M3, kE4M3>(p, s, name, "fp8_rows_row", "fp8_tile_row");
    default: return sg::launch<kF8_BLOCK, kE4M3, kE4M3>(p, s, name, "fp8_rows_block", "fp8_tile_block");
  }
}

hipError_t launch_mx6_quant(int elem, const Fp8QuantParams& p, hipStream_t s, const char** name) {
  const int64_t total = p.M * (p.K / 8);
  if (total == 0) return hipSuccess;
  if ((total + 255) / 256 > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 block(256), grid((unsigned)((total + 255) / 256));
  const bool f32 = p.in_f32 != 0;
  if (elem == sg::kE2M3) {
    *name = f32 ? "mx6_quant_e2m3_f32" : "mx6_quant_e2m3_bf16";
    if (f32) hipLaunchKernelGGL((mx6_quant_kernel<sg::kE2M3, float>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((mx6_quant_kernel<sg::kE2M3, uint16_t>), grid, block, 0, s, p);
  } else {
    *name = f32 ? "mx6_quant_e3m2_f32" : "mx6_quant_e3m2_bf16";
    if (f32) hipLaunchKernelGGL((mx6_quant_kernel<sg::kE3M2, float>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((mx6_quant_kernel<sg::kE3M2, uint16_t>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace fp4
