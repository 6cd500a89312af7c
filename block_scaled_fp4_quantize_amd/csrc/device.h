// Device-side helpers shared by the gfx950 kernels: bf16 conversion, block-scale
// decode and the round-to-nearest-even e2m1 / e4m3 encoders.
//
// Formats: "vLLM on the NVIDIA DGX Spark (GB10 / sm_121): A Complete Technical
// Guide", §6.1 (NVFP4: e2m1 elements with max 6.0, e4m3 scale per 16 along K) and
// §6.4 (MXFP4: 32-element blocks, exponent-only e8m0 scale).  E4M3 is the OCP
// e4m3fn variant (bias 7, max 448) that gfx950 also uses natively.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// Two fp32 values -> bf16 pair (a in the low half), round to nearest even, by gfx950's
// pair conversion.  A device probe over 2^24 random bit patterns plus ties at every
// exponent, denormals, infinities and NaNs matched rounding the bit pattern to nearest
// even (NaNs stay NaN).
__device__ __forceinline__ uint32_t bf16_pack2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)a, (__bf16)b});
}

// e4m3fn code of sf >= 0 (finite or +inf): round to nearest even, saturating at 448
// (code 0x7E).  Normal range: keep 3 mantissa bits of the fp32 pattern with
// round-half-even at bit 20 and rebias the exponent (127 -> 7).  Below 2^-6 the
// grid is m * 2^-9: scale exactly by 2^9 and round half-even to an integer (8 is
// the smallest normal, code 0x08, so the carry works out).
__device__ __forceinline__ uint32_t e4m3_code_pos(float sf) {
  if (!(sf < 448.0f)) return 0x7Eu;
  if (sf < 0.015625f) return (uint32_t)__builtin_rintf(sf * 512.0f);
  uint32_t u = __float_as_uint(sf);
  uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);
  uint32_t code = (r >> 20) - (120u << 3);
  return code > 0x7Eu ? 0x7Eu : code;
}

// Value of a non-negative e4m3fn code (0..0x7E).
__device__ __forceinline__ float e4m3_value_pos(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  // both forms computed and selected: a branch here would split every MFMA loop
  // that decodes scales into exec-masked pieces
  const float sub = (float)m * 0.001953125f;                         // m * 2^-9
  const float nrm = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return e == 0 ? sub : nrm;
}
// Value of an e4m3 code of either sign (0x7F / 0xFF, NaN, are outside the contract)
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  return __uint_as_float(__float_as_uint(e4m3_value_pos(c & 0x7Fu)) | ((c & 0x80u) << 24));
}

// ---- one quantization block, given its amax ---------------------------------------
// NVFP4 (activation quantizer order): sf = fp32(fp32(amax * g) / 6) -> e4m3 code sc
// (RNE, saturating); elements are scaled by r = fp32(g / scale).  A zero scale gives
// r = 0, for which q_nv_pack2 gives magnitude 0 with the sign kept (e2m1 of 0).
__device__ __forceinline__ uint32_t q_nv_scale(float amax, float g, float* r);
__device__ __forceinline__ uint32_t q_nv_pack2(float v0, float v1, float r);
// MXFP4 (OCP MX): E = clamp(floor(log2 amax) - 2, -127, 127), code E + 127, read off
// the exponent field (zero and subnormal amax give code 0); elements are v * 2^-E.
__device__ __forceinline__ uint32_t q_mx_scale(float amax, int* E);
__device__ __forceinline__ uint32_t q_mx_pack2(float v0, float v1, int E);
// (q_*_pack2: the codes of two elements in one byte, the first in the low nibble)

// Value 2^(c-127) of an e8m0 code (c = 0 gives the fp32 subnormal 2^-127).
__device__ __forceinline__ float e8m0_value(uint32_t c) {
  return c == 0 ? __uint_as_float(0x00400000u) : __uint_as_float((c & 0xFFu) << 23);
}

// gfx950's scaled fp4 conversions apply only the exponent of their fp32 scale
// operand (an e4m3 scale of 1.25 acts as 1.0), which is exactly an e8m0 scale.
// So: MXFP4 codes decode in one instruction with the e8m0 scale; NVFP4 codes are
// converted at unit scale and multiplied by the e4m3 block scale separately.

// 8 e2m1 codes (one dword, low nibble first) times an e8m0 scale -> bf16x8.
__device__ __forceinline__ bf16x8 decode8_bf16_pow2(uint32_t packed, float scale) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, scale, 0);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, scale, 1);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, scale, 2);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, scale, 3);
  bf16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// 8 e2m1 codes times an arbitrary (e4m3) scale -> fp16x8, exactly: every product of
// an e2m1 value and an e4m3 value lies in [2^-10, 2688] with at most six
// significant bits, so it is an fp16 number.  One unit-scale convert and one
// packed fp16 multiply per pair.
__device__ __forceinline__ f16x8 decode8_f16(uint32_t packed, f16x2 scale2) {
  f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 0) * scale2;
  f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 1) * scale2;
  f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 2) * scale2;
  f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 3) * scale2;
  f16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// The two e4m3 scale codes in bytes 0 and 1 of w -> their values as an fp16 pair
// {value(byte 0), value(byte 1)}, by gfx950's fp8 -> fp16 pair conversion at unit
// scale (exact: every e4m3 value is an fp16 number).  A device probe of all 256 codes
// in both bytes of both words matched the e4m3fn definition (bias 7, subnormals,
// sign; 0x7F / 0xFF give NaN).  Issued as inline asm: this compiler's builtin for the
// conversion hands back the low half in both halves of its result.
__device__ __forceinline__ f16x2 e4m3_pair_f16(uint32_t w) {
  uint32_t r;
  asm("v_cvt_scalef32_pk_f16_fp8 %0, %1, 1.0" : "=v"(r) : "v"(w));
  return __builtin_bit_cast(f16x2, r);
}
// {p.x, p.x} or {p.y, p.y}
__device__ __forceinline__ f16x2 f16_bcast(f16x2 p, int hi) {
  return hi ? f16x2{p.y, p.y} : f16x2{p.x, p.x};
}

// 8 e2m1 codes times an arbitrary fp32 scale -> bf16x8 (for bf16 MFMA against bf16
// activations).  The products are exact in fp32 and representable in bf16, so
// keeping the upper half of each fp32 pattern is exact.
__device__ __forceinline__ uint32_t pack_bf16_exact(float lo, float hi) {
  return (__float_as_uint(hi) & 0xFFFF0000u) | (__float_as_uint(lo) >> 16);
}

template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_bf16_scaled(uint32_t packed, float scale) {
  v2f v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, SEL);
  return pack_bf16_exact(v[0] * scale, v[1] * scale);
}

__device__ __forceinline__ bf16x8 decode8_bf16(uint32_t packed, float scale) {
  uint32_t w[4] = {fp4x2_bf16_scaled<0>(packed, scale), fp4x2_bf16_scaled<1>(packed, scale),
                   fp4x2_bf16_scaled<2>(packed, scale), fp4x2_bf16_scaled<3>(packed, scale)};
  bf16x8 r;
  __builtin_memcpy(&r, w, 16);
  return r;
}

__device__ __forceinline__ uint32_t dword_of(const uint4& q, int j) {
  return j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w;
}
__device__ __forceinline__ uint32_t dword_of_v(const u32x4& q, int j) {
  return j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w;
}

// An e4m3 block-scale value as a packed fp16 pair (exact: e4m3 values are fp16 numbers).
__device__ __forceinline__ f16x2 f16_pair(float v) {
  const _Float16 h = (_Float16)v;
  return f16x2{h, h};
}

__device__ __forceinline__ bf16x8 bits_to_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}


// 8 consecutive elements (bf16 bits or fp32) as fp32, one or two 16-byte loads
template <typename Tin>
__device__ __forceinline__ void load8(const Tin* p, float v[8]);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float v[8]) {
  uint4 q = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
    v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
  }
}

template <>
__device__ __forceinline__ void load8<float>(const float* p, float v[8]) {
  float4 a = reinterpret_cast<const float4*>(p)[0];
  float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// SwiGLU of one gate/up pair: SiLU(z) * u with SiLU(z) = z / (1 + e^-z), in fp32.
__device__ __forceinline__ float swiglu1(float z, float u) {
  const float silu = z / (1.0f + expf(-z));
  return silu * u;
}

// ---- block quantization helpers (declared above) ---------------------------------
__device__ __forceinline__ uint32_t q_nv_scale(float amax, float g, float* r) {
  const float sf = (amax * g) / 6.0f;
  const uint32_t sc = e4m3_code_pos(sf);
  const float sd = e4m3_value_pos(sc);
  *r = sd != 0.0f ? g / sd : 0.0f;
  return sc;
}
// Two e2m1 codes in one byte (low nibble y0), by gfx950's fp32 -> fp4 conversion at
// unit scale: the magnitude is the nearest of {0, .5, 1, 1.5, 2, 3, 4, 6}, a midpoint
// going to the neighbour with mantissa bit 0, values above 6 saturating to 6; the sign
// bit is y's (so -0 and small negatives give 0x8).  Checked on the device against
// that rule for every midpoint and its neighbouring floats, both signs, zeros,
// infinities and subnormals; NaN, outside the quantizers' contract, comes out as 6.
// The upper bytes of the result are zero.
__device__ __forceinline__ uint32_t e2m1_pack2(float y0, float y1) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y0, y1, 1.0f, 0);
}
// elements times r (r >= 0: the product keeps the element's sign)
__device__ __forceinline__ uint32_t q_nv_pack2(float v0, float v1, float r) {
  return e2m1_pack2(v0 * r, v1 * r);
}
__device__ __forceinline__ uint32_t q_mx_scale(float amax, int* E) {
  const uint32_t eb = (__float_as_uint(amax) >> 23) & 0xFFu;
  const int code = eb == 0 ? 0 : max((int)eb - 2, 0);
  *E = code - 127;
  return (uint32_t)code;
}
// elements times 2^-E, exactly (|v| * 2^-E < 8 for the block's E)
__device__ __forceinline__ uint32_t q_mx_pack2(float v0, float v1, int E) {
  return e2m1_pack2(ldexpf(v0, -E), ldexpf(v1, -E));
}
}  // namespace fp4
