// Internal launcher interface between the C-ABI layer (api.cpp) and the kernels.
// Not installed; the public interface is include/fp4.h.
#pragma once

#include <hip/hip_runtime.h>
#include <atomic>
#include <stddef.h>
#include <stdint.h>

namespace fp4 {

// Raise a kernel's dynamic-LDS limit on the current device, once per device (the
// attribute belongs to the device the call is made on).  Concurrent first calls both
// set it, which is harmless.
inline hipError_t ensure_dynamic_lds(const void* fn, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (1ull << dev) : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  if (bit) done.fetch_or(bit, std::memory_order_release);
  return hipSuccess;
}

enum Fmt : int { kNV = 0, kMX = 1 };

// ---- activation / weight quantization --------------------------------------------
struct QuantParams {
  const void* x;            // bf16 bits or fp32, [rows of the source, ldx]
  int in_f32;               // 0: bf16 input, 1: fp32 input
  int64_t M, K, ldx;
  float g;                  // NVFP4 quantize multiplier 1/input_scale (scalar)
  const int32_t* row_src;   // optional: source row of output row r
  const int32_t* row_grp;   // optional: group of output row r, selects grp_g
  const float* grp_g;       // per-group multiplier (device)
  uint8_t* codes;           // [M, K/2]
  uint8_t* scales;          // [M, K/G]
};
hipError_t launch_quant(int fmt, const QuantParams& p, hipStream_t s, const char** name);
// One-time weight preparation: codes [N, K/2] -> the prepared layout of the decode
// kernels (N % 16 == 0, K % 128 == 0); *bad (zeroed by the caller) set to 1 when a
// block scale is a NaN code.
hipError_t launch_prepare(int fmt, const uint8_t* w_codes, const uint8_t* w_scales, int64_t N,
                          int64_t K, uint8_t* out, int32_t* bad, hipStream_t s);

// ---- block-scaled matmul ----------------------------------------------------------
struct GemmParams {
  int64_t M, N, K;
  // activations: fp4 codes/scales, or bf16 bits with row stride lda
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const uint16_t* a_bf16;
  int64_t lda;
  const int32_t* a_gather;  // optional: source row of virtual row p
  // weights, one [N, K] matrix per group at these strides; w_tiled: codes in the
  // prepared layout (16-row x 128-element blocks in lane order; N % 16 == 0, K % 128 == 0)
  int w_tiled;
  const uint8_t* w_codes;
  const uint8_t* w_scales;
  int64_t w_estride_codes, w_estride_scales;
  // grouping: dense when mblk_expert == nullptr
  const int32_t* mblk_expert;     // [n_mblocks] group of each row block (-1 = none)
  const int32_t* mblk_row0;       // [n_mblocks] first virtual row of each row block
  const int32_t* group_end;       // [groups]: one past the last virtual row of each group
  int64_t n_mblocks;
  int bm;                          // rows per row block the table was built for
  const float* alpha_g;           // optional per-group alpha (device)
  float alpha;
  void* out;
  int64_t ldo;
  int out_f32;
  // Fused SwiGLU + requant of a gate/up GEMM (tiled kernel, fp4 activations): the
  // weight rows are gate [0, I) and up [I, 2I) (N = 2I, I % 128 == 0); instead of
  // `out`, h = SiLU(alpha g) * (alpha u) is quantized into h_codes / h_scales, whose
  // rows are indexed like the output rows.
  int fuse_swiglu;
  int64_t I;
  const float* h_grp_g;   // per-group NVFP4 quantize multiplier (1 / a2_scale), or null
  float h_g;              // scalar multiplier when h_grp_g is null (MXFP4: unused)
  uint8_t* h_codes;       // [rows, I/2]
  uint8_t* h_scales;      // [rows, I/G]
  // Optional block scales in the 256 x 256 tile's stage order (scale_relayout): when
  // both are set, that kernel copies each stage's scales as contiguous 256-byte pieces
  // instead of gathering one word from each row.
  const uint8_t* a_scales_t;
  const uint8_t* w_scales_t;
};
enum AKind : int { kA_FP4 = 0, kA_BF16 = 1 };
// Whether a gate/up GEMM of this shape takes the fused SwiGLU + requant epilogue: on
// the tiled kernel (grouped: 128-row blocks; dense: more than 64 rows), else on the
// streaming kernel when the plain GEMM would run there too or has at most 16 rows.
bool gemm_can_fuse_swiglu(int fmt, int akind, int64_t M, int64_t K, int64_t I, bool grouped,
                          int bm, int64_t n_mblocks);
// Row-block height of the block table for grouped (MoE) GEMMs of these shapes
// (GEMM1 has K = H, GEMM2 has K = I); launch_gemm picks its kernel from it.
int gemm_block_rows(int fmt, int akind, int64_t rows_per_group, int64_t H, int64_t I);
// W4A16 for many rows (bf16 activations, dense above 64 rows or grouped 128-row expert
// blocks, K % 128 == 0, lda % 8 == 0): the LDS-tiled bf16-MFMA kernel;
// w4a16_tiled_ok says whether a GEMM qualifies.
bool w4a16_tiled_ok(const GemmParams& p);
// Dense fp4-activation GEMMs with at least 256 tiles of 256 x 256 run on the 4-wave
// 256 x 256 tile kernel (K % 128 == 0).  Its block scales can first be re-laid into
// stage order: scale_relayout_bytes(R, K) bytes per side (rows padded to 256), written
// by launch_scale_relayout for the activations (rows in order) and the weights (rows
// in the kernel's pair order).
bool gemm_big_tile(int fmt, int64_t M, int64_t N, int64_t K);
size_t scale_relayout_bytes(int fmt, int64_t R, int64_t K);
hipError_t launch_scale_relayout(int fmt, const uint8_t* a_scales, int64_t M,
                                 const uint8_t* w_scales, int64_t N, int64_t K, uint8_t* a_t,
                                 uint8_t* w_t, hipStream_t s);
hipError_t launch_gemm_w4a16_tiled(int fmt, const GemmParams& p, hipStream_t s, const char** name);
hipError_t launch_gemm(int fmt, int akind, const GemmParams& p, hipStream_t s,
                       const char** name);
// decode kernel with the activations resident in LDS (fp4 activations, one 16-row
// tile per workgroup: mt must be 1); usable when resident_fits()
constexpr int64_t kResidentMaxLds = 160 * 1024;
int64_t resident_lds_bytes(int fmt, int mt, int ksplit, int64_t K);
// nblk: row blocks of the launch (the expert table's capacity, or 1 when dense)
int resident_ksplit(int64_t M, int64_t N, int64_t K, int64_t nblk);   // 1, 2 or 4 waves split K
bool resident_fits(int fmt, int mt, int64_t M, int64_t N, int64_t K, int64_t nblk);
hipError_t launch_gemm_resident(int fmt, int mt, const GemmParams& p, hipStream_t s,
                                const char** name);
// tiled kernel for many activation rows (fp4 activations, K % 128 == 0, 128-row
// activation blocks)
hipError_t launch_gemm_tiled(int fmt, const GemmParams& p, hipStream_t s, const char** name);

// ---- MXFP8 and FP8 W8A8 (e4m3 operands) ---------------------------------------------
// scaling modes, in the order of the C ABI's fp8_scaling
enum Fp8Mode : int { kF8_MX = 0, kF8_TENSOR = 1, kF8_ROW = 2, kF8_BLOCK = 3 };
struct Fp8QuantParams {
  const void* x;            // bf16 bits or fp32 [M, ldx]
  int in_f32;
  int64_t M, K, ldx;
  int weight_blocks;        // BLOCK: 128 x 128 blocks (weights) instead of 1 x 128
  float tensor_scale;       // TENSOR: the divisor
  uint8_t* codes;           // e4m3 [M, K]
  uint8_t* mx_scales;       // MX: e8m0 [M, K/32]
  float* f_scales;          // ROW: [M]; BLOCK: [M, K/128] or [ceil(M/128), K/128]
};
hipError_t launch_fp8_quant(int mode, const Fp8QuantParams& p, hipStream_t s, const char** name);
struct Fp8GemmParams {
  int64_t M, N, K;
  const uint8_t* a_codes;   // [M, K]
  const uint8_t* w_codes;   // [N, K]
  const uint8_t* a_mx;      // MX: e8m0 [M, K/32]
  const uint8_t* w_mx;      // MX: e8m0 [N, K/32]
  const float* a_s;         // ROW: [M]; BLOCK: [M, K/128]
  const float* w_s;         // ROW: [N]; BLOCK: [ceil(N/128), K/128]
  float alpha;              // TENSOR: a_scale * w_scale; MX and BLOCK: 1
  int unit_scale;           // the e8m0 code of 1.0 (127), passed at run time
  void* out;
  int64_t ldo;
  int out_f32;
};
// K % 128 == 0
hipError_t launch_fp8_gemm(int mode, const Fp8GemmParams& p, hipStream_t s, const char** name);

// MX formats of any element type.  Element types are the scaled MFMA's codes: 0 e4m3,
// 2 e2m3, 3 e3m2, 4 e2m1.  MXFP6 quantization (elem 2 or 3) writes 24 bytes of codes per
// 32 elements (element i at bits [6 i, 6 i + 6) of the little-endian group) and one e8m0
// byte per 32 into mx_scales; K % 32 == 0.
hipError_t launch_mx6_quant(int elem, const Fp8QuantParams& p, hipStream_t s, const char** name);
// MX matmul with element types fa (activations) and fw (weights): a_mx / w_mx scales,
// alpha 1, unit_scale unused; K % 128 == 0.  (e4m3 x e4m3 is launch_fp8_gemm's MX mode.)
hipError_t launch_mx_gemm(int fa, int fw, const Fp8GemmParams& p, hipStream_t s, const char** name);

// ---- MoE stages ------------------------------------------------------------------
hipError_t launch_topk_softmax(const float* logits, int64_t T, int64_t E, int k,
                               int renormalize, int32_t* ids, float* w, hipStream_t s,
                               const char** name);

struct PermuteParams {
  const int32_t* ids;      // [T*k]
  int64_t T;
  int k;
  int64_t E;
  int bm;                  // row-block height for the block table
  int64_t n_mblocks;       // capacity of the block table
  int32_t* expert_offsets; // [E+1]
  int32_t* sorted_rows;    // [T*k]
  int32_t* inverse;        // [T*k]
  int32_t* row_expert;     // [T*k]
  int32_t* src_token;      // [T*k]
  int32_t* mblk_expert;    // [n_mblocks]
  int32_t* mblk_row0;      // [n_mblocks]
  int32_t* group_end;      // [E]
  int32_t* chunk_base;     // [ceil(T*k / kPermuteChunk)][E] scratch
  // Work folded into the one-workgroup dispatch of small slot counts (optional):
  //  * up_n floats (the host values passed to launch_permute) stored to up_dst;
  //  * quantization of the GEMM1 activations when they are few (q_fmt >= 0): output
  //    row j is hidden row src(j) under multiplier g(j), with, for q_routed, src(j) =
  //    the token of sorted slot j and g(j) = host value q_g_off + its expert (routed
  //    NVFP4 rows; slots past the routed count are not written), else src(j) = j and
  //    g = q_g (one row per token).
  float* up_dst;
  int up_n;
  int q_fmt;
  int q_routed;
  int q_g_off;
  float q_g;
  const uint16_t* q_x;     // bf16 [., q_K]
  int64_t q_K, q_rows;
  uint8_t* q_codes;        // [q_rows, q_K/2]
  uint8_t* q_scales;       // [q_rows, q_K/G]
};
constexpr int kPermuteChunk = 256;   // routed slots per histogram / scatter chunk
// Activation elements up to which the one-workgroup dispatch also quantizes them.
constexpr int64_t kPermuteQuantMax = 65536;
// Dispatch; *quantized tells whether the activation quantization was done in it (when
// it was not, the caller runs the quantization pass).  up_host: the up_n floats.
hipError_t launch_permute(const PermuteParams& p, const float* up_host, hipStream_t s,
                          const char** name, bool* quantized);

struct SwigluParams {
  const float* gu;          // [R, 2I] fp32
  int64_t R, I;
  int mode_w4a16;           // 1: write bf16 h, 0: quantize h
  int fmt;
  const int32_t* row_grp;   // optional: group (expert) of each row -> grp_g
  const float* grp_g;       // per-group quantize multiplier (NVFP4)
  float g;                  // scalar multiplier when row_grp == nullptr
  uint8_t* h_codes;         // [R, I/2]
  uint8_t* h_scales;        // [R, I/G]
  uint16_t* h_bf16;         // [R, I]
};
hipError_t launch_swiglu(const SwigluParams& p, hipStream_t s, const char** name);

struct CombineParams {
  const float* y;           // [P + T (shared), H] fp32 in sorted order
  const int32_t* inverse;   // [T*k]
  const float* w;           // [T, k]
  int64_t T, H;
  int k;
  const float* y_shared;    // [T, H] or nullptr
  uint16_t* out;            // [T, H] bf16
};
hipError_t launch_combine(const CombineParams& p, hipStream_t s, const char** name);

hipError_t launch_upload_floats(float* dst, const float* host_vals, int64_t n,
                                hipStream_t s);

// ---- a whole NVFP4 W4A4 MoE layer for a few routed slots (moe_small.hip) ----------
// Two launches: gate/up with routing, activation quantization and SwiGLU + requant;
// down projection with the weighted combine.  The workspace rows named here are
// written as the general path writes them (sorted positions).
constexpr int kSmallSlots = 32;     // routed slots T k, at most
constexpr int kSmallTokens = 4;     // tokens, at most
constexpr int64_t kSmallMaxH = 4096;
constexpr int64_t kSmallMaxI = 2048;
struct MoeSmallParams {
  int64_t T, H, I, E;
  int k;
  const uint16_t* hidden;          // bf16 [T, H]
  const int32_t* ids;              // [T, k]
  const float* w;                  // [T, k]
  const uint8_t *w13_codes, *w13_scales, *w2_codes, *w2_scales;
  int32_t* expert_offsets;         // [E + 1]
  int32_t* sorted_rows;            // [T k]
  int32_t* inverse;                // [T k]
  uint8_t *x_codes, *x_scales;     // [T k, H/2], [T k, H/16] at sorted positions
  uint8_t *h_codes, *h_scales;     // [T k, I/2], [T k, I/16]
  float* y;                        // [T k, H]
  uint16_t* out;                   // bf16 [T, H]
};
bool moe_small_fits(int64_t T, int k, int64_t E, int64_t H, int64_t I);
// scal_host: the 4 E per-expert scalars g13, alpha13, g2, alpha2
hipError_t launch_moe_small(const MoeSmallParams& p, const float* scal_host, hipStream_t s,
                            const char** name);

}  // namespace fp4
