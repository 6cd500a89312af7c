// C-ABI entry points of libfp4 (declared and documented in include/fp4.h):
// host-side validation, the device check, and the launch sequences.
//
// Failure behaviour follows the pages' lessons: an unsupported device fails
// loudly ("vLLM on the NVIDIA DGX Spark (GB10 / sm_121): A Complete Technical
// Guide", §6.3: the FP4 entry point raises instead of running a wrong kernel); a
// missing or zero activation scale is refused instead of silently zeroing the
// experts ("GLM-5.3-Flash on vLLM, on GB10"); and there is no silent fallback to
// another precision ("vLLM per-format kernel capability matrix derived from
// source", THE EMULATION COLUMN) -- weight-only execution of a W4A4 request
// happens only when the caller opts in, and is reported in the status.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "fp4.h"
#include "fp8.h"
#include "mx.h"
#include "internal.h"

namespace {

thread_local const char* t_last_kernel = "";

constexpr float kScaleMin = 0x1p-100f;
constexpr float kScaleMax = 0x1p100f;

bool scale_ok(float s) { return std::isfinite(s) && s >= kScaleMin && s <= kScaleMax; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool fmt_ok(int f) { return f == FP4_NVFP4 || f == FP4_MXFP4; }
bool mode_ok(int m) { return m == FP4_W4A4 || m == FP4_W4A16; }
int64_t group_of(int fmt) { return fmt == FP4_NVFP4 ? 16 : 32; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

fp4_status device_check() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return FP4_ERR_DEVICE;
  }
  static std::atomic<int> cache[64];  // 0 unknown, 1 supported, 2 not
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c == 1) return FP4_OK;
    if (c == 2) return FP4_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return FP4_ERR_DEVICE;
  }
  const int ok = fp4_arch_supported(prop.gcnArchName);
  if (dev < 64) cache[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? FP4_OK : FP4_ERR_DEVICE;
}

fp4_status launched(hipError_t e, const char* name) {
  t_last_kernel = name ? name : "";
  return e == hipSuccess ? FP4_OK : FP4_ERR_LAUNCH;
}

size_t gemm_ws_bytes(int fmt, int64_t M, int64_t K) {
  return align256((size_t)M * (size_t)(K / 2)) + align256((size_t)M * (size_t)(K / group_of(fmt)));
}
// The stage-ordered block scales of both operands, for W4A4 GEMMs that run on the
// 256 x 256 tile kernel (0 otherwise).
size_t gemm_relayout_bytes(int fmt, int64_t M, int64_t N, int64_t K) {
  const int ifmt = fmt == FP4_NVFP4 ? fp4::kNV : fp4::kMX;
  if (!fp4::gemm_big_tile(ifmt, M, N, K)) return 0;
  return align256(fp4::scale_relayout_bytes(ifmt, M, K)) + align256(fp4::scale_relayout_bytes(ifmt, N, K));
}

// ---- MoE workspace layout ----------------------------------------------------------
struct MoePlan {
  fp4_moe_layout L;
  size_t scal;          // float [4][E]: g13, alpha13, g2, alpha2
  size_t group_end;     // int32 [E]
  size_t row_expert;    // int32 [P]
  size_t src_token;     // int32 [P]
  size_t mblk_expert;   // int32 [n_mblocks]
  size_t mblk_row0;     // int32 [n_mblocks]
  size_t chunk_base;    // int32 [ceil(P / kPermuteChunk)][E]
  int64_t P, R;         // routed rows, routed + shared rows
  int64_t n_mblocks;
  int bm;
  bool shared;
  bool w4a4;            // effective mode (after an allowed fallback)
  bool fuse_routed;     // routed gate/up GEMM takes the fused SwiGLU epilogue
  bool fuse_shared;     // shared expert's gate/up GEMM does
};

bool moe_shared(const fp4_moe_args* a) {
  return a->sh_w13_codes || a->sh_w13_scales || a->sh_w2_codes || a->sh_w2_scales;
}

// The layout reserves the W4A4 and the W4A16 regions the call may need.
void moe_plan(const fp4_moe_args* a, bool w4a4, bool may_w4a16, MoePlan* pl) {
  const int64_t G = group_of(a->fmt);
  const int64_t P = a->T * a->k;
  const bool sh = moe_shared(a);
  const int64_t R = P + (sh ? a->T : 0);
  const int bm = fp4::gemm_block_rows(a->fmt, w4a4 ? fp4::kA_FP4 : fp4::kA_BF16,
                                      a->E > 0 ? P / a->E : P, a->H, a->I);
  // row-block table capacity: an expert with c > 0 rows takes ceil(c / bm) < c / bm + 1
  // blocks, and at most min(E, P) experts have rows, so fewer than P / bm + min(E, P)
  // blocks are ever used (every grouped GEMM launches this many row blocks, so the
  // bound matters when few tokens are routed)
  const int64_t nmb = (P + bm - 1) / bm + (a->E < P ? a->E : P);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  std::memset(&pl->L, 0, sizeof(pl->L));
  pl->scal = take(sizeof(float) * 4 * (size_t)a->E);
  pl->L.expert_offsets = take(sizeof(int32_t) * (size_t)(a->E + 1));
  pl->group_end = take(sizeof(int32_t) * (size_t)a->E);
  pl->L.sorted_rows = take(sizeof(int32_t) * (size_t)P);
  pl->L.inverse = take(sizeof(int32_t) * (size_t)P);
  pl->row_expert = take(sizeof(int32_t) * (size_t)P);
  pl->src_token = take(sizeof(int32_t) * (size_t)P);
  pl->mblk_expert = take(sizeof(int32_t) * (size_t)nmb);
  pl->mblk_row0 = take(sizeof(int32_t) * (size_t)nmb);
  pl->chunk_base = take(sizeof(int32_t) * (size_t)((P + fp4::kPermuteChunk - 1) /
                                                   fp4::kPermuteChunk) * (size_t)a->E);
  const int64_t x_rows = a->fmt == FP4_MXFP4 ? a->T : R;
  pl->L.x_rows = x_rows;
  pl->L.x_codes = take((size_t)x_rows * (size_t)(a->H / 2));
  pl->L.x_scales = take((size_t)x_rows * (size_t)(a->H / G));
  const int akind = w4a4 ? fp4::kA_FP4 : fp4::kA_BF16;
  pl->fuse_routed = fp4::gemm_can_fuse_swiglu(a->fmt, akind, P, a->H, a->I, true, bm, nmb);
  pl->fuse_shared = sh && fp4::gemm_can_fuse_swiglu(a->fmt, akind, a->T, a->H, a->I, false, bm, 1);
  const int64_t gu_rows = (pl->fuse_routed ? 0 : P) + (sh && !pl->fuse_shared ? a->T : 0);
  pl->L.gu_rows = gu_rows;
  pl->L.swiglu_fused = (pl->fuse_routed ? 1 : 0) | (pl->fuse_shared ? 2 : 0);
  pl->L.gu = take(sizeof(float) * (size_t)gu_rows * (size_t)(2 * a->I));
  pl->L.h_codes = take((size_t)R * (size_t)(a->I / 2));
  pl->L.h_scales = take((size_t)R * (size_t)(a->I / G));
  pl->L.h_bf16 = may_w4a16 ? take(sizeof(uint16_t) * (size_t)R * (size_t)a->I) : 0;
  pl->L.y = take(sizeof(float) * (size_t)R * (size_t)a->H);
  pl->L.total_bytes = off;
  pl->P = P;
  pl->R = R;
  pl->n_mblocks = nmb;
  pl->bm = bm;
  pl->shared = sh;
  pl->w4a4 = w4a4;
}

// Validation shared by the size/layout queries and the call itself.  Sets
// *w4a4_eff to the mode the call will run in and *may_w4a16 to whether the layout
// needs the bf16 intermediate region.
fp4_status moe_validate(const fp4_moe_args* a, bool* w4a4_eff, bool* may_w4a16) {
  if (!a) return FP4_ERR_NULL;
  if (!fmt_ok(a->fmt) || !mode_ok(a->mode) || (a->flags & ~FP4_FLAG_ALLOW_W4A16_FALLBACK))
    return FP4_ERR_FORMAT;
  const int64_t G = group_of(a->fmt);
  if (a->T < 0 || a->H <= 0 || a->I <= 0 || a->E <= 0 || a->E > 1024 || a->k < 1 ||
      a->k > a->E || a->k > 32 || a->H % G || a->I % G)
    return FP4_ERR_SHAPE;
  if (!a->hidden_bf16 || !a->topk_ids || !a->topk_w || !a->w13_codes || !a->w13_scales ||
      !a->w2_codes || !a->w2_scales || !a->out_bf16)
    return FP4_ERR_NULL;
  const bool sh = moe_shared(a);
  if (sh && !(a->sh_w13_codes && a->sh_w13_scales && a->sh_w2_codes && a->sh_w2_scales))
    return FP4_ERR_NULL;
  const void* ptrs[] = {a->hidden_bf16, a->topk_ids, a->topk_w, a->w13_codes, a->w13_scales,
                        a->w2_codes, a->w2_scales, a->out_bf16, a->sh_w13_codes,
                        a->sh_w13_scales, a->sh_w2_codes, a->sh_w2_scales};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return FP4_ERR_ALIGN;
  const bool nv = a->fmt == FP4_NVFP4;
  if (nv) {
    if (!a->w13_scale_2 || !a->w2_scale_2) return FP4_ERR_WEIGHT_SCALE;
    for (int64_t e = 0; e < a->E; ++e)
      if (!scale_ok(a->w13_scale_2[e]) || !scale_ok(a->w2_scale_2[e])) return FP4_ERR_WEIGHT_SCALE;
    if (sh && (!scale_ok(a->sh_w13_scale_2) || !scale_ok(a->sh_w2_scale_2)))
      return FP4_ERR_WEIGHT_SCALE;
  } else {
    if (a->w13_scale_2 || a->w2_scale_2 || a->a13_scale || a->a2_scale) return FP4_ERR_FORMAT;
    if (sh && (a->sh_w13_scale_2 != 1.0f || a->sh_w2_scale_2 != 1.0f)) return FP4_ERR_FORMAT;
    if (sh && a->mode == FP4_W4A4 && (a->sh_a13_scale != 1.0f || a->sh_a2_scale != 1.0f))
      return FP4_ERR_FORMAT;
  }
  bool w4a4 = a->mode == FP4_W4A4;
  bool may16 = !w4a4;
  if (w4a4 && nv) {
    bool ok = a->a13_scale && a->a2_scale;
    for (int64_t e = 0; ok && e < a->E; ++e)
      ok = scale_ok(a->a13_scale[e]) && scale_ok(a->a2_scale[e]);
    if (ok && sh) ok = scale_ok(a->sh_a13_scale) && scale_ok(a->sh_a2_scale);
    const bool allow = (a->flags & FP4_FLAG_ALLOW_W4A16_FALLBACK) != 0;
    if (allow) may16 = true;
    if (!ok) {
      if (!allow) return FP4_ERR_INPUT_SCALE;
      w4a4 = false;
    }
  }
  *w4a4_eff = w4a4;
  *may_w4a16 = may16;
  return FP4_OK;
}

}  // namespace

extern "C" {

int fp4_arch_supported(const char* name) {
  if (!name) return 0;
  if (std::strncmp(name, "gfx950", 6) != 0) return 0;
  return name[6] == '\0' || name[6] == ':';
}

const char* fp4_status_str(fp4_status s) {
  switch (s) {
    case FP4_OK: return "FP4_OK";
    case FP4_OK_FELL_BACK_W4A16: return "FP4_OK_FELL_BACK_W4A16";
    case FP4_ERR_NULL: return "FP4_ERR_NULL";
    case FP4_ERR_SHAPE: return "FP4_ERR_SHAPE";
    case FP4_ERR_ALIGN: return "FP4_ERR_ALIGN";
    case FP4_ERR_INPUT_SCALE: return "FP4_ERR_INPUT_SCALE";
    case FP4_ERR_WEIGHT_SCALE: return "FP4_ERR_WEIGHT_SCALE";
    case FP4_ERR_FORMAT: return "FP4_ERR_FORMAT";
    case FP4_ERR_WORKSPACE: return "FP4_ERR_WORKSPACE";
    case FP4_ERR_DEVICE: return "FP4_ERR_DEVICE";
    case FP4_ERR_LAUNCH: return "FP4_ERR_LAUNCH";
  }
  return "FP4_UNKNOWN_STATUS";
}

const char* fp4_last_kernel(void) { return t_last_kernel; }

static fp4_status quantize_common(fp4_format fmt, const void* x, int in_f32, int64_t M,
                                  int64_t K, int64_t ldx, float scale, uint8_t* codes,
                                  uint8_t* scales, void* stream, fp4_status bad_scale) {
  if (!fmt_ok(fmt)) return FP4_ERR_FORMAT;
  const int64_t G = group_of(fmt);
  if (M < 0 || K < 0 || K % G) return FP4_ERR_SHAPE;
  if (M == 0 || K == 0) return FP4_OK;
  if (ldx < K) return FP4_ERR_SHAPE;
  if (!x || !codes || !scales) return FP4_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales) || ldx % (in_f32 ? 4 : 8))
    return FP4_ERR_ALIGN;
  if (fmt == FP4_NVFP4) {
    if (!scale_ok(scale)) return bad_scale;
  } else if (scale != 1.0f) {
    return FP4_ERR_FORMAT;
  }
  fp4_status st = device_check();
  if (st != FP4_OK) return st;
  fp4::QuantParams p{};
  p.x = x;
  p.in_f32 = in_f32;
  p.M = M;
  p.K = K;
  p.ldx = ldx;
  p.g = fmt == FP4_NVFP4 ? 1.0f / scale : 1.0f;
  p.codes = codes;
  p.scales = scales;
  const char* name = "";
  hipError_t e = fp4::launch_quant(fmt, p, (hipStream_t)stream, &name);
  return launched(e, name);
}

fp4_status fp4_quantize_act(fp4_format fmt, const void* x_bf16, int64_t M, int64_t K,
                            int64_t ldx, float input_scale, uint8_t* codes, uint8_t* scales,
                            void* stream) {
  return quantize_common(fmt, x_bf16, 0, M, K, ldx, input_scale, codes, scales, stream,
                         FP4_ERR_INPUT_SCALE);
}

fp4_status fp4_quantize_weight(fp4_format fmt, const float* w, int64_t N, int64_t K,
                               int64_t ldw, float weight_scale_2, uint8_t* codes,
                               uint8_t* scales, void* stream) {
  return quantize_common(fmt, w, 1, N, K, ldw, weight_scale_2, codes, scales, stream,
                         FP4_ERR_WEIGHT_SCALE);
}

size_t fp4_gemm_workspace_size(fp4_format fmt, fp4_mode mode, int64_t M, int64_t K,
                               int has_a_bf16) {
  if (!fmt_ok(fmt) || !mode_ok(mode) || M <= 0 || K <= 0) return 0;
  if (mode != FP4_W4A4 || !has_a_bf16) return 0;
  return gemm_ws_bytes(fmt, M, K);
}

size_t fp4_gemm_workspace_size_mnk(fp4_format fmt, fp4_mode mode, int64_t M, int64_t N,
                                   int64_t K, int has_a_bf16) {
  if (!fmt_ok(fmt) || !mode_ok(mode) || M <= 0 || N <= 0 || K <= 0) return 0;
  if (mode != FP4_W4A4 || K % group_of(fmt)) return 0;
  return (has_a_bf16 ? gemm_ws_bytes(fmt, M, K) : 0) + gemm_relayout_bytes(fmt, M, N, K);
}

}  // extern "C"

namespace {

// ---- the allocation-free variant's scratch ------------------------------------------
// One array per device (each device's code object holds its own copy), holding the
// fused W4A4 GEMM's quantized activations.  Host code never uses the symbol itself:
// its host-side name is a stand-in, not a device address.  The device address is
// resolved once per device, with that device current, and kept here.
static __device__ __align__(256) uint8_t scratch[FP4_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];

// Device address of the current device's scratch array (FP4_ERR_DEVICE if it cannot
// be resolved).
fp4_status scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return FP4_ERR_DEVICE;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return FP4_ERR_DEVICE;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FP4_OK;
}

// fp4_gemm and fp4_gemm_noalloc: with use_scratch the fused quantization writes into
// the device's scratch array (workspace / workspace_bytes are ignored, the capacity is
// FP4_NOALLOC_SCRATCH_BYTES) instead of a caller workspace.
fp4_status gemm_call(fp4_format fmt, fp4_mode mode, int64_t M, int64_t N, int64_t K,
                     const void* a_bf16, int64_t lda, const uint8_t* a_codes,
                     const uint8_t* a_scales, const uint8_t* w_codes, const uint8_t* w_scales,
                     float weight_scale_2, float input_scale, void* out, int64_t ldo,
                     fp4_out out_dtype, uint32_t flags, void* workspace,
                     size_t workspace_bytes, void* stream, bool use_scratch) {
  if (use_scratch) {
    workspace = nullptr;
    workspace_bytes = FP4_NOALLOC_SCRATCH_BYTES;
  }
  const bool prepared = (flags & FP4_FLAG_PREPARED_WEIGHTS) != 0;
  if (!fmt_ok(fmt) || !mode_ok(mode) || (out_dtype != FP4_OUT_BF16 && out_dtype != FP4_OUT_F32) ||
      (flags & ~(FP4_FLAG_ALLOW_W4A16_FALLBACK | FP4_FLAG_PREPARED_WEIGHTS)))
    return FP4_ERR_FORMAT;
  const int64_t G = group_of(fmt);
  if (M < 0 || N < 0 || K <= 0 || K % G) return FP4_ERR_SHAPE;
  // prepared weights feed the decode kernels: W4A4, at most 64 rows, whole blocks
  if (prepared && (mode != FP4_W4A4 || (flags & FP4_FLAG_ALLOW_W4A16_FALLBACK)))
    return FP4_ERR_FORMAT;
  if (prepared && (M > 64 || N % 16 || K % 128)) return FP4_ERR_SHAPE;
  if (M == 0 || N == 0) return FP4_OK;
  if (ldo < N) return FP4_ERR_SHAPE;
  const bool need_bf16 = mode == FP4_W4A16;
  if (!w_codes || !w_scales || !out) return FP4_ERR_NULL;
  if (need_bf16 && !a_bf16) return FP4_ERR_NULL;
  if (!a_bf16 && (!a_codes || !a_scales)) return FP4_ERR_NULL;
  if (a_bf16 && lda < K) return FP4_ERR_SHAPE;
  const void* ptrs[] = {a_bf16, a_codes, a_scales, w_codes, w_scales, out};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return FP4_ERR_ALIGN;
  if (a_bf16 && lda % 8) return FP4_ERR_ALIGN;
  const bool nv = fmt == FP4_NVFP4;
  if (nv) {
    if (!scale_ok(weight_scale_2)) return FP4_ERR_WEIGHT_SCALE;
  } else if (weight_scale_2 != 1.0f || (mode == FP4_W4A4 && input_scale != 1.0f)) {
    return FP4_ERR_FORMAT;
  }
  bool w4a4 = mode == FP4_W4A4;
  fp4_status ok_status = FP4_OK;
  if (w4a4 && nv && !scale_ok(input_scale)) {
    if (!(flags & FP4_FLAG_ALLOW_W4A16_FALLBACK) || !a_bf16) return FP4_ERR_INPUT_SCALE;
    w4a4 = false;
    ok_status = FP4_OK_FELL_BACK_W4A16;
  }
  const bool fused = w4a4 && a_bf16;
  if (fused) {
    if ((!use_scratch && !workspace) || workspace_bytes < gemm_ws_bytes(fmt, M, K))
      return FP4_ERR_WORKSPACE;
    if (!use_scratch && !aligned16(workspace)) return FP4_ERR_ALIGN;
  }
  fp4_status st = device_check();
  if (st != FP4_OK) return st;
  if (fused && use_scratch) {
    st = scratch_for_current_device(&workspace);
    if (st != FP4_OK) return st;
  }

  // Room for the stage-ordered scales after the fused quantization's area: used when
  // the GEMM runs on the 256 x 256 tile (else its scales are gathered row by row)
  const size_t fused_bytes = fused ? gemm_ws_bytes(fmt, M, K) : 0;
  const size_t relayout_bytes = w4a4 ? gemm_relayout_bytes(fmt, M, N, K) : 0;
  bool relayout = false;
  if (relayout_bytes && (use_scratch || (workspace && aligned16(workspace))) &&
      workspace_bytes >= fused_bytes + relayout_bytes) {
    if (use_scratch && !fused) {
      st = scratch_for_current_device(&workspace);
      if (st != FP4_OK) return st;
    }
    relayout = true;
  }

  hipStream_t s = (hipStream_t)stream;
  const char* name = "";
  const uint8_t* ac = a_codes;
  const uint8_t* as = a_scales;
  if (fused) {
    uint8_t* wsb = static_cast<uint8_t*>(workspace);
    fp4::QuantParams q{};
    q.x = a_bf16;
    q.in_f32 = 0;
    q.M = M;
    q.K = K;
    q.ldx = lda;
    q.g = nv ? 1.0f / input_scale : 1.0f;
    q.codes = wsb;
    q.scales = wsb + align256((size_t)M * (size_t)(K / 2));
    hipError_t e = fp4::launch_quant(fmt, q, s, &name);
    if (e != hipSuccess) return launched(e, name);
    ac = q.codes;
    as = q.scales;
  }
  fp4::GemmParams p{};
  p.M = M;
  p.N = N;
  p.K = K;
  p.a_codes = ac;
  p.a_scales = as;
  p.a_bf16 = static_cast<const uint16_t*>(a_bf16);
  p.lda = lda;
  p.w_tiled = prepared ? 1 : 0;
  p.w_codes = w_codes;
  p.w_scales = w_scales;
  p.alpha = nv ? (w4a4 ? weight_scale_2 * input_scale : weight_scale_2) : 1.0f;
  p.out = out;
  p.ldo = ldo;
  p.out_f32 = out_dtype == FP4_OUT_F32;
  if (relayout) {
    uint8_t* a_t = static_cast<uint8_t*>(workspace) + fused_bytes;
    uint8_t* w_t = a_t + align256(fp4::scale_relayout_bytes(nv ? fp4::kNV : fp4::kMX, M, K));
    hipError_t e = fp4::launch_scale_relayout(nv ? fp4::kNV : fp4::kMX, as, M, w_scales, N, K,
                                              a_t, w_t, s);
    if (e != hipSuccess) return launched(e, "scale_relayout");
    p.a_scales_t = a_t;
    p.w_scales_t = w_t;
  }
  hipError_t e = fp4::launch_gemm(fmt, w4a4 ? fp4::kA_FP4 : fp4::kA_BF16, p, s, &name);
  st = launched(e, name);
  return st == FP4_OK ? ok_status : st;
}

}  // namespace

extern "C" {

fp4_status fp4_gemm(fp4_format fmt, fp4_mode mode, int64_t M, int64_t N, int64_t K,
                    const void* a_bf16, int64_t lda, const uint8_t* a_codes,
                    const uint8_t* a_scales, const uint8_t* w_codes, const uint8_t* w_scales,
                    float weight_scale_2, float input_scale, void* out, int64_t ldo,
                    fp4_out out_dtype, uint32_t flags, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return gemm_call(fmt, mode, M, N, K, a_bf16, lda, a_codes, a_scales, w_codes, w_scales,
                   weight_scale_2, input_scale, out, ldo, out_dtype, flags, workspace,
                   workspace_bytes, stream, false);
}

fp4_status fp4_gemm_noalloc(fp4_format fmt, fp4_mode mode, int64_t M, int64_t N, int64_t K,
                            const void* a_bf16, int64_t lda, const uint8_t* a_codes,
                            const uint8_t* a_scales, const uint8_t* w_codes,
                            const uint8_t* w_scales, float weight_scale_2, float input_scale,
                            void* out, int64_t ldo, fp4_out out_dtype, uint32_t flags,
                            void* stream) {
  return gemm_call(fmt, mode, M, N, K, a_bf16, lda, a_codes, a_scales, w_codes, w_scales,
                   weight_scale_2, input_scale, out, ldo, out_dtype, flags, nullptr, 0, stream,
                   true);
}

size_t fp4_prepared_weight_bytes(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || N % 16 || K % 128) return 0;
  return (size_t)N * (size_t)(K / 2);
}

fp4_status fp4_prepare_weights(fp4_format fmt, const uint8_t* w_codes, const uint8_t* w_scales,
                               int64_t N, int64_t K, uint8_t* prepared_codes, int32_t* check,
                               void* stream) {
  if (!fmt_ok(fmt)) return FP4_ERR_FORMAT;
  if (N <= 0 || K <= 0 || N % 16 || K % 128) return FP4_ERR_SHAPE;
  if (!w_codes || !w_scales || !prepared_codes || !check) return FP4_ERR_NULL;
  if (!aligned16(w_codes) || !aligned16(w_scales) || !aligned16(prepared_codes) ||
      (reinterpret_cast<uintptr_t>(check) & 3u))
    return FP4_ERR_ALIGN;
  fp4_status st = device_check();
  if (st != FP4_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (hipMemsetAsync(check, 0, sizeof(int32_t), s) != hipSuccess) return launched(hipGetLastError(), "");
  hipError_t e = fp4::launch_prepare(fmt, w_codes, w_scales, N, K, prepared_codes, check, s);
  st = launched(e, "prepare_weights");
  if (st != FP4_OK) return st;
  int32_t bad = 0;
  if (hipMemcpyAsync(&bad, check, sizeof(bad), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess) {
    (void)hipGetLastError();
    return FP4_ERR_LAUNCH;
  }
  return bad ? FP4_ERR_WEIGHT_SCALE : FP4_OK;
}

fp4_status fp4_moe_topk_softmax(const float* logits, int64_t T, int64_t E, int k,
                                int renormalize, int32_t* topk_ids, float* topk_w,
                                void* stream) {
  if (T < 0 || E <= 0 || E > 1024 || k < 1 || k > E || k > 32) return FP4_ERR_SHAPE;
  if (T == 0) return FP4_OK;
  if (!logits || !topk_ids || !topk_w) return FP4_ERR_NULL;
  if (!aligned16(logits) || !aligned16(topk_ids) || !aligned16(topk_w)) return FP4_ERR_ALIGN;
  fp4_status st = device_check();
  if (st != FP4_OK) return st;
  const char* name = "";
  hipError_t e = fp4::launch_topk_softmax(logits, T, E, k, renormalize, topk_ids, topk_w,
                                          (hipStream_t)stream, &name);
  return launched(e, name);
}

size_t fp4_moe_workspace_size(const fp4_moe_args* a) {
  bool w4a4 = false, may16 = false;
  if (moe_validate(a, &w4a4, &may16) != FP4_OK) return 0;
  MoePlan pl;
  moe_plan(a, w4a4, may16, &pl);
  return pl.L.total_bytes;
}

fp4_status fp4_moe_workspace_layout(const fp4_moe_args* a, fp4_moe_layout* layout) {
  if (!layout) return FP4_ERR_NULL;
  bool w4a4 = false, may16 = false;
  fp4_status st = moe_validate(a, &w4a4, &may16);
  if (st != FP4_OK) return st;
  MoePlan pl;
  moe_plan(a, w4a4, may16, &pl);
  *layout = pl.L;
  return FP4_OK;
}

fp4_status fp4_moe_grouped_gemm(const fp4_moe_args* a, void* workspace, size_t ws_bytes,
                                void* stream) {
  bool w4a4 = false, may16 = false;
  fp4_status st = moe_validate(a, &w4a4, &may16);
  if (st != FP4_OK) return st;
  if (a->T == 0) return FP4_OK;
  MoePlan pl;
  moe_plan(a, w4a4, may16, &pl);
  if (!workspace || ws_bytes < pl.L.total_bytes) return FP4_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FP4_ERR_ALIGN;
  st = device_check();
  if (st != FP4_OK) return st;
  const fp4_status ok_status =
      (a->mode == FP4_W4A4 && !w4a4) ? FP4_OK_FELL_BACK_W4A16 : FP4_OK;

  hipStream_t s = (hipStream_t)stream;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const bool nv = a->fmt == FP4_NVFP4;
  const int fmt = a->fmt;
  const int64_t E = a->E, T = a->T, H = a->H, I = a->I, G = group_of(fmt);
  const int64_t P = pl.P;
  const char* name = "";
  hipError_t e;
#define FP4_TRY(expr)                          \
  do {                                         \
    e = (expr);                                \
    if (e != hipSuccess) return launched(e, name); \
  } while (0)

  // 1. per-expert scalars: quantize multipliers 1/a_scale and dequant alphas
  float* scal = reinterpret_cast<float*>(ws + pl.scal);
  float* g13 = scal;
  float* alpha13 = scal + E;
  float* g2 = scal + 2 * E;
  float* alpha2 = scal + 3 * E;
  std::vector<float> h;
  if (nv) {   // (MXFP4 reads none of them: alpha and the block-scale rule are fixed)
    h.assign(4 * (size_t)E, 1.0f);
    for (int64_t x = 0; x < E; ++x) {
      if (nv) {
        const float w13 = a->w13_scale_2[x], w2 = a->w2_scale_2[x];
        if (w4a4) {
          h[x] = 1.0f / a->a13_scale[x];
          h[E + x] = w13 * a->a13_scale[x];
          h[2 * E + x] = 1.0f / a->a2_scale[x];
          h[3 * E + x] = w2 * a->a2_scale[x];
        } else {
          h[E + x] = w13;
          h[3 * E + x] = w2;
        }
      }
    }
  }
  const float sh_g13 = (nv && w4a4) ? 1.0f / a->sh_a13_scale : 1.0f;
  const float sh_g2 = (nv && w4a4) ? 1.0f / a->sh_a2_scale : 1.0f;
  const float sh_alpha13 = nv ? (w4a4 ? a->sh_w13_scale_2 * a->sh_a13_scale : a->sh_w13_scale_2) : 1.0f;
  const float sh_alpha2 = nv ? (w4a4 ? a->sh_w2_scale_2 * a->sh_a2_scale : a->sh_w2_scale_2) : 1.0f;

  // 2. dispatch bookkeeping
  bool act_quantized = false;
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + pl.L.expert_offsets);
  int32_t* group_end = reinterpret_cast<int32_t*>(ws + pl.group_end);
  int32_t* sorted_rows = reinterpret_cast<int32_t*>(ws + pl.L.sorted_rows);
  int32_t* inverse = reinterpret_cast<int32_t*>(ws + pl.L.inverse);
  int32_t* row_expert = reinterpret_cast<int32_t*>(ws + pl.row_expert);
  int32_t* src_token = reinterpret_cast<int32_t*>(ws + pl.src_token);
  int32_t* mblk_expert = reinterpret_cast<int32_t*>(ws + pl.mblk_expert);
  int32_t* mblk_row0 = reinterpret_cast<int32_t*>(ws + pl.mblk_row0);
  // a few routed slots of an NVFP4 W4A4 layer without a shared expert: the whole
  // layer in two launches (the workspace rows it writes are the ones below)
  if (nv && w4a4 && !pl.shared && pl.fuse_routed &&
      fp4::moe_small_fits(T, a->k, E, H, I)) {
    fp4::MoeSmallParams q{};
    q.T = T;
    q.H = H;
    q.I = I;
    q.E = E;
    q.k = a->k;
    q.hidden = static_cast<const uint16_t*>(a->hidden_bf16);
    q.ids = a->topk_ids;
    q.w = a->topk_w;
    q.w13_codes = a->w13_codes;
    q.w13_scales = a->w13_scales;
    q.w2_codes = a->w2_codes;
    q.w2_scales = a->w2_scales;
    q.expert_offsets = offsets;
    q.sorted_rows = sorted_rows;
    q.inverse = inverse;
    q.x_codes = ws + pl.L.x_codes;
    q.x_scales = ws + pl.L.x_scales;
    q.h_codes = ws + pl.L.h_codes;
    q.h_scales = ws + pl.L.h_scales;
    q.y = reinterpret_cast<float*>(ws + pl.L.y);
    q.out = static_cast<uint16_t*>(a->out_bf16);
    FP4_TRY(fp4::launch_moe_small(q, h.data(), s, &name));
    return ok_status;
  }
  {
    fp4::PermuteParams pp{};
    pp.ids = a->topk_ids;
    pp.T = T;
    pp.k = a->k;
    pp.E = E;
    pp.bm = pl.bm;
    pp.n_mblocks = pl.n_mblocks;
    pp.expert_offsets = offsets;
    pp.sorted_rows = sorted_rows;
    pp.inverse = inverse;
    pp.row_expert = row_expert;
    pp.src_token = src_token;
    pp.mblk_expert = mblk_expert;
    pp.mblk_row0 = mblk_row0;
    pp.group_end = group_end;
    pp.chunk_base = reinterpret_cast<int32_t*>(ws + pl.chunk_base);
    // the scalar upload travels with the dispatch launch (its own launch only when
    // the dispatch takes several), and so may the GEMM1 activation quantization
    pp.up_dst = nv ? scal : nullptr;
    pp.up_n = nv ? (int)(4 * E) : 0;
    pp.q_fmt = -1;
    if (w4a4) {
      pp.q_fmt = fmt;
      pp.q_x = static_cast<const uint16_t*>(a->hidden_bf16);
      pp.q_K = H;
      pp.q_codes = ws + pl.L.x_codes;
      pp.q_scales = ws + pl.L.x_scales;
      pp.q_routed = nv ? 1 : 0;      // NVFP4: each routed row under its expert's scale
      pp.q_rows = nv ? P : T;        // MXFP4: each token once
      pp.q_g_off = 0;                // 1/a13_scale[e] are the first E uploaded values
      pp.q_g = 1.0f;
    }
    FP4_TRY(fp4::launch_permute(pp, nv ? h.data() : nullptr, s, &name, &act_quantized));
  }

  // 3. GEMM1 input
  uint8_t* x_codes = ws + pl.L.x_codes;
  uint8_t* x_scales = ws + pl.L.x_scales;
  if (w4a4) {
    fp4::QuantParams q{};
    q.x = a->hidden_bf16;
    q.in_f32 = 0;
    q.K = H;
    q.ldx = H;
    q.codes = x_codes;
    q.scales = x_scales;
    if (!nv) {  // MXFP4: each token once, shared by all its experts
      q.M = T;
      q.g = 1.0f;
      if (!act_quantized) FP4_TRY(fp4::launch_quant(fmt, q, s, &name));
    } else {    // NVFP4: each routed row under its expert's activation scale
      q.M = P;
      q.row_src = src_token;
      q.row_grp = row_expert;
      q.grp_g = g13;
      if (!act_quantized) FP4_TRY(fp4::launch_quant(fmt, q, s, &name));
      if (pl.shared) {
        fp4::QuantParams qs{};
        qs.x = a->hidden_bf16;
        qs.K = H;
        qs.ldx = H;
        qs.M = T;
        qs.g = sh_g13;
        qs.codes = x_codes + (size_t)P * (H / 2);
        qs.scales = x_scales + (size_t)P * (H / G);
        FP4_TRY(fp4::launch_quant(fmt, qs, s, &name));
      }
    }
  }
  const int akind = w4a4 ? fp4::kA_FP4 : fp4::kA_BF16;

  // 4. grouped GEMM1 (gate and up) into gu fp32, or straight into the quantized h
  //    when the SwiGLU + requant epilogue is fused
  float* gu = reinterpret_cast<float*>(ws + pl.L.gu);
  float* gu_shared = gu + (size_t)(pl.fuse_routed ? 0 : P) * (size_t)(2 * I);
  uint8_t* h_codes = ws + pl.L.h_codes;
  uint8_t* h_scales = ws + pl.L.h_scales;
  uint16_t* h_bf16 = pl.L.h_bf16 ? reinterpret_cast<uint16_t*>(ws + pl.L.h_bf16) : nullptr;
  {
    fp4::GemmParams p{};
    p.M = P;
    p.N = 2 * I;
    p.K = H;
    if (w4a4) {
      p.a_codes = x_codes;
      p.a_scales = x_scales;
      p.a_gather = nv ? nullptr : src_token;
    } else {
      p.a_bf16 = static_cast<const uint16_t*>(a->hidden_bf16);
      p.lda = H;
      p.a_gather = src_token;
    }
    p.w_codes = a->w13_codes;
    p.w_scales = a->w13_scales;
    p.w_estride_codes = 2 * I * (H / 2);
    p.w_estride_scales = 2 * I * (H / G);
    p.mblk_expert = mblk_expert;
    p.mblk_row0 = mblk_row0;
    p.group_end = group_end;
    p.n_mblocks = pl.n_mblocks;
    p.bm = pl.bm;
    p.alpha_g = nv ? alpha13 : nullptr;
    p.alpha = 1.0f;
    if (pl.fuse_routed) {
      p.fuse_swiglu = 1;
      p.I = I;
      p.h_grp_g = nv ? g2 : nullptr;
      p.h_g = 1.0f;
      p.h_codes = h_codes;
      p.h_scales = h_scales;
    } else {
      p.out = gu;
      p.ldo = 2 * I;
      p.out_f32 = 1;
    }
    FP4_TRY(fp4::launch_gemm(fmt, akind, p, s, &name));
    if (pl.shared) {
      fp4::GemmParams q{};
      q.M = T;
      q.N = 2 * I;
      q.K = H;
      if (w4a4) {
        const int64_t r0 = nv ? P : 0;
        q.a_codes = x_codes + (size_t)r0 * (H / 2);
        q.a_scales = x_scales + (size_t)r0 * (H / G);
      } else {
        q.a_bf16 = static_cast<const uint16_t*>(a->hidden_bf16);
        q.lda = H;
      }
      q.w_codes = a->sh_w13_codes;
      q.w_scales = a->sh_w13_scales;
      q.alpha = sh_alpha13;
      if (pl.fuse_shared) {
        q.fuse_swiglu = 1;
        q.I = I;
        q.h_g = sh_g2;
        q.h_codes = h_codes + (size_t)P * (I / 2);
        q.h_scales = h_scales + (size_t)P * (I / G);
      } else {
        q.out = gu_shared;
        q.ldo = 2 * I;
        q.out_f32 = 1;
      }
      FP4_TRY(fp4::launch_gemm(fmt, akind, q, s, &name));
    }
  }

  // 5. SwiGLU + requant (or bf16) of the intermediate, for the unfused parts
  {
    fp4::SwigluParams sp{};
    sp.gu = gu;
    sp.R = P;
    sp.I = I;
    sp.mode_w4a16 = !w4a4;
    sp.fmt = fmt;
    sp.row_grp = nv ? row_expert : nullptr;
    sp.grp_g = g2;
    sp.g = 1.0f;
    sp.h_codes = h_codes;
    sp.h_scales = h_scales;
    sp.h_bf16 = h_bf16;
    if (!pl.fuse_routed) FP4_TRY(fp4::launch_swiglu(sp, s, &name));
    if (pl.shared && !pl.fuse_shared) {
      fp4::SwigluParams ss = sp;
      ss.gu = gu_shared;
      ss.R = T;
      ss.row_grp = nullptr;
      ss.g = sh_g2;
      ss.h_codes = h_codes + (size_t)P * (I / 2);
      ss.h_scales = h_scales + (size_t)P * (I / G);
      ss.h_bf16 = h_bf16 ? h_bf16 + (size_t)P * I : nullptr;
      FP4_TRY(fp4::launch_swiglu(ss, s, &name));
    }
  }

  // 6. grouped GEMM2 (down) into y [R, H] fp32
  float* y = reinterpret_cast<float*>(ws + pl.L.y);
  {
    fp4::GemmParams p{};
    p.M = P;
    p.N = H;
    p.K = I;
    if (w4a4) {
      p.a_codes = h_codes;
      p.a_scales = h_scales;
    } else {
      p.a_bf16 = h_bf16;
      p.lda = I;
    }
    p.w_codes = a->w2_codes;
    p.w_scales = a->w2_scales;
    p.w_estride_codes = H * (I / 2);
    p.w_estride_scales = H * (I / G);
    p.mblk_expert = mblk_expert;
    p.mblk_row0 = mblk_row0;
    p.group_end = group_end;
    p.n_mblocks = pl.n_mblocks;
    p.bm = pl.bm;
    p.alpha_g = nv ? alpha2 : nullptr;
    p.alpha = 1.0f;
    p.out = y;
    p.ldo = H;
    p.out_f32 = 1;
    FP4_TRY(fp4::launch_gemm(fmt, akind, p, s, &name));
    if (pl.shared) {
      fp4::GemmParams q{};
      q.M = T;
      q.N = H;
      q.K = I;
      if (w4a4) {
        q.a_codes = h_codes + (size_t)P * (I / 2);
        q.a_scales = h_scales + (size_t)P * (I / G);
      } else {
        q.a_bf16 = h_bf16 + (size_t)P * I;
        q.lda = I;
      }
      q.w_codes = a->sh_w2_codes;
      q.w_scales = a->sh_w2_scales;
      q.alpha = sh_alpha2;
      q.out = y + (size_t)P * H;
      q.ldo = H;
      q.out_f32 = 1;
      FP4_TRY(fp4::launch_gemm(fmt, akind, q, s, &name));
    }
  }

  // 7. combine
  {
    fp4::CombineParams cp{};
    cp.y = y;
    cp.inverse = inverse;
    cp.w = a->topk_w;
    cp.T = T;
    cp.H = H;
    cp.k = a->k;
    cp.y_shared = pl.shared ? y + (size_t)P * H : nullptr;
    cp.out = static_cast<uint16_t*>(a->out_bf16);
    FP4_TRY(fp4::launch_combine(cp, s, &name));
  }
#undef FP4_TRY
  t_last_kernel = "moe";
  return ok_status;
}

}  // extern "C"

// ---- FP8 family (MXFP8, FP8 W8A8) ---------------------------------------------------
namespace {

static_assert(FP8_MX == fp4::kF8_MX && FP8_PER_TENSOR == fp4::kF8_TENSOR &&
                  FP8_ROWWISE == fp4::kF8_ROW && FP8_BLOCK == fp4::kF8_BLOCK,
              "fp8_scaling codes are the kernels' mode numbers");

bool f8mode_ok(int m) { return m == FP8_MX || m == FP8_PER_TENSOR || m == FP8_ROWWISE || m == FP8_BLOCK; }
int64_t f8_kmult(int m) { return m == FP8_MX ? 32 : (m == FP8_BLOCK ? 128 : 8); }

fp4_status fp8_quantize_common(int mode, const void* x, bool weight, int64_t M, int64_t K,
                               int64_t ldx, float ts, uint8_t* codes, void* scales,
                               void* stream, fp4_status bad_scale) {
  if (!f8mode_ok(mode)) return FP4_ERR_FORMAT;
  if (M < 0 || K < 0 || K % f8_kmult(mode)) return FP4_ERR_SHAPE;
  if (M == 0 || K == 0) return FP4_OK;
  if (ldx < K) return FP4_ERR_SHAPE;
  const bool tensor = mode == FP8_PER_TENSOR;
  if (!x || !codes || (!tensor && !scales)) return FP4_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes) || (scales && !aligned16(scales)) ||
      ldx % (weight ? 4 : 8))
    return FP4_ERR_ALIGN;
  if (tensor) {
    if (!scale_ok(ts)) return bad_scale;
    if (scales) return FP4_ERR_FORMAT;
  } else if (ts != 1.0f) {
    return FP4_ERR_FORMAT;
  }
  fp4_status st = device_check();
  if (st != FP4_OK) return st;
  fp4::Fp8QuantParams p{};
  p.x = x;
  p.in_f32 = weight ? 1 : 0;
  p.M = M;
  p.K = K;
  p.ldx = ldx;
  p.weight_blocks = weight && mode == FP8_BLOCK;
  p.tensor_scale = ts;
  p.codes = codes;
  p.mx_scales = mode == FP8_MX ? static_cast<uint8_t*>(scales) : nullptr;
  p.f_scales = (mode == FP8_ROWWISE || mode == FP8_BLOCK) ? static_cast<float*>(scales) : nullptr;
  const char* name = "";
  hipError_t e = fp4::launch_fp8_quant(mode, p, (hipStream_t)stream, &name);
  return launched(e, name);
}

}  // namespace

extern "C" {

fp4_status fp8_quantize_act(fp8_scaling mode, const void* x_bf16, int64_t M, int64_t K,
                            int64_t ldx, float tensor_scale, uint8_t* codes, void* scales,
                            void* stream) {
  return fp8_quantize_common(mode, x_bf16, false, M, K, ldx, tensor_scale, codes, scales,
                             stream, FP4_ERR_INPUT_SCALE);
}

fp4_status fp8_quantize_weight(fp8_scaling mode, const float* w, int64_t N, int64_t K,
                               int64_t ldw, float tensor_scale, uint8_t* codes, void* scales,
                               void* stream) {
  return fp8_quantize_common(mode, w, true, N, K, ldw, tensor_scale, codes, scales, stream,
                             FP4_ERR_WEIGHT_SCALE);
}

fp4_status fp8_gemm(fp8_scaling mode, int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                    const void* a_scales, float a_tensor_scale, const uint8_t* w_codes,
                    const void* w_scales, float w_tensor_scale, void* out, int64_t ldo,
                    fp4_out out_dtype, void* stream) {
  if (!f8mode_ok(mode) || (out_dtype != FP4_OUT_BF16 && out_dtype != FP4_OUT_F32))
    return FP4_ERR_FORMAT;
  if (M < 0 || N < 0 || K <= 0 || K % 128) return FP4_ERR_SHAPE;
  if (M == 0 || N == 0) return FP4_OK;
  if (ldo < N) return FP4_ERR_SHAPE;
  const bool tensor = mode == FP8_PER_TENSOR;
  if (!a_codes || !w_codes || !out || (!tensor && (!a_scales || !w_scales))) return FP4_ERR_NULL;
  const void* ptrs[] = {a_codes, a_scales, w_codes, w_scales, out};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return FP4_ERR_ALIGN;
  float alpha = 1.0f;
  if (tensor) {
    if (!scale_ok(a_tensor_scale)) return FP4_ERR_INPUT_SCALE;
    if (!scale_ok(w_tensor_scale)) return FP4_ERR_WEIGHT_SCALE;
    alpha = a_tensor_scale * w_tensor_scale;
    // the product is applied once per output: it must be a finite normal fp32
    if (!std::isfinite(alpha) || alpha < 0x1p-126f) return FP4_ERR_INPUT_SCALE;
    if (a_scales || w_scales) return FP4_ERR_FORMAT;
  } else if (a_tensor_scale != 1.0f || w_tensor_scale != 1.0f) {
    return FP4_ERR_FORMAT;
  }
  fp4_status st = device_check();
  if (st != FP4_OK) return st;
  fp4::Fp8GemmParams p{};
  p.M = M;
  p.N = N;
  p.K = K;
  p.a_codes = a_codes;
  p.w_codes = w_codes;
  if (mode == FP8_MX) {
    p.a_mx = static_cast<const uint8_t*>(a_scales);
    p.w_mx = static_cast<const uint8_t*>(w_scales);
  } else if (!tensor) {
    p.a_s = static_cast<const float*>(a_scales);
    p.w_s = static_cast<const float*>(w_scales);
  }
  p.alpha = alpha;
  p.unit_scale = 127;   // e8m0 code of 1.0: the MFMA's block scale for non-MX modes
  p.out = out;
  p.ldo = ldo;
  p.out_f32 = out_dtype == FP4_OUT_F32;
  const char* name = "";
  hipError_t e = fp4::launch_fp8_gemm(mode, p, (hipStream_t)stream, &name);
  return launched(e, name);
}

}  // extern "C"

// ---- MX formats of any element type --------------------------------------------------
namespace {

// the scaled MFMA's element-type code of each mx_elem (e4m3 0, e2m3 2, e3m2 3, e2m1 4)
int mfma_code(int t) { return t == MX_E2M1 ? 4 : (t == MX_E2M3 ? 2 : (t == MX_E3M2 ? 3 : 0)); }
bool elem_ok(int t) { return t == MX_E2M1 || t == MX_E2M3 || t == MX_E3M2 || t == MX_E4M3; }

fp4_status mx_quantize_common(int t, const void* x, bool weight, int64_t M, int64_t K,
                              int64_t ldx, uint8_t* codes, uint8_t* scales, void* stream) {
  if (!elem_ok(t)) return FP4_ERR_FORMAT;
  if (M < 0 || K < 0 || K % 32) return FP4_ERR_SHAPE;
  if (M == 0 || K == 0) return FP4_OK;
  if (ldx < K) return FP4_ERR_SHAPE;
  if (!x || !codes || !scales) return FP4_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales) || ldx % (weight ? 4 : 8))
    return FP4_ERR_ALIGN;
  fp4_status st = device_check();
  if (st != FP4_OK) return st;
  const hipStream_t s = (hipStream_t)stream;
  const char* name = "";
  hipError_t e;
  if (t == MX_E2M1) {                     // the MXFP4 quantizer of fp4_quantize_act
    fp4::QuantParams q{};
    q.x = x;
    q.in_f32 = weight ? 1 : 0;
    q.M = M;
    q.K = K;
    q.ldx = ldx;
    q.g = 1.0f;
    q.codes = codes;
    q.scales = scales;
    e = fp4::launch_quant(FP4_MXFP4, q, s, &name);
  } else {
    fp4::Fp8QuantParams q{};
    q.x = x;
    q.in_f32 = weight ? 1 : 0;
    q.M = M;
    q.K = K;
    q.ldx = ldx;
    q.tensor_scale = 1.0f;
    q.codes = codes;
    q.mx_scales = scales;
    e = t == MX_E4M3 ? fp4::launch_fp8_quant(fp4::kF8_MX, q, s, &name)
                     : fp4::launch_mx6_quant(mfma_code(t), q, s, &name);
  }
  return launched(e, name);
}

}  // namespace

extern "C" {

fp4_status mx_quantize_act(mx_elem t, const void* x_bf16, int64_t M, int64_t K, int64_t ldx,
                           uint8_t* codes, uint8_t* scales, void* stream) {
  return mx_quantize_common(t, x_bf16, false, M, K, ldx, codes, scales, stream);
}

fp4_status mx_quantize_weight(mx_elem t, const float* w, int64_t N, int64_t K, int64_t ldw,
                              uint8_t* codes, uint8_t* scales, void* stream) {
  return mx_quantize_common(t, w, true, N, K, ldw, codes, scales, stream);
}

fp4_status mx_gemm(mx_elem a_t, mx_elem w_t, int64_t M, int64_t N, int64_t K,
                   const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* w_codes,
                   const uint8_t* w_scales, void* out, int64_t ldo, fp4_out out_dtype,
                   void* stream) {
  if (!elem_ok(a_t) || !elem_ok(w_t) || (out_dtype != FP4_OUT_BF16 && out_dtype != FP4_OUT_F32))
    return FP4_ERR_FORMAT;
  if (M < 0 || N < 0 || K <= 0 || K % 128) return FP4_ERR_SHAPE;
  if (M == 0 || N == 0) return FP4_OK;
  if (ldo < N) return FP4_ERR_SHAPE;
  if (!a_codes || !a_scales || !w_codes || !w_scales || !out) return FP4_ERR_NULL;
  const void* ptrs[] = {a_codes, a_scales, w_codes, w_scales, out};
  for (const void* q : ptrs)
    if (!aligned16(q)) return FP4_ERR_ALIGN;
  fp4_status st = device_check();
  if (st != FP4_OK) return st;
  fp4::Fp8GemmParams p{};
  p.M = M;
  p.N = N;
  p.K = K;
  p.a_codes = a_codes;
  p.w_codes = w_codes;
  p.a_mx = a_scales;
  p.w_mx = w_scales;
  p.alpha = 1.0f;
  p.unit_scale = 127;
  p.out = out;
  p.ldo = ldo;
  p.out_f32 = out_dtype == FP4_OUT_F32;
  const char* name = "";
  hipError_t e = fp4::launch_mx_gemm(mfma_code(a_t), mfma_code(w_t), p, (hipStream_t)stream, &name);
  return launched(e, name);
}

}  // extern "C"
