// W4A16 for many activation rows: bf16 activations times FP4 weights (NVFP4 or MXFP4)
// decoded exactly to bf16, on gfx950's bf16 32x32x16 MFMA ("vLLM on the DGX Spark, the
// Hard Way: Seven Months of GB10 Field Notes", the rule that explains the FP4
// confusion: a weight-only checkpoint multiplies 16-bit activations by the dequantized
// weights, which is what costs it prefill; "vLLM per-format kernel capability matrix
// derived from source", THE EMULATION COLUMN: dequantize, multiply in high precision).
//
// Exactness: an e2m1 value times an e4m3 scale has at most six significant bits and lies
// in [2^-10, 2688], a bf16 number; an e2m1 value times an e8m0 scale is a bf16 number
// unless the product leaves bf16's exponent range (scale codes above 253).  The
// products are summed by the MFMA in fp32.
//
// Tiling.  A workgroup of 8 waves owns 256 weight rows and 128 activation rows; wave w
// holds weight rows 32 w .. 32 w + 31 against all 128 activation rows (four 32 x 32
// accumulator blocks), so each decoded weight operand feeds four MFMAs and the bf16
// activations need no conversion.  K advances in stages of 128.  Inside a stage the
// MFMA's 16 K slots of step t (t < 8) are K 64 h + 8 t + [0, 8) for lane half h, the
// same for both operands (the sum over K does not depend on the order, and the block
// scales are applied during the decode): a weight lane's codes for the whole stage are
// 32 contiguous bytes and an activation lane reads one 16-byte piece per step.
// Stage data goes global -> LDS with global_load_lds copies (acts 256 bytes per row,
// 16 pieces, XOR-swizzled by r & 15; codes 64 bytes per row, 4 pieces, swizzled by
// (r >> 2) & 3; scales one or two dwords per row), NBUF stages resident, one barrier
// per stage.
#include "device.h"
#include "internal.h"

namespace fp4 {

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));

struct W16Cfg {
  static constexpr int WAVES = 8, BN = 256, BM = 128, NB = 4;
  static constexpr int ASLOTS = BM * 16;              // 16-byte slots of bf16 activations
  static constexpr int WSLOTS = BN * 4;               // of weight codes
  static constexpr int CODES = 16 * (ASLOTS + WSLOTS);
  static constexpr int NCOP = (ASLOTS + WSLOTS) / 64; // 1 KB copies per stage
  static constexpr int CPW = NCOP / WAVES;
  static constexpr int SCALES = 256 * WAVES;          // one 256-byte scale copy per wave
  static constexpr int STAGE = CODES + SCALES;
  static constexpr int NBUF = 3;
  static constexpr int LDS = NBUF * STAGE;
  static_assert(NCOP % WAVES == 0, "copies spread evenly over the waves");
  static_assert(LDS <= 160 * 1024, "LDS per CU");
};

__device__ __forceinline__ int w16_aslot(int r, int p) { return 16 * r + (p ^ (r & 15)); }
__device__ __forceinline__ int w16_wslot(int r, int p) { return 4 * r + (p ^ ((r >> 2) & 3)); }

#define FP4_W16_LDS(p) ((__attribute__((address_space(3))) void*)(p))
__device__ __forceinline__ void w16_copy16(const void* g, uint8_t* lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)FP4_W16_LDS(lds));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(m0v), "v"(g) : "memory", "m0");
}
__device__ __forceinline__ void w16_copy4(const void* g, uint8_t* lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)FP4_W16_LDS(lds));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :: "s"(m0v), "v"(g) : "memory", "m0");
}
constexpr int w16_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

template <int FMT>
__global__ __launch_bounds__(512, 1) void w4a16_tile_kernel(GemmParams p) {
  using C = W16Cfg;
  constexpr int G = FMT == kNV ? 16 : 32;
  constexpr int SPR = 128 / G;                          // scale bytes per row per stage
  constexpr int OPS = C::CPW + 1;                       // copies per stage per wave
  extern __shared__ __attribute__((aligned(16))) uint8_t wsm[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t ntiles = (p.N + C::BN - 1) / C::BN;
  const int64_t mb = (int64_t)blockIdx.x / ntiles;
  const int64_t nt = (int64_t)blockIdx.x - mb * ntiles;
  // dense, or one 128-row block of one expert (grouped MoE GEMMs: the block table gives
  // the expert and its rows; activation rows may be gathered)
  int grp = 0;
  int64_t row0 = mb * C::BM, row_end = p.M;
  if (p.mblk_expert) {
    grp = p.mblk_expert[mb];
    if (grp < 0) return;  // uniform over the workgroup
    row0 = p.mblk_row0[mb];
    row_end = p.group_end[grp];
  }
  const float alpha = p.alpha_g ? p.alpha_g[grp] : p.alpha;
  const uint8_t* wcodes = p.w_codes + grp * p.w_estride_codes;
  const uint8_t* wscales = p.w_scales + grp * p.w_estride_scales;
  const int64_t K = p.K, nst = K / 128;
  const int64_t KB = K / 2, KS = K / G;
  // the lane's source of each copy of a stage (slot 64 (wave + 8 q) + lane)
  const uint8_t* dsrc[C::CPW];
  int dstep[C::CPW];
#pragma unroll
  for (int q = 0; q < C::CPW; ++q) {
    const int s = 64 * (wave + C::WAVES * q) + lane;
    if (s < C::ASLOTS) {
      const int r = s >> 4, pc = (s & 15) ^ (r & 15);
      const int64_t v = row0 + r < row_end ? row0 + r : row_end - 1;
      const int64_t m = p.a_gather ? (int64_t)p.a_gather[v] : v;
      dsrc[q] = reinterpret_cast<const uint8_t*>(p.a_bf16 + m * p.lda) + 16 * pc;
      dstep[q] = 256;
    } else {
      const int w = s - C::ASLOTS, r = w >> 2, pc = (w & 3) ^ ((r >> 2) & 3);
      const int64_t n = nt * C::BN + r < p.N ? nt * C::BN + r : p.N - 1;
      dsrc[q] = wcodes + n * KB + 16 * pc;
      dstep[q] = 64;
    }
  }
  // scales: dword d of the stage (SPR / 4 per row) comes from row d / (SPR / 4); MXFP4's
  // 256 dwords are copied twice (waves 4-7 into the unused second half)
  const uint8_t* ssrc;
  {
    constexpr int DPR = SPR / 4;
    const int d = (64 * wave + lane) % (C::BN * DPR);
    const int r = d / DPR, j = d % DPR;
    const int64_t n = nt * C::BN + r < p.N ? nt * C::BN + r : p.N - 1;
    ssrc = wscales + n * KS + 4 * j;
  }
  auto issue = [&](int64_t t) {
    uint8_t* buf = wsm + (int)(t % C::NBUF) * C::STAGE;
#pragma unroll
    for (int q = 0; q < C::CPW; ++q) w16_copy16(dsrc[q] + t * dstep[q], buf + (wave + C::WAVES * q) * 1024);
    w16_copy4(ssrc + t * SPR, buf + C::CODES + wave * 256);
  };
  auto sync = [&](int64_t ahead) {
    if (ahead >= 2) __builtin_amdgcn_s_waitcnt(w16_vmcnt(2 * OPS));
    else if (ahead >= 1) __builtin_amdgcn_s_waitcnt(w16_vmcnt(OPS));
    else __builtin_amdgcn_s_waitcnt(w16_vmcnt(0));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  const int r = lane & 31, h = lane >> 5;
  const int wr = wave * 32 + r;                          // the lane's weight row in the tile
  v16f acc[C::NB];
#pragma unroll
  for (int i = 0; i < C::NB; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;

#pragma unroll
  for (int s = 0; s < C::NBUF; ++s)
    if (s < nst) issue(s);
  for (int64_t st = 0; st < nst; ++st) {
    {
      const int64_t last = st + C::NBUF - 1 < nst ? st + C::NBUF - 1 : nst - 1;
      sync(last - st);                                   // stage st landed
    }
    const uint8_t* cur = wsm + (int)(st % C::NBUF) * C::STAGE;
    const uint8_t* wreg = cur + 16 * C::ASLOTS;
    // the lane's codes of the stage (K 64 h .. 64 h + 63 of row wr) and its scales
    const u32x4 c0 = *reinterpret_cast<const u32x4*>(wreg + 16 * w16_wslot(wr, 2 * h));
    const u32x4 c1 = *reinterpret_cast<const u32x4*>(wreg + 16 * w16_wslot(wr, 2 * h + 1));
    uint32_t sw;
    if (FMT == kNV) sw = *reinterpret_cast<const uint32_t*>(cur + C::CODES + wr * 8 + 4 * h);
    else sw = *reinterpret_cast<const uint32_t*>(cur + C::CODES + wr * 4) >> (16 * h);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t code = t < 4 ? dword_of_v(c0, t) : dword_of_v(c1, t - 4);
      bf16x8 wop;
      if (FMT == kNV) wop = decode8_bf16(code, e4m3_value((sw >> (8 * (t >> 1))) & 0xFFu));
      else wop = decode8_bf16_pow2(code, e8m0_value((sw >> (8 * (t >> 2))) & 0xFFu));
#pragma unroll
      for (int i = 0; i < C::NB; ++i) {
        const uint4 a = *reinterpret_cast<const uint4*>(cur + 16 * w16_aslot(32 * i + r, 8 * h + t));
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wop, bits_to_bf16x8(a), acc[i], 0, 0, 0);
      }
    }
    // every wave is done with stage st before its buffer is refilled
    if (st + C::NBUF < nst) {
      __builtin_amdgcn_s_waitcnt(0xC07F);                // lgkmcnt(0): this wave's reads done
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      issue(st + C::NBUF);
    }
  }

  // lane l, register j = weight row 8 (j / 4) + 4 h + j % 4 of the wave's 32, activation
  // row l % 32 of block i
  const bool vec = (p.ldo & 3) == 0 &&
                   (reinterpret_cast<uintptr_t>(p.out) & (p.out_f32 ? 15 : 7)) == 0;
#pragma unroll
  for (int i = 0; i < C::NB; ++i) {
    const int64_t m = row0 + 32 * i + r;
    if (m >= row_end) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t n = nt * C::BN + wave * 32 + 8 * q + 4 * h;
      const float x0 = acc[i][4 * q] * alpha, x1 = acc[i][4 * q + 1] * alpha;
      const float x2 = acc[i][4 * q + 2] * alpha, x3 = acc[i][4 * q + 3] * alpha;
      if (vec && n + 3 < p.N) {
        if (p.out_f32)
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + m * p.ldo + n) =
              make_float4(x0, x1, x2, x3);
        else
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + m * p.ldo + n) =
              make_uint2(bf16_pack2(x0, x1), bf16_pack2(x2, x3));
        continue;
      }
      const float xs[4] = {x0, x1, x2, x3};
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (n + v >= p.N) continue;
        if (p.out_f32)
          reinterpret_cast<float*>(p.out)[m * p.ldo + n + v] = xs[v];
        else
          reinterpret_cast<uint16_t*>(p.out)[m * p.ldo + n + v] = f32_to_bf16_rne(xs[v]);
      }
    }
  }
}

}  // namespace

bool w4a16_tiled_ok(const GemmParams& p) {
  const bool rows_ok = p.mblk_expert ? p.bm == W16Cfg::BM : (p.M > 64 && !p.a_gather);
  return rows_ok && p.K % 128 == 0 && (p.lda % 8) == 0;
}

hipError_t launch_gemm_w4a16_tiled(int fmt, const GemmParams& p, hipStream_t s, const char** name) {
  using C = W16Cfg;
  const int64_t mblocks = p.mblk_expert ? p.n_mblocks : (p.M + C::BM - 1) / C::BM;
  const int64_t grid = ((p.N + C::BN - 1) / C::BN) * mblocks;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF || !w4a16_tiled_ok(p)) return hipErrorInvalidConfiguration;
  static std::atomic<uint64_t> lds_nv{0}, lds_mx{0};
  if (fmt == kNV) {
    *name = "w4a16_tile_nvfp4";
    hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&w4a16_tile_kernel<kNV>), C::LDS, lds_nv);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((w4a16_tile_kernel<kNV>), dim3((unsigned)grid), dim3(512), C::LDS, s, p);
  } else {
    *name = "w4a16_tile_mxfp4";
    hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&w4a16_tile_kernel<kMX>), C::LDS, lds_mx);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((w4a16_tile_kernel<kMX>), dim3((unsigned)grid), dim3(512), C::LDS, s, p);
  }
  return hipGetLastError();
}

}  // namespace fp4
