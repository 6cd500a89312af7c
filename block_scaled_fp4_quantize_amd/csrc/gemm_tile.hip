// Tiled block-scaled FP4 GEMM for many activation rows (prefill, and MoE experts
// with many routed rows), fp4 activations, K a multiple of 128.
//
// Definition as in gemm.hip: out[m, n] = alpha * sum_k a_hat[m, k] * w_hat[n, k]
// ("vLLM per-format kernel capability matrix derived from source", THE EMULATION
// COLUMN), with MXFP4 on gfx950's scaled FP4 MFMA and NVFP4 decoded exactly to
// fp16 for fp16 MFMA ("vLLM on the NVIDIA DGX Spark (GB10 / sm_121): A Complete
// Technical Guide", §6.1 and §6.4 for the two block-scale formats).
//
// Tiling: a workgroup (4 waves, 2 x 2) owns 256 weight rows and BM activation rows
// (BM = 128: MXFP4 runs two such workgroups per CU; a 256-row MXFP4 variant is
// kept for callers that ask for it).
// Each wave computes a 128 x BM/2 tile with 16x16 MFMAs (weights as the A operand,
// so a lane ends up holding 4 consecutive output columns).  K advances in stages
// of 128: the packed codes (64 bytes per row) and block scales of the BM + 256
// rows are staged in LDS, double-buffered, with the next stage's global loads in
// flight while the current one is multiplied.  Codes travel at 4.5 bits per
// element all the way into registers; NVFP4 is decoded to fp16 right before the
// MFMA (unit-scale convert, then one packed fp16 multiply by the e4m3 scale --
// exact), MXFP4 needs no decode at all.
#include "device.h"
#include "internal.h"

namespace fp4 {

namespace {

constexpr int kTBK = 128;        // K per stage
constexpr int kTBN = 256;        // weight rows per workgroup
constexpr int kTCS = 80;         // LDS row stride of staged codes: 64 bytes + 16 pad

template <int FMT, int BM>
struct TileCfg {
  static constexpr int G = FMT == kNV ? 16 : 32;
  static constexpr int SB = kTBK / G;          // scale bytes per row per stage (8 / 4)
  static constexpr int MI = BM / 32;           // 16-row activation tiles per wave
  static constexpr int NJ = 8;                 // 16-row weight tiles per wave
  static constexpr int ROWS = BM + kTBN;       // staged rows: activations, then weights
  static constexpr int CODE_BYTES = ROWS * kTCS;
  static constexpr int STAGE = CODE_BYTES + ROWS * SB;
  static constexpr int CP = ROWS * 4 / 256;    // 16-byte code pieces per thread per stage
  static constexpr int SPT = ROWS * SB / 4;    // 4-byte scale pieces per stage
  static constexpr int SP = (SPT + 255) / 256; // scale pieces per thread (last one guarded)
};

// Global -> register half of staging one K stage: this thread's code pieces (16
// bytes of one row) and scale pieces (4 bytes), at stage st.
template <class C>
__device__ __forceinline__ void stage_load(u32x4 (&creg)[C::CP], uint32_t (&sreg)[C::SP],
                                           const uint8_t* const (&cptr)[C::CP],
                                           const uint8_t* const (&sptr)[C::SP], int64_t st) {
  const int64_t kb = st * (kTBK / 2);
#pragma unroll
  for (int i = 0; i < C::CP; ++i) creg[i] = *reinterpret_cast<const u32x4*>(cptr[i] + kb);
  const int64_t ks = st * C::SB;
#pragma unroll
  for (int i = 0; i < C::SP; ++i) sreg[i] = *reinterpret_cast<const uint32_t*>(sptr[i] + ks);
}

// Register -> LDS half: code piece i of thread t is row t/4 + 64 i, bytes 16 (t%4)..;
// scale piece t + 256 i is the 4-byte word at that index of the stage's scale area.
template <class C>
__device__ __forceinline__ void stage_store(uint8_t* base, const u32x4 (&creg)[C::CP],
                                            const uint32_t (&sreg)[C::SP], int tid) {
#pragma unroll
  for (int i = 0; i < C::CP; ++i)
    *reinterpret_cast<u32x4*>(base + ((tid >> 2) + 64 * i) * kTCS + (tid & 3) * 16) = creg[i];
#pragma unroll
  for (int i = 0; i < C::SP; ++i)
    if (tid + 256 * i < C::SPT)
      *reinterpret_cast<uint32_t*>(base + C::CODE_BYTES + (tid + 256 * i) * 4) = sreg[i];
}

// MXFP4 128-row tiles fit in 256 registers, so two workgroups share a CU and one
// computes while the other waits for its next stage (NVFP4 would spill).
// FUSE: the gate/up GEMM of an MoE expert with SwiGLU + requant in the epilogue.  The
// workgroup's 256 weight rows are then 128 gate rows and the matching 128 up rows of
// h columns [128 nt, 128 nt + 128): wave column wn takes h columns 64 wn + [0, 64),
// its weight tiles 0-3 being the gate rows and 4-7 the up rows of the same columns,
// so a lane holds gate and up of the same (m, h column) in registers.
template <int FMT, int BM, bool FUSE>
__global__ __launch_bounds__(256, (FMT == kMX && BM == 128) ? 2 : 1) void tile_gemm(GemmParams p) {
  using C = TileCfg<FMT, BM>;
  extern __shared__ __attribute__((aligned(16))) uint8_t tsm[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int wm = wave & 1;
  const int wn = wave >> 1;
  const int64_t ntiles = (p.N + kTBN - 1) / kTBN;
  const int64_t mb = (int64_t)blockIdx.x / ntiles;
  const int64_t nt = (int64_t)blockIdx.x - mb * ntiles;
  int grp = 0;
  int64_t row0, row_end;
  if (p.mblk_expert) {
    grp = p.mblk_expert[mb];
    if (grp < 0) return;  // uniform over the workgroup
    row0 = p.mblk_row0[mb];
    row_end = p.group_end[grp];
  } else {
    row0 = mb * BM;
    row_end = p.M;
  }
  const int64_t K = p.K;
  const int64_t KB = K >> 1;
  const int64_t KS = K / C::G;
  const uint8_t* wcodes = p.w_codes + grp * p.w_estride_codes;
  const uint8_t* wscales = p.w_scales + grp * p.w_estride_scales;

  // global source rows of this thread's staging pieces (fixed for all stages);
  // rows past the end are clamped to the last valid one (outputs not stored)
  auto src_row = [&](int rr) -> int64_t {
    if (rr < BM) {
      int64_t pv = row0 + rr;
      if (pv >= row_end) pv = row_end - 1;
      return p.a_gather ? (int64_t)p.a_gather[pv] : pv;
    }
    int64_t n;
    if (FUSE) {
      const int w = rr - BM, within = w & 127;
      const int64_t col = nt * 128 + (w >> 7) * 64 + (within & 63);
      n = within < 64 ? col : p.I + col;
    } else {
      n = nt * kTBN + (rr - BM);
    }
    return n < p.N ? n : p.N - 1;
  };
  const int cseg = tid & 3;
  const uint8_t* cptr[C::CP];
#pragma unroll
  for (int i = 0; i < C::CP; ++i) {
    const int rr = (tid >> 2) + 64 * i;
    cptr[i] = (rr < BM ? p.a_codes : wcodes) + src_row(rr) * KB + cseg * 16;
  }
  const uint8_t* sptr[C::SP];
#pragma unroll
  for (int i = 0; i < C::SP; ++i) {
    int pc = tid + 256 * i;
    if (pc >= C::SPT) pc = C::SPT - 1;
    const int rr = pc / (C::SB / 4);
    sptr[i] = (rr < BM ? p.a_scales : wscales) + src_row(rr) * KS + (pc - rr * (C::SB / 4)) * 4;
  }

  v4f acc[C::NJ][C::MI];
#pragma unroll
  for (int j = 0; j < C::NJ; ++j)
#pragma unroll
    for (int i = 0; i < C::MI; ++i) acc[j][i] = v4f{0.f, 0.f, 0.f, 0.f};

  const int r = lane & 15;
  const int gq = lane >> 4;
  const int64_t nstages = K / kTBK;
  uint8_t* buf0 = tsm;
  uint8_t* buf1 = tsm + C::STAGE;

  {
    u32x4 creg[C::CP];
    uint32_t sreg[C::SP];
    stage_load<C>(creg, sreg, cptr, sptr, 0);
    stage_store<C>(buf0, creg, sreg, tid);
  }
  __syncthreads();
  for (int64_t st = 0; st < nstages; ++st) {
    uint8_t* cur = (st & 1) ? buf1 : buf0;
    uint8_t* nxt = (st & 1) ? buf0 : buf1;
    u32x4 creg[C::CP];
    uint32_t sreg[C::SP];
    // clamped prefetch of the next stage (the last iteration reloads its own stage)
    stage_load<C>(creg, sreg, cptr, sptr, st + 1 < nstages ? st + 1 : st);
    __builtin_amdgcn_sched_barrier(0);

    // fragments of this stage: weights (A operand) and activations (B operand)
    uint4 wf[C::NJ];
    uint32_t wsb[C::NJ];
    uint4 af[C::MI];
    uint32_t asb[C::MI];
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) {
      const int rr = BM + wn * 128 + 16 * j + r;
      wf[j] = *reinterpret_cast<const uint4*>(cur + rr * kTCS + gq * 16);
      if (FMT == kMX)
        wsb[j] = cur[C::CODE_BYTES + rr * C::SB + gq];
      else
        wsb[j] = *reinterpret_cast<const uint16_t*>(cur + C::CODE_BYTES + rr * C::SB + gq * 2);
    }
#pragma unroll
    for (int i = 0; i < C::MI; ++i) {
      const int rr = wm * (BM / 2) + 16 * i + r;
      af[i] = *reinterpret_cast<const uint4*>(cur + rr * kTCS + gq * 16);
      if (FMT == kMX)
        asb[i] = cur[C::CODE_BYTES + rr * C::SB + gq];
      else
        asb[i] = *reinterpret_cast<const uint16_t*>(cur + C::CODE_BYTES + rr * C::SB + gq * 2);
    }

    if (FMT == kMX) {
#pragma unroll
      for (int j = 0; j < C::NJ; ++j) {
        const v8i wop = {(int)wf[j].x, (int)wf[j].y, (int)wf[j].z, (int)wf[j].w, 0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < C::MI; ++i) {
          const v8i aop = {(int)af[i].x, (int)af[i].y, (int)af[i].z, (int)af[i].w, 0, 0, 0, 0};
          acc[j][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              wop, aop, acc[j][i], 4, 4, 0, (int)wsb[j], 0, (int)asb[i]);
        }
      }
    } else {
      // lane group gq holds elements [32 gq, 32 gq + 32) of the stage; k-step s uses
      // its dword s (block 2 gq + s/2), the same k slots for both operands
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        f16x8 aop[C::MI];
#pragma unroll
        for (int i = 0; i < C::MI; ++i)
          aop[i] = decode8_f16(dword_of(af[i], s),
                               f16_pair(e4m3_value_pos((asb[i] >> (8 * (s >> 1))) & 0xFFu)));
#pragma unroll
        for (int j = 0; j < C::NJ; ++j) {
          const f16x8 wop = decode8_f16(dword_of(wf[j], s),
                                        f16_pair(e4m3_value_pos((wsb[j] >> (8 * (s >> 1))) & 0xFFu)));
#pragma unroll
          for (int i = 0; i < C::MI; ++i)
            acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wop, aop[i], acc[j][i], 0, 0, 0);
        }
      }
    }

    stage_store<C>(nxt, creg, sreg, tid);   // (waits only for the staging loads issued above)
    __syncthreads();
  }

  const float alpha = p.alpha_g ? p.alpha_g[grp] : p.alpha;
  if (FUSE) {
    // h = SiLU(alpha g) * (alpha u) for this lane's 4 consecutive h columns of each
    // gate tile j; a quantization block (16 or 32 columns of one row) spans the lanes
    // r, r + 16, r + 32, r + 48 (and, for MXFP4, gate tiles j and j + 1), so its amax is
    // two lane exchanges away.  Every lane takes part in the exchanges; only rows
    // that exist are stored.
    const float g = p.h_grp_g ? p.h_grp_g[grp] : p.h_g;
    const int64_t hrow = p.I / 2;
#pragma unroll
    for (int i = 0; i < C::MI; ++i) {
      const int64_t m = row0 + wm * (BM / 2) + 16 * i + r;
      const bool store = m < row_end;
      float h[4][4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) h[j][v] = swiglu1(acc[j][i][v] * alpha, acc[j + 4][i][v] * alpha);
      const int64_t hc0 = nt * 128 + wn * 64 + 4 * gq;   // + 16 j: this lane's first column
      if (FMT == kNV) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float amax = fmaxf(fmaxf(fabsf(h[j][0]), fabsf(h[j][1])), fmaxf(fabsf(h[j][2]), fabsf(h[j][3])));
          amax = fmaxf(amax, __shfl_xor(amax, 16));
          amax = fmaxf(amax, __shfl_xor(amax, 32));
          float rs;
          const uint32_t sc = q_nv_scale(amax, g, &rs);
          uint32_t q = 0;
#pragma unroll
          for (int v = 0; v < 4; ++v) q |= q_nv_code(h[j][v], rs) << (4 * v);
          if (store) {
            const int64_t hc = hc0 + 16 * j;
            *reinterpret_cast<uint16_t*>(p.h_codes + m * hrow + hc / 2) = (uint16_t)q;
            if (gq == 0) p.h_scales[m * (p.I / 16) + hc / 16] = (uint8_t)sc;
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; j += 2) {
          float amax = 0.0f;
#pragma unroll
          for (int v = 0; v < 4; ++v) amax = fmaxf(amax, fmaxf(fabsf(h[j][v]), fabsf(h[j + 1][v])));
          amax = fmaxf(amax, __shfl_xor(amax, 16));
          amax = fmaxf(amax, __shfl_xor(amax, 32));
          int E;
          const uint32_t sc = q_mx_scale(amax, &E);
          uint32_t q0 = 0, q1 = 0;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            q0 |= q_mx_code(h[j][v], E) << (4 * v);
            q1 |= q_mx_code(h[j + 1][v], E) << (4 * v);
          }
          if (store) {
            const int64_t hc = hc0 + 16 * j;
            *reinterpret_cast<uint16_t*>(p.h_codes + m * hrow + hc / 2) = (uint16_t)q0;
            *reinterpret_cast<uint16_t*>(p.h_codes + m * hrow + (hc + 16) / 2) = (uint16_t)q1;
            if (gq == 0) p.h_scales[m * (p.I / 32) + hc / 32] = (uint8_t)sc;
          }
        }
      }
    }
    return;
  }

  // epilogue: lane holds out[m][n .. n+3], m = rows of activation tile i,
  // n = 4 consecutive columns of weight tile j
  const bool vec = (p.ldo & 3) == 0 && ((reinterpret_cast<uintptr_t>(p.out) & 15) == 0);
#pragma unroll
  for (int i = 0; i < C::MI; ++i) {
    const int64_t m = row0 + wm * (BM / 2) + 16 * i + r;
    if (m >= row_end) continue;
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) {
      const int64_t n = nt * kTBN + wn * 128 + 16 * j + 4 * gq;
      if (n >= p.N) continue;
      const float x0 = acc[j][i][0] * alpha, x1 = acc[j][i][1] * alpha;
      const float x2 = acc[j][i][2] * alpha, x3 = acc[j][i][3] * alpha;
      if (p.out_f32) {
        float* o = reinterpret_cast<float*>(p.out) + m * p.ldo + n;
        if (vec && n + 3 < p.N) {
          *reinterpret_cast<float4*>(o) = make_float4(x0, x1, x2, x3);
        } else {
          o[0] = x0;
          if (n + 1 < p.N) o[1] = x1;
          if (n + 2 < p.N) o[2] = x2;
          if (n + 3 < p.N) o[3] = x3;
        }
      } else {
        uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + m * p.ldo + n;
        const uint16_t b0 = f32_to_bf16_rne(x0), b1 = f32_to_bf16_rne(x1);
        const uint16_t b2 = f32_to_bf16_rne(x2), b3 = f32_to_bf16_rne(x3);
        if (vec && n + 3 < p.N) {
          *reinterpret_cast<uint2*>(o) = make_uint2((uint32_t)b0 | ((uint32_t)b1 << 16),
                                                    (uint32_t)b2 | ((uint32_t)b3 << 16));
        } else {
          o[0] = b0;
          if (n + 1 < p.N) o[1] = b1;
          if (n + 2 < p.N) o[2] = b2;
          if (n + 3 < p.N) o[3] = b3;
        }
      }
    }
  }
}

template <int FMT, int BM, bool FUSE>
hipError_t launch_tile(const GemmParams& p, hipStream_t s, const char** name) {
  using C = TileCfg<FMT, BM>;
  const int64_t ntiles = (p.N + kTBN - 1) / kTBN;
  const int64_t mblocks = p.mblk_expert ? p.n_mblocks : (p.M + BM - 1) / BM;
  const int64_t grid = ntiles * mblocks;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  static const char* names[2][2] = {{"tile_nvfp4_m128", "tile_nvfp4_m256"},
                                    {"tile_mxfp4_m128", "tile_mxfp4_m256"}};
  *name = FUSE ? (FMT == kNV ? "tile_nvfp4_m128_swiglu" : "tile_mxfp4_m128_swiglu")
               : names[FMT][BM == 256 ? 1 : 0];
  if (p.K % kTBK != 0 || p.K <= 0) return hipErrorInvalidValue;
  if (FUSE && (p.I <= 0 || p.I % 128 != 0 || p.N != 2 * p.I || !p.h_codes || !p.h_scales))
    return hipErrorInvalidValue;
  const size_t lds = 2 * (size_t)C::STAGE;
  static bool attr_set = false;  // once per instantiation (idempotent, so races are harmless)
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&tile_gemm<FMT, BM, FUSE>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((tile_gemm<FMT, BM, FUSE>), dim3((unsigned)grid), dim3(256), lds, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_tiled(int fmt, int bm, const GemmParams& p, hipStream_t s,
                             const char** name) {
  // NVFP4 runs on fp16 MFMAs (four per 128-deep stage where MXFP4 needs one), so
  // 128-row tiles already give it enough MFMA work per staged byte; 256-row NVFP4
  // tiles would also exceed the register file.
  if (p.fuse_swiglu)
    return fmt == kNV ? launch_tile<kNV, 128, true>(p, s, name) : launch_tile<kMX, 128, true>(p, s, name);
  if (fmt == kNV || bm != 256) return fmt == kNV ? launch_tile<kNV, 128, false>(p, s, name)
                                                 : launch_tile<kMX, 128, false>(p, s, name);
  return launch_tile<kMX, 256, false>(p, s, name);
}

}  // namespace fp4
