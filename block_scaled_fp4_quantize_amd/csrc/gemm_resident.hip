// Decode-shaped block-scaled FP4 GEMM: few activation rows (one 16-row tile per
// workgroup), fp4 activations, K a multiple of 128.  The weights are read exactly
// once, so the kernel is bound by HBM bandwidth and its job is to keep as many
// weight bytes in flight as the register file allows.
//
// Definition as in gemm.hip: out[m, n] = alpha * sum_k a_hat[m, k] * w_hat[n, k]
// ("vLLM per-format kernel capability matrix derived from source", THE EMULATION
// COLUMN); MXFP4 on the scaled FP4 MFMA, NVFP4 decoded exactly to fp16 ("vLLM on
// the NVIDIA DGX Spark (GB10 / sm_121): A Complete Technical Guide", §6.1, §6.4).
//
// A workgroup owns 16 * 4 / KSPLIT weight rows and 16*MT activation rows: its 4 waves
// form 4 / KSPLIT row groups of 16 weight rows, each split over KSPLIT contiguous
// ranges of K (one wave per range); the partial tiles are added through LDS in wave
// order (bitwise reproducible).  Splitting K gives decode-sized N enough workgroups to
// occupy every CU: N = 14336 is 224 workgroups at 64 rows, 448 at 32.
//  * Activation codes, activation scales and the workgroup's weight scales for the
//    whole K are copied into LDS once, by LDS-direct 16-byte loads (no registers).
//  * Each wave keeps a ring of RING K-steps (128 elements, 16 bytes per lane) of
//    its weight codes in flight in registers.  All of the ring is issued before the
//    first barrier; each step is refilled with the step RING ahead as soon as it
//    has been multiplied, so a lane has up to RING loads outstanding throughout.
//  * The one barrier waits only for the LDS copies (issued first); the weight
//    loads behind them stay in flight.
//
// LDS layout (bytes):
//   act codes   [16*MT rows][ASTR]        row-major, ASTR = K/2 rounded up to 1 KB,
//                                          plus 16: a copy is 1 KB of one row (a
//                                          partial last copy spills only into the
//                                          row's own padding), and the 16-byte pad
//                                          puts the 16 rows of an MFMA operand read
//                                          on distinct banks.  Only rows that exist
//                                          are copied: padded rows of a partial
//                                          tile feed output columns never stored.
//   act scales  [K/G/16][16*MT rows][16]  16-byte groups of a row's scales, group-
//   w scales    [K/G/16][RROWS][16]       major: a 16-byte global piece lands whole,
//                                          and one step's scale reads across 16
//                                          rows are 16 bytes apart (distinct banks)
// The two scale sections are padded to whole 1 KB copies: the lanes of a last,
// partial copy write into the padding (copies of different waves are unordered).
//   partials    [KSPLIT-1][4/KSPLIT][MT][64 lanes][16]  the K-split partial tiles
#include "device.h"
#include "internal.h"

namespace fp4 {

namespace {

#define FP4_LDS(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int kRStep = 128;   // K per step (one scaled MFMA, or four fp16 MFMAs)
constexpr int kResPieces = 16;  // max 16-byte activation pieces staged per thread

template <int FMT, int MT, int KSPLIT = 1>
struct ResCfg {
  static constexpr int G = FMT == kNV ? 16 : 32;
  static constexpr int AROWS = 16 * MT;
  static constexpr int RG = 4 / KSPLIT;      // 16-row weight groups per workgroup
  static constexpr int RROWS = 16 * RG;      // weight rows per workgroup
  // activation rows staged in LDS: the four-way split serves at most 4 rows, which
  // keeps its LDS small enough for all of its workgroups to be resident at once
  static constexpr int ALDS = KSPLIT == 4 ? 4 : AROWS;
  static_assert(KSPLIT == 1 || KSPLIT == 2 || KSPLIT == 4, "4 waves split K evenly");
};

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima)
__host__ __device__ constexpr int64_t round_kb(int64_t b) { return (b + 1023) / 1024 * 1024; }

constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// One 16-byte LDS-direct copy per lane: lane l writes lds_base + 16 l (M0 holds the
// wave-uniform LDS base; one wait state separates the M0 write from its use).
// Written as inline asm so that the compiler's wait-count insertion does not treat
// every later LDS read as dependent on it (it would drain the whole weight ring
// with vmcnt(0)).  Correctness: every copy is issued before the weight ring, so
// waiting for any ring load also waits for all copies, and the explicit vmcnt wait
// before the barrier covers the LDS reads that follow it.
__device__ __forceinline__ void lds_copy16(const void* g, uint8_t* lds_base) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)FP4_LDS(lds_base));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(m0v), "v"(g) : "memory", "m0");
}

// LDS operands of one step: activation codes and scales of the MT tiles, and the
// weight scale(s) of the lane's row.  Fetched one step ahead of their MFMAs.
template <int MT>
struct StepOps {
  u32x4 aq[MT];
  uint32_t asb[MT];
  uint32_t wsb;
};

// padded LDS row stride of the activation codes
__host__ __device__ constexpr int64_t res_astr(int64_t K) { return round_kb(K / 2) + 16; }

template <int FMT, int MT, int RROWS, int ALDS>
__device__ __forceinline__ StepOps<MT> res_fetch(const uint8_t* __restrict__ a_lds,
                                                 const uint8_t* __restrict__ as_lds,
                                                 const uint8_t* __restrict__ ws_lds, int KS,
                                                 int astr, int64_t jc, int wrow, int r,
                                                 int gq) {
  using C = ResCfg<FMT, MT>;
  StepOps<MT> o;
  // scale byte b of a row sits in group b / 16 at byte b % 16; the step's bytes are
  // 4 jc + gq (MXFP4, block of the lane's 32 elements) or 8 jc + 2 gq, + 1 (NVFP4)
  const int sb = FMT == kMX ? 4 * (int)jc + gq : 8 * (int)jc + 2 * gq;
  const int sgrp = sb >> 4, sbyte = sb & 15;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    // operand rows past the staged ones re-read the last (outputs never stored)
    const int ar = 16 * t + r < ALDS ? 16 * t + r : ALDS - 1;
    o.aq[t] = *reinterpret_cast<const u32x4*>(a_lds + ar * astr + jc * 64 + gq * 16);
    const uint8_t* ap = as_lds + (sgrp * ALDS + ar) * 16 + sbyte;
    o.asb[t] = FMT == kMX ? (uint32_t)*ap : (uint32_t)*reinterpret_cast<const uint16_t*>(ap);
  }
  const uint8_t* wp = ws_lds + (sgrp * RROWS + wrow) * 16 + sbyte;
  o.wsb = FMT == kMX ? (uint32_t)*wp : (uint32_t)*reinterpret_cast<const uint16_t*>(wp);
  return o;
}

// Accumulators: kNAcc independent chains per tile (an MFMA waits for the previous
// one on its accumulator, so a single chain would serialize on MFMA latency).
// MXFP4 steps rotate over the chains; NVFP4 sub-steps take one chain each.
constexpr int kNAcc = 4;

template <int FMT, int MT>
__device__ __forceinline__ void res_mma(const StepOps<MT>& o, uint32_t keep, u32x4 wq,
                                        v4f (&acc)[MT][kNAcc], int chain) {
  const u32x4 w = wq & keep;
  if (FMT == kMX) {
    const v8i wop = {(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const v8i aop = {(int)o.aq[t].x, (int)o.aq[t].y, (int)o.aq[t].z, (int)o.aq[t].w,
                       0, 0, 0, 0};
      acc[t][chain] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          wop, aop, acc[t][chain], 4, 4, 0, (int)o.wsb, 0, (int)o.asb[t]);
    }
  } else {
    const f16x2 wsp = e4m3_pair_f16(o.wsb);
    const f16x2 ws_lo = f16_bcast(wsp, 0);
    const f16x2 ws_hi = f16_bcast(wsp, 1);
    f16x2 asp[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) asp[t] = e4m3_pair_f16(o.asb[t]);
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      const f16x8 wop = decode8_f16(w[sub], sub < 2 ? ws_lo : ws_hi);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const f16x8 aop = decode8_f16(o.aq[t][sub], f16_bcast(asp[t], sub >> 1));
        acc[t][sub] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wop, aop, acc[t][sub], 0, 0, 0);
      }
    }
  }
}

// A four-way split has four times the workgroups of the unsplit kernel (896 for
// N = 14336); asking for four workgroups per CU (at most 128 registers) keeps them all
// resident at once instead of leaving a second, partial round.
template <int FMT, int MT, int RING, int KSPLIT>
__global__ __launch_bounds__(256, KSPLIT == 4 ? 4 : 1) void resident_gemm(GemmParams p) {
  using C = ResCfg<FMT, MT, KSPLIT>;
  extern __shared__ __attribute__((aligned(16))) uint8_t res_smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int64_t ntiles = (p.N + C::RROWS - 1) / C::RROWS;
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
    row0 = mb * C::AROWS;
    row_end = p.M;
  }
  // per-group scalars fetched up front, not after the main loop
  const float alpha = p.alpha_g ? p.alpha_g[grp] : p.alpha;
  const int64_t K = p.K;
  const int64_t KB = K >> 1;
  const int KS = (int)(K / C::G);
  const int64_t NS = K / kRStep;
  const int astr = (int)res_astr(K);
  uint8_t* a_lds = res_smem;                                            // ALDS * astr
  uint8_t* as_lds = a_lds + (size_t)C::ALDS * astr;                     // ALDS * KS
  uint8_t* ws_lds = as_lds + round_kb((int64_t)C::ALDS * KS);           // RROWS * KS
  uint8_t* red_lds = ws_lds + round_kb((int64_t)C::RROWS * KS);         // partial tiles
  const uint8_t* wcodes = p.w_codes + grp * p.w_estride_codes;
  const uint8_t* wscales = p.w_scales + grp * p.w_estride_scales;

  // ---- LDS-direct copies (issued first, so the one wait below leaves the weight
  // loads issued after them in flight) ----
  // act codes: 16-byte piece P = 64 c + lane of copy c sits at LDS byte 16 P, i.e.
  // step P / (4 AROWS), row (P / 4) % AROWS, bytes 16 (P % 4) of the step
  // source row of activation row rr (padded rows repeat the last valid row): lane
  // rr looks it up once, the others read it with a lane shuffle
  int src_mine;
  {
    int64_t pv = row0 + (lane < C::AROWS ? lane : C::AROWS - 1);
    if (pv >= row_end) pv = row_end - 1;
    src_mine = p.a_gather ? p.a_gather[pv] : (int)pv;
  }
  // resolved here, while nothing else is outstanding: later shuffles of it must not
  // wait on the loads issued after this point
  asm volatile("" : "+v"(src_mine));
  auto act_src = [&](int rr) -> int64_t { return (int64_t)__shfl(src_mine, rr, 64); };
  // act codes through registers (issued first; stored to LDS after the ring loads
  // are in flight): the rows_valid * K/32 16-byte pieces of the existing rows,
  // piece u * 256 + tid of this thread, rotated by the workgroup index (every
  // workgroup reads the same rows).  nper is uniform over the workgroup.
  const uint32_t rows_valid = (uint32_t)(row_end - row0 < C::ALDS ? row_end - row0 : C::ALDS);
  const uint32_t ppr = (uint32_t)(KB / 16);       // pieces per row
  const uint32_t apieces = rows_valid * ppr;      // <= 256 * kResPieces (resident_fits)
  const int nper = (int)((apieces + 255) / 256);
  const uint32_t arot = ((uint32_t)blockIdx.x * 64u) % apieces;
  // piece u of this thread is (u * 256 + tid + arot) mod apieces, walked as a
  // (row, column) pair: one division up front, then steps of 256 pieces
  const uint32_t step_r = 256u / ppr, step_c = 256u - step_r * ppr;
  // (steps happen only when apieces > 256, where step_r < rows_valid and one wrap
  // suffices; surplus threads of smaller tiles start at a valid piece too)
  const uint32_t pc0 = ((uint32_t)tid + arot) % apieces;
  const uint32_t arow0 = pc0 / ppr, acol0 = pc0 - arow0 * ppr;
  u32x4 areg[kResPieces];
  {
    uint32_t rr = arow0, cc = acol0;
#pragma unroll
    for (int u = 0; u < kResPieces; ++u) {
      if (u < nper) {
        // a piece past the end (u * 256 + tid >= apieces) is re-read, not stored
        areg[u] = *reinterpret_cast<const u32x4*>(p.a_codes + act_src((int)rr) * KB +
                                                  (int64_t)cc * 16);
        cc += step_c;
        rr += step_r;
        if (cc >= ppr) { cc -= ppr; ++rr; }
        if (rr >= rows_valid) rr -= rows_valid;
      }
    }
  }
  // act scales and weight scales: 16-byte piece P = 64 c + lane of copy c is group
  // P / rows, row P % rows (KS % 16 == 0, so a row has KS / 16 whole groups)
  {
    const int64_t apieces = (int64_t)C::ALDS * (KS / 16);
    for (int64_t c = wave; c * 64 < apieces; c += 4) {
      int64_t pc = c * 64 + lane;
      if (pc >= apieces) pc = apieces - 1;       // surplus lanes re-copy the last piece
      const int rr = (int)(pc % C::ALDS);
      const int64_t g = pc / C::ALDS;
      lds_copy16(p.a_scales + act_src(rr) * KS + g * 16, as_lds + c * 1024);
    }
    const int64_t wpieces = (int64_t)C::RROWS * (KS / 16);
    for (int64_t c = wave; c * 64 < wpieces; c += 4) {
      int64_t pc = c * 64 + lane;
      if (pc >= wpieces) pc = wpieces - 1;
      const int rr = (int)(pc % C::RROWS);
      const int64_t g = pc / C::RROWS;
      int64_t n = nt * C::RROWS + rr;
      if (n >= p.N) n = p.N - 1;
      lds_copy16(wscales + n * KS + g * 16, ws_lds + c * 1024);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- the weight ring: steps s0 .. s0+RING-1 of this wave's K range [s0, s1)
  // (steps past the end are clamped re-reads, multiplied by zero) ----
  const int r = lane & 15;
  const int gq = lane >> 4;
  const int rg = wave % C::RG;          // row group
  const int kh = wave / C::RG;          // K range
  const int64_t s0 = KSPLIT == 1 ? 0 : kh * NS / KSPLIT;                // NS >= KSPLIT
  const int64_t s1 = KSPLIT == 1 ? NS : (kh + 1) * NS / KSPLIT;
  const int wrow = rg * 16 + r;
  const int64_t wn_raw = nt * C::RROWS + wrow;
  const int64_t wn = wn_raw < p.N ? wn_raw : p.N - 1;   // padded rows: outputs not stored
  // row-major codes (64 bytes per step), or the prepared layout of 16-row x 128-element
  // blocks in lane order (1 KB per step, contiguous over the wave)
  const uint8_t* wsrc = p.w_tiled ? wcodes + (((wn >> 4) * NS) * 64 + (wn & 15) + 16 * gq) * 16
                                  : wcodes + wn * KB + gq * 16;
  const int64_t wstep = p.w_tiled ? 1024 : 64;
  u32x4 wq[RING];
#pragma unroll
  for (int i = 0; i < RING; ++i)
    wq[i] = *reinterpret_cast<const u32x4*>(wsrc + (s0 + i < s1 ? s0 + i : s1 - 1) * wstep);
  __builtin_amdgcn_sched_barrier(0);
  // every activation load and LDS-direct copy of this wave has landed once at most
  // RING loads remain
  __builtin_amdgcn_s_waitcnt(vmcnt_only(RING));
  {
    uint32_t rr = arow0, cc = acol0;
#pragma unroll
    for (int u = 0; u < kResPieces; ++u) {
      if (u < nper) {
        if ((uint32_t)u * 256u + (uint32_t)tid < apieces)
          *reinterpret_cast<u32x4*>(a_lds + rr * astr + cc * 16) = areg[u];
        cc += step_c;
        rr += step_r;
        if (cc >= ppr) { cc -= ppr; ++rr; }
        if (rr >= rows_valid) rr -= rows_valid;
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the LDS stores are done
  asm volatile("" ::: "memory");   // no LDS access moves across the barrier
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  v4f acc[MT][kNAcc];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int c = 0; c < kNAcc; ++c) acc[t][c] = v4f{0.f, 0.f, 0.f, 0.f};

  // The LDS operands of step j + 1 are fetched before the MFMAs of step j, and a
  // scheduling barrier closes every step: the lookahead stays at one step, which
  // keeps the ring, the operands and the accumulators in ordinary registers.
  int64_t base = s0;
  StepOps<MT> cur = res_fetch<FMT, MT, C::RROWS, C::ALDS>(a_lds, as_lds, ws_lds, KS, astr, s0, wrow, r, gq);
  // full ring passes that refill: step base + i, then load step base + i + RING
  for (; base + RING < s1; base += RING) {
#pragma unroll
    for (int i = 0; i < RING; ++i) {
      const int64_t j = base + i;
      const StepOps<MT> nxt =
          res_fetch<FMT, MT, C::RROWS, C::ALDS>(a_lds, as_lds, ws_lds, KS, astr, j + 1, wrow, r, gq);
      res_mma<FMT, MT>(cur, 0xFFFFFFFFu, wq[i], acc, i % kNAcc);
      const int64_t jn = j + RING < s1 ? j + RING : s1 - 1;
      wq[i] = *reinterpret_cast<const u32x4*>(wsrc + jn * wstep);
      cur = nxt;
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // last pass: no refills; steps at or past s1 contribute zero (operands of the
  // clamped last step)
#pragma unroll
  for (int i = 0; i < RING; ++i) {
    const int64_t j = base + i;
    const int64_t jn = j + 1 < s1 ? j + 1 : s1 - 1;
    const StepOps<MT> nxt =
        res_fetch<FMT, MT, C::RROWS, C::ALDS>(a_lds, as_lds, ws_lds, KS, astr, jn, wrow, r, gq);
    res_mma<FMT, MT>(cur, j < s1 ? 0xFFFFFFFFu : 0u, wq[i], acc, i % kNAcc);
    cur = nxt;
    __builtin_amdgcn_sched_barrier(0);
  }

  // The accumulators pass through an opaque asm statement before the stores.  The
  // last pass is straight-line code that only feeds the stores below, and without
  // this the compiler sinks it into the store branch (m < row_end): the MFMAs
  // would then run with the lanes of padded rows masked off, whose LDS operand
  // reads never happen, while an MFMA still reads every lane's registers.
  v4f sum[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    sum[t] = (acc[t][0] + acc[t][1]) + (acc[t][2] + acc[t][3]);
    asm volatile("" : "+v"(sum[t]));
  }
  if (KSPLIT > 1) {
    // the waves of K ranges 1.. park their partial tiles in LDS (a region no wave
    // reads in its loop); the range-0 wave of each row group adds them in order
    if (kh > 0) {
#pragma unroll
      for (int t = 0; t < MT; ++t)
        *reinterpret_cast<v4f*>(red_lds + ((((kh - 1) * C::RG + rg) * MT + t) * 64 + lane) * 16) =
            sum[t];
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kh > 0) return;   // uniform per wave
#pragma unroll
    for (int k = 1; k < KSPLIT; ++k)
#pragma unroll
      for (int t = 0; t < MT; ++t)
        sum[t] += *reinterpret_cast<const v4f*>(
            red_lds + ((((k - 1) * C::RG + rg) * MT + t) * 64 + lane) * 16);
  }

  // a lane holds out[m][n .. n+3]: one 8-byte (bf16) or 16-byte (fp32) store when
  // the row stride and base allow it
  const bool vec = (p.ldo & 3) == 0 &&
                   (reinterpret_cast<uintptr_t>(p.out) & (p.out_f32 ? 15 : 7)) == 0;
  const int64_t n = nt * C::RROWS + rg * 16 + 4 * gq;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int64_t m = row0 + 16 * t + r;
    if (m >= row_end || n >= p.N) continue;
    const float x0 = sum[t][0] * alpha, x1 = sum[t][1] * alpha;
    const float x2 = sum[t][2] * alpha, x3 = sum[t][3] * alpha;
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
      const uint32_t b01 = bf16_pack2(x0, x1), b23 = bf16_pack2(x2, x3);
      const uint16_t b0 = (uint16_t)b01, b1 = (uint16_t)(b01 >> 16);
      const uint16_t b2 = (uint16_t)b23, b3 = (uint16_t)(b23 >> 16);
      if (vec && n + 3 < p.N) {
        *reinterpret_cast<uint2*>(o) = make_uint2(b01, b23);
      } else {
        o[0] = b0;
        if (n + 1 < p.N) o[1] = b1;
        if (n + 2 < p.N) o[2] = b2;
        if (n + 3 < p.N) o[3] = b3;
      }
    }
  }
}

template <int FMT, int MT, int RING, int KSPLIT>
hipError_t launch_res(const GemmParams& p, hipStream_t s, const char** name) {
  using C = ResCfg<FMT, MT, KSPLIT>;
  const int64_t ntiles = (p.N + C::RROWS - 1) / C::RROWS;
  const int64_t mblocks = p.mblk_expert ? p.n_mblocks : (p.M + 16 * MT - 1) / (16 * MT);
  const int64_t grid = ntiles * mblocks;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (p.K / kRStep < KSPLIT) return hipErrorInvalidValue;
  if (C::ALDS < C::AROWS && (p.mblk_expert || p.M > C::ALDS)) return hipErrorInvalidValue;
  static const char* names[2][2] = {{"resident_nvfp4_m16", "resident_nvfp4_m32"},
                                    {"resident_mxfp4_m16", "resident_mxfp4_m32"}};
  *name = names[FMT][MT - 1];
  const int64_t lds = resident_lds_bytes(FMT, MT, KSPLIT, p.K);
  static std::atomic<uint64_t> lds_set{0};   // devices done, per instantiation
  hipError_t e = ensure_dynamic_lds(
      reinterpret_cast<const void*>(&resident_gemm<FMT, MT, RING, KSPLIT>), (int)kResidentMaxLds, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((resident_gemm<FMT, MT, RING, KSPLIT>), dim3((unsigned)grid), dim3(256),
                     (size_t)lds, s, p);
  return hipGetLastError();
}

// ring depth: the steps of one wave's K range, up to 32 (8 for the four-way split,
// whose 128-register budget holds no deeper ring)
template <int FMT, int MT, int KSPLIT>
hipError_t launch_res_ring(const GemmParams& p, hipStream_t s, const char** name) {
  if constexpr (KSPLIT == 4) {
    return launch_res<FMT, MT, 8, KSPLIT>(p, s, name);
  } else {
    const int64_t ns = p.K / kRStep / KSPLIT;
    if (ns >= 32) return launch_res<FMT, MT, 32, KSPLIT>(p, s, name);
    if (ns >= 16) return launch_res<FMT, MT, 16, KSPLIT>(p, s, name);
    return launch_res<FMT, MT, 8, KSPLIT>(p, s, name);
  }
}

template <int FMT, int MT>
hipError_t launch_res_split(int ksplit, const GemmParams& p, hipStream_t s, const char** name) {
  if constexpr (MT == 1)
    if (ksplit == 4) return launch_res_ring<FMT, MT, 4>(p, s, name);
  if (ksplit == 2) return launch_res_ring<FMT, MT, 2>(p, s, name);
  return launch_res_ring<FMT, MT, 1>(p, s, name);
}

}  // namespace

int64_t resident_lds_bytes(int fmt, int mt, int ksplit, int64_t K) {
  const int64_t G = fmt == kNV ? 16 : 32;
  const int64_t arows = ksplit == 4 ? 4 : 16 * mt;   // staged activation rows
  const int64_t rrows = 64 / ksplit;
  return arows * res_astr(K) + round_kb(arows * (K / G)) + round_kb(rrows * (K / G)) +
         (int64_t)(ksplit - 1) * (4 / ksplit) * mt * 1024;
}

int resident_ksplit(int64_t M, int64_t N, int64_t K, int64_t nblk) {
  // split K while the workgroups (nblk row blocks times the weight tiles) would not
  // cover every CU twice and each wave keeps at least 8 steps; four ways only for at
  // most 4 rows (measured at N = 14336, K = 4096: four ways is best for 1 row, two
  // ways from 8 rows on).  Expert tables count all their row blocks: NVFP4 MoE at
  // T = 64 (160 row blocks) runs unsplit, 117.5 -> 112 us, and at T = 1 (9) split.
  const int64_t ns = K / kRStep;
  const int kmax = M <= 4 ? 4 : 2;   // (so two-tile blocks never split four ways)
  int ks = 1;
  while (ks < kmax && ns / (2 * ks) >= 8 &&
         nblk * ((N + 16 * (4 / ks) - 1) / (16 * (4 / ks))) < 512)
    ks *= 2;
  return ks;
}

bool resident_fits(int fmt, int mt, int64_t M, int64_t N, int64_t K, int64_t nblk) {
  const int64_t G = fmt == kNV ? 16 : 32;
  const int64_t pieces = 16 * mt * (K / 32);          // 16-byte activation pieces
  return K % kRStep == 0 && (K / G) % 16 == 0 && pieces <= 256 * kResPieces &&
         resident_lds_bytes(fmt, mt, resident_ksplit(M, N, K, nblk), K) <= kResidentMaxLds;
}

hipError_t launch_gemm_resident(int fmt, int mt, const GemmParams& p, hipStream_t s,
                                const char** name) {
  // one 16-row activation tile per workgroup (two-tile blocks measured faster on the
  // streaming kernel, so only MT = 1 is built)
  if (mt != 1) return hipErrorInvalidValue;
  const int64_t rows = p.mblk_expert ? 16 : p.M;   // rows per block, at most
  const int64_t nblk = p.mblk_expert ? p.n_mblocks : 1;
  if (!resident_fits(fmt, 1, rows, p.N, p.K, nblk)) return hipErrorInvalidValue;
  const int ks = resident_ksplit(rows, p.N, p.K, nblk);
  return fmt == kNV ? launch_res_split<kNV, 1>(ks, p, s, name)
                    : launch_res_split<kMX, 1>(ks, p, s, name);
}

}  // namespace fp4
