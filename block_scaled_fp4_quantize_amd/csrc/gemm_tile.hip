// Tiled block-scaled FP4 GEMM for many activation rows (prefill, and MoE experts
// with many routed rows), fp4 activations, K a multiple of 128.
//
// Definition as in gemm.hip: out[m, n] = alpha * sum_k a_hat[m, k] * w_hat[n, k]
// ("vLLM per-format kernel capability matrix derived from source", THE EMULATION
// COLUMN), with MXFP4 on gfx950's scaled FP4 MFMA and NVFP4 decoded exactly to
// fp16 for fp16 MFMA ("vLLM on the NVIDIA DGX Spark (GB10 / sm_121): A Complete
// Technical Guide", §6.1 and §6.4 for the two block-scale formats).
//
// Tiling: a workgroup (4 waves, 2 x 2) owns 256 weight rows and 128 activation rows
// (MXFP4 runs two such workgroups per CU).  Each wave computes a 128 x 64 tile with
// 16x16 MFMAs (weights as the A operand, so a lane ends up holding 4 consecutive
// output columns).  K advances in stages of 128: the packed codes (64 bytes per row)
// and block scales of the 384 rows are copied straight from global memory into LDS
// (no staging registers), with NBUF stages in LDS so that the copies of the next
// NBUF - 2 stages are in flight while one stage is multiplied.  Codes travel at 4.5
// bits per element all the way into registers; NVFP4 is decoded to fp16 right before
// the MFMA (unit-scale convert, then one packed fp16 multiply by the e4m3 scale --
// exact), MXFP4 needs no decode at all.
#include <type_traits>

#include "device.h"
#include "internal.h"

namespace fp4 {

namespace {

constexpr int kTBK = 128;        // K per stage

// Staged LDS layout of one K stage (no staging registers: global -> LDS copies).
// Codes: unpadded 64-byte rows; the 16-byte column c of row x is stored at column
// c ^ tile_swz(x & 15), which makes the MFMA fragment reads (16 rows x one column per
// 16 lanes) bank-conflict-free whether the LDS serves 128 or 256 bytes per clock.  A
// copy is 16 rows x 64 bytes, the swizzle applied through each lane's source address.
// Scales: the 4-byte words of a row (MXFP4: one word = the row's 4 block scales of the
// stage; NVFP4: two words, stored as two planes of ROWS words) are stored at word
// tile_sslot(x), which puts the words of rows 16 j + r, j = 4 k .. 4 k + 3, of a 64-row
// block next to each other: a lane (row r) then gets its 4 tiles' scales with one
// 16-byte read, and 16 lanes read 256 consecutive bytes.  Every wave issues the same
// number OPS of copies per stage (pad copies repeat copy 0 into a pad area), so one
// compile-time vmcnt serves all waves.  NBUF stages live in LDS at once.
__device__ __forceinline__ int tile_swz(int r) {
  return ((r >> 2) & 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 1);
}
__device__ __forceinline__ int tile_sslot(int x) {
  return (x & ~63) | ((x & 15) << 2) | ((x >> 4) & 3);
}
__device__ __forceinline__ int tile_srow(int slot) {   // inverse of tile_sslot
  return (slot & ~63) | ((slot & 3) << 4) | ((slot >> 2) & 15);
}

// BM activation rows x BN weight rows per workgroup.  NVFP4 128 x 128 tiles take half
// the registers of 128 x 256 ones, so two workgroups share a CU (as for MXFP4 at 128 x
// 256) and one computes while the other waits.
template <int FMT, int BM, int BN>
struct TileCfg {
  static constexpr int G = FMT == kNV ? 16 : 32;
  static constexpr int SB = kTBK / G;                  // scale bytes per row per stage
  static constexpr int WM = BM / 64;                   // waves along the activation rows
  static constexpr int WAVES = 2 * WM;                 // (two along the weight rows)
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int MI = 4;                         // 16-row activation tiles per wave
  static constexpr int NJ = BN / 32;                   // 16-row weight tiles per wave
  static constexpr int ROWS = BM + BN;                 // staged rows: activations, then weights
  static constexpr int CCOP = ROWS / 16;               // 1 KB code copies per stage
  static constexpr int CPW = CCOP / WAVES;             // ... per wave
  static constexpr int SDW = ROWS * SB / 4;            // scale words per stage
  static constexpr int SCOP = (SDW + 63) / 64;         // 256-byte scale copies
  static constexpr int SPW = (SCOP + WAVES - 1) / WAVES;  // ... per wave (padded)
  static constexpr int PLANES = SB / 4;                // scale words per row per stage
  // Grouped scales (the 8-wave tile, whose LDS has room for them): a copy moves the
  // words of 16 rows for 4 consecutive stages (16 bytes of each row), so each scale
  // line is fetched once per 4 stages instead of once per stage.  A group (4 stages)
  // takes SGI copies, issued a quarter per stage, into one of 3 group buffers.
  static constexpr bool SGRP = BM == 256 && FMT == kMX;
  static constexpr int SGI = ROWS / 16 * PLANES;       // 256-byte copies per group
  static constexpr int SGW = SGI / 4 / WAVES;          // ... per wave per stage
  static constexpr int ISTR = 320;                     // LDS stride of those copies
  static constexpr int SGBYTES = SGI * ISTR;           // one group buffer
  static constexpr int OPS = CPW + (SGRP ? SGW : SPW);  // copies per wave per stage
  static constexpr int CODES = ROWS * 64;
  static constexpr int STAGE = CODES + (SGRP ? 0 : WAVES * SPW * 256);  // bytes per LDS stage
  // LDS stride between the scale words of consecutive 64-row blocks (as seen by a lane)
  static constexpr int SBLK = SGRP ? 4 * ISTR : 256;
  // workgroups per CU (the register budget follows from it: 512 / (PER_CU * WAVES /
  // 4) per lane): 4-wave tiles that fit in 256 registers run two per CU (MXFP4 128 x
  // 256, NVFP4 128 x 128), MXFP4 128 x 128 three; 8-wave tiles one.  Four stages
  // in LDS when they fit next to the other workgroups, else three.
  static constexpr int PER_CU =
      BM == 128 ? (BN == 128 ? (FMT == kMX ? 3 : 2) : (FMT == kMX ? 2 : 1)) : 1;
  static constexpr int NBUF = PER_CU * 4 * STAGE <= 160 * 1024 ? 4 : 3;
  static constexpr int SGOFF = NBUF * STAGE;           // group buffers follow the stages
  static constexpr int LDS = NBUF * STAGE + (SGRP ? 3 * SGBYTES : 0);
  static_assert(!SGRP || SGI % (4 * WAVES) == 0, "group copies split evenly over stages and waves");
  static_assert(CCOP % WAVES == 0, "code copies split evenly over the waves");
  static_assert(BM % 128 == 0 && BN % 128 == 0, "64-row scale blocks, 4-tile weight groups");
  static_assert(NBUF >= 3 && NBUF <= 4, "the stage waits cover up to two stages in flight");
  static_assert(PER_CU * LDS <= 160 * 1024, "LDS per CU");
  static_assert(THREADS == 2 * BM, "launch bounds of tile_gemm");
};

#define FP4_TILE_LDS(p) ((__attribute__((address_space(3))) void*)(p))
// One LDS-direct copy per lane: 16 bytes to lds + 16 lane, or 4 bytes to lds + 4 lane
// (M0 = the wave-uniform LDS base, one wait state before its use).  Issued from
// inline asm: the compiler's wait-count pass would otherwise drain every load before
// any later LDS read; the kernel waits for these copies itself.
__device__ __forceinline__ void tile_copy16(const void* g, uint8_t* lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)FP4_TILE_LDS(lds));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(m0v), "v"(g) : "memory", "m0");
}
__device__ __forceinline__ void tile_copy4(const void* g, uint8_t* lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)FP4_TILE_LDS(lds));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :: "s"(m0v), "v"(g) : "memory", "m0");
}
// s_waitcnt vmcnt(n) lgkmcnt(0) (gfx9 encoding): this wave's copies except the last n
// have landed and its own LDS reads are done, so after the barrier that follows, the
// buffer just read may be overwritten
constexpr int tile_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

// The MFMA work of one staged K step: fragment reads (codes at row * 64 + ccol; the
// 16 scale bytes of this lane's row in the 4 tiles of 64-row block b at sc + b * SBLK)
// and the MFMAs into acc.
// PART: only the first nv (wave-uniform) 16-row activation tiles of the wave hold
// rows that exist (a row block cut short, as an MoE expert's last one is); the others
// are neither read nor multiplied, and their accumulators stay zero (never stored).
template <int FMT, int BM, int BN, bool PART = false>
__device__ __forceinline__ void tile_step(
    const uint8_t* cur, const uint8_t* sc, int ccol, int r, int gq, int wm, int wn,
    v4f (&acc)[TileCfg<FMT, BM, BN>::NJ][TileCfg<FMT, BM, BN>::MI], int nv = TileCfg<FMT, BM, BN>::MI) {
  using C = TileCfg<FMT, BM, BN>;
  // fragments of this stage: weights (A operand) and activations (B operand).  The
  // scale word of tile j of this lane's row holds its 4 (MXFP4) or 2 (NVFP4 plane
  // gq / 2) block scales; the lane's own block starts at bit 8 gq or 16 (gq & 1).
  uint4 wf[C::NJ];
  uint32_t wsb[C::NJ];
  uint4 af[C::MI];
  uint32_t asb[C::MI];
  const int ssh = FMT == kNV ? 16 * (gq & 1) : 8 * gq;
#pragma unroll
  for (int j = 0; j < C::NJ; ++j)
    wf[j] = *reinterpret_cast<const uint4*>(cur + (BM + wn * (BN / 2) + 16 * j + r) * 64 + ccol);
#pragma unroll
  for (int k = 0; k < C::NJ / 4; ++k) {
    const uint4 w4 = *reinterpret_cast<const uint4*>(sc + ((BM + wn * (BN / 2)) / 64 + k) * C::SBLK);
    wsb[4 * k + 0] = w4.x >> ssh;
    wsb[4 * k + 1] = w4.y >> ssh;
    wsb[4 * k + 2] = w4.z >> ssh;
    wsb[4 * k + 3] = w4.w >> ssh;
  }
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
    if (!PART || i < nv)
      af[i] = *reinterpret_cast<const uint4*>(cur + (wm * 64 + 16 * i + r) * 64 + ccol);
  {
    const uint4 a4 = *reinterpret_cast<const uint4*>(sc + wm * C::SBLK);
    asb[0] = a4.x >> ssh;
    asb[1] = a4.y >> ssh;
    asb[2] = a4.z >> ssh;
    asb[3] = a4.w >> ssh;
  }
  static_assert(C::MI == 4 && C::NJ % 4 == 0, "scale words are read 4 tiles at a time");

  if (FMT == kMX) {
    if (PART) {   // activation tile outermost: one uniform branch per tile
#pragma unroll
      for (int i = 0; i < C::MI; ++i) {
        if (i >= nv) break;
        const v8i aop = {(int)af[i].x, (int)af[i].y, (int)af[i].z, (int)af[i].w, 0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < C::NJ; ++j) {
          const v8i wop = {(int)wf[j].x, (int)wf[j].y, (int)wf[j].z, (int)wf[j].w, 0, 0, 0, 0};
          acc[j][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              wop, aop, acc[j][i], 4, 4, 0, (int)wsb[j], 0, (int)asb[i]);
        }
      }
      return;
    }
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
    // the lane's two block scales of each tile (bytes 0 and 1 of its scale word)
    f16x2 asc[C::MI], wsc[C::NJ];
#pragma unroll
    for (int i = 0; i < C::MI; ++i) asc[i] = e4m3_pair_f16(asb[i]);
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) wsc[j] = e4m3_pair_f16(wsb[j]);
    if (PART) {   // activation tile outermost: one uniform branch per tile
#pragma unroll
      for (int i = 0; i < C::MI; ++i) {
        if (i >= nv) break;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const f16x8 aop = decode8_f16(dword_of(af[i], s), f16_bcast(asc[i], s >> 1));
#pragma unroll
          for (int j = 0; j < C::NJ; ++j) {
            const f16x8 wop = decode8_f16(dword_of(wf[j], s), f16_bcast(wsc[j], s >> 1));
            acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wop, aop, acc[j][i], 0, 0, 0);
          }
        }
      }
      return;
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      f16x8 aop[C::MI];
#pragma unroll
      for (int i = 0; i < C::MI; ++i)
        aop[i] = decode8_f16(dword_of(af[i], s), f16_bcast(asc[i], s >> 1));
#pragma unroll
      for (int j = 0; j < C::NJ; ++j) {
        const f16x8 wop = decode8_f16(dword_of(wf[j], s), f16_bcast(wsc[j], s >> 1));
#pragma unroll
        for (int i = 0; i < C::MI; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wop, aop[i], acc[j][i], 0, 0, 0);
      }
    }
  }

}

// Each wave holds a BN/2 (weight rows) x 64 (activation rows) accumulator tile.
// MXFP4 128 x 256 and NVFP4 128 x 128 tiles fit in 256 registers, so two workgroups
// share a CU and one computes while the other waits at a barrier; MXFP4 256 x 256
// tiles use 8 waves (two per SIMD) on one CU, sharing each staged weight row between
// twice as many activation rows.
// FUSE: the gate/up GEMM of an MoE expert with SwiGLU + requant in the epilogue.  The
// workgroup's BN weight rows are then BN/2 gate rows and the matching BN/2 up rows of
// h columns [BN/2 nt, BN/2 nt + BN/2): wave column wn takes h columns BN/4 wn + [0,
// BN/4), its weight tiles 0 .. NJ/2-1 being the gate rows and NJ/2 .. NJ-1 the up rows
// of the same columns, so a lane holds gate and up of the same (m, h column).
template <int FMT, int BM, int BN, bool FUSE>
__global__ __launch_bounds__(2 * BM, (TileCfg<FMT, BM, BN>::PER_CU)) void tile_gemm(GemmParams p) {
  using C = TileCfg<FMT, BM, BN>;
  extern __shared__ __attribute__((aligned(16))) uint8_t tsm[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int wm = wave % C::WM;
  const int wn = wave / C::WM;
  const int64_t ntiles = (p.N + BN - 1) / BN;
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
  // per-group scalars fetched up front, not after the main loop
  const float alpha = p.alpha_g ? p.alpha_g[grp] : p.alpha;
  const float hg = FUSE ? (p.h_grp_g ? p.h_grp_g[grp] : p.h_g) : 0.0f;
  const int64_t K = p.K;
  const int64_t KB = K >> 1;
  const int64_t KS = K / C::G;
  const uint8_t* wcodes = p.w_codes + grp * p.w_estride_codes;
  const uint8_t* wscales = p.w_scales + grp * p.w_estride_scales;

  // global source row of staged row rr (fixed for all stages); rows past the end are
  // clamped to the last valid one (their outputs are not stored)
  auto src_row = [&](int rr) -> int64_t {
    if (rr < BM) {
      int64_t pv = row0 + rr;
      if (pv >= row_end) pv = row_end - 1;
      return p.a_gather ? (int64_t)p.a_gather[pv] : pv;
    }
    int64_t n;
    if (FUSE) {
      const int w = rr - BM, within = w % (BN / 2);
      const int64_t col = nt * (BN / 2) + (w / (BN / 2)) * (BN / 4) + within % (BN / 4);
      n = within < BN / 4 ? col : p.I + col;
    } else {
      n = nt * BN + (rr - BM);
    }
    return n < p.N ? n : p.N - 1;
  };
  // code copy q of this wave is copy c = wave + WAVES q (staged rows 16 c ..): lane l
  // fetches row 16 c + l/4, column (l & 3) ^ tile_swz(l/4) into LDS slot l.  Scale
  // copy q is c = wave + WAVES q (a pad copy past the last repeats copy 0): lane l
  // fills scale word e = 64 c + l (clamped to the last one), i.e. plane e / ROWS,
  // staged row tile_srow(e % ROWS).
  const uint8_t* dcode[C::CPW];
  const uint8_t* dscale[C::SPW];
#pragma unroll
  for (int q = 0; q < C::CPW; ++q) {
    const int rr = 16 * (wave + C::WAVES * q) + (lane >> 2);
    const int col = (lane & 3) ^ tile_swz(lane >> 2);
    dcode[q] = (rr < BM ? p.a_codes : wcodes) + src_row(rr) * KB + col * 16;
  }
#pragma unroll
  for (int q = 0; q < C::SPW; ++q) {
    int c = wave + C::WAVES * q;
    if (c >= C::SCOP) c = 0;
    int e = 64 * c + lane;
    if (e >= C::SDW) e = C::SDW - 1;
    const int plane = e / C::ROWS;
    const int rr = tile_srow(e - plane * C::ROWS);
    dscale[q] = (rr < BM ? p.a_scales : wscales) + src_row(rr) * KS + plane * 4;
  }

  // Grouped scales: copy c of a group (c = SGI/4 q + wave + WAVES w for quarter q) is
  // plane c / (ROWS/16), 64-row block b = (c % (ROWS/16)) / 4 and rows 4 (c % 4) ..
  // +3 of each of the block's 4 tiles; lane l fetches stage 4 g + l / 16 of tile l % 4,
  // row 4 (c % 4) + (l / 4) % 4, so the 256 bytes land as [stage][row][tile] words and
  // a lane reads its row's 4 tile words of one stage with one 16-byte read.
  const uint8_t* gsrc[4][C::SGW > 0 ? C::SGW : 1];
  if constexpr (C::SGRP) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int w = 0; w < C::SGW; ++w) {
        const int c = (C::SGI / 4) * q + wave + C::WAVES * w;
        const int plane = c / (C::ROWS / 16), rem = c % (C::ROWS / 16);
        const int rr = (rem / 4) * 64 + (lane & 3) * 16 + 4 * (rem % 4) + ((lane >> 2) & 3);
        gsrc[q][w] = (rr < BM ? p.a_scales : wscales) + src_row(rr) * KS + plane * 4;
      }
  }
  v4f acc[C::NJ][C::MI];
#pragma unroll
  for (int j = 0; j < C::NJ; ++j)
#pragma unroll
    for (int i = 0; i < C::MI; ++i) acc[j][i] = v4f{0.f, 0.f, 0.f, 0.f};

  const int r = lane & 15;
  const int gq = lane >> 4;
  const int64_t nstages = K / kTBK;

  // Stage t lives in buffer t % NBUF.  Iteration st issues stage st + NBUF - 1 (if it
  // exists) into the buffer computed at st - 1, computes stage st, then waits until
  // stage st + 1 has landed -- the stages after it may stay in flight -- and syncs.
  // The last iteration waits for everything, so no copy is outstanding after the loop.
  // quarter q of scale group gi into group buffer gi % 3 (stages past the end re-read
  // the last one: a group past the end is padding, its buffer free like any other)
  auto issue_grp = [&](int64_t gi, int q, int w) {
    uint8_t* gb = tsm + C::SGOFF + (int)(gi % 3) * C::SGBYTES;
    int64_t stg = 4 * gi + (lane >> 4);
    if (stg >= nstages) stg = nstages - 1;
    tile_copy4(gsrc[q][w] + stg * C::SB, gb + ((C::SGI / 4) * q + wave + C::WAVES * w) * C::ISTR);
  };
  // copy u (0 .. OPS-1) of stage t: the code copies, then the scale copies
  auto issue_part = [&](int64_t t, int u) {
    uint8_t* buf = tsm + (int)(t % C::NBUF) * C::STAGE;
    if (u < C::CPW) {
      tile_copy16(dcode[u] + t * 64, buf + (wave + C::WAVES * u) * 1024);
    } else if constexpr (C::SGRP) {
      issue_grp(t / 4 + 1, (int)(t % 4), u - C::CPW);
    } else {
      tile_copy4(dscale[u - C::CPW] + t * C::SB, buf + C::CODES + (wave + C::WAVES * (u - C::CPW)) * 256);
    }
  };
  auto issue = [&](int64_t t) {
#pragma unroll
    for (int u = 0; u < C::OPS; ++u) issue_part(t, u);
  };
  auto sync = [&](int64_t ahead) {   // stages issued after the one needed next
    if (ahead >= 3)
      __builtin_amdgcn_s_waitcnt(tile_vmcnt(3 * C::OPS));
    else if (ahead >= 2)
      __builtin_amdgcn_s_waitcnt(tile_vmcnt(2 * C::OPS));
    else if (ahead >= 1)
      __builtin_amdgcn_s_waitcnt(tile_vmcnt(C::OPS));
    else
      __builtin_amdgcn_s_waitcnt(tile_vmcnt(0));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // fragment rows are 16-row tile starts + r, so their swizzle is tile_swz(r)
  const int gcol = (gq ^ tile_swz(r)) << 4;
  // 16-row activation tiles of this wave that hold existing rows (uniform per wave)
  int nvt;
  {
    const int64_t left = row_end - (row0 + wm * 64);
    nvt = left >= 64 ? 4 : (left <= 0 ? 0 : (int)((left + 15) / 16));
    nvt = __builtin_amdgcn_readfirstlane(nvt);
  }
  // this lane's scale words: plane gq / 2 (NVFP4), row r
  const int splane = FMT == kNV ? (gq >> 1) : 0;
  const int srd = C::SGRP ? splane * (C::ROWS / 16) * C::ISTR + (r >> 2) * C::ISTR + (r & 3) * 16
                          : C::CODES + splane * C::ROWS * 4 + r * 16;
  auto stage_scales = [&](int64_t s, const uint8_t* cur) -> const uint8_t* {
    return C::SGRP ? tsm + C::SGOFF + (int)((s / 4) % 3) * C::SGBYTES + (int)(s % 4) * 64 + srd
                   : cur + srd;
  };
  // Scale group g is issued with code stages 4 g - 4 .. 4 g - 1 (group 0 up front) and
  // read by stages 4 g .. 4 g + 3; its buffer last held group g - 3, whose reads all
  // ended before the barrier that precedes the first of those issues.
  if constexpr (C::SGRP) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int w = 0; w < C::SGW; ++w) issue_grp(0, q, w);
  }

  if constexpr (FMT == kMX && C::NBUF == 4) {
    // Software-pipelined: the LDS operands of stage st + 1 are read while the MFMAs of
    // stage st run, each into the registers of an operand right after its last MFMA
    // (weight tile j after tile j's MFMAs, activation tile i during the last weight
    // tile's), so a stage's MFMAs never wait on LDS.  Stage st's buffer is free once
    // its operands are in registers: iteration st refills it with stage st + NBUF, and
    // waits (before its barrier) until stage st + 2 has landed.  Only with four stage
    // buffers: with three, the copies would get one stage less to land than in the
    // plain loop below, which measured faster there (MoE 128-row tiles).
    const int wrow0 = BM + wn * (BN / 2);
    u32x4 wf[C::NJ];
    uint32_t wsb[C::NJ];
    u32x4 af[C::MI];
    uint32_t asb[C::MI];
    const int ssh = 8 * gq;
    auto rd_w = [&](const uint8_t* cur, int j) {
      return *reinterpret_cast<const u32x4*>(cur + (wrow0 + 16 * j + r) * 64 + gcol);
    };
    auto rd_ws = [&](const uint8_t* sc, int k) {   // weight tiles 4 k .. 4 k + 3
      const u32x4 w4 = *reinterpret_cast<const u32x4*>(sc + (wrow0 / 64 + k) * C::SBLK);
      wsb[4 * k + 0] = w4.x >> ssh;
      wsb[4 * k + 1] = w4.y >> ssh;
      wsb[4 * k + 2] = w4.z >> ssh;
      wsb[4 * k + 3] = w4.w >> ssh;
    };
    auto rd_a = [&](const uint8_t* cur, int i) {
      return *reinterpret_cast<const u32x4*>(cur + (wm * 64 + 16 * i + r) * 64 + gcol);
    };
    auto rd_as = [&](const uint8_t* sc) {
      const u32x4 a4 = *reinterpret_cast<const u32x4*>(sc + wm * C::SBLK);
      asb[0] = a4.x >> ssh;
      asb[1] = a4.y >> ssh;
      asb[2] = a4.z >> ssh;
      asb[3] = a4.w >> ssh;
    };
    auto mma = [&](int j, int i) {
      const v8i wop = {(int)wf[j].x, (int)wf[j].y, (int)wf[j].z, (int)wf[j].w, 0, 0, 0, 0};
      const v8i aop = {(int)af[i].x, (int)af[i].y, (int)af[i].z, (int)af[i].w, 0, 0, 0, 0};
      acc[j][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          wop, aop, acc[j][i], 4, 4, 0, (int)wsb[j], 0, (int)asb[i]);
    };
    static_assert(C::MI == 4 && C::NJ % 4 == 0, "scale words are read 4 tiles at a time");
#pragma unroll
    for (int t = 0; t < C::NBUF; ++t)
      if (t < nstages) issue(t);
    sync(nstages - 1 < C::NBUF - 1 ? nstages - 1 : C::NBUF - 1);   // stage 0 landed
    {
      const uint8_t* sc = stage_scales(0, tsm);
#pragma unroll
      for (int j = 0; j < C::NJ; ++j) wf[j] = rd_w(tsm, j);
#pragma unroll
      for (int k = 0; k < C::NJ / 4; ++k) rd_ws(sc, k);
#pragma unroll
      for (int i = 0; i < C::MI; ++i) af[i] = rd_a(tsm, i);
      rd_as(sc);
    }
    // stage 1 landed; every wave's reads of buffer 0 done
    sync(nstages - 1 < C::NBUF - 1 ? (nstages - 1 > 0 ? nstages - 2 : 0) : C::NBUF - 2);
    // copy u goes after MFMA group u (NJ - 1) / OPS <= NJ - 2: every copy is issued
    static_assert(C::NJ >= 2, "at least two weight tiles per wave");
    for (int64_t st = 0; st < nstages; ++st) {
      // stage st + NBUF refills this stage's buffer; its OPS copies are spread over
      // the MFMA groups below (issued in one burst, the copies of the 8 waves queue
      // up in the texture unit and stall the waves behind them)
      const bool refill = st + C::NBUF < nstages;
      // operands of stage st + 1 (or stage st again after the last: its buffer is not
      // refilled then, and the values go unused)
      const int64_t sn = st + 1 < nstages ? st + 1 : st;
      const uint8_t* cur = tsm + (int)(sn % C::NBUF) * C::STAGE;
      const uint8_t* sc = stage_scales(sn, cur);
#pragma unroll
      for (int j = 0; j < C::NJ - 1; ++j) {
#pragma unroll
        for (int i = 0; i < C::MI; ++i) mma(j, i);
        // pins the order: the MFMAs above (their results pass through here), then the
        // reads below (the memory clobber keeps them from being hoisted)
        asm volatile("" : "+v"(acc[j][0]), "+v"(acc[j][1]), "+v"(acc[j][2]), "+v"(acc[j][3])
                     :: "memory");
#pragma unroll
        for (int u = 0; u < C::OPS; ++u)
          if (u * (C::NJ - 1) / C::OPS == j && refill) issue_part(st + C::NBUF, u);
        wf[j] = rd_w(cur, j);
        if (j % 4 == 3) rd_ws(sc, j / 4);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < C::MI; ++i) {
        mma(C::NJ - 1, i);
        asm volatile("" : "+v"(acc[C::NJ - 1][i]) :: "memory");
        af[i] = rd_a(cur, i);
      }
      wf[C::NJ - 1] = rd_w(cur, C::NJ - 1);
      rd_ws(sc, C::NJ / 4 - 1);
      rd_as(sc);
      __builtin_amdgcn_sched_barrier(0);
      // stage st + 2 landed (the stages issued after it may stay in flight)
      const int64_t last = st + C::NBUF < nstages ? st + C::NBUF : nstages - 1;
      sync(st + 2 <= nstages - 1 ? last - (st + 2) : 0);
    }
  } else {
    // Row blocks cut short take the per-tile form of the step through their own copy
    // of the loop (two forms in one loop would double the live registers)
    auto plain = [&](auto partial) {
      constexpr bool PART = decltype(partial)::value;
#pragma unroll
      for (int t = 0; t < C::NBUF - 1; ++t)
        if (t < nstages) issue(t);
      sync(nstages - 1 < C::NBUF - 2 ? nstages - 1 : C::NBUF - 2);
      for (int64_t st = 0; st < nstages; ++st) {
        const int64_t t = st + C::NBUF - 1;
        if (t < nstages) issue(t);
        const uint8_t* cur = tsm + (int)(st % C::NBUF) * C::STAGE;
        tile_step<FMT, BM, BN, PART>(cur, stage_scales(st, cur), gcol, r, gq, wm, wn, acc, nvt);
        sync((t < nstages ? t : nstages - 1) - (st + 1));
      }
    };
    if constexpr (BM == 128) {   // (the 256-row tile: dense only, no copy)
      if (nvt < C::MI) {
        plain(std::true_type{});
      } else {
        plain(std::false_type{});
      }
    } else {
      plain(std::false_type{});
    }
  }

  if (FUSE) {
    // h = SiLU(alpha g) * (alpha u) for this lane's 4 consecutive h columns of each
    // gate tile j (up tile j + NJ/2); a quantization block (16 or 32 columns of one
    // row) spans the lanes r, r + 16, r + 32, r + 48 (and, for MXFP4, gate tiles j and
    // j + 1), so its amax is two lane exchanges away.  Every lane takes part in the
    // exchanges; only rows that exist are stored.
    constexpr int NG = C::NJ / 2;   // gate tiles per wave
    static_assert(NG % 2 == 0, "MXFP4 blocks pair gate tiles");
    const float g = hg;
    const int64_t hrow = p.I / 2;
#pragma unroll
    for (int i = 0; i < C::MI; ++i) {
      const int64_t m = row0 + wm * 64 + 16 * i + r;
      const bool store = m < row_end;
      float h[NG][4];
#pragma unroll
      for (int j = 0; j < NG; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) h[j][v] = swiglu1(acc[j][i][v] * alpha, acc[j + NG][i][v] * alpha);
      // + 16 j: this lane's first column
      const int64_t hc0 = nt * (BN / 2) + wn * (BN / 4) + 4 * gq;
      if (FMT == kNV) {
#pragma unroll
        for (int j = 0; j < NG; ++j) {
          float amax = fmaxf(fmaxf(fabsf(h[j][0]), fabsf(h[j][1])), fmaxf(fabsf(h[j][2]), fabsf(h[j][3])));
          amax = fmaxf(amax, __shfl_xor(amax, 16));
          amax = fmaxf(amax, __shfl_xor(amax, 32));
          float rs;
          const uint32_t sc = q_nv_scale(amax, g, &rs);
          const uint32_t q = q_nv_pack2(h[j][0], h[j][1], rs) | (q_nv_pack2(h[j][2], h[j][3], rs) << 8);
          if (store) {
            const int64_t hc = hc0 + 16 * j;
            *reinterpret_cast<uint16_t*>(p.h_codes + m * hrow + hc / 2) = (uint16_t)q;
            if (gq == 0) p.h_scales[m * (p.I / 16) + hc / 16] = (uint8_t)sc;
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < NG; j += 2) {
          float amax = 0.0f;
#pragma unroll
          for (int v = 0; v < 4; ++v) amax = fmaxf(amax, fmaxf(fabsf(h[j][v]), fabsf(h[j + 1][v])));
          amax = fmaxf(amax, __shfl_xor(amax, 16));
          amax = fmaxf(amax, __shfl_xor(amax, 32));
          int E;
          const uint32_t sc = q_mx_scale(amax, &E);
          const uint32_t q0 = q_mx_pack2(h[j][0], h[j][1], E) | (q_mx_pack2(h[j][2], h[j][3], E) << 8);
          const uint32_t q1 =
              q_mx_pack2(h[j + 1][0], h[j + 1][1], E) | (q_mx_pack2(h[j + 1][2], h[j + 1][3], E) << 8);
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
  // the wave's BN/2 columns inside the output and aligned: stores without per-column
  // checks (uniform decision), rows checked per lane only if the block is cut short
  {
    const int64_t m_lo = row0 + wm * 64, n_lo = nt * BN + wn * (BN / 2);
    if (vec && n_lo + BN / 2 <= p.N) {
      const bool rows_full = m_lo + 64 <= row_end;
#pragma unroll
      for (int i = 0; i < C::MI; ++i) {
        if (!rows_full && m_lo + 16 * i + r >= row_end) continue;
        const int64_t off = (m_lo + 16 * i + r) * p.ldo + n_lo + 4 * gq;
#pragma unroll
        for (int j = 0; j < C::NJ; ++j) {
          const float x0 = acc[j][i][0] * alpha, x1 = acc[j][i][1] * alpha;
          const float x2 = acc[j][i][2] * alpha, x3 = acc[j][i][3] * alpha;
          if (p.out_f32)
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + off + 16 * j) =
                make_float4(x0, x1, x2, x3);
          else
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + off + 16 * j) =
                make_uint2(bf16_pack2(x0, x1), bf16_pack2(x2, x3));
        }
      }
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < C::MI; ++i) {
    const int64_t m = row0 + wm * 64 + 16 * i + r;
    if (m >= row_end) continue;
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) {
      const int64_t n = nt * BN + wn * (BN / 2) + 16 * j + 4 * gq;
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
}

template <int FMT, int BM, int BN, bool FUSE>
hipError_t launch_tile(const GemmParams& p, hipStream_t s, const char** name) {
  using C = TileCfg<FMT, BM, BN>;
  const int64_t ntiles = (p.N + BN - 1) / BN;
  const int64_t mblocks = p.mblk_expert ? p.n_mblocks : (p.M + BM - 1) / BM;
  const int64_t grid = ntiles * mblocks;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (FMT == kNV)
    *name = FUSE ? (BN == 128 ? "tile_nvfp4_m128_n128_swiglu" : "tile_nvfp4_m128_swiglu")
                 : (BM == 256 ? "tile_nvfp4_m256" : (BN == 128 ? "tile_nvfp4_m128_n128" : "tile_nvfp4_m128"));
  else
    *name = FUSE ? "tile_mxfp4_m128_swiglu" : (BM == 256 ? "tile_mxfp4_m256" : "tile_mxfp4_m128");
  if (p.K % kTBK != 0 || p.K <= 0) return hipErrorInvalidValue;
  if (FUSE && (p.I <= 0 || p.I % 128 != 0 || p.N != 2 * p.I || !p.h_codes || !p.h_scales))
    return hipErrorInvalidValue;
  const size_t lds = C::LDS;
  static std::atomic<uint64_t> lds_set{0};   // devices done, per instantiation
  hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&tile_gemm<FMT, BM, BN, FUSE>),
                                    (int)lds, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((tile_gemm<FMT, BM, BN, FUSE>), dim3((unsigned)grid), dim3(C::THREADS), lds,
                     s, p);
  return hipGetLastError();
}

// NVFP4 weight-tile width (128: two workgroups per CU)
constexpr int kNvTileN = 128;

}  // namespace

hipError_t launch_gemm_tiled(int fmt, const GemmParams& p, hipStream_t s, const char** name) {
  const int64_t ntiles256 = (p.N + 255) / 256;
  const bool big = !p.mblk_expert && ((p.M + 255) / 256) * ntiles256 >= 256;
  if (fmt == kNV) {
    if (p.fuse_swiglu) return launch_tile<kNV, 128, kNvTileN, true>(p, s, name);
    if (big) return launch_tile<kNV, 256, 256, false>(p, s, name);
    return launch_tile<kNV, 128, kNvTileN, false>(p, s, name);
  }
  if (p.fuse_swiglu) return launch_tile<kMX, 128, 256, true>(p, s, name);
  // dense MXFP4 with enough 256 x 256 tiles to give every CU one: the 8-wave tile
  if (big) return launch_tile<kMX, 256, 256, false>(p, s, name);
  return launch_tile<kMX, 128, 256, false>(p, s, name);
}

}  // namespace fp4
