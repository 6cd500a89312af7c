// Tiled block-scaled FP4 GEMM for many activation rows (prefill, and MoE experts
// with many routed rows), fp4 activations, K a multiple of 128.
//
// Definition as in gemm.hip: out[m, n] = alpha * sum_k a_hat[m, k] * w_hat[n, k]
// ("vLLM per-format kernel capability matrix derived from source", THE EMULATION
// COLUMN), with MXFP4 on gfx950's scaled FP4 MFMA and NVFP4 decoded exactly to
// fp16 for fp16 MFMA ("vLLM on the NVIDIA DGX Spark (GB10 / sm_121): A Complete
// Technical Guide", §6.1 and §6.4 for the two block-scale formats).
//
// Two tile kernels.  Dense problems with at least 256 tiles of 256 x 256 run big_gemm
// (below): 4 waves, each 128 x 128 outputs, one workgroup per CU.  The rest (MoE
// expert blocks, mid-size dense problems) run tile_gemm:
// a workgroup (4 waves, 2 x 2) owns 256 weight rows and 128 activation rows
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
#include <utility>

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
  static constexpr int OPS = CPW + SPW;                // copies per wave per stage
  static constexpr int CODES = ROWS * 64;
  static constexpr int STAGE = CODES + WAVES * SPW * 256;  // bytes per LDS stage
  // LDS stride between the scale words of consecutive 64-row blocks (as seen by a lane)
  static constexpr int SBLK = 256;
  // workgroups per CU (the register budget follows from it: 512 / (PER_CU * WAVES /
  // 4) per lane): tiles that fit in 256 registers run two per CU (MXFP4 128 x 256,
  // NVFP4 128 x 128), MXFP4 128 x 128 three.  Four stages in LDS when they fit next
  // to the other workgroups, else three.
  static constexpr int PER_CU = BN == 128 ? (FMT == kMX ? 3 : 2) : (FMT == kMX ? 2 : 1);
  static constexpr int NBUF = PER_CU * 4 * STAGE <= 160 * 1024 ? 4 : 3;
  static constexpr int LDS = NBUF * STAGE;
  static_assert(CCOP % WAVES == 0, "code copies split evenly over the waves");
  static_assert(BM == 128 && BN % 128 == 0, "64-row scale blocks, 4-tile weight groups");
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
  // copy u (0 .. OPS-1) of stage t: the code copies, then the scale copies
  auto issue_part = [&](int64_t t, int u) {
    uint8_t* buf = tsm + (int)(t % C::NBUF) * C::STAGE;
    if (u < C::CPW) {
      tile_copy16(dcode[u] + t * 64, buf + (wave + C::WAVES * u) * 1024);
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
  const int srd = C::CODES + splane * C::ROWS * 4 + r * 16;

  {
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
        tile_step<FMT, BM, BN, PART>(cur, cur + srd, gcol, r, gq, wm, wn, acc, nvt);
        sync((t < nstages ? t : nstages - 1) - (st + 1));
      }
    };
    if (nvt < C::MI) {
      plain(std::true_type{});
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
                 : (BN == 128 ? "tile_nvfp4_m128_n128" : "tile_nvfp4_m128");
  else
    *name = FUSE ? "tile_mxfp4_m128_swiglu" : "tile_mxfp4_m128";
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

// ---- dense problems with many 256 x 256 tiles: a 4-wave tile, 128 x 128 per wave ----
// One wave per SIMD; wave (wm, wn) computes 128 activation rows x 128 weight rows as
// 8 x 8 16x16 MFMA tiles (256 accumulator registers), so each LDS operand read feeds 8
// MFMAs (the 8-wave tile's feed 4 or 8) and, for NVFP4, each decoded operand tile too.
// The staged LDS layout is the one above (64-byte code rows, XOR-swizzled columns, scale
// words in tile_sslot order), four stage buffers.  Weight rows are staged in pair order:
// in each 32-row group, 16-row tile 2p holds rows 8q + v and tile 2p + 1 rows 8q + 4 + v
// (q, v = 0..3), so a lane's accumulators of the two tiles are 8 consecutive output
// columns (one 16-byte bf16 store).
// Global row (within its 256-row tile) of staged weight row w.  MXFP4 (16x16 MFMAs, a
// lane holds rows 4 gq + v of a 16-row tile): tile 2p holds rows 32 p + 8 q + v and
// tile 2p + 1 rows 32 p + 8 q + 4 + v.  NVFP4 (32x32 MFMAs, a lane holds rows 8 g +
// 4 h + v of a 32-row tile, g = 0..3): row 8 g + 4 h + v of tile T is 32 T + 16 (g >> 1)
// + 8 h + 4 (g & 1) + v.  Either way a lane's accumulators cover runs of 8 consecutive
// output columns.
template <int FMT>
__device__ __forceinline__ int big_wperm(int w) {
  if (FMT == kMX) {
    const int t = w >> 4, rho = w & 15;
    return 32 * (t >> 1) + 8 * (rho >> 2) + 4 * (t & 1) + (rho & 3);
  }
  const int T = w >> 5, rho = w & 31, g = rho >> 3;
  return 32 * T + 16 * (g >> 1) + 8 * ((rho >> 2) & 1) + 4 * (g & 1) + (rho & 3);
}

template <int FMT>
struct BigCfg {
  static constexpr int G = FMT == kNV ? 16 : 32;
  static constexpr int SB = kTBK / G;           // scale bytes per row per stage
  static constexpr int PLANES = SB / 4;         // scale words per row per stage
  static constexpr int WAVES = 4;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int MI = 8, NJ = 8;          // 16-row activation / weight tiles per wave
  static constexpr int ROWS = 512;              // staged rows: 256 activation, 256 weight
  static constexpr int CPW = ROWS / 16 / WAVES; // 1 KB code copies per wave per stage
  static constexpr int SDW = ROWS * PLANES;     // scale words per stage
  static constexpr int SPW = SDW / 64 / WAVES;  // 256-byte scale copies per wave per stage
  static constexpr int OPS = CPW + SPW;
  static constexpr int CODES = ROWS * 64;
  static constexpr int STAGE = CODES + SDW * 4;
  static constexpr int NBUF = 4;
  static constexpr int LDS = NBUF * STAGE;
  static_assert(LDS <= 160 * 1024, "LDS per CU");
  static_assert(SDW % (64 * WAVES) == 0, "scale copies split evenly over the waves");
  static_assert(3 * OPS <= 63, "the stage waits fit the vmcnt field");
};

// Scheduling groups of one MXFP4 stage (in order): for each weight tile j < 7, its 8
// MFMAs, the copies spread onto it and its LDS reads (plus the first scale read after
// tile 3); then each MFMA of tile 7 followed by one activation read; then the last
// four reads.  Masks: 0x008 MFMA, 0x020 vector memory read, 0x100 LDS read.
template <int OPS, int J>
__device__ __forceinline__ void big_mx_group() {
  constexpr int nc = [] {
    int n = 0;
    for (int u = 0; u < OPS; ++u) n += u * 7 / OPS == J;
    return n;
  }();
  __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  if constexpr (nc > 0) __builtin_amdgcn_sched_group_barrier(0x020, nc, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, J == 3 ? 2 : 1, 0);
}
template <int OPS, int... J>
__device__ __forceinline__ void big_mx_order(std::integer_sequence<int, J...>) {
  (big_mx_group<OPS, J>(), ...);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
}

// Scheduling groups of the NVFP4 k-step 7 (in order): the next stage's activation
// code and scale reads (12 LDS reads), then per weight tile u: its decode (8 VALU), the
// reads of its next-stage codes, its 4 MFMAs each followed by two VALU of the next
// stage's first activation decode, and the copies spread onto it.
template <int OPS, int U>
__device__ __forceinline__ void big_nv_group7() {
  constexpr int nc = [] {
    int n = 0;
    for (int q = 0; q < OPS; ++q) n += q * 4 / OPS == U;
    return n;
  }();
  __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
  }
  if constexpr (nc > 0) __builtin_amdgcn_sched_group_barrier(0x020, nc, 0);
}
template <int OPS, int... U>
__device__ __forceinline__ void big_nv_order7(std::integer_sequence<int, U...>) {
  __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
  (big_nv_group7<OPS, U>(), ...);
}

// Eight consecutive outputs out[m][n .. n + 7] (alpha applied): one 16-byte bf16 store
// (or two fp32 ones) when aligned and inside the matrix, else element by element.
__device__ __forceinline__ void big_store8(const GemmParams& p, int64_t m, int64_t n,
                                           const float (&x)[8], bool vec) {
  if (vec && n + 7 < p.N) {
    if (p.out_f32) {
      float* o = reinterpret_cast<float*>(p.out) + m * p.ldo + n;
      *reinterpret_cast<float4*>(o) = make_float4(x[0], x[1], x[2], x[3]);
      *reinterpret_cast<float4*>(o + 4) = make_float4(x[4], x[5], x[6], x[7]);
    } else {
      uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + m * p.ldo + n;
      *reinterpret_cast<uint4*>(o) = make_uint4(bf16_pack2(x[0], x[1]), bf16_pack2(x[2], x[3]),
                                                bf16_pack2(x[4], x[5]), bf16_pack2(x[6], x[7]));
    }
    return;
  }
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    if (n + v >= p.N) break;
    if (p.out_f32)
      reinterpret_cast<float*>(p.out)[m * p.ldo + n + v] = x[v];
    else
      reinterpret_cast<uint16_t*>(p.out)[m * p.ldo + n + v] = (uint16_t)(bf16_pack2(x[v], 0.0f) & 0xFFFFu);
  }
}

typedef float v16f __attribute__((ext_vector_type(16)));

template <int FMT>
__global__ __launch_bounds__(256, 1) void big_gemm(GemmParams p) {
  using C = BigCfg<FMT>;
  extern __shared__ __attribute__((aligned(16))) uint8_t tsm[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int64_t ntiles = (p.N + 255) / 256;
  const int64_t mb = (int64_t)blockIdx.x / ntiles;
  const int64_t nt = (int64_t)blockIdx.x - mb * ntiles;
  const int64_t row0 = mb * 256;
  const int64_t K = p.K, KB = K >> 1, KS = K / C::G;
  const int64_t nstages = K / kTBK;
  const float alpha = p.alpha;

  // global row of staged row rr: activations 0..255 in order, weights in pair order;
  // rows past the end are clamped to the last one (their outputs are not stored)
  auto src_row = [&](int rr) -> int64_t {
    if (rr < 256) {
      const int64_t m = row0 + rr;
      return m < p.M ? m : p.M - 1;
    }
    const int64_t n = nt * 256 + big_wperm<FMT>(rr - 256);
    return n < p.N ? n : p.N - 1;
  };
  // code copy q of this wave is copy c = wave + 4 q (staged rows 16 c ..): lane l
  // fetches row 16 c + l/4, column (l & 3) ^ tile_swz(l/4) into LDS slot l; scale copy
  // q (c = wave + 4 q) fills scale words 64 c + l.
  const uint8_t* dcode[C::CPW];
  const uint8_t* dscale[C::SPW];
#pragma unroll
  for (int q = 0; q < C::CPW; ++q) {
    const int rr = 16 * (wave + C::WAVES * q) + (lane >> 2);
    const int col = (lane & 3) ^ tile_swz(lane >> 2);
    dcode[q] = (rr < 256 ? p.a_codes : p.w_codes) + src_row(rr) * KB + col * 16;
  }
  // scale copy q (c = wave + 4 q) fills the 64 words of plane c / 8, 64-row block c % 8
  // of the stage: gathered from the rows (one word per row), or one contiguous 256-byte
  // piece of the stage-ordered scales ([64-row block][stage][plane][64 words])
  const bool stile = p.a_scales_t && p.w_scales_t;
  const int64_t sstride = stile ? C::PLANES * 256 : C::SB;   // bytes per stage
#pragma unroll
  for (int q = 0; q < C::SPW; ++q) {
    const int c = wave + C::WAVES * q;
    const int e = 64 * c + lane;
    const int plane = e / C::ROWS;
    if (stile) {
      const int blk = c % 8;   // 0..3 activation blocks, 4..7 weight blocks
      const int64_t rb = blk < 4 ? mb * 4 + blk : nt * 4 + blk - 4;
      dscale[q] = (blk < 4 ? p.a_scales_t : p.w_scales_t) + (rb * nstages * C::PLANES + plane) * 256 + lane * 4;
    } else {
      const int rr = tile_srow(e - plane * C::ROWS);
      dscale[q] = (rr < 256 ? p.a_scales : p.w_scales) + src_row(rr) * KS + plane * 4;
    }
  }
  // Stages past the last are issued too, as copies that all read one line (the
  // first weight bytes): every iteration then issues the same copies and waits with
  // the same counts, so the loop has no branches.  Their buffers are never read.
  auto issue_part = [&](int64_t t, int u) {
    uint8_t* buf = tsm + (int)(t % C::NBUF) * C::STAGE;
    const bool real = t < nstages;
    if (u < C::CPW) {
      const uint8_t* src = real ? dcode[u] + t * 64 : p.w_codes;
      tile_copy16(src, buf + (wave + C::WAVES * u) * 1024);
    } else {
      const uint8_t* src = real ? dscale[u - C::CPW] + t * sstride : p.w_scales;
      tile_copy4(src, buf + C::CODES + (wave + C::WAVES * (u - C::CPW)) * 256);
    }
  };
  // wait until all but the last AHEAD stages issued have landed, then barrier
  auto sync = [&](auto ahead_tag) {
    constexpr int AHEAD = decltype(ahead_tag)::value;
    __builtin_amdgcn_s_waitcnt(tile_vmcnt(AHEAD * C::OPS));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  const int r = lane & 15;
  const int gq = lane >> 4;
  const int gcol = (gq ^ tile_swz(r)) << 4;
  const int wrow0 = 256 + wn * 128;   // this wave's staged weight rows
  const int arow0 = wm * 128;         // ... and activation rows
  // scale words of plane pl, 64-row block starting at staged row b0, this lane's row r:
  // the 4 tiles' words in one 16-byte read
  auto rd_s4 = [&](const uint8_t* cur, int pl, int b0) {
    return *reinterpret_cast<const u32x4*>(cur + C::CODES + (pl * C::ROWS + b0 + 4 * r) * 4);
  };
  auto rd_w = [&](const uint8_t* cur, int j) {
    return *reinterpret_cast<const u32x4*>(cur + (wrow0 + 16 * j + r) * 64 + gcol);
  };
  auto rd_a = [&](const uint8_t* cur, int i) {
    return *reinterpret_cast<const u32x4*>(cur + (arow0 + 16 * i + r) * 64 + gcol);
  };

#pragma unroll
  for (int t = 0; t < C::NBUF; ++t)
#pragma unroll
    for (int u = 0; u < C::OPS; ++u) issue_part(t, u);
  using A1 = std::integral_constant<int, 1>;
  using A2 = std::integral_constant<int, 2>;
  using A3 = std::integral_constant<int, 3>;

  if constexpr (FMT == kMX) {
    v4f acc[C::NJ][C::MI];
#pragma unroll
    for (int j = 0; j < C::NJ; ++j)
#pragma unroll
      for (int i = 0; i < C::MI; ++i) acc[j][i] = v4f{0.f, 0.f, 0.f, 0.f};
    // The LDS operands of stage st + 1 are read while the MFMAs of stage st run, each
    // into the registers of an operand right after its last MFMA; stage st's buffer
    // is refilled (stage st + 4) from iteration st on, and iteration st ends by waiting
    // until stage st + 2 has landed.
    u32x4 wf[C::NJ], af[C::MI];
    uint32_t wsb[C::NJ], asb[C::MI];
    const int ssh = 8 * gq;
    auto rd_ws = [&](const uint8_t* cur, int k) {
      const u32x4 w4 = rd_s4(cur, 0, wrow0 + 64 * k);
      wsb[4 * k + 0] = w4.x >> ssh;
      wsb[4 * k + 1] = w4.y >> ssh;
      wsb[4 * k + 2] = w4.z >> ssh;
      wsb[4 * k + 3] = w4.w >> ssh;
    };
    auto rd_as = [&](const uint8_t* cur, int k) {
      const u32x4 a4 = rd_s4(cur, 0, arow0 + 64 * k);
      asb[4 * k + 0] = a4.x >> ssh;
      asb[4 * k + 1] = a4.y >> ssh;
      asb[4 * k + 2] = a4.z >> ssh;
      asb[4 * k + 3] = a4.w >> ssh;
    };
    auto mma = [&](int j, int i) {
      const v8i wop = {(int)wf[j].x, (int)wf[j].y, (int)wf[j].z, (int)wf[j].w, 0, 0, 0, 0};
      const v8i aop = {(int)af[i].x, (int)af[i].y, (int)af[i].z, (int)af[i].w, 0, 0, 0, 0};
      acc[j][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          wop, aop, acc[j][i], 4, 4, 0, (int)wsb[j], 0, (int)asb[i]);
    };
    sync(A3{});   // stage 0 landed
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) wf[j] = rd_w(tsm, j);
    rd_ws(tsm, 0);
    rd_ws(tsm, 1);
#pragma unroll
    for (int i = 0; i < C::MI; ++i) af[i] = rd_a(tsm, i);
    rd_as(tsm, 0);
    rd_as(tsm, 1);
    sync(A2{});   // stage 1 landed; every wave's reads of buffer 0 done
    for (int64_t st = 0; st < nstages; ++st) {
      // operands of stage st + 1 (after the last stage: a dummy stage, unused)
      const uint8_t* cur = tsm + (int)((st + 1) % C::NBUF) * C::STAGE;
#pragma unroll
      for (int j = 0; j < C::NJ - 1; ++j) {
#pragma unroll
        for (int i = 0; i < C::MI; ++i) mma(j, i);
#pragma unroll
        for (int u = 0; u < C::OPS; ++u)
          if (u * (C::NJ - 1) / C::OPS == j) issue_part(st + C::NBUF, u);
        wf[j] = rd_w(cur, j);
        if (j == 3) rd_ws(cur, 0);
      }
#pragma unroll
      for (int i = 0; i < C::MI; ++i) {
        mma(C::NJ - 1, i);
        af[i] = rd_a(cur, i);
      }
      wf[C::NJ - 1] = rd_w(cur, C::NJ - 1);
      rd_ws(cur, 1);
      rd_as(cur, 0);
      rd_as(cur, 1);
      // the order of the body: 8 MFMAs, then weight tile j's copies and LDS reads, for
      // each j; then each MFMA of the last weight tile followed by one activation read
      big_mx_order<C::OPS>(std::make_integer_sequence<int, C::NJ - 1>{});
      sync(A2{});   // stage st + 2 landed, st + 3 and st + 4 in flight
    }
    // the copies of the dummy stages must land before the workgroup ends
    __builtin_amdgcn_s_waitcnt(tile_vmcnt(0));

    // epilogue: lane holds out[m][n .. n+3] of weight tile j (n per the pair order) for
    // activation row m = 16 i + r; tiles 2 q and 2 q + 1 give 8 consecutive columns
    const bool vec = (p.ldo & 7) == 0 && ((reinterpret_cast<uintptr_t>(p.out) & 15) == 0);
#pragma unroll
    for (int i = 0; i < C::MI; ++i) {
      const int64_t m = row0 + arow0 + 16 * i + r;
      if (m >= p.M) continue;
#pragma unroll
      for (int q = 0; q < C::NJ / 2; ++q) {
        const int64_t n = nt * 256 + 32 * (4 * wn + q) + 8 * gq;
        float x[8];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          x[v] = acc[2 * q][i][v] * alpha;
          x[4 + v] = acc[2 * q + 1][i][v] * alpha;
        }
        big_store8(p, m, n, x, vec);
      }
    }
  } else {
    // NVFP4 on 32x32x16 fp16 MFMAs: wave tile = 4 weight x 4 activation tiles of 32
    // rows (lane row rho = lane % 32).  Lane half h = lane / 32 holds elements [64 h,
    // 64 h + 64) of the stage (16-byte columns 2 h and 2 h + 1 of its row); k-step s =
    // 0..7 uses its elements 64 h + 8 s .. + 8, i.e. block 4 h + s / 2, the same k slots
    // for both operands.  The activation tiles of k-step s + 1 are decoded while the
    // MFMAs of k-step s run, each weight tile right before its 4 MFMAs.  K-step 7 of
    // stage st starts with a barrier after which stage st + 1 has landed and every wave
    // has finished reading stage st (whose buffer then takes stage st + 4); its MFMAs
    // run while stage st + 1's operands are read and its first activation k-step decoded.
    constexpr int T4 = 4;
    v16f acc2[T4][T4];
#pragma unroll
    for (int u = 0; u < T4; ++u)
#pragma unroll
      for (int i = 0; i < T4; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc2[u][i][v] = 0.0f;
    const int rho = lane & 31, h = lane >> 5;
    const int c0 = ((2 * h) ^ tile_swz(rho & 15)) << 4;
    const int c1 = ((2 * h + 1) ^ tile_swz(rho & 15)) << 4;
    const int tsel = rho >> 4;   // word of a 64-row block's 4 that holds this lane's row
    u32x4 wf[T4][2], af[T4][2];
    f16x2 wsc[T4][2], asc[T4][2];
    auto rd_codes = [&](const uint8_t* cur, int row0_, u32x4 (&f)[T4][2], int u) {
      const uint8_t* rp = cur + (row0_ + 32 * u + rho) * 64;
      f[u][0] = *reinterpret_cast<const u32x4*>(rp + c0);
      f[u][1] = *reinterpret_cast<const u32x4*>(rp + c1);
    };
    // scale words of plane h for the 4 tiles of a side (two 64-row blocks, two tiles
    // each), as two fp16 pairs per tile (blocks 4 h, 4 h + 1 and 4 h + 2, 4 h + 3)
    auto rd_sc = [&](const uint8_t* cur, int row0_, f16x2 (&sc)[T4][2]) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const u32x4 w4 = rd_s4(cur, h, row0_ + 64 * k);
        const uint32_t e0 = tsel ? w4.y : w4.x, e1 = tsel ? w4.w : w4.z;
        sc[2 * k][0] = e4m3_pair_f16(e0);
        sc[2 * k][1] = e4m3_pair_f16(e0 >> 16);
        sc[2 * k + 1][0] = e4m3_pair_f16(e1);
        sc[2 * k + 1][1] = e4m3_pair_f16(e1 >> 16);
      }
    };
    auto dec = [&](const u32x4 (&f)[2], const f16x2 (&sc)[2], int s) {
      return decode8_f16(dword_of_v(f[s >> 2], s & 3), f16_bcast(sc[s >> 2], (s >> 1) & 1));
    };
    f16x8 ad[T4];
    sync(A3{});   // stage 0 landed
#pragma unroll
    for (int u = 0; u < T4; ++u) {
      rd_codes(tsm, arow0, af, u);
      rd_codes(tsm, wrow0, wf, u);
    }
    rd_sc(tsm, arow0, asc);
    rd_sc(tsm, wrow0, wsc);
#pragma unroll
    for (int i = 0; i < T4; ++i) ad[i] = dec(af[i], asc[i], 0);
    for (int64_t st = 0; st < nstages; ++st) {
#pragma unroll
      for (int s = 0; s < 7; ++s) {
        f16x8 an[T4];
#pragma unroll
        for (int u = 0; u < T4; ++u) {
          const f16x8 wd = dec(wf[u], wsc[u], s);
#pragma unroll
          for (int i = 0; i < T4; ++i)
            acc2[u][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wd, ad[i], acc2[u][i], 0, 0, 0);
          an[u] = dec(af[u], asc[u], s + 1);   // activation tile u of k-step s + 1
        }
#pragma unroll
        for (int i = 0; i < T4; ++i) ad[i] = an[i];
      }
      // k-steps 0..6: per weight tile, its decode (8 VALU), then its 4 MFMAs each
      // followed by two of the 8 VALU decoding an activation tile of the next k-step
#pragma unroll
      for (int g = 0; g < 7 * T4; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
#pragma unroll
        for (int i = 0; i < T4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        }
      }
      sync(A2{});   // stage st + 1 landed, st + 2 and st + 3 in flight
      // operands of stage st + 1 (after the last stage: a dummy stage, unused)
      const uint8_t* nxt = tsm + (int)((st + 1) % C::NBUF) * C::STAGE;
#pragma unroll
      for (int u = 0; u < T4; ++u) rd_codes(nxt, arow0, af, u);
      f16x2 wsn[T4][2], asn[T4][2];
      rd_sc(nxt, arow0, asn);
      rd_sc(nxt, wrow0, wsn);
      f16x8 an[T4];
#pragma unroll
      for (int u = 0; u < T4; ++u) {
        const f16x8 wd = dec(wf[u], wsc[u], 7);
        rd_codes(nxt, wrow0, wf, u);
#pragma unroll
        for (int i = 0; i < T4; ++i)
          acc2[u][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wd, ad[i], acc2[u][i], 0, 0, 0);
        an[u] = dec(af[u], asn[u], 0);
#pragma unroll
        for (int q = 0; q < C::OPS; ++q)
          if (q * T4 / C::OPS == u) issue_part(st + C::NBUF, q);
      }
      big_nv_order7<C::OPS>(std::make_integer_sequence<int, T4>{});
#pragma unroll
      for (int u = 0; u < T4; ++u) {
        ad[u] = an[u];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          asc[u][k] = asn[u][k];
          wsc[u][k] = wsn[u][k];
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(tile_vmcnt(0));
    // epilogue: lane holds, for weight tile u and activation tile i, out[m][n0 + 0..7]
    // (accumulators 0..7) and out[m][n0 + 16 + 0..7] (8..15), m = 32 i + rho, n0 = 32 u
    // + 8 h (the staging order above)
    const bool vec = (p.ldo & 7) == 0 && ((reinterpret_cast<uintptr_t>(p.out) & 15) == 0);
#pragma unroll
    for (int i = 0; i < T4; ++i) {
      const int64_t m = row0 + arow0 + 32 * i + rho;
      if (m >= p.M) continue;
#pragma unroll
      for (int u = 0; u < T4; ++u)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int64_t n = nt * 256 + wn * 128 + 32 * u + 16 * q + 8 * h;
          float x[8];
#pragma unroll
          for (int v = 0; v < 8; ++v) x[v] = acc2[u][i][8 * q + v] * alpha;
          big_store8(p, m, n, x, vec);
        }
    }
    return;
  }


}

// Block scales in the 256 x 256 tile's stage order: word (64-row block rb, stage t,
// plane pl, slot) at ((rb * nstages + t) * PLANES + pl) * 64 + slot holds the scale
// bytes [t SB + 4 pl, +4) of the row staged at position 64 rb + tile_srow(slot) --
// rows in order for the activations, in the pair order within each 256-row tile for
// the weights; rows past the end get zero words.
// One workgroup per (64-row block of one side, 8 stages): the rows' scale bytes of
// those stages are read whole into LDS (coalesced), then written out in stage order.
constexpr int kRelayStages = 8;
template <int FMT>
__global__ __launch_bounds__(256) void scale_relayout_kernel(
    const uint8_t* __restrict__ a_sc, int64_t M, const uint8_t* __restrict__ w_sc, int64_t N,
    int64_t K, uint8_t* __restrict__ a_t, uint8_t* __restrict__ w_t, int64_t a_blocks) {
  using C = BigCfg<FMT>;
  constexpr int RB = kRelayStages * C::SB;   // bytes of a row in one workgroup's stages
  __shared__ __attribute__((aligned(16))) uint8_t rows[64 * RB];
  const int64_t nst = K / kTBK, KS = K / C::G;
  const int64_t nchunk = (nst + kRelayStages - 1) / kRelayStages;
  const int64_t blk = (int64_t)blockIdx.x / nchunk;
  const int64_t t0 = ((int64_t)blockIdx.x - blk * nchunk) * kRelayStages;
  const int nt_ = (int)(nst - t0 < kRelayStages ? nst - t0 : kRelayStages);   // stages here
  const bool wside = blk >= a_blocks;
  const int64_t rb = wside ? blk - a_blocks : blk;
  const int64_t R = wside ? N : M;
  const uint8_t* sc = wside ? w_sc : a_sc;
  uint8_t* out = wside ? w_t : a_t;
  // load: words, row-major over the 64 staged rows of the block (a row's bytes of these
  // stages are contiguous)
  const int rwords = nt_ * C::SB / 4;
  for (int q = threadIdx.x; q < 64 * rwords; q += 256) {
    const int i = q / rwords, w = q - i * rwords;
    const int64_t sr = rb * 64 + i;   // staged row
    const int64_t row = wside ? (sr & ~(int64_t)255) + big_wperm<FMT>((int)(sr & 255)) : sr;
    const uint32_t v = row < R ? reinterpret_cast<const uint32_t*>(sc + row * KS + t0 * C::SB)[w] : 0u;
    reinterpret_cast<uint32_t*>(rows + i * RB)[w] = v;
  }
  __syncthreads();
  // write: word slot of stage t0 + tt, plane pl holds the bytes [tt SB + 4 pl, +4) of
  // the row staged at tile_srow(slot)
  const int words = nt_ * C::PLANES * 64;
  for (int e = threadIdx.x; e < words; e += 256) {
    const int slot = e & 63, pl = (e >> 6) % C::PLANES, tt = (e >> 6) / C::PLANES;
    const uint32_t v = *reinterpret_cast<const uint32_t*>(rows + tile_srow(slot) * RB + tt * C::SB + 4 * pl);
    reinterpret_cast<uint32_t*>(out)[((rb * nst + t0 + tt) * C::PLANES + pl) * 64 + slot] = v;
  }
}

template <int FMT>
hipError_t launch_big(const GemmParams& p, hipStream_t s, const char** name) {
  using C = BigCfg<FMT>;
  const int64_t grid = ((p.N + 255) / 256) * ((p.M + 255) / 256);
  *name = FMT == kNV ? "big_nvfp4_256" : "big_mxfp4_256";
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (p.K % kTBK != 0 || p.K <= 0 || p.mblk_expert || p.a_gather || p.fuse_swiglu)
    return hipErrorInvalidValue;
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&big_gemm<FMT>), C::LDS, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((big_gemm<FMT>), dim3((unsigned)grid), dim3(C::THREADS), C::LDS, s, p);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_relayout(const uint8_t* a_sc, int64_t M, const uint8_t* w_sc, int64_t N,
                           int64_t K, uint8_t* a_t, uint8_t* w_t, hipStream_t s) {
  const int64_t a_blocks = (M + 255) / 256 * 4, w_blocks = (N + 255) / 256 * 4;
  const int64_t nchunk = (K / kTBK + kRelayStages - 1) / kRelayStages;
  const int64_t grid = (a_blocks + w_blocks) * nchunk;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((scale_relayout_kernel<FMT>), dim3((unsigned)grid), dim3(256), 0, s, a_sc, M,
                     w_sc, N, K, a_t, w_t, a_blocks);
  return hipGetLastError();
}

// NVFP4 weight-tile width (128: two workgroups per CU)
constexpr int kNvTileN = 128;

}  // namespace

bool gemm_big_tile(int fmt, int64_t M, int64_t N, int64_t K) {
  (void)fmt;
  return M > 64 && K > 0 && K % kTBK == 0 && ((M + 255) / 256) * ((N + 255) / 256) >= 256;
}

size_t scale_relayout_bytes(int fmt, int64_t R, int64_t K) {
  return (size_t)((R + 255) / 256 * 256) * (size_t)(K / (fmt == kNV ? 16 : 32));
}

hipError_t launch_scale_relayout(int fmt, const uint8_t* a_scales, int64_t M,
                                 const uint8_t* w_scales, int64_t N, int64_t K, uint8_t* a_t,
                                 uint8_t* w_t, hipStream_t s) {
  if (K <= 0 || K % kTBK) return hipErrorInvalidValue;
  return fmt == kNV ? launch_relayout<kNV>(a_scales, M, w_scales, N, K, a_t, w_t, s)
                    : launch_relayout<kMX>(a_scales, M, w_scales, N, K, a_t, w_t, s);
}

hipError_t launch_gemm_tiled(int fmt, const GemmParams& p, hipStream_t s, const char** name) {
  // dense problems with enough 256 x 256 tiles to give every CU one: the 4-wave tile
  const bool big = !p.mblk_expert && !p.a_gather && !p.fuse_swiglu && gemm_big_tile(fmt, p.M, p.N, p.K);
  if (fmt == kNV) {
    if (p.fuse_swiglu) return launch_tile<kNV, 128, kNvTileN, true>(p, s, name);
    if (big) return launch_big<kNV>(p, s, name);
    return launch_tile<kNV, 128, kNvTileN, false>(p, s, name);
  }
  if (p.fuse_swiglu) return launch_tile<kMX, 128, 256, true>(p, s, name);
  if (big) return launch_big<kMX>(p, s, name);
  return launch_tile<kMX, 128, 256, false>(p, s, name);
}

}  // namespace fp4
