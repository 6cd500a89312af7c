// The scaled-MFMA matmul engine shared by FP8 W8A8 (all four scaling modes) and the MX
// formats of any element type (MXFP4, MXFP6, MXFP8, mixed between the two operands).
//
// out[m, n] = sum_k a_hat[m, k] * w_hat[n, k] on gfx950's scaled 32x32x64 MFMA, whose two
// operands each name their element type: e4m3 (8 bits), e2m3 or e3m2 (6 bits), e2m1
// (4 bits).  MX scales (e8m0 per 32 along K) are the instruction's block scales; the
// FP8 modes pass the unit scale and apply their fp32 scales outside it -- per-tensor and
// rowwise in the epilogue, block scales per 128-deep K block onto that block's partial
// sum.
//
// Operand layout of the MFMA (checked on the device lane by lane), lane l, h = l / 32,
// row l % 32:
//   e4m3: dwords 0-3 hold K [16 h, 16 h + 16), dwords 4-7 K [32 + 16 h, 48 + 16 h);
//   e2m3 / e3m2: dwords 0-5 hold K [32 h, 32 h + 32), element i at bits [6 i, 6 i + 6);
//   e2m1: dwords 0-3 hold K [32 h, 32 h + 32), element i in nibble i;
// the lane's scale byte covers K block h of the instruction's 64.  Result: lane l,
// register j = first-operand row 8 (j / 4) + 4 h + j % 4, second-operand row l % 32.
// Packed rows therefore stream into registers unchanged: e2m1 two per byte (low nibble
// first), e2m3 / e3m2 32 elements in 24 bytes, e4m3 one per byte.
#pragma once

#include "device.h"
#include "internal.h"

namespace fp4 {
namespace sg {

typedef float v16f __attribute__((ext_vector_type(16)));

// MFMA element-type codes of the scaled f8f6f4 instruction
constexpr int kE4M3 = 0, kE2M3 = 2, kE3M2 = 3, kE2M1 = 4;

template <int F>
struct Fmt {
  static constexpr int BITS = F == kE4M3 ? 8 : (F == kE2M1 ? 4 : 6);
  static constexpr int PIECES = BITS;          // 16-byte pieces per row per 128-deep stage
  static constexpr int RB = 16 * BITS;         // bytes per row per stage
};

// ---- operand fetch ----------------------------------------------------------------
// The lane's operand of the 64-deep step at k0 (a multiple of 64) of a packed row.
template <int F>
__device__ __forceinline__ v8i ld_lane(const uint8_t* row, int64_t k0, int h) {
  if constexpr (F == kE4M3) {
    const uint4 x0 = *reinterpret_cast<const uint4*>(row + k0 + 16 * h);
    const uint4 x1 = *reinterpret_cast<const uint4*>(row + k0 + 32 + 16 * h);
    return v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
  } else if constexpr (F == kE2M1) {
    const uint4 x = *reinterpret_cast<const uint4*>(row + (k0 / 32 + h) * 16);
    return v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
  } else {
    const uint2* p = reinterpret_cast<const uint2*>(row + (k0 / 32 + h) * 24);
    const uint2 x0 = p[0], x1 = p[1], x2 = p[2];
    return v8i{(int)x0.x, (int)x0.y, (int)x1.x, (int)x1.y, (int)x2.x, (int)x2.y, 0, 0};
  }
}

// Slot (16-byte unit) of piece p of row r inside an LDS region, and its inverse.  The
// maps make the per-chunk reads of 32 consecutive rows free of bank conflicts:
//   e4m3 (8 pieces): XOR swizzle (r >> 1) & 7;  e2m1 (4 pieces): (r >> 2) & 3;
//   6-bit (6 pieces): groups of 8 rows stored piece-major, odd groups rotated by 8 slots,
//   so that 16 lanes reading one piece of 16 consecutive rows cover all 16 slot classes.
template <int F>
__device__ __forceinline__ int slot_of(int r, int p) {
  if constexpr (F == kE4M3) return 8 * r + (p ^ ((r >> 1) & 7));
  else if constexpr (F == kE2M1) return 4 * r + (p ^ ((r >> 2) & 3));
  else {
    const int g = r >> 3;
    return 48 * g + (8 * p + (r & 7) + 8 * (g & 1)) % 48;
  }
}
template <int F>
__device__ __forceinline__ void piece_of(int s, int& r, int& p) {
  if constexpr (F == kE4M3) {
    r = s >> 3;
    p = (s & 7) ^ ((r >> 1) & 7);
  } else if constexpr (F == kE2M1) {
    r = s >> 2;
    p = (s & 3) ^ ((r >> 2) & 3);
  } else {
    const int g = s / 48, u = (s % 48 - 8 * (g & 1) + 48) % 48;
    p = u >> 3;
    r = 8 * g + (u & 7);
  }
}

// The lane's operand of 64-deep chunk c (0, 1) of a staged row r.
template <int F>
__device__ __forceinline__ v8i lds_lane(const uint8_t* region, int r, int c, int h) {
  auto piece = [&](int p) { return *reinterpret_cast<const uint4*>(region + 16 * slot_of<F>(r, p)); };
  if constexpr (F == kE4M3) {
    const uint4 a = piece(4 * c + h), b = piece(4 * c + 2 + h);
    return v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
  } else if constexpr (F == kE2M1) {
    const uint4 a = piece(2 * c + h);
    return v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  } else {
    // 24 bytes at 24 (2 c + h): pieces 3 c and the low half of 3 c + 1 (h = 0), or the
    // high half of 3 c + 1 and piece 3 c + 2 (h = 1)
    const uint4 a = piece(3 * c + h), b = piece(3 * c + 1 + h);
    if (h == 0) return v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, 0, 0};
    return v8i{(int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0};
  }
}

// scale operands are passed as run-time values (a compile-time constant scale operand is
// read as an f32 inline constant by this compiler)
template <int FW, int FA>
__device__ __forceinline__ v16f mfma(const v8i& w, const v8i& a, const v16f& c, int ws, int as) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w, a, c, FW, FA, 0, ws, 0, as);
}

// epilogue of one 32 x 32 block held by a lane: weight rows n0 + 8 q + 4 h + v (q, v <
// 4), activation row m; ROW mode scales by a_s[m] * w_s[n], the others by fa
template <int MODE>
__device__ __forceinline__ void store_block(const Fp8GemmParams& p, const v16f& acc, int64_t m,
                                            int64_t n0, int h, float fa) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t n = n0 + 8 * q + 4 * h;
    float x[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float f = fa;
      if (MODE == kF8_ROW) f = fa * p.w_s[n + v < p.N ? n + v : p.N - 1];
      x[v] = acc[4 * q + v] * f;
    }
    const bool vec = n + 3 < p.N && (p.ldo & 3) == 0 &&
                     (reinterpret_cast<uintptr_t>(p.out) & (p.out_f32 ? 15 : 7)) == 0;
    if (vec) {
      if (p.out_f32)
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + m * p.ldo + n) =
            make_float4(x[0], x[1], x[2], x[3]);
      else
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + m * p.ldo + n) =
            make_uint2(bf16_pack2(x[0], x[1]), bf16_pack2(x[2], x[3]));
      continue;
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if (n + v >= p.N) continue;
      if (p.out_f32)
        reinterpret_cast<float*>(p.out)[m * p.ldo + n + v] = x[v];
      else
        reinterpret_cast<uint16_t*>(p.out)[m * p.ldo + n + v] = f32_to_bf16_rne(x[v]);
    }
  }
}

// global -> LDS copies (the address of the LDS destination goes in M0): 16 bytes or 4
// bytes per lane
#define FP4_SG_LDS(p) ((__attribute__((address_space(3))) void*)(p))
__device__ __forceinline__ void copy16(const void* g, uint8_t* lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)FP4_SG_LDS(lds));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(m0v), "v"(g) : "memory", "m0");
}
__device__ __forceinline__ void copy4(const void* g, uint8_t* lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)FP4_SG_LDS(lds));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :: "s"(m0v), "v"(g) : "memory", "m0");
}
constexpr int vmcnt_enc(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

// ---- few activation rows (decode): one workgroup = 32 NW weight rows x 32 activation
// rows, its 4 waves splitting K by 128-deep blocks (wave w takes blocks w, w + 4, ...).
// Each wave stages its blocks (the activation rows and its NW 32-row weight tiles)
// through its own two LDS buffers with global_load_lds copies of whole cache lines (8
// rows x 128 bytes, or 16 x 64, per kilobyte), the next block in flight while the
// current one multiplies; no barrier until the partial sums are added through LDS in
// wave order (bitwise reproducible).  Weights are read once per 32 activation rows;
// each staged activation block serves NW weight tiles.
constexpr int kRowsWaves = 4;

template <int FA, int FW, int NW>
struct RowsCfg {
  static constexpr int ASLOTS = 32 * Fmt<FA>::PIECES;     // 16-byte slots of one block
  static constexpr int WSLOTS = 32 * NW * Fmt<FW>::PIECES;
  static constexpr int NCA = ASLOTS / 64, NCW = WSLOTS / 64;   // 1 KB copies
  static constexpr int SW = NW == 1 ? 256 : 512;               // MX scale words
  static constexpr int BUF = 16 * (ASLOTS + WSLOTS) + SW;
  static constexpr int RED = (kRowsWaves - 1) * NW * 64 * 64;  // partial sums (v16f)
  static constexpr int LDS = kRowsWaves * 2 * BUF + RED;
  static_assert(ASLOTS % 64 == 0 && WSLOTS % 64 == 0, "whole 1 KB copies");
  static_assert(NW == 1 || NW == 2, "one or two weight tiles per wave");
};

template <int MODE, int FA, int FW, int NW>
__global__ __launch_bounds__(64 * kRowsWaves) void rows_kernel(Fp8GemmParams p) {
  using C = RowsCfg<FA, FW, NW>;
  constexpr bool MX = MODE == kF8_MX;
  constexpr int OPS = C::NCA + C::NCW + (MX ? NW : 0);       // copies per block (all rows)
  constexpr int WR = 32 * NW;                                // weight rows per workgroup
  extern __shared__ __attribute__((aligned(16))) uint8_t rsm[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t ntiles = (p.N + WR - 1) / WR;
  const int64_t mb = (int64_t)blockIdx.x / ntiles;
  const int64_t nt = (int64_t)blockIdx.x - mb * ntiles;
  const int r = lane & 31, h = lane >> 5;
  const int64_t m = mb * 32 + r;
  const int64_t mc = m < p.M ? m : p.M - 1;
  const int64_t a_rowb = p.K * Fmt<FA>::BITS / 8, w_rowb = p.K * Fmt<FW>::BITS / 8;
  const int64_t nkb = p.K / 128;
  const int one = p.unit_scale;
  // the weight block of these rows (BLOCK): 128-row blocks hold whole 32 NW-row tiles
  const int64_t wblk = (nt * WR) / 128;
  uint8_t* mybuf = rsm + wave * 2 * C::BUF;
  // the lane's copy sources: slot 64 c + lane of the activation / weight region
  const uint8_t* asrc[C::NCA];
  const uint8_t* wsrc[C::NCW];
#pragma unroll
  for (int c = 0; c < C::NCA; ++c) {
    int rr, pc;
    piece_of<FA>(64 * c + lane, rr, pc);
    const int64_t mm = mb * 32 + rr < p.M ? mb * 32 + rr : p.M - 1;
    asrc[c] = p.a_codes + mm * a_rowb + 16 * pc;
  }
#pragma unroll
  for (int c = 0; c < C::NCW; ++c) {
    int rr, pc;
    piece_of<FW>(64 * c + lane, rr, pc);
    const int64_t nn = nt * WR + rr < p.N ? nt * WR + rr : p.N - 1;
    wsrc[c] = p.w_codes + nn * w_rowb + 16 * pc;
  }
  // MX scale words of a block.  One tile: lanes 0-31 copy the weight rows' e8m0 word,
  // lanes 32-63 the activation rows' (words 0-31 weights, 32-63 activations).  Two
  // tiles: one copy of the 64 weight rows' words, one of the 32 activation rows'
  // (lanes 32-63 repeat them into padding): words 0-63 weights, 64-95 activations.
  const uint8_t* ssrc = nullptr;
  const uint8_t* ssrc2 = nullptr;
  if (MX) {
    if (NW == 1) {
      const int64_t nc = nt * 32 + r < p.N ? nt * 32 + r : p.N - 1;
      ssrc = h == 0 ? p.w_mx + nc * (p.K / 32) : p.a_mx + mc * (p.K / 32);
    } else {
      const int64_t nl = nt * WR + lane < p.N ? nt * WR + lane : p.N - 1;
      ssrc = p.w_mx + nl * (p.K / 32);
      ssrc2 = p.a_mx + mc * (p.K / 32);
    }
  }
  constexpr int AW = NW == 1 ? 128 : 256;   // byte offset of the activation words
  // activation copies that hold rows that exist (e4m3 / e2m1 copies hold whole rows: 8
  // or 16 per kilobyte); the lanes of absent rows read stale LDS, which only reaches
  // output rows that are not stored
  constexpr int RPC = FA == kE4M3 ? 8 : (FA == kE2M1 ? 16 : 0);
  const int64_t mrows = p.M - mb * 32 < 32 ? p.M - mb * 32 : 32;
  const int nca = RPC ? (int)((mrows + RPC - 1) / RPC) : C::NCA;   // uniform
  auto issue = [&](int64_t kb, int slot) {
    uint8_t* buf = mybuf + slot * C::BUF;
#pragma unroll
    for (int c = 0; c < C::NCA; ++c)
      if (c < nca) copy16(asrc[c] + kb * Fmt<FA>::RB, buf + c * 1024);
#pragma unroll
    for (int c = 0; c < C::NCW; ++c) copy16(wsrc[c] + kb * Fmt<FW>::RB, buf + 16 * C::ASLOTS + c * 1024);
    if (MX) {
      copy4(ssrc + kb * 4, buf + 16 * (C::ASLOTS + C::WSLOTS));
      if (NW == 2) copy4(ssrc2 + kb * 4, buf + 16 * (C::ASLOTS + C::WSLOTS) + AW);
    }
  };
  v16f acc[NW];
#pragma unroll
  for (int j = 0; j < NW; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[j][v] = 0.0f;
  int64_t kb = wave;
  if (kb < nkb) issue(kb, 0);
  for (int slot = 0; kb < nkb; kb += kRowsWaves, slot ^= 1) {
    const int64_t nxt = kb + kRowsWaves;
    // this wave's LDS reads of the other buffer are done before it is refilled
    __builtin_amdgcn_s_waitcnt(0xC07F);
    if (nxt < nkb) {
      issue(nxt, slot ^ 1);
      // block kb landed: at most the next block's copies outstanding
      if (nca == C::NCA) __builtin_amdgcn_s_waitcnt(vmcnt_enc(OPS));
      else if (nca == 1) __builtin_amdgcn_s_waitcnt(vmcnt_enc(OPS - C::NCA + 1));
      else if (nca == 2) __builtin_amdgcn_s_waitcnt(vmcnt_enc(OPS - C::NCA + 2));
      else __builtin_amdgcn_s_waitcnt(vmcnt_enc(OPS - C::NCA + 3));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_enc(0));
    }
    asm volatile("" ::: "memory");
    const uint8_t* buf = mybuf + slot * C::BUF;
    const v8i a0 = lds_lane<FA>(buf, r, 0, h), a1 = lds_lane<FA>(buf, r, 1, h);
    int as0 = one, as1 = one;
    const uint8_t* sw = buf + 16 * (C::ASLOTS + C::WSLOTS);
    if (MX) {
      const uint32_t asw = *reinterpret_cast<const uint32_t*>(sw + AW + 4 * r);
      as0 = (int)((asw >> (8 * h)) & 0xFFu);
      as1 = (int)((asw >> (8 * (2 + h))) & 0xFFu);
    }
    // this block's scales (BLOCK: activation row m, the weight block of the tiles)
    const float bf = MODE == kF8_BLOCK ? p.a_s[mc * nkb + kb] * p.w_s[wblk * nkb + kb] : 0.0f;
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      const uint8_t* wreg = buf + 16 * C::ASLOTS;
      const v8i w0 = lds_lane<FW>(wreg, 32 * j + r, 0, h), w1 = lds_lane<FW>(wreg, 32 * j + r, 1, h);
      int ws0 = one, ws1 = one;
      if (MX) {
        const uint32_t wsw = *reinterpret_cast<const uint32_t*>(sw + 4 * (32 * j + r));
        ws0 = (int)((wsw >> (8 * h)) & 0xFFu);
        ws1 = (int)((wsw >> (8 * (2 + h))) & 0xFFu);
      }
      if (MODE == kF8_BLOCK) {
        v16f t;
#pragma unroll
        for (int v = 0; v < 16; ++v) t[v] = 0.0f;
        t = mfma<FW, FA>(w0, a0, t, ws0, as0);
        t = mfma<FW, FA>(w1, a1, t, ws1, as1);
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[j][v] += t[v] * bf;
      } else {
        acc[j] = mfma<FW, FA>(w0, a0, acc[j], ws0, as0);
        acc[j] = mfma<FW, FA>(w1, a1, acc[j], ws1, as1);
      }
    }
  }
  v16f* red = reinterpret_cast<v16f*>(rsm + kRowsWaves * 2 * C::BUF);
  if (wave > 0) {
#pragma unroll
    for (int j = 0; j < NW; ++j) red[((wave - 1) * NW + j) * 64 + lane] = acc[j];
  }
  __syncthreads();
  if (wave != 0 || m >= p.M) return;
  const float fa = MODE == kF8_ROW ? p.a_s[m] : p.alpha;
#pragma unroll
  for (int j = 0; j < NW; ++j) {
#pragma unroll
    for (int wv = 0; wv < kRowsWaves - 1; ++wv) {
      const v16f o = red[(wv * NW + j) * 64 + lane];
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][v] += o[v];
    }
    store_block<MODE>(p, acc[j], m, nt * WR + 32 * j, h, fa);
  }
}

// ---- many activation rows (prefill): LDS-tiled -------------------------------------
// A workgroup of 8 waves owns 256 weight rows and BM = 128 activation rows; wave (wn,
// wm), wn < 2, wm < 4, computes 128 weight rows x 32 activation rows as four 32 x 32
// blocks.  K advances in stages of 128; a stage holds each row's packed codes (RB bytes
// = 16 pieces of 16 bytes per 8 bits of element) at the slots of slot_of, and for MX
// the rows' e8m0 words.  Everything goes global -> LDS with global_load_lds copies of
// 1 KB (64 lanes x 16 bytes), NBUF stages resident.  A stage is two 64-deep chunks:
// the wave reads chunk 1 while chunk 0 multiplies, passes one barrier (after which the
// stage's buffer is refilled with stage st + NBUF), then reads chunk 0 of the next
// stage while chunk 1 multiplies.
template <int FA, int FW>
struct TileCfg {
  static constexpr int BM = 128, BN = 256, WAVES = 8, WM = 4, NA = 4;
  static constexpr int ASLOTS = BM * Fmt<FA>::PIECES;           // 16-byte slots per stage
  static constexpr int WSLOTS = BN * Fmt<FW>::PIECES;
  static constexpr int CODES = 16 * (ASLOTS + WSLOTS);
  static constexpr int NCOP = (ASLOTS + WSLOTS) / 64;          // 1 KB copies per stage
  static constexpr int CPW_LO = NCOP / WAVES;                    // copies of waves >= XW
  static constexpr int XW = NCOP % WAVES;                        // waves < XW do one more
  static constexpr int CPW = CPW_LO + (XW ? 1 : 0);
  static constexpr int ROWS = BM + BN;
  static constexpr int SCALES = 256 * WAVES;                     // e8m0 words (MX): one
                                                                 // 256-byte copy per wave
  static constexpr int STAGE = CODES + SCALES;
  static constexpr int NBUF = 4 * STAGE <= 160 * 1024 ? 4 : (3 * STAGE <= 160 * 1024 ? 3 : 2);
  static constexpr int LDS = NBUF * STAGE;
  static_assert((ASLOTS % 64) == 0 && (WSLOTS % 64) == 0, "1 KB copies per region");
  static_assert(ROWS % 64 == 0 && ROWS / 64 <= WAVES, "one scale copy per wave");
  static_assert(LDS <= 160 * 1024, "LDS per CU");
};

// staged row of scale-word slot s: activation rows in order, weight rows ordered so that
// lane r of weight half wn reads the words of rows wn * 128 + 32 j + r (j < 4) as one
// 16-byte load
__device__ __forceinline__ int scale_row(int s) {
  constexpr int BM = 128;
  if (s < BM) return s;
  const int w = s - BM, g = w / 128, t = w % 128;
  return BM + g * 128 + 32 * (t % 4) + t / 4;
}


template <int MODE, int FA, int FW>
__global__ __launch_bounds__(512, 1) void tile_kernel(Fp8GemmParams p) {
  using C = TileCfg<FA, FW>;
  constexpr int BM = C::BM, NA = C::NA;
  constexpr bool MX = MODE == kF8_MX;
  // copy operations per stage of a wave issuing CPW_LO + 1 (waves < XW) or CPW_LO copies
  constexpr int OPS_HI = C::CPW_LO + 1 + (MX ? 1 : 0), OPS_LO = C::CPW_LO + (MX ? 1 : 0);
  extern __shared__ __attribute__((aligned(16))) uint8_t fsm[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % C::WM, wn = wave / C::WM;
  const int64_t ntiles = (p.N + C::BN - 1) / C::BN;
  const int64_t mb = (int64_t)blockIdx.x / ntiles;
  const int64_t nt = (int64_t)blockIdx.x - mb * ntiles;
  const int64_t row0 = mb * BM, K = p.K, nst = K / 128;
  const int64_t a_rowb = K * Fmt<FA>::BITS / 8, w_rowb = K * Fmt<FW>::BITS / 8;
  const bool more = wave < C::XW;
  // the lane's source of copy q (slots 64 (wave + 8 q) + lane of the stage) and how far
  // it moves per stage (the row bytes per stage of its operand)
  const uint8_t* dcode[C::CPW];
  int dstep[C::CPW];
#pragma unroll
  for (int q = 0; q < C::CPW; ++q) {
    const int g = wave + C::WAVES * q;
    int s = 64 * g + lane;
    if (s >= C::ASLOTS + C::WSLOTS) s = 0;            // (a copy this wave does not issue)
    int r, pc;
    if (s < C::ASLOTS) {
      piece_of<FA>(s, r, pc);
      const int64_t m = row0 + r;
      dcode[q] = p.a_codes + (m < p.M ? m : p.M - 1) * a_rowb + 16 * pc;
      dstep[q] = Fmt<FA>::RB;
    } else {
      piece_of<FW>(s - C::ASLOTS, r, pc);
      const int64_t n = nt * C::BN + r;
      dcode[q] = p.w_codes + (n < p.N ? n : p.N - 1) * w_rowb + 16 * pc;
      dstep[q] = Fmt<FW>::RB;
    }
  }
  const uint8_t* dscale = p.a_codes;
  if (MX) {
    int w = 64 * wave + lane;
    if (w >= C::ROWS) w = C::ROWS - 1;
    const int x = scale_row(w);
    if (x < BM) {
      const int64_t m = row0 + x;
      dscale = p.a_mx + (m < p.M ? m : p.M - 1) * (K / 32);
    } else {
      const int64_t n = nt * C::BN + (x - BM);
      dscale = p.w_mx + (n < p.N ? n : p.N - 1) * (K / 32);
    }
  }
  auto issue = [&](int64_t t) {
    uint8_t* buf = fsm + (int)(t % C::NBUF) * C::STAGE;
#pragma unroll
    for (int q = 0; q < C::CPW_LO; ++q)
      copy16(dcode[q] + t * dstep[q], buf + (wave + C::WAVES * q) * 1024);
    if (C::XW && more)
      copy16(dcode[C::CPW - 1] + t * dstep[C::CPW - 1], buf + (wave + C::WAVES * C::CPW_LO) * 1024);
    if (MX) copy4(dscale + t * 4, buf + C::CODES + wave * 256);
  };
  // wait until the oldest stage in flight has landed, `ahead` later stages may stay in
  // flight, then a workgroup barrier
  auto sync = [&](int64_t ahead) {
    if (more) {
      if (ahead >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_enc(2 * OPS_HI));
      else if (ahead >= 1) __builtin_amdgcn_s_waitcnt(vmcnt_enc(OPS_HI));
      else __builtin_amdgcn_s_waitcnt(vmcnt_enc(0));
    } else {
      if (ahead >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_enc(2 * OPS_LO));
      else if (ahead >= 1) __builtin_amdgcn_s_waitcnt(vmcnt_enc(OPS_LO));
      else __builtin_amdgcn_s_waitcnt(vmcnt_enc(0));
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  const int r = lane & 31, h = lane >> 5;
  const int wrow0 = wn * 128, arow = wm * 32 + r;
  const int wsc_off = C::CODES + (BM + wrow0 + 4 * r) * 4;
  const int asc_off = C::CODES + arow * 4;
  const int one = p.unit_scale;
  const int64_t nkb = nst;
  // BLOCK: the wave's 128 weight rows are one weight block
  const int64_t nwb = (p.N + 127) / 128;
  const int64_t wblk = (nt * C::BN + wrow0) / 128;
  const int64_t wblk_c = wblk < nwb ? wblk : nwb - 1;
  const int64_t am = row0 + arow < p.M ? row0 + arow : p.M - 1;

  v16f acc[NA];
#pragma unroll
  for (int j = 0; j < NA; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[j][v] = 0.0f;

  v8i wq[2][NA], aq[2];                       // [chunk]
  uint32_t wsw[NA] = {}, wsn[NA] = {}, asw = 0, asn = 0;
  auto rd_chunk = [&](const uint8_t* cur, int c) {
#pragma unroll
    for (int j = 0; j < NA; ++j) wq[c][j] = lds_lane<FW>(cur + 16 * C::ASLOTS, wrow0 + 32 * j + r, c, h);
    aq[c] = lds_lane<FA>(cur, arow, c, h);
  };
  auto rd_scales = [&](const uint8_t* cur) {   // MX: the rows' e8m0 words of a stage
    if (!MX) return;
    const u32x4 w4 = *reinterpret_cast<const u32x4*>(cur + wsc_off);
    wsn[0] = w4.x; wsn[1] = w4.y; wsn[2] = w4.z; wsn[3] = w4.w;
    asn = *reinterpret_cast<const uint32_t*>(cur + asc_off);
  };
  // BLOCK: this stage's factor a_s[m, kb] * w_s[block, kb]
  float bf = 0.0f, bfn = 0.0f;
  auto ld_blockf = [&](int64_t kb) {
    if (MODE == kF8_BLOCK) bfn = p.a_s[am * nkb + kb] * p.w_s[wblk_c * nkb + kb];
  };
  v16f t[NA];
  auto mma_chunk = [&](int c) {
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const int ws = MX ? (int)((wsw[j] >> (8 * (2 * c + h))) & 0xFFu) : one;
      const int as = MX ? (int)((asw >> (8 * (2 * c + h))) & 0xFFu) : one;
      if (MODE == kF8_BLOCK) {
        if (c == 0) {
#pragma unroll
          for (int v = 0; v < 16; ++v) t[j][v] = 0.0f;
        }
        t[j] = mfma<FW, FA>(wq[c][j], aq[c], t[j], ws, as);
      } else {
        acc[j] = mfma<FW, FA>(wq[c][j], aq[c], acc[j], ws, as);
      }
    }
  };

#pragma unroll
  for (int s = 0; s < C::NBUF; ++s)
    if (s < nst) issue(s);
  sync(nst - 1 < C::NBUF - 1 ? nst - 1 : C::NBUF - 1);   // stage 0 landed
  rd_chunk(fsm, 0);
  rd_scales(fsm);
  ld_blockf(0);
  for (int64_t st = 0; st < nst; ++st) {
    const uint8_t* cur = fsm + (int)(st % C::NBUF) * C::STAGE;
#pragma unroll
    for (int j = 0; j < NA; ++j) wsw[j] = wsn[j];
    asw = asn;
    bf = bfn;
    rd_chunk(cur, 1);
    __builtin_amdgcn_sched_barrier(0);
    mma_chunk(0);
    __builtin_amdgcn_sched_barrier(0);
    if (st + 1 < nst) {
      // stage st + 1 landed (later stages may stay in flight); every wave done with st
      const int64_t last = st + C::NBUF - 1 < nst ? st + C::NBUF - 1 : nst - 1;
      sync(last - (st + 1));
      if (st + C::NBUF < nst) issue(st + C::NBUF);
      const uint8_t* nxt = fsm + (int)((st + 1) % C::NBUF) * C::STAGE;
      rd_chunk(nxt, 0);
      rd_scales(nxt);
      ld_blockf(st + 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    mma_chunk(1);
    if (MODE == kF8_BLOCK) {
#pragma unroll
      for (int j = 0; j < NA; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[j][v] += t[j][v] * bf;
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  const int64_t m = row0 + arow;
  if (m >= p.M) return;
  const float fa = MODE == kF8_ROW ? p.a_s[m] : (MODE == kF8_BLOCK ? 1.0f : p.alpha);
#pragma unroll
  for (int j = 0; j < NA; ++j) store_block<MODE>(p, acc[j], m, nt * C::BN + wrow0 + 32 * j, h, fa);
}

template <int MODE, int FA, int FW, int NW>
hipError_t launch_rows(const Fp8GemmParams& p, hipStream_t s) {
  const int64_t grid = ((p.N + 32 * NW - 1) / (32 * NW)) * ((p.M + 31) / 32);
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  constexpr int lds = RowsCfg<FA, FW, NW>::LDS;
  static std::atomic<uint64_t> rows_lds{0};
  hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&rows_kernel<MODE, FA, FW, NW>), lds,
                                    rows_lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((rows_kernel<MODE, FA, FW, NW>), dim3((unsigned)grid), dim3(64 * kRowsWaves), lds,
                     s, p);
  return hipGetLastError();
}

template <int MODE, int FA, int FW>
hipError_t launch(const Fp8GemmParams& p, hipStream_t s, const char** name, const char* rows_name,
                  const char* tile_name) {
  if (p.M <= 32) {
    *name = rows_name;
    // two weight tiles per wave halve the activation staging per weight byte, and the
    // workgroups: measured faster for MX operands above 16 rows (M = 32: MXFP8 17.7 ->
    // 16.6 us, FP4 weights x FP8 activations 13.6 -> 12.8 us at N = 14336, K = 4096),
    // slower with fewer rows (fewer workgroups than CUs) and no faster for rowwise FP8
    if (MODE == kF8_MX && p.M > 16) return launch_rows<MODE, FA, FW, 2>(p, s);
    return launch_rows<MODE, FA, FW, 1>(p, s);
  }
  using C = TileCfg<FA, FW>;
  *name = tile_name;
  const int64_t grid = ((p.N + C::BN - 1) / C::BN) * ((p.M + C::BM - 1) / C::BM);
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&tile_kernel<MODE, FA, FW>), C::LDS,
                                    lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((tile_kernel<MODE, FA, FW>), dim3((unsigned)grid), dim3(512), C::LDS, s, p);
  return hipGetLastError();
}

}  // namespace sg
}  // namespace fp4
