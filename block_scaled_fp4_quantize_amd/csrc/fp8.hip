// MXFP8 and FP8 W8A8 on gfx950: quantization and matmul with e4m3 operands.
//
// What is computed ("vLLM per-format kernel capability matrix derived from source"):
//  * MXFP8 -- e4m3 elements with an e8m0 scale per 32 along K (the MX group size of its
//    group-size note; the MXFP8 section: the one MX format with a native path on gfx95);
//  * FP8 W8A8 with one of the three scaling modes of its "FP8, THREE SCALING MODES"
//    section: per-tensor; rowwise (per token for activations, per output channel for
//    weights, dynamic); block (1 x 128 activation blocks, 128 x 128 weight blocks).
// out[m, n] = sum_k a_hat[m, k] * w_hat[n, k], each operand dequantized with its own
// scales (the emulation definition of THE EMULATION COLUMN), accumulated in fp32.
//
// All four modes run on gfx950's scaled 32x32x64 MFMA with e4m3 operands: MXFP8 passes
// its e8m0 bytes as the instruction's block scales; the other modes pass the unit scale
// (code 127) and apply their fp32 scales outside the MFMA -- per-tensor and rowwise in
// the epilogue, block scales per 128-deep K block onto that block's partial sum.
//
// Operand layout of the e4m3 MFMA (checked on the device lane by lane): lane l holds
// row l % 32; with h = l / 32, its dwords 0-3 are K [16 h, 16 h + 16) and dwords 4-7
// K [32 + 16 h, 48 + 16 h) of the instruction's 64; its scale byte covers K block h.
// Result: lane l, register j = weight row 8 (j / 4) + 4 h + j % 4, activation row l % 32.
// The e4m3 dot products inside the MFMA are not exact fp32 sums (the device showed up
// to 1.4e-4 of the sum of |products| per instruction), well inside the GEMM tolerance.
#include "device.h"
#include "internal.h"

#pragma clang fp contract(off)

namespace fp4 {

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));

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

// ---- matmul: shared pieces -----------------------------------------------------------
// scale operand of the MFMA: MX passes the lane's e8m0 byte, the others the unit code
// 127 -- as a run-time value (a compile-time constant scale operand is read as an f32
// inline constant by this compiler)
template <int MODE>
__device__ __forceinline__ v16f fp8_mfma(const v8i& w, const v8i& a, const v16f& c, int ws, int as) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w, a, c, 0, 0, 0, ws, 0, as);
}

// epilogue of one 32 x 32 block held by a lane: weight rows n0 + 8 q + 4 h + v (q, v <
// 4), activation row m; ROW mode scales by a_s[m] * w_s[n], the others by alpha
template <int MODE>
__device__ __forceinline__ void fp8_store_block(const Fp8GemmParams& p, const v16f& acc, int64_t m,
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

// ---- matmul for few activation rows (decode): one workgroup = 32 weight rows x 32
// activation rows, its 4 waves splitting K by 128-deep blocks (kb = wave, wave + 4,
// ...), operands loaded straight from global memory, partial sums added through LDS in
// wave order (bitwise reproducible).  Weights are read once per 32 activation rows.
template <int MODE>
__global__ __launch_bounds__(256) void fp8_rows_kernel(Fp8GemmParams p) {
  __shared__ v16f red[3][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t ntiles = (p.N + 31) / 32;
  const int64_t mb = (int64_t)blockIdx.x / ntiles;
  const int64_t nt = (int64_t)blockIdx.x - mb * ntiles;
  const int r = lane & 31, h = lane >> 5;
  const int64_t n = nt * 32 + r, m = mb * 32 + r;
  const int64_t nc = n < p.N ? n : p.N - 1, mc = m < p.M ? m : p.M - 1;
  const uint8_t* wrow = p.w_codes + nc * p.K;
  const uint8_t* arow = p.a_codes + mc * p.K;
  const int64_t nkb = p.K / 128;
  const int one = p.unit_scale;
  // the weight block of these 32 rows (BLOCK): 128-row blocks hold whole 32-row tiles
  const int64_t wblk = (nt * 32) / 128;
  v16f acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  auto ld = [&](const uint8_t* row, int64_t k0) {   // the lane's operand of a 64-K step
    const uint4 x0 = *reinterpret_cast<const uint4*>(row + k0 + 16 * h);
    const uint4 x1 = *reinterpret_cast<const uint4*>(row + k0 + 32 + 16 * h);
    return v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
  };
  for (int64_t kb = wave; kb < nkb; kb += 4) {
    const int64_t k0 = kb * 128;
    const v8i w0 = ld(wrow, k0), w1 = ld(wrow, k0 + 64);
    const v8i a0 = ld(arow, k0), a1 = ld(arow, k0 + 64);
    int ws0 = one, ws1 = one, as0 = one, as1 = one;
    if (MODE == kF8_MX) {
      const uint32_t wsw = *reinterpret_cast<const uint32_t*>(p.w_mx + nc * (p.K / 32) + kb * 4);
      const uint32_t asw = *reinterpret_cast<const uint32_t*>(p.a_mx + mc * (p.K / 32) + kb * 4);
      ws0 = (int)((wsw >> (8 * h)) & 0xFFu);
      ws1 = (int)((wsw >> (8 * (2 + h))) & 0xFFu);
      as0 = (int)((asw >> (8 * h)) & 0xFFu);
      as1 = (int)((asw >> (8 * (2 + h))) & 0xFFu);
    }
    if (MODE == kF8_BLOCK) {
      v16f t;
#pragma unroll
      for (int v = 0; v < 16; ++v) t[v] = 0.0f;
      t = fp8_mfma<MODE>(w0, a0, t, ws0, as0);
      t = fp8_mfma<MODE>(w1, a1, t, ws1, as1);
      // this block's partial sum times its two scales (activation row m, weight block)
      const float f = p.a_s[mc * nkb + kb] * p.w_s[wblk * nkb + kb];
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[v] += t[v] * f;
    } else {
      acc = fp8_mfma<MODE>(w0, a0, acc, ws0, as0);
      acc = fp8_mfma<MODE>(w1, a1, acc, ws1, as1);
    }
  }
  if (wave > 0) red[wave - 1][lane] = acc;
  __syncthreads();
  if (wave != 0 || m >= p.M) return;
#pragma unroll
  for (int wv = 0; wv < 3; ++wv) {
    const v16f o = red[wv][lane];
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] += o[v];
  }
  const float fa = MODE == kF8_ROW ? p.a_s[m] : p.alpha;
  fp8_store_block<MODE>(p, acc, m, nt * 32, h, fa);
}

// ---- matmul for many activation rows (prefill): LDS-tiled ----------------------------
// A workgroup of 8 waves owns 256 weight rows and BM = 128 activation rows; wave (wn,
// wm), wn < 2, wm < 4, computes 128 weight rows x 32 activation rows as 32 x 32 blocks.
// K advances in stages of 128 (128 bytes of codes per row, 8 columns of 16 bytes,
// XOR-swizzled by (row >> 1) & 7 -- conflict-free for the lane pattern of the MFMA
// reads, measured on the device); the codes (and MXFP8's e8m0 words) go global -> LDS
// with global_load_lds copies, NBUF stages resident.  A stage is two 64-K chunks: the
// wave reads chunk 1 while chunk 0 multiplies, passes one barrier (after which the
// stage's buffer is refilled with stage st + NBUF), then reads chunk 0 of the next
// stage while chunk 1 multiplies.
template <int BM>
struct Fp8TileCfg {
  static constexpr int WAVES = 8, WM = 4, NA = 4;
  static constexpr int NB = BM / (32 * WM);           // 32-row activation blocks per wave
  static constexpr int ROWS = BM + 256;
  static constexpr int CODES = ROWS * 128;
  static constexpr int CCOP = ROWS / 8;                // 1 KB code copies per stage
  static constexpr int CPW = CCOP / WAVES;
  static constexpr int SCOP = ROWS / 64;               // 256-byte e8m0 copies (MXFP8)
  static constexpr int SPW = (SCOP + WAVES - 1) / WAVES;
  static constexpr int SCALES = WAVES * SPW * 256;
  static constexpr int STAGE = CODES + SCALES;
  static constexpr int NBUF = 4 * STAGE <= 160 * 1024 ? 4 : (3 * STAGE <= 160 * 1024 ? 3 : 2);
  static constexpr int LDS = NBUF * STAGE;
  static_assert(NB >= 1 && CCOP % WAVES == 0, "tile shape");
  static_assert(LDS <= 160 * 1024, "LDS per CU");
};

__device__ __forceinline__ int fp8_swz(int r) { return (r >> 1) & 7; }

template <int BM>
__device__ __forceinline__ int fp8_srow(int s) {   // staged row of scale-word slot s
  constexpr int NB = Fp8TileCfg<BM>::NB;
  if (s < BM) {
    const int g = s / (32 * NB), t = s % (32 * NB);
    return g * 32 * NB + 32 * (t % NB) + t / NB;
  }
  const int w = s - BM, g = w / 128, t = w % 128;
  return BM + g * 128 + 32 * (t % 4) + t / 4;
}

#define FP4_F8_LDS(p) ((__attribute__((address_space(3))) void*)(p))
__device__ __forceinline__ void f8_copy16(const void* g, uint8_t* lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)FP4_F8_LDS(lds));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(m0v), "v"(g) : "memory", "m0");
}
__device__ __forceinline__ void f8_copy4(const void* g, uint8_t* lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)FP4_F8_LDS(lds));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :: "s"(m0v), "v"(g) : "memory", "m0");
}
constexpr int f8_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

template <int MODE, int BM>
__global__ __launch_bounds__(512, 1) void fp8_tile_kernel(Fp8GemmParams p) {
  using C = Fp8TileCfg<BM>;
  constexpr int NA = C::NA, NB = C::NB;
  constexpr bool MX = MODE == kF8_MX;
  constexpr int OPS = C::CPW + (MX ? C::SPW : 0);
  extern __shared__ __attribute__((aligned(16))) uint8_t fsm[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % C::WM, wn = wave / C::WM;
  const int64_t ntiles = (p.N + 255) / 256;
  const int64_t mb = (int64_t)blockIdx.x / ntiles;
  const int64_t nt = (int64_t)blockIdx.x - mb * ntiles;
  const int64_t row0 = mb * BM, K = p.K, nst = K / 128;
  auto src_row = [&](int x) -> int64_t {
    if (x < BM) {
      const int64_t m = row0 + x;
      return m < p.M ? m : p.M - 1;
    }
    const int64_t n = nt * 256 + (x - BM);
    return n < p.N ? n : p.N - 1;
  };
  const uint8_t* dcode[C::CPW];
#pragma unroll
  for (int q = 0; q < C::CPW; ++q) {
    const int x = 8 * (wave + C::WAVES * q) + (lane >> 3);
    const int col = (lane & 7) ^ fp8_swz(x);
    dcode[q] = (x < BM ? p.a_codes : p.w_codes) + src_row(x) * K + col * 16;
  }
  const uint8_t* dscale[C::SPW];
  if (MX) {
#pragma unroll
    for (int q = 0; q < C::SPW; ++q) {
      int w = 64 * (wave + C::WAVES * q) + lane;
      if (w >= C::ROWS) w = C::ROWS - 1;
      const int x = fp8_srow<BM>(w);
      dscale[q] = (x < BM ? p.a_mx : p.w_mx) + src_row(x) * (K / 32);
    }
  }
  auto issue = [&](int64_t t) {
    uint8_t* buf = fsm + (int)(t % C::NBUF) * C::STAGE;
#pragma unroll
    for (int q = 0; q < C::CPW; ++q) f8_copy16(dcode[q] + t * 128, buf + (wave + C::WAVES * q) * 1024);
    if (MX) {
#pragma unroll
      for (int q = 0; q < C::SPW; ++q)
        f8_copy4(dscale[q] + t * 4, buf + C::CODES + (wave + C::WAVES * q) * 256);
    }
  };
  auto sync = [&](int64_t ahead) {
    if (ahead >= 2)
      __builtin_amdgcn_s_waitcnt(f8_vmcnt(2 * OPS));
    else if (ahead >= 1)
      __builtin_amdgcn_s_waitcnt(f8_vmcnt(OPS));
    else
      __builtin_amdgcn_s_waitcnt(f8_vmcnt(0));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  const int r = lane & 31, h = lane >> 5;
  const int swz = fp8_swz(r);
  const int wrow0 = BM + wn * 128, arow0 = wm * 32 * NB;
  // chunk c of a stage: columns 4c + h and 4c + 2 + h of the lane's row
  const int c00 = ((0 + h) ^ swz) << 4, c01 = ((2 + h) ^ swz) << 4;
  const int c10 = ((4 + h) ^ swz) << 4, c11 = ((6 + h) ^ swz) << 4;
  const int wsc_off = C::CODES + (wrow0 + 4 * r) * 4;
  const int asc_off = C::CODES + (arow0 + NB * r) * 4;
  const int one = p.unit_scale;
  const int64_t nkb = nst;
  // BLOCK: the wave's 128 weight rows are one weight block
  const int64_t wblk = (nt * 256 + wn * 128) / 128;
  const int64_t wblk_c = wblk < (p.N + 127) / 128 ? wblk : (p.N + 127) / 128 - 1;
  int64_t am[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int64_t m = row0 + arow0 + 32 * i + r;
    am[i] = m < p.M ? m : p.M - 1;
  }

  v16f acc[NA][NB];
#pragma unroll
  for (int j = 0; j < NA; ++j)
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][i][v] = 0.0f;

  v8i wq[2][NA], aq[2][NB];                       // [chunk]
  uint32_t wsw[NA] = {}, asw[NB] = {}, wsn[NA] = {}, asn[NB] = {};
  auto rd_chunk = [&](const uint8_t* cur, int c) {
    const int x0 = c ? c10 : c00, x1 = c ? c11 : c01;
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const uint8_t* row = cur + (wrow0 + 32 * j + r) * 128;
      const uint4 a = *reinterpret_cast<const uint4*>(row + x0);
      const uint4 b = *reinterpret_cast<const uint4*>(row + x1);
      wq[c][j] = v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const uint8_t* row = cur + (arow0 + 32 * i + r) * 128;
      const uint4 a = *reinterpret_cast<const uint4*>(row + x0);
      const uint4 b = *reinterpret_cast<const uint4*>(row + x1);
      aq[c][i] = v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
    }
  };
  auto rd_scales = [&](const uint8_t* cur) {   // MXFP8: the rows' e8m0 words of a stage
    if (!MX) return;
    const u32x4 w4 = *reinterpret_cast<const u32x4*>(cur + wsc_off);
    wsn[0] = w4.x; wsn[1] = w4.y; wsn[2] = w4.z; wsn[3] = w4.w;
    static_assert(NB == 1, "one activation block per wave");
    asn[0] = *reinterpret_cast<const uint32_t*>(cur + asc_off);
  };
  // BLOCK: this stage's factor a_s[m, kb] * w_s[block, kb] per activation block
  float bf[NB], bfn[NB];
  auto ld_blockf = [&](int64_t kb, float (&f)[NB]) {
    if (MODE != kF8_BLOCK) return;
    const float wsv = p.w_s[wblk_c * nkb + kb];
#pragma unroll
    for (int i = 0; i < NB; ++i) f[i] = p.a_s[am[i] * nkb + kb] * wsv;
  };
  // the MFMAs of chunk c (BLOCK: into the stage's partial sums t)
  v16f t[NA][NB];
  auto mma_chunk = [&](int c) {
#pragma unroll
    for (int j = 0; j < NA; ++j)
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int ws = MX ? (int)((wsw[j] >> (8 * (2 * c + h))) & 0xFFu) : one;
        const int as = MX ? (int)((asw[i] >> (8 * (2 * c + h))) & 0xFFu) : one;
        if (MODE == kF8_BLOCK) {
          if (c == 0) {
#pragma unroll
            for (int v = 0; v < 16; ++v) t[j][i][v] = 0.0f;
          }
          t[j][i] = fp8_mfma<MODE>(wq[c][j], aq[c][i], t[j][i], ws, as);
        } else {
          acc[j][i] = fp8_mfma<MODE>(wq[c][j], aq[c][i], acc[j][i], ws, as);
        }
      }
  };

#pragma unroll
  for (int s = 0; s < C::NBUF; ++s)
    if (s < nst) issue(s);
  sync(nst - 1 < C::NBUF - 1 ? nst - 1 : C::NBUF - 1);   // stage 0 landed
  rd_chunk(fsm, 0);
  rd_scales(fsm);
  ld_blockf(0, bfn);
  for (int64_t st = 0; st < nst; ++st) {
    const uint8_t* cur = fsm + (int)(st % C::NBUF) * C::STAGE;
#pragma unroll
    for (int j = 0; j < NA; ++j) wsw[j] = wsn[j];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      asw[i] = asn[i];
      bf[i] = bfn[i];
    }
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
      ld_blockf(st + 1, bfn);
    }
    __builtin_amdgcn_sched_barrier(0);
    mma_chunk(1);
    if (MODE == kF8_BLOCK) {
#pragma unroll
      for (int j = 0; j < NA; ++j)
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[j][i][v] += t[j][i][v] * bf[i];
    }
    __builtin_amdgcn_sched_barrier(0);
  }

#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int64_t m = row0 + arow0 + 32 * i + r;
    if (m >= p.M) continue;
    const float fa = MODE == kF8_ROW ? p.a_s[m] : (MODE == kF8_BLOCK ? 1.0f : p.alpha);
#pragma unroll
    for (int j = 0; j < NA; ++j) fp8_store_block<MODE>(p, acc[j][i], m, nt * 256 + wn * 128 + 32 * j, h, fa);
  }
}

template <int MODE, int BM>
hipError_t launch_fp8_tile(const Fp8GemmParams& p, hipStream_t s) {
  using C = Fp8TileCfg<BM>;
  const int64_t grid = ((p.N + 255) / 256) * ((p.M + BM - 1) / BM);
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&fp8_tile_kernel<MODE, BM>), C::LDS,
                                    lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fp8_tile_kernel<MODE, BM>), dim3((unsigned)grid), dim3(512), C::LDS, s, p);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_fp8_mode(const Fp8GemmParams& p, hipStream_t s, const char** name) {
  static const char* rows_names[4] = {"fp8_rows_mx", "fp8_rows_tensor", "fp8_rows_row", "fp8_rows_block"};
  static const char* tile_names[4] = {"fp8_tile_mx", "fp8_tile_tensor", "fp8_tile_row", "fp8_tile_block"};
  if (p.M <= 32) {
    *name = rows_names[MODE];
    const int64_t grid = ((p.N + 31) / 32) * ((p.M + 31) / 32);
    if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((fp8_rows_kernel<MODE>), dim3((unsigned)grid), dim3(256), 0, s, p);
    return hipGetLastError();
  }
  // 128-row tiles: two waves per SIMD hold the 128 accumulators and two chunks of
  // operands of a 128 x 32 wave tile in their 256 registers (256-row tiles spill)
  *name = tile_names[MODE];
  return launch_fp8_tile<MODE, 128>(p, s);
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
  switch (mode) {
    case kF8_MX: return launch_fp8_mode<kF8_MX>(p, s, name);
    case kF8_TENSOR: return launch_fp8_mode<kF8_TENSOR>(p, s, name);
    case kF8_ROW: return launch_fp8_mode<kF8_ROW>(p, s, name);
    default: return launch_fp8_mode<kF8_BLOCK>(p, s, name);
  }
}

}  // namespace fp4
