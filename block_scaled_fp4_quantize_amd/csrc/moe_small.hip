// A whole NVFP4 W4A4 MoE layer for a few routed slots (decode token counts) in two
// launches ("vLLM on the NVIDIA DGX Spark (GB10 / sm_121): A Complete Technical Guide",
// §4.3: one fused kernel does token dispatch, both expert GEMMs, SwiGLU and the top-k
// weighted reduction; here the work splits at the one point where every gate/up result
// must be complete before any down projection starts).
//
//  1. moe_small_gateup_nv: workgroup (slot s, 16 intermediate columns).  Every
//     workgroup routes the few slots itself (a stable counting sort by expert, the
//     general dispatch's order), quantizes its token's hidden row under its expert's
//     input scale into LDS (the quantization pass's arithmetic), streams the 16 gate and
//     16 up weight rows of that expert with all of their K-steps in flight, and applies
//     SwiGLU + requant to the one output row.  The workgroups of the first column tile
//     also write the dispatch bookkeeping and the quantized GEMM1 input.
//  2. moe_small_down_nv: workgroup (8 output columns), 8 waves taking the slots in
//     pairs (one MFMA serves both slots of a pair): each down projection of a slot,
//     times its expert's alpha, is written as a y row and added, times its routing
//     weight, into the wave's per-token partial sums; the partials are added in slot
//     order and stored as bf16.  No reduction crosses workgroups, so no grid-wide
//     synchronization is needed.
//
// The workspace rows the general path writes are written here too, at the same sorted
// positions (offsets, sorted rows, inverse map, GEMM1 input codes, h codes, y rows), so
// the layer's stages stay checkable.  Slots whose id is outside [0, E) are dropped.
#include "device.h"
#include "internal.h"

namespace fp4 {

namespace {

constexpr int kSmallPack = 768;   // 4 per-expert scalars: g13, alpha13, g2, alpha2
struct SmallPack {
  float v[kSmallPack];
};

// Routing of the few slots inside one wave: lane j < n holds slot j's expert id (-1
// outside [0, E)).  A slot's sorted position is the number of routed slots before it in
// expert order, slots of one expert in slot order (the general dispatch's order).  The
// load is branch-free and its check separate, so that other loads can be issued between
// the two.
__device__ __forceinline__ int small_ids_load(const MoeSmallParams& p, int n, int lane) {
  return p.ids[lane < n ? lane : 0];
}
__device__ __forceinline__ int small_ids_check(int raw, int n, int lane, int64_t E) {
  return lane < n && raw >= 0 && raw < E ? raw : -1;
}
__device__ __forceinline__ int small_pos(int ej, int lane, int s, int es) {
  const bool before = ej >= 0 && (ej < es || (ej == es && lane < s));
  return __builtin_popcountll(__ballot(before));
}

// Cross-lane steps by DPP within a row of 16 lanes: the value of lane ^ 1, and the
// maximum over the row (xor 1, xor 2, then the mirrors of 8 and of 16 lanes)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float lane_xor1(float v) { return dpp_f<0xB1>(v); }
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));    // quad_perm [1, 0, 3, 2]
  v = fmaxf(v, dpp_f<0x4E>(v));    // quad_perm [2, 3, 0, 1]
  v = fmaxf(v, dpp_f<0x141>(v));   // row_half_mirror
  return fmaxf(v, dpp_f<0x140>(v));   // row_mirror
}

// Gate/up: 8 waves, wave w takes the 16 gate rows (w even) or the matching 16 up rows
// (w odd) of columns nt*16 + [0, 16) over K quarter w >> 1; K-steps of 128 elements, at
// most SMAX per wave, all of a lane's 16-byte weight pieces in flight.  16 columns per
// workgroup give 2 x 8 x I / 16 workgroups for 8 slots (384 at I = 768), enough to
// keep every CU streaming.  Every wave quantizes its own K quarter of the hidden row
// into its own LDS slice (two waves share a quarter: the work is repeated, a workgroup
// barrier is not needed), so its MFMA loop starts as soon as its piece of the row has
// arrived and decodes the weight steps in the order they land.
template <int SMAX>
__global__ __launch_bounds__(512) void moe_small_gateup_nv(MoeSmallParams p, SmallPack pk) {
  constexpr int XR = (SMAX * 16 + 63) / 64;   // 8-element row chunks per lane
  // each wave's K half of the quantized row, decoded exactly to fp16 (its MFMA operand)
  __shared__ __attribute__((aligned(16))) _Float16 xw[8][SMAX * 128];
  __shared__ float kp[4][2][16];   // [K quarter][gate, up][column]: the partial dot products
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = (int)(p.T * p.k);
  const int64_t H = p.H, I = p.I, E = p.E;
  const int ntiles = (int)(I / 16);
  const int s = (int)(blockIdx.x / ntiles);
  const int nt = (int)(blockIdx.x - (int64_t)s * ntiles);
  const int64_t t = s / p.k;
  const int r = lane & 15, gq = lane >> 4;
  const int rg = wave & 1, kq = wave >> 1;   // gate (0) or up (1) rows; K quarter
  const int S = (int)(H / 128);
  const int s0 = kq * S / 4, s1 = (kq + 1) * S / 4;   // this wave's K-steps [s0, s1)
  const int nq = (s1 - s0) * 16;                        // its row chunks
  // loads first, in the order they are needed: the wave's piece of the token's hidden
  // row (known from the block index), all slots' ids, this slot's expert id, that
  // expert's weight rows.  Loads complete in issue order, so the routing and the
  // quantization below wait for the first two only and run while the weights stream in.
  const uint16_t* xrow = p.hidden + t * H + (int64_t)s0 * 128;
  float xv[XR][8];
#pragma unroll
  for (int j = 0; j < XR; ++j) {   // chunk lane + 64 j of the piece (past it: its last)
    const int q = lane + 64 * j < nq ? lane + 64 * j : (nq > 0 ? nq - 1 : 0);
    load8<uint16_t>(xrow + q * 8, xv[j]);
  }
  const int ej_raw = small_ids_load(p, n, lane);
  int e = p.ids[s];
  e = (e >= 0 && e < E) ? e : -1;
  const int64_t wn = rg == 0 ? nt * 16 + r : I + nt * 16 + r;
  const int ec = e >= 0 ? e : 0;   // a dropped slot's workgroup loads expert 0 and exits
  const uint8_t* wrow = p.w13_codes + ec * (2 * I) * (H / 2) + wn * (H / 2) + gq * 16;
  const uint8_t* wsrow = p.w13_scales + ec * (2 * I) * (H / 16) + wn * (H / 16) + 2 * gq;
  uint4 wq[SMAX];
  uint32_t wsb[SMAX];
#pragma unroll
  for (int i = 0; i < SMAX; ++i) {
    const int st = s0 + i < s1 ? s0 + i : (s1 > s0 ? s1 - 1 : 0);   // past the range: zeroed below
    wq[i] = *reinterpret_cast<const uint4*>(wrow + st * 64);
    wsb[i] = *reinterpret_cast<const uint16_t*>(wsrow + st * 8);
  }
  __builtin_amdgcn_sched_barrier(0);
  const int ej = small_ids_check(ej_raw, n, lane, E);

  const int pos = small_pos(ej, lane, s, e);   // uniform; meaningful when e >= 0
  if (nt == 0 && wave == 0) {
    // dispatch bookkeeping, each entry written once: the slot's own entries by its
    // first tile; offsets and the dropped tail of sorted_rows by slot 0's first tile
    if (lane == 0) {
      p.inverse[s] = e >= 0 ? pos : -1;
      if (e >= 0) p.sorted_rows[pos] = s;
    }
    if (s == 0) {
      const int routed = __builtin_popcountll(__ballot(ej >= 0));
      if (lane >= routed && lane < n) p.sorted_rows[lane] = -1;
      // lane x: routed slots of experts < x (the loop is uniform over the wave, so every
      // lane takes part in the shuffles)
      for (int64_t x0 = 0; x0 <= E; x0 += 64) {
        const int64_t x = x0 + lane;
        int off = 0;
        for (int j = 0; j < n; ++j) {
          const int f = __shfl(ej, j);
          off += (f >= 0 && f < x) ? 1 : 0;
        }
        if (x <= E) p.expert_offsets[x] = off;
      }
    }
  }
  if (e < 0) return;   // dropped slot (uniform over the workgroup)
  const float g13 = pk.v[e], alpha13 = pk.v[E + e], g2 = pk.v[2 * E + e];

  // the wave's piece of the hidden row, quantized under g13 as the quantization pass
  // does it (8 elements per lane and chunk, the 16-element block's amax across a lane
  // pair), and decoded back to its exact fp16 values; the first tile's row-group-0
  // waves also store the GEMM1 input codes and scales
  _Float16* xs = xw[wave];
  if (nq == 0 && lane < 16) *reinterpret_cast<f16x8*>(xs + lane * 8) = f16x8{};   // (no steps: zeros for the masked reads)
#pragma unroll
  for (int j = 0; j < XR; ++j) {
    const int q = lane + 64 * j;
    const bool active = q < nq;
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, active ? fabsf(xv[j][i]) : 0.0f);
    amax = fmaxf(amax, lane_xor1(amax));
    float rq;
    const uint32_t sc = q_nv_scale(amax, g13, &rq);
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) packed |= q_nv_pack2(xv[j][2 * i], xv[j][2 * i + 1], rq) << (8 * i);
    if (active) {
      const f16x2 sp = e4m3_pair_f16(sc);   // this lane pair's scale value
      *reinterpret_cast<f16x8*>(xs + q * 8) = decode8_f16(packed, f16_bcast(sp, 0));
      if (nt == 0 && rg == 0) {
        const int64_t qa = (int64_t)s0 * 16 + q;   // the chunk's index in the row
        *reinterpret_cast<uint32_t*>(p.x_codes + (int64_t)pos * (H / 2) + qa * 4) = packed;
        if ((q & 1) == 0) p.x_scales[(int64_t)pos * (H / 16) + qa / 2] = (uint8_t)sc;
      }
    }
  }
  __builtin_amdgcn_wave_barrier();   // the slice is the wave's own: LDS keeps its order

  // gate/up: fp16 MFMAs, the weights decoded exactly, the activation operand read as it
  // is (every lane reads the one row: the 16 rows of the operand are copies); branch-free
  // over SMAX steps (a data-dependent exit would let the compiler sink each step's weight
  // load into the step): steps past the wave's range multiply zero codes
  v4f acc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < SMAX; ++i) {
    const bool in = s0 + i < s1;
    const int ia = in ? i : 0;
    const uint32_t keep = in ? 0xFFFFFFFFu : 0u;
    const uint4 wj = make_uint4(wq[i].x & keep, wq[i].y & keep, wq[i].z & keep, wq[i].w & keep);
    const f16x2 wsp = e4m3_pair_f16(wsb[i]);
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      const f16x8 wop = decode8_f16(dword_of(wj, sub), f16_bcast(wsp, sub >> 1));
      // elements 128 (s0 + ia) + 32 gq + 8 sub .. + 7 of the row: this lane's K slots
      const f16x8 aop = *reinterpret_cast<const f16x8*>(xs + ia * 128 + gq * 32 + sub * 8);
      acc[sub] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wop, aop, acc[sub], 0, 0, 0);
    }
  }
  v4f sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  asm volatile("" : "+v"(sum));
  // lane (row r, gq) holds columns 4 gq .. + 3 of the group's 16 (every r alike)
  if (r == 0) {
#pragma unroll
    for (int v = 0; v < 4; ++v) kp[kq][rg][4 * gq + v] = sum[v];
  }
  __syncthreads();
  // SwiGLU + requant under g2, the arithmetic of the SwiGLU epilogues: lane c < 16 of
  // wave 0 takes h column nt * 16 + c; the 16-column block is a row of 16 lanes, a code
  // byte a lane pair
  if (wave == 0) {
    const int c = lane & 15;
    const float g = ((kp[0][0][c] + kp[1][0][c]) + (kp[2][0][c] + kp[3][0][c])) * alpha13;
    const float u = ((kp[0][1][c] + kp[1][1][c]) + (kp[2][1][c] + kp[3][1][c])) * alpha13;
    const float h = swiglu1(g, u);
    const float amax = max16(fabsf(h));
    float rq;
    const uint32_t sc = q_nv_scale(amax, g2, &rq);
    const float h1 = lane_xor1(h);
    if (lane < 16) {
      if ((lane & 1) == 0)
        p.h_codes[(int64_t)pos * (I / 2) + nt * 8 + lane / 2] = (uint8_t)q_nv_pack2(h, h1, rq);
      if (c == 0) p.h_scales[(int64_t)pos * (I / 16) + nt] = (uint8_t)sc;
    }
  }
}

// Down projection + weighted combine: workgroup = 8 output columns n0 .. n0 + 7, wave w
// takes the slot pairs (2 m, 2 m + 1), m = w, w + 8, ..  One 16x16x32 MFMA serves both
// slots of a pair: its rows 0-7 are the first slot's weight rows n0 .. n0 + 7 and rows
// 8-15 the second's, its columns 0-7 copies of the first slot's h row and 8-15 of the
// second's (the products across the two slots are computed and not used).  K-steps of
// 128: S <= SMAX.  The wave decodes both h rows once, exactly to fp16, into its own LDS
// rows (8-element chunks q = lane, lane + 64, ..), and every lane reads its MFMA operand
// from there.  A dropped slot's weights are masked to zero and its h row is zero.
template <int SMAX>
__global__ __launch_bounds__(512) void moe_small_down_nv(MoeSmallParams p, SmallPack pk) {
  constexpr int WAVES = 8;
  constexpr int HR = (SMAX * 16 + 63) / 64;   // chunks of one h row per lane
  __shared__ float part[WAVES][2][kSmallTokens][8];
  __shared__ __attribute__((aligned(16))) _Float16 hrow[WAVES][2][SMAX * 128];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = (int)(p.T * p.k);
  const int64_t H = p.H, I = p.I, E = p.E;
  const int64_t n0 = (int64_t)blockIdx.x * 8;
  const int r = lane & 15, gq = lane >> 4;
  const int hf = r >> 3;   // the lane's slot of the pair: its A row and its B column
  const int S = (int)(I / 128);
  v4f tok[kSmallTokens];
#pragma unroll
  for (int x = 0; x < kSmallTokens; ++x) tok[x] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int m = wave; 2 * m < n; m += WAVES) {
    // both slots' experts, sorted positions (the gate/up launch's routing; -1: dropped)
    // and weights, fetched together
    const int sa = 2 * m, sb = 2 * m + 1 < n ? 2 * m + 1 : 2 * m;
    const int ea = p.ids[sa], eb = p.ids[sb];
    const int pa = p.inverse[sa], pb = p.inverse[sb];
    float wa = p.w[sa], wb = p.w[sb];
    asm volatile("" : "+v"(wa), "+v"(wb));    // (keeps the loads ahead of the branch)
    const bool va = pa >= 0 && ea >= 0 && ea < E;
    const bool vb = 2 * m + 1 < n && pb >= 0 && eb >= 0 && eb < E;
    if (!va && !vb) continue;   // (uniform per wave)
    const int eac = va ? ea : 0, ebc = vb ? eb : 0;
    const bool vm = hf ? vb : va;
    const int em = hf ? ebc : eac;
    const uint8_t* wrow = p.w2_codes + em * H * (I / 2) + (n0 + (r & 7)) * (I / 2) + gq * 16;
    const uint8_t* wsrow = p.w2_scales + em * H * (I / 16) + (n0 + (r & 7)) * (I / 16) + 2 * gq;
    const int64_t ra = va ? pa : 0, rb = vb ? pb : 0;
    uint4 wq[SMAX];
    uint32_t wsb[SMAX], hc[2][HR], hs[2][HR];
#pragma unroll
    for (int j = 0; j < HR; ++j) {   // (chunks past the row: its last, not stored)
      const int q = lane + 64 * j < S * 16 ? lane + 64 * j : S * 16 - 1;
      hc[0][j] = *reinterpret_cast<const uint32_t*>(p.h_codes + ra * (I / 2) + q * 4);
      hs[0][j] = p.h_scales[ra * (I / 16) + q / 2];
      hc[1][j] = *reinterpret_cast<const uint32_t*>(p.h_codes + rb * (I / 2) + q * 4);
      hs[1][j] = p.h_scales[rb * (I / 16) + q / 2];
    }
#pragma unroll
    for (int st = 0; st < SMAX; ++st) {
      const int sc = st < S ? st : S - 1;
      wq[st] = *reinterpret_cast<const uint4*>(wrow + sc * 64);
      wsb[st] = *reinterpret_cast<const uint16_t*>(wsrow + sc * 8);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const bool vh = hh ? vb : va;
      _Float16* hw = hrow[wave][hh];
#pragma unroll
      for (int j = 0; j < HR; ++j)
        if (lane + 64 * j < S * 16) {
          const f16x8 d = decode8_f16(hc[hh][j], f16_bcast(e4m3_pair_f16(hs[hh][j]), 0));
          *reinterpret_cast<f16x8*>(hw + (lane + 64 * j) * 8) = vh ? d : f16x8{};
        }
    }
    __builtin_amdgcn_wave_barrier();   // the rows are the wave's own: LDS keeps its order
    const _Float16* hw = hrow[wave][hf];
    v4f acc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < SMAX; ++st) {   // branch-free: steps past S multiply zero codes
      const uint32_t keep = st < S && vm ? 0xFFFFFFFFu : 0u;
      const uint4 wj = make_uint4(wq[st].x & keep, wq[st].y & keep, wq[st].z & keep, wq[st].w & keep);
      const f16x2 wsp = e4m3_pair_f16(wsb[st]);
      const int sa2 = st < S ? st : 0;
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) {
        const f16x8 wop = decode8_f16(dword_of(wj, sub), f16_bcast(wsp, sub >> 1));
        // elements 128 sa2 + 32 gq + 8 sub .. + 7 of the lane's h row
        const f16x8 aop = *reinterpret_cast<const f16x8*>(hw + sa2 * 128 + gq * 32 + sub * 8);
        acc[sub] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wop, aop, acc[sub], 0, 0, 0);
      }
    }
    v4f y = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    asm volatile("" : "+v"(y));
    // lane (column r, gq) holds rows 4 gq .. + 3: lanes 0 and 16 the first slot's columns
    // n0 + 4 (gq & 1) .. + 3 (rows 0-7, column 0), lanes 40 and 56 the second's (rows
    // 8-15, column 8)
    const float alpha2 = hf ? pk.v[3 * E + ebc] : pk.v[3 * E + eac];
    y = y * alpha2;
    const bool outl = (r == 0 && gq < 2) || (r == 8 && gq >= 2);
    if (outl && vm)
      *reinterpret_cast<float4*>(p.y + (hf ? rb : ra) * H + n0 + 4 * (gq & 1)) =
          make_float4(y[0], y[1], y[2], y[3]);
    const int tm = (hf ? sb : sa) / p.k;
    const float wm = vm ? (hf ? wb : wa) : 0.0f;
#pragma unroll
    for (int x = 0; x < kSmallTokens; ++x)
      if (x == tm) tok[x] += y * wm;
  }
  if ((r == 0 && gq < 2) || (r == 8 && gq >= 2)) {
#pragma unroll
    for (int x = 0; x < kSmallTokens; ++x)
#pragma unroll
      for (int v = 0; v < 4; ++v) part[wave][hf][x][4 * (gq & 1) + v] = tok[x][v];
  }
  __syncthreads();
  if (tid < p.T * 8) {   // the pairs' partials in slot order
    const int x = tid >> 3, c = tid & 7;
    float o = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      o += part[w][0][x][c];
      o += part[w][1][x][c];
    }
    p.out[x * H + n0 + c] = f32_to_bf16_rne(o);
  }
}

}  // namespace

bool moe_small_fits(int64_t T, int k, int64_t E, int64_t H, int64_t I) {
  return T >= 1 && T <= kSmallTokens && T * k <= kSmallSlots && 4 * E <= kSmallPack &&
         H % 128 == 0 && H <= kSmallMaxH && I % 128 == 0 && I <= kSmallMaxI;
}

hipError_t launch_moe_small(const MoeSmallParams& p, const float* scal_host, hipStream_t s,
                            const char** name) {
  if (!moe_small_fits(p.T, p.k, p.E, p.H, p.I)) return hipErrorInvalidValue;
  SmallPack pk;
  for (int i = 0; i < kSmallPack; ++i) pk.v[i] = i < 4 * p.E ? scal_host[i] : 0.0f;
  const int64_t n = p.T * p.k;
  *name = "moe_small_gateup_nvfp4";
  // K-steps per wave, the smallest instance that covers them: a quarter of H / 128
  // (rounded up) for gate/up, I / 128 for down (steps past them are masked, not skipped)
  const dim3 g1((unsigned)(n * (p.I / 16)));
  const int64_t s1 = (p.H / 128 + 3) / 4;
  if (s1 <= 4)
    hipLaunchKernelGGL(moe_small_gateup_nv<4>, g1, dim3(512), 0, s, p, pk);
  else if (s1 <= 8)
    hipLaunchKernelGGL(moe_small_gateup_nv<8>, g1, dim3(512), 0, s, p, pk);
  else if (s1 <= 12)
    hipLaunchKernelGGL(moe_small_gateup_nv<12>, g1, dim3(512), 0, s, p, pk);
  else
    hipLaunchKernelGGL(moe_small_gateup_nv<16>, g1, dim3(512), 0, s, p, pk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  *name = "moe_small_down_nvfp4";
  const dim3 g2((unsigned)(p.H / 8));
  const int64_t s2 = p.I / 128;
  if (s2 <= 4)
    hipLaunchKernelGGL(moe_small_down_nv<4>, g2, dim3(512), 0, s, p, pk);
  else if (s2 <= 6)
    hipLaunchKernelGGL(moe_small_down_nv<6>, g2, dim3(512), 0, s, p, pk);
  else if (s2 <= 8)
    hipLaunchKernelGGL(moe_small_down_nv<8>, g2, dim3(512), 0, s, p, pk);
  else if (s2 <= 12)
    hipLaunchKernelGGL(moe_small_down_nv<12>, g2, dim3(512), 0, s, p, pk);
  else
    hipLaunchKernelGGL(moe_small_down_nv<16>, g2, dim3(512), 0, s, p, pk);
  return hipGetLastError();
}

}  // namespace fp4
