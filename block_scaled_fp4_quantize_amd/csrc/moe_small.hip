// A whole NVFP4 W4A4 MoE layer for a few routed slots (decode token counts) in two
// launches ("vLLM on the NVIDIA DGX Spark (GB10 / sm_121): A Complete Technical Guide",
// §4.3: one fused kernel does token dispatch, both expert GEMMs, SwiGLU and the top-k
// weighted reduction; here the work splits at the one point where every gate/up result
// must be complete before any down projection starts).
//
//  1. moe_small_gateup_nv: workgroup (slot s, 32 intermediate columns).  Every
//     workgroup routes the few slots itself (a stable counting sort by expert, the
//     general dispatch's order), quantizes its token's hidden row under its expert's
//     input scale into LDS (the quantization pass's arithmetic), streams the 32 gate and
//     32 up weight rows of that expert with all of their K-steps in flight, and applies
//     SwiGLU + requant to the one output row.  The workgroups of the first column tile
//     also write the dispatch bookkeeping and the quantized GEMM1 input.
//  2. moe_small_down_nv: workgroup (16 output columns), 8 waves taking the slots in
//     turn: each down projection of a slot, times its expert's alpha, is written as a
//     y row and added, times its routing weight, into the wave's per-token partial
//     sums; the waves' partials are added in wave order and stored as bf16.  No
//     reduction crosses workgroups, so no grid-wide synchronization is needed.
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

// Gate/up: 8 waves, wave w takes weight rows of group w & 3 (gate columns nt*32 +
// [0, 32) for groups 0-1, the matching up rows for 2-3) over K half w >> 2; K-steps of
// 128 elements, at most SMAX per wave, all of a lane's 16-byte weight pieces in flight.
template <int SMAX>
__global__ __launch_bounds__(512) void moe_small_gateup_nv(MoeSmallParams p, SmallPack pk) {
  // the quantized row, decoded exactly to fp16 (its MFMA operand, shared by all lanes)
  __shared__ __attribute__((aligned(16))) _Float16 x16[kSmallMaxH];
  __shared__ float kp[2][4][16];   // [K half][row group][column]: the partial dot products
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = (int)(p.T * p.k);
  const int64_t H = p.H, I = p.I, E = p.E;
  const int ntiles = (int)(I / 32);
  const int s = (int)(blockIdx.x / ntiles);
  const int nt = (int)(blockIdx.x - (int64_t)s * ntiles);
  const int64_t t = s / p.k;
  // loads first, in the order they are needed: the token's hidden row (known from the
  // block index), all slots' ids, this slot's expert id, that expert's weight rows.
  // Loads complete in issue order, so the routing and the quantization below wait for
  // the first two only and run while the weights stream in.
  const uint16_t* xrow = p.hidden + t * H;
  const int64_t nch = H / 8;   // 8-element chunks of the row; thread tid takes chunk tid
  float xv[8];
  load8<uint16_t>(xrow + (tid < nch ? tid : nch - 1) * 8, xv);   // (past the row: its last)
  const int ej_raw = small_ids_load(p, n, lane);
  int e = p.ids[s];
  e = (e >= 0 && e < E) ? e : -1;
  const int r = lane & 15, gq = lane >> 4;
  const int rg = wave & 3, kh = wave >> 2;
  const int64_t wn = rg < 2 ? nt * 32 + rg * 16 + r : I + nt * 32 + (rg - 2) * 16 + r;
  const int S = (int)(H / 128);
  const int s0 = kh * (S / 2), s1 = kh ? S : S / 2;   // this wave's K-steps [s0, s1)
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

  // the token's hidden row, quantized under g13 as the quantization pass does it (one
  // lane per 8 elements, the 16-element block's amax across a lane pair), and decoded
  // back to its exact fp16 values
  {
    const bool active = tid < nch;
    float amax = 0.0f;
#pragma unroll
    for (int q = 0; q < 8; ++q) amax = fmaxf(amax, active ? fabsf(xv[q]) : 0.0f);
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    if (active) {
      float rq;
      const uint32_t sc = q_nv_scale(amax, g13, &rq);
      uint32_t packed = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) packed |= q_nv_pack2(xv[2 * q], xv[2 * q + 1], rq) << (8 * q);
      const f16x2 sp = e4m3_pair_f16(sc);   // this lane pair's scale value
      *reinterpret_cast<f16x8*>(x16 + tid * 8) = decode8_f16(packed, f16_bcast(sp, 0));
      if (nt == 0) {
        *reinterpret_cast<uint32_t*>(p.x_codes + (int64_t)pos * (H / 2) + tid * 4) = packed;
        if ((tid & 1) == 0) p.x_scales[(int64_t)pos * (H / 16) + tid / 2] = (uint8_t)sc;
      }
    }
  }
  __syncthreads();

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
    const int sa = in ? s0 + i : 0;
    const uint32_t keep = in ? 0xFFFFFFFFu : 0u;
    const uint4 wj = make_uint4(wq[i].x & keep, wq[i].y & keep, wq[i].z & keep, wq[i].w & keep);
    const f16x2 wsp = e4m3_pair_f16(wsb[i]);
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      const f16x8 wop = decode8_f16(dword_of(wj, sub), f16_bcast(wsp, sub >> 1));
      // elements 128 sa + 32 gq + 8 sub .. + 7 of the row: this lane's K slots
      const f16x8 aop = *reinterpret_cast<const f16x8*>(x16 + sa * 128 + gq * 32 + sub * 8);
      acc[sub] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wop, aop, acc[sub], 0, 0, 0);
    }
  }
  v4f sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  asm volatile("" : "+v"(sum));
  // lane (row r, gq) holds columns 4 gq .. + 3 of the group's 16 (every r alike)
  if (r == 0) {
#pragma unroll
    for (int v = 0; v < 4; ++v) kp[kh][rg][4 * gq + v] = sum[v];
  }
  __syncthreads();
  // SwiGLU + requant under g2, the arithmetic of the SwiGLU epilogues: lane c < 32 of
  // wave 0 takes h column nt * 32 + c; a 16-column block is 16 lanes, a code byte a
  // lane pair
  if (tid < 32) {
    const int c = tid & 15, b = tid >> 4;
    const float g = (kp[0][b][c] + kp[1][b][c]) * alpha13;
    const float u = (kp[0][2 + b][c] + kp[1][2 + b][c]) * alpha13;
    const float h = swiglu1(g, u);
    float amax = fabsf(h);
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
    float rq;
    const uint32_t sc = q_nv_scale(amax, g2, &rq);
    const float h1 = __shfl_xor(h, 1);
    if ((tid & 1) == 0)
      p.h_codes[(int64_t)pos * (I / 2) + nt * 16 + tid / 2] = (uint8_t)q_nv_pack2(h, h1, rq);
    if (c == 0) p.h_scales[(int64_t)pos * (I / 16) + nt * 2 + b] = (uint8_t)sc;
  }
}

// down projection + weighted combine; K-steps of 128: S <= SMAX.  A wave decodes its
// slot's h row once, exactly to fp16, into its own LDS row (8-element chunks q = lane,
// lane + 64, ..), and every lane reads its MFMA operand from there.
template <int SMAX>
__global__ __launch_bounds__(512) void moe_small_down_nv(MoeSmallParams p, SmallPack pk) {
  constexpr int WAVES = 8;
  constexpr int HR = (SMAX * 16 + 63) / 64;   // h chunks per lane
  __shared__ float part[WAVES][kSmallTokens][16];
  __shared__ __attribute__((aligned(16))) _Float16 hrow[WAVES][SMAX * 128];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = (int)(p.T * p.k);
  const int64_t H = p.H, I = p.I, E = p.E;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int r = lane & 15, gq = lane >> 4;
  const int S = (int)(I / 128);
  v4f tok[kSmallTokens];
#pragma unroll
  for (int x = 0; x < kSmallTokens; ++x) tok[x] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int s = wave; s < n; s += WAVES) {
    // the slot's expert, sorted position (the gate/up launch's routing; -1: dropped)
    // and weight, fetched together
    const int e = p.ids[s];
    const int pos = p.inverse[s];
    float wt = p.w[s];
    asm volatile("" : "+v"(wt));    // (keeps the three loads ahead of the branch)
    if (pos < 0 || e < 0 || e >= E) continue;   // dropped slot (uniform per wave)
    const int t = s / p.k;
    const float alpha2 = pk.v[3 * E + e];
    const uint8_t* wrow = p.w2_codes + e * H * (I / 2) + (n0 + r) * (I / 2) + gq * 16;
    const uint8_t* wsrow = p.w2_scales + e * H * (I / 16) + (n0 + r) * (I / 16) + 2 * gq;
    const uint8_t* arow = p.h_codes + (int64_t)pos * (I / 2);
    const uint8_t* asrow = p.h_scales + (int64_t)pos * (I / 16);
    uint4 wq[SMAX];
    uint32_t wsb[SMAX], hc[HR], hs[HR];
#pragma unroll
    for (int j = 0; j < HR; ++j) {   // (chunks past the row: its last, not stored)
      const int q = lane + 64 * j < S * 16 ? lane + 64 * j : S * 16 - 1;
      hc[j] = *reinterpret_cast<const uint32_t*>(arow + q * 4);
      hs[j] = asrow[q / 2];
    }
#pragma unroll
    for (int st = 0; st < SMAX; ++st) {
      const int sc = st < S ? st : S - 1;
      wq[st] = *reinterpret_cast<const uint4*>(wrow + sc * 64);
      wsb[st] = *reinterpret_cast<const uint16_t*>(wsrow + sc * 8);
    }
    __builtin_amdgcn_sched_barrier(0);
    _Float16* hw = hrow[wave];
#pragma unroll
    for (int j = 0; j < HR; ++j)
      if (lane + 64 * j < S * 16)
        *reinterpret_cast<f16x8*>(hw + (lane + 64 * j) * 8) = decode8_f16(hc[j], f16_bcast(e4m3_pair_f16(hs[j]), 0));
    __builtin_amdgcn_wave_barrier();   // the row is the wave's own: LDS keeps its order
    v4f acc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < SMAX; ++st) {   // branch-free: steps past S multiply zero codes
      const uint32_t keep = st < S ? 0xFFFFFFFFu : 0u;
      const uint4 wj = make_uint4(wq[st].x & keep, wq[st].y & keep, wq[st].z & keep, wq[st].w & keep);
      const f16x2 wsp = e4m3_pair_f16(wsb[st]);
      const int sa = st < S ? st : 0;
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) {
        const f16x8 wop = decode8_f16(dword_of(wj, sub), f16_bcast(wsp, sub >> 1));
        // elements 128 sa + 32 gq + 8 sub .. + 7 of the h row
        const f16x8 aop = *reinterpret_cast<const f16x8*>(hw + sa * 128 + gq * 32 + sub * 8);
        acc[sub] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wop, aop, acc[sub], 0, 0, 0);
      }
    }
    v4f y = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    asm volatile("" : "+v"(y));
    y = y * alpha2;
    // lane (row r, gq) holds columns n0 + 4 gq .. + 3; row 0 is the slot's
    if (r == 0)
      *reinterpret_cast<float4*>(p.y + (int64_t)pos * H + n0 + 4 * gq) = make_float4(y[0], y[1], y[2], y[3]);
#pragma unroll
    for (int x = 0; x < kSmallTokens; ++x)
      if (x == t) tok[x] += y * wt;
  }
  if (r == 0) {
#pragma unroll
    for (int x = 0; x < kSmallTokens; ++x)
#pragma unroll
      for (int v = 0; v < 4; ++v) part[wave][x][4 * gq + v] = tok[x][v];
  }
  __syncthreads();
  if (tid < p.T * 16) {
    const int x = tid >> 4, c = tid & 15;
    float o = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) o += part[w][x][c];
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
  // K-steps per wave, the smallest instance that covers them: half of H / 128 for
  // gate/up, I / 128 for down (steps past them are masked, not skipped)
  const dim3 g1((unsigned)(n * (p.I / 32)));
  const int64_t s1 = p.H / 256 + (p.H % 256 ? 1 : 0);
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
  const dim3 g2((unsigned)(p.H / 16));
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
