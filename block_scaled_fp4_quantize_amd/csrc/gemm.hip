// Block-scaled FP4 matmul on gfx950 (dense, or grouped over experts).
//
// Definition: out[m, n] = alpha * sum_k a_hat[m, k] * w_hat[n, k] -- the
// dequantize-then-multiply semantics of the "vLLM per-format kernel capability
// matrix derived from source", THE EMULATION COLUMN, computed natively:
//  * MXFP4 W4A4 maps 1:1 onto gfx950's scaled MFMA: e2m1 codes go in raw and each
//    lane's e8m0 block scale (one 32-element block per lane per instruction) is
//    the instruction's scale operand ("vLLM on the NVIDIA DGX Spark ... Technical
//    Guide", §6.4: MXFP4 = e2m1 + e8m0 per 32).
//  * NVFP4 (e4m3 scale per 16) has no such mapping: e2m1 x e4m3 needs up to six
//    significant bits, more than an fp8 operand holds.  For W4A4 both operands
//    are decoded exactly to fp16 (all such products are fp16 numbers) and
//    multiplied with fp16 MFMA.  W4A16 ("vLLM on the DGX Spark, the Hard Way:
//    Seven Months of GB10 Field Notes": weight-only checkpoints keep 16-bit
//    activations) decodes the weights exactly to bf16 and uses bf16 MFMA against
//    the bf16 activations as given.
//
// This file holds the "row-block" kernel: a workgroup owns one 16-row tile of W
// and 16*MT rows of activations, its 4 waves split K and reduce through LDS in a
// fixed order (bitwise reproducible).  Weight bytes are streamed once per row
// block with 16-byte loads (4 lanes cover 64 contiguous bytes of a row), which is
// what decode-shaped problems need.  Grouped problems (MoE experts) enumerate
// (row block, n tile) pairs from a device-side table, so no host sync is needed.
#include <stdlib.h>

#include "device.h"
#include "internal.h"

namespace fp4 {

namespace {

constexpr int kKStep = 128;  // K elements per lane-group step (4 lanes x 32)

template <bool GEN>
__device__ __forceinline__ uint4 load_codes32(const uint8_t* row, int64_t k0, int64_t K,
                                              bool ok) {
  if (!ok) return make_uint4(0, 0, 0, 0);
  if (!GEN) return *reinterpret_cast<const uint4*>(row + (k0 >> 1));
  uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (k0 + 2 * i < K) w[i >> 2] |= (uint32_t)row[(k0 >> 1) + i] << (8 * (i & 3));
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Scale bytes for a lane's 32-element chunk starting at k0: MXFP4 one e8m0 byte,
// NVFP4 two e4m3 bytes (low byte = first 16 elements).  Out-of-range lanes get a
// neutral scale (their codes are zero).
template <int FMT>
__device__ __forceinline__ uint32_t load_scales32(const uint8_t* srow, int64_t k0,
                                                  int64_t K, bool ok) {
  if (FMT == kMX) {
    if (!ok) return 127u;
    return srow[k0 >> 5];
  } else {
    if (!ok) return 0x3838u;
    uint32_t b0 = srow[k0 >> 4];
    uint32_t b1 = (k0 + 16 < K) ? (uint32_t)srow[(k0 >> 4) + 1] : 0x38u;
    return b0 | (b1 << 8);
  }
}

template <bool GEN>
__device__ __forceinline__ void load_bf16x32(const uint16_t* row, int64_t k0, int64_t K,
                                             bool ok, uint4 out[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (!ok) {
      out[j] = make_uint4(0, 0, 0, 0);
    } else if (!GEN) {
      out[j] = *reinterpret_cast<const uint4*>(row + k0 + 8 * j);
    } else {
      uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t k = k0 + 8 * j + i;
        if (k < K) w[i >> 1] |= (uint32_t)row[k] << (16 * (i & 1));
      }
      out[j] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}


// Block scale of sub-step `sub` (8 elements) of a lane's 32-element chunk.
template <int FMT>
__device__ __forceinline__ float scale_value(uint32_t sb, int sub) {
  if (FMT == kMX) return e8m0_value(sb & 0xFFu);
  return e4m3_value((sb >> (8 * (sub >> 1))) & 0xFFu);
}


// FMT: kNV / kMX.  AK: kA_FP4 (activation codes) / kA_BF16.  MT: 16-row
// activation tiles per workgroup.  GEN: K not a multiple of 128 (byte loads).
// U: K steps whose loads are issued together per wave.
template <int FMT, int AK, int MT, bool GEN, int U>
__global__ __launch_bounds__(256) void rowblock_gemm(GemmParams p) {
  constexpr int G = FMT == kNV ? 16 : 32;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int64_t ntiles = (p.N + 15) >> 4;
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
    row0 = mb * (16 * MT);
    row_end = p.M;
  }
  // per-group scalars fetched up front, not after the main loop
  const float alpha = p.alpha_g ? p.alpha_g[grp] : p.alpha;

  const int64_t K = p.K;
  const int r = lane & 15;
  const int gq = lane >> 4;
  const int64_t wn = nt * 16 + r;
  const bool wvalid = wn < p.N;
  const uint8_t* wrow = p.w_codes + grp * p.w_estride_codes + (wvalid ? wn : 0) * (K >> 1);
  const uint8_t* wsrow = p.w_scales + grp * p.w_estride_scales + (wvalid ? wn : 0) * (K / G);

  const uint8_t* arow[MT];
  const uint8_t* asrow[MT];
  const uint16_t* abrow[MT];
  bool avalid[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int64_t pv = row0 + t * 16 + r;
    avalid[t] = pv < row_end;
    const int64_t src = avalid[t] ? (p.a_gather ? (int64_t)p.a_gather[pv] : pv) : 0;
    if (AK == kA_FP4) {
      arow[t] = p.a_codes + src * (K >> 1);
      asrow[t] = p.a_scales + src * (K / G);
    } else {
      abrow[t] = p.a_bf16 + src * p.lda;
    }
  }

  v4f acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};

  const int64_t nsteps = (K + kKStep - 1) / kKStep;
  for (int64_t s0 = wave; s0 < nsteps; s0 += 4 * U) {
    uint4 wq[U];
    uint32_t wsb[U];
    uint4 aq[U][MT];
    uint32_t asb[U][MT];
    uint4 ab[U][MT][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t s = s0 + 4 * u;
      const bool in = s < nsteps;
      const int64_t k0 = s * kKStep + gq * 32;
      const bool kin = in && k0 < K;
      wq[u] = load_codes32<GEN>(wrow, k0, K, wvalid && kin);
      wsb[u] = load_scales32<FMT>(wsrow, k0, K, wvalid && kin);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        if (AK == kA_FP4) {
          aq[u][t] = load_codes32<GEN>(arow[t], k0, K, avalid[t] && kin);
          asb[u][t] = load_scales32<FMT>(asrow[t], k0, K, avalid[t] && kin);
        } else {
          load_bf16x32<GEN>(abrow[t], k0, K, avalid[t] && kin, ab[u][t]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + 4 * u >= nsteps) break;
      if (FMT == kMX && AK == kA_FP4) {
        const v8i wop = {(int)wq[u].x, (int)wq[u].y, (int)wq[u].z, (int)wq[u].w, 0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const v8i aop = {(int)aq[u][t].x, (int)aq[u][t].y, (int)aq[u][t].z,
                           (int)aq[u][t].w, 0, 0, 0, 0};
          acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              wop, aop, acc[t], 4, 4, 0, (int)wsb[u], 0, (int)asb[u][t]);
        }
      } else if (FMT == kNV && AK == kA_FP4) {
        // NVFP4 W4A4: both operands decoded exactly to fp16, fp16 MFMA
        const f16x2 wsp = e4m3_pair_f16(wsb[u]);
        const f16x2 ws_lo = f16_bcast(wsp, 0);
        const f16x2 ws_hi = f16_bcast(wsp, 1);
        f16x2 as_lo[MT], as_hi[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const f16x2 asp = e4m3_pair_f16(asb[u][t]);
          as_lo[t] = f16_bcast(asp, 0);
          as_hi[t] = f16_bcast(asp, 1);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f16x8 wop = decode8_f16(dword_of(wq[u], j), j < 2 ? ws_lo : ws_hi);
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            const f16x8 aop = decode8_f16(dword_of(aq[u][t], j), j < 2 ? as_lo[t] : as_hi[t]);
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wop, aop, acc[t], 0, 0, 0);
          }
        }
      } else {
        // W4A16: weights decoded exactly to bf16, bf16 activations as given
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x8 wop = FMT == kMX ? decode8_bf16_pow2(dword_of(wq[u], j), scale_value<FMT>(wsb[u], j))
                                        : decode8_bf16(dword_of(wq[u], j), scale_value<FMT>(wsb[u], j));
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            const bf16x8 aop = bits_to_bf16x8(ab[u][t][j]);
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wop, aop, acc[t], 0, 0, 0);
          }
        }
      }
    }
  }

  // split-K reduction across the 4 waves, in wave order
  __shared__ float red[3][MT][64][4];
  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[wave - 1][t][lane][v] = acc[t][v];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    // lane holds out[m = row0 + 16t + (lane & 15)][n = 16 nt + 4 (lane >> 4) + v]
    const int64_t m = row0 + t * 16 + (lane & 15);
    if (m >= row_end) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float x = acc[t][v];
      x += red[0][t][lane][v];
      x += red[1][t][lane][v];
      x += red[2][t][lane][v];
      x *= alpha;
      const int64_t n = nt * 16 + 4 * (lane >> 4) + v;
      if (n >= p.N) continue;
      if (p.out_f32)
        reinterpret_cast<float*>(p.out)[m * p.ldo + n] = x;
      else
        reinterpret_cast<uint16_t*>(p.out)[m * p.ldo + n] = f32_to_bf16_rne(x);
    }
  }
}

// ---------------------------------------------------------------------------------
// Streaming kernel for few activation rows (decode, and MoE experts at decode token
// counts), fp4 activations, K a multiple of 128.  A workgroup owns 64 weight rows
// (16 per wave, the full K range, so no cross-wave reduction) and 16*MT activation
// rows.  The activation codes and scales are staged once per workgroup in LDS, in
// chunks of 1024 K (double-buffered), instead of being re-read by every wave; each
// wave keeps the next chunk's eight 16-byte weight loads per lane in flight while it
// computes the current chunk (two register buffers used in turn).
//
// No load is predicated: a predicated load becomes a divergent branch, after which
// the compiler waits for every outstanding load.  Rows past the end are clamped to
// the last valid row (they only reach outputs that are not stored), and offsets
// past K are clamped to chunks already read (those steps are not computed).
// ---------------------------------------------------------------------------------
constexpr int kSKC = 1024;               // K per staged chunk
constexpr int kSSteps = kSKC / kKStep;   // 8 MFMA K-steps per chunk

template <int FMT, int MT>
struct StreamCfg {
  static constexpr int G = FMT == kNV ? 16 : 32;
  static constexpr int AROWS = 16 * MT;
  static constexpr int ASTR = kSKC / 2 + 16;   // padded LDS row stride of staged codes
  static constexpr int SSTR = kSKC / G;        // scale bytes per staged row per chunk
  static constexpr int SDW = SSTR / 16;        // 16-byte scale loads per lane per chunk
  static constexpr int TPR = 256 / AROWS;      // staging threads per activation row
  static constexpr int CBT = (kSKC / 2) / TPR; // code bytes staged per thread (64 or 32)
  static constexpr int NCL = CBT / 16;         // 16-byte code loads per staging thread
  static constexpr int SBT = SSTR / TPR;       // scale bytes staged per thread (2, 4 or 8)
  static constexpr int NSW = (SBT + 3) / 4;    // scale dwords per staging thread
};

// Activation staging of one chunk: every thread of the workgroup moves CBT code
// bytes and SBT scale bytes of one activation row (global -> registers -> LDS).
// The register copy is held in named variables (an array here ends up on the
// stack, whose reloads the in-order load counter cannot wait for separately).
struct StageRegs {
  uint4 c0, c1, c2, c3, c4, c5, c6, c7;
  uint32_t s0, s1, s2, s3;
};

template <int FMT, int MT>
__device__ __forceinline__ StageRegs stage_load(const uint8_t* codes, const uint8_t* scales,
                                                int64_t c, int64_t KB, int64_t KS, int sseg) {
  using C = StreamCfg<FMT, MT>;
  static_assert(C::NCL <= 8 && C::SBT <= 16 && C::SBT >= 2, "staging registers");
  StageRegs rg;
  const int64_t kb0 = c * (kSKC / 2) + sseg * C::CBT;
  auto ld16 = [&](int i) {
    const int64_t off = kb0 + i * 16;
    return *reinterpret_cast<const uint4*>(codes + (off < KB ? off : 0));
  };
  const int64_t so = c * C::SSTR + sseg * C::SBT;
  auto ld4 = [&](int i) {
    const int64_t o = so + 4 * i;
    return *reinterpret_cast<const uint32_t*>(scales + (o < KS ? o : 0));
  };
  rg.c0 = ld16(0); rg.c1 = ld16(1);
  if (C::NCL > 2) { rg.c2 = ld16(2); rg.c3 = ld16(3); }
  if (C::NCL > 4) { rg.c4 = ld16(4); rg.c5 = ld16(5); rg.c6 = ld16(6); rg.c7 = ld16(7); }
  if (C::SBT == 2)  // KS is a multiple of 4, so so < KS implies so + 2 <= KS
    rg.s0 = *reinterpret_cast<const uint16_t*>(scales + (so < KS ? so : 0));
  else
    rg.s0 = ld4(0);
  if (C::SBT >= 8) rg.s1 = ld4(1);
  if (C::SBT >= 16) { rg.s2 = ld4(2); rg.s3 = ld4(3); }
  return rg;
}

template <int FMT, int MT>
__device__ __forceinline__ void stage_store(uint8_t* a_lds, uint8_t* s_lds, int srow, int sseg,
                                            const StageRegs& rg) {
  using C = StreamCfg<FMT, MT>;
  uint8_t* a = a_lds + srow * C::ASTR + sseg * C::CBT;
  *reinterpret_cast<uint4*>(a) = rg.c0;
  *reinterpret_cast<uint4*>(a + 16) = rg.c1;
  if (C::NCL > 2) {
    *reinterpret_cast<uint4*>(a + 32) = rg.c2;
    *reinterpret_cast<uint4*>(a + 48) = rg.c3;
  }
  if (C::NCL > 4) {
    *reinterpret_cast<uint4*>(a + 64) = rg.c4;
    *reinterpret_cast<uint4*>(a + 80) = rg.c5;
    *reinterpret_cast<uint4*>(a + 96) = rg.c6;
    *reinterpret_cast<uint4*>(a + 112) = rg.c7;
  }
  if (C::SBT == 2) {
    *reinterpret_cast<uint16_t*>(s_lds + srow * C::SSTR + sseg * C::SBT) = (uint16_t)rg.s0;
    return;
  }
  uint32_t* sp = reinterpret_cast<uint32_t*>(s_lds + srow * C::SSTR + sseg * C::SBT);
  sp[0] = rg.s0;
  if (C::SBT >= 8) sp[1] = rg.s1;
  if (C::SBT >= 16) { sp[2] = rg.s2; sp[3] = rg.s3; }
}

// The lane's 16-byte code piece of step st (128 elements) sits at wbase + st * wstride:
// row-major codes (stride 64 bytes), or the prepared layout of 16-row x 128-element
// blocks stored in lane order (stride 1 KB, one contiguous kilobyte per wave).  Steps
// at or past the end read step 0 (their operand is zeroed in stream_compute).
template <int FMT, bool SVEC>
__device__ __forceinline__ void stream_w_load(const uint8_t* wbase, int64_t wstride,
                                              const uint8_t* wsrow, int64_t c, int64_t K,
                                              int64_t KS, uint4 (&q)[kSSteps],
                                              uint4 (&sc)[StreamCfg<FMT, 1>::SDW]) {
  constexpr int SSTR = StreamCfg<FMT, 1>::SSTR;
  const int64_t S = K / kKStep;
#pragma unroll
  for (int j = 0; j < kSSteps; ++j) {
    const int64_t st = c * kSSteps + j;
    q[j] = *reinterpret_cast<const uint4*>(wbase + (st < S ? st : 0) * wstride);
  }
#pragma unroll
  for (int i = 0; i < StreamCfg<FMT, 1>::SDW; ++i) {
    const int64_t so = c * SSTR + i * 16;
    if (SVEC) {  // scale rows a multiple of 16 bytes: so < KS implies so + 16 <= KS
      sc[i] = *reinterpret_cast<const uint4*>(wsrow + (so < KS ? so : 0));
    } else {     // 4-byte granularity (KS is a multiple of 4)
      uint32_t d[4];
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        const int64_t o = so + 4 * q2;
        d[q2] = *reinterpret_cast<const uint32_t*>(wsrow + (o < KS ? o : 0));
      }
      sc[i] = make_uint4(d[0], d[1], d[2], d[3]);
    }
  }
}

// Branch-free over all kSSteps steps (a data-dependent exit would stop the full
// unroll and turn the register buffers into stack memory); steps at or past
// nsteps get an all-zero weight operand.
template <int FMT, int MT>
__device__ __forceinline__ void stream_compute(
    const uint8_t* a_lds, const uint8_t* s_lds, const uint4 (&wq)[kSSteps],
    const uint4 (&wsc)[StreamCfg<FMT, 1>::SDW], int nsteps, int r, int gq, v4f (&acc)[MT]) {
  using C = StreamCfg<FMT, MT>;
#pragma unroll
  for (int j = 0; j < kSSteps; ++j) {
    const uint32_t keep = j < nsteps ? 0xFFFFFFFFu : 0u;
    const uint4 wj = make_uint4(wq[j].x & keep, wq[j].y & keep, wq[j].z & keep, wq[j].w & keep);
    if (FMT == kMX) {
      // scale byte 4j + gq of the chunk: dword j of the scale window
      const uint32_t wsd = dword_of(wsc[j >> 2], j & 3);
      const uint32_t wsb = (wsd >> (8 * gq)) & 0xFFu;
      const v8i wop = {(int)wj.x, (int)wj.y, (int)wj.z, (int)wj.w, 0, 0, 0, 0};
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int ar = t * 16 + r;
        const uint4 aq = *reinterpret_cast<const uint4*>(a_lds + ar * C::ASTR + j * 64 + gq * 16);
        const uint32_t asb = s_lds[ar * C::SSTR + j * 4 + gq];
        const v8i aop = {(int)aq.x, (int)aq.y, (int)aq.z, (int)aq.w, 0, 0, 0, 0};
        acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wop, aop, acc[t], 4, 4, 0,
                                                                   (int)wsb, 0, (int)asb);
      }
    } else {
      // scale bytes 8j + 2gq, +1 of the chunk: dword 2j + gq/2 of the scale window
      const uint32_t d0 = dword_of(wsc[(2 * j) >> 2], (2 * j) & 3);
      const uint32_t d1 = dword_of(wsc[(2 * j + 1) >> 2], (2 * j + 1) & 3);
      const uint32_t wsd2 = (gq >> 1) ? d1 : d0;
      const uint32_t wsb = (wsd2 >> (16 * (gq & 1))) & 0xFFFFu;
      const f16x2 wsp = e4m3_pair_f16(wsb);
      const f16x2 ws_lo = f16_bcast(wsp, 0);
      const f16x2 ws_hi = f16_bcast(wsp, 1);
      uint4 aq[MT];
      f16x2 as_lo[MT], as_hi[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int ar = t * 16 + r;
        aq[t] = *reinterpret_cast<const uint4*>(a_lds + ar * C::ASTR + j * 64 + gq * 16);
        const uint32_t asb = *reinterpret_cast<const uint16_t*>(s_lds + ar * C::SSTR + j * 8 + gq * 2);
        const f16x2 asp = e4m3_pair_f16(asb);
        as_lo[t] = f16_bcast(asp, 0);
        as_hi[t] = f16_bcast(asp, 1);
      }
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) {
        const f16x8 wop = decode8_f16(dword_of(wj, sub), sub < 2 ? ws_lo : ws_hi);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const f16x8 aop = decode8_f16(dword_of(aq[t], sub), sub < 2 ? as_lo[t] : as_hi[t]);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wop, aop, acc[t], 0, 0, 0);
        }
      }
    }
  }
}

// Fused SwiGLU + requant epilogue of a gate/up GEMM on the streaming kernel: waves 0-1
// hold gate columns c0 .. c0 + 31 and waves 2-3 the matching up columns (c0 = 32 nt);
// h = SiLU(alpha g) * (alpha u) is formed through LDS and quantized 8 columns per lane
// (2 lanes per NVFP4 block of 16, 4 per MXFP4 block of 32), the arithmetic of the
// stand-alone SwiGLU kernel, into h_codes / h_scales at the rows of the output.
template <int FMT, int MT>
__device__ __forceinline__ void stream_swiglu_epilogue(const GemmParams& p, const v4f (&acc)[MT],
                                                       float alpha, int grp, int64_t row0,
                                                       int64_t row_end, int64_t nt, int wave,
                                                       int lane, float* up, float* hb) {
  constexpr int LD = 33;                   // padded row of 32 columns
  constexpr int LPG = FMT == kNV ? 2 : 4;
  const int r = lane & 15, cq = 4 * (lane >> 4);
  __syncthreads();                         // every wave is done with the staging buffers
  if (wave >= 2) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) up[(t * 16 + r) * LD + (wave - 2) * 16 + cq + v] = acc[t][v] * alpha;
  }
  __syncthreads();
  if (wave < 2) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int o = (t * 16 + r) * LD + wave * 16 + cq + v;
        hb[o] = swiglu1(acc[t][v] * alpha, up[o]);
      }
  }
  __syncthreads();
  const int tid = wave * 64 + lane;
  if (wave >= MT) return;                  // 64 MT lanes: 16 MT rows x 4 chunks of 8
  const int row = tid >> 2, chunk = tid & 3;
  float h[8];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h[i] = hb[row * LD + chunk * 8 + i];
    amax = fmaxf(amax, fabsf(h[i]));
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  if (LPG == 4) amax = fmaxf(amax, __shfl_xor(amax, 2));
  const int64_t m = row0 + row;
  if (m >= row_end) return;
  const float g = p.h_grp_g ? p.h_grp_g[grp] : p.h_g;
  uint32_t packed = 0, sc;
  if (FMT == kNV) {
    float rr;
    sc = q_nv_scale(amax, g, &rr);
#pragma unroll
    for (int i = 0; i < 4; ++i) packed |= q_nv_pack2(h[2 * i], h[2 * i + 1], rr) << (8 * i);
  } else {
    int E;
    sc = q_mx_scale(amax, &E);
#pragma unroll
    for (int i = 0; i < 4; ++i) packed |= q_mx_pack2(h[2 * i], h[2 * i + 1], E) << (8 * i);
  }
  const int64_t col = nt * 32 + chunk * 8;
  *reinterpret_cast<uint32_t*>(p.h_codes + m * (p.I / 2) + col / 2) = packed;
  if ((chunk & (LPG - 1)) == 0) {
    constexpr int G = FMT == kNV ? 16 : 32;
    p.h_scales[m * (p.I / G) + col / G] = (uint8_t)sc;
  }
}

template <int FMT, int MT, bool SVEC>
__global__ __launch_bounds__(256) void stream_gemm(GemmParams p) {
  using C = StreamCfg<FMT, MT>;
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[2][C::AROWS * C::ASTR];
  __shared__ __attribute__((aligned(16))) uint8_t s_lds[2][C::AROWS * C::SSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  // fused SwiGLU: a workgroup owns 32 intermediate columns (their gate and up rows)
  const int64_t ntiles = p.fuse_swiglu ? p.I / 32 : (p.N + 63) >> 6;
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
  const int64_t KS = K / C::G;

  const int r = lane & 15;
  const int gq = lane >> 4;
  const int64_t wn_raw = !p.fuse_swiglu ? nt * 64 + wave * 16 + r
                         : (wave < 2 ? nt * 32 + wave * 16 + r : p.I + nt * 32 + (wave - 2) * 16 + r);
  const int64_t wn = wn_raw < p.N ? wn_raw : p.N - 1;
  const uint8_t* wcodes = p.w_codes + grp * p.w_estride_codes;
  const uint8_t* wbase = p.w_tiled
      ? wcodes + (((wn >> 4) * (K / kKStep)) * 64 + (wn & 15) + 16 * gq) * 16
      : wcodes + wn * KB + gq * 16;
  const int64_t wstride = p.w_tiled ? 1024 : kKStep / 2;
  const uint8_t* wsrow = p.w_scales + grp * p.w_estride_scales + wn * KS;

  // activation staging: thread -> (row, segment of the row's chunk)
  const int srow = tid / C::TPR;
  const int sseg = tid % C::TPR;
  int64_t pv = row0 + srow;
  if (pv >= row_end) pv = row_end - 1;  // row0 < row_end for every block
  const int64_t s_src = p.a_gather ? (int64_t)p.a_gather[pv] : pv;
  const uint8_t* s_codes = p.a_codes + s_src * KB;
  const uint8_t* s_scales = p.a_scales + s_src * KS;
  const int64_t nchunks = (K + kSKC - 1) / kSKC;
  StageRegs st;

  v4f acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};

  uint4 wA[kSSteps], wB[kSSteps];
  uint4 sA[C::SDW], sB[C::SDW];
  auto steps_of = [&](int64_t c) {
    const int64_t rem = (K - c * kSKC) / kKStep;
    return rem < kSSteps ? (int)rem : kSSteps;
  };

  st = stage_load<FMT, MT>(s_codes, s_scales, 0, KB, KS, sseg);
  stream_w_load<FMT, SVEC>(wbase, wstride, wsrow, 0, K, KS, wA, sA);
  stage_store<FMT, MT>(a_lds[0], s_lds[0], srow, sseg, st);
  __syncthreads();
  // (the prefetch of the chunk after the last one is skipped: it would only make the
  // last waves wait for loads nothing uses)
  for (int64_t c = 0; c < nchunks; c += 2) {
    // chunk c from (buffer 0, wA); prefetch chunk c+1 into (buffer 1, wB)
    if (c + 1 < nchunks) {
      // issued before the weight loads, so waiting for it leaves those in flight
      st = stage_load<FMT, MT>(s_codes, s_scales, c + 1, KB, KS, sseg);
      __builtin_amdgcn_sched_barrier(0);  // keep the staging loads ahead of the weight loads
      stream_w_load<FMT, SVEC>(wbase, wstride, wsrow, c + 1, K, KS, wB, sB);
      stream_compute<FMT, MT>(a_lds[0], s_lds[0], wA, sA, steps_of(c), r, gq, acc);
      stage_store<FMT, MT>(a_lds[1], s_lds[1], srow, sseg, st);
      __syncthreads();
    } else {
      stream_compute<FMT, MT>(a_lds[0], s_lds[0], wA, sA, steps_of(c), r, gq, acc);
      break;
    }
    // chunk c+1 from (buffer 1, wB); prefetch chunk c+2 into (buffer 0, wA)
    if (c + 2 < nchunks) {
      st = stage_load<FMT, MT>(s_codes, s_scales, c + 2, KB, KS, sseg);
      __builtin_amdgcn_sched_barrier(0);
      stream_w_load<FMT, SVEC>(wbase, wstride, wsrow, c + 2, K, KS, wA, sA);
      stream_compute<FMT, MT>(a_lds[1], s_lds[1], wB, sB, steps_of(c + 1), r, gq, acc);
      stage_store<FMT, MT>(a_lds[0], s_lds[0], srow, sseg, st);
      __syncthreads();
    } else {
      stream_compute<FMT, MT>(a_lds[1], s_lds[1], wB, sB, steps_of(c + 1), r, gq, acc);
      break;
    }
  }

  if (p.fuse_swiglu) {
    stream_swiglu_epilogue<FMT, MT>(p, acc, alpha, grp, row0, row_end, nt, wave, lane,
                                    reinterpret_cast<float*>(a_lds[0]),
                                    reinterpret_cast<float*>(a_lds[1]));
    return;
  }
  const int64_t n0 = nt * 64 + wave * 16 + 4 * (lane >> 4);
  // a lane holds out[m][n0 .. n0+3]: one 8-byte (bf16) or 16-byte (fp32) store when the
  // four columns exist and the row stride and base allow it
  const bool vec = (p.ldo & 3) == 0 &&
                   (reinterpret_cast<uintptr_t>(p.out) & (p.out_f32 ? 15 : 7)) == 0;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int64_t m = row0 + t * 16 + (lane & 15);
    if (m >= row_end) continue;
    const float x0 = acc[t][0] * alpha, x1 = acc[t][1] * alpha;
    const float x2 = acc[t][2] * alpha, x3 = acc[t][3] * alpha;
    if (vec && n0 + 3 < p.N) {
      if (p.out_f32)
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + m * p.ldo + n0) =
            make_float4(x0, x1, x2, x3);
      else
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + m * p.ldo + n0) =
            make_uint2(bf16_pack2(x0, x1), bf16_pack2(x2, x3));
      continue;
    }
    const float xs[4] = {x0, x1, x2, x3};
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t n = n0 + v;
      if (n >= p.N) continue;
      if (p.out_f32)
        reinterpret_cast<float*>(p.out)[m * p.ldo + n] = xs[v];
      else
        reinterpret_cast<uint16_t*>(p.out)[m * p.ldo + n] = f32_to_bf16_rne(xs[v]);
    }
  }
}

template <int FMT, int MT>
hipError_t launch_stream(const GemmParams& p, hipStream_t s, const char** name) {
  const int64_t ntiles = p.fuse_swiglu ? p.I / 32 : (p.N + 63) / 64;
  const int64_t mblocks = p.mblk_expert ? p.n_mblocks : (p.M + 16 * MT - 1) / (16 * MT);
  const int64_t grid = ntiles * mblocks;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  *name = FMT == kNV ? (MT == 1 ? "stream_nvfp4_m16" : "stream_nvfp4_m32")
                     : (MT == 1 ? "stream_mxfp4_m16" : "stream_mxfp4_m32");
  const bool svec = ((p.K / StreamCfg<FMT, MT>::G) % 16) == 0;
  if (svec)
    hipLaunchKernelGGL((stream_gemm<FMT, MT, true>), dim3((unsigned)grid), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((stream_gemm<FMT, MT, false>), dim3((unsigned)grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int FMT, int AK, int MT>
hipError_t launch_rowblock(const GemmParams& p, hipStream_t s, const char** name) {
  const int64_t ntiles = (p.N + 15) / 16;
  const int64_t mblocks = p.mblk_expert ? p.n_mblocks : (p.M + 16 * MT - 1) / (16 * MT);
  const int64_t grid = ntiles * mblocks;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const bool gen = (p.K % kKStep) != 0;
  constexpr int U = AK == kA_FP4 ? 4 : 2;
  static const char* names[2][2][2] = {
      {{"rowblock_nvfp4_a4", "rowblock_nvfp4_a4_gen"}, {"rowblock_nvfp4_a16", "rowblock_nvfp4_a16_gen"}},
      {{"rowblock_mxfp4_a4", "rowblock_mxfp4_a4_gen"}, {"rowblock_mxfp4_a16", "rowblock_mxfp4_a16_gen"}}};
  *name = names[FMT][AK][gen ? 1 : 0];
  if (gen)
    hipLaunchKernelGGL((rowblock_gemm<FMT, AK, MT, true, U>), dim3((unsigned)grid), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((rowblock_gemm<FMT, AK, MT, false, U>), dim3((unsigned)grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

int gemm_block_rows(int /*fmt*/, int akind, int64_t rows_per_group, int64_t H, int64_t I) {
  // experts averaging at least 48 rows: 128-row tiles; at most 16: one 16-row tile per
  // block (half the activation decode and MFMA work of a 32-row block); else 32
  // (fp4 activations: the FP4 tile kernel; bf16 activations: the W4A16 tile kernel)
  const bool tiled = H % kKStep == 0 && I % kKStep == 0;
  if (tiled && rows_per_group >= 48) return 128;
  return rows_per_group <= 16 ? 16 : 32;
}

bool gemm_can_fuse_swiglu(int fmt, int akind, int64_t M, int64_t K, int64_t I, bool grouped,
                          int bm, int64_t n_mblocks) {
  if (akind != kA_FP4 || K % kKStep != 0 || I <= 0 || I % 128 != 0) return false;
  if (grouped ? bm == 128 : M > 64) return true;          // the tiled kernel
  if (grouped && bm != 16 && bm != 32) return false;
  // the streaming kernel: where the unfused GEMM would run on it anyway, or for at most
  // 16 rows, where saving the SwiGLU launch outweighs the resident kernel's faster
  // stream (measured: NVFP4, 8 routed rows, 12.6 -> 9.1 us; 512 rows, 53 -> 68 us)
  const bool one = grouped ? bm == 16 : M <= 16;
  const bool resident = one && !(grouped && fmt == kMX) &&
                        resident_fits(fmt, 1, grouped ? 16 : M, 2 * I, K, grouped ? n_mblocks : 1);
  return !resident || M <= 16;
}

hipError_t launch_gemm(int fmt, int akind, const GemmParams& p, hipStream_t s,
                       const char** name) {
  if (p.fuse_swiglu) {   // the tiled or the streaming kernel
    if (!gemm_can_fuse_swiglu(fmt, akind, p.M, p.K, p.I, p.mblk_expert != nullptr, p.bm,
                              p.n_mblocks))
      return hipErrorInvalidValue;
    if (p.mblk_expert ? p.bm == 128 : p.M > 64) return launch_gemm_tiled(fmt, p, s, name);
    if (p.mblk_expert && p.bm != 16 && p.bm != 32) return hipErrorInvalidValue;
    const bool one1 = p.mblk_expert ? p.bm == 16 : p.M <= 16;
    if (fmt == kNV) return one1 ? launch_stream<kNV, 1>(p, s, name) : launch_stream<kNV, 2>(p, s, name);
    return one1 ? launch_stream<kMX, 1>(p, s, name) : launch_stream<kMX, 2>(p, s, name);
  }
  // prepared weights: only the decode kernels (streaming, resident) read that layout
  if (p.w_tiled && (akind != kA_FP4 || p.mblk_expert || p.M > 64 || p.K % kKStep || p.N % 16))
    return hipErrorInvalidValue;
  // bf16 activations, many rows (or 128-row expert blocks): the LDS-tiled bf16-MFMA kernel
  if (akind == kA_BF16 && w4a16_tiled_ok(p)) return launch_gemm_w4a16_tiled(fmt, p, s, name);
  // row blocks of 32 (two 16-row activation tiles); dense problems of at most 16
  // rows, and expert tables of 16-row blocks, use one tile
  const bool one = p.mblk_expert ? p.bm == 16 : p.M <= 16;
  // fp4 activations with K a multiple of 128 take the streaming kernel, or the
  // LDS-tiled one when there are many activation rows
  const bool fast = akind == kA_FP4 && p.K % kKStep == 0;
  if (p.mblk_expert && p.bm != 32 && p.bm != 16) {
    if (p.bm != 128 || !fast) return hipErrorInvalidValue;
    return launch_gemm_tiled(fmt, p, s, name);
  }
  if (fast && !p.mblk_expert && p.M > 64) return launch_gemm_tiled(fmt, p, s, name);
  // at most 16 rows (one 16-row activation tile): activations resident in LDS with
  // a deep weight stream, when they fit; two-tile blocks measure faster on the
  // streaming kernel below, and so do MXFP4 expert tables of 16-row blocks (many
  // experts with a few rows each: 64 weight rows per workgroup amortize the staging),
  // and short-K NVFP4 expert tables of at most 32 blocks (a few routed tokens: the
  // resident kernel's per-block staging of the activations is not repaid by K < 1024)
  const bool grouped_mx = p.mblk_expert && fmt == kMX;
  const bool few_short = p.mblk_expert && p.K < 1024 && p.n_mblocks <= 32;
  if (fast && one && !grouped_mx && !few_short &&
      resident_fits(fmt, 1, p.mblk_expert ? 16 : p.M, p.N, p.K, p.mblk_expert ? p.n_mblocks : 1))
    return launch_gemm_resident(fmt, 1, p, s, name);
  if (fast) {
    if (fmt == kNV) return one ? launch_stream<kNV, 1>(p, s, name) : launch_stream<kNV, 2>(p, s, name);
    return one ? launch_stream<kMX, 1>(p, s, name) : launch_stream<kMX, 2>(p, s, name);
  }
  if (fmt == kNV) {
    if (akind == kA_FP4)
      return one ? launch_rowblock<kNV, kA_FP4, 1>(p, s, name) : launch_rowblock<kNV, kA_FP4, 2>(p, s, name);
    return one ? launch_rowblock<kNV, kA_BF16, 1>(p, s, name) : launch_rowblock<kNV, kA_BF16, 2>(p, s, name);
  }
  if (akind == kA_FP4)
    return one ? launch_rowblock<kMX, kA_FP4, 1>(p, s, name) : launch_rowblock<kMX, kA_FP4, 2>(p, s, name);
  return one ? launch_rowblock<kMX, kA_BF16, 1>(p, s, name) : launch_rowblock<kMX, kA_BF16, 2>(p, s, name);
}

}  // namespace fp4
