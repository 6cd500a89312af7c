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

__device__ __forceinline__ uint32_t dword_of(const uint4& q, int j) {
  return j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w;
}

// Block scale of sub-step `sub` (8 elements) of a lane's 32-element chunk.
template <int FMT>
__device__ __forceinline__ float scale_value(uint32_t sb, int sub) {
  if (FMT == kMX) return e8m0_value(sb & 0xFFu);
  return e4m3_value_pos((sb >> (8 * (sub >> 1))) & 0xFFu);
}

__device__ __forceinline__ f16x2 f16_pair(float v) {
  const _Float16 h = (_Float16)v;  // exact: e4m3 values are fp16 numbers
  return f16x2{h, h};
}

// FMT: kNV / kMX.  AK: kA_FP4 (activation codes) / kA_BF16.  MT: 16-row
// activation tiles per workgroup.  GEN: K not a multiple of 128 (byte loads).
// U: K steps whose loads are issued together per wave.
template <int FMT, int AK, int MT, bool GEN, int U>
__global__ __launch_bounds__(256) void rowblock_gemm(GemmParams p) {
  constexpr int G = FMT == kNV ? 16 : 32;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
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
        const f16x2 ws_lo = f16_pair(scale_value<FMT>(wsb[u], 0));
        const f16x2 ws_hi = f16_pair(scale_value<FMT>(wsb[u], 2));
        f16x2 as_lo[MT], as_hi[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          as_lo[t] = f16_pair(scale_value<FMT>(asb[u][t], 0));
          as_hi[t] = f16_pair(scale_value<FMT>(asb[u][t], 2));
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
  const float alpha = p.alpha_g ? p.alpha_g[grp] : p.alpha;
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

int gemm_block_rows(int /*fmt*/, int /*akind*/, int64_t /*M_hint*/) { return 32; }

hipError_t launch_gemm(int fmt, int akind, const GemmParams& p, hipStream_t s,
                       const char** name) {
  // row blocks of 32 (two 16-row activation tiles); dense problems of at most 16
  // rows use one tile
  const bool one = !p.mblk_expert && p.M <= 16;
  if (p.mblk_expert && p.bm != 32) return hipErrorInvalidValue;
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
