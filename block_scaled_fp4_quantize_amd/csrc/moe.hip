// Mixture-of-experts stages on gfx950: router, dispatch bookkeeping, SwiGLU with
// requantization, and the top-k weighted combine.
//
// Stage structure: "vLLM on the NVIDIA DGX Spark (GB10 / sm_121): A Complete
// Technical Guide", §7.1 (Router -> Quantize-Dispatch -> Permute-Experts-
// Unpermute -> Combine) and §4.3 (the fused expert: token dispatch, two GEMMs,
// SwiGLU, top-k weight reduction, in-kernel BF16->FP4 quantization).  The expert
// GEMMs themselves run in gemm.hip.
//
// Everything here is deterministic: routing ties go to the lower expert index,
// the dispatch is a stable counting sort, and every reduction has a fixed order.
#include <math.h>

#include "device.h"
#include "internal.h"

#pragma clang fp contract(off)

namespace fp4 {

namespace {

// ---- router: one wave per token -----------------------------------------------
constexpr int kMaxPerLane = 16;  // E <= 1024

__global__ __launch_bounds__(256) void topk_softmax_kernel(const float* __restrict__ logits,
                                                           int64_t T, int E, int k, int renorm,
                                                           int32_t* __restrict__ ids,
                                                           float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform over the wave
  const float* row = logits + t * E;
  const int per = (E + 63) / 64;
  float v[kMaxPerLane];
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + 64 * i;
    v[i] = (i < per && e < E) ? row[e] : -INFINITY;
  }
  uint32_t taken = 0;
  int my_e = 0;
  float my_v = 0.f;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + 64 * i;
      if (i < per && e < E && !((taken >> i) & 1u)) {
        if (v[i] > bv || (v[i] == bv && e < be)) {
          bv = v[i];
          be = e;
        }
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oe = __shfl_xor(be, off);
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == j) {
      my_e = be;
      my_v = bv;
    }
  }
  // softmax over all E, evaluated at the chosen experts
  const float mx = __shfl(my_v, 0);
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + 64 * i;
    if (i < per && e < E) sum += expf(v[i] - mx);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  float wj = lane < k ? expf(my_v - mx) / sum : 0.f;
  if (renorm) {
    float s = wj;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    wj = wj / s;
  }
  if (lane < k) {
    ids[t * k + lane] = my_e;
    w[t * k + lane] = wj;
  }
}

// ---- dispatch: counts, offsets and the row-block table (one workgroup) ---------
constexpr int kScanThreads = 1024;

__device__ int block_exclusive_scan(int x, int* buf) {
  // exclusive scan over kScanThreads values: an inclusive scan within each wave by
  // lane shuffles, a scan of the wave totals by wave 0, then the earlier waves' total
  // added (integer sums: the same result as any other order); three barriers
  constexpr int kWaves = kScanThreads / 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int v = x;
#pragma unroll 1
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(v, off, 64);
    if (lane >= off) v += y;
  }
  if (lane == 63) buf[w] = v;
  __syncthreads();
  if (w == 0) {
    int t = lane < kWaves ? buf[lane] : 0;
#pragma unroll 1
    for (int off = 1; off < kWaves; off <<= 1) {
      const int y = __shfl_up(t, off, 64);
      if (lane >= off) t += y;
    }
    if (lane < kWaves) buf[kWaves + lane] = t;
  }
  __syncthreads();
  const int incl = v + (w > 0 ? buf[kWaves + w - 1] : 0);
  __syncthreads();  // (buf is reused by the next scan)
  return incl - x;
}

// ---- dispatch: stable counting sort over the flat slot index i = t*k + j -------
// (1) per-chunk expert histograms; (2) one workgroup turns them into each chunk's
// first position per expert, and builds the offsets and the row-block table;
// (3) per chunk, slot i goes to base[chunk][e] + (number of earlier slots of the
// chunk routed to e).  Positions follow i within every expert, as the stable
// order requires.  Ids outside [0, E) are dropped (inverse -1).
// Sorted positions past the routed count exist only when some ids were dropped.
// Passes that walk every one of the T*k positions (the NVFP4 GEMM1 quantization, the
// unfused SwiGLU) read their token and expert there, so those get token 0 / expert 0
// (valid indices; the rows they produce are never gathered by the GEMMs or the
// combine), and sorted_rows gets -1.
__device__ __forceinline__ void fill_dropped_tail(const PermuteParams& p, int64_t routed,
                                                  int64_t n, int tid, int nthreads) {
  for (int64_t i = routed + tid; i < n; i += nthreads) {
    p.sorted_rows[i] = -1;
    p.row_expert[i] = 0;
    p.src_token[i] = 0;
  }
}

__global__ __launch_bounds__(kPermuteChunk) void permute_hist_kernel(PermuteParams p) {
  __shared__ int cnt[1024];
  const int tid = threadIdx.x;
  for (int e = tid; e < p.E; e += kPermuteChunk) cnt[e] = 0;
  __syncthreads();
  const int64_t n = p.T * p.k;
  const int64_t i = (int64_t)blockIdx.x * kPermuteChunk + tid;
  if (i < n) {
    const int e = p.ids[i];
    if (e >= 0 && e < p.E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  int32_t* out = p.chunk_base + (int64_t)blockIdx.x * p.E;
  for (int e = tid; e < p.E; e += kPermuteChunk) out[e] = cnt[e];
}

// Sum (or, with write_base, turn into running positions starting at base) the
// chunk histogram entries [ch0, ch1) of expert e, 16 loads in flight at a time.
__device__ __forceinline__ int chunk_walk(int32_t* hist, int64_t E, int e, int64_t ch0,
                                          int64_t ch1, bool write_base, int base) {
  int run = base;
  for (int64_t c0 = ch0; c0 < ch1; c0 += 16) {
    int v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int64_t ch = c0 + u < ch1 ? c0 + u : ch1 - 1;
      v[u] = hist[ch * E + e];
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if (c0 + u < ch1) {
        if (write_base) hist[(c0 + u) * E + e] = run;
        run += v[u];
      }
    }
  }
  return run - base;
}

__global__ __launch_bounds__(kScanThreads) void permute_count_kernel(PermuteParams p) {
  __shared__ int buf[kScanThreads];
  __shared__ int partsum[kScanThreads];
  __shared__ int ebase[1024];
  __shared__ int total_mb;
  __shared__ int total_rows;
  const int tid = threadIdx.x;
  const int64_t n = p.T * p.k;
  const int64_t nchunks = (n + kPermuteChunk - 1) / kPermuteChunk;
  // thread = (part, expert): the chunks of each expert are split into `parts`
  // contiguous ranges, one per thread
  const int E = (int)p.E;
  const int parts = kScanThreads / E;          // >= 1 (E <= 1024)
  const int e = tid % E, part = tid / E;
  const bool act = part < parts;
  const int64_t cpp = (nchunks + parts - 1) / parts;
  const int64_t ch0 = act ? (int64_t)part * cpp : 0;
  const int64_t ch1 = act ? (ch0 + cpp < nchunks ? ch0 + cpp : nchunks) : 0;
  partsum[tid] = act && ch0 < ch1 ? chunk_walk(p.chunk_base, E, e, ch0, ch1, false, 0) : 0;
  __syncthreads();
  int c = 0;
  if (tid < E)
    for (int q = 0; q < parts; ++q) c += partsum[q * E + tid];
  const int off = block_exclusive_scan(c, buf);
  if (tid < E) {
    p.expert_offsets[tid] = off;
    p.group_end[tid] = off + c;
    ebase[tid] = off;
  }
  __syncthreads();
  // each chunk histogram entry becomes the chunk's first position for its expert
  if (act && ch0 < ch1) {
    int base = ebase[e];
    for (int q = 0; q < part; ++q) base += partsum[q * E + e];
    chunk_walk(p.chunk_base, E, e, ch0, ch1, true, base);
  }
  if (tid == E - 1) {
    p.expert_offsets[E] = off + c;
    total_rows = off + c;
  }
  const int nmb = (c + p.bm - 1) / p.bm;
  const int mbo = block_exclusive_scan(nmb, buf);
  if (tid == kScanThreads - 1) total_mb = mbo + nmb;
  if (tid < p.E) {
    for (int j = 0; j < nmb; ++j) {
      p.mblk_expert[mbo + j] = tid;
      p.mblk_row0[mbo + j] = off + j * p.bm;
    }
  }
  __syncthreads();
  for (int64_t i = total_mb + tid; i < p.n_mblocks; i += kScanThreads) {
    p.mblk_expert[i] = -1;
    p.mblk_row0[i] = 0;
  }
  fill_dropped_tail(p, total_rows, n, tid, kScanThreads);
}

__global__ __launch_bounds__(kPermuteChunk) void permute_scatter_kernel(PermuteParams p) {
  __shared__ __attribute__((aligned(16))) int ids[kPermuteChunk];
  const int tid = threadIdx.x;
  const int64_t n = p.T * p.k;
  const int64_t i = (int64_t)blockIdx.x * kPermuteChunk + tid;
  int e = -1;
  if (i < n) {
    e = p.ids[i];
    if (e < 0 || e >= p.E) e = -1;
  }
  ids[tid] = e;
  __syncthreads();
  if (i >= n) return;
  if (e < 0) {
    p.inverse[i] = -1;
    return;
  }
  // earlier slots of this chunk routed to the same expert, four at a time
  int rank = 0;
  const int4* ids4 = reinterpret_cast<const int4*>(ids);
  for (int q = 0; q < (tid >> 2); ++q) {
    const int4 v = ids4[q];
    rank += (v.x == e) + (v.y == e) + (v.z == e) + (v.w == e);
  }
  for (int s2 = tid & ~3; s2 < tid; ++s2) rank += ids[s2] == e;
  const int pos = p.chunk_base[(int64_t)blockIdx.x * p.E + e] + rank;
  p.sorted_rows[pos] = (int32_t)i;
  p.inverse[i] = pos;
  p.row_expert[pos] = e;
  p.src_token[pos] = (int32_t)(i / p.k);
}

constexpr int kRankE = 256;  // experts up to which the dispatch ranks by wave histograms

// ---- per-expert host scalars -> device, passed by value (3 KB of kernel arguments,
// under the 4 KB limit: the four scalars of up to 192 experts in one launch) ---------
constexpr int kPackFloats = 768;
struct FloatPack {
  float v[kPackFloats];
};

// One quantization block (G elements of one row) for the folded activation
// quantization: the quantization pass's rules and helpers, one thread per block.
template <int FMT>
__device__ __forceinline__ void quant_block(const uint16_t* x, float g, uint8_t* codes,
                                            uint8_t* scale) {
  constexpr int G = FMT == kNV ? 16 : 32;
  float v[G];
#pragma unroll
  for (int q = 0; q < G / 8; ++q) {
    const uint4 d = *reinterpret_cast<const uint4*>(x + 8 * q);
    const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[8 * q + 2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
      v[8 * q + 2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < G; ++i) amax = fmaxf(amax, fabsf(v[i]));
  uint32_t out[G / 8];
  uint32_t sc;
  if (FMT == kNV) {
    float r;
    sc = q_nv_scale(amax, g, &r);
#pragma unroll
    for (int q = 0; q < G / 8; ++q) {
      uint32_t pk = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pk |= q_nv_pack2(v[8 * q + 2 * i], v[8 * q + 2 * i + 1], r) << (8 * i);
      out[q] = pk;
    }
    *reinterpret_cast<uint2*>(codes) = make_uint2(out[0], out[1]);
  } else {
    int E;
    sc = q_mx_scale(amax, &E);
#pragma unroll
    for (int q = 0; q < G / 8; ++q) {
      uint32_t pk = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pk |= q_mx_pack2(v[8 * q + 2 * i], v[8 * q + 2 * i + 1], E) << (8 * i);
      out[q] = pk;
    }
    *reinterpret_cast<uint4*>(codes) = make_uint4(out[0], out[1], out[2], out[3]);
  }
  *scale = (uint8_t)sc;
}

// ---- dispatch for at most kScanThreads slots (decode token counts): counts,
// offsets, the row-block table and the scatter in one workgroup, the same results
// as the three kernels above; also the per-expert scalar upload and, for few rows,
// the GEMM1 activation quantization (saving their launches) ----------------------------
__global__ __launch_bounds__(kScanThreads) void permute_small_kernel(PermuteParams p,
                                                                     FloatPack pk) {
  __shared__ int buf[kScanThreads];
  __shared__ __attribute__((aligned(16))) int ids[kScanThreads];
  __shared__ int cnt[1024];
  __shared__ int ebase[1024];
  __shared__ int q_src[kScanThreads];
  __shared__ int q_exp[kScanThreads];
  __shared__ int whist[kScanThreads / 64][kRankE];
  __shared__ int total_mb;
  const int tid = threadIdx.x;
  for (int i = tid; i < p.up_n; i += kScanThreads) p.up_dst[i] = pk.v[i];
  const int n = (int)(p.T * p.k);   // <= kScanThreads
  const int E = (int)p.E;           // <= 1024
  int e = -1;
  if (tid < n) {
    e = p.ids[tid];
    if (e < 0 || e >= E) e = -1;
  }
  ids[tid] = e;
  if (tid < E) cnt[tid] = 0;
  __syncthreads();
  if (e >= 0) atomicAdd(&cnt[e], 1);
  __syncthreads();
  const int c = tid < E ? cnt[tid] : 0;
  const int off = block_exclusive_scan(c, buf);
  if (tid < E) {
    p.expert_offsets[tid] = off;
    p.group_end[tid] = off + c;
    ebase[tid] = off;
  }
  if (tid == E - 1) p.expert_offsets[E] = off + c;
  const int nmb = (c + p.bm - 1) / p.bm;
  const int mbo = block_exclusive_scan(nmb, buf);
  if (tid == kScanThreads - 1) total_mb = mbo + nmb;
  if (tid < E) {
    for (int j = 0; j < nmb; ++j) {
      p.mblk_expert[mbo + j] = tid;
      p.mblk_row0[mbo + j] = off + j * p.bm;
    }
  }
  __syncthreads();
  for (int64_t i = total_mb + tid; i < p.n_mblocks; i += kScanThreads) {
    p.mblk_expert[i] = -1;
    p.mblk_row0[i] = 0;
  }
  // rank of a slot among the earlier slots routed to the same expert: with at most
  // kRankE experts, the count over earlier waves comes from per-wave histograms and
  // only the own wave's earlier lanes are compared; else all earlier slots are
  const bool whist_ok = E <= kRankE;
  if (whist_ok) {
    for (int i = tid; i < (kScanThreads / 64) * kRankE; i += kScanThreads) (&whist[0][0])[i] = 0;
    __syncthreads();
    if (e >= 0) atomicAdd(&whist[tid >> 6][e], 1);
    __syncthreads();
    if (tid < E) {  // exclusive prefix over the waves, per expert
      int run = 0;
      for (int w = 0; w < kScanThreads / 64; ++w) {
        const int c2 = whist[w][tid];
        whist[w][tid] = run;
        run += c2;
      }
    }
    __syncthreads();
  }
  if (tid < n) {
    if (e < 0) {
      p.inverse[tid] = -1;
    } else {
      int rank = 0;
      const int4* ids4 = reinterpret_cast<const int4*>(ids);
      const int q0 = whist_ok ? (tid & ~63) >> 2 : 0;   // first int4 to compare
      if (whist_ok) rank = whist[tid >> 6][e];
      for (int q = q0; q < (tid >> 2); ++q) {
        const int4 v = ids4[q];
        rank += (v.x == e) + (v.y == e) + (v.z == e) + (v.w == e);
      }
      for (int s2 = tid & ~3; s2 < tid; ++s2) rank += ids[s2] == e;
      const int pos = ebase[e] + rank;
      p.sorted_rows[pos] = tid;
      p.inverse[tid] = pos;
      p.row_expert[pos] = e;
      p.src_token[pos] = (int32_t)(tid / p.k);
      q_src[pos] = tid / p.k;
      q_exp[pos] = e;
    }
  }
  // (ebase and cnt are final: the barriers inside the scans follow their last writes)
  const int routed = ebase[E - 1] + cnt[E - 1];
  fill_dropped_tail(p, routed, n, tid, kScanThreads);
  if (p.q_fmt < 0) return;  // uniform over the workgroup
  __syncthreads();
  // routed rows: the slots that hold a valid expert (the routed count)
  const int64_t rows = p.q_routed ? (int64_t)routed : p.q_rows;
  const int G = p.q_fmt == kNV ? 16 : 32;
  const int64_t bpr = p.q_K / G;
  for (int64_t b = tid; b < rows * bpr; b += kScanThreads) {
    const int64_t j = b / bpr, kb = b - j * bpr;
    const int64_t src = p.q_routed ? q_src[j] : j;
    const float g = p.q_routed ? pk.v[p.q_g_off + q_exp[j]] : p.q_g;
    const uint16_t* x = p.q_x + src * p.q_K + kb * G;
    uint8_t* codes = p.q_codes + j * (p.q_K / 2) + kb * (G / 2);
    uint8_t* scale = p.q_scales + j * bpr + kb;
    if (p.q_fmt == kNV)
      quant_block<kNV>(x, g, codes, scale);
    else
      quant_block<kMX>(x, g, codes, scale);
  }
}

// ---- SwiGLU + requant: one lane = 8 consecutive intermediate columns -----------
template <int FMT, bool W4A16>
__global__ __launch_bounds__(256) void swiglu_kernel(SwigluParams p) {
  constexpr int LPG = FMT == kNV ? 2 : 4;
  const int64_t chunks = p.I / 8;
  const int64_t total = p.R * chunks;
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool active = c < total;
  const int64_t row = active ? c / chunks : 0;
  const int64_t kc = active ? c - row * chunks : 0;
  float h[8];
  float amax = 0.f;
  float g = p.g;
  if (active) {
    const float* gate = p.gu + row * (2 * p.I) + kc * 8;
    const float* up = gate + p.I;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      h[i] = swiglu1(gate[i], up[i]);
      amax = fmaxf(amax, fabsf(h[i]));
    }
    if (p.row_grp) g = p.grp_g[p.row_grp[row]];
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = 0.f;
  }
  if (W4A16) {
    if (!active) return;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = bf16_pack2(h[2 * i], h[2 * i + 1]);
    *reinterpret_cast<uint4*>(p.h_bf16 + row * p.I + kc * 8) = make_uint4(w[0], w[1], w[2], w[3]);
    return;
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  if (LPG == 4) amax = fmaxf(amax, __shfl_xor(amax, 2));
  if (!active) return;
  uint32_t packed = 0, sc;
  if (FMT == kNV) {
    float r;
    sc = q_nv_scale(amax, g, &r);
#pragma unroll
    for (int i = 0; i < 4; ++i) packed |= q_nv_pack2(h[2 * i], h[2 * i + 1], r) << (8 * i);
  } else {
    int E;
    sc = q_mx_scale(amax, &E);
#pragma unroll
    for (int i = 0; i < 4; ++i) packed |= q_mx_pack2(h[2 * i], h[2 * i + 1], E) << (8 * i);
  }
  *reinterpret_cast<uint32_t*>(p.h_codes + row * (p.I / 2) + kc * 4) = packed;
  if ((kc & (LPG - 1)) == 0) {
    constexpr int G = FMT == kNV ? 16 : 32;
    p.h_scales[row * (p.I / G) + kc / LPG] = (uint8_t)sc;
  }
}

// ---- combine: out[t] = sum_j w[t,j] * y[inverse[t,j]] (+ shared) -> bf16 ------
// The k routed rows of a token are fetched eight at a time with every load of a
// group in flight together (the slot indices first, then the rows at clamped
// addresses), and added in slot order; a dropped slot (expert id out of range)
// contributes nothing.
constexpr int kCombineGroup = 8;

__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  const int64_t chunks = p.H / 8;
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= p.T * chunks) return;
  const int64_t t = c / chunks;
  const int64_t col = (c - t * chunks) * 8;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int j0 = 0; j0 < p.k; j0 += kCombineGroup) {
    int32_t pos[kCombineGroup];
    float wj[kCombineGroup];
#pragma unroll
    for (int u = 0; u < kCombineGroup; ++u) {
      const int j = j0 + u < p.k ? j0 + u : p.k - 1;
      pos[u] = p.inverse[t * p.k + j];
      wj[u] = p.w[t * p.k + j];
      if (j0 + u >= p.k) pos[u] = -1;
    }
    float4 a[kCombineGroup], b[kCombineGroup];
#pragma unroll
    for (int u = 0; u < kCombineGroup; ++u) {
      const float* yr = p.y + (int64_t)(pos[u] >= 0 ? pos[u] : 0) * p.H + col;
      a[u] = reinterpret_cast<const float4*>(yr)[0];
      b[u] = reinterpret_cast<const float4*>(yr)[1];
    }
#pragma unroll
    for (int u = 0; u < kCombineGroup; ++u) {
      if (pos[u] < 0) continue;
      acc[0] += wj[u] * a[u].x; acc[1] += wj[u] * a[u].y;
      acc[2] += wj[u] * a[u].z; acc[3] += wj[u] * a[u].w;
      acc[4] += wj[u] * b[u].x; acc[5] += wj[u] * b[u].y;
      acc[6] += wj[u] * b[u].z; acc[7] += wj[u] * b[u].w;
    }
  }
  if (p.y_shared) {
    const float* yr = p.y_shared + t * p.H + col;
    const float4 a = reinterpret_cast<const float4*>(yr)[0];
    const float4 b = reinterpret_cast<const float4*>(yr)[1];
    acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
    acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
  }
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = bf16_pack2(acc[2 * i], acc[2 * i + 1]);
  *reinterpret_cast<uint4*>(p.out + t * p.H + col) = make_uint4(w[0], w[1], w[2], w[3]);
}

__global__ __launch_bounds__(256) void upload_kernel(float* dst, int n, FloatPack pk) {
  for (int i = threadIdx.x; i < n; i += 256) dst[i] = pk.v[i];
}

}  // namespace

hipError_t launch_topk_softmax(const float* logits, int64_t T, int64_t E, int k,
                               int renormalize, int32_t* ids, float* w, hipStream_t s,
                               const char** name) {
  if (T == 0) return hipSuccess;
  *name = "topk_softmax";
  hipLaunchKernelGGL(topk_softmax_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s,
                     logits, T, (int)E, k, renormalize, ids, w);
  return hipGetLastError();
}

hipError_t launch_permute(const PermuteParams& p, const float* up_host, hipStream_t s,
                          const char** name, bool* quantized) {
  *name = "permute";
  *quantized = false;
  const int64_t n = p.T * p.k;
  if (p.E > 1024 || p.up_n < 0) return hipErrorInvalidValue;
  if (n <= kScanThreads && p.up_n <= kPackFloats) {
    PermuteParams q = p;
    const bool fold_q = p.q_fmt >= 0 && p.q_rows * p.q_K <= kPermuteQuantMax &&
                        p.q_rows <= kScanThreads &&
                        (!p.q_routed || p.q_g_off + p.E <= p.up_n);
    if (!fold_q) q.q_fmt = -1;
    FloatPack pk;
    for (int i = 0; i < kPackFloats; ++i) pk.v[i] = i < p.up_n ? up_host[i] : 0.f;
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(kScanThreads), 0, s, q, pk);
    *quantized = fold_q;
    return hipGetLastError();
  }
  if (p.up_n > 0) {
    hipError_t err = launch_upload_floats(p.up_dst, up_host, p.up_n, s);
    if (err != hipSuccess) return err;
  }
  const int64_t nchunks = (n + kPermuteChunk - 1) / kPermuteChunk;
  if (nchunks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (nchunks > 0) {
    hipLaunchKernelGGL(permute_hist_kernel, dim3((unsigned)nchunks), dim3(kPermuteChunk), 0, s, p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(permute_count_kernel, dim3(1), dim3(kScanThreads), 0, s, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || nchunks == 0) return err;
  hipLaunchKernelGGL(permute_scatter_kernel, dim3((unsigned)nchunks), dim3(kPermuteChunk), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_swiglu(const SwigluParams& p, hipStream_t s, const char** name) {
  const int64_t total = p.R * (p.I / 8);
  if (total == 0) return hipSuccess;
  const dim3 grid((unsigned)((total + 255) / 256)), block(256);
  if (p.mode_w4a16) {
    *name = "swiglu_bf16";
    hipLaunchKernelGGL((swiglu_kernel<kNV, true>), grid, block, 0, s, p);
  } else if (p.fmt == kNV) {
    *name = "swiglu_quant_nvfp4";
    hipLaunchKernelGGL((swiglu_kernel<kNV, false>), grid, block, 0, s, p);
  } else {
    *name = "swiglu_quant_mxfp4";
    hipLaunchKernelGGL((swiglu_kernel<kMX, false>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, hipStream_t s, const char** name) {
  const int64_t total = p.T * (p.H / 8);
  if (total == 0) return hipSuccess;
  *name = "combine";
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_upload_floats(float* dst, const float* host_vals, int64_t n, hipStream_t s) {
  for (int64_t base = 0; base < n; base += kPackFloats) {
    FloatPack pk;
    const int cnt = (int)((n - base) < kPackFloats ? (n - base) : kPackFloats);
    for (int i = 0; i < kPackFloats; ++i) pk.v[i] = i < cnt ? host_vals[base + i] : 0.f;
    hipLaunchKernelGGL(upload_kernel, dim3(1), dim3(256), 0, s, dst + base, cnt, pk);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace fp4
