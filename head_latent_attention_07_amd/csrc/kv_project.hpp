// Down-projection of the new tokens and their cache append: the latent
// c_KV = W_DKV h_t ("DeepSeek AI efficiency, architecture, benchmarks",
// section "Architectural Innovations: Multi-Head Latent Attention (MLA)",
// equation for c_KV) and the RoPE key k^R = RoPE(W_KR h_t), both computed
// from the token's hidden state h_t ("How DeepSeek Rewrote the Transformer
// [MLA]", section "MLA: compress the pair, not the heads", diagram), then
// written to the cache as the append does.
//
// y[b, n] = sum_k W[n, k] h[b, k] for the 576 outputs n (rows 0..511 of W are
// W_DKV, rows 512..575 W_KR) is a GEMM with M = batch, N = 576 and
// K = d_model whose cost is the single pass over the weights (8.3 MB in bf16
// at d_model 7168; 2 * batch flops per weight element, under the MFMA ridge
// for any batch up to ~300). So the kernel is laid out for the weight
// stream:
//   * grid = 18 column tiles of 32 outputs x S slices of K (x batch groups
//     of 128): every weight element is read by exactly one workgroup, and
//     each workgroup covers the whole batch group, so no weight is read
//     twice;
//   * both operands are contiguous along K, so each lane loads its MFMA
//     operands straight from global memory (no LDS staging): lane l of a
//     wave reads 32 consecutive k of row l % 32 (half l / 32 of a 64-wide
//     chunk), and the four MFMAs of the chunk pair those k identically for
//     the weight and the hidden row (the contraction order inside a chunk
//     is a permutation of k, which a sum does not see);
//   * the four waves of a workgroup take interleaved chunks of its K slice
//     and are reduced through LDS in a fixed order (the result does not
//     depend on timing); each slice writes an fp32 partial [S, B, 576]. The
//     LDS reduction and the partials grow with the accumulator volume, so
//     a workgroup holds one 32-wide column tile (64-wide tiles measured no
//     faster and double both);
//   * a second kernel (one workgroup per sequence) sums the S partials in a
//     fixed order and hands the fp32 row to the append's rotate-and-store.
#pragma once

#include "append.hpp"

namespace mla {

constexpr int PJ_CHUNK = 64;               // k per chunk (two lane halves of 32)
constexpr int PJ_NSUB = 1;                 // 32-wide MFMA column tiles per workgroup
constexpr int PJ_NT = 32 * PJ_NSUB;        // outputs per workgroup
constexpr int PJ_NTILES = D_QK / PJ_NT;    // the W_KR rows (512..575) fill whole tiles
constexpr int PJ_CH = 1;                   // chunks whose loads a wave has in flight at once
constexpr int PJ_MG = 128;                 // batch rows per batch group: four 32-row tiles
constexpr int PJ_WAVES = 4;

struct ProjectParams {
  const void* h;      // [B, D] hidden states, row stride D
  const void* w_dkv;  // [512, D]
  const void* w_kr;   // [64, D]
  float* part;        // [S, B, 576] fp32 partial sums, one per K slice
  int B, D;
  int S;              // K slices
  int cps;            // 64-wide chunks per slice
};

// Per-type operand traffic: a lane's 32 consecutive k of one row are LOADS
// 16-byte loads; mfma_chunk contracts a tile pair over those 32 k (and the
// other half's 32 k held by lanes 32..63).
template <typename T>
struct PjOps;

template <>
struct PjOps<bf16> {
  static constexpr int LOADS = 4;
  __device__ __forceinline__ static void mfma_chunk(f32x16& acc, const u32x4 (&a)[LOADS],
                                                    const u32x4 (&b)[LOADS]) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[i]),
                                                    __builtin_bit_cast(bf16x8, b[i]), acc, 0, 0, 0);
  }
};

template <>
struct PjOps<float> {
  static constexpr int LOADS = 8;
  __device__ __forceinline__ static void mfma_chunk(f32x16& acc, const u32x4 (&a)[LOADS],
                                                    const u32x4 (&b)[LOADS]) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[i][e]),
                                                   __uint_as_float(b[i][e]), acc, 0, 0, 0);
  }
};

// Workgroups whose ids share the dispatcher's round-robin XCD (id mod 8) get
// consecutive tile indices, so the column tiles of a K slice, which
// read the same hidden-state columns, meet in one XCD's L2. A bijection of
// [0, G).
__device__ __forceinline__ int pj_tile_index(int bid, int G) {
  const int xcd = bid & 7, slot = bid >> 3, q = G >> 3, rem = G & 7;
  return xcd * q + (xcd < rem ? xcd : rem) + slot;
}

template <typename T, int MSUB>
__global__ __launch_bounds__(256) void mla_kv_project_kernel(ProjectParams p) {
  using Ops = PjOps<T>;
  constexpr int L = Ops::LOADS;
  constexpr int E = MSUB * PJ_NSUB * 16;   // accumulator values per lane
  __shared__ float red[PJ_WAVES][E][64];

  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, r = l & 31, g = l >> 5;
  const int G = (int)gridDim.x;
  int t = pj_tile_index((int)blockIdx.x, G);
  const int nt = t % PJ_NTILES;
  t /= PJ_NTILES;
  const int s = t % p.S;
  const int mg = t / p.S;
  const int nchunks = p.D / PJ_CHUNK;
  const int c0 = s * p.cps;
  const int c1 = min(c0 + p.cps, nchunks);

  const T* wrow[PJ_NSUB];
#pragma unroll
  for (int ns = 0; ns < PJ_NSUB; ++ns) {
    const int n = nt * PJ_NT + 32 * ns + r;
    wrow[ns] = (n < D_C) ? (const T*)p.w_dkv + (int64_t)n * p.D
                         : (const T*)p.w_kr + (int64_t)(n - D_C) * p.D;
  }
  const T* hrow[MSUB];
#pragma unroll
  for (int ms = 0; ms < MSUB; ++ms) {
    const int m = min(mg * PJ_MG + 32 * ms + r, p.B - 1);   // rows past the batch: discarded
    hrow[ms] = (const T*)p.h + (int64_t)m * p.D;
  }

  f32x16 acc[MSUB][PJ_NSUB];
#pragma unroll
  for (int ms = 0; ms < MSUB; ++ms)
#pragma unroll
    for (int ns = 0; ns < PJ_NSUB; ++ns)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[ms][ns][j] = 0.f;

  // wave w takes chunks w, w+4, ... of the slice, PJ_CH of them per pass
  // (a pass's chunks past the slice load its last chunk again and skip it)
  for (int c = c0 + w; c < c1; c += PJ_WAVES * PJ_CH) {
    u32x4 bw[PJ_CH][PJ_NSUB][L], ah[PJ_CH][MSUB][L];
#pragma unroll
    for (int ch = 0; ch < PJ_CH; ++ch) {
      const int k = min(c + PJ_WAVES * ch, c1 - 1) * PJ_CHUNK + 32 * g;
#pragma unroll
      for (int ns = 0; ns < PJ_NSUB; ++ns)
#pragma unroll
        for (int i = 0; i < L; ++i)
          bw[ch][ns][i] = *(const u32x4*)((const char*)(wrow[ns] + k) + 16 * i);
#pragma unroll
      for (int ms = 0; ms < MSUB; ++ms)
#pragma unroll
        for (int i = 0; i < L; ++i)
          ah[ch][ms][i] = *(const u32x4*)((const char*)(hrow[ms] + k) + 16 * i);
    }
    // every load of the pass is issued before the first MFMA waits on one
    // (left to itself the scheduler interleaves them and pays the memory
    // latency several times per chunk)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ch = 0; ch < PJ_CH; ++ch) {
      if (ch > 0 && c + PJ_WAVES * ch >= c1) break;
#pragma unroll
      for (int ms = 0; ms < MSUB; ++ms)
#pragma unroll
        for (int ns = 0; ns < PJ_NSUB; ++ns) Ops::mfma_chunk(acc[ms][ns], ah[ch][ms], bw[ch][ns]);
    }
  }

  // reduce the four waves' sums: wave w adds entries [w E/4, (w+1) E/4) of
  // all four in wave order and stores them
#pragma unroll
  for (int i = 0; i < E; ++i) red[w][i][l] = acc[i / (16 * PJ_NSUB)][(i >> 4) % PJ_NSUB][i & 15];
  __syncthreads();
#pragma unroll
  for (int q = 0; q < E / PJ_WAVES; ++q) {
    const int i = w * (E / PJ_WAVES) + q;
    const float v = ((red[0][i][l] + red[1][i][l]) + red[2][i][l]) + red[3][i][l];
    const int ms = i / (16 * PJ_NSUB), ns = (i >> 4) % PJ_NSUB, j = i & 15;
    // 32x32 accumulator layout: lane l holds column l % 32, rows
    // 8 (j / 4) + 4 (l / 32) + j % 4
    const int m = mg * PJ_MG + 32 * ms + 8 * (j >> 2) + 4 * g + (j & 3);
    const int n = nt * PJ_NT + 32 * ns + r;
    if (m < p.B) p.part[((int64_t)s * p.B + m) * D_QK + n] = v;
  }
}

// One workgroup per sequence: wave w sums slices w, w+4, ... of the partials
// (the loads of up to eight slices in flight at once, clamped to valid
// slices, the extra ones discarded), the waves are added in order, and wave
// 0 stores the row. The RoPE angle needs only the position: it is computed
// while the loads are in flight.
constexpr int PJ_FIN_U = 8;

struct PjRound {
  f32x4 v0[PJ_FIN_U], v1[PJ_FIN_U];
  f32x2 pr[PJ_FIN_U];
};

__device__ __forceinline__ void pj_fin_load(PjRound& q, const float* __restrict__ part, int s0,
                                            int S, int B, int b, int l, int lp) {
#pragma unroll
  for (int u = 0; u < PJ_FIN_U; ++u) {
    const int s = min(s0 + PJ_WAVES * u, S - 1);
    const float* row = part + ((int64_t)s * B + b) * D_QK;
    q.v0[u] = *(const f32x4*)(row + 8 * l);
    q.v1[u] = *(const f32x4*)(row + 8 * l + 4);
    q.pr[u] = *(const f32x2*)(row + D_C + 2 * lp);
  }
}

__device__ __forceinline__ void pj_fin_add(const PjRound& q, int s0, int S, float (&x)[8],
                                           float& xe, float& xo) {
#pragma unroll
  for (int u = 0; u < PJ_FIN_U; ++u) {
    if (s0 + PJ_WAVES * u < S) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] += q.v0[u][i];
        x[4 + i] += q.v1[u][i];
      }
      xe += q.pr[u][0];
      xo += q.pr[u][1];
    }
  }
}

__global__ __launch_bounds__(256) void mla_project_append_kernel(const float* __restrict__ part,
                                                                 int S, int B, AppendParams a) {
  const int b = blockIdx.x, w = threadIdx.x >> 6, l = threadIdx.x & 63, lp = l & (D_R / 2 - 1);
  float x[8], xe = 0.f, xo = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = 0.f;
  PjRound q;
  // first round outside the loop, so that the angle (loop-invariant) is
  // computed after its loads are issued rather than before the loop
  pj_fin_load(q, part, w, S, B, b, l, lp);
  __builtin_amdgcn_sched_barrier(0);
  RopeAngle ang{};
  if (w == 0) ang = append_angle(a, b, l);
  pj_fin_add(q, w, S, x, xe, xo);
  for (int s0 = w + PJ_FIN_U * PJ_WAVES; s0 < S; s0 += PJ_FIN_U * PJ_WAVES) {
    pj_fin_load(q, part, s0, S, B, b, l, lp);
    pj_fin_add(q, s0, S, x, xe, xo);
  }
  __shared__ float red[PJ_WAVES - 1][10][64];
  if (w > 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) red[w - 1][i][l] = x[i];
    red[w - 1][8][l] = xe;
    red[w - 1][9][l] = xo;
  }
  __syncthreads();
  if (w != 0) return;
#pragma unroll
  for (int v = 0; v < PJ_WAVES - 1; ++v) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] += red[v][i][l];
    xe += red[v][8][l];
    xo += red[v][9][l];
  }
  append_write(a, b, l, x, (double)xe, (double)xo, ang);
}

}  // namespace mla
