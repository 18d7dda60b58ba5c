// Decode with W_UK and W_UV absorbed offline into the query and output
// projections ("How DeepSeek Rewrote the Transformer [MLA]", section "MLA:
// compress the pair, not the heads": by associativity W_UK can be absorbed
// into the Q matrix and W_UV into the output matrix W_O before serving).
//
// With per-head fused weights W_QK[h] = W_UK[h]^T W_Q[h] [512, d_model] and
// W_VO[h] = W_UV[h] W_O[h] [512, d_model], a decode step goes from the
// token's model-width input x to its model-width output y:
//   q_lat[b, h]  = W_QK[h] x[b]                       (GEMM, K = d_model)
//   o_lat[b, h]  = attention over the latent cache     (the decode kernels)
//   y[b]         = sum_h o_lat[b, h] W_VO[h]          (GEMM, K = 512 H)
//
// Kernels:
//   * mla_fuse_weights_kernel: the offline products (fp32 vector ALU, one
//     64 x 64 output tile of one head per workgroup, the 128-long
//     contraction staged in LDS); run once per set of weights;
//   * mla_skinny_gemm_kernel: Y = X W^T for a small batch M and large N, K,
//     both operands contiguous along K (the fused weights are stored so):
//     the operand scheme of the down-projection GEMM (each lane loads its
//     MFMA operands straight from global memory, 32 consecutive k of one
//     row, the same k permutation for both operands), 32 output columns per
//     workgroup, K cut into slices that write fp32 partial sums [S, M, N]
//     (summed in a fixed order by the finishing kernels);
//   * mla_fused_q_finish_kernel: sums the query partials into the attention
//     kernels' query-operand layout, pre-scaled, plus the RoPE query part;
//   * mla_merge_latent_kernel: merges the attention splits into o_lat
//     [B, H * 512] bf16 (no W_UV: it is inside W_VO);
//   * mla_fused_out_finish_kernel: sums the output partials into y (bf16).
#pragma once

#include "common.hpp"

namespace mla {

// ---------------------------------------------------------------------------
// Offline fusion: for each head h, C_h[m, n] = sum_k A_h(k, m) B_h(k, n) with
// k over 128 (d_nope or d_v), all operands addressed through strides
// (elements), bf16 in and out, fp32 accumulation.
// ---------------------------------------------------------------------------
struct FuseParams {
  const bf16* a;
  int64_t a_sk, a_sm, a_sh;
  const bf16* b;
  int64_t b_sk, b_sn, b_sh;
  bf16* c;
  int64_t c_sm, c_sn, c_sh;
  int M, N, H;
};

__global__ __launch_bounds__(256) void mla_fuse_weights_kernel(FuseParams p) {
  __shared__ float as[128][64 + 4];
  __shared__ float bs[128][64 + 4];
  const int tid = threadIdx.x;
  const int mt = p.M / 64, nt = p.N / 64;
  const int blk = blockIdx.x;
  const int h = blk / (mt * nt), r = blk % (mt * nt);
  const int m0 = (r / nt) * 64, n0 = (r % nt) * 64;
  if (h >= p.H) return;
  const bf16* a = p.a + (int64_t)h * p.a_sh;
  const bf16* b = p.b + (int64_t)h * p.b_sh;
  for (int i = tid; i < 128 * 64; i += 256) {
    const int k = i >> 6, j = i & 63;
    as[k][j] = (float)a[(int64_t)k * p.a_sk + (int64_t)(m0 + j) * p.a_sm];
    bs[k][j] = (float)b[(int64_t)k * p.b_sk + (int64_t)(n0 + j) * p.b_sn];
  }
  __syncthreads();
  const int tm = tid >> 4, tn = tid & 15;
  float acc[4][4] = {};
  for (int k = 0; k < 128; ++k) {
    float av[4], bv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) av[i] = as[k][4 * tm + i];
#pragma unroll
    for (int i = 0; i < 4; ++i) bv[i] = bs[k][4 * tn + i];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
  }
  bf16* c = p.c + (int64_t)h * p.c_sh;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      c[(int64_t)(m0 + 4 * tm + i) * p.c_sm + (int64_t)(n0 + 4 * tn + j) * p.c_sn] = (bf16)acc[i][j];
}

// ---------------------------------------------------------------------------
// Weight-streaming GEMM: part[s, m, n] = sum over the k of slice s of
// X[m, k] W[n, k].
// ---------------------------------------------------------------------------
struct SkinnyParams {
  const bf16* x;    // [M, K], row stride ldx
  const bf16* w;    // [N, K], row stride ldw
  float* part;      // [S, M, N]
  int64_t ldx, ldw;
  int M, N, K;
  int S, cps;       // slices, 64-wide chunks per slice
};

constexpr int SG_CHUNK = 64;
constexpr int SG_MG = 128;      // batch rows per group (four 32-row tiles)
constexpr int SG_CH = 2;        // chunks a wave has in flight at once

template <int MSUB>
__global__ __launch_bounds__(256) void mla_skinny_gemm_kernel(SkinnyParams p) {
  constexpr int E = MSUB * 16;
  __shared__ float red[4][E][64];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, r = l & 31, g = l >> 5;
  const int ntile = p.N / 32;
  // XCD-major: the workgroups of one XCD (id mod 8) take consecutive tiles
  // of one slice, which read the same X columns
  const int G = (int)gridDim.x;
  int t;
  {
    const int xcd = (int)blockIdx.x & 7, slot = (int)blockIdx.x >> 3, q = G >> 3, rem = G & 7;
    t = xcd * q + (xcd < rem ? xcd : rem) + slot;
  }
  const int nt = t % ntile;
  t /= ntile;
  const int s = t % p.S;
  const int mg = t / p.S;
  const int nchunks = p.K / SG_CHUNK;
  const int c0 = s * p.cps, c1 = min(c0 + p.cps, nchunks);
  const bf16* wrow = p.w + (int64_t)(nt * 32 + r) * p.ldw;
  const bf16* xrow[MSUB];
#pragma unroll
  for (int ms = 0; ms < MSUB; ++ms)
    xrow[ms] = p.x + (int64_t)min(mg * SG_MG + 32 * ms + r, p.M - 1) * p.ldx;
  f32x16 acc[MSUB];
#pragma unroll
  for (int ms = 0; ms < MSUB; ++ms) acc[ms] = f32x16{};
  for (int c = c0 + w; c < c1; c += 4 * SG_CH) {
    u32x4 bw[SG_CH][4], ax[SG_CH][MSUB][4];
#pragma unroll
    for (int ch = 0; ch < SG_CH; ++ch) {
      const int k = min(c + 4 * ch, c1 - 1) * SG_CHUNK + 32 * g;
#pragma unroll
      for (int i = 0; i < 4; ++i) bw[ch][i] = *(const u32x4*)((const char*)(wrow + k) + 16 * i);
#pragma unroll
      for (int ms = 0; ms < MSUB; ++ms)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          ax[ch][ms][i] = *(const u32x4*)((const char*)(xrow[ms] + k) + 16 * i);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ch = 0; ch < SG_CH; ++ch) {
      if (ch > 0 && c + 4 * ch >= c1) break;
#pragma unroll
      for (int ms = 0; ms < MSUB; ++ms)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[ms] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ax[ch][ms][i]),
                                                            __builtin_bit_cast(bf16x8, bw[ch][i]),
                                                            acc[ms], 0, 0, 0);
    }
  }
  // the four waves' sums, added in wave order
#pragma unroll
  for (int i = 0; i < E; ++i) red[w][i][l] = acc[i >> 4][i & 15];
  __syncthreads();
#pragma unroll
  for (int q = 0; q < E / 4; ++q) {
    const int i = w * (E / 4) + q;
    const float v = ((red[0][i][l] + red[1][i][l]) + red[2][i][l]) + red[3][i][l];
    const int ms = i >> 4, j = i & 15;
    // accumulator: lane l holds column (weight row) l % 32, batch rows
    // 8 (j / 4) + 4 (l / 32) + j % 4
    const int m = mg * SG_MG + 32 * ms + 8 * (j >> 2) + 4 * g + (j & 3);
    const int n = nt * 32 + r;
    if (m < p.M) p.part[((int64_t)s * p.M + m) * p.N + n] = v;
  }
}

// ---------------------------------------------------------------------------
// Query finish: q[qop_index(b, h, c)] = bf16(cs * sum_s part[s, b, 512 h + c])
// for c < 512, and bf16(cs * q_pe[b, h, c - 512]) for the RoPE part; one
// thread per 8 consecutive c (a contiguous 16-byte piece of the layout).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mla_fused_q_finish_kernel(const float* __restrict__ part,
                                                                 int S, const bf16* __restrict__ q_pe,
                                                                 bf16* __restrict__ q, int B, int H,
                                                                 float cs) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // over B * H * 72 pieces
  if (i >= (int64_t)B * H * 72) return;
  const int piece = (int)(i % 72);
  const int64_t bh = i / 72;
  const int b = (int)(bh / H), h = (int)(bh % H);
  const int c = 8 * piece;
  float v[8];
  if (c < D_C) {
    const int64_t N = (int64_t)H * D_C;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.f;
    for (int s = 0; s < S; ++s) {
      const float* src = part + ((int64_t)s * B + b) * N + (int64_t)h * D_C + c;
      const f32x4 a = *(const f32x4*)src, a2 = *(const f32x4*)(src + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] += a[e];
        v[4 + e] += a2[e];
      }
    }
  } else {
    const bf16x8 x = *(const bf16x8*)(q_pe + bh * D_R + (c - D_C));
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (float)x[e];
  }
  bf16x8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (bf16)(v[e] * cs);
  *(bf16x8*)(q + qop_index(b, h, c, H)) = o;
}

// ---------------------------------------------------------------------------
// Merge of the attention splits into the mixed latent row o_lat (bf16,
// [B, H * 512]) and lse: the same weights as the decode's merge,
// 2^(lse_s - L) x factor_s / sum_s' 2^(lse_s' - L). One workgroup of 128
// threads per (sequence, head), four dims per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(128) void mla_merge_latent_kernel(
    const _Float16* __restrict__ part_o, const float* __restrict__ part_scale,
    const float* __restrict__ part_lse, bf16* __restrict__ o_lat, float* __restrict__ lse, int B,
    int H, int S) {
  const int bh = blockIdx.x, b = bh / H, h = bh % H, tid = threadIdx.x;
  float L = -INFINITY;
  for (int s = 0; s < S; ++s) L = fmaxf(L, part_lse[((int64_t)b * S + s) * H + h]);
  float wsum = 0.f;
  if (L > -INFINITY)
    for (int s = 0; s < S; ++s) wsum += fast_exp2(part_lse[((int64_t)b * S + s) * H + h] - L);
  const float inv = (L > -INFINITY && wsum > 0.f) ? 1.0f / wsum : 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  if (inv > 0.f) {
    for (int s = 0; s < S; ++s) {
      const int64_t row = ((int64_t)b * S + s) * H + h;
      const float wgt = fast_exp2(part_lse[row] - L) * part_scale[row] * inv;
      const f16x4 v = *(const f16x4*)(part_o + row * D_C + 4 * tid);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += wgt * (float)v[e];
    }
  }
  const bf16x4 o = {(bf16)acc[0], (bf16)acc[1], (bf16)acc[2], (bf16)acc[3]};
  *(bf16x4*)(o_lat + ((int64_t)b * H + h) * D_C + 4 * tid) = o;
  if (tid == 0 && lse)
    lse[(int64_t)b * H + h] = (L > -INFINITY) ? (L + __builtin_log2f(wsum)) * LN2 : -INFINITY;
}

// Output finish: y[m, n] = bf16(sum_s part[s, m, n]), four outputs per thread.
__global__ __launch_bounds__(256) void mla_fused_out_finish_kernel(const float* __restrict__ part,
                                                                   int S, bf16* __restrict__ y,
                                                                   int M, int N) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= (int64_t)M * N) return;
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < S; ++s) {
    const f32x4 a = *(const f32x4*)(part + (int64_t)s * M * N + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] += a[e];
  }
  const bf16x4 o = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
  *(bf16x4*)(y + i) = o;
}

}  // namespace mla
