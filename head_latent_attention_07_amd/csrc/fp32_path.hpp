// fp32 MLA decode on the vector ALUs (queries, weights, cache and output all
// binary32). Same three stages as the bf16 path (absorb, split attention,
// merge + W_UV) with plain fp32 FMA arithmetic; used for fp32 workloads, where
// the MFMA operand types would lose precision.
#pragma once

#include "common.hpp"

namespace mla {

// q[b,h,0:512] = (q_nope[b,h,:] . W_UK[h]) * c ; q[b,h,512:576] = q_pe * c
// one workgroup (256 threads) per (b, h); thread owns columns tid, tid+256
__global__ __launch_bounds__(256) void mla_absorb_f32_kernel(const float* __restrict__ q_nope,
                                                             const float* __restrict__ q_pe,
                                                             const float* __restrict__ w_uk,
                                                             float* __restrict__ q, int H, float c) {
  __shared__ float qn[D_N];
  const int bh = blockIdx.x, head = bh % H, tid = threadIdx.x;
  if (tid < D_N) qn[tid] = q_nope[(int64_t)bh * D_N + tid];
  __syncthreads();
  const float* w = w_uk + (int64_t)head * D_N * D_C;
  float a0 = 0.f, a1 = 0.f;
  for (int k = 0; k < D_N; ++k) {
    a0 = fmaf(qn[k], w[k * D_C + tid], a0);
    a1 = fmaf(qn[k], w[k * D_C + tid + 256], a1);
  }
  float* qo = q + (int64_t)bh * D_QK;
  qo[tid] = a0 * c;
  qo[tid + 256] = a1 * c;
  if (tid < D_R) qo[D_C + tid] = q_pe[(int64_t)bh * D_R + tid] * c;
}

struct DecodeF32Params {
  const float* q;           // [B, H, 576] pre-scaled by softmax_scale*log2(e)
  const float* latent;
  int64_t latent_stride;
  const float* rope;
  int64_t rope_stride;
  int64_t rows, seq_capacity;
  const int32_t* block_table;
  int max_blocks, block_size;
  const int32_t* lengths;
  int max_len;
  int B, H, S, tokens_per_split;
  float* part_o;            // [B, S, H, 512]
  float* part_lse;          // [B, S, H] log2
};

constexpr int F32_MAX_SPLIT = 1024;

// one workgroup (256 threads) per (b, h, split)
__global__ __launch_bounds__(256) void mla_decode_f32_kernel(DecodeF32Params p) {
  __shared__ float qs[D_QK];
  __shared__ float sc[F32_MAX_SPLIT];
  __shared__ int64_t rowof[F32_MAX_SPLIT];
  __shared__ float red[4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int s = blockIdx.x % p.S;
  const int bh = blockIdx.x / p.S;
  const int b = bh / p.H, head = bh % p.H;
  const int len = min(max(p.lengths[b], 0), p.max_len);
  const int t0 = s * p.tokens_per_split;
  const int t1 = min(t0 + p.tokens_per_split, len);
  float* po = p.part_o + (((int64_t)b * p.S + s) * p.H + head) * D_C;
  float* pl = p.part_lse + ((int64_t)b * p.S + s) * p.H + head;
  if (t0 >= t1) {
    for (int d = tid; d < D_C; d += 256) po[d] = 0.f;
    if (tid == 0) *pl = -INFINITY;
    return;
  }
  const int n = t1 - t0;
  for (int d = tid; d < D_QK; d += 256) qs[d] = p.q[(int64_t)bh * D_QK + d];
  for (int t = tid; t < n; t += 256)
    rowof[t] = cache_row(b, t0 + t, p.seq_capacity, p.block_table, p.max_blocks, p.block_size, p.rows);
  __syncthreads();
  // scores: one token per thread
  float mloc = -INFINITY;
  for (int t = tid; t < n; t += 256) {
    const float* c = p.latent + rowof[t] * p.latent_stride;
    const float* r = p.rope + rowof[t] * p.rope_stride;
    float a = 0.f;
    for (int d = 0; d < D_C; ++d) a = fmaf(qs[d], c[d], a);
    for (int d = 0; d < D_R; ++d) a = fmaf(qs[D_C + d], r[d], a);
    sc[t] = a;
    mloc = fmaxf(mloc, a);
  }
  mloc = wave_max(mloc);
  if (lane == 0) red[wv] = mloc;
  __syncthreads();
  const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float lloc = 0.f;
  for (int t = tid; t < n; t += 256) {
    const float e = exp2f(sc[t] - m);
    sc[t] = e;
    lloc += e;
  }
  lloc = wave_sum(lloc);
  if (lane == 0) red[wv] = lloc;
  __syncthreads();
  const float lsum = red[0] + red[1] + red[2] + red[3];
  const float inv = 1.0f / lsum;
  // O[d] = sum_t p_t c_t[d]; thread owns dims tid, tid+256
  float o0 = 0.f, o1 = 0.f;
  for (int t = 0; t < n; ++t) {
    const float* c = p.latent + rowof[t] * p.latent_stride;
    o0 = fmaf(sc[t], c[tid], o0);
    o1 = fmaf(sc[t], c[tid + 256], o1);
  }
  po[tid] = o0 * inv;
  po[tid + 256] = o1 * inv;
  if (tid == 0) *pl = m + log2f(lsum);
}

// merge of the splits + W_UV; one workgroup (128 threads) per (b, h)
__global__ __launch_bounds__(128) void mla_combine_f32_kernel(const float* __restrict__ part_o,
                                                              const float* __restrict__ part_lse,
                                                              const float* __restrict__ w_uv,
                                                              float* __restrict__ out,
                                                              float* __restrict__ lse, int H, int S) {
  __shared__ float ol[D_C];
  const int bh = blockIdx.x, b = bh / H, head = bh % H, tid = threadIdx.x;
  float L = -INFINITY;
  for (int s = 0; s < S; ++s) L = fmaxf(L, part_lse[((int64_t)b * S + s) * H + head]);
  float wsum = 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  if (L > -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const float wgt = exp2f(part_lse[((int64_t)b * S + s) * H + head] - L);
      wsum += wgt;
      const float* o = part_o + (((int64_t)b * S + s) * H + head) * D_C;
      for (int k = 0; k < 4; ++k) acc[k] = fmaf(wgt, o[tid + 128 * k], acc[k]);
    }
    for (int k = 0; k < 4; ++k) ol[tid + 128 * k] = acc[k] / wsum;
  } else {
    for (int k = 0; k < 4; ++k) ol[tid + 128 * k] = 0.f;
  }
  __syncthreads();
  const float* w = w_uv + (int64_t)head * D_C * D_V;
  float a = 0.f;
  for (int k = 0; k < D_C; ++k) a = fmaf(ol[k], w[k * D_V + tid], a);
  out[(int64_t)bh * D_V + tid] = a;
  if (tid == 0 && lse) lse[bh] = (L > -INFINITY) ? (L + log2f(wsum)) * LN2 : -INFINITY;
}

}  // namespace mla
