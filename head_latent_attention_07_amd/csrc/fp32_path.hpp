// fp32 MLA decode on the vector ALUs (queries, weights, cache and output all
// binary32). Same three stages as the bf16 path (absorb, split attention,
// merge + W_UV) with plain fp32 FMA arithmetic; used for fp32 workloads, where
// the MFMA operand types would lose precision.
#pragma once

#include "common.hpp"

namespace mla {

// q[b,h,0:512] = (q_nope[b,h,:] . W_UK[h]) * c ; q[b,h,512:576] = q_pe * c
// Four workgroups (256 threads) per (b, h), one per 128 output columns, so
// that the 256 KB of W_UK[h] stream through four CUs: thread (kh, col) =
// (tid / 128, tid % 128) sums the 64 contraction rows 64 kh .. 64 kh + 63 of
// its column with four independent partial sums (one coalesced 512-byte
// row segment per step across the half-workgroup, 16 loads in flight per
// thread), and the two halves are added through LDS.
__global__ __launch_bounds__(256) void mla_absorb_f32_kernel(const float* __restrict__ q_nope,
                                                             const float* __restrict__ q_pe,
                                                             const float* __restrict__ w_uk,
                                                             float* __restrict__ q, int H, float c) {
  __shared__ float qn[D_N];
  __shared__ float half[128];
  const int bh = blockIdx.x >> 2, quarter = blockIdx.x & 3, head = bh % H, tid = threadIdx.x;
  if (tid < D_N) qn[tid] = q_nope[(int64_t)bh * D_N + tid];
  __syncthreads();
  const int kh = tid >> 7, col = 128 * quarter + (tid & 127);
  const float* w = w_uk + (int64_t)head * D_N * D_C + (int64_t)(64 * kh) * D_C + col;
  float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 16
  for (int k = 0; k < 64; ++k) a[k & 3] = fmaf(qn[64 * kh + k], w[(int64_t)k * D_C], a[k & 3]);
  const float sum = (a[0] + a[1]) + (a[2] + a[3]);
  if (kh == 1) half[tid & 127] = sum;
  __syncthreads();
  float* qo = q + (int64_t)bh * D_QK;
  if (kh == 0) qo[col] = (sum + half[tid]) * c;
  if (quarter == 0 && tid >= 128 && tid < 128 + D_R)
    qo[D_C + tid - 128] = q_pe[(int64_t)bh * D_R + tid - 128] * c;
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
constexpr int F32_U = 8;   // tokens per wave per step of the score loop

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
  const int raw_len = p.lengths[b];
  debug_flag(raw_len < 0 || raw_len > p.max_len, DBG_LENGTH);
  const int len = min(max(raw_len, 0), p.max_len);
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
  // scores: wave wv takes tokens F32_U wv .. F32_U wv + F32_U - 1, then
  // 4 F32_U further, ...; its 64 lanes read a row together (lane l: latent
  // dims l + 64 k, RoPE dim l: 9 coalesced 256-byte reads per row) against
  // their 9 query values in registers, and the dot product is summed across
  // the wave
  float qv[9];
#pragma unroll
  for (int k = 0; k < 8; ++k) qv[k] = qs[lane + 64 * k];
  qv[8] = qs[D_C + lane];
  // (F32_U tokens at a time, so that their loads are in flight together and
  // their reductions overlap; a token past the split's end repeats the last
  // one and is not stored)
  float mloc = -INFINITY;
  for (int t = F32_U * wv; t < n; t += 4 * F32_U) {
    float a[F32_U];
#pragma unroll
    for (int u = 0; u < F32_U; ++u) {
      const int64_t row = rowof[min(t + u, n - 1)];
      const float* c = p.latent + row * p.latent_stride;
      const float* r = p.rope + row * p.rope_stride;
      a[u] = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) a[u] = fmaf(qv[k], c[lane + 64 * k], a[u]);
      a[u] = fmaf(qv[8], r[lane], a[u]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
#pragma unroll
      for (int u = 0; u < F32_U; ++u) a[u] += __shfl_xor(a[u], o, 64);
#pragma unroll
    for (int u = 0; u < F32_U; ++u) {
      if (t + u < n) {
        if (lane == 0) sc[t + u] = a[u];
        mloc = fmaxf(mloc, a[u]);
      }
    }
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
#pragma unroll 16
  for (int t = 0; t < n; ++t) {   // (16 rows' loads in flight)
    const float* c = p.latent + rowof[t] * p.latent_stride;
    o0 = fmaf(sc[t], c[tid], o0);
    o1 = fmaf(sc[t], c[tid + 256], o1);
  }
  po[tid] = o0 * inv;
  po[tid + 256] = o1 * inv;
  if (tid == 0) *pl = m + log2f(lsum);
}

// merge of the splits + W_UV. Four workgroups (256 threads) per (b, h), one
// per 32 output columns, so that the 256 KB of W_UV[h] stream through four
// CUs: each merges the S split rows into the 512 latent values (thread tid:
// dims tid and tid + 256; eight splits' loads in flight),
// then thread (kq, col) = (tid / 32, tid % 32) sums the contraction rows
// 64 kq .. 64 kq + 63 of its column with four independent partial sums
// (128-byte row segments, 16 loads in flight), and the eight partial sums of
// a column are added through LDS.
__global__ __launch_bounds__(256) void mla_combine_f32_kernel(const float* __restrict__ part_o,
                                                              const float* __restrict__ part_lse,
                                                              const float* __restrict__ w_uv,
                                                              float* __restrict__ out,
                                                              float* __restrict__ lse, int H, int S) {
  __shared__ float ol[D_C];
  __shared__ float red[8][32];
  __shared__ float mred[4];
  const int bh = blockIdx.x >> 2, quarter = blockIdx.x & 3, b = bh / H, head = bh % H;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const float* pl = part_lse + (int64_t)b * S * H + head;   // split s at pl[s * H]
  // L = max of the splits' lse values (loaded S / 256 per thread at a time)
  float mx = -INFINITY;
  for (int s = tid; s < S; s += 256) mx = fmaxf(mx, pl[(int64_t)s * H]);
  mx = wave_max(mx);
  if (lane == 0) mred[wv] = mx;
  __syncthreads();
  const float L = fmaxf(fmaxf(mred[0], mred[1]), fmaxf(mred[2], mred[3]));
  float wsum = 0.f;
  float acc[2] = {0.f, 0.f};
  const float* o = part_o + ((int64_t)b * S * H + head) * D_C + tid;
#pragma unroll 8
  for (int s = 0; s < S; ++s) {
    const float wgt = (L > -INFINITY) ? exp2f(pl[(int64_t)s * H] - L) : 0.f;
    wsum += wgt;
    for (int k = 0; k < 2; ++k) acc[k] = fmaf(wgt, o[(int64_t)s * H * D_C + 256 * k], acc[k]);
  }
  for (int k = 0; k < 2; ++k) ol[tid + 256 * k] = (wsum > 0.f) ? acc[k] / wsum : 0.f;
  __syncthreads();
  const int kq = tid >> 5, col = 32 * quarter + (tid & 31);
  const float* w = w_uv + (int64_t)head * D_C * D_V + (int64_t)(64 * kq) * D_V + col;
  float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 16
  for (int k = 0; k < 64; ++k) a[k & 3] = fmaf(ol[64 * kq + k], w[(int64_t)k * D_V], a[k & 3]);
  red[kq][tid & 31] = (a[0] + a[1]) + (a[2] + a[3]);
  __syncthreads();
  if (tid < 32) {
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) sum += red[q][tid];
    out[(int64_t)bh * D_V + col] = sum;
  }
  if (quarter == 0 && tid == 0 && lse)
    lse[bh] = (L > -INFINITY) ? (L + log2f(wsum)) * LN2 : -INFINITY;
}

}  // namespace mla
