// The two per-head projections around the attention kernel (bf16 MFMA):
//
//   absorb:  q[b,h,0:512]   = (q_nope[b,h,:] . W_UK[h]) * c,  q[b,h,512:576] = q_pe[b,h,:] * c
//            with c = softmax_scale * log2(e)  (the query absorption of
//            "How DeepSeek Rewrote the Transformer [MLA]", section "MLA:
//            compress the pair, not the heads")
//   combine: o_lat[b,h,:]   = sum_s 2^(lse_s - L) O_s / sum_s 2^(lse_s - L)
//            out[b,h,:]     = o_lat[b,h,:] . W_UV[h],  lse = L' ln 2
//            (merge of the split partials, then the value up-projection)
//
// Both are a batch of small GEMMs, one per head, with M = up to 32
// sequences. The weight is row-major with the contraction index as its slow
// index, so it is staged through LDS and fed to the MFMA with the transposing
// LDS read (ds_read_b64_tr_b16), which gives each lane 4 consecutive rows of
// one column.
#pragma once

#include "common.hpp"

namespace mla {

__device__ __forceinline__ bf16x8 tr_read_8(const char* p_lo, const char* p_hi) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p_lo);
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p_hi);
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

// ----------------------------------------------------------------------------
// absorb: one workgroup (4 waves) per (head, chunk of 32 sequences)
// ----------------------------------------------------------------------------
struct AbsorbParams {
  const bf16* q_nope;  // [B, H, 128]
  const bf16* q_pe;    // [B, H, 64]
  const bf16* w_uk;    // [H, 128, 512]
  bf16* q;             // [B, H, 576]
  int B, H, nbc;       // nbc = number of 32-sequence chunks
  float c;             // softmax_scale * log2(e)
};

constexpr int AB_KC = 32;                  // W_UK rows per LDS stage
constexpr int AB_WPITCH = D_C * 2 + 32;    // 1056 B: 4 rows' 32-byte spans hit distinct banks
constexpr int AB_APITCH = D_N * 2 + 16;    // 272 B: 8 rows' 16-byte chunks hit distinct banks

__global__ __launch_bounds__(256) void mla_absorb_kernel(AbsorbParams p) {
  __shared__ __attribute__((aligned(16))) char a_lds[32 * AB_APITCH];
  __shared__ __attribute__((aligned(16))) char w_lds[AB_KC * AB_WPITCH];
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  const int h = l >> 5, l32 = l & 31, jj = l & 15, g16 = l >> 4;
  // the nbc chunks of one head share its W_UK rows: keep them on one XCD
  int head, bc;
  {
    const int x = blockIdx.x;
    const int q_lo = x & 7, rest = x >> 3;
    bc = rest % p.nbc;
    head = (rest / p.nbc) * 8 + q_lo;
    if (head >= p.H) return;
  }
  const int b0 = bc * 32;

  // q_nope rows of the chunk -> LDS (zero rows past B); q_pe scaled copy
  for (int i = tid; i < 32 * (D_N / 8); i += 256) {
    const int r = i / (D_N / 8), c = i % (D_N / 8);
    u32x4 v = {0, 0, 0, 0};
    if (b0 + r < p.B) v = *(const u32x4*)(p.q_nope + ((int64_t)(b0 + r) * p.H + head) * D_N + 8 * c);
    *(u32x4*)(a_lds + r * AB_APITCH + 16 * c) = v;
  }
  for (int i = tid; i < 32 * D_R; i += 256) {
    const int r = i / D_R, c = i % D_R;
    if (b0 + r < p.B) {
      const int64_t bh = (int64_t)(b0 + r) * p.H + head;
      p.q[bh * D_QK + D_C + c] = (bf16)((float)p.q_pe[bh * D_R + c] * p.c);
    }
  }

  f32x16 acc[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x16{};
  const bf16* wsrc = p.w_uk + (int64_t)head * D_N * D_C;
  for (int k0 = 0; k0 < D_N; k0 += AB_KC) {
    __syncthreads();
    for (int i = tid; i < AB_KC * (D_C / 8); i += 256) {
      const int r = i / (D_C / 8), c = i % (D_C / 8);
      *(u32x4*)(w_lds + r * AB_WPITCH + 16 * c) = *(const u32x4*)(wsrc + (int64_t)(k0 + r) * D_C + 8 * c);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < AB_KC / 16; ++ks) {
      const bf16x8 a = *(const bf16x8*)(a_lds + l32 * AB_APITCH + 2 * (k0 + 16 * ks + 8 * h));
      const int r1 = 16 * ks + 8 * h + (jj >> 2);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int col = 32 * (4 * w + nt) + 16 * (g16 & 1) + 4 * (jj & 3);
        const bf16x8 bop = tr_read_8(w_lds + r1 * AB_WPITCH + 2 * col,
                                     w_lds + (r1 + 4) * AB_WPITCH + 2 * col);
        acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bop, acc[nt], 0, 0, 0);
      }
    }
  }
  // lane holds column n, rows b = 8(r/4) + 4h + r%4
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int n = 32 * (4 * w + nt) + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int bb = b0 + 8 * (r >> 2) + 4 * h + (r & 3);
      if (bb < p.B) p.q[((int64_t)bb * p.H + head) * D_QK + n] = (bf16)(acc[nt][r] * p.c);
    }
  }
}

// ----------------------------------------------------------------------------
// combine + W_UV: one workgroup (4 waves) per (head, chunk of 32 sequences)
// ----------------------------------------------------------------------------
struct CombineParams {
  const float* part_o;    // [B, S, H, 512]
  const float* part_lse;  // [B, S, H] log2 domain
  const bf16* w_uv;       // [H, 512, 128]
  bf16* out;              // [B, H, 128]
  float* lse;             // [B, H] natural log, or nullptr
  int B, H, S, nbc;
};

constexpr int CB_KC = 64;                   // W_UV rows per LDS stage
constexpr int CB_WPITCH = D_V * 2 + 32;     // 288 B
constexpr int CB_APITCH = D_C * 2 + 16;     // 1040 B

__global__ __launch_bounds__(256) void mla_combine_kernel(CombineParams p) {
  __shared__ __attribute__((aligned(16))) char a_lds[32 * CB_APITCH];
  __shared__ __attribute__((aligned(16))) char w_lds[CB_KC * CB_WPITCH];
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  const int h = l >> 5, l32 = l & 31, jj = l & 15, g16 = l >> 4;
  int head, bc;
  {
    const int x = blockIdx.x;
    const int q_lo = x & 7, rest = x >> 3;
    bc = rest % p.nbc;
    head = (rest / p.nbc) * 8 + q_lo;
    if (head >= p.H) return;
  }
  const int b0 = bc * 32;

  // merge the splits of the 32 sequences into a bf16 A tile: o_lat[b][0:512]
  for (int r = 0; r < 32; ++r) {
    const int b = b0 + r;
    float2 acc = {0.f, 0.f};
    if (b < p.B) {
      const float* lse_s = p.part_lse + (int64_t)b * p.S * p.H + head;
      float L = -INFINITY;
      for (int s = 0; s < p.S; ++s) L = fmaxf(L, lse_s[(int64_t)s * p.H]);
      if (L > -INFINITY) {
        float wsum = 0.f;
        for (int s = 0; s < p.S; ++s) {
          const float ls = lse_s[(int64_t)s * p.H];
          const float wgt = fast_exp2(ls - L);
          wsum += wgt;
          const float2 v = *(const float2*)(p.part_o + (((int64_t)b * p.S + s) * p.H + head) * D_C + 2 * tid);
          acc.x += wgt * v.x;
          acc.y += wgt * v.y;
        }
        const float inv = 1.0f / wsum;
        acc.x *= inv;
        acc.y *= inv;
        if (tid == 0 && p.lse) p.lse[(int64_t)b * p.H + head] = (L + __builtin_log2f(wsum)) * LN2;
      } else if (tid == 0 && p.lse) {
        p.lse[(int64_t)b * p.H + head] = -INFINITY;
      }
    }
    bf16x2 pk = {(bf16)acc.x, (bf16)acc.y};
    *(bf16x2*)(a_lds + r * CB_APITCH + 4 * tid) = pk;
  }

  f32x16 acc = f32x16{};
  const bf16* wsrc = p.w_uv + (int64_t)head * D_C * D_V;
  for (int k0 = 0; k0 < D_C; k0 += CB_KC) {
    __syncthreads();
    for (int i = tid; i < CB_KC * (D_V / 8); i += 256) {
      const int r = i / (D_V / 8), c = i % (D_V / 8);
      *(u32x4*)(w_lds + r * CB_WPITCH + 16 * c) = *(const u32x4*)(wsrc + (int64_t)(k0 + r) * D_V + 8 * c);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < CB_KC / 16; ++ks) {
      const bf16x8 a = *(const bf16x8*)(a_lds + l32 * CB_APITCH + 2 * (k0 + 16 * ks + 8 * h));
      const int r1 = 16 * ks + 8 * h + (jj >> 2);
      const int col = 32 * w + 16 * (g16 & 1) + 4 * (jj & 3);
      const bf16x8 bop = tr_read_8(w_lds + r1 * CB_WPITCH + 2 * col, w_lds + (r1 + 4) * CB_WPITCH + 2 * col);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bop, acc, 0, 0, 0);
    }
  }
  const int n = 32 * w + l32;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int bb = b0 + 8 * (r >> 2) + 4 * h + (r & 3);
    if (bb < p.B) p.out[((int64_t)bb * p.H + head) * D_V + n] = (bf16)acc[r];
  }
}

}  // namespace mla
