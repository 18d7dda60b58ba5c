// Cache append: write the new token's latent row and RoPE-rotated key into the
// cache ("How DeepSeek Rewrote the Transformer [MLA]", section "MLA: compress
// the pair, not the heads": c_KV and the decoupled key k^R both go to the
// cache, 576 numbers per token per layer).
#pragma once

#include "common.hpp"

namespace mla {

struct AppendParams {
  const void* c_kv;           // [B, 512]
  const void* k_pe;           // [B, 64], un-rotated
  int in_bf16;                // input type: 1 bf16, 0 f32
  const int32_t* positions;   // [B]
  void* latent;
  int64_t latent_stride;
  void* rope;
  int64_t rope_stride;
  bf16* scales;               // fp8 cache only
  int cache_kind;             // CacheKind
  int64_t rows, seq_capacity;
  const int32_t* block_table;
  int max_blocks, block_size;
  double theta;
  // instead of c_kv / k_pe: the fp32 partial sums [S, B, 576] that a
  // down-projection left in its workspace (nullptr: use c_kv / k_pe)
  const float* part;
  int part_slices;
  int rows_in_batch;   // B of the partials' [S, B, 576] layout
};

// OCP e4m3fn code of v, round to nearest even, saturating to +-448.
__device__ __forceinline__ uint32_t e4m3fn_encode(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  if (a >= 448.0f) return sign | 0x7Eu;
  if (a < 0.015625f) {                      // below 2^-6: subnormal step 2^-9
    return sign | (uint32_t)rintf(a * 512.0f);  // 8 lands on 0x08 = 2^-6
  }
  int e;
  const float m = frexpf(a, &e);            // a = m 2^e, m in [0.5, 1)
  int E = e - 1;                            // a = (2m) 2^E, 2m in [1, 2)
  float q = rintf((2.0f * m - 1.0f) * 8.0f);
  if (q == 8.0f) { q = 0.0f; E += 1; }
  return sign | (uint32_t)(((E + 7) << 3) | (int)q);
}

// Rotate and store one row, given its values in fp32: lane l of the wave
// holds latent values x = c[8l .. 8l+7] and (xe, xo) = the un-rotated RoPE
// pair (2l', 2l'+1), l' = l mod 32 (lanes 32..63 repeat a pair and do not
// store it). The rotation angle is computed before the destination row is
// known (its latency overlaps that of the position and block-table reads).
__device__ __forceinline__ void append_store(const AppendParams& p, int b, int l,
                                             const float (&x)[8], double xe, double xo);

// The token's position and the rotation of lane l's pair, (cos, sin) of
// pos * theta^(-2 l' / 64) in double precision: needs only the position, so
// a caller can start it before the row's values are known.
struct RopeAngle {
  int pos;
  double cs, sn;
};

__device__ __forceinline__ RopeAngle append_angle(const AppendParams& p, int b, int l) {
  const int lp = l & (D_R / 2 - 1);
  RopeAngle a;
  a.pos = p.positions[b];
  const double freq = pow(p.theta, -2.0 * (double)lp / (double)D_R);
  sincos((double)a.pos * freq, &a.sn, &a.cs);
  return a;
}

__device__ __forceinline__ void append_write(const AppendParams& p, int b, int l,
                                             const float (&x)[8], double xe, double xo,
                                             const RopeAngle& ang);

// Cache row of the new token of sequence b at position pos (contiguous or
// paged); false if it falls outside the cache (then nothing is written).
__device__ __forceinline__ bool append_dest(const AppendParams& p, int b, int pos, int64_t* row) {
  int64_t r;
  if (p.block_table) {
    const bool in_cap = pos >= 0 && pos / p.block_size < p.max_blocks;
    debug_flag(!in_cap, DBG_POSITION);
    if (!in_cap) return false;
    r = (int64_t)p.block_table[(int64_t)b * p.max_blocks + pos / p.block_size] * p.block_size +
        pos % p.block_size;
  } else {
    const bool in_cap = pos >= 0 && pos < p.seq_capacity;
    debug_flag(!in_cap, DBG_POSITION);
    if (!in_cap) return false;
    r = (int64_t)b * p.seq_capacity + pos;
  }
  debug_flag(r < 0 || r >= p.rows, DBG_BLOCK);
  if (r < 0 || r >= p.rows) return false;
  *row = r;
  return true;
}

// The row of sequence b as the sum of a down-projection's S partials, added
// in the order of the down-projection's own append kernel (slices of each
// residue mod 4 in increasing order, then the four residues in order), so
// both give the same bits. Lane layout as in append_row.
__device__ __forceinline__ void append_row_projected(const AppendParams& p, int b, int l) {
  const int lp = l & (D_R / 2 - 1), S = p.part_slices;
  float acc[4][10];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int i = 0; i < 10; ++i) acc[r][i] = 0.f;
  for (int s0 = 0; s0 < S; s0 += 4) {
    f32x4 v0[4], v1[4];
    f32x2 pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {   // clamped loads, the extra ones discarded
      const float* row = p.part + ((int64_t)min(s0 + r, S - 1) * p.rows_in_batch + b) * D_QK;
      v0[r] = *(const f32x4*)(row + 8 * l);
      v1[r] = *(const f32x4*)(row + 8 * l + 4);
      pr[r] = *(const f32x2*)(row + D_C + 2 * lp);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (s0 + r < S) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[r][i] += v0[r][i];
          acc[r][4 + i] += v1[r][i];
        }
        acc[r][8] += pr[r][0];
        acc[r][9] += pr[r][1];
      }
    }
  }
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = ((acc[0][i] + acc[1][i]) + acc[2][i]) + acc[3][i];
  const float xe = ((acc[0][8] + acc[1][8]) + acc[2][8]) + acc[3][8];
  const float xo = ((acc[0][9] + acc[1][9]) + acc[2][9]) + acc[3][9];
  append_store(p, b, l, x, (double)xe, (double)xo);
}

// one wave per sequence: lane l owns latent values 8l..8l+7 and, for l < 32,
// the RoPE pair (2l, 2l+1), read from the c_kv / k_pe inputs.
__device__ __forceinline__ void append_row(const AppendParams& p, int b, int l) {
  if (p.part) {
    append_row_projected(p, b, l);
    return;
  }
  float x[8];
  if (p.in_bf16) {
    const bf16x8 v = *(const bf16x8*)((const bf16*)p.c_kv + (int64_t)b * D_C + 8 * l);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)v[i];
  } else {
    const f32x4* src = (const f32x4*)((const float*)p.c_kv + (int64_t)b * D_C + 8 * l);
    const f32x4 v0 = src[0], v1 = src[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[i] = v0[i]; x[4 + i] = v1[i]; }
  }
  double xe = 0.0, xo = 0.0;
  const int lp = l & (D_R / 2 - 1);   // lanes 32..63 repeat a pair (unused)
  if (p.in_bf16) {
    const bf16* k = (const bf16*)p.k_pe + (int64_t)b * D_R;
    xe = (float)k[2 * lp];
    xo = (float)k[2 * lp + 1];
  } else {
    const float* k = (const float*)p.k_pe + (int64_t)b * D_R;
    xe = k[2 * lp];
    xo = k[2 * lp + 1];
  }
  append_store(p, b, l, x, xe, xo);
}

__device__ __forceinline__ void append_store(const AppendParams& p, int b, int l,
                                             const float (&x)[8], double xe, double xo) {
  append_write(p, b, l, x, xe, xo, append_angle(p, b, l));
}

__device__ __forceinline__ void append_write(const AppendParams& p, int b, int l,
                                             const float (&x)[8], double xe, double xo,
                                             const RopeAngle& ang) {
  const int pos = ang.pos;
  const double cs = ang.cs, sn = ang.sn;
  const float r0 = (float)(xe * cs - xo * sn);
  const float r1 = (float)(xe * sn + xo * cs);

  int64_t r;
  if (!append_dest(p, b, pos, &r)) return;

  if (p.cache_kind == CACHE_F32) {
    float* dst = (float*)p.latent + r * p.latent_stride + 8 * l;
    *(f32x4*)dst = f32x4{x[0], x[1], x[2], x[3]};
    *(f32x4*)(dst + 4) = f32x4{x[4], x[5], x[6], x[7]};
    if (l < D_R / 2) *(f32x2*)((float*)p.rope + r * p.rope_stride + 2 * l) = f32x2{r0, r1};
  } else if (p.cache_kind == CACHE_BF16) {
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (bf16)x[i];
    *(bf16x8*)((bf16*)p.latent + r * p.latent_stride + 8 * l) = v;
    if (l < D_R / 2) *(bf16x2*)((bf16*)p.rope + r * p.rope_stride + 2 * l) = bf16x2{(bf16)r0, (bf16)r1};
  } else {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
    if (l < D_R / 2) amax = fmaxf(amax, fmaxf(fabsf(r0), fabsf(r1)));
    amax = wave_max(amax);
    float s;
    if (amax == 0.f) {
      s = 1.0f;
    } else {
      const float s32 = amax / 448.0f;
      s = (s32 < 1.17549435e-38f) ? 1.17549435e-38f : (float)(bf16)s32;
    }
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= e4m3fn_encode(x[i] / s) << (8 * i);
      hi |= e4m3fn_encode(x[4 + i] / s) << (8 * i);
    }
    *(u32x2*)((uint8_t*)p.latent + r * p.latent_stride + 8 * l) = u32x2{lo, hi};
    if (l < D_R / 2) {
      const uint32_t c0 = e4m3fn_encode(r0 / s), c1 = e4m3fn_encode(r1 / s);
      *(uint16_t*)((uint8_t*)p.rope + r * p.rope_stride + 2 * l) = (uint16_t)(c0 | (c1 << 8));
    }
    if (l == 0) p.scales[r] = (bf16)s;
  }
}

__global__ __launch_bounds__(64) void mla_append_kernel(AppendParams p) {
  append_row(p, blockIdx.x, threadIdx.x);
}

}  // namespace mla
