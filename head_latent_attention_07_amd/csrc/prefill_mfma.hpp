// Prefill (and chunked prefill) of MLA attention in the recompute mode, on
// gfx950 bf16 MFMA.
//
// For a chunk of T new queries per sequence whose rows are the last T of the
// sequence's n cached rows, query i (position n - T + i) attends to rows
// 0 .. n - T + i: softmax(Q K^T / sqrt(d_k) + M) V with the causal mask M
// ("How DeepSeek Rewrote the Transformer [MLA]", section "Classic attention
// and the cost of the KV cache"). With many queries per sequence the keys
// and values are worth decompressing once per head (the "recompute" mode of
// "Como a MLA da DeepSeek cortou 93% da memoria", section "O preco da
// economia: mais contas"): K_h = C W_UK[h]^T and V_h = C W_UV[h] ("DeepSeek
// AI efficiency, architecture, benchmarks", section "Architectural
// Innovations: Multi-Head Latent Attention (MLA)", the equations for K and
// V), so attention runs at d_qk = 128 + 64 (the decoupled RoPE key, shared by
// all heads) and d_v = 128 instead of over the 576-wide latent.
//
// Three launches:
//   * mla_wuv_transpose_kernel: W_UV[h] [512, 128] -> [128, 512], so that
//     both decompressions take their weight rows with the contraction index
//     contiguous;
//   * mla_prefill_expand_kernel: for a tile of 128 tokens and one head,
//     [K_h | V_h]^T = [W_UK[h] ; W_UV[h]^T] C^T on bf16 MFMA (A = weight
//     rows, B = latent rows, both read 16 bytes at a time from swizzled LDS
//     stages); K_h is stored as fp16 [B, H, cap, 128], V_h transposed, as
//     fp16 [B, H, 128, cap] with the tokens of every 16 in the order the PV
//     product consumes them (vt_pos), so that the attention kernel reads its
//     PV operand with plain 16-byte LDS reads; the head-0 workgroups also
//     copy the tokens' RoPE keys to a contiguous fp16 [B, cap, 64] array;
//   * mla_prefill_attn_kernel: causal flash attention for 128 queries of one
//     (sequence, head) (4 waves x 32 queries). Key tiles of 64 keys (K | k^R
//     | V^T, 40 KB) stream through two LDS stages with direct-to-LDS loads;
//     S^T = K Q^T and O^T += V^T P^T run on v_mfma_f32_32x32x16_f16 with the
//     same token-slot permutation as the decode kernel (the S^T accumulator
//     is the PV B operand as is), online softmax in base 2 with one rescale
//     of the 64 O^T registers per tile.
//
// The attention operands (queries, decompressed keys and values, weights P)
// are fp16, not bf16: the f16 and bf16 matrix instructions have the same
// rate, and fp16's 11-bit significand makes the rounding of K, V and P 8x
// smaller than bf16's, which would otherwise each add about the error of
// the bf16 output itself. Values are well inside fp16's range here (K and V
// are latent rows times weight rows, P lies in [0, 1]); larger magnitudes
// saturate at +-65504.
#pragma once

#include "common.hpp"
#include "decode_mfma.hpp"

namespace mla {

// ---------------------------------------------------------------------------
// W_UV[h] transposed: [H, 512, 128] -> [H, 128, 512]; one workgroup per
// (head, 64 x 64 block), through LDS.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mla_wuv_transpose_kernel(const bf16* __restrict__ w_uv,
                                                                bf16* __restrict__ w_uvt, int H) {
  __shared__ bf16 t[64][66];
  const int blk = blockIdx.x, head = blk / 16, rb = (blk / 2) % 8, cb = blk % 2;
  if (head >= H) return;
  const bf16* src = w_uv + (int64_t)head * D_C * D_V;
  bf16* dst = w_uvt + (int64_t)head * D_V * D_C;
  const int tid = threadIdx.x;
  for (int i = tid; i < 64 * 64; i += 256) {
    const int r = i >> 6, c = i & 63;   // r over latent dims, c over value dims
    t[r][c] = src[(int64_t)(64 * rb + r) * D_V + 64 * cb + c];
  }
  __syncthreads();
  for (int i = tid; i < 64 * 64; i += 256) {
    const int r = i >> 6, c = i & 63;   // r over value dims, c over latent dims
    dst[(int64_t)(64 * cb + r) * D_C + 64 * rb + c] = t[c][r];
  }
}

// ---------------------------------------------------------------------------
// Decompression GEMM
// ---------------------------------------------------------------------------
struct ExpandParams {
  const bf16* latent;
  int64_t latent_stride;
  const bf16* rope;
  int64_t rope_stride;
  int64_t rows, seq_capacity;
  const int32_t* block_table;
  int max_blocks, block_size;
  const int32_t* lengths;
  const bf16* w_uk;    // [H, 128, 512]
  const bf16* w_uvt;   // [H, 128, 512]
  _Float16* kx;        // [B, H, cap, 128]
  _Float16* vx;        // [B, H, 128, cap], tokens in vt_pos order
  _Float16* kpx;       // [B, cap, 64]
  int B, H, cap, max_len;
};

// Position of token k of an aligned group of 16 in the transposed values:
// the PV B operand (the S^T accumulator as is) gives lane half h of k-step
// ks the tokens 4h .. 4h+3 and 8+4h .. 8+4h+3 of its 16, in that order, so
// they are stored at 8h .. 8h+7: order 0-3, 8-11, 4-7, 12-15.
__host__ __device__ constexpr int vt_pos(int k) {
  return 8 * ((k >> 2) & 1) + 4 * ((k >> 3) & 1) + (k & 3);
}

__device__ __forceinline__ _Float16 f16_sat(float x) {
  return (_Float16)fminf(fmaxf(x, -65504.0f), 65504.0f);
}

constexpr int EX_ROWS = 128;                       // tokens per workgroup
constexpr int EX_KC = 32;                          // contraction elements per stage
constexpr int EX_A_BYTES = EX_ROWS * EX_KC * 2;    // 8 KB of latent rows
constexpr int EX_B_BYTES = 2 * D_N * EX_KC * 2;    // 16 KB of weight rows (K rows, then V rows)
constexpr int EX_STAGE = EX_A_BYTES + EX_B_BYTES;  // 24 KB

// 64-byte rows of 4 chunks: chunk c of row r at c ^ ((r >> 2) & 3), so a
// 16-byte read of one chunk from 16 consecutive rows hits 16 distinct
// 16-byte bank groups.
__device__ __forceinline__ int ex_swz(int r) { return (r >> 2) & 3; }

__device__ __forceinline__ int64_t prefill_row(const int32_t* __restrict__ table, int b, int t,
                                               int64_t seq_capacity, int max_blocks,
                                               int block_size, int64_t rows) {
  int64_t r;
  if (table) {
    const int bi = min(t / block_size, max_blocks - 1);
    r = (int64_t)table[(int64_t)b * max_blocks + bi] * block_size + t % block_size;
  } else {
    r = (int64_t)b * seq_capacity + t;
  }
  // (every caller passes a token of the sequence: t < its length)
  const bool ok = r >= 0 && r < rows;
  debug_flag(!ok, DBG_BLOCK);
  return ok ? r : 0;
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mla_prefill_expand_kernel(ExpandParams p) {
  __shared__ __attribute__((aligned(16))) char lds[2 * EX_STAGE];
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ntile = (p.max_len + EX_ROWS - 1) / EX_ROWS;
  // XCD-major work order (workgroups go round-robin to the 8 XCDs): XCD x
  // takes the heads h = x mod 8, each over all sequences and token tiles, so
  // a head's 256 KB of weight rows stays in that XCD's L2 while its tiles run
  const int xcd = blockIdx.x & 7, i = blockIdx.x >> 3;
  const int per_head = p.B * ntile;
  const int hl = i / per_head, rem = i - hl * per_head;
  const int head = hl * 8 + xcd;
  const int b = rem / ntile, rt = rem - b * ntile;
  if (head >= p.H) return;
  const int raw_len = p.lengths[b];
  debug_flag(raw_len < 0 || raw_len > p.max_len, DBG_LENGTH);
  const int len = min(max(raw_len, 0), p.max_len);
  const int t0 = rt * EX_ROWS;
  if (t0 >= len) return;

  // this thread's global pieces of a stage: latent rows r = tid / 4 and
  // 64 + tid / 4 (chunk tid % 4), weight rows tid / 4 + 64 m (m = 0..3)
  const int cc = tid & 3, r0 = tid >> 2;
  const bf16* arow[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int t = min(t0 + r0 + 64 * m, len - 1);
    arow[m] = p.latent + prefill_row(p.block_table, b, t, p.seq_capacity, p.max_blocks,
                                     p.block_size, p.rows) * p.latent_stride + 8 * cc;
  }
  const bf16* brow[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int d = r0 + 64 * m;   // 0..255: K rows, then V rows
    brow[m] = (d < D_N ? p.w_uk + ((int64_t)head * D_N + d) * D_C
                       : p.w_uvt + ((int64_t)head * D_N + d - D_N) * D_C) + 8 * cc;
  }
  u32x4 ga[2], gb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int m = 0; m < 2; ++m) ga[m] = *(const u32x4*)(arow[m] + k0);
#pragma unroll
    for (int m = 0; m < 4; ++m) gb[m] = *(const u32x4*)(brow[m] + k0);
  };
  auto lstore = [&](char* st) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int r = r0 + 64 * m;
      *(u32x4*)(st + r * 64 + 16 * (cc ^ ex_swz(r))) = ga[m];
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int r = r0 + 64 * m;
      *(u32x4*)(st + EX_A_BYTES + r * 64 + 16 * (cc ^ ex_swz(r))) = gb[m];
    }
  };

  // wave (wr, wc): tokens 64 wr .. 64 wr + 63 (two 32-token tiles), output
  // rows 128 wc .. 128 wc + 127 (wc 0: K, 1: V; four 32-row tiles)
  const int wr = w & 1, wc = w >> 1;
  const int kg = l >> 5, l32 = l & 31;
  f32x16 acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int u = 0; u < 2; ++u) acc[a][u] = f32x16{};

  gload(0);
  lstore(lds);
  __syncthreads();
  constexpr int NCH = D_C / EX_KC;   // 16 stages of 32
  for (int kc = 0; kc < NCH; ++kc) {
    char* st = lds + (kc & 1) * EX_STAGE;
    if (kc + 1 < NCH) gload((kc + 1) * EX_KC);
#pragma unroll
    for (int ks = 0; ks < EX_KC / 16; ++ks) {
      const int c = 2 * ks + kg;
      bf16x8 bop[2], aop[4];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int r = 64 * wr + 32 * u + l32;
        bop[u] = *(const bf16x8*)(st + r * 64 + 16 * (c ^ ex_swz(r)));
      }
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int r = 128 * wc + 32 * a + l32;
        aop[a] = *(const bf16x8*)(st + EX_A_BYTES + r * 64 + 16 * (c ^ ex_swz(r)));
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int u = 0; u < 2; ++u)
          acc[a][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[a], bop[u], acc[a][u], 0, 0, 0);
    }
    if (kc + 1 < NCH) lstore(lds + ((kc + 1) & 1) * EX_STAGE);
    __syncthreads();
  }

  // acc[a][u]: lane holds token t = t0 + 64 wr + 32 u + l32 and output rows
  // 32 a + 8 g + 4 kg + (0..3) in registers 4 g .. 4 g + 3
  if (wc == 0) {
    _Float16* dst = p.kx + ((int64_t)b * p.H + head) * p.cap * D_N;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = t0 + 64 * wr + 32 * u + l32;
      if (t < len) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f16x4 v = {f16_sat(acc[a][u][4 * g]), f16_sat(acc[a][u][4 * g + 1]),
                             f16_sat(acc[a][u][4 * g + 2]), f16_sat(acc[a][u][4 * g + 3])};
            *(f16x4*)(dst + (int64_t)t * D_N + 32 * a + 8 * g + 4 * kg) = v;
          }
      }
    }
  } else {
    // V^T of this wave's 64 tokens: through its own 16 KB of the (now idle)
    // stages as [128 rows][64 tokens in vt_pos order], then out as 16-byte
    // runs of 8 tokens. Every token of the tile is stored (those past the
    // sequence's end from its last row: finite, and weighted 0 by the
    // attention's mask).
    char* const tb = lds + wr * (D_V * 128);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int tl = 32 * u + l32;
      const int pos = (tl & ~15) + vt_pos(tl & 15);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 32 * a + 8 * (r >> 2) + 4 * kg + (r & 3);
          *(_Float16*)(tb + row * 128 + 2 * pos) = f16_sat(acc[a][u][r]);
        }
    }
    _Float16* dst = p.vx + ((int64_t)b * p.H + head) * D_V * p.cap + t0 + 64 * wr;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int id = 64 * i + l, row = id >> 3, c = id & 7;
      const u32x4 v = *(const u32x4*)(tb + row * 128 + 16 * c);
      *(u32x4*)(dst + (int64_t)row * p.cap + 8 * c) = v;
    }
  }
  // the RoPE keys of the tile, once (head 0), to a contiguous array
  if (head == 0) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int i2 = tid + 256 * m, r = i2 >> 3, c = i2 & 7;
      const int t = t0 + r;
      if (t < len) {
        const int64_t row = prefill_row(p.block_table, b, t, p.seq_capacity, p.max_blocks,
                                        p.block_size, p.rows);
        const bf16x8 x = *(const bf16x8*)(p.rope + row * p.rope_stride + 8 * c);
        f16x8 y;
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = f16_sat((float)x[e]);
        *(f16x8*)(p.kpx + ((int64_t)b * p.cap + t) * D_R + 8 * c) = y;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Causal attention over the decompressed keys and values
// ---------------------------------------------------------------------------
struct PrefillParams {
  const bf16* q_nope;   // [B, T, H, 128]
  const bf16* q_pe;     // [B, T, H, 64] (already rotated)
  const _Float16* kx;   // [B, H, cap, 128]
  const _Float16* vx;   // [B, H, cap, 128]
  const _Float16* kpx;  // [B, cap, 64]
  const int32_t* lengths;
  int B, H, T, cap, max_len;
  float c;              // softmax_scale * log2(e)
  int order;            // work order, see pf_work
  bf16* out;            // [B, T, H, 128]
  float* lse;           // [B, T, H] natural log, or nullptr
};

constexpr int PF_Q = 128;                        // queries per workgroup (4 waves x 32)
constexpr int PF_KEYS = 64;                      // keys per LDS tile
constexpr int PF_KN = 0;                         // K rows: 64 x 256 B
constexpr int PF_KP = PF_KEYS * 256;             // RoPE keys: 64 x 128 B
constexpr int PF_V = PF_KP + PF_KEYS * 128;      // V^T rows: 128 x 128 B
constexpr int PF_STAGE = PF_V + PF_KEYS * 256;   // 40 KB

// Swizzles (16-byte chunk XOR per row):
//   K rows (256 B), read 16 bytes per lane from 16 consecutive keys:  c ^ (key & 15)
//   RoPE keys (128 B), same reads:                                    c ^ ((key >> 1) & 7)
//   V^T rows (128 B = 64 keys of one value dim), same reads:          c ^ ((dim >> 1) & 7)
__device__ __forceinline__ int pf_kswz(int k) { return k & 15; }

// (sequence, head) pair and query tile of this workgroup. XCD x takes the
// pairs = x mod 8 (their keys and values are read through that XCD's L2).
// order 1 (the default): the longest query tiles of all the XCD's pairs
// first, then the next longest, so that no long tile starts near the end of
// the launch; order 0: each pair with all its query tiles (longest first)
// in a row.
__device__ __forceinline__ void pf_work(const PrefillParams& p, int nqt, int& pr, int& qt) {
  const int xcd = blockIdx.x & 7, i = blockIdx.x >> 3;
  if (p.order == 0) {
    pr = (i / nqt) * 8 + xcd;
    qt = nqt - 1 - (i % nqt);
  } else {
    const int nh = (p.B * p.H + 7) / 8;
    pr = (i % nh) * 8 + xcd;
    qt = nqt - 1 - i / nh;
  }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mla_prefill_attn_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(1024))) char lds[2 * PF_STAGE];
  const int tid = threadIdx.x, l = tid & 63, h = l >> 5, l32 = l & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nqt = (p.T + PF_Q - 1) / PF_Q;
  int pr, qt;
  pf_work(p, nqt, pr, qt);
  if (pr >= p.B * p.H) return;
  const int b = pr / p.H, head = pr - b * p.H;
  const int raw_len = p.lengths[b];
  debug_flag(raw_len < 0 || raw_len > p.max_len, DBG_LENGTH);
  const int len = min(max(raw_len, 0), p.max_len);
  const int p0 = len - p.T;                    // position of chunk query 0
  const int q0 = qt * PF_Q, qw0 = q0 + 32 * w;
  const int q = qw0 + l32;                     // this lane's query
  const int pos = p0 + q;
  // keys the workgroup reads, and the last key any query of this wave sees
  const int kmax = min(len, max(p0 + q0 + PF_Q, 0));
  const int wkmax = min(len, max(p0 + qw0 + 32, 0));
  const int ntiles = (kmax + PF_KEYS - 1) / PF_KEYS;

  // queries of this lane, in fp16 and pre-multiplied by softmax_scale
  // log2(e), so the scores come out of the products in log2 units (clamped
  // past the chunk: never stored)
  f16x8 qop[12];
  {
    const int qc = min(q, p.T - 1);
    const int64_t qi = ((int64_t)b * p.T + qc) * p.H + head;
    bf16x8 x[12];
#pragma unroll
    for (int s = 0; s < 8; ++s) x[s] = *(const bf16x8*)(p.q_nope + qi * D_N + 16 * s + 8 * h);
#pragma unroll
    for (int s = 0; s < 4; ++s) x[8 + s] = *(const bf16x8*)(p.q_pe + qi * D_R + 16 * s + 8 * h);
#pragma unroll
    for (int s = 0; s < 12; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) qop[s][e] = f16_sat((float)x[s][e] * p.c);
  }

  // per-lane offsets of this wave's direct-to-LDS pieces of a tile (relative
  // to the tile's first key): 4 K pieces (4 keys x 256 B), 2 RoPE-key pieces
  // (8 keys x 128 B), 4 V^T pieces (8 value dims x 64 keys x 2 B)
  int vo_k[4], vo_p[2], vo_v[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int key = 4 * (4 * w + m) + (l >> 4);
    vo_k[m] = key * 256 + 16 * ((l & 15) ^ pf_kswz(key));
    const int dim = 8 * (4 * w + m) + (l >> 3);
    vo_v[m] = dim * (p.cap * 2) + 16 * ((l & 7) ^ rope_swz(dim));
  }
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int key = 8 * (2 * w + m) + (l >> 3);
    vo_p[m] = key * 128 + 16 * ((l & 7) ^ rope_swz(key));
  }
  const _Float16* kbase = p.kx + ((int64_t)b * p.H + head) * p.cap * D_N;
  const _Float16* vbase = p.vx + ((int64_t)b * p.H + head) * D_V * p.cap;
  const _Float16* pbase = p.kpx + (int64_t)b * p.cap * D_R;
  auto issue = [&](int j) {
    char* st = lds + (j & 1) * PF_STAGE;
    const int key0 = j * PF_KEYS;
    const int nv = __builtin_amdgcn_readfirstlane(max(min(len - key0, PF_KEYS), 0));
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + (int64_t)key0 * D_N, (int64_t)nv * 256);
    // (V^T: the 64-key segments of 128 rows; keys past the end are finite
    // values the mask weights 0)
    const __amdgpu_buffer_rsrc_t rv =
        make_rsrc(vbase + key0, (int64_t)(D_V - 1) * p.cap * 2 + PF_KEYS * 2);
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(pbase + (int64_t)key0 * D_R, (int64_t)nv * 128);
    const uint32_t mk = __builtin_amdgcn_readfirstlane(lds_u32(st + PF_KN) + 4 * w * 1024);
    const uint32_t mp = __builtin_amdgcn_readfirstlane(lds_u32(st + PF_KP) + 2 * w * 1024);
    const uint32_t mv = __builtin_amdgcn_readfirstlane(lds_u32(st + PF_V) + 4 * w * 1024);
    dma16_m0<0>(rk, mk, vo_k[0]);
    dma16_m0<1024>(rk, mk, vo_k[1]);
    dma16_m0<2048>(rk, mk, vo_k[2]);
    dma16_m0<3072>(rk, mk, vo_k[3]);
    dma16_m0<0>(rp, mp, vo_p[0]);
    dma16_m0<1024>(rp, mp, vo_p[1]);
    dma16_m0<0>(rv, mv, vo_v[0]);
    dma16_m0<1024>(rv, mv, vo_v[1]);
    dma16_m0<2048>(rv, mv, vo_v[2]);
    dma16_m0<3072>(rv, mv, vo_v[3]);
  };

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  if (ntiles > 0) issue(0);
  wait_vm_lgkm0<0>();
  __builtin_amdgcn_s_barrier();
  compiler_fence();

  // LDS read offsets of this lane (relative to a stage): S^T A operand (key
  // row l32 of a 32-key block, chunk 2 s + h), PV A operand (V^T row
  // 32 dt + l32, chunk 2 ks + h: the lane half's 8 keys of k-step ks)
  const int vsw = rope_swz(l32);
  for (int j = 0; j < ntiles; ++j) {
    const char* st = lds + (j & 1) * PF_STAGE;
    if (j + 1 < ntiles) issue(j + 1);
    const int kt0 = j * PF_KEYS;
    f32x16 sacc[2];
    bool act[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      act[kb] = kt0 + 32 * kb < wkmax;   // wave-uniform
      if (act[kb]) {
        const int key = 32 * kb + l32;
#pragma unroll
        for (int s = 0; s < 12; ++s) {
          f16x8 a;
          if (s < 8) {
            const int c = 2 * s + h;
            a = *(const f16x8*)(st + PF_KN + key * 256 + 16 * (c ^ pf_kswz(key)));
          } else {
            const int c = 2 * (s - 8) + h;
            a = *(const f16x8*)(st + PF_KP + key * 128 + 16 * (c ^ rope_swz(key)));
          }
          sacc[kb] = (s == 0) ? __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qop[s], f32x16{}, 0, 0, 0)
                              : __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qop[s], sacc[kb], 0, 0, 0);
        }
      }
    }
    if (act[0]) {
      // scores (log2 units); register r of block kb is key
      // kt0 + 32 kb + 8 (r / 4) + 4 h + r % 4. Only tiles that reach past the
      // wave's first query position are masked (wave-uniform test).
      if (!act[1]) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[1][r] = -INFINITY;
      }
      if (kt0 + PF_KEYS - 1 > p0 + qw0) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kt0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
            sacc[kb][r] = (key > pos) ? -INFINITY : sacc[kb][r];
          }
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, sacc[kb][r]);
      tmax = pair_max(tmax);
      // The exponent reference m_run moves only when a tile's maximum exceeds
      // it by more than LAZY (log2 units): the weights stay below 2^LAZY
      // (exact enough in fp16, far from its range), and the accumulator is
      // rescaled only in the rare tiles where some lane's reference moved.
      constexpr float LAZY = 8.0f;
      const bool up = tmax > m_run + LAZY;
      const float m_new = up ? tmax : m_run;
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = up ? fast_exp2(m_run - m_use) : 1.0f;
      m_run = m_new;
      f16x8 pb[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) pb[kb][r >> 3][r & 7] = (_Float16)fast_exp2(sacc[kb][r] - m_use);
      // the denominator sums the fp16 weights the PV product uses, two per
      // v_dot2_f32_f16
      typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
      const f16x2 one2 = {(_Float16)1.0f, (_Float16)1.0f};
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int e = 0; e < 8; e += 2)
            psum = __builtin_amdgcn_fdot2(f16x2{pb[kb][hf][e], pb[kb][hf][e + 1]}, one2, psum, false);
      l_run = l_run * alpha + psum;
      if (__any(up)) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (act[kb]) {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const int ks = 2 * kb + hf;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
              const f16x8 v = *(const f16x8*)(st + PF_V + (32 * dt + l32) * 128 +
                                              16 * ((2 * ks + h) ^ vsw));
              o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(v, pb[kb][hf], o[dt], 0, 0, 0);
            }
          }
        }
      }
    }
    // the next tile has landed everywhere, and every wave is done with this one
    wait_vm_lgkm0<0>();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
  }

  // both half-waves hold the same query: total denominator, then the output
  const unsigned ul = __builtin_bit_cast(unsigned, l_run);
  const auto sw = __builtin_amdgcn_permlane32_swap(ul, ul, false, false);
  const float ltot = __builtin_bit_cast(float, (unsigned)sw[0]) + __builtin_bit_cast(float, (unsigned)sw[1]);
  if (q < p.T) {
    const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
    bf16* orow = p.out + (((int64_t)b * p.T + q) * p.H + head) * D_V;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const bf16x4 v = {(bf16)(o[dt][4 * g] * inv), (bf16)(o[dt][4 * g + 1] * inv),
                          (bf16)(o[dt][4 * g + 2] * inv), (bf16)(o[dt][4 * g + 3] * inv)};
        *(bf16x4*)(orow + 32 * dt + 8 * g + 4 * h) = v;
      }
    if (p.lse && h == 0)
      p.lse[((int64_t)b * p.T + q) * p.H + head] =
          ltot > 0.f ? (m_run + __builtin_log2f(ltot)) * LN2 : -INFINITY;
  }
}

}  // namespace mla
