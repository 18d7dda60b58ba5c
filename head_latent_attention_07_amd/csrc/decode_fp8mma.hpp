// Split-KV flash decode over an fp8 (e4m3) cache on gfx950's fp8 matrix
// cores (v_mfma_scale_f32_32x32x64_f8f6f4), without widening the cache.
//
// The cache rows are e4m3 codes with one bf16 scale per row ("Como a MLA da
// DeepSeek cortou 93% da memoria", section "De onde vem o 93%": serving with
// an FP8 / ~6-bit cache; "DeepSeek AI efficiency, architecture, benchmarks",
// section "Training Pipeline and FP8 Execution": FP8 with fine-grained
// scaling). The codes are exact e4m3 values, so they go to the matrix cores
// as stored; the other operand of each product is split into two e4m3
// parts, hi and lo, each with a power-of-two scale per 32-wide contraction
// block (the scale operands of the instruction):
//
//   S^T[t, h] = s_t * sum_d code_t[d] (q_hi[h, d] 2^-e + q_lo[h, d] 2^-(e+4))
//   O^T[d, h] += sum_t code_t[d] (P'_hi[t, h] 2^-f + P'_lo[t, h] 2^-(f+4)),
//                P'[t, h] = s_t 2^(S^T[t, h] - m_ref[h])
//
// hi carries the leading 4 significant bits and lo the next 4 (of the
// remainder, 16 times larger), so each product sees about 8 significant
// bits of the query and of the weights, as the bf16 kernel does. Two fp8
// MFMAs of 64 cycles do the work of one 32x32x64 bf16 product (two bf16
// MFMAs of 32 cycles): the matrix-core time equals the bf16 kernel's, and the
// cache never leaves its 1-byte form (no widening pass, half the LDS bytes
// per token).
//
// Work decomposition (as the bf16 kernel): workgroup = (sequence, split),
// four waves of 32 heads each; O^T (32 heads x 512 dims, fp32) fills the 256
// AGPRs; the token range streams through LDS in tiles of 64 rows (64 x 576
// bytes), two buffers, with direct-to-LDS loads of the next tile issued at
// the start of each step. The query's hi parts stay in VGPRs (72), its lo
// parts in LDS (18 KB per wave, read one k-step ahead).
//
// Layouts. For the 32x32x64 f8 instruction, lane (r, g) = (l % 32, l / 32)
// holds row r of A (column r of B) and k = 16g..16g+15 (bytes 0..15),
// 32+16g..32+16g+15 (bytes 16..31) of the 64-wide step; block kb = k / 32
// takes its scale from lane (r, kb).
//   * S^T = K Q^T: A = token rows of the tile. Row i of a 32-token half is
//     token f8_tok(i), so that accumulator register r of lane (j, g) is
//     token 16 g + r: the lane's 16 scores of each half are exactly the 16
//     P^T bytes it supplies to the PV product (bytes 0..15 from the first
//     half, 16..31 from the second), with no cross-lane traffic.
//   * O^T += V^T P^T: A = V^T from ds_read_b64_tr_b8 (each lane gets 8
//     consecutive tokens of one latent column), tokens in natural order.
//   * LDS swizzle of a 512-byte latent row (16-byte chunks): c ^ f8_lat_swz(t)
//     makes both the QK reads (16 rows, one chunk) and the transposed PV
//     reads (8 consecutive rows, 32 bytes) conflict-free; the 64-byte RoPE
//     rows use c ^ f8_rope_swz(t).
#pragma once

#include "decode_mfma.hpp"

namespace mla {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int F8_TILE = 64;                               // tokens per tile
constexpr int F8_LAT_BYTES = F8_TILE * D_C;               // 32 KB of latent codes
constexpr int F8_TILE_BYTES = F8_LAT_BYTES + F8_TILE * D_R;   // + 4 KB of RoPE codes
constexpr int F8_KS = D_QK / 64;                          // 9 contraction steps of 64
constexpr int F8_QLO_WAVE = F8_KS * 2048;                 // lo query parts of a wave (18 KB)
constexpr int F8_MAX_TILES = 64;                          // 4096 tokens per split (one tile row per lane)
constexpr uint32_t F8_UNIT_SCALE = 0x7F7F7F7Fu;           // E8M0 127 = 2^0 in every byte

__device__ __forceinline__ int f8_lat_swz(int t) { return ((t & 7) << 1) | ((t >> 4) & 1); }
__device__ __forceinline__ int f8_rope_swz(int t) { return ((t >> 2) & 1) | ((t >> 3) & 2); }
__device__ __forceinline__ int f8_tok(int i) { return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3); }

__device__ __forceinline__ f32x16 mfma_f8(const i32x8& a, const i32x8& b, const f32x16& c,
                                          int sb, int opsel_b) {
  switch (opsel_b) {   // the byte of the scale register (compile-time after unrolling)
    case 0: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, (int)F8_UNIT_SCALE, 0, sb);
    case 1: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, (int)F8_UNIT_SCALE, 1, sb);
    case 2: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, (int)F8_UNIT_SCALE, 2, sb);
    default: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, (int)F8_UNIT_SCALE, 3, sb);
  }
}

// The S^T chain in VGPRs (inline assembly fixes the register class: the 256
// AGPRs hold O^T, and the compiler would otherwise move an O^T tile through
// VGPRs every step). OPSEL picks the byte of the B scale register; the A
// scale is 2^0. The compiler does not see these as MFMAs: f8_settle inserts
// the wait states a vector read of the result needs (more than the 17 of
// this 16-pass instruction), bound to the accumulator. Back-to-back MFMAs
// accumulating into the same registers need none.
#define F8_MFMA_ASM(OPS)                                                             \
  "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4" OPS
template <int OPSEL>
__device__ __forceinline__ void f8_mfma_vgpr(f32x16& acc, const i32x8& a, const i32x8& b,
                                             uint32_t sa, uint32_t sb) {
  if constexpr (OPSEL == 0)
    asm volatile(F8_MFMA_ASM("") : "+v"(acc) : "v"(a), "v"(b), "v"(sa), "v"(sb));
  else if constexpr (OPSEL == 1)
    asm volatile(F8_MFMA_ASM(" op_sel:[0,1,0]") : "+v"(acc) : "v"(a), "v"(b), "v"(sa), "v"(sb));
  else if constexpr (OPSEL == 2)
    asm volatile(F8_MFMA_ASM(" op_sel_hi:[0,1,0]") : "+v"(acc) : "v"(a), "v"(b), "v"(sa), "v"(sb));
  else
    asm volatile(F8_MFMA_ASM(" op_sel:[0,1,0] op_sel_hi:[0,1,0]")
                 : "+v"(acc) : "v"(a), "v"(b), "v"(sa), "v"(sb));
}
#undef F8_MFMA_ASM
__device__ __forceinline__ void f8_settle(f32x16& acc) {
  asm volatile("s_nop 15\n\ts_nop 7" : "+v"(acc));
}

// Power-of-two exponent e with amax * 2^e < 256 (0 for amax == 0 or
// non-finite): e4m3 holds up to 448, so hi parts never saturate.
__device__ __forceinline__ int f8_exp(float amax) {
  if (!(amax > 0.f) || !(amax < INFINITY)) return 0;
  int x;
  (void)frexpf(amax, &x);   // amax < 2^x
  return min(max(8 - x, -100), 100);
}

// e4m3 hi and lo parts of v (already multiplied by 2^e): hi = rne(v),
// lo = rne(16 (v - hi)), two values at a time into half HIGH of the words.
template <bool HIGH>
__device__ __forceinline__ void f8_split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  const uint32_t h = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, hi, HIGH);
  // the hi codes back to fp32, to form the remainders
  const float ha = __builtin_amdgcn_cvt_f32_fp8(h, HIGH ? 2 : 0);
  const float hb = __builtin_amdgcn_cvt_f32_fp8(h, HIGH ? 3 : 1);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(16.f * (a - ha), 16.f * (b - hb), lo, HIGH);
  hi = h;
}

// Physical rows of the first token of each 64-token tile of the split, tile i
// in lane i (at most 32 tiles).
__device__ __forceinline__ int f8_tile_rows_lanes(const DecodeParams& p, int b, int t0, int t1,
                                                  const int* tab, int first_blk, int l) {
  const int t = t0 + F8_TILE * min(l, max((t1 - t0 + F8_TILE - 1) / F8_TILE - 1, 0));
  if (p.block_table) return tab[t / p.block_size - first_blk] * p.block_size + (t % p.block_size);
  return (int)((int64_t)b * p.seq_capacity + t);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_decode_fp8mma_kernel(DecodeParams p) {
  constexpr int NW = 4, NT = 256;
  __shared__ __attribute__((aligned(1024))) char bufs[2 * F8_TILE_BYTES];     // 72 KB
  __shared__ __attribute__((aligned(1024))) char qlo_all[NW * F8_QLO_WAVE];   // 72 KB
  __shared__ __attribute__((aligned(16))) float scl_all[F8_MAX_TILES * F8_TILE];   // 16 KB
  // (160 KB in all: the split's block table borrows tile buffer 1 in the
  // prologue, before that buffer's first load; the overflow flags borrow the
  // end of tile buffer 0 after the last tile, past write_partial's staging)
  int* const blk_tab = (int*)(bufs + F8_TILE_BYTES);
  int* const flags = (int*)(bufs + F8_TILE_BYTES - 64);
  static_assert(2 * PART_SCR_BYTES <= F8_TILE_BYTES - 64, "flags past the partial staging");
  static_assert(MAX_SPLIT_BLOCKS * 4 <= F8_TILE_BYTES, "block table fits in a tile buffer");

  const int tid = threadIdx.x, l = tid & 63, g = l >> 5, r32 = l & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  WorkItem wi;
  if (!work_item<NW>(p, w, l, wi)) return;
  if (wi.t0 >= wi.t1) {
    write_empty(wi, g);
    return;
  }
  const int ntiles = (wi.t1 - wi.t0 + F8_TILE - 1) / F8_TILE;
  auto nvalid = [&](int k) { return min(max(wi.t1 - (wi.t0 + k * F8_TILE), 0), F8_TILE); };

  // This wave's 9 direct-to-LDS pieces of a tile: 8 latent pieces (rows
  // 16w + 2i and +1: lane l fills LDS chunk l % 32 of row l / 32, which
  // holds the chunk the swizzle places there) and one RoPE piece (rows
  // 16w .. 16w+15). The lane offsets are recomputed at each issue (a few
  // ALU operations) from an opaque copy of the lane index: kept live across
  // the loop they would be spilled, and a reload would wait for the tile
  // loads in flight.
  auto issue = [&](char* buf, int row0, int nv) {
    const TileRsrc rs = tile_rsrc(p, row0, nv, 1);
    const uint32_t ml = __builtin_amdgcn_readfirstlane(lds_u32(buf) + 16 * w * 512);
    const uint32_t mr = __builtin_amdgcn_readfirstlane(lds_u32(buf) + F8_LAT_BYTES + 16 * w * 64);
    int lv = l;
    asm volatile("" : "+v"(lv));
    const int lsb = (int)p.latent_stride, rsb = (int)p.rope_stride;
    auto lat_off = [&](int i) {
      const int t = 16 * w + 2 * i + (lv >> 5);
      return t * lsb + 16 * ((lv & 31) ^ f8_lat_swz(t));
    };
    dma16_m0<0>(rs.lat, ml, lat_off(0));
    dma16_m0<1024>(rs.lat, ml, lat_off(1));
    dma16_m0<2048>(rs.lat, ml, lat_off(2));
    dma16_m0<3072>(rs.lat, ml, lat_off(3));
    dma16_m0<4096>(rs.lat, ml, lat_off(4));
    dma16_m0<5120>(rs.lat, ml, lat_off(5));
    dma16_m0<6144>(rs.lat, ml, lat_off(6));
    dma16_m0<7168>(rs.lat, ml, lat_off(7));
    const int tr = 16 * w + (lv >> 2);
    dma16_m0<0>(rs.rope, mr, tr * rsb + 16 * ((lv & 3) ^ f8_rope_swz(tr)));
  };

  // Prologue: tile 0's loads, the split's block table, the queries (hi
  // parts into registers, lo parts into LDS, block scales), one wait.
  issue(bufs, (int)tile_base_row_direct(p, wi.b, wi.t0), nvalid(0));
  load_block_table<NT>(p, wi.b, wi.t0, wi.t1, blk_tab, tid);
  i32x8 qhi[F8_KS];
  uint32_t sc_hi[3] = {F8_UNIT_SCALE, F8_UNIT_SCALE, F8_UNIT_SCALE};
  uint32_t sc_lo[3] = {F8_UNIT_SCALE, F8_UNIT_SCALE, F8_UNIT_SCALE};
  char* const qlo = qlo_all + w * F8_QLO_WAVE;
  {
    const int hd = wi.head;   // this lane's head
#pragma unroll
    for (int ks = 0; ks < F8_KS; ++ks) {
      // dims 64 ks + 16 g .. +15 (bytes 0..15) and 64 ks + 32 + 16 g .. +15
      float v[32];
#pragma unroll
      for (int part = 0; part < 2; ++part)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int n = 64 * ks + 32 * part + 16 * g + 8 * hf;
          const bf16x8 x = *(const bf16x8*)(p.q + qop_index(wi.b, hd, n, p.H));
#pragma unroll
          for (int e = 0; e < 8; ++e) v[16 * part + 8 * hf + e] = (float)x[e];
        }
      // block kb of the step is dims 32 kb .. 32 kb + 31: this lane's bytes
      // 16 kb .. 16 kb + 15 and its partner's (lane l ^ 32)
      float am[2] = {0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 32; ++e) am[e >> 4] = fmaxf(am[e >> 4], fabsf(v[e]));
      const int e0 = f8_exp(pair_max(am[0])), e1 = f8_exp(pair_max(am[1]));
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        hi[k] = 0;
        lo[k] = 0;
        const float m = ldexpf(1.0f, k < 4 ? e0 : e1);
        f8_split2<false>(v[4 * k] * m, v[4 * k + 1] * m, hi[k], lo[k]);
        f8_split2<true>(v[4 * k + 2] * m, v[4 * k + 3] * m, hi[k], lo[k]);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) qhi[ks][k] = (int)hi[k];
      *(u32x4*)(qlo + 2048 * ks + 16 * l) = u32x4{lo[0], lo[1], lo[2], lo[3]};
      *(u32x4*)(qlo + 2048 * ks + 1024 + 16 * l) = u32x4{lo[4], lo[5], lo[6], lo[7]};
      // this lane supplies the scale of block g of its column
      const int e = g ? e1 : e0;
      const uint32_t shi = (uint32_t)(127 - e), slo = (uint32_t)(127 - e - 4);
      const int word = ks >> 2, sh = 8 * (ks & 3);
      sc_hi[word] = (sc_hi[word] & ~(0xFFu << sh)) | (shi << sh);
      sc_lo[word] = (sc_lo[word] & ~(0xFFu << sh)) | (slo << sh);
    }
  }
  WaveState st;
  reset_state(st, -INFINITY);
  wait_vm_lgkm0<0>();
  __builtin_amdgcn_s_barrier();
  compiler_fence();
  const int trow = f8_tile_rows_lanes(p, wi.b, wi.t0, wi.t1, blk_tab, first_blk_of(p, wi.t0), l);
  for (int i = tid; i < ntiles * F8_TILE; i += NT) {
    const int k = i >> 6, rr = i & 63;
    const int last = wi.t1 - 1 - (wi.t0 + k * F8_TILE);
    int64_t row = (int64_t)__shfl(trow, k, 64) + min(rr, last);
    row = (row >= 0 && row < p.rows) ? row : 0;
    scl_all[i] = (float)p.scales[row];
  }
  wait_vm_lgkm0<0>();
  __builtin_amdgcn_s_barrier();   // every row scale is in LDS before any is read
  compiler_fence();

  // LDS offsets of this lane's operand reads (relative to a tile buffer)
  int qa[2];       // S^T A operand, half u: token row 32 u + f8_tok(r32)
  int qr[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int t = 32 * u + f8_tok(r32);
    qa[u] = t * D_C;
    qr[u] = F8_LAT_BYTES + t * D_R;
  }
  auto k_operand = [&](const char* buf, int u, int ks) {
    const int t = 32 * u + f8_tok(r32);
    i32x8 a;
    u32x4 x0, x1;
    if (ks < 8) {
      const int sw = f8_lat_swz(t);
      x0 = *(const u32x4*)(buf + qa[u] + 16 * ((4 * ks + g) ^ sw));
      x1 = *(const u32x4*)(buf + qa[u] + 16 * ((4 * ks + 2 + g) ^ sw));
    } else {
      const int sw = f8_rope_swz(t);
      x0 = *(const u32x4*)(buf + qr[u] + 16 * (g ^ sw));
      x1 = *(const u32x4*)(buf + qr[u] + 16 * ((2 + g) ^ sw));
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      a[k] = (int)x0[k];
      a[4 + k] = (int)x1[k];
    }
    return a;
  };
  auto qlo_operand = [&](int ks) {
    const u32x4 x0 = *(const u32x4*)(qlo + 2048 * ks + 16 * l);
    const u32x4 x1 = *(const u32x4*)(qlo + 2048 * ks + 1024 + 16 * l);
    i32x8 b;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      b[k] = (int)x0[k];
      b[4 + k] = (int)x1[k];
    }
    return b;
  };
  // V^T A operand of latent column tile dt: tokens 16 g .. 16 g + 15 (bytes
  // 0..15) and 32 + 16 g .. (bytes 16..31), 8 tokens per transposing read;
  // lanes 2m, 2m+1 of a 16-lane group supply row m, 8 bytes each
  const int jj = l & 15, g16 = l >> 4;
  auto v_operand = [&](const char* buf, int dt) {
    i32x8 a;
#pragma unroll
    for (int rd = 0; rd < 4; ++rd) {
      const int t = 16 * g + 8 * (rd & 1) + 32 * (rd >> 1) + (jj >> 1);
      const int c = (2 * dt + (g16 & 1)) ^ f8_lat_swz(t);
      typedef int i32x2 __attribute__((ext_vector_type(2)));
      const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (__attribute__((address_space(3))) i32x2*)(buf + t * D_C + 16 * c + 8 * (jj & 1)));
      a[2 * rd] = x[0];
      a[2 * rd + 1] = x[1];
    }
    return a;
  };

  // scores of one tile (both halves), scaled by the rows' scales, masked
  // past the split's end
  const uint32_t unit = F8_UNIT_SCALE;
  // scores of half u of tile k: the rows' scales applied, masked past the
  // split's end (register r is token 32 u + 16 g + r)
  auto scale_mask = [&](int k, int u, f32x16& s) {
    const float* sc = scl_all + F8_TILE * k;
    const int tk0 = wi.t0 + F8_TILE * k;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4 s4 = *(const f32x4*)(sc + 32 * u + 16 * g + 4 * q4);
#pragma unroll
      for (int e = 0; e < 4; ++e) s[4 * q4 + e] *= s4[e];
    }
    if (tk0 + F8_TILE > wi.t1) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (tk0 + 32 * u + 16 * g + r >= wi.t1) s[r] = -INFINITY;
    }
  };
  auto half_scores = [&](const char* buf, int k, int u, f32x16& s) {
    s = f32x16{};
    static_for<F8_KS>([&](auto kc) {
      constexpr int ks = decltype(kc)::value;
      const i32x8 a = k_operand(buf, u, ks);
      const i32x8 bl = qlo_operand(ks);
      f8_mfma_vgpr<ks & 3>(s, a, qhi[ks], unit, sc_hi[ks >> 2]);
      f8_mfma_vgpr<ks & 3>(s, a, bl, unit, sc_lo[ks >> 2]);
    });
    f8_settle(s);
    scale_mask(k, u, s);
  };
  auto tile_scores = [&](const char* buf, int k, f32x16 (&s)[2]) {
    half_scores(buf, k, 0, s[0]);
    half_scores(buf, k, 1, s[1]);
  };

  for (int attempt = 0; attempt < 2; ++attempt) {
    if (attempt > 0) {
      issue(bufs, __builtin_amdgcn_readlane(trow, 0), nvalid(0));
      wait_vm_lgkm0<0>();
      __builtin_amdgcn_s_barrier();
      compiler_fence();
    }
    for (int j = 0; j < ntiles; ++j) {
      const char* buf = bufs + (j & 1) * F8_TILE_BYTES;
      if (j + 1 < ntiles)
        issue(bufs + ((j + 1) & 1) * F8_TILE_BYTES,
              __builtin_amdgcn_readlane(trow, min(j + 1, ntiles - 1)), nvalid(j + 1));
      // S^T of the tile's first half; then the second half's chain, under
      // whose MFMAs the first half's weights are formed and split (slices
      // pinned between the MFMAs); then the second half's weights.
      const float* sc = scl_all + F8_TILE * j;
      f32x16 s0, s1;
      half_scores(buf, j, 0, s0);
      if (st.m_ref == -INFINITY) {   // the split's first half-tile fixes the reference
        float m = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, s0[r]);
        st.m_ref = pair_max(m);
      }
      i32x8 phi, plo;
      float pw0[16];
      float am0 = 0.f;
      int f0 = 0;
      s1 = f32x16{};
      __builtin_amdgcn_sched_barrier(0);
      static_for<F8_KS>([&](auto kc) {
        constexpr int ks = decltype(kc)::value;
        const i32x8 a = k_operand(buf, 1, ks);
        const i32x8 bl = qlo_operand(ks);
        f8_mfma_vgpr<ks & 3>(s1, a, qhi[ks], unit, sc_hi[ks >> 2]);
        f8_mfma_vgpr<ks & 3>(s1, a, bl, unit, sc_lo[ks >> 2]);
        if constexpr (ks < 4) {   // weights of tokens 16 g + 4 ks .. +3
          const f32x4 s4 = *(const f32x4*)(sc + 16 * g + 4 * ks);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float pr = fast_exp2(s0[4 * ks + e] - st.m_ref);
            st.lsum += pr;
            pw0[4 * ks + e] = pr * s4[e];
            am0 = fmaxf(am0, pw0[4 * ks + e]);
          }
        } else if constexpr (ks == 4) {
          f0 = f8_exp(pair_max(am0));
        } else {                  // hi / lo of word ks - 5
          constexpr int k = ks - 5;
          const float m = ldexpf(1.0f, f0);
          uint32_t hi = 0, lo = 0;
          f8_split2<false>(pw0[4 * k] * m, pw0[4 * k + 1] * m, hi, lo);
          f8_split2<true>(pw0[4 * k + 2] * m, pw0[4 * k + 3] * m, hi, lo);
          phi[k] = (int)hi;
          plo[k] = (int)lo;
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      f8_settle(s1);
      scale_mask(j, 1, s1);
      float pw1[16];
      float am1 = 0.f;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 s4 = *(const f32x4*)(sc + 32 + 16 * g + 4 * q4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pr = fast_exp2(s1[4 * q4 + e] - st.m_ref);
          st.lsum += pr;
          pw1[4 * q4 + e] = pr * s4[e];
          am1 = fmaxf(am1, pw1[4 * q4 + e]);
        }
      }
      const int f1 = f8_exp(pair_max(am1));
      {
        const float m = ldexpf(1.0f, f1);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          uint32_t hi = 0, lo = 0;
          f8_split2<false>(pw1[4 * k] * m, pw1[4 * k + 1] * m, hi, lo);
          f8_split2<true>(pw1[4 * k + 2] * m, pw1[4 * k + 3] * m, hi, lo);
          phi[4 + k] = (int)hi;
          plo[4 + k] = (int)lo;
        }
      }
      const int fe = g ? f1 : f0;
      const int pshi = 127 - fe, pslo = 127 - fe - 4;
#pragma unroll
      for (int dt = 0; dt < D_C / 32; ++dt) {
        const i32x8 a = v_operand(buf, dt);
        st.o[dt] = mfma_f8(a, phi, st.o[dt], pshi, 0);
        st.o[dt] = mfma_f8(a, plo, st.o[dt], pslo, 0);
      }
      // the next tile has landed everywhere; every wave is done with this one
      wait_vm_lgkm0<0>();
      __builtin_amdgcn_s_barrier();
      compiler_fence();
    }
    const bool ovf = split_overflowed(st);
    if (l == 0) flags[w] = ovf ? 1 : 0;
    wait_vm_lgkm0<0>();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    int any_ovf = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) any_ovf |= flags[i];
    any_ovf = __builtin_amdgcn_readfirstlane(any_ovf);
    if (any_ovf == 0) break;
    // Rare path (see the bf16 kernel): each head's true maximum over the
    // split (scores only), then the split again against it.
    float mtrue = -INFINITY;
    for (int k = 0; k < ntiles; ++k) {
      __builtin_amdgcn_s_barrier();   // buffer 0 and the flags are no longer read
      compiler_fence();
      issue(bufs, __builtin_amdgcn_readlane(trow, k), nvalid(k));
      wait_vm_lgkm0<0>();
      __builtin_amdgcn_s_barrier();
      compiler_fence();
      f32x16 s[2];
      tile_scores(bufs, k, s);
      float m = -INFINITY;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, s[u][r]);
      mtrue = fmaxf(mtrue, pair_max(m));
    }
    reset_state(st, mtrue);
    wait_vm_lgkm0<0>();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
  }
  write_partial(wi, st, g, l, (w < 2 ? bufs : bufs + F8_TILE_BYTES) + (w & 1) * PART_SCR_BYTES);
}

}  // namespace mla
