// Split-KV flash-decode for MLA on gfx950 (bf16 MFMA, bf16 or fp8 cache).
//
// Absorbed MLA decode ("How DeepSeek Rewrote the Transformer [MLA]", section
// "MLA: compress the pair, not the heads"): every head scores its absorbed
// query q = [q_nope W_UK[h] | q_pe] against the same cached rows
// [c_t | k^R_t] and mixes the same latent rows c_t, so the head dimension is
// the N dimension of two dense contractions that share one operand stream:
//
//   S^T[t, h]  = sum_d  K[t, d] Q^T[d, h]        (d over 576)
//   O^T[d, h] += sum_t  C^T[d, t] P^T[t, h]      (d over 512)
//
// Work decomposition
//   * workgroup = (sequence b, token split s, head group g), NW waves; wave
//     w owns 32 heads: its absorbed queries are the S^T B operand (latent
//     k-steps in registers, RoPE k-steps in LDS) and its O^T accumulator
//     (32 heads x 512 dims, fp32) fills the 256 AGPRs as 16 32x32 tiles.
//   * the workgroup streams its token range through LDS in tiles of 32 rows
//     (32 x 1152 bytes, row-major, 16-byte chunks XOR-swizzled per row so
//     both read patterns are free of bank conflicts), loaded with
//     direct-to-LDS buffer loads issued between the MFMAs (two tiles ahead).
//   * S^T reads the tile with ds_read_b128 (token-major A operand); PV reads
//     the same bytes with ds_read_b64_tr_b16, the gfx950 transposing LDS
//     read, which hands each lane 4 consecutive tokens of one latent column.
//     The token order inside a 16-token k-step is permuted to match the
//     32x32 accumulator layout of S^T, so P^T goes from the S^T accumulator
//     to the PV B operand without any cross-lane traffic.
//   * softmax in base 2 (the absorbed query is pre-scaled by softmax_scale *
//     log2 e) against a fixed exponent reference, the split's first-tile
//     max: the accumulators are never rescaled; a split whose weights reach
//     2^64 is recomputed against its true max.
//   * bf16 cache: a cross-tile software pipeline (pipe_step) interleaves the
//     PV of tile j-1 with the S^T of tile j in one stream of MFMAs.
//   * fp8 cache: the same pipeline over tiles widened (exactly) to the bf16
//     tile layout: each lane widens the raw e4m3 pieces its own loads
//     staged, in the step's early MFMA slots; the per-row scale multiplies
//     the row's scores and, after the softmax sum, its weights, so both
//     MFMAs see exact e4m3 values.
//   * each split writes its normalised partial O (fp16 relative to the row
//     max, with the fp32 factor) and its log2 sum-exp; a separate kernel
//     merges the splits and applies W_UV.
#pragma once

#include <type_traits>
#include <utility>

#include "common.hpp"

namespace mla {

// One work item of a length-aware split plan: sequence b's token range
// [t0, t1), written to its partial slot s (t0 >= t1: an empty sequence).
struct __attribute__((aligned(16))) SplitItem {
  int b, s, t0, t1;
};

struct DecodeParams {
  const bf16* q;               // [B, H, 576] absorbed query, pre-scaled
  const void* latent;          // cache latent array
  int64_t latent_stride;       // elements
  const void* rope;            // cache RoPE-key array
  int64_t rope_stride;         // elements
  const bf16* scales;          // fp8 cache: bf16 scale per row
  int64_t rows;                // rows in the cache arrays
  int64_t seq_capacity;        // contiguous cache: rows per sequence
  const int32_t* block_table;  // paged cache: [B, max_blocks] (nullptr: contiguous)
  int max_blocks;
  int block_size;
  const int32_t* lengths;      // [B]
  int max_len;
  int B, H, S, tokens_per_split, G;   // S: partial slots per sequence
  const SplitItem* items;      // length-aware plan: work item q of the launch (b < 0: none),
  int nitems;                  // or nullptr: item q is split q % S of sequence q / S
  _Float16* part_o;            // [B, S, H, 512] normalised partial outputs / part_scale
  float* part_scale;           // [B, S, H] max |normalised output| of each partial row
  float* part_lse;             // [B, S, H] log2 sum-exp of each split
};


constexpr int TILE = 32;                    // tokens per LDS tile
constexpr int LAT_ROW = D_C * 2;            // 1024 B: bf16 latent row in LDS
constexpr int ROPE_ROW = D_R * 2;           // 128 B: bf16 RoPE-key row in LDS
constexpr int ROPE_OFF = TILE * LAT_ROW;    // RoPE rows follow the 32 latent rows
constexpr int TILE_BYTES = ROPE_OFF + TILE * ROPE_ROW;  // 36864

// The absorbed query of a lane's head is the QK^T B operand: all 36 k-steps
// stay in registers (144 VGPRs: 32 latent k-steps in qreg, the 4 RoPE
// k-steps in qpe), so the only LDS reads of the loop are the tile's.
constexpr int QREG = D_C / 16;           // latent k-steps of Q
constexpr int QLDS = D_QK / 16 - QREG;   // RoPE k-steps of Q

// LDS swizzles (gfx950 LDS: 64 banks of 4 bytes, 256 bytes per cycle).
// Latent rows are 1 KB (64 chunks of 16 bytes); chunk c of row r is stored at
// c ^ lat_swz(r), an XOR on the low four bits, so that
//   * a ds_read_b128 of one chunk from 16 consecutive rows (QK^T A operand,
//     16 lanes per cycle) touches 16 distinct 16-byte bank groups, and
//   * a ds_read_b64_tr_b16 of 64 bytes from each of 4 consecutive rows (PV A
//     operand, 32 lanes per cycle) touches 4 distinct 64-byte bank groups.
// RoPE-key rows are 128 bytes (8 chunks), chunk c of row r at c ^ rope_swz(r):
// 16 consecutive rows then cover the 256 bytes of banks exactly once.
__device__ __forceinline__ int lat_swz(int row) { return 4 * (row & 3) + ((row >> 2) & 3); }
__device__ __forceinline__ int rope_swz(int row) { return (row >> 1) & 7; }

// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding, expcnt left at its maximum):
// this wave's LDS traffic is done and at most N of its global loads remain.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

// Per-lane LDS byte offsets of the MFMA operand reads (relative to a tile).
// QK^T A operand, k-step j: latent (j < 32) at qb[j & 7] + 256 (j >> 3),
// RoPE key (j >= 32) at rb[j - 32]. PV A operand (transposing read) for
// 32-dim tile dt and 16-token k-step ks: lower 4 tokens at
// tb[0][dt & 3] + 256 (dt >> 2) + 16 KB ks, upper 4 tokens (8 rows further)
// at tb[1][...] (the swizzle of row+8 differs from that of row).
struct LaneAddr {
  int qb[8];
  int rb[4];
  int tb[2][4];
};

__device__ __forceinline__ LaneAddr lane_addr(int l) {
  LaneAddr a;
  const int h = l >> 5, l32 = l & 31, jj = l & 15, g16 = l >> 4;
  const int sw = lat_swz(l32), rsw = rope_swz(l32);
#pragma unroll
  for (int k = 0; k < 8; ++k) a.qb[k] = l32 * LAT_ROW + 16 * ((2 * k + h) ^ sw);
#pragma unroll
  for (int k = 0; k < 4; ++k) a.rb[k] = ROPE_OFF + l32 * ROPE_ROW + 16 * ((2 * k + h) ^ rsw);
  const int row1 = 4 * h + (jj >> 2);
  const int cbase = 2 * (g16 & 1) + ((jj & 3) >> 1);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = row1 + 8 * u;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      a.tb[u][e] = row * LAT_ROW + 16 * ((4 * e + cbase) ^ lat_swz(row)) + 8 * (jj & 1);
  }
  return a;
}

__device__ __forceinline__ bf16x8 lds_tr8(const char* lo, const char* hi) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)lo);
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)hi);
  return __builtin_bit_cast(bf16x8, (i16x8)__builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Softmax state and output accumulator of one wave (32 heads).
//
// The exponent reference m_ref of each head is fixed at the max of its first
// tile and never moves, so the accumulator is never rescaled (a rescale
// would need vector ALU passes over all 256 accumulator registers). A later
// score may exceed m_ref by up to OVERFLOW_SLACK (p <= 2^64, far from fp32 or
// bf16 overflow); a larger excess is reported and the workgroup recomputes
// the split with m_ref set to the split's true maximum.
constexpr float OVERFLOW_SLACK = 64.0f;  // log2 units

struct WaveState {
  f32x16 o[D_C / 32];   // O^T tiles: lane holds head l%32, dims 32dt + 8(r/4) + 4h + r%4
  float m_ref;          // exponent reference (log2 units), -inf before the first tile
  float lsum;           // this lane's share of the softmax denominator
};

// max(x[l], x[l ^ 32]): the two half-waves hold the two token halves of the
// same heads. v_permlane32_swap exchanges lanes 32-63 of its first operand
// with lanes 0-31 of its second, so with both operands x the two results
// hold, in every lane, x of that lane and x of its partner.
__device__ __forceinline__ float pair_max(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)sw[0]), __builtin_bit_cast(float, (unsigned)sw[1]));
}

// The S^T accumulator of the QK^T chain is kept in VGPRs (the 256 AGPRs
// hold O^T; the compiler would otherwise park an O^T tile in VGPRs and copy
// it back and forth around every tile, and copy S^T out of AGPRs). Inline
// assembly fixes the register class; the compiler does not see these as
// MFMAs, so the wait states an XDL result needs before a vector ALU read are
// inserted explicitly (mfma_vgpr_settle, bound to the accumulator so no read
// moves above it). Back-to-back MFMAs accumulating into the same registers
// need none.
__device__ __forceinline__ void mfma_vgpr_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_vgpr_acc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_vgpr_settle(f32x16& acc) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(acc));
}

// S^T = K Q^T for one tile: this lane's 16 scores (scaled for fp8; masked
// past the split's end, which only its last tile reaches). With FIRST the
// tile's max of this lane's head is returned (the exponent reference comes
// from the first tile); otherwise no max is taken. The A operands are read
// from LDS three k-steps ahead of the MFMA that consumes them (a software
// pipeline pinned with scheduling barriers), so LDS latency overlaps the
// MFMA chain. `issue(j)` runs after k-step j's MFMA (the main loop issues
// the next tile's loads there).
template <int CK, bool FIRST, typename Issue>
__device__ __forceinline__ float tile_scores(const char* tile, const float* scale, int tile_t0,
                                             int t1, const bf16x8 (&qreg)[QREG],
                                             const bf16x8 (&qpe)[QLDS], const LaneAddr& la, int h,
                                             float (&sv)[16], const Issue& issue) {
  constexpr int NJ = D_QK / 16;   // 36 k-steps
  constexpr int AHEAD = 3;
  auto a_off = [&](int j) { return (j < 32) ? la.qb[j & 7] + 256 * (j >> 3) : la.rb[j - 32]; };
  bf16x8 ring[AHEAD + 1];
#pragma unroll
  for (int j = 0; j < AHEAD; ++j) ring[j] = *(const bf16x8*)(tile + a_off(j));
  f32x16 sacc;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    if (j + AHEAD < NJ) ring[(j + AHEAD) % (AHEAD + 1)] = *(const bf16x8*)(tile + a_off(j + AHEAD));
    const bf16x8 bq = (j < QREG) ? qreg[j < QREG ? j : 0] : qpe[j < QREG ? 0 : j - QREG];
    if (j == 0) mfma_vgpr_first(sacc, ring[0], bq);
    else mfma_vgpr_acc(sacc, ring[j % (AHEAD + 1)], bq);
    issue(j);
    __builtin_amdgcn_sched_barrier(0);
  }
  mfma_vgpr_settle(sacc);
  // accumulator row r of this lane is token 8(r/4) + 4h + r%4 of the tile
  // fp8 cache: the row scales of this lane's 16 rows, 4 consecutive rows per
  // 16-byte read
  f32x4 sc4[4];
  if (CK == CACHE_FP8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sc4[i] = *(const f32x4*)(scale + 8 * i + 4 * h);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) sv[r] = (CK == CACHE_FP8) ? sacc[r] * sc4[r >> 2][r & 3] : sacc[r];
  if (tile_t0 + TILE > t1) {   // wave-uniform: the split's last tile only
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (tile_t0 + 8 * (r >> 2) + 4 * h + (r & 3) >= t1) sv[r] = -INFINITY;
  }
  if (!FIRST) return 0.f;
  float m4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    m4[i] = fmaxf(fmaxf(sv[4 * i], sv[4 * i + 1]), fmaxf(sv[4 * i + 2], sv[4 * i + 3]));
  return pair_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
}

// Every weight of a split is 2^(score - m_ref) <= its lane's share of the
// softmax denominator, so a share below 2^64 bounds every weight (and the
// accumulators) far from fp32 and bf16 overflow. A share at or above it
// (or NaN) can only come from a score well above the first tile's max: the
// workgroup then recomputes the split against the true max.
__device__ __forceinline__ bool split_overflowed(const WaveState& st) {
  return __any(!(st.lsum < 0x1p64f));
}

// Compile-time loop: f(std::integral_constant<int, i>) for i in [0, N).
template <typename F, int... I>
__device__ __forceinline__ void static_for_(const F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(const F& f) {
  static_for_(f, std::make_integer_sequence<int, N>{});
}

// Slot schedule of a pipelined step with nq S^T MFMAs and np PV MFMAs
// (both nonzero): two PV slots first (their operands were read before the
// step's barrier; the step's own K operands are still in flight), then the
// S^T chain spread evenly over the slots up to the last `tail` ones, which
// are PV (they cover the softmax work after the chain's end).
constexpr int SLOT_HEAD = 2, SLOT_TAIL = 6;
constexpr bool slot_is_q(int t, int nq, int np) {
  if (!nq) return false;
  if (!np) return true;
  const int span = nq + np - SLOT_HEAD - SLOT_TAIL;   // slots holding all S^T MFMAs
  if (t < SLOT_HEAD || t >= SLOT_HEAD + span) return false;
  const int u = t - SLOT_HEAD;
  return ((u + 1) * nq) / span != (u * nq) / span;   // nq of the span's slots, evenly
}
constexpr int slot_q_index(int t, int nq, int np) {
  int c = 0;
  for (int i = 0; i < t; ++i) c += slot_is_q(i, nq, np) ? 1 : 0;
  return c;
}

// Cross-tile software pipeline (bf16 kernel). Step j runs, in one stream of
// MFMA slots,
//   * O^T += C^T P^T of tile j-1 (32 MFMAs into 16 independent
//     accumulators), with the weights of its last 16 tokens formed between
//     the first of them (those of its first 16 came from step j-1);
//   * S^T of tile j into sn (36 MFMAs, one dependent chain), and after it
//     the first half of tile j's softmax (masked past the split's end on its
//     last tile; on the split's first tile its max becomes the exponent
//     reference) into pb[0], and the first PV operands of tile j into pring,
//     all before the step's barrier.
// The next step thus starts with PV MFMAs whose operands are in registers
// while its K operands are read, and the matrix pipe stays fed through the
// softmax and across step boundaries. The first step only computes S^T,
// the last only PV. `issue(t, n)` runs after slot t of the step's n.
// SCALED (fp8 cache, tiles holding the widened codes): `kscl` / `vscl` are
// the row scales of the S^T tile and of the PV tile (LDS); a row's scale
// multiplies its scores and, after the softmax sums, its weights.
template <bool DO_QK, bool DO_PV, bool K_FIRST, bool SCALED = false, typename Issue>
__device__ __forceinline__ void pipe_step(const char* kt, const char* vt, int k_t0, int t1,
                                          const bf16x8 (&qreg)[QREG], const char* qpe,
                                          const LaneAddr& la, int h, WaveState& st,
                                          f32x16& sn, f32x16& sp, bf16x8 (&pb)[2],
                                          bf16x8 (&pring)[3], const Issue& issue,
                                          const float* kscl = nullptr,
                                          const float* vscl = nullptr) {
  constexpr int NQ = DO_QK ? D_QK / 16 : 0, NP = DO_PV ? 32 : 0, NSLOT = NQ + NP;
  constexpr int QA = 2, PA = 2;   // LDS read lookahead, in MFMAs of each chain
  auto a_off = [&](int j) { return (j < 32) ? la.qb[j & 7] + 256 * (j >> 3) : la.rb[j - 32]; };
  auto v_op = [&](const char* tile, int s) {
    const int ks = s >> 4, dt = s & 15;
    const int off = 256 * (dt >> 2) + ks * 16 * LAT_ROW;
    return lds_tr8(tile + la.tb[0][dt & 3] + off, tile + la.tb[1][dt & 3] + off);
  };
  // qring: K operands; rring: the RoPE k-steps' query operands (from LDS,
  // `qpe` is this lane's slot, k-step i at +1 KB i)
  bf16x8 qring[QA + 1], rring[QA + 1];
  if (DO_QK) {
#pragma unroll
    for (int j = 0; j < QA; ++j) qring[j] = *(const bf16x8*)(kt + a_off(j));
  }
  const float mref_pv = st.m_ref;
  auto half_sum = [&](f32x16& v, int r0) {
    float half = ((v[r0] + v[r0 + 1]) + (v[r0 + 2] + v[r0 + 3])) +
                 ((v[r0 + 4] + v[r0 + 5]) + (v[r0 + 6] + v[r0 + 7]));
    asm volatile("" : "+v"(half));
    st.lsum += half;
  };
  auto pack = [&](const f32x16& v, int r) {   // rows r, r+1 into the B operand
    pb[r >> 3][r & 7] = (bf16)v[r];
    pb[r >> 3][(r & 7) + 1] = (bf16)v[r + 1];
  };
  // register r of a score / weight fragment is token row 8(r/4) + 4h + r%4:
  // rows 4h + 0..3 + 8i are the f32x4 at 8i + 4h of the tile's scales
  f32x4 ksc[4], vsc[2];
  auto load_ksc = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) ksc[i] = *(const f32x4*)(kscl + 8 * i + 4 * h);
  };
  auto pack_scaled = [&](const f32x16& v, int r, const f32x4& sc) {   // rows r, r+1 (r even)
    pb[r >> 3][r & 7] = (bf16)(v[r] * sc[r & 3]);
    pb[r >> 3][(r & 7) + 1] = (bf16)(v[r + 1] * sc[(r & 3) + 1]);
  };
  // after the S^T chain (sn settled): mask, reference, first-half weights
  float mref_k = 0.f;
  auto softmax_head = [&]() {
    if constexpr (SCALED) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sn[r] *= ksc[r >> 2][r & 3];
    }
    if (k_t0 + TILE > t1) {   // wave-uniform: the split's last tile only
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (k_t0 + 8 * (r >> 2) + 4 * h + (r & 3) >= t1) sn[r] = -INFINITY;
    }
    if (K_FIRST) {
      float m4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        m4[i] = fmaxf(fmaxf(sn[4 * i], sn[4 * i + 1]), fmaxf(sn[4 * i + 2], sn[4 * i + 3]));
      const float tmax = pair_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
      st.m_ref = (st.m_ref == -INFINITY) ? tmax : st.m_ref;
    }
    mref_k = st.m_ref;
  };
  // S^T-only step: everything after the chain
  constexpr int HEAD_AT = DO_PV ? SLOT_HEAD + (NQ + NP - SLOT_HEAD - SLOT_TAIL) : NQ;
  __builtin_amdgcn_sched_barrier(0);
  static_for<NSLOT>([&](auto tc) {
    constexpr int t = decltype(tc)::value;
    constexpr bool is_q = slot_is_q(t, NQ, NP);
    constexpr int qi = slot_q_index(t, NQ, NP);
    constexpr int pi = t - qi;
    if constexpr (is_q) {
      if constexpr (qi == 0) {
        mfma_vgpr_first(sn, qring[0], qreg[0]);
      } else if constexpr (qi < QREG) {
        mfma_vgpr_acc(sn, qring[qi % (QA + 1)], qreg[qi]);
      } else {
        mfma_vgpr_acc(sn, qring[qi % (QA + 1)], rring[qi % (QA + 1)]);
      }
      if constexpr (qi + QA < NQ) qring[(qi + QA) % (QA + 1)] = *(const bf16x8*)(kt + a_off(qi + QA));
      if constexpr (qi + QA >= QREG && qi + QA < NQ)
        rring[(qi + QA) % (QA + 1)] = *(const bf16x8*)(qpe + 1024 * (qi + QA - QREG));
      if constexpr (qi == NQ - 1) mfma_vgpr_settle(sn);
    } else {
      constexpr int dt = pi & 15;
      st.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pring[pi % (PA + 1)], pb[pi >> 4], st.o[dt], 0, 0, 0);
      if constexpr (pi + PA < NP) pring[(pi + PA) % (PA + 1)] = v_op(vt, pi + PA);
      // second half of tile j-1's weights
      if constexpr (pi < 8) sp[8 + pi] = fast_exp2(sp[8 + pi] - mref_pv);
      if constexpr (pi == 8) half_sum(sp, 8);
      if constexpr (SCALED && pi == 4) {
        vsc[0] = *(const f32x4*)(vscl + 16 + 4 * h);
        vsc[1] = *(const f32x4*)(vscl + 24 + 4 * h);
      }
      if constexpr (pi >= 9 && pi < 13) {
        if constexpr (SCALED)
          pack_scaled(sp, 8 + 2 * (pi - 9), vsc[(pi - 9) >> 1]);
        else
          pack(sp, 8 + 2 * (pi - 9));
      }
    }
    // tile j's softmax head over the tail slots, and its first PV operands
    // once the last two PV MFMAs have read the ring entries they replace
    if constexpr (DO_QK && DO_PV) {
      constexpr int u = t - (HEAD_AT - 1);   // 0 at the chain's last slot
      if constexpr (SCALED && u == -4) load_ksc();
      if constexpr (u == 0) softmax_head();
      if constexpr (u >= 0 && u < 4) {
        sn[2 * u] = fast_exp2(sn[2 * u] - mref_k);
        sn[2 * u + 1] = fast_exp2(sn[2 * u + 1] - mref_k);
      }
      if constexpr (u == 3) {
        half_sum(sn, 0);
#pragma unroll
        for (int r = 0; r < 8; r += 2) {
          if constexpr (SCALED)
            pack_scaled(sn, r, ksc[r >> 2]);
          else
            pack(sn, r);
        }
      }
      if constexpr (t == NSLOT - 2) pring[0] = v_op(kt, 0);
      if constexpr (t == NSLOT - 1) pring[1] = v_op(kt, 1);
    }
    issue(t, NSLOT);
    __builtin_amdgcn_sched_barrier(0);
  });
  if constexpr (DO_QK && !DO_PV) {   // S^T-only step: the head after the chain
    if constexpr (SCALED) load_ksc();
    softmax_head();
#pragma unroll
    for (int r = 0; r < 8; ++r) sn[r] = fast_exp2(sn[r] - mref_k);
    half_sum(sn, 0);
#pragma unroll
    for (int r = 0; r < 8; r += 2) {
      if constexpr (SCALED)
        pack_scaled(sn, r, ksc[r >> 2]);
      else
        pack(sn, r);
    }
    pring[0] = v_op(kt, 0);
    pring[1] = v_op(kt, 1);
  }
}

// Map a flat workgroup id to (sequence*split index q, head group g).
// Workgroups are dispatched round-robin over the 8 XCDs (x mod 8), each with
// its own L2; every XCD gets a contiguous range of q, so the head groups and
// the splits of one sequence (which share its queries and rows) run on the
// same XCD. `per` = ceil(B*S / 8); the grid is 8 * per * G workgroups.
__device__ __forceinline__ void xcd_map(int x, int G, int per, int& q, int& g) {
  const int rest = x >> 3;
  g = rest % G;
  q = (x & 7) * per + rest / G;
}

// Paged caches: the block-table entries a split touches are copied to LDS
// once (at most MAX_SPLIT_BLOCKS; the split planner keeps every split within
// that), so finding a tile's physical row is an LDS read instead of a global
// or scalar load in the loop. Returns the first block index of the split.
constexpr int MAX_SPLIT_BLOCKS = 64;

template <int NT>
__device__ __forceinline__ int load_block_table(const DecodeParams& p, int b, int t0, int t1,
                                                int* tab, int tid) {
  if (!p.block_table) return 0;
  const int first = t0 / p.block_size;
  const int nblk = min((t1 - 1) / p.block_size - first + 1, MAX_SPLIT_BLOCKS);
  const int32_t* src = p.block_table + (int64_t)b * p.max_blocks + first;
#if MLA_DEBUG_CHECKS
  const int64_t nblocks = p.rows / p.block_size;
  for (int i = tid; i < nblk; i += NT) {
    tab[i] = src[i];
    debug_flag(src[i] < 0 || src[i] >= nblocks, DBG_BLOCK);
  }
#else
  for (int i = tid; i < nblk; i += NT) tab[i] = src[i];
#endif
  return first;
}

__device__ __forceinline__ int first_blk_of(const DecodeParams& p, int t0) {
  return p.block_table ? t0 / p.block_size : 0;
}

// Scalar (SMEM) load of a wave-uniform int, waited for inside the asm block
// (counted on lgkmcnt, so it does not wait for tile loads in flight).
__device__ __forceinline__ int scalar_load_i32(const int32_t* ptr) {
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(ptr) : "memory");
  return v;
}

// Physical rows of the first tokens of two tiles, reading their block
// entries from global memory with one wait (before the split's table is in
// LDS).
__device__ __forceinline__ void tile_base_rows_direct2(const DecodeParams& p, int b, int ta, int tb,
                                                      int& ra, int& rb) {
  if (p.block_table) {
    const int ia = __builtin_amdgcn_readfirstlane(b * p.max_blocks + ta / p.block_size);
    const int ib = __builtin_amdgcn_readfirstlane(b * p.max_blocks + tb / p.block_size);
    int va, vb;
    asm volatile("s_load_dword %0, %2, 0x0\n\ts_load_dword %1, %3, 0x0\n\ts_waitcnt lgkmcnt(0)"
                 : "=&s"(va), "=&s"(vb)
                 : "s"(p.block_table + ia), "s"(p.block_table + ib)
                 : "memory");
    ra = va * p.block_size + (ta % p.block_size);
    rb = vb * p.block_size + (tb % p.block_size);
  } else {
    ra = (int)((int64_t)b * p.seq_capacity + ta);
    rb = (int)((int64_t)b * p.seq_capacity + tb);
  }
}

// Physical row of the first token of a tile, reading the block entry from
// global memory (before the split's table is in LDS).
__device__ __forceinline__ int64_t tile_base_row_direct(const DecodeParams& p, int b, int tile_t0) {
  if (p.block_table) {
    const int idx = __builtin_amdgcn_readfirstlane(b * p.max_blocks + tile_t0 / p.block_size);
    const int blk = scalar_load_i32(p.block_table + idx);
    return (int64_t)blk * p.block_size + (tile_t0 % p.block_size);
  }
  return (int64_t)b * p.seq_capacity + tile_t0;
}

// Physical rows of the first token of each tile of a split, tile i in lane
// i (a split has at most 64 tiles: the split planner keeps it so), so a
// tile's row in the loop is one v_readlane. Rows fit in 32 bits (the ABI
// rejects larger caches). `tab` is the split's block table in LDS.
__device__ __forceinline__ int tile_rows_lanes(const DecodeParams& p, int b, int t0, int t1,
                                               const int* tab, int first_blk, int l) {
  const int t = t0 + TILE * min(l, max((t1 - t0 + TILE - 1) / TILE - 1, 0));
  if (p.block_table) return tab[t / p.block_size - first_blk] * p.block_size + (t % p.block_size);
  return (int)((int64_t)b * p.seq_capacity + t);
}

// Buffer resource over [base, base + bytes) for raw buffer loads: accesses at
// or past `bytes` return zeros instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int32_t n = (int32_t)min(max(bytes, (int64_t)0), (int64_t)0x7FFFFFF0);
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, n, 0x00020000);
}

// Buffer resources of one tile: the latent and RoPE-key arrays rebased at the
// tile's first physical row, with a record count of `nvalid` rows, so rows
// past the split's end (all rows of a tile past the split: nvalid = 0) read
// as zeros. A row index outside the cache reads row 0 instead (never faults).
// Row strides are below 2^24 bytes (the ABI checks), so every offset inside
// a tile fits in 32 bits.
struct TileRsrc {
  __amdgpu_buffer_rsrc_t lat, rope;
};

__device__ __forceinline__ TileRsrc tile_rsrc(const DecodeParams& p, int row0, int nvalid,
                                              int esize) {
  TileRsrc t;
  const int rows = (int)p.rows;   // below 2^31 (the ABI checks)
  row0 = __builtin_amdgcn_readfirstlane((row0 >= 0 && row0 < rows) ? row0 : 0);
  nvalid = __builtin_amdgcn_readfirstlane(max(min(nvalid, rows - row0), 0));
  const int lsb = (int)p.latent_stride * esize, rsb = (int)p.rope_stride * esize;
  t.lat = __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)p.latent + (int64_t)row0 * lsb),
                                            (short)0, nvalid * lsb, 0x00020000);
  t.rope = __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)p.rope + (int64_t)row0 * rsb),
                                             (short)0, nvalid * rsb, 0x00020000);
  return t;
}

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// One wave-wide direct-to-LDS load: 16 bytes per lane from rsrc + voffset
// (zeros past the resource's records) to LDS at m0_base + IMM + 16 * lane
// (m0_base wave-uniform).
//
// Written as inline assembly so that the compiler's wait-count tracking does
// not see it: it cannot tell which LDS buffer each pending load targets once
// control flow merges, and would then wait for every load in flight before
// each LDS read. The kernels wait for these loads themselves (vmcnt) before
// the barrier that publishes a tile, and fence the compiler there.
//
// M0 is written without being saved: the compiler uses M0 for nothing in the
// decode kernels (the library build checks the generated code for this and
// fails otherwise). The s_nop covers the M0-write hazard; the add writes SCC
// (declared, so no scalar condition is kept across the block).
template <int IMM>
__device__ __forceinline__ void dma16_m0(__amdgpu_buffer_rsrc_t rsrc, uint32_t m0_base, int voffset) {
  asm volatile(
      "s_add_u32 m0, %0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(m0_base), "v"(voffset), "s"(rsrc), "n"(IMM)
      : "memory", "scc");
}

// Compiler-only fence: no memory access moves across it (emits nothing).
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// bf16 cache: direct global->LDS loads (16 bytes per lane), 36 wave-wide
// loads per tile (32 latent rows of 1 KB, 4 groups of 8 RoPE-key rows), of
// which each of the NW waves issues PIECES: piece i < RPW is latent row
// u = w*RPW + i, the others are RoPE-key groups. Lane i writes LDS slot i of
// its 1 KB, so it fetches the chunk that the swizzle places there. The lane
// offsets of a wave's pieces relative to a tile's first row are the same for
// every tile (tile_piece_offsets, kept in registers); a tile only brings its
// two buffer resources.
//
// A wave that issues several direct-to-LDS loads back to back stalls at issue
// until the CU's memory pipeline accepts them, and issues nothing else
// meanwhile. The main loop therefore spreads the next tile's pieces through
// the MFMA chains of the current one (step(t) after MFMA t), where a stall
// only delays MFMAs already queued.
template <int NW>
struct TileLoad {
  static constexpr int RPW = TILE / NW;          // latent rows per wave
  static constexpr int GPW = 4 / NW;             // RoPE-key row groups per wave
  static constexpr int PIECES = RPW + GPW;       // 9, 18, 36
  TileRsrc rs;
  uint32_t m_lat, m_rope;   // LDS address of this wave's first latent row / RoPE group
  const int* voff;          // lane offsets of the pieces

  template <int I>
  __device__ __forceinline__ void piece() const {
    if constexpr (I < RPW) dma16_m0<I * LAT_ROW>(rs.lat, m_lat, voff[I]);
    else dma16_m0<(I - RPW) * 8 * ROPE_ROW>(rs.rope, m_rope, voff[I]);
  }
  template <int... I>
  __device__ __forceinline__ void all_(std::integer_sequence<int, I...>) const {
    (piece<I>(), ...);
  }
  __device__ __forceinline__ void all() const { all_(std::make_integer_sequence<int, PIECES>{}); }
  // after slot t of a pipelined step of n slots: piece i at
  // t = 1 + i * span / PIECES, span = min(n - 2, 2 PIECES) (every other slot
  // from the step's start while there is room), so the tile has most of two
  // steps to land; every piece goes out for any n >= 3
  template <int... I>
  __device__ __forceinline__ void step_n_(int t, int n, std::integer_sequence<int, I...>) const {
    const int span = min(n - 2, 2 * PIECES);
    ((t == 1 + (I * span) / PIECES ? piece<I>() : void()), ...);
  }
  __device__ __forceinline__ void step_n(int t, int n) const {
    step_n_(t, n, std::make_integer_sequence<int, PIECES>{});
  }
};

template <int NW>
__device__ __forceinline__ void tile_piece_offsets(const DecodeParams& p, int w, int l,
                                                   int (&voff)[TileLoad<NW>::PIECES]) {
  constexpr int RPW = TileLoad<NW>::RPW, GPW = TileLoad<NW>::GPW;
  const int lsb = (int)p.latent_stride * 2, rsb = (int)p.rope_stride * 2;
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int u = w * RPW + i;
    voff[i] = u * lsb + 16 * (l ^ lat_swz(u));
  }
#pragma unroll
  for (int i = 0; i < GPW; ++i) {
    const int row = 8 * (w * GPW + i) + (l >> 3);
    voff[RPW + i] = row * rsb + 16 * ((l & 7) ^ rope_swz(row));
  }
}

// Loads of one tile (first physical row row0, nvalid valid rows) into `tile`.
template <int NW>
__device__ __forceinline__ TileLoad<NW> tile_load(const DecodeParams& p, char* tile, int row0,
                                                  int nvalid, int w, const int* voff) {
  TileLoad<NW> t;
  t.rs = tile_rsrc(p, row0, nvalid, 2);
  t.m_lat = __builtin_amdgcn_readfirstlane(lds_u32(tile) + w * TileLoad<NW>::RPW * LAT_ROW);
  t.m_rope = __builtin_amdgcn_readfirstlane(lds_u32(tile) + ROPE_OFF +
                                            w * TileLoad<NW>::GPW * 8 * ROPE_ROW);
  t.voff = voff;
  return t;
}


// fp8 cache: the raw codes of a tile (32 rows x 576 bytes) and its 32 bf16
// row scales are brought into an LDS staging area with direct global->LDS
// loads, then widened to bf16 (exactly: e4m3 values are a subset of bf16)
// into the same swizzled tile layout as a bf16 cache, so the MFMA path is
// shared. Staging layout: latent [32][512], RoPE key [32][64], scales [32].
constexpr int STG_ROPE = TILE * D_C;                 // 16384
constexpr int STG_SCALE = STG_ROPE + TILE * D_R;     // 18432
constexpr int STG_BYTES = STG_SCALE;                 // codes only (18 KB)

// Per tile and wave: 16/NW latent pieces (two 512-byte rows each) and
// ceil(2/NW) RoPE-key pieces (16 rows each; with four waves, waves 2 and 3
// issue an empty load into a dummy area instead, so every wave issues the
// same number and the vmcnt waits stay exact). Loads are the direct-to-LDS
// loads of the bf16 kernel (resources rebased per tile, zeros past the
// split's end, per-piece lane offsets kept in registers); the row scales of
// the whole split are loaded into LDS by the prologue.
template <int NW>
struct Fp8Load {
  static constexpr int LAT = 16 / NW;
  static constexpr int ROPE = (2 + NW - 1) / NW;
  static constexpr int PIECES = LAT + ROPE;
  TileRsrc rs;                // rope: an empty resource on waves that only issue dummy loads
  uint32_t m_lat, m_rope;
  const int* voff;

  template <int I>
  __device__ __forceinline__ void piece() const {
    if constexpr (I < LAT) dma16_m0<I * 2 * D_C>(rs.lat, m_lat, voff[I]);
    else dma16_m0<(I - LAT) * 16 * D_R>(rs.rope, m_rope, voff[I]);
  }
  template <int... I>
  __device__ __forceinline__ void all_(std::integer_sequence<int, I...>) const {
    (piece<I>(), ...);
  }
  __device__ __forceinline__ void all() const { all_(std::make_integer_sequence<int, PIECES>{}); }
  template <int... I>
  __device__ __forceinline__ void step_(int t, std::integer_sequence<int, I...>) const {
    ((t == 2 + (64 * I) / PIECES ? piece<I>() : void()), ...);
  }
  // after MFMA t (0..67) of the tile being computed
  __device__ __forceinline__ void step(int t) const {
    step_(t, std::make_integer_sequence<int, PIECES>{});
  }
};

template <int NW>
__device__ __forceinline__ void fp8_piece_offsets(const DecodeParams& p, int w, int l,
                                                  int (&voff)[Fp8Load<NW>::PIECES]) {
  constexpr int LAT = Fp8Load<NW>::LAT, ROPE = Fp8Load<NW>::ROPE;
  const int lsb = (int)p.latent_stride, rsb = (int)p.rope_stride;
#pragma unroll
  for (int i = 0; i < LAT; ++i) voff[i] = (2 * (w * LAT + i) + (l >> 5)) * lsb + 16 * (l & 31);
#pragma unroll
  for (int i = 0; i < ROPE; ++i) {
    const int pc = min(w * ROPE + i, 1);
    voff[LAT + i] = (16 * pc + (l >> 2)) * rsb + 16 * (l & 3);
  }
}

template <int NW>
__device__ __forceinline__ Fp8Load<NW> fp8_load(const DecodeParams& p, char* stage, char* dummy,
                                                int row0, int nvalid, int w, const int* voff) {
  Fp8Load<NW> t;
  t.rs = tile_rsrc(p, row0, nvalid, 1);
  const bool real = w * Fp8Load<NW>::ROPE < 2;   // wave-uniform
  if (!real) t.rs.rope = make_rsrc(p.rope, 0);
  t.m_lat = __builtin_amdgcn_readfirstlane(lds_u32(stage) + w * Fp8Load<NW>::LAT * 2 * D_C);
  t.m_rope = __builtin_amdgcn_readfirstlane(
      real ? lds_u32(stage) + STG_ROPE + w * Fp8Load<NW>::ROPE * 16 * D_R : lds_u32(dummy));
  t.voff = voff;
  return t;
}


// Common prologue: work item of this workgroup, the empty-split case, the
// absorbed queries of this lane's head.
struct WorkItem {
  int b, s, t0, t1, head;
  _Float16* po;       // this lane's head row (+4 values for the upper half-wave)
  _Float16* po_wave;  // the row of the wave's first head
  float* pl;
  float* ps;
};

template <int NW>
__device__ __forceinline__ bool work_item(const DecodeParams& p, int w, int l, WorkItem& wi) {
  int q, g;
  const int nq = p.items ? p.nitems : p.B * p.S;
  xcd_map(blockIdx.x, p.G, (nq + 7) / 8, q, g);
  if (q >= nq) return false;
  if (p.items) {
    // (the planning kernel clamped the lengths and checked them)
    const SplitItem it = p.items[q];
    if (__builtin_amdgcn_readfirstlane(it.b) < 0) return false;
    wi.b = __builtin_amdgcn_readfirstlane(it.b);
    wi.s = __builtin_amdgcn_readfirstlane(it.s);
    wi.t0 = __builtin_amdgcn_readfirstlane(it.t0);
    wi.t1 = __builtin_amdgcn_readfirstlane(it.t1);
  } else {
    wi.b = __builtin_amdgcn_readfirstlane(q / p.S);
    wi.s = __builtin_amdgcn_readfirstlane(q - wi.b * p.S);
    const int raw_len = __builtin_amdgcn_readfirstlane(p.lengths[wi.b]);
    debug_flag(raw_len < 0 || raw_len > p.max_len, DBG_LENGTH);
    const int len = min(max(raw_len, 0), p.max_len);
    wi.t0 = wi.s * p.tokens_per_split;
    wi.t1 = min(wi.t0 + p.tokens_per_split, len);
  }
  wi.head = (g * NW + w) * 32 + (l & 31);
  wi.po = p.part_o + (((int64_t)wi.b * p.S + wi.s) * p.H + wi.head) * D_C + 4 * (l >> 5);
  wi.po_wave = p.part_o + (((int64_t)wi.b * p.S + wi.s) * p.H + (g * NW + w) * 32) * D_C;
  wi.pl = p.part_lse + ((int64_t)wi.b * p.S + wi.s) * p.H + wi.head;
  wi.ps = p.part_scale + ((int64_t)wi.b * p.S + wi.s) * p.H + wi.head;
  return true;
}

__device__ __forceinline__ void write_empty(const WorkItem& wi, int h) {
#pragma unroll
  for (int dt = 0; dt < 16; ++dt)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) *(f16x4*)(wi.po + 32 * dt + 8 * rq) = f16x4{0, 0, 0, 0};
  if (h == 0) {
    *wi.pl = -INFINITY;
    *wi.ps = 0.f;
  }
}

// The wave's normalised partial output (32 heads x 512 latent dims) is
// stored as fp16 relative to its row maximum (values in [-1, 1], the fp32
// factor in part_scale): half the bytes of fp32, and a rounding error
// (2^-11 of the row maximum) far below that of the bf16 operand the merge
// later feeds to the W_UV product. It goes out through LDS, 128 dims at a
// time: the accumulator layout puts the 32 heads across lanes (each store
// instruction would touch 32 rows 1 KB apart), so the values are first
// written to a [32 heads][128 dims] LDS block (rows padded by 16 bytes), then
// read back row-wise, and every store instruction writes four contiguous
// 256-byte row segments. `scr` is PART_SCR_BYTES of LDS owned by this wave.
constexpr int PART_ROW = 2 * 128 + 16;
constexpr int PART_SCR_BYTES = 32 * PART_ROW;   // 8704
constexpr int FLAG_OFF = 2 * PART_SCR_BYTES;     // overflow flags in a tile buffer
static_assert(FLAG_OFF + 64 <= TILE_BYTES, "flags fit in a tile buffer");

__device__ __forceinline__ void write_partial(const WorkItem& wi, const WaveState& st, int h,
                                              int l, char* scr) {
  const unsigned ul = __builtin_bit_cast(unsigned, st.lsum);
  const auto sw = __builtin_amdgcn_permlane32_swap(ul, ul, false, false);
  const float ltot = __builtin_bit_cast(float, (unsigned)sw[0]) + __builtin_bit_cast(float, (unsigned)sw[1]);
  float mx = 0.f;
#pragma unroll
  for (int dt = 0; dt < D_C / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fabsf(st.o[dt][r]));
  mx = pair_max(mx);
  const float f = (mx > 0.f) ? 1.0f / mx : 0.f;
  const int head = l & 31;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const f32x16& o = st.o[4 * c + d];
        const f16x4 v = {(_Float16)(o[4 * rq] * f), (_Float16)(o[4 * rq + 1] * f),
                         (_Float16)(o[4 * rq + 2] * f), (_Float16)(o[4 * rq + 3] * f)};
        *(f16x4*)(scr + head * PART_ROW + 2 * (32 * d + 8 * rq + 4 * h)) = v;
      }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 4 * i + (l >> 4);
      const u32x4 v = *(const u32x4*)(scr + row * PART_ROW + 16 * (l & 15));
      *(u32x4*)(wi.po_wave + row * D_C + 128 * c + 8 * (l & 15)) = v;
    }
  }
  if (h == 0) {
    *wi.pl = st.m_ref + __builtin_log2f(ltot);
    *wi.ps = mx / ltot;
  }
}

// Queries of this wave's 32 heads (operand layout, see qop_index): the 32
// latent k-steps into qreg, the 4 RoPE k-steps into qpe.
__device__ __forceinline__ void load_q(const DecodeParams& p, const WorkItem& wi, int l,
                                       bf16x8 (&qreg)[QREG], bf16x8 (&qpe)[QLDS]) {
  const bf16* qp = p.q + qop_index(wi.b, wi.head - (l & 31), 0, p.H) + 8 * l;
#pragma unroll
  for (int j = 0; j < QREG; ++j) qreg[j] = *(const bf16x8*)(qp + 512 * j);
#pragma unroll
  for (int j = 0; j < QLDS; ++j) qpe[j] = *(const bf16x8*)(qp + 512 * (QREG + j));
}

__device__ __forceinline__ void reset_state(WaveState& st, float m_ref) {
#pragma unroll
  for (int dt = 0; dt < D_C / 32; ++dt) st.o[dt] = f32x16{};
  st.m_ref = m_ref;
  st.lsum = 0.f;
}

// ---------------------------------------------------------------------------
// bf16 cache: three LDS tile buffers, two tiles of DMA in flight
// ---------------------------------------------------------------------------
template <int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_decode_bf16_kernel(DecodeParams p) {
  // four tile buffers and the RoPE k-steps of the queries (160 KB with four
  // waves); the split's block table and the waves' overflow flags borrow tile
  // buffer space while it is idle (the prologue; the end of a pass, in the
  // buffer after the last tile's, past the partial-output staging)
  __shared__ __attribute__((aligned(1024))) char bufs[4 * TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char qpe_all[NW * QLDS * 1024];
  constexpr int NT = 64 * NW;
  constexpr int DMA_PER_TILE = TileLoad<NW>::PIECES;  // wave-wide loads per tile per wave
  char* const buf0 = bufs;
  char* const buf1 = bufs + TILE_BYTES;
  char* const buf2 = bufs + 2 * TILE_BYTES;
  char* const buf3 = bufs + 3 * TILE_BYTES;
  int* const blk_tab = (int*)buf3;   // prologue only (tile 3 is loaded after it is read)

  const int tid = threadIdx.x, l = tid & 63, h = l >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  WorkItem wi;
  if (!work_item<NW>(p, w, l, wi)) return;
  if (wi.t0 >= wi.t1) {
    write_empty(wi, h);
    return;
  }
  const int ntiles = (wi.t1 - wi.t0 + TILE - 1) / TILE;
  int voff[DMA_PER_TILE];
  tile_piece_offsets<NW>(p, w, l, voff);
  // valid rows of tile k (0 past the split: its loads read nothing)
  auto nvalid = [&](int k) { return min(max(wi.t1 - (wi.t0 + k * TILE), 0), TILE); };
  int trow = 0;   // lane i: physical row of tile i's first token (set in the prologue)
  auto load = [&](char* tile, int k) {
    return tile_load<NW>(p, tile, __builtin_amdgcn_readlane(trow, min(k, ntiles - 1)), nvalid(k),
                         w, voff);
  };
  const auto no_issue = [](int) {};

  // Prologue: the queries (independent of everything else), the block
  // entries of tiles 0 and 1 (scalar path, one wait), their loads, the rest
  // of the split's block table; then one wait for all of it. The compiler
  // does not count the tile loads, so a wait it placed for the query loads
  // inside the loop would drain every tile load in flight. The tile buffers
  // need no clearing: a tile's loads write all of its bytes (zeros past the
  // split's end).
  bf16x8 qreg[QREG], qtmp[QLDS];
  load_q(p, wi, l, qreg, qtmp);
  {
    int r0, r1;
    tile_base_rows_direct2(p, wi.b, wi.t0, wi.t0 + min(1, ntiles - 1) * TILE, r0, r1);
    tile_load<NW>(p, buf0, r0, nvalid(0), w, voff).all();
    tile_load<NW>(p, buf1, r1, nvalid(1), w, voff).all();
  }
  load_block_table<NT>(p, wi.b, wi.t0, wi.t1, blk_tab, tid);
  char* const qpe = qpe_all + w * (QLDS * 1024) + 16 * l;   // this lane's RoPE query slot
  const LaneAddr la = lane_addr(l);
  WaveState st;
  reset_state(st, -INFINITY);
  wait_vm_lgkm0<0>();
#pragma unroll
  for (int j = 0; j < QLDS; ++j) *(bf16x8*)(qpe + 1024 * j) = qtmp[j];
  __builtin_amdgcn_s_barrier();
  compiler_fence();
  // (buffer 3 holds the table until tile 3's loads, issued after every wave
  // has passed step 0's barrier)
  trow = tile_rows_lanes(p, wi.b, wi.t0, wi.t1, blk_tab, first_blk_of(p, wi.t0), l);

  for (int attempt = 0; attempt < 2; ++attempt) {
    if (attempt > 0) {
      load(buf0, 0).all();
      load(buf1, 1).all();
      wait_vm_lgkm0<DMA_PER_TILE>();   // tile 0 landed (tile 1 may be in flight)
      __builtin_amdgcn_s_barrier();
      compiler_fence();
    }
    // Tile t lives in buffer t mod 4. Step j computes S^T of tile j and PV of
    // tile j-1 (see pipe_step) while tile j+2 loads into the buffer of tile
    // j-2, then waits for tile j+1 and meets the other waves at the barrier,
    // after which tile j-1's buffer is free. Every real step issues the same
    // number of loads (those of tiles past the split read nothing), so the
    // vmcnt waits stay exact; steps past the last tile, which only come
    // after every real one, do nothing (a load there could land in the last
    // tile's buffer before the final step reads it).
    f32x16 s0, s1;    // scores of even / odd tiles
    bf16x8 pb[2];     // PV B operand (weights of the tile whose PV is next)
    bf16x8 pring[3];  // PV A operands in flight
    auto step_end = [&]() {
      // tile j+1 landed, tile j+2 may be in flight
      wait_vm_lgkm0<DMA_PER_TILE>();
      __builtin_amdgcn_s_barrier();
      compiler_fence();               // no LDS read of tile j+1 moves above this
    };
    // the next tile's loader is set up after the step's first MFMA (its
    // scalar work hides behind it; the first load goes out after slot 1)
    {
      TileLoad<NW> next;
      pipe_step<true, false, true>(buf0, nullptr, wi.t0, wi.t1, qreg, qpe, la, h, st, s0, s1, pb,
                                   pring, [&](int t, int n) {
                               if (t == 0) next = load(buf2, 2);
                               next.step_n(t, n);
                             });
      step_end();
    }
    auto step = [&](char* K, char* V, char* Z, int j, f32x16& sn, f32x16& sp) {
      if (j < ntiles) {
        TileLoad<NW> next;
        pipe_step<true, true, false>(K, V, wi.t0 + j * TILE, wi.t1, qreg, qpe, la, h, st, sn, sp,
                                     pb, pring, [&](int t, int n) {
                                if (t == 0) next = load(Z, j + 2);
                                next.step_n(t, n);
                              });
        step_end();
      }
    };
    for (int j = 1; j < ntiles; j += 4) {
      step(buf1, buf0, buf3, j, s1, s0);
      step(buf2, buf1, buf0, j + 1, s0, s1);
      step(buf3, buf2, buf1, j + 2, s1, s0);
      step(buf0, buf3, buf2, j + 3, s0, s1);
    }
    {   // softmax and PV of the last tile
      const int last = ntiles - 1;
      f32x16 sl = (last & 1) ? s1 : s0;
      pipe_step<false, true, false>(nullptr, bufs + (last & 3) * TILE_BYTES, 0, wi.t1, qreg, qpe,
                                    la, h, st, sl, sl, pb, pring, [](int, int) {});
    }
    // The waves' overflow flags go through the buffer after the last tile's
    // (no step reads it; the loads of the tiles past the end, which write
    // zeros there, are drained first), past the bytes write_partial stages
    // in. After the one barrier every wave is also done reading tiles.
    const bool ovf = split_overflowed(st);
    int* const flags = (int*)(bufs + (ntiles & 3) * TILE_BYTES + FLAG_OFF);
    wait_vm_lgkm0<0>();
    if (l == 0) flags[w] = ovf ? 1 : 0;
    wait_vm_lgkm0<0>();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    int any_ovf = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) any_ovf |= flags[i];
    any_ovf = __builtin_amdgcn_readfirstlane(any_ovf);
    if (any_ovf == 0) break;
    wait_vm_lgkm0<0>();
    __builtin_amdgcn_s_barrier();   // every wave has read the flags
    compiler_fence();

    // Rare path: a weight reached 2^64 against the first tile's max (or the
    // sum is NaN). Drain the loads in flight, find each head's true maximum
    // over the split (scores only), then recompute the split against it.
    float mtrue = -INFINITY;
    for (int k = 0; k < ntiles; ++k) {
      load(buf0, k).all();
      wait_vm_lgkm0<0>();
      __builtin_amdgcn_s_barrier();
      compiler_fence();
      float sv[16];
      bf16x8 qp[QLDS];
#pragma unroll
      for (int j = 0; j < QLDS; ++j) qp[j] = *(const bf16x8*)(qpe + 1024 * j);
      mtrue = fmaxf(mtrue, tile_scores<CACHE_BF16, true>(buf0, nullptr, wi.t0 + k * TILE, wi.t1,
                                                         qreg, qp, la, h, sv, no_issue));
      __builtin_amdgcn_s_barrier();
      compiler_fence();
    }
    reset_state(st, mtrue);
  }
  // (every load has landed and every wave is past its last tile read: the
  // flag exchange above ended with both)
  write_partial(wi, st, h, l, (w < 2 ? buf0 : buf1) + (w & 1) * PART_SCR_BYTES);
}

// ---------------------------------------------------------------------------
// fp8 cache, pipelined: the bf16 kernel's cross-tile pipeline (pipe_step,
// SCALED) over tiles widened to bf16 in LDS. Tile t lives in bf16 buffer
// t mod 3: step j reads tile j (S^T) and tile j-1 (PV) and widens tile j+1
// into the third buffer, which step j-1 finished reading. The raw codes of
// one tile at a time wait in a staging tile, filled by the direct-to-LDS
// loads of Fp8Load: every lane widens exactly the 16-byte pieces its own
// loads wrote there, so as soon as its reads are done it loads the next
// tile's codes into the same bytes, with no barrier. The widening runs in
// the step's early MFMA slots, the next tile's loads right after it (they
// then have the rest of the step and the next step's first slots to land).
// The row scales of the split sit in LDS; pipe_step applies them to the
// scores and the weights (SCALED).
// ---------------------------------------------------------------------------

// Widen piece I (a 16-byte chunk of 16 codes) of this lane's share of a
// staged tile into a bf16 tile (e4m3 codes are exact in bf16; the row scales
// are applied in the attention math). Latent pieces I < LAT (row
// 2(w LAT + I) + l/32, codes 16 (l mod 32) ..), RoPE piece I = LAT (row
// 16 pc + l/4, codes 16 (l mod 4) .., only on the waves whose RoPE loads are
// real).
template <int NW, int I>
__device__ __forceinline__ void widen_own_piece(const char* stg, char* tile, int w, int l) {
  constexpr int LAT = Fp8Load<NW>::LAT, ROPE = Fp8Load<NW>::ROPE;
  // addresses are recomputed at each use (a few ALU operations): kept live
  // across the loop they would not fit in the registers
  asm volatile("" : "+v"(l));
  const char* src;
  char* row_base;
  int c, sw;
  if constexpr (I < LAT) {
    const int row = 2 * (w * LAT + I) + (l >> 5);
    c = l & 31;
    sw = lat_swz(row);
    src = stg + (w * LAT + I) * 1024 + 16 * l;
    row_base = tile + row * LAT_ROW;
  } else {
    const int pc = w * ROPE + (I - LAT);
    const int row = 16 * pc + (l >> 2);
    c = l & 3;
    sw = rope_swz(row);
    src = stg + STG_ROPE + pc * 1024 + 16 * l;
    row_base = tile + ROPE_OFF + row * ROPE_ROW;
  }
  const u32x4 v = *(const u32x4*)src;
  u32x4 lo, hi;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    lo[2 * j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[j], 1.0f, false));
    lo[2 * j + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[j], 1.0f, true));
    hi[2 * j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[j + 2], 1.0f, false));
    hi[2 * j + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[j + 2], 1.0f, true));
  }
  // the read has returned before anything after this point (the next
  // tile's loads into the same staging bytes) is issued
  asm volatile("" ::"v"(lo[0]), "v"(hi[0]));
  *(u32x4*)(row_base + 16 * ((2 * c) ^ sw)) = lo;
  *(u32x4*)(row_base + 16 * ((2 * c + 1) ^ sw)) = hi;
}

// Every piece of this lane's share (the RoPE piece only where it is real).
template <int NW, int... I>
__device__ __forceinline__ void widen_own_all_(const char* stg, char* tile, int w, int l,
                                               bool rope_real, std::integer_sequence<int, I...>) {
  ((I < Fp8Load<NW>::LAT || rope_real ? widen_own_piece<NW, I>(stg, tile, w, l) : void()), ...);
}
template <int NW>
__device__ __forceinline__ void widen_own_all(const char* stg, char* tile, int w, int l,
                                              bool rope_real) {
  widen_own_all_<NW>(stg, tile, w, l, rope_real,
                     std::make_integer_sequence<int, Fp8Load<NW>::PIECES>{});
}
// The same, piece I after MFMA slot 2 + 3 I of a step.
constexpr int WIDEN_SLOT0 = 2, WIDEN_EVERY = 3;
constexpr int fp8_load_slot(int pieces) { return WIDEN_SLOT0 + WIDEN_EVERY * pieces; }
template <int NW, int... I>
__device__ __forceinline__ void widen_own_at_(int t, const char* stg, char* tile, int w, int l,
                                              bool rope_real, std::integer_sequence<int, I...>) {
  ((t == WIDEN_SLOT0 + WIDEN_EVERY * I && (I < Fp8Load<NW>::LAT || rope_real)
        ? widen_own_piece<NW, I>(stg, tile, w, l)
        : void()),
   ...);
}

template <int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_decode_fp8_kernel(DecodeParams p) {
  constexpr int NT = 64 * NW;
  constexpr int P = Fp8Load<NW>::PIECES;
  constexpr int LOAD_SLOT = fp8_load_slot(P);   // after the widening's last piece
  __shared__ __attribute__((aligned(1024))) char bufs[3 * TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char qpe_all[NW * QLDS * 1024];
  __shared__ __attribute__((aligned(1024))) char stage[STG_BYTES];
  __shared__ __attribute__((aligned(1024))) char dummy[1024];
  __shared__ __attribute__((aligned(16))) float scl_all[64 * TILE];   // tile i at 32 i
  __shared__ int blk_tab[MAX_SPLIT_BLOCKS];
  __shared__ int flags[NW];
  char* const buf0 = bufs;
  char* const buf1 = bufs + TILE_BYTES;
  char* const buf2 = bufs + 2 * TILE_BYTES;

  const int tid = threadIdx.x, l = tid & 63, h = l >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  WorkItem wi;
  if (!work_item<NW>(p, w, l, wi)) return;
  if (wi.t0 >= wi.t1) {
    write_empty(wi, h);
    return;
  }
  const int ntiles = (wi.t1 - wi.t0 + TILE - 1) / TILE;
  const bool rope_real = w * Fp8Load<NW>::ROPE < 2;   // wave-uniform
  int voff[P];
  fp8_piece_offsets<NW>(p, w, l, voff);
  auto nvalid = [&](int k) { return min(max(wi.t1 - (wi.t0 + k * TILE), 0), TILE); };
  int trow = 0;   // lane i: physical row of tile i's first token (set in the prologue)
  auto load_raw = [&](char* stg, int k) {
    return fp8_load<NW>(p, stg, dummy, __builtin_amdgcn_readlane(trow, min(k, ntiles - 1)),
                        nvalid(k), w, voff);
  };

  // Prologue: raw tile 0 into the staging tile, raw tile 1 into buffer 2
  // (idle until step 1 widens tile 2 into it), the queries, the block table;
  // one wait; the RoPE query k-steps and the split's row scales into LDS;
  // tile 0 widened into buffer 0.
  fp8_load<NW>(p, stage, dummy, (int)tile_base_row_direct(p, wi.b, wi.t0), nvalid(0), w, voff).all();
  fp8_load<NW>(p, buf2, dummy, (int)tile_base_row_direct(p, wi.b, wi.t0 + min(1, ntiles - 1) * TILE),
               nvalid(1), w, voff)
      .all();
  bf16x8 qreg[QREG], qtmp[QLDS];
  load_q(p, wi, l, qreg, qtmp);
  load_block_table<NT>(p, wi.b, wi.t0, wi.t1, blk_tab, tid);
  char* const qpe = qpe_all + w * (QLDS * 1024) + 16 * l;   // this lane's RoPE query slot
  const LaneAddr la = lane_addr(l);
  WaveState st;
  reset_state(st, -INFINITY);
  wait_vm_lgkm0<0>();
#pragma unroll
  for (int j = 0; j < QLDS; ++j) *(bf16x8*)(qpe + 1024 * j) = qtmp[j];
  __builtin_amdgcn_s_barrier();
  compiler_fence();
  trow = tile_rows_lanes(p, wi.b, wi.t0, wi.t1, blk_tab, first_blk_of(p, wi.t0), l);
  for (int i = tid; i < ntiles * TILE; i += NT) {
    const int k = i >> 5, r = i & 31;
    const int last = wi.t1 - 1 - (wi.t0 + k * TILE);
    int64_t row = (int64_t)__shfl(trow, k, 64) + min(r, last);
    row = (row >= 0 && row < p.rows) ? row : 0;
    scl_all[i] = (float)p.scales[row];
  }
  wait_vm_lgkm0<0>();
  __builtin_amdgcn_s_barrier();   // every row scale is in LDS before any is read
  compiler_fence();
  widen_own_all<NW>(stage, buf0, w, l, rope_real);
  wait_vm_lgkm0<0>();
  __builtin_amdgcn_s_barrier();
  compiler_fence();

  for (int attempt = 0; attempt < 2; ++attempt) {
    if (attempt > 0) {
      load_raw(stage, 0).all();
      load_raw(buf2, 1).all();
      wait_vm_lgkm0<0>();
      widen_own_all<NW>(stage, buf0, w, l, rope_real);
      wait_vm_lgkm0<0>();
      __builtin_amdgcn_s_barrier();
      compiler_fence();
    }
    f32x16 s0, s1;    // scores of even / odd tiles
    bf16x8 pb[2];     // PV B operand (weights of the tile whose PV is next)
    bf16x8 pring[3];  // PV A operands in flight
    // a step's extra work: wait for its raw tile, widen it, load the one after
    auto extra = [&](int t, const char* raw, char* dst, int j) {
      if (j + 1 < ntiles) {
        if (t == WIDEN_SLOT0 - 1) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        widen_own_at_<NW>(t, raw, dst, w, l, rope_real, std::make_integer_sequence<int, P>{});
      }
      if (t == LOAD_SLOT && j + 2 < ntiles) {
        int lv = l;   // lane offsets recomputed here, for the same reason
        asm volatile("" : "+v"(lv));
        int vo[P];
        fp8_piece_offsets<NW>(p, w, lv, vo);
        fp8_load<NW>(p, stage, dummy, __builtin_amdgcn_readlane(trow, min(j + 2, ntiles - 1)),
                     nvalid(j + 2), w, vo)
            .all();
      }
    };
    auto step_end = [&]() {   // tile j+1 widened everywhere, tile j-1 read everywhere
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      compiler_fence();
    };
    pipe_step<true, false, true, true>(buf0, nullptr, wi.t0, wi.t1, qreg, qpe, la, h, st, s0, s1,
                                       pb, pring, [&](int t, int) { extra(t, buf2, buf1, 0); },
                                       scl_all);
    // (with few waves a lane's pieces outnumber the S^T-only step's slots:
    // the rest of its extra work follows the step)
    static_for<(LOAD_SLOT + 1 > D_QK / 16) ? LOAD_SLOT + 1 - D_QK / 16 : 0>(
        [&](auto tc) { extra(D_QK / 16 + decltype(tc)::value, buf2, buf1, 0); });
    step_end();
    auto step = [&](char* K, char* V, char* W, int j, f32x16& sn, f32x16& sp) {
      if (j < ntiles) {
        pipe_step<true, true, false, true>(K, V, wi.t0 + j * TILE, wi.t1, qreg, qpe, la, h, st, sn,
                                           sp, pb, pring, [&](int t, int) { extra(t, stage, W, j); },
                                           scl_all + TILE * j, scl_all + TILE * (j - 1));
        step_end();
      }
    };
    for (int j = 1; j < ntiles; j += 6) {
      step(buf1, buf0, buf2, j, s1, s0);
      step(buf2, buf1, buf0, j + 1, s0, s1);
      step(buf0, buf2, buf1, j + 2, s1, s0);
      step(buf1, buf0, buf2, j + 3, s0, s1);
      step(buf2, buf1, buf0, j + 4, s1, s0);
      step(buf0, buf2, buf1, j + 5, s0, s1);
    }
    {   // softmax and PV of the last tile
      const int last = ntiles - 1;
      f32x16 sl = (last & 1) ? s1 : s0;
      pipe_step<false, true, false, true>(nullptr, bufs + (last % 3) * TILE_BYTES, 0, wi.t1, qreg,
                                          qpe, la, h, st, sl, sl, pb, pring, [](int, int) {},
                                          nullptr, scl_all + TILE * last);
    }
    // overflow flags (own LDS words); after the barrier every wave is also
    // past its last tile read, and no load is in flight
    const bool ovf = split_overflowed(st);
    wait_vm_lgkm0<0>();
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
      load_raw(stage, k).all();
      wait_vm_lgkm0<0>();
      widen_own_all<NW>(stage, buf0, w, l, rope_real);
      wait_vm_lgkm0<0>();
      __builtin_amdgcn_s_barrier();
      compiler_fence();
      float sv[16];
      bf16x8 qp[QLDS];
#pragma unroll
      for (int j = 0; j < QLDS; ++j) qp[j] = *(const bf16x8*)(qpe + 1024 * j);
      mtrue = fmaxf(mtrue, tile_scores<CACHE_FP8, true>(buf0, scl_all + TILE * k, wi.t0 + k * TILE,
                                                        wi.t1, qreg, qp, la, h, sv, [](int) {}));
    }
    reset_state(st, mtrue);
    wait_vm_lgkm0<0>();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
  }
  write_partial(wi, st, h, l, (w < 2 ? buf0 : buf1) + (w & 1) * PART_SCR_BYTES);
}


}  // namespace mla
