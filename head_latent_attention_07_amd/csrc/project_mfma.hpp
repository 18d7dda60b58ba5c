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

#include <type_traits>

#include "append.hpp"
#include "common.hpp"
#include "split_plan.hpp"

namespace mla {

__device__ __forceinline__ bf16x8 tr_read_8(const char* p_lo, const char* p_hi) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p_lo);
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p_hi);
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

// Buffer resource for raw buffer loads (bounds-checked: reads past `bytes`
// return zeros).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t proj_rsrc(const void* base, int64_t bytes) {
  const int32_t n = (int32_t)min(max(bytes, (int64_t)0), (int64_t)0x7FFFFFF0);
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, n, 0x00020000);
}

// XOR swizzle of 16-byte chunks within a 1 KB weight row in LDS (same scheme
// as the attention tiles): ds_read_b64_tr_b16 over 4 consecutive rows hits 4
// distinct 32-byte bank groups.
__device__ __forceinline__ int wrow_swizzle(int row) { return 2 * (row & 3) + ((row >> 2) & 1); }

// ----------------------------------------------------------------------------
// absorb: four workgroups (4 waves each) per head, each owning 128 of the 512
// output columns; its slice of W_UK[h] (128 rows x 256 B = 32 KB) is brought
// into LDS by direct-to-LDS loads, then every chunk of 32 sequences is
// multiplied against it (wave w: columns 32w..32w+31 of the slice).
// ----------------------------------------------------------------------------
struct AbsorbParams {
  const bf16* q_nope;  // [B, H, 128]
  const bf16* q_pe;    // [B, H, 64]
  const bf16* w_uk;    // [H, 128, 512]
  bf16* q;             // [B, H, 576] in the operand layout of qop_index
  int B, H, nbc;       // nbc: unused (kept for the launch code)
  float c;             // softmax_scale * log2(e)
  BalanceParams plan;  // a length-aware split plan to make in the same launch (or items == nullptr)
};

// Workgroups of the absorb launch before the absorb (and append) ones that
// make the length-aware split plan: 8 (one working), so that the others keep
// their XCD placement.
__host__ __device__ constexpr int plan_blocks(bool planned) { return planned ? 8 : 0; }

constexpr int AB_APITCH = D_N * 2 + 16;    // 272 B: 8 rows' 16-byte chunks hit distinct banks
constexpr int AB_COLS = 128;               // output columns per workgroup
constexpr int AB_ROW = AB_COLS * 2;        // 256 B per W row slice in LDS
constexpr int AB_OPITCH = 32 * 2 + 16;     // 80 B: output staging row (32 bf16 + pad)

__device__ __forceinline__ void absorb_workgroup(const AbsorbParams& p, int x) {
  __shared__ __attribute__((aligned(1024))) char w_lds[D_N * AB_ROW];   // 32 KB
  // two chunks of 32 sequences; after a pass's products every wave stages
  // its outputs (32 sequences x 32 columns) in its own 2.5 KB of this space,
  // so the workgroup takes 49 KB of LDS and three fit on a CU (with the
  // cache-append workgroups of the same launch, 4 H + B / 4 workgroups at
  // H = 128 all run at once)
  __shared__ __attribute__((aligned(16))) char a_lds[2][32 * AB_APITCH];
  static_assert(4 * 32 * AB_OPITCH <= 2 * 32 * AB_APITCH, "output staging fits");
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = l >> 5, l32 = l & 31, jj = l & 15, g16 = l >> 4;
  // (head, quarter) from the flat id: workgroups are dispatched round-robin
  // over the 8 XCDs; the 16 workgroups of 4 consecutive heads (which write
  // interleaved 16-byte pieces of the same lines of the query layout) share
  // one XCD, so its L2 merges them into whole lines
  int head, quarter;
  {
    const int xcd = x & 7, i = x >> 3;
    const int cluster = (i >> 4) * 8 + xcd;
    head = cluster * 4 + ((i & 15) >> 2);
    quarter = i & 3;
  }
  if (head >= p.H) return;

  // W_UK[h][:, 128 q .. 128 q + 127]: wave w loads rows 32w..32w+31, four
  // rows (4 x 256 B) per wave-wide load; lane l fills LDS slot l & 15 of row
  // 4k + (l >> 4), which holds the chunk the swizzle places there
  {
    const __amdgpu_buffer_rsrc_t rs = proj_rsrc(p.w_uk + (int64_t)head * D_N * D_C, D_N * D_C * 2);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int row0 = w * 32 + 4 * k, row = row0 + (l >> 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(w_lds + row0 * AB_ROW), 16,
          row * (D_C * 2) + quarter * AB_ROW + 16 * ((l & 15) ^ wrow_swizzle(row)), 0, 0, 0);
    }
  }
  // tr-read bases for this lane's B operand
  const int r1 = 8 * h + (jj >> 2);                    // + 16 ks, and + 4 for the upper half
  const int chunk = 4 * w + (2 * (g16 & 1) + ((jj & 3) >> 1));
  const int off = 8 * (jj & 1);
  // passes of 64 sequences: both chunks' q_nope rows are loaded (one wait
  // for them and the weight slice), then multiplied chunk by chunk
  for (int b0 = 0; b0 < p.B; b0 += 64) {
    {
      u32x4 v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {   // 64 rows x 16 pieces of 16 bytes, 4 per thread
        const int i = tid + 256 * k, r = i >> 4, c = i & 15;
        v[k] = u32x4{0, 0, 0, 0};
        if (b0 + r < p.B) v[k] = *(const u32x4*)(p.q_nope + ((int64_t)(b0 + r) * p.H + head) * D_N + 8 * c);
      }
      if (quarter == 0) {
        // q_pe: 8 consecutive values per thread (64 rows x 64, two per thread)
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int r = (tid >> 3) + 32 * k, c = 8 * (tid & 7);
          if (b0 + r < p.B) {
            const int64_t bh = (int64_t)(b0 + r) * p.H + head;
            const bf16x8 x = *(const bf16x8*)(p.q_pe + bh * D_R + c);
            bf16x8 o;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = (bf16)((float)x[e] * p.c);
            *(bf16x8*)(p.q + qop_index(b0 + r, head, D_C + c, p.H)) = o;
          }
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int i = tid + 256 * k, r = i >> 4, c = i & 15;
        *(u32x4*)(a_lds[r >> 5] + (r & 31) * AB_APITCH + 16 * c) = v[k];
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // W_UK slice landed (first pass)
    __syncthreads();
    f32x16 acc[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      acc[cb] = f32x16{};
      if (b0 + 32 * cb >= p.B) continue;   // (uniform)
#pragma unroll
      for (int ks = 0; ks < D_N / 16; ++ks) {
        const bf16x8 a = *(const bf16x8*)(a_lds[cb] + l32 * AB_APITCH + 2 * (16 * ks + 8 * h));
        const int ra = 16 * ks + r1, rb = ra + 4;
        const bf16x8 bop = tr_read_8(w_lds + ra * AB_ROW + 16 * (chunk ^ wrow_swizzle(ra)) + off,
                                     w_lds + rb * AB_ROW + 16 * (chunk ^ wrow_swizzle(rb)) + off);
        acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bop, acc[cb], 0, 0, 0);
      }
    }
    __syncthreads();   // every wave is done reading a_lds
    // lane holds column 32w + l32 of the slice, rows b = 8(r/4) + 4h + r%4:
    // transpose through LDS so each lane stores 8 consecutive columns of one
    // sequence (one 16-byte piece of the query layout)
    char* const ol = &a_lds[0][0] + w * (32 * AB_OPITCH);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int bc0 = b0 + 32 * cb;
      if (bc0 >= p.B) break;   // (uniform)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        *(bf16*)(ol + (8 * (r >> 2) + 4 * h + (r & 3)) * AB_OPITCH + 2 * l32) = (bf16)(acc[cb][r] * p.c);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int id = l + 64 * i, r = id >> 2, c8 = id & 3;
        const u32x4 v = *(const u32x4*)(ol + r * AB_OPITCH + 16 * c8);
        if (bc0 + r < p.B)
          *(u32x4*)(p.q + qop_index(bc0 + r, head, quarter * AB_COLS + 32 * w + 8 * c8, p.H)) = v;
      }
    }
    __syncthreads();   // a_lds is rewritten by the next pass
  }
}

__global__ __launch_bounds__(256) void mla_absorb_kernel(AbsorbParams p) {
  const int np = plan_blocks(p.plan.items != nullptr);
  if ((int)blockIdx.x < np) {
    if (blockIdx.x == 0) balance_plan(p.plan);
    return;
  }
  absorb_workgroup(p, blockIdx.x - np);
}

// absorb and cache append in one launch (the absorb neither reads nor
// writes the cache, so the two are independent). The append workgroups come
// first (one sequence per wave, their count rounded up to a multiple of 8 so
// the absorb workgroups keep their XCD placement) and run beside the absorb
// from the start: at 128 heads the launch's 512 + B/4 workgroups are all
// resident at once (three fit per CU).
__host__ __device__ constexpr int append_blocks(int B) { return ((B + 3) / 4 + 7) / 8 * 8; }

__global__ __launch_bounds__(256) void mla_absorb_append_kernel(AbsorbParams p, AppendParams a) {
  const int np = plan_blocks(p.plan.items != nullptr);
  if ((int)blockIdx.x < np) {
    if (blockIdx.x == 0) balance_plan(p.plan);
    return;
  }
  const int x = (int)blockIdx.x - np;
  const int na = append_blocks(p.B);
  if (x < na) {
    const int b = x * 4 + (int)(threadIdx.x >> 6);
    if (b < p.B) append_row(a, b, threadIdx.x & 63);
    return;
  }
  absorb_workgroup(p, x - na);
}

// ----------------------------------------------------------------------------
// merge + W_UV: one workgroup of 8 waves per (head, chunk of 32 sequences);
// the chunks of one head run on one XCD, so W_UV[h] comes from HBM once and
// from that XCD's L2 after.
//
// The kernel streams 256 KB per workgroup (128 KB of fp16 partials at S = 4,
// 128 KB of W_UV) and does a little arithmetic on it. A wave stalls while
// its loads queue up, so the work is spread over two waves per SIMD: while
// one waits on memory the other merges. At entry each thread issues the lse
// and scale of its share of the first 64 splits, the partials of the first
// group of 4 splits, its part of the W_UV DMA and the partials of the second
// group. The merge weights 2^(lse_s - L) * scale_s / sum_s' 2^(lse_s' - L)
// go into an LDS table [32 sequences][64 splits]; the partials are merged
// group by group, each group loaded two groups ahead. More than 64 splits
// are merged in chunks of 64 (the table refilled per chunk). Each half of
// the product is split over the two wave sets by its contraction index and
// the two accumulators are summed through LDS at the end.
// ----------------------------------------------------------------------------
struct CombineParams {
  const _Float16* part_o;   // [B, sp, H, 512] fp16, relative to part_scale
  const float* part_scale;  // [B, sp, H]
  const float* part_lse;    // [B, sp, H] log2 domain
  const bf16* w_uv;       // [H, 512, 128]
  bf16* out;              // [B, H, 128]
  float* lse;             // [B, H] natural log, or nullptr
  int B, H, S, nbc;       // S: partials merged per sequence; nbc: chunks of 32 sequences
  int sp, ss;             // split slots per sequence in the arrays; partial s is slot s * ss
                          // (mla_combine_kernel: sp == S, ss == 1)
  const int32_t* nsplit;  // mla_combine_kernel: [B] partials of each sequence (slots
                          // 0 .. nsplit[b] - 1; a length-aware plan), or nullptr: all S
};

constexpr int CB_THREADS = 512;       // 8 waves
constexpr int CB_APITCH = D_C + 16;   // 528 B: half a merged row (256 dims) + pad
constexpr int CB_CHUNK = 64;          // splits per weight table
constexpr int CB_G = 4;               // splits per merge group
constexpr int CB_R = 2;               // sequences per thread in the merge
constexpr int CB_WJ = 4;              // table entries per thread (64 splits / 16)

// Position in the merge order (half of the 512 dims, chunk of 64 splits,
// group of 4 splits, in that nesting); s0 is the group's first split.
struct CbUnit {
  int half, c0, s0;
  __device__ bool valid() const { return half < 2; }
  __device__ void next(int S) {
    s0 += CB_G;
    if (s0 < min(c0 + CB_CHUNK, S)) return;
    c0 += CB_CHUNK;
    s0 = c0;
    if (c0 < S) return;
    ++half;
    c0 = s0 = 0;
  }
};

// Workgroup barrier for LDS hand-offs only: this workgroup's LDS writes are
// complete and visible, outstanding global loads stay in flight (the
// __syncthreads fences would also wait for every global load).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The partials of one group for this thread: sequences rq + 16i, dims
// half*256 + 8*d8 .. +7, splits s0 .. s0+3. A sequence or split past the end
// reads the last one again (unused, or weighted 0): the loads stay
// unconditional, so the compiler's wait counts stay exact.
__device__ __forceinline__ void cb_load(const CombineParams& p, const _Float16* const (&po)[CB_R],
                                        const int (&nrow)[CB_R], const CbUnit& u, int d8,
                                        f16x8 (&v)[CB_R][CB_G]) {
#pragma unroll
  for (int k = 0; k < CB_G; ++k) {
#pragma unroll
    for (int i = 0; i < CB_R; ++i) {
      const int64_t so = (int64_t)min(u.s0 + k, nrow[i] - 1) * p.H * D_C + u.half * 256 + 8 * d8;
      v[i][k] = *(const f16x8*)(po[i] + so);
    }
  }
}

__global__ __launch_bounds__(CB_THREADS) void mla_combine_kernel(CombineParams p) {
  __shared__ __attribute__((aligned(1024))) char w_lds[D_C * D_V * 2];   // 128 KB
  __shared__ __attribute__((aligned(16))) char a_lds[32 * CB_APITCH];    // 32 seq x 256 dims
  __shared__ __attribute__((aligned(16))) float wts[32 * CB_CHUNK];      // merge weights
  __shared__ float red[2][16][32];                                       // max, sum partials
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = l >> 5, l32 = l & 31, jj = l & 15, g16 = l >> 4;
  // (head, chunk of 32 sequences); the chunks of one head share an XCD (L2)
  int head, bc;
  {
    const int x = blockIdx.x;
    const int q_lo = x & 7, rest = x >> 3;
    bc = __builtin_amdgcn_readfirstlane(rest % p.nbc);
    head = __builtin_amdgcn_readfirstlane((rest / p.nbc) * 8 + q_lo);
    if (head >= p.H) return;
  }
  const int S = p.S, b0 = bc * 32, nrows = min(32, p.B - b0);
  // 1. Loads. Weight-table role: sequence wr, splits wp + 16j of a chunk.
  const int wr = tid & 31, wp = tid >> 5;
  const int wb = b0 + wr;
  const bool wrow = wb < p.B;
  const int64_t wrow0 = (int64_t)min(wb, p.B - 1) * S * p.H + head;
  // partials of this role's sequence: the first wS slots (all S without a
  // length-aware plan); later slots are never read (a load past them reads
  // the last one again, with weight 0)
  const int wS = p.nsplit ? min(max(p.nsplit[min(wb, p.B - 1)], 1), S) : S;
  float lv[CB_WJ], sv[CB_WJ];
#pragma unroll
  for (int j = 0; j < CB_WJ; ++j) {
    const int64_t ix = wrow0 + (int64_t)min(wp + 16 * j, wS - 1) * p.H;
    lv[j] = p.part_lse[ix];   // masked below, after the issue
    sv[j] = p.part_scale[ix];
  }
  // merge role: sequences rq + 16i, dims 8*d8 .. +7 of each half
  const int rq = tid >> 5, d8 = tid & 31;
  const _Float16* po[CB_R];
  int nrow[CB_R];
#pragma unroll
  for (int i = 0; i < CB_R; ++i) {
    const int bi = min(b0 + rq + 16 * i, p.B - 1);
    po[i] = p.part_o + ((int64_t)bi * S * p.H + head) * D_C;
    nrow[i] = p.nsplit ? min(max(p.nsplit[bi], 1), S) : S;
  }
  auto load_w = [&]() {
    const __amdgpu_buffer_rsrc_t rs = proj_rsrc(p.w_uv + (int64_t)head * D_C * D_V, D_C * D_V * 2);
#pragma unroll
    for (int k = 0; k < 16; ++k) {   // 128 lines of 1 KB (4 rows each), 16 per wave
      const int line = w * 16 + k;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(w_lds + line * 1024), 16, 16 * l,
          line * 1024, 0, 0);
    }
    asm volatile("" ::: "memory");   // later loads stay behind the DMA
  };
  // The first group, W_UV, the second group, in that order; every later
  // group is loaded two groups ahead of its merge. With S <= 4 there are
  // just two groups (one per half) and no loop, so that each step waits
  // only for what it reads.
  const bool one_group = S <= CB_G;
  f16x8 va[CB_R][CB_G], vb[CB_R][CB_G];
  CbUnit ua{0, 0, 0};
  CbUnit ub = ua;
  ub.next(S);
  CbUnit un = ub;   // the next unit to load
  un.next(S);
  cb_load(p, po, nrow, ua, d8, va);
  load_w();
  cb_load(p, po, nrow, ub, d8, vb);
#pragma unroll
  for (int j = 0; j < CB_WJ; ++j) {   // (kept here: the issue above does not wait for these)
    asm volatile("" : "+v"(lv[j]));
    lv[j] = (wrow && wp + 16 * j < wS) ? lv[j] : -INFINITY;
  }
  // 2. L = max over all splits, wsum = sum of 2^(lse - L), per sequence;
  //    the weight table of the first chunk.
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < CB_WJ; ++j) mx = fmaxf(mx, lv[j]);
  if (wrow)
    for (int s = CB_CHUNK + wp; s < wS; s += 16) mx = fmaxf(mx, p.part_lse[wrow0 + (int64_t)s * p.H]);
  red[0][wp][wr] = mx;
  lds_barrier();
  float L = -INFINITY;
#pragma unroll
  for (int k = 0; k < 16; ++k) L = fmaxf(L, red[0][k][wr]);
  float sum = 0.f;
  if (L > -INFINITY) {
#pragma unroll
    for (int j = 0; j < CB_WJ; ++j) sum += fast_exp2(lv[j] - L);
    if (wrow)
      for (int s = CB_CHUNK + wp; s < wS; s += 16)
        sum += fast_exp2(p.part_lse[wrow0 + (int64_t)s * p.H] - L);
  }
  red[1][wp][wr] = sum;
  lds_barrier();
  float wsum = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) wsum += red[1][k][wr];
  const float inv = (L > -INFINITY && wsum > 0.f) ? 1.0f / wsum : 0.f;
  if (wp == 0 && wrow && p.lse)
    p.lse[(int64_t)wb * p.H + head] = (L > -INFINITY) ? (L + __builtin_log2f(wsum)) * LN2 : -INFINITY;
#pragma unroll
  for (int j = 0; j < CB_WJ; ++j)
    wts[wr * CB_CHUNK + wp + 16 * j] = (inv > 0.f) ? fast_exp2(lv[j] - L) * sv[j] * inv : 0.f;
  lds_barrier();

  // 3. Merge group by group; after the last group of a half, that half of
  //    the merged rows times the matching 256 rows of W_UV[h] (waves w and
  //    w + 4: output columns 32(w mod 4) .. +31, contraction steps
  //    8(w div 4) .. +7 of the half's 16).
  int table_c0 = 0;   // the chunk whose weights are in wts
  int issued = 1;     // groups loaded after the W_UV DMA
  f32x8 m[CB_R];
#pragma unroll
  for (int i = 0; i < CB_R; ++i) m[i] = f32x8{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int colb = 32 * (w & 3) + 16 * (g16 & 1) + 4 * (jj & 3);   // B-operand column base
  const int ks0 = 8 * (w >> 2);
  f32x16 acc = f32x16{};
  auto merge = [&](const CbUnit& u, const f16x8 (&v)[CB_R][CB_G], auto looped) {
    if (looped && u.c0 != table_c0) {   // weights of another chunk of splits (S > 64)
      lds_barrier();                    // the table in use is no longer read
#pragma unroll
      for (int j = 0; j < CB_WJ; ++j) {
        const int s = u.c0 + wp + 16 * j;
        const int64_t ix = wrow0 + (int64_t)min(s, wS - 1) * p.H;
        const float x = (wrow && s < wS) ? p.part_lse[ix] : -INFINITY;
        wts[wr * CB_CHUNK + wp + 16 * j] = (inv > 0.f) ? fast_exp2(x - L) * p.part_scale[ix] * inv : 0.f;
      }
      lds_barrier();
      table_c0 = u.c0;
    }
    const int g = u.s0 - u.c0;
#pragma unroll
    for (int i = 0; i < CB_R; ++i) {
      if (rq + 16 * i < nrows) {
        const f32x4 w4 = *(const f32x4*)(wts + (rq + 16 * i) * CB_CHUNK + g);
#pragma unroll
        for (int k = 0; k < CB_G; ++k)
#pragma unroll
          for (int e = 0; e < 8; ++e) m[i][e] += w4[k] * (float)v[i][k][e];
      }
    }
    if (looped) {
      CbUnit nx = u;
      nx.next(S);
      if (nx.half == u.half) return;
    }
#pragma unroll
    for (int i = 0; i < CB_R; ++i) {
      bf16x8 pk;
#pragma unroll
      for (int k = 0; k < 8; ++k) pk[k] = (bf16)m[i][k];
      *(bf16x8*)(a_lds + (rq + 16 * i) * CB_APITCH + 16 * d8) = pk;
      m[i] = f32x8{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    }
    // W_UV has landed once at most the groups loaded after it are pending:
    // they are the youngest loads, at most two groups of 8 (before the
    // half-0 product without the loop: the 8 of the half-1 group)
    if (issued >= 2)
      asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else if (u.half == 0)
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
#pragma unroll
    for (int ks = ks0; ks < ks0 + 8; ++ks) {
      const bf16x8 a = *(const bf16x8*)(a_lds + l32 * CB_APITCH + 2 * (16 * ks + 8 * h));
      const int ra = u.half * 256 + 16 * ks + 8 * h + (jj >> 2);
      const bf16x8 bop = tr_read_8(w_lds + ra * 256 + 2 * colb, w_lds + (ra + 4) * 256 + 2 * colb);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bop, acc, 0, 0, 0);
    }
    lds_barrier();   // a_lds is rewritten next
  };
  if (one_group) {
    merge(ua, va, std::false_type{});
    merge(ub, vb, std::false_type{});
  } else {
    // units alternate between the buffers va and vb (named at compile
    // time); after a unit is merged its buffer takes the unit two on
    while (ua.valid()) {
      merge(ua, va, std::true_type{});
      ua = un;
      if (un.valid()) {
        cb_load(p, po, nrow, un, d8, va);
        un.next(S);
        ++issued;
      }
      if (!ub.valid()) break;
      merge(ub, vb, std::true_type{});
      ub = un;
      if (un.valid()) {
        cb_load(p, po, nrow, un, d8, vb);
        un.next(S);
        ++issued;
      }
    }
  }
  // 4. Sum the two contraction halves (waves w + 4 hand theirs to wave w
  //    through the now unused a_lds) and store.
  f32x16* const xch = (f32x16*)a_lds + ((w & 3) * 64 + l);
  if (w >= 4) *xch = acc;
  lds_barrier();
  if (w < 4) {
    acc += *xch;
    const int n = 32 * w + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int bb = b0 + 8 * (r >> 2) + 4 * h + (r & 3);
      if (bb < p.B) p.out[((int64_t)bb * p.H + head) * D_V + n] = (bf16)acc[r];
    }
  }
}

// ----------------------------------------------------------------------------
// First merge level for rows with many splits: the splits of each
// (sequence, head) row are cut into NG groups of G consecutive splits, and
// one wave merges one group into one partial of the same form (fp16 values
// relative to the row maximum, the fp32 factor, the log2-domain lse), which
// it writes over the group's first split. mla_combine_s4_kernel then merges
// the NG group partials, G slots apart, and applies W_UV. Merging in groups
// is exact up to rounding: the lse of a union of splits is the lse of the
// groups' lse values, and each group's output is its splits' outputs
// weighted by 2^(lse_s - lse_group). It spreads the partial bytes over
// B * H * NG waves, where mla_combine_kernel has one workgroup per
// (head, 32 sequences) walk its splits group after group.
//
// Lane l holds dims 8l .. 8l+7 of the row. The group is read MS_CH splits
// at a time with a running maximum of the lse; past the group's last split
// the loads read that split again with weight 0, so every load is
// unconditional and issued before the weights are known. An empty split
// (lse -inf, zeros, written by the attention kernels) weighs 0; a group of
// empty splits gives zeros, factor 0 and lse -inf.
// ----------------------------------------------------------------------------
struct MergeSplitsParams {
  _Float16* part_o;    // [B, S, H, 512] fp16, relative to part_scale
  float* part_scale;   // [B, S, H]
  float* part_lse;     // [B, S, H] log2 domain
  int B, H, S, G, NG;  // splits, splits per group, groups (NG = ceil(S / G))
};

constexpr int MS_WAVES = 4;   // waves per workgroup (consecutive heads)

template <int MS_CH>
__global__ __launch_bounds__(64 * MS_WAVES) __attribute__((amdgpu_waves_per_eu(1, 4)))
void mla_merge_splits_kernel(MergeSplitsParams p) {
  const int l = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane((int)blockIdx.x * MS_WAVES + (int)(threadIdx.x >> 6));
  const int head = wid % p.H, rest = wid / p.H;   // (b, group, head), head fastest
  const int g = rest % p.NG, b = rest / p.NG;
  if (b >= p.B) return;
  const int s0 = g * p.G, n = min(p.G, p.S - s0);
  const int64_t row0 = ((int64_t)b * p.S + s0) * p.H + head;   // the group's first split
  float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float L = -INFINITY, wsum = 0.f;
  for (int c = 0; c < n; c += MS_CH) {
    f16x8 v[MS_CH];
#pragma unroll
    for (int k = 0; k < MS_CH; ++k)
      v[k] = *(const f16x8*)(p.part_o + (row0 + (int64_t)min(c + k, n - 1) * p.H) * D_C + 8 * l);
    // lane l holds the lse and factor of split c + (l mod MS_CH): one load
    // per lane instead of a chain of uniform loads
    const int kl = c + (l & (MS_CH - 1));
    const int64_t ixl = row0 + (int64_t)min(kl, n - 1) * p.H;
    float lvl = p.part_lse[ixl];
    const float svl = p.part_scale[ixl];
    lvl = (kl < n) ? lvl : -INFINITY;
    float cm = fmaxf(L, lvl);
#pragma unroll
    for (int o = MS_CH / 2; o > 0; o >>= 1) cm = fmaxf(cm, __shfl_xor(cm, o, 64));
    // a new maximum rescales what is merged so far (0 when nothing is)
    const float alpha = (L > -INFINITY) ? fast_exp2(L - cm) : 0.f;
    L = cm;
    float el = (lvl > -INFINITY) ? fast_exp2(lvl - L) : 0.f;
    const float wl = el * svl;
#pragma unroll
    for (int o = MS_CH / 2; o > 0; o >>= 1) el += __shfl_xor(el, o, 64);
    wsum = wsum * alpha + el;
#pragma unroll
    for (int e = 0; e < 8; ++e) m[e] *= alpha;
#pragma unroll
    for (int k = 0; k < MS_CH; ++k) {
      const float wk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), k));
#pragma unroll
      for (int e = 0; e < 8; ++e) m[e] += wk * (float)v[k][e];
    }
  }
  float mx = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(m[e]));
  mx = wave_max(mx);
  const float f = (mx > 0.f) ? 1.0f / mx : 0.f;
  f16x8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (_Float16)(m[e] * f);
  // every read of the group's rows is done: each value stored depends on all of them
  *(f16x8*)(p.part_o + row0 * D_C + 8 * l) = o;
  if (l == 0) {
    p.part_lse[row0] = (wsum > 0.f) ? L + __builtin_log2f(wsum) : -INFINITY;
    p.part_scale[row0] = (wsum > 0.f) ? mx / wsum : 0.f;
  }
}

// ----------------------------------------------------------------------------
// merge + W_UV for S <= 4 splits (the many-sequence case, or the groups of
// mla_merge_splits_kernel, split s at slot s * ss), same grid and
// work split as above but without the weight table and the A staging: wave
// w owns dims 32w .. 32w+31 of each half of the latent, lane l the sequence
// l mod 32. A lane computes its sequence's weights from the (at most 4)
// split lse values itself, merges its 16 dims of each half straight into
// the MFMA A operand, and multiplies them by the 64 rows of W_UV[h] it
// loaded into LDS itself, for the workgroup's 32 NCB output columns. The 8
// waves' partial products are summed through LDS (the W_UV buffer, free by
// then). NCB = 4: one workgroup per (head, 32 sequences) takes all 128
// columns; NCB = 2: two workgroups take 64 columns each (half of W_UV[h] in
// LDS each, twice the workgroups where one per (head, 32 sequences) would
// leave CUs idle; both merge the same partials, the second from L2).
// ----------------------------------------------------------------------------
template <int NCB, int G>
__global__ __launch_bounds__(CB_THREADS) void mla_combine_s4_kernel(CombineParams p) {
  constexpr int NCS = 4 / NCB;         // workgroups per (head, 32 sequences)
  constexpr int ROWB = 64 * NCB;       // bytes of this workgroup's slice of a W_UV row
  constexpr int RPI = 1024 / ROWB;     // slice rows per 1 KB direct load
  constexpr int NI = 64 / RPI;         // direct loads per wave (its 64 rows)
  __shared__ __attribute__((aligned(1024))) char w_lds[D_C * ROWB];   // 128 or 64 KB
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = l >> 5, l32 = l & 31, jj = l & 15, g16 = l >> 4;
  int head, bc, cs;
  {
    const int x = blockIdx.x;
    const int q_lo = x & 7, rest = x >> 3;
    bc = __builtin_amdgcn_readfirstlane(rest % p.nbc);
    const int r2 = rest / p.nbc;
    cs = __builtin_amdgcn_readfirstlane(r2 % NCS);
    head = __builtin_amdgcn_readfirstlane((r2 / NCS) * 8 + q_lo);
    if (head >= p.H) return;
  }
  const int b = bc * 32 + l32;
  const bool brow = b < p.B;
  // partials of this lane's sequence: p.S, or its own count (a length-aware
  // plan; later slots are never read: a load past them reads the last one
  // again, weighted 0)
  const int S = p.nsplit ? min(max(p.nsplit[min(b, p.B - 1)], 1), p.S) : p.S;
  const int64_t row0 = (int64_t)min(b, p.B - 1) * p.sp * p.H + head;   // (b, split 0, head)
  const int64_t sstep = (int64_t)p.ss * p.H;                            // split s: + s * sstep
  // loads: lse and scale, half-0 partials, this wave's W_UV rows, half-1
  // partials (v[half][step][split]: dims 256 half + 32 w + 16 step + 8 h)
  float lv[G], sv[G];
#pragma unroll
  for (int s = 0; s < G; ++s) {
    const int64_t ix = row0 + min(s, S - 1) * sstep;
    lv[s] = p.part_lse[ix];
    sv[s] = p.part_scale[ix];
  }
  f16x8 v[2][2][G];
  auto load_half = [&](int hf) {
#pragma unroll
    for (int s = 0; s < G; ++s)
#pragma unroll
      for (int t = 0; t < 2; ++t)
        v[hf][t][s] = *(const f16x8*)(p.part_o + (row0 + min(s, S - 1) * sstep) * D_C +
                                      256 * hf + 32 * w + 16 * t + 8 * h);
  };
  load_half(0);
  {
    // rows 256 hf + 32 w .. +31 of W_UV[h], columns 32 NCB cs .. +32 NCB - 1
    // (ROWB bytes of each 256-byte row), to the same rows of the LDS copy
    // (rows ROWB apart), RPI rows per 1 KB load
    const __amdgpu_buffer_rsrc_t rs = proj_rsrc(p.w_uv + (int64_t)head * D_C * D_V, D_C * D_V * 2);
    const int vo = 256 * (l / (ROWB / 16)) + 16 * (l % (ROWB / 16));
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int r0 = 256 * (k / (NI / 2)) + 32 * w + RPI * (k % (NI / 2));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(w_lds + r0 * ROWB), 16, vo,
          r0 * 256 + cs * ROWB, 0, 0);
    }
    asm volatile("" ::: "memory");   // later loads stay behind the DMA
  }
  load_half(1);
  // weights of this lane's sequence
  float L = -INFINITY;
#pragma unroll
  for (int s = 0; s < G; ++s) {
    lv[s] = (brow && s < S) ? lv[s] : -INFINITY;
    L = fmaxf(L, lv[s]);
  }
  float e[G], wsum = 0.f;
#pragma unroll
  for (int s = 0; s < G; ++s) {
    e[s] = (L > -INFINITY) ? fast_exp2(lv[s] - L) : 0.f;
    wsum += e[s];
  }
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  float wt[G];
#pragma unroll
  for (int s = 0; s < G; ++s) wt[s] = e[s] * sv[s] * inv;
  if (cs == 0 && w == 0 && h == 0 && brow && p.lse)
    p.lse[(int64_t)b * p.H + head] = (L > -INFINITY) ? (L + __builtin_log2f(wsum)) * LN2 : -INFINITY;

  f32x16 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x16{};
  const int colb0 = 16 * (g16 & 1) + 4 * (jj & 3);   // + 32 cb: B-operand column base
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    bf16x8 a[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < G; ++s)
#pragma unroll
        for (int k = 0; k < 8; ++k) m[k] += wt[s] * (float)v[hf][t][s][k];
#pragma unroll
      for (int k = 0; k < 8; ++k) a[t][k] = (bf16)m[k];
    }
    // this wave's W_UV rows have landed once only the 8 half-1 loads, which
    // follow them, may be pending
    if (hf == 0) {
      __builtin_amdgcn_sched_barrier(0);   // the half-0 merge stays ahead of the wait
      if constexpr (G == 4)
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int ra = 256 * hf + 32 * w + 16 * t + 8 * h + (jj >> 2);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int colb = 32 * cb + colb0;
        const bf16x8 bop = tr_read_8(w_lds + ra * ROWB + 2 * colb, w_lds + (ra + 4) * ROWB + 2 * colb);
        acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[t], bop, acc[cb], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);   // half 1 waits for its loads only after this
  }
  // sum over the 8 waves: wave w' stores acc[cb] registers 4 r4 .. 4 r4 + 3
  // of lane l at f32x4 slot ((w' * NCB + cb) * 4 + r4) * 64 + l (8 NCB
  // 4 KB slots: the whole W_UV buffer); wave w then adds up slots
  // j = RPW w .. RPW w + RPW - 1 of the 4 NCB (column block j / 4,
  // registers 4 (j mod 4) .. +3)
  constexpr int RPW = NCB / 2;
  lds_barrier();   // every wave is done with W_UV
  f32x4* const xch = (f32x4*)w_lds;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      xch[((w * NCB + cb) * 4 + r4) * 64 + l] =
          f32x4{acc[cb][4 * r4], acc[cb][4 * r4 + 1], acc[cb][4 * r4 + 2], acc[cb][4 * r4 + 3]};
  lds_barrier();
#pragma unroll
  for (int q = 0; q < RPW; ++q) {
    const int j = RPW * w + q, cb = j >> 2, r4 = j & 3;
    f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ww = 0; ww < 8; ++ww) sum += xch[((ww * NCB + cb) * 4 + r4) * 64 + l];
    const int n = 32 * NCB * cs + 32 * cb + l32;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int bb = bc * 32 + 8 * r4 + 4 * h + c;   // accumulator register 4 r4 + c
      if (bb < p.B) p.out[((int64_t)bb * p.H + head) * D_V + n] = (bf16)sum[c];
    }
  }
}

// ----------------------------------------------------------------------------
// merge + W_UV for at most G partials per row, reading whole partial rows:
// the grid and the W_UV staging of mla_combine_s4_kernel, but wave w merges
// sequences 4w .. 4w+3 of the workgroup's 32, one 1 KB partial row per load
// instruction (lane l: dims 8l .. 8l+7), where the lane-per-sequence layout
// of mla_combine_s4_kernel makes each load touch 32 rows 32 bytes at a time
// (four times the cache lines per instruction, and the memory pipeline, not
// HBM, then bounds that merge). The merged rows go to LDS as bf16 (16-byte
// chunks XOR-swizzled by the row, so the MFMA A reads of 32 rows hit
// distinct banks), and waves 0 .. NCB-1 multiply them by the W_UV columns
// of their 32-column block over the whole 512-long contraction. A row's
// partial count is the plan's (p.nsplit, wave-uniform here) or p.S; the
// loads past it are not issued.
// ----------------------------------------------------------------------------
template <int NCB, int G>
__global__ __launch_bounds__(CB_THREADS) void mla_combine_rows_kernel(CombineParams p) {
  constexpr int NCS = 4 / NCB;         // workgroups per (head, 32 sequences)
  constexpr int ROWB = 64 * NCB;       // bytes of this workgroup's slice of a W_UV row
  constexpr int RPI = 1024 / ROWB;     // slice rows per 1 KB direct load
  constexpr int NI = 64 / RPI;         // direct loads per wave (its 64 rows)
  static_assert(4 * G <= 64, "one lane per (sequence, partial) of a wave");
  __shared__ __attribute__((aligned(1024))) char w_lds[D_C * ROWB];   // 128 or 64 KB
  __shared__ __attribute__((aligned(1024))) char a_lds[32 * D_C * 2];  // 32 merged rows, bf16
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = l >> 5, l32 = l & 31, jj = l & 15, g16 = l >> 4;
  int head, bc, cs;
  {
    const int x = blockIdx.x;
    const int q_lo = x & 7, rest = x >> 3;
    bc = __builtin_amdgcn_readfirstlane(rest % p.nbc);
    const int r2 = rest / p.nbc;
    cs = __builtin_amdgcn_readfirstlane(r2 % NCS);
    head = __builtin_amdgcn_readfirstlane((r2 / NCS) * 8 + q_lo);
    if (head >= p.H) return;
  }
  const int b_lo = bc * 32 + 4 * w;   // this wave's first sequence
  // partials per sequence (wave-uniform; 0 past the batch) and the rows of
  // partial 0
  int nb[4];
  int64_t row[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = min(b_lo + i, p.B - 1);
    nb[i] = b_lo + i >= p.B ? 0 : p.nsplit ? min(max(p.nsplit[b], 1), p.S) : p.S;
    row[i] = (int64_t)b * p.sp * p.H + head;
  }
  const int64_t sstep = (int64_t)p.ss * p.H;
  // lse and factor of (sequence i, partial s) in lane i G + s
  float lse_l = -INFINITY, scl_l = 0.f;
  if (l < 4 * G) {
    const int i = l / G, s = l % G;
    int n = nb[0];
#pragma unroll
    for (int k = 1; k < 4; ++k) n = (i == k) ? nb[k] : n;
    int64_t r0 = row[0];
#pragma unroll
    for (int k = 1; k < 4; ++k) r0 = (i == k) ? row[k] : r0;
    const int64_t ix = r0 + min(s, max(n, 1) - 1) * sstep;
    const float x = p.part_lse[ix];
    scl_l = p.part_scale[ix];
    lse_l = (s < n) ? x : -INFINITY;
  }
  // whole partial rows (the loads past a row's count are not issued: the
  // count is uniform over the wave)
  f16x8 v[4][G];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int s = 0; s < G; ++s) {
      v[i][s] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
      if (s < nb[i]) v[i][s] = *(const f16x8*)(p.part_o + (row[i] + s * sstep) * D_C + 8 * l);
    }
  {
    // rows 256 hf + 32 w .. +31 of W_UV[h], columns 32 NCB cs .. +32 NCB - 1
    // (ROWB bytes of each 256-byte row), to the same rows of the LDS copy
    // (rows ROWB apart), RPI rows per 1 KB load
    const __amdgpu_buffer_rsrc_t rs = proj_rsrc(p.w_uv + (int64_t)head * D_C * D_V, D_C * D_V * 2);
    const int vo = 256 * (l / (ROWB / 16)) + 16 * (l % (ROWB / 16));
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int r0 = 256 * (k / (NI / 2)) + 32 * w + RPI * (k % (NI / 2));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(w_lds + r0 * ROWB), 16, vo,
          r0 * 256 + cs * ROWB, 0, 0);
    }
    asm volatile("" ::: "memory");
  }
  // weights of each sequence's partials: 2^(lse_s - L) * factor_s / sum
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float lv[G], L = -INFINITY;
#pragma unroll
    for (int s = 0; s < G; ++s) {
      lv[s] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                            __builtin_bit_cast(int, lse_l), i * G + s));
      L = fmaxf(L, lv[s]);
    }
    float e[G], wsum = 0.f;
#pragma unroll
    for (int s = 0; s < G; ++s) {
      e[s] = (L > -INFINITY) ? fast_exp2(lv[s] - L) : 0.f;
      wsum += e[s];
    }
    const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
    float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < G; ++s) {
      const float sc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                     __builtin_bit_cast(int, scl_l), i * G + s));
      const float wt = e[s] * sc * inv;
#pragma unroll
      for (int k = 0; k < 8; ++k) m[k] += wt * (float)v[i][s][k];
    }
    const int r = 4 * w + i;   // row of the merged block
    bf16x8 pk;
#pragma unroll
    for (int k = 0; k < 8; ++k) pk[k] = (bf16)m[k];
    *(bf16x8*)(a_lds + r * (D_C * 2) + 16 * (l ^ (r & 15))) = pk;
    if (cs == 0 && l == 0 && b_lo + i < p.B && p.lse)
      p.lse[(int64_t)(b_lo + i) * p.H + head] =
          (L > -INFINITY) ? (L + __builtin_log2f(wsum)) * LN2 : -INFINITY;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's W_UV rows landed
  lds_barrier();
  if (w >= NCB) return;
  // output columns 32 NCB cs + 32 w .. +31: two chains (even, odd k-steps)
  const int colb = 32 * w + 16 * (g16 & 1) + 4 * (jj & 3);   // B-operand column base
  f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
  for (int ks = 0; ks < D_C / 16; ++ks) {
    const int c = 2 * ks + h;   // 16-byte chunk of the row: dims 16 ks + 8 h .. +7
    const bf16x8 a = *(const bf16x8*)(a_lds + l32 * (D_C * 2) + 16 * (c ^ (l32 & 15)));
    const int ra = 16 * ks + 8 * h + (jj >> 2);
    const bf16x8 bop = tr_read_8(w_lds + ra * ROWB + 2 * colb, w_lds + (ra + 4) * ROWB + 2 * colb);
    acc[ks & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bop, acc[ks & 1], 0, 0, 0);
  }
  const int n = 32 * NCB * cs + 32 * w + l32;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int bb = bc * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
    if (bb < p.B) p.out[((int64_t)bb * p.H + head) * D_V + n] = (bf16)(acc[0][r] + acc[1][r]);
  }
}

}  // namespace mla
