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

#include "append.hpp"
#include "common.hpp"

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
};

constexpr int AB_APITCH = D_N * 2 + 16;    // 272 B: 8 rows' 16-byte chunks hit distinct banks
constexpr int AB_COLS = 128;               // output columns per workgroup
constexpr int AB_ROW = AB_COLS * 2;        // 256 B per W row slice in LDS
constexpr int AB_OPITCH = 32 * 2 + 16;     // 80 B: output staging row (32 bf16 + pad)

__device__ __forceinline__ void absorb_workgroup(const AbsorbParams& p, int x) {
  __shared__ __attribute__((aligned(1024))) char w_lds[D_N * AB_ROW];   // 32 KB
  __shared__ __attribute__((aligned(16))) char a_lds[2][32 * AB_APITCH];  // two chunks of 32 seq
  __shared__ __attribute__((aligned(16))) char o_lds[4][32 * AB_OPITCH];  // per wave: 32 seq x 32 cols
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
    for (int cb = 0; cb < 2 && b0 + 32 * cb < p.B; ++cb) {
      const int bc0 = b0 + 32 * cb;
      f32x16 acc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < D_N / 16; ++ks) {
        const bf16x8 a = *(const bf16x8*)(a_lds[cb] + l32 * AB_APITCH + 2 * (16 * ks + 8 * h));
        const int ra = 16 * ks + r1, rb = ra + 4;
        const bf16x8 bop = tr_read_8(w_lds + ra * AB_ROW + 16 * (chunk ^ wrow_swizzle(ra)) + off,
                                     w_lds + rb * AB_ROW + 16 * (chunk ^ wrow_swizzle(rb)) + off);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bop, acc, 0, 0, 0);
      }
      // lane holds column 32w + l32 of the slice, rows b = 8(r/4) + 4h + r%4:
      // transpose through LDS so each lane stores 8 consecutive columns of
      // one sequence (one 16-byte piece of the query layout)
      char* ol = o_lds[w];
#pragma unroll
      for (int r = 0; r < 16; ++r)
        *(bf16*)(ol + (8 * (r >> 2) + 4 * h + (r & 3)) * AB_OPITCH + 2 * l32) = (bf16)(acc[r] * p.c);
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
  absorb_workgroup(p, blockIdx.x);
}

// absorb and cache append in one launch: workgroups past the absorb grid
// append the new rows, one sequence per wave (the absorb neither reads nor
// writes the cache, so the two halves are independent)
__global__ __launch_bounds__(256) void mla_absorb_append_kernel(AbsorbParams p, AppendParams a,
                                                               int absorb_blocks) {
  if ((int)blockIdx.x < absorb_blocks) {
    absorb_workgroup(p, blockIdx.x);
  } else {
    const int b = ((int)blockIdx.x - absorb_blocks) * 4 + (int)(threadIdx.x >> 6);
    if (b < p.B) append_row(a, b, threadIdx.x & 63);
  }
}

// ----------------------------------------------------------------------------
// merge + W_UV: one workgroup (4 waves) per head; W_UV[h] (512 rows x 256 B)
// is brought into LDS whole by direct-to-LDS loads while the splits of the
// first chunk of 32 sequences are merged.
// ----------------------------------------------------------------------------
struct CombineParams {
  const _Float16* part_o;   // [B, S, H, 512] fp16, relative to part_scale
  const float* part_scale;  // [B, S, H]
  const float* part_lse;    // [B, S, H] log2 domain
  const bf16* w_uv;       // [H, 512, 128]
  bf16* out;              // [B, H, 128]
  float* lse;             // [B, H] natural log, or nullptr
  int B, H, S, nbc;
};

constexpr int CB_APITCH = D_C + 16;         // 528 B: half a merged row (256 dims) + pad

__global__ __launch_bounds__(256) void mla_combine_kernel(CombineParams p) {
  __shared__ __attribute__((aligned(1024))) char w_lds[D_C * D_V * 2];   // 128 KB
  __shared__ __attribute__((aligned(16))) char a_lds[32 * CB_APITCH];    // 32 seq x 256 dims
  __shared__ float lmax[32], winv[32];   // per sequence of the chunk: max lse, 1/sum of weights
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = l >> 5, l32 = l & 31, jj = l & 15, g16 = l >> 4;
  // (head, chunk of 32 sequences); the chunks of one head share an XCD (L2)
  int head, bc;
  {
    const int x = blockIdx.x;
    const int q_lo = x & 7, rest = x >> 3;
    bc = rest % p.nbc;
    head = (rest / p.nbc) * 8 + q_lo;
    if (head >= p.H) return;
  }
  {
    const __amdgpu_buffer_rsrc_t rs = proj_rsrc(p.w_uv + (int64_t)head * D_C * D_V, D_C * D_V * 2);
#pragma unroll
    for (int k = 0; k < 32; ++k) {   // 128 lines of 1 KB (4 rows each), 32 per wave
      const int line = w * 32 + k;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(w_lds + line * 1024), 16, 16 * l,
          line * 1024, 0, 0);
    }
  }
  const int colb = 32 * w + 16 * (g16 & 1) + 4 * (jj & 3);   // B-operand column base
  {
    const int b0 = bc * 32;
    // merge weights: per sequence, 2^(lse_s - L) / sum over splits
    if (tid < 32) {
      const int b = b0 + tid;
      float L = -INFINITY, wsum = 0.f;
      if (b < p.B) {
        const float* ls = p.part_lse + (int64_t)b * p.S * p.H + head;
        for (int s = 0; s < p.S; ++s) L = fmaxf(L, ls[(int64_t)s * p.H]);
        if (L > -INFINITY)
          for (int s = 0; s < p.S; ++s) wsum += fast_exp2(ls[(int64_t)s * p.H] - L);
        if (p.lse)
          p.lse[(int64_t)b * p.H + head] =
              (L > -INFINITY) ? (L + __builtin_log2f(wsum)) * LN2 : -INFINITY;
      }
      winv[tid] = (L > -INFINITY) ? 1.0f / wsum : 0.0f;
      lmax[tid] = L;
    }
    __syncthreads();
    f32x16 acc = f32x16{};
    for (int half = 0; half < 2; ++half) {
      // thread: dims half*256 + 8*(tid%32) .. +7 of sequences b0 + tid/32 + 8i
      const int d8 = tid & 31;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = (tid >> 5) + 8 * i;
        const int b = b0 + r;
        f32x8 m = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (b < p.B && winv[r] > 0.f) {
          const float L = lmax[r];
          const int64_t row0 = (int64_t)b * p.S * p.H + head;
          const _Float16* po = p.part_o + row0 * D_C + half * 256 + 8 * d8;
#pragma unroll 4
          for (int s = 0; s < p.S; ++s) {
            const int64_t rs_ = row0 + (int64_t)s * p.H;
            const float wgt = fast_exp2(p.part_lse[rs_] - L) * p.part_scale[rs_];
            const f16x8 v = *(const f16x8*)(po + (int64_t)s * p.H * D_C);
#pragma unroll
            for (int k = 0; k < 8; ++k) m[k] += wgt * (float)v[k];
          }
          m *= winv[r];
        }
        bf16x8 pk;
#pragma unroll
        for (int k = 0; k < 8; ++k) pk[k] = (bf16)m[k];
        *(bf16x8*)(a_lds + r * CB_APITCH + 16 * d8) = pk;
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // W_UV landed (first pass)
      __syncthreads();
#pragma unroll 4
      for (int ks = 0; ks < 16; ++ks) {
        const bf16x8 a = *(const bf16x8*)(a_lds + l32 * CB_APITCH + 2 * (16 * ks + 8 * h));
        const int ra = half * 256 + 16 * ks + 8 * h + (jj >> 2);
        const bf16x8 bop = tr_read_8(w_lds + ra * 256 + 2 * colb, w_lds + (ra + 4) * 256 + 2 * colb);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bop, acc, 0, 0, 0);
      }
      __syncthreads();   // a_lds is rewritten next
    }
    const int n = 32 * w + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int bb = b0 + 8 * (r >> 2) + 4 * h + (r & 3);
      if (bb < p.B) p.out[((int64_t)bb * p.H + head) * D_V + n] = (bf16)acc[r];
    }
  }
}

}  // namespace mla
