// Shared device types and helpers for the gfx950 MLA kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int D_C = 512;      // latent width
constexpr int D_R = 64;       // decoupled RoPE key width
constexpr int D_QK = D_C + D_R;
constexpr int D_N = 128;      // no-RoPE query/key width
constexpr int D_V = 128;      // value width
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

enum CacheKind { CACHE_F32 = 0, CACHE_BF16 = 1, CACHE_FP8 = 2 };

// Debug-checks build (MLA_DEBUG_CHECKS=1): the device-resident integers that
// the host cannot validate without a synchronisation (sequence lengths,
// block-table entries, append positions) are checked where the kernels read
// them, and each violation sets its bit in a per-device error word (read
// and cleared by mla_debug_errors). The kernels clamp such values in every
// build, so a violation never makes them access memory out of bounds; the
// word only reports it. Release builds compile the checks away.
#ifndef MLA_DEBUG_CHECKS
#define MLA_DEBUG_CHECKS 0
#endif
enum DebugBit : unsigned {
  DBG_LENGTH = 1u,       // lengths[b] outside [0, max_len]
  DBG_BLOCK = 2u,        // block-table entry (or the row it gives) outside the cache
  DBG_POSITION = 4u,     // append position outside the sequence's capacity
};
#if MLA_DEBUG_CHECKS
__device__ unsigned int g_debug_word;
__device__ __forceinline__ void debug_flag(bool bad, unsigned bit) {
  if (bad) atomicOr(&g_debug_word, bit);
}
#else
__device__ __forceinline__ void debug_flag(bool, unsigned) {}
#endif

// 64-lane wavefront helpers
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Physical cache row of token t of sequence b (contiguous or paged), clamped
// into [0, rows) so that malformed device-side tables cannot fault.
__device__ __forceinline__ int64_t cache_row(int b, int t, int64_t seq_capacity,
                                             const int32_t* __restrict__ block_table,
                                             int max_blocks, int block_size, int64_t rows) {
  int64_t r;
  if (block_table) {
    int blk = block_table[(int64_t)b * max_blocks + t / block_size];
    r = (int64_t)blk * block_size + (t % block_size);
  } else {
    r = (int64_t)b * seq_capacity + t;
  }
  const bool ok = r >= 0 && r < rows;
  debug_flag(!ok, DBG_BLOCK);
  return ok ? r : 0;
}

// Absorbed-query layout in the workspace (written by the absorb kernel,
// read by the attention kernels): per (sequence, group of 32 heads), the 36
// k-steps of the QK^T B operand in lane order, so that a wave loads k-step j
// as one contiguous 1 KB. Lane l holds head 32 g + (l % 32), dims
// 16 j + 8 (l / 32) .. +7. Element n (0..575) of head hd of sequence b:
__device__ __forceinline__ int64_t qop_index(int b, int hd, int n, int H) {
  const int lane = (hd & 31) + 32 * ((n >> 3) & 1);
  return ((((int64_t)b * (H >> 5) + (hd >> 5)) * (D_QK / 16) + (n >> 4)) * 64 + lane) * 8 + (n & 7);
}

}  // namespace mla
