// Length-aware split plan, made on the device from the sequences' actual
// lengths (the host knows only max_len). The attention launch keeps its
// number of workgroups (nitems per head group); what changes is how the
// sequences are cut: one split length c for the whole batch (a multiple of
// the 32-token tile, at most the default split length ts_max and at least
// max_len / slots), the smallest for which the splits of all sequences,
// n_b = max(1, ceil(len_b / c)) each, fit in the nitems work items. Long
// sequences then get more splits than short ones and every workgroup walks
// about the same number of tokens, where the default plan gives every
// sequence the same split count and the launch lasts as long as a full
// split of the longest one.
//
// It runs as one workgroup of 256 threads inside the launch of the query
// absorption (which the attention launch follows on the stream), beside the
// absorb workgroups.
//
// Outputs: items[q] = (b, s, t0, t1) for the splits in sequence order
// (consecutive items of a sequence share an XCD under the attention
// kernels' workgroup mapping), b = -1 past the last one; nsplit[b] = n_b,
// the number of partial slots of sequence b that the merge reads.
#pragma once

#include "common.hpp"
#include "decode_mfma.hpp"

namespace mla {

struct BalanceParams {   // items == nullptr: no plan
  const int32_t* lengths;  // [B] device
  int B, max_len;
  int nitems;              // work items of the attention launch
  int slots;               // partial slots per sequence (n_b <= slots)
  int ts_max;              // the default split length (tokens, multiple of TILE)
  SplitItem* items;        // [nitems]
  int32_t* nsplit;         // [B]
};

constexpr int BP_THREADS = 256;

__device__ __forceinline__ int bp_len(const BalanceParams& p, int b) {
  const int raw = p.lengths[b];
  return min(max(raw, 0), p.max_len);
}

// Sum of v over the workgroup (every thread gets it); `red` holds 4 ints.
__device__ __forceinline__ int bp_block_sum(int v, int* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

__device__ __forceinline__ void balance_plan(const BalanceParams& p) {
  __shared__ int red[4];
  __shared__ int scan[BP_THREADS / 64];
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
#if MLA_DEBUG_CHECKS
  for (int b = tid; b < p.B; b += BP_THREADS) {
    const int raw = p.lengths[b];
    debug_flag(raw < 0 || raw > p.max_len, DBG_LENGTH);
  }
#endif
  // splits of the whole batch at split length c tokens
  auto count = [&](int c) {
    int n = 0;
    for (int b = tid; b < p.B; b += BP_THREADS) n += max(1, (bp_len(p, b) + c - 1) / c);
    return bp_block_sum(n, red);
  };
  // smallest c (in tiles) in [lo, hi] whose splits fit; hi always does (the
  // default plan: at most ceil(max_len / ts_max) splits per sequence)
  const int hi_t = p.ts_max / TILE;
  const int min_c = (p.max_len + p.slots - 1) / p.slots;
  int lo = min(max((min_c + TILE - 1) / TILE, 1), hi_t), hi = hi_t;
  while (lo < hi) {
    const int mid = (lo + hi) / 2;
    if (count(mid * TILE) <= p.nitems) hi = mid;
    else lo = mid + 1;
  }
  const int c = hi * TILE;
  // items in sequence order: exclusive prefix sum of n_b, 256 sequences per round
  int base = 0;
  for (int b0 = 0; b0 < p.B; b0 += BP_THREADS) {
    const int b = b0 + tid;
    const int len = b < p.B ? bp_len(p, b) : 0;
    const int n = b < p.B ? max(1, (len + c - 1) / c) : 0;
    int incl = n;   // inclusive scan within the wave, then across the 4 waves
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (l >= o) incl += y;
    }
    __syncthreads();
    if (l == 63) scan[w] = incl;
    __syncthreads();
    int before = base;
    for (int k = 0; k < w; ++k) before += scan[k];
    const int first = before + incl - n;
    if (b < p.B) {
      p.nsplit[b] = n;
      for (int s = 0; s < n; ++s) {
        SplitItem it;
        it.b = b;
        it.s = s;
        it.t0 = s * c;
        it.t1 = min((s + 1) * c, len);
        p.items[first + s] = it;
      }
    }
    base += scan[0] + scan[1] + scan[2] + scan[3];
  }
  for (int q = base + tid; q < p.nitems; q += BP_THREADS) {
    SplitItem it;
    it.b = -1;
    it.s = it.t0 = it.t1 = 0;
    p.items[q] = it;
  }
}

}  // namespace mla
