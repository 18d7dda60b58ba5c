// C ABI of the MLA decode library: argument validation, split planning and
// kernel launches on the caller's stream. See include/mla.h for the contract.
#include <atomic>
#include <mutex>
#include <cmath>
#include <cstdlib>
#include <cstring>

#include <hip/hip_ext.h>

#include "mla.h"
#include "append.hpp"
#include "decode_fp8mma.hpp"
#include "decode_mfma.hpp"
#include "fp32_path.hpp"
#include "fused_io.hpp"
#include "kv_project.hpp"
#include "prefill_mfma.hpp"
#include "project_mfma.hpp"
#include "split_plan.hpp"

using namespace mla;

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev >= kMaxDevices) dev = kMaxDevices - 1;
  int v = g_cu_count[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  g_cu_count[dev].store(n, std::memory_order_relaxed);
  return n;
}

int env_int(const char* name) {
  const char* s = std::getenv(name);
  return s ? std::atoi(s) : 0;
}

int env_int_or(const char* name, int dflt) {
  const char* s = std::getenv(name);
  return s ? std::atoi(s) : dflt;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool dims_supported(const mla_dims* d) {
  return d && d->d_c == D_C && d->d_rope == D_R && d->d_nope == D_N && d->d_v == D_V && d->heads >= 1;
}

size_t elem_size(mla_dtype t) {
  switch (t) {
    case MLA_F32: return 4;
    case MLA_BF16: return 2;
    case MLA_FP8_E4M3: return 1;
  }
  return 0;
}

// Split plan: how many token ranges each sequence is cut into, and how many
// waves / head groups each workgroup covers.
struct Plan {
  int S = 1;          // splits per sequence
  int TS = TILE;      // tokens per split (multiple of the 32-token tile)
  int NW = 4;         // waves per workgroup (bf16 path)
  int G = 1;          // head groups (bf16 path)
  // length-aware plan (made on the device, split_plan.hpp): S is then the
  // partial slots per sequence, nitems the attention launch's work items per
  // head group, TS the longest split
  bool length_aware = false;
  int nitems = 0;
};

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

Plan make_plan(int B, int H, int max_len, mla_dtype act, const mla_decode_options* opts,
               int nw = 0) {
  Plan pl;
  const int cus = device_cu_count();
  const int len = max_len > 0 ? max_len : 1;
  int S;
  if (act == MLA_F32) {
    pl.NW = 0;
    pl.G = 1;
    const int min_tok = 64;
    S = std::max(ceil_div(len, F32_MAX_SPLIT),
                 std::min(ceil_div(cus, (int64_t)B * H), ceil_div(len, min_tok)));
  } else {
    const int hw = H / 32;
    pl.NW = (hw % 4 == 0) ? 4 : (hw % 2 == 0) ? 2 : 1;
    if (nw > 0 && hw % nw == 0) pl.NW = nw;
    const int fw = env_int("MLA_WAVES");   // A/B only: waves (32 heads each) per workgroup
    if ((fw == 1 || fw == 2 || fw == 4) && hw % fw == 0) pl.NW = fw;
    pl.G = hw / pl.NW;
    // one resident workgroup per CU; splits no shorter than 64 tokens (at
    // B=1 N=4096, 64 splits of 64 tokens beat 16 of 256: 33.0 vs 38.5 us
    // for the step's kernels)
    const int groups = B * pl.G;
    S = std::min(ceil_div(cus, groups), ceil_div(len, 64));
  }
  int forced = (opts && opts->num_splits > 0) ? opts->num_splits : env_int("MLA_SPLITS");
  if (forced > 0) S = forced;
  S = std::max(1, std::min(S, ceil_div(len, TILE)));
  // a split has at most 64 tiles (the attention kernel keeps one tile row per
  // lane): ceil(len / S) <= 2048, which stays <= 2048 when rounded up to 32
  if (act != MLA_F32) S = std::max(S, ceil_div(len, 64 * TILE));
  int ts = ceil_div(len, S);
  ts = ceil_div(ts, TILE) * TILE;
  if (act == MLA_F32) ts = std::min(ts, F32_MAX_SPLIT);
  pl.TS = ts;
  pl.S = ceil_div(len, ts);
  return pl;
}

// Rows of more than 8 splits (5-8 take the row merge with 8 slots, see
// run_decode) are merged in one level (mla_combine_kernel) or two
// (mla_merge_splits_kernel folds each row's splits into groups,
// mla_combine_s4_kernel merges the groups and applies W_UV). Measured: two
// levels win above 16 splits (2 groups), and from 5 splits when there are
// at most 32 sequences (1 group; mla_combine_kernel then has only one
// workgroup per head); with more sequences and 5-16 splits one level is
// faster. Returns the group count, 0 for one level; MLA_MERGE_GROUPS (0-4)
// overrides.
int merge_groups(int S, int nbc) {
  const char* e = std::getenv("MLA_MERGE_GROUPS");
  if (e) return std::max(0, std::min(std::atoi(e), CB_G));
  if (S > 16) return 2;
  return nbc == 1 ? 1 : 0;
}

// Column split of the S <= 4 merge: when its grid has fewer workgroups than
// the device has CUs. MLA_COMBINE_COLS (1 or 2 workgroups per head and
// chunk of sequences) overrides.
bool combine_col_split(int workgroups) {
  const char* e = std::getenv("MLA_COMBINE_COLS");
  if (e) return std::atoi(e) == 2;
  return workgroups < device_cu_count();
}

// Merge + W_UV of at most G partials per row: mla_combine_s4_kernel (a lane
// per sequence) for up to 4, mla_combine_rows_kernel (whole partial rows per
// load; it issues no load past a row's own partial count) for up to 8
// (measured: equal at 4 partials, 5 us faster at 8 slots holding 2-6);
// MLA_SHORT_MERGE=lanes or rows overrides. Two workgroups per (head, 32
// sequences), each for half of the output columns, where one each would
// leave CUs idle.
template <int G>
void launch_short_merge(const CombineParams& cp, dim3 cgrid, hipStream_t stream) {
  const bool col_split = combine_col_split((int)cgrid.x);
  const char* e = std::getenv("MLA_SHORT_MERGE");
  const bool lanes = e ? std::strcmp(e, "lanes") == 0 : G <= CB_G;
  const dim3 grid(col_split ? 2 * cgrid.x : cgrid.x), block(CB_THREADS);
  if (lanes) {
    if (col_split) hipLaunchKernelGGL((mla_combine_s4_kernel<2, G>), grid, block, 0, stream, cp);
    else hipLaunchKernelGGL((mla_combine_s4_kernel<4, G>), grid, block, 0, stream, cp);
  } else {
    if (col_split) hipLaunchKernelGGL((mla_combine_rows_kernel<2, G>), grid, block, 0, stream, cp);
    else hipLaunchKernelGGL((mla_combine_rows_kernel<4, G>), grid, block, 0, stream, cp);
  }
}

// The fp8 cache goes to the fp8 matrix cores (decode_fp8mma.hpp) when its
// layout fits that kernel: four waves of 32 heads per workgroup, splits of
// whole 64-token tiles (at most 64 of them), and page blocks holding whole
// tiles; MLA_FP8_KERNEL=widen selects the widening kernel instead.
bool use_fp8mma(mla_dtype cdt, const Plan& pl, const int32_t* block_table, int block_size) {
  if (cdt != MLA_FP8_E4M3 || pl.NW != 4) return false;
  if (block_table && block_size % F8_TILE != 0) return false;
  const char* e = std::getenv("MLA_FP8_KERNEL");
  return !(e && std::strcmp(e, "widen") == 0);
}

// Plan of a decode call: make_plan; for the fp8 matrix-core kernel, splits
// of whole 64-token tiles, as long as 64 of them (that kernel keeps one tile
// row per lane of 64-token tiles, where the bf16 kernel's tiles hold 32), so
// a sequence needs no more splits than filling the CUs asks for (never more
// than make_plan's, so the workspace make_plan sizes is enough).
Plan decode_plan(int B, int H, int max_len, mla_dtype act, mla_dtype cdt,
                 const int32_t* block_table, int block_size, const mla_decode_options* opts) {
  Plan pl = make_plan(B, H, max_len, act, opts);
  // bf16 cache with at most half of the CUs holding a workgroup (a batch of
  // one or two sequences): workgroups of two waves (64 heads), twice as many
  // of them, each with half the queries to load and half the partial to
  // write. Measured at B=1 N=4096: 14.2-14.4 vs 15.8-17.1 us per attention
  // launch, 33.5 vs 34.8 us per step replayed from a graph. Never more
  // splits than make_plan's (the splits fill the CUs for twice the groups).
  if (act == MLA_BF16 && cdt == MLA_BF16 && pl.NW == 4 && !env_int("MLA_WAVES") &&
      (int64_t)B * pl.S * pl.G * 2 <= device_cu_count())
    pl = make_plan(B, H, max_len, act, opts, 2);
  if (act != MLA_F32 && use_fp8mma(cdt, pl, block_table, block_size)) {
    const int len = max_len > 0 ? max_len : 1;
    const bool forced = (opts && opts->num_splits > 0) || env_int("MLA_SPLITS") > 0;
    int S = pl.S;
    if (!forced) {
      const int fill = std::min(ceil_div(device_cu_count(), (int64_t)B * pl.G), ceil_div(len, 64));
      S = std::min(S, std::max(fill, ceil_div(len, F8_MAX_TILES * F8_TILE)));
    }
    pl.TS = std::min(ceil_div(ceil_div(len, S), F8_TILE) * F8_TILE, F8_MAX_TILES * F8_TILE);
    pl.S = ceil_div(len, pl.TS);
  }
  return pl;
}

// The length-aware plan (mla_decode_options.length_aware) on the bf16 cache:
// as many work items as the default plan has splits (so the launch keeps its
// workgroups), twice its split slots per sequence (split lengths from half
// the default one up).
void apply_length_aware(Plan& pl, int B, mla_dtype act, mla_dtype cdt,
                        const mla_decode_options* opts) {
  if (!opts || !opts->length_aware || act != MLA_BF16 || cdt != MLA_BF16 || pl.S < 2) return;
  pl.length_aware = true;
  pl.nitems = B * pl.S;
  pl.S = 2 * pl.S;
}

// Workspace: absorbed queries [B, H, 576] (activation dtype), split partials
// [B, S, H, 512] (fp32 on the fp32 path; fp16 relative to a per-row fp32
// scale [B, S, H] otherwise), split lse [B, S, H] fp32; with a length-aware
// plan, its work items [nitems] and the splits per sequence [B].
struct WsLayout {
  size_t q_off, po_off, ps_off, pl_off, items_off, nsplit_off, total;
};

WsLayout ws_layout(int B, int H, const Plan& pl, mla_dtype act) {
  WsLayout w;
  const size_t qe = (act == MLA_F32) ? 4 : 2;
  const size_t pe = (act == MLA_F32) ? 4 : 2;
  const size_t rows = (size_t)B * pl.S * H;
  w.q_off = 0;
  w.po_off = align_up((size_t)B * H * D_QK * qe, 256);
  w.ps_off = align_up(w.po_off + rows * D_C * pe, 256);
  w.pl_off = align_up(w.ps_off + (act == MLA_F32 ? 0 : rows * 4), 256);
  w.items_off = align_up(w.pl_off + rows * 4, 256);
  w.nsplit_off = align_up(w.items_off + (pl.length_aware ? (size_t)pl.nitems * sizeof(SplitItem) : 0), 256);
  w.total = align_up(w.nsplit_off + (pl.length_aware ? (size_t)B * 4 : 0), 256);
  return w;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Largest row stride (bytes) of a cache array that a decode call accepts:
// the attention kernels form a tile's buffer records and lane offsets as
// 32-bit products of up to 32 rows times the stride.
constexpr int64_t kMaxRowStrideBytes = (int64_t)1 << 24;

// Prefill workspace: W_UV transposed [H, 128, 512] (bf16), decompressed keys
// and values [B, H, cap, 128] each, RoPE keys [B, cap, 64] (fp16), with cap
// = max_len rounded up to the expansion tile.
struct PrefillWs {
  size_t wuvt, kx, vx, kpx, total;
  int cap;
};

PrefillWs prefill_ws(int B, int H, int max_len) {
  PrefillWs w;
  w.cap = (int)(((int64_t)max_len + EX_ROWS - 1) / EX_ROWS * EX_ROWS);
  const size_t kv = (size_t)B * H * w.cap * D_N * 2;
  w.wuvt = 0;
  w.kx = align_up((size_t)H * D_V * D_C * 2, 256);
  w.vx = align_up(w.kx + kv, 256);
  w.kpx = align_up(w.vx + kv, 256);
  w.total = align_up(w.kpx + (size_t)B * w.cap * D_R * 2, 256);
  return w;
}

// Scratch of mla_decode_paged_noalloc: the absorbed queries and split
// partials that mla_decode_paged keeps in the caller's workspace. Each device
// holds its own copy (from the module's load until the process ends). Host
// code never uses the array's name as an address: the device address comes
// from hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // guarded by g_scratch_mu

mla_status scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MLA_ERR_HIP;
    if (((uintptr_t)p & 255) != 0) return MLA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
}

mla_status launch_status() {
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

#define MLA_TRY(x)                         \
  do {                                     \
    mla_status _s = (x);                   \
    if (_s != MLA_OK) return _s;           \
  } while (0)

// Validation of a cache append (mla_cache_append, or the append of a decode
// call); fills the kernel parameters.
mla_status check_append(const mla_dims* dims, const void* c_kv, const void* k_pe,
                        mla_dtype in_dtype, const int32_t* positions, int32_t batch,
                        void* latent, int64_t ls, void* rope, int64_t rs, void* scales,
                        mla_dtype cdt, int64_t rows, int64_t seq_capacity,
                        const int32_t* block_table, int32_t max_blocks, int32_t block_size,
                        float rope_theta, AppendParams* out) {
  if (!dims || batch < 0) return MLA_ERR_INVALID_ARG;
  if (!dims_supported(dims)) return MLA_ERR_UNSUPPORTED;
  if (in_dtype != MLA_F32 && in_dtype != MLA_BF16) return MLA_ERR_UNSUPPORTED;
  const size_t ce = elem_size(cdt);
  if (!ce) return MLA_ERR_UNSUPPORTED;
  if (!std::isfinite(rope_theta) || rope_theta <= 0.f) return MLA_ERR_INVALID_ARG;
  if (batch == 0) return MLA_OK;
  if (!c_kv || !k_pe || !positions || !latent || !rope) return MLA_ERR_INVALID_ARG;
  if (cdt == MLA_FP8_E4M3 && !scales) return MLA_ERR_INVALID_ARG;
  if (ls < D_C || rs < D_R || rows < 1) return MLA_ERR_INVALID_ARG;
  if (!aligned16(latent) || !aligned16(rope) || (ls * ce) % 16 != 0 || (rs * ce) % 16 != 0 ||
      !aligned16(c_kv) || ((uintptr_t)k_pe & 3) != 0)
    return MLA_ERR_INVALID_ARG;
  if (block_table) {
    if (block_size <= 0 || max_blocks <= 0) return MLA_ERR_INVALID_ARG;
  } else {
    if (seq_capacity < 1 || (int64_t)batch * seq_capacity > rows) return MLA_ERR_INVALID_ARG;
  }
  out->c_kv = c_kv;
  out->k_pe = k_pe;
  out->in_bf16 = (in_dtype == MLA_BF16);
  out->positions = positions;
  out->latent = latent;
  out->latent_stride = ls;
  out->rope = rope;
  out->rope_stride = rs;
  out->scales = (bf16*)scales;
  out->cache_kind = (cdt == MLA_F32) ? CACHE_F32 : (cdt == MLA_BF16) ? CACHE_BF16 : CACHE_FP8;
  out->rows = rows;
  out->seq_capacity = seq_capacity;
  out->block_table = block_table;
  out->max_blocks = max_blocks;
  out->block_size = block_size;
  out->theta = (double)rope_theta;
  out->part = nullptr;
  out->part_slices = 0;
  out->rows_in_batch = batch;
  return MLA_OK;
}

// Split of the down-projection's K (d_model) into slices: about 256
// workgroups (18 column tiles x slices x batch groups) so that one wave of
// workgroups covers the chip and reads the weights once; every slice is
// non-empty. MLA_PROJECT_SPLITS overrides the slice count (for tuning).
struct ProjPlan {
  int S, cps, mgroups, msub;
};

ProjPlan project_plan(int B, int D) {
  ProjPlan pl;
  const int nchunks = D / PJ_CHUNK;
  pl.mgroups = ceil_div(B, PJ_MG);
  pl.msub = pl.mgroups > 1 ? 4 : ceil_div(B, 32);
  int target = env_int("MLA_PROJECT_SPLITS");
  if (target <= 0) target = 256 / (PJ_NTILES * pl.mgroups);
  target = std::max(1, std::min(target, nchunks));
  pl.cps = ceil_div(nchunks, target);
  pl.S = ceil_div(nchunks, pl.cps);
  return pl;
}

size_t project_ws_bytes(int B, int D) {
  const ProjPlan pl = project_plan(B, D);
  return align_up((size_t)pl.S * B * D_QK * sizeof(float), 256);
}

template <typename T>
void launch_project(const ProjectParams& pp, int msub, int grid, hipStream_t stream) {
  switch (msub) {
    case 1: hipLaunchKernelGGL((mla_kv_project_kernel<T, 1>), dim3(grid), dim3(256), 0, stream, pp); break;
    case 2: hipLaunchKernelGGL((mla_kv_project_kernel<T, 2>), dim3(grid), dim3(256), 0, stream, pp); break;
    case 3: hipLaunchKernelGGL((mla_kv_project_kernel<T, 3>), dim3(grid), dim3(256), 0, stream, pp); break;
    default: hipLaunchKernelGGL((mla_kv_project_kernel<T, 4>), dim3(grid), dim3(256), 0, stream, pp); break;
  }
}

// Validation shared by both decode entry points.
mla_status check_decode(const mla_dims* dims, const void* q_nope, const void* q_pe,
                        const void* w_uk, const void* w_uv, mla_dtype act, const void* latent,
                        int64_t ls, const void* rope, int64_t rs, const void* scales,
                        mla_dtype cdt, int64_t rows, const int32_t* lengths, int32_t batch,
                        int32_t max_len, float softmax_scale, const void* out) {
  if (!dims) return MLA_ERR_INVALID_ARG;
  if (batch < 0 || max_len < 0 || max_len > (1 << 30)) return MLA_ERR_INVALID_ARG;
  if (!std::isfinite(softmax_scale)) return MLA_ERR_INVALID_ARG;
  if (!dims_supported(dims)) return MLA_ERR_UNSUPPORTED;
  const bool combo = (act == MLA_F32 && cdt == MLA_F32) || (act == MLA_BF16 && cdt == MLA_BF16) ||
                     (act == MLA_BF16 && cdt == MLA_FP8_E4M3);
  if (!combo) return MLA_ERR_UNSUPPORTED;
  if (act == MLA_BF16 && dims->heads % 32 != 0) return MLA_ERR_UNSUPPORTED;
  if (batch == 0) return MLA_OK;
  if (!q_nope || !q_pe || !w_uk || !w_uv || !latent || !rope || !lengths || !out)
    return MLA_ERR_INVALID_ARG;
  if (cdt == MLA_FP8_E4M3 && !scales) return MLA_ERR_INVALID_ARG;
  const size_t ce = elem_size(cdt);
  if (ls < D_C || rs < D_R || rows < 1) return MLA_ERR_INVALID_ARG;
  if (rows > INT32_MAX) return MLA_ERR_UNSUPPORTED;   // row indices are 32-bit in the kernels
  if (!aligned16(latent) || !aligned16(rope) || (ls * ce) % 16 != 0 || (rs * ce) % 16 != 0)
    return MLA_ERR_INVALID_ARG;
  // the attention kernels address a tile's rows with 32-bit byte offsets
  if (ls * (int64_t)ce >= kMaxRowStrideBytes || rs * (int64_t)ce >= kMaxRowStrideBytes)
    return MLA_ERR_UNSUPPORTED;
  const size_t ae = elem_size(act);
  if (((uintptr_t)q_nope | (uintptr_t)q_pe | (uintptr_t)w_uk | (uintptr_t)w_uv | (uintptr_t)out) %
          16 != 0 &&
      ae == 2)
    return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

// Parameters of the split attention kernels (bf16 / fp8 cache).
DecodeParams decode_params(const bf16* q, const void* latent, int64_t ls, const void* rope,
                           int64_t rs, const void* scales, int64_t rows, int64_t seq_capacity,
                           const int32_t* block_table, int32_t max_blocks, int32_t block_size,
                           const int32_t* lengths, int32_t max_len, int B, int H, const Plan& pl,
                           _Float16* part_h, float* part_scale, float* part_lse) {
  DecodeParams dp;
  dp.q = q;
  dp.latent = latent;
  dp.latent_stride = ls;
  dp.rope = rope;
  dp.rope_stride = rs;
  dp.scales = (const bf16*)scales;
  dp.rows = rows;
  dp.seq_capacity = seq_capacity;
  dp.block_table = block_table;
  dp.max_blocks = max_blocks;
  dp.block_size = block_size;
  dp.lengths = lengths;
  dp.max_len = max_len;
  dp.B = B;
  dp.H = H;
  dp.S = pl.S;
  dp.tokens_per_split = pl.TS;
  dp.G = pl.G;
  dp.items = nullptr;
  dp.nitems = 0;
  dp.part_o = part_h;
  dp.part_scale = part_scale;
  dp.part_lse = part_lse;
  return dp;
}

// Launch of the split attention kernel for the plan; with timing events, the
// launch itself records the kernel's start and end (the dispatch's own
// timestamps, not those of separate event packets).
mla_status launch_attention(const DecodeParams& dp, const Plan& pl, bool fp8,
                            const mla_decode_options* opts, hipStream_t stream) {
  const bool mma = fp8 && use_fp8mma(MLA_FP8_E4M3, pl, dp.block_table, dp.block_size);
  const int nq = pl.length_aware ? pl.nitems : dp.B * pl.S;
  const dim3 grid(ceil_div(nq, 8) * 8 * pl.G);
  hipEvent_t ev0 = opts ? opts->attn_begin : nullptr, ev1 = opts ? opts->attn_end : nullptr;
  auto launch = [&](auto kern, int threads) {
    if (ev0 || ev1)
      hipExtLaunchKernelGGL(kern, grid, dim3(threads), 0, stream, ev0, ev1, 0, dp);
    else
      hipLaunchKernelGGL(kern, grid, dim3(threads), 0, stream, dp);
  };
  if (mma) {
    launch(mla_decode_fp8mma_kernel, 256);
    return launch_status();
  }
  switch (pl.NW * 2 + (fp8 ? 1 : 0)) {
    case 8: launch(mla_decode_bf16_kernel<4>, 256); break;
    case 9: launch(mla_decode_fp8_kernel<4>, 256); break;
    case 4: launch(mla_decode_bf16_kernel<2>, 128); break;
    case 5: launch(mla_decode_fp8_kernel<2>, 128); break;
    case 2: launch(mla_decode_bf16_kernel<1>, 64); break;
    case 3: launch(mla_decode_fp8_kernel<1>, 64); break;
    default: return MLA_ERR_UNSUPPORTED;
  }
  return launch_status();
}

// Split-K plan of a weight-streaming GEMM (M x K) . (N x K)^T: enough
// workgroups (32-column tiles x K slices x batch groups of 128) to cover the
// chip several times; every slice non-empty.
struct SkPlan {
  int S, cps, mgroups, msub;
};

SkPlan skinny_plan(int M, int N, int K) {
  SkPlan pl;
  const int nchunks = K / SG_CHUNK;
  pl.mgroups = ceil_div(M, SG_MG);
  pl.msub = pl.mgroups > 1 ? 4 : ceil_div(M, 32);
  const int tiles = (N / 32) * pl.mgroups;
  int S = std::max(1, std::min(ceil_div(1024, tiles), nchunks));
  pl.cps = ceil_div(nchunks, S);
  pl.S = ceil_div(nchunks, pl.cps);
  return pl;
}

void launch_skinny(const SkinnyParams& sp, const SkPlan& pl, hipStream_t stream) {
  const dim3 grid((unsigned)((sp.N / 32) * pl.S * pl.mgroups));
  switch (pl.msub) {
    case 1: hipLaunchKernelGGL(mla_skinny_gemm_kernel<1>, grid, dim3(256), 0, stream, sp); break;
    case 2: hipLaunchKernelGGL(mla_skinny_gemm_kernel<2>, grid, dim3(256), 0, stream, sp); break;
    case 3: hipLaunchKernelGGL(mla_skinny_gemm_kernel<3>, grid, dim3(256), 0, stream, sp); break;
    default: hipLaunchKernelGGL(mla_skinny_gemm_kernel<4>, grid, dim3(256), 0, stream, sp); break;
  }
}

// Workspace of mla_decode_fused: that of the decode (queries, split
// partials) followed by the query GEMM's partials [Sq, B, 512 H] fp32, the
// merged latent rows [B, 512 H] bf16 and the output GEMM's partials
// [So, B, d_model] fp32.
struct FusedWs {
  WsLayout dec;
  SkPlan qp, op;
  size_t qpart, olat, opart, total;
};

FusedWs fused_ws(int B, int H, int D, const Plan& pl) {
  FusedWs f;
  f.dec = ws_layout(B, H, pl, MLA_BF16);
  f.qp = skinny_plan(B, H * D_C, D);
  f.op = skinny_plan(B, D, H * D_C);
  f.qpart = f.dec.total;
  f.olat = align_up(f.qpart + (size_t)f.qp.S * B * H * D_C * 4, 256);
  f.opart = align_up(f.olat + (size_t)B * H * D_C * 2, 256);
  f.total = align_up(f.opart + (size_t)f.op.S * B * D * 4, 256);
  return f;
}

mla_status run_decode(const mla_dims* dims, const void* q_nope, const void* q_pe,
                      const void* w_uk, const void* w_uv, mla_dtype act, const void* latent,
                      int64_t ls, const void* rope, int64_t rs, const void* scales,
                      mla_dtype cdt, int64_t rows, int64_t seq_capacity,
                      const int32_t* block_table, int32_t max_blocks, int32_t block_size,
                      const int32_t* lengths, int32_t batch, int32_t max_len,
                      float softmax_scale, void* out, float* lse, void* workspace,
                      size_t workspace_bytes, const mla_decode_options* opts,
                      hipStream_t stream) {
  const int B = batch, H = dims->heads;
  AppendParams app;
  const bool do_append = opts && opts->append;
  if (do_append) {
    const mla_append_args* a = opts->append;
    // rows from a down-projection's workspace: its partials stand in for the
    // inputs in the checks, and the row values are their sums
    const void* ci = a->projected ? a->projected : a->c_kv;
    const void* ki = a->projected ? a->projected : a->k_pe;
    const mla_dtype in_dt = a->projected ? MLA_F32 : a->in_dtype;
    MLA_TRY(check_append(dims, ci, ki, in_dt, a->positions, batch, const_cast<void*>(latent), ls,
                         const_cast<void*>(rope), rs, const_cast<void*>(scales), cdt, rows,
                         seq_capacity, block_table, max_blocks, block_size, a->rope_theta, &app));
    if (a->projected) {
      if (a->d_model <= 0 || a->d_model % PJ_CHUNK != 0) return MLA_ERR_INVALID_ARG;
      app.part = (const float*)a->projected;
      app.part_slices = project_plan(batch, a->d_model).S;
    }
  }
  Plan pl = decode_plan(B, H, max_len, act, cdt, block_table, block_size, opts);
  apply_length_aware(pl, B, act, cdt, opts);
  const WsLayout wl = ws_layout(B, H, pl, act);
  if (!workspace || workspace_bytes < wl.total || ((uintptr_t)workspace & 255) != 0)
    return MLA_ERR_WORKSPACE;
  if (do_append && opts->append->projected) {
    // the partial sums must all be there (their slice count follows from
    // batch and d_model), and must not share bytes with the workspace, whose
    // absorbed queries are written in the launch that reads the sums
    const mla_append_args* a = opts->append;
    if (a->projected_bytes < project_ws_bytes(batch, a->d_model)) return MLA_ERR_WORKSPACE;
    const uintptr_t p0 = (uintptr_t)a->projected, p1 = p0 + a->projected_bytes;
    const uintptr_t w0 = (uintptr_t)workspace, w1 = w0 + wl.total;
    if (p0 < w1 && w0 < p1) return MLA_ERR_WORKSPACE;
  }
  char* ws = (char*)workspace;
  float* part_o = (float*)(ws + wl.po_off);           // fp32 path
  _Float16* part_h = (_Float16*)(ws + wl.po_off);     // bf16 path
  float* part_scale = (float*)(ws + wl.ps_off);
  float* part_lse = (float*)(ws + wl.pl_off);
  // 0 selects 1/sqrt(key width), the key being [k_nope | k_pe]
  if (softmax_scale == 0.f) softmax_scale = 1.0f / std::sqrt((float)(D_N + D_R));
  const float c = softmax_scale * LOG2E;
  (void)hipGetLastError();  // start from a clean launch-error state

  if (act == MLA_F32) {
    if (do_append) {
      hipLaunchKernelGGL(mla_append_kernel, dim3(B), dim3(64), 0, stream, app);
      MLA_TRY(launch_status());
    }
    float* q = (float*)(ws + wl.q_off);
    hipLaunchKernelGGL(mla_absorb_f32_kernel, dim3(4 * B * H), dim3(256), 0, stream,
                       (const float*)q_nope, (const float*)q_pe, (const float*)w_uk, q, H, c);
    MLA_TRY(launch_status());
    DecodeF32Params dp;
    dp.q = q;
    dp.latent = (const float*)latent;
    dp.latent_stride = ls;
    dp.rope = (const float*)rope;
    dp.rope_stride = rs;
    dp.rows = rows;
    dp.seq_capacity = seq_capacity;
    dp.block_table = block_table;
    dp.max_blocks = max_blocks;
    dp.block_size = block_size;
    dp.lengths = lengths;
    dp.max_len = max_len;
    dp.B = B;
    dp.H = H;
    dp.S = pl.S;
    dp.tokens_per_split = pl.TS;
    dp.part_o = part_o;
    dp.part_lse = part_lse;
    if (opts && opts->attn_begin) (void)hipEventRecord(opts->attn_begin, stream);
    hipLaunchKernelGGL(mla_decode_f32_kernel, dim3(B * H * pl.S), dim3(256), 0, stream, dp);
    MLA_TRY(launch_status());
    if (opts && opts->attn_end) (void)hipEventRecord(opts->attn_end, stream);
    hipLaunchKernelGGL(mla_combine_f32_kernel, dim3(4 * B * H), dim3(256), 0, stream, part_o,
                       part_lse, (const float*)w_uv, (float*)out, lse, H, pl.S);
    return launch_status();
  }

  bf16* q = (bf16*)(ws + wl.q_off);
  const int nbc = ceil_div(B, 32);
  AbsorbParams ap{(const bf16*)q_nope, (const bf16*)q_pe, (const bf16*)w_uk, q, B, H, nbc, c, {}};
  DecodeParams dp = decode_params(q, latent, ls, rope, rs, scales, rows, seq_capacity,
                                  block_table, max_blocks, block_size, lengths, max_len, B, H, pl,
                                  part_h, part_scale, part_lse);
  int32_t* nsplit = nullptr;
  if (pl.length_aware) {
    // one extra workgroup of the absorb launch makes the plan; it reads only
    // the lengths, which the append of the same launch does not touch
    SplitItem* items = (SplitItem*)(ws + wl.items_off);
    nsplit = (int32_t*)(ws + wl.nsplit_off);
    ap.plan = BalanceParams{lengths, B, max_len, pl.nitems, pl.S, pl.TS, items, nsplit};
    dp.items = items;
    dp.nitems = pl.nitems;
  }
  const int absorb_blocks = plan_blocks(pl.length_aware) + ceil_div(H, 32) * 128;
  if (do_append)
    hipLaunchKernelGGL(mla_absorb_append_kernel, dim3(append_blocks(B) + absorb_blocks), dim3(256),
                       0, stream, ap, app);
  else
    hipLaunchKernelGGL(mla_absorb_kernel, dim3(absorb_blocks), dim3(256), 0, stream, ap);
  MLA_TRY(launch_status());
  MLA_TRY(launch_attention(dp, pl, cdt == MLA_FP8_E4M3, opts, stream));

  CombineParams cp{part_h, part_scale, part_lse, (const bf16*)w_uv, (bf16*)out, lse, B, H, pl.S, nbc,
                   pl.S, 1, nullptr};
  const dim3 cgrid(ceil_div(H, 8) * 8 * nbc);
  if (pl.length_aware) {
    // one level over the slots each sequence filled: up to 8 per row in
    // registers, more through the general merge
    cp.nsplit = nsplit;
    if (pl.S <= 2 * CB_G) {
      launch_short_merge<2 * CB_G>(cp, cgrid, stream);
    } else {
      hipLaunchKernelGGL(mla_combine_kernel, cgrid, dim3(CB_THREADS), 0, stream, cp);
    }
    return launch_status();
  }
  auto launch_s4 = [&]() { launch_short_merge<CB_G>(cp, cgrid, stream); };
  if (pl.S <= CB_G) {
    launch_s4();
    return launch_status();
  }
  // 5-8 partials per row: one launch of the row merge with 8 slots (which
  // issues no load past the row's count); MLA_MERGE8=0, or a merge grouping
  // asked for with MLA_MERGE_GROUPS, selects the paths below
  if (pl.S <= 2 * CB_G && env_int_or("MLA_MERGE8", 1) != 0 && !std::getenv("MLA_MERGE_GROUPS")) {
    launch_short_merge<2 * CB_G>(cp, cgrid, stream);
    return launch_status();
  }
  const int ng = merge_groups(pl.S, nbc);
  if (ng == 0) {
    hipLaunchKernelGGL(mla_combine_kernel, cgrid, dim3(CB_THREADS), 0, stream, cp);
    return launch_status();
  }
  MergeSplitsParams mp{part_h, part_scale, part_lse, B, H, pl.S, ceil_div(pl.S, ng), 0};
  mp.NG = ceil_div(pl.S, mp.G);
  const dim3 mgrid((unsigned)ceil_div((int64_t)B * mp.NG * H, MS_WAVES));
  if (mp.G <= 4)
    hipLaunchKernelGGL(mla_merge_splits_kernel<4>, mgrid, dim3(64 * MS_WAVES), 0, stream, mp);
  else if (mp.G <= 8)
    hipLaunchKernelGGL(mla_merge_splits_kernel<8>, mgrid, dim3(64 * MS_WAVES), 0, stream, mp);
  else
    hipLaunchKernelGGL(mla_merge_splits_kernel<16>, mgrid, dim3(64 * MS_WAVES), 0, stream, mp);
  MLA_TRY(launch_status());
  cp.S = mp.NG;
  cp.ss = mp.G;
  launch_s4();
  return launch_status();
}

}  // namespace

extern "C" {

mla_status mla_debug_errors(uint32_t* word, hipStream_t stream) {
  if (!word) return MLA_ERR_INVALID_ARG;
  *word = 0;
#if MLA_DEBUG_CHECKS
  void* dev_word = nullptr;
  if (hipGetSymbolAddress(&dev_word, HIP_SYMBOL(mla::g_debug_word)) != hipSuccess || !dev_word)
    return MLA_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return MLA_ERR_HIP;
  uint32_t v = 0;
  const uint32_t zero = 0;
  if (hipMemcpy(&v, dev_word, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return MLA_ERR_HIP;
  if (hipMemcpy(dev_word, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess)
    return MLA_ERR_HIP;
  *word = v;
  return MLA_OK;
#else
  (void)stream;
  return MLA_ERR_UNSUPPORTED;
#endif
}

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG: invalid argument";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: unsupported dims, dtype or layout";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: HIP launch failure";
  }
  return "MLA_ERR_UNKNOWN";
}

size_t mla_cache_bytes_per_token(mla_dtype cdt, int32_t d_c, int32_t d_rope) {
  if (d_c <= 0 || d_rope <= 0) return 0;
  const size_t e = elem_size(cdt);
  if (!e) return 0;
  return (size_t)(d_c + d_rope) * e + (cdt == MLA_FP8_E4M3 ? 2 : 0);
}

size_t mla_decode_workspace_size(const mla_dims* dims, int32_t batch, int32_t max_len,
                                 mla_dtype act, mla_dtype cdt, const mla_decode_options* opts) {
  if (!dims_supported(dims) || batch < 0 || max_len < 0) return 0;
  if (act != MLA_F32 && act != MLA_BF16) return 0;
  if (batch == 0) return 256;
  Plan pl = make_plan(batch, dims->heads, max_len, act, opts);
  apply_length_aware(pl, batch, act, cdt, opts);
  return ws_layout(batch, dims->heads, pl, act).total;
}

mla_status mla_decode(const mla_dims* dims, const void* q_nope, const void* q_pe,
                      const void* w_uk, const void* w_uv, mla_dtype act, const void* latent,
                      int64_t ls, const void* rope, int64_t rs, const void* scales,
                      mla_dtype cdt, int64_t rows, int64_t seq_capacity, const int32_t* lengths,
                      int32_t batch, int32_t max_len, float softmax_scale, void* out,
                      float* lse, void* workspace, size_t workspace_bytes,
                      const mla_decode_options* opts, hipStream_t stream) {
  MLA_TRY(check_decode(dims, q_nope, q_pe, w_uk, w_uv, act, latent, ls, rope, rs, scales, cdt,
                       rows, lengths, batch, max_len, softmax_scale, out));
  if (batch == 0) return MLA_OK;
  if (seq_capacity < max_len || seq_capacity < 1 || (int64_t)batch * seq_capacity > rows)
    return MLA_ERR_INVALID_ARG;
  return run_decode(dims, q_nope, q_pe, w_uk, w_uv, act, latent, ls, rope, rs, scales, cdt, rows,
                    seq_capacity, nullptr, 0, TILE, lengths, batch, max_len, softmax_scale, out,
                    lse, workspace, workspace_bytes, opts, stream);
}

mla_status mla_decode_paged(const mla_dims* dims, const void* q_nope, const void* q_pe,
                            const void* w_uk, const void* w_uv, mla_dtype act,
                            const void* latent, int64_t ls, const void* rope, int64_t rs,
                            const void* scales, mla_dtype cdt, int64_t rows,
                            const int32_t* block_table, int32_t max_blocks, int32_t block_size,
                            const int32_t* lengths, int32_t batch, int32_t max_len,
                            float softmax_scale, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, const mla_decode_options* opts,
                            hipStream_t stream) {
  MLA_TRY(check_decode(dims, q_nope, q_pe, w_uk, w_uv, act, latent, ls, rope, rs, scales, cdt,
                       rows, lengths, batch, max_len, softmax_scale, out));
  if (batch == 0) return MLA_OK;
  if (!block_table || block_size <= 0 || block_size % TILE != 0 || max_blocks <= 0 ||
      (int64_t)max_blocks * block_size < max_len || rows < block_size)
    return MLA_ERR_INVALID_ARG;
  return run_decode(dims, q_nope, q_pe, w_uk, w_uv, act, latent, ls, rope, rs, scales, cdt, rows,
                    0, block_table, max_blocks, block_size, lengths, batch, max_len,
                    softmax_scale, out, lse, workspace, workspace_bytes, opts, stream);
}

mla_status mla_decode_paged_noalloc(const mla_dims* dims, const void* q_nope, const void* q_pe,
                                    const void* w_uk, const void* w_uv, mla_dtype act,
                                    const void* latent, int64_t ls, const void* rope, int64_t rs,
                                    const void* scales, mla_dtype cdt, int64_t rows,
                                    const int32_t* block_table, int32_t max_blocks,
                                    int32_t block_size, const int32_t* lengths, int32_t batch,
                                    int32_t max_len, float softmax_scale, void* out, float* lse,
                                    const mla_decode_options* opts, hipStream_t stream) {
  MLA_TRY(check_decode(dims, q_nope, q_pe, w_uk, w_uv, act, latent, ls, rope, rs, scales, cdt,
                       rows, lengths, batch, max_len, softmax_scale, out));
  if (batch == 0) return MLA_OK;
  if (!block_table || block_size <= 0 || block_size % TILE != 0 || max_blocks <= 0 ||
      (int64_t)max_blocks * block_size < max_len || rows < block_size)
    return MLA_ERR_INVALID_ARG;
  // the scratch this call needs, before touching the device's copy
  Plan npl = make_plan(batch, dims->heads, max_len, act, opts);
  apply_length_aware(npl, batch, act, cdt, opts);
  const size_t need = ws_layout(batch, dims->heads, npl, act).total;
  if (need > kScratchBytes) return MLA_ERR_WORKSPACE;
  void* ws = nullptr;
  MLA_TRY(scratch_address(&ws));
  return run_decode(dims, q_nope, q_pe, w_uk, w_uv, act, latent, ls, rope, rs, scales, cdt, rows,
                    0, block_table, max_blocks, block_size, lengths, batch, max_len,
                    softmax_scale, out, lse, ws, kScratchBytes, opts, stream);
}

size_t mla_prefill_workspace_size(const mla_dims* dims, int32_t batch, int32_t max_len) {
  if (!dims_supported(dims) || batch < 0 || max_len < 0 || max_len > (1 << 30)) return 0;
  if (batch == 0 || max_len == 0) return 256;
  return prefill_ws(batch, dims->heads, max_len).total;
}

mla_status mla_prefill(const mla_dims* dims, const void* q_nope, const void* q_pe,
                       const void* w_uk, const void* w_uv, mla_dtype act, const void* latent,
                       int64_t ls, const void* rope, int64_t rs, mla_dtype cdt, int64_t rows,
                       int64_t seq_capacity, const int32_t* block_table, int32_t max_blocks,
                       int32_t block_size, const int32_t* lengths, int32_t batch, int32_t chunk,
                       int32_t max_len, float softmax_scale, void* out, float* lse,
                       void* workspace, size_t workspace_bytes, const mla_prefill_options* opts,
                       hipStream_t stream) {
  if (!dims) return MLA_ERR_INVALID_ARG;
  if (batch < 0 || chunk < 0 || max_len < 0 || max_len > (1 << 30)) return MLA_ERR_INVALID_ARG;
  if (!std::isfinite(softmax_scale)) return MLA_ERR_INVALID_ARG;
  if (!dims_supported(dims)) return MLA_ERR_UNSUPPORTED;
  if (act != MLA_BF16 || cdt != MLA_BF16) return MLA_ERR_UNSUPPORTED;
  if (dims->heads % 32 != 0) return MLA_ERR_UNSUPPORTED;
  if (batch == 0 || chunk == 0) return MLA_OK;
  if (chunk > max_len) return MLA_ERR_INVALID_ARG;
  if (!q_nope || !q_pe || !w_uk || !w_uv || !latent || !rope || !lengths || !out)
    return MLA_ERR_INVALID_ARG;
  if (ls < D_C || rs < D_R || rows < 1 || rows > INT32_MAX) return MLA_ERR_INVALID_ARG;
  if (!aligned16(latent) || !aligned16(rope) || (ls * 2) % 16 != 0 || (rs * 2) % 16 != 0)
    return MLA_ERR_INVALID_ARG;
  if (((uintptr_t)q_nope | (uintptr_t)q_pe | (uintptr_t)w_uk | (uintptr_t)w_uv |
       (uintptr_t)out) % 16 != 0)
    return MLA_ERR_INVALID_ARG;
  if (block_table) {
    if (block_size <= 0 || block_size % TILE != 0 || max_blocks <= 0 ||
        (int64_t)max_blocks * block_size < max_len || rows < block_size)
      return MLA_ERR_INVALID_ARG;
  } else {
    if (seq_capacity < max_len || seq_capacity < 1 || (int64_t)batch * seq_capacity > rows)
      return MLA_ERR_INVALID_ARG;
  }
  const int B = batch, H = dims->heads;
  const PrefillWs wl = prefill_ws(B, H, max_len);
  if (!workspace || workspace_bytes < wl.total || ((uintptr_t)workspace & 255) != 0)
    return MLA_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  if (softmax_scale == 0.f) softmax_scale = 1.0f / std::sqrt((float)(D_N + D_R));
  (void)hipGetLastError();

  bf16* wuvt = (bf16*)(ws + wl.wuvt);
  hipLaunchKernelGGL(mla_wuv_transpose_kernel, dim3(H * 16), dim3(256), 0, stream,
                     (const bf16*)w_uv, wuvt, H);
  MLA_TRY(launch_status());

  ExpandParams ep;
  ep.latent = (const bf16*)latent;
  ep.latent_stride = ls;
  ep.rope = (const bf16*)rope;
  ep.rope_stride = rs;
  ep.rows = rows;
  ep.seq_capacity = seq_capacity;
  ep.block_table = block_table;
  ep.max_blocks = max_blocks;
  ep.block_size = block_size;
  ep.lengths = lengths;
  ep.w_uk = (const bf16*)w_uk;
  ep.w_uvt = wuvt;
  ep.kx = (_Float16*)(ws + wl.kx);
  ep.vx = (_Float16*)(ws + wl.vx);
  ep.kpx = (_Float16*)(ws + wl.kpx);
  ep.B = B;
  ep.H = H;
  ep.cap = wl.cap;
  ep.max_len = max_len;
  const int ntile = ceil_div(max_len, EX_ROWS);
  const dim3 egrid((unsigned)((int64_t)8 * (H / 8) * B * ntile));
  hipEvent_t e0 = opts ? opts->expand_begin : nullptr, e1 = opts ? opts->expand_end : nullptr;
  if (e0 || e1)
    hipExtLaunchKernelGGL(mla_prefill_expand_kernel, egrid, dim3(256), 0, stream, e0, e1, 0, ep);
  else
    hipLaunchKernelGGL(mla_prefill_expand_kernel, egrid, dim3(256), 0, stream, ep);
  MLA_TRY(launch_status());

  PrefillParams pp;
  pp.q_nope = (const bf16*)q_nope;
  pp.q_pe = (const bf16*)q_pe;
  pp.kx = ep.kx;
  pp.vx = ep.vx;
  pp.kpx = ep.kpx;
  pp.lengths = lengths;
  pp.B = B;
  pp.H = H;
  pp.T = chunk;
  pp.cap = wl.cap;
  pp.max_len = max_len;
  pp.c = softmax_scale * LOG2E;
  pp.out = (bf16*)out;
  pp.lse = lse;
  // longest query tiles first unless MLA_PREFILL_ORDER=0
  const char* oe = std::getenv("MLA_PREFILL_ORDER");
  pp.order = (oe && std::atoi(oe) == 0) ? 0 : 1;
  const int nqt = ceil_div(chunk, PF_Q);
  const dim3 agrid((unsigned)((int64_t)8 * ceil_div((int64_t)B * H, 8) * nqt));
  hipEvent_t a0 = opts ? opts->attn_begin : nullptr, a1 = opts ? opts->attn_end : nullptr;
  if (a0 || a1)
    hipExtLaunchKernelGGL(mla_prefill_attn_kernel, agrid, dim3(256), 0, stream, a0, a1, 0, pp);
  else
    hipLaunchKernelGGL(mla_prefill_attn_kernel, agrid, dim3(256), 0, stream, pp);
  return launch_status();
}

mla_status mla_fuse_weights(const mla_dims* dims, int32_t d_model, const void* w_q,
                            const void* w_uk, const void* w_uv, const void* w_o, mla_dtype act,
                            void* w_qk, void* w_vo, hipStream_t stream) {
  if (!dims) return MLA_ERR_INVALID_ARG;
  if (!dims_supported(dims)) return MLA_ERR_UNSUPPORTED;
  if (act != MLA_BF16) return MLA_ERR_UNSUPPORTED;
  if (d_model <= 0 || d_model % 64 != 0) return MLA_ERR_INVALID_ARG;
  if (!w_q || !w_uk || !w_uv || !w_o || !w_qk || !w_vo) return MLA_ERR_INVALID_ARG;
  const int H = dims->heads, D = d_model;
  (void)hipGetLastError();
  const int per_head = (D_C / 64) * (D / 64);
  // W_QK[h][c][k] = sum_j W_UK[h][j][c] W_Q[h][j][k]
  FuseParams fq{(const bf16*)w_uk, D_C, 1, (int64_t)D_N * D_C,
                (const bf16*)w_q, D, 1, (int64_t)D_N * D,
                (bf16*)w_qk, D, 1, (int64_t)D_C * D, D_C, D, H};
  hipLaunchKernelGGL(mla_fuse_weights_kernel, dim3(H * per_head), dim3(256), 0, stream, fq);
  MLA_TRY(launch_status());
  // W_VO stored [d_model][512 H]: entry (n, 512 h + c) = sum_j W_UV[h][c][j] W_O[h][j][n]
  FuseParams fo{(const bf16*)w_uv, 1, D_V, (int64_t)D_C * D_V,
                (const bf16*)w_o, D, 1, (int64_t)D_V * D,
                (bf16*)w_vo, 1, (int64_t)H * D_C, D_C, D_C, D, H};
  hipLaunchKernelGGL(mla_fuse_weights_kernel, dim3(H * per_head), dim3(256), 0, stream, fo);
  return launch_status();
}

size_t mla_decode_fused_workspace_size(const mla_dims* dims, int32_t batch, int32_t max_len,
                                       int32_t d_model, const mla_decode_options* opts) {
  if (!dims_supported(dims) || batch < 0 || max_len < 0 || d_model <= 0 || d_model % 64 != 0)
    return 0;
  if (batch == 0) return 256;
  const Plan pl = make_plan(batch, dims->heads, max_len, MLA_BF16, opts);
  return fused_ws(batch, dims->heads, d_model, pl).total;
}

mla_status mla_decode_fused(const mla_dims* dims, const void* x, const void* q_pe,
                            const void* w_qk, const void* w_vo, int32_t d_model, mla_dtype act,
                            const void* latent, int64_t ls, const void* rope, int64_t rs,
                            const void* scales, mla_dtype cdt, int64_t rows, int64_t seq_capacity,
                            const int32_t* block_table, int32_t max_blocks, int32_t block_size,
                            const int32_t* lengths, int32_t batch, int32_t max_len,
                            float softmax_scale, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, const mla_decode_options* opts,
                            hipStream_t stream) {
  // the decode's own checks (x and the fused weights stand in for the
  // query and weight arguments), then those of the fused form
  MLA_TRY(check_decode(dims, x, q_pe, w_qk, w_vo, act, latent, ls, rope, rs, scales, cdt, rows,
                       lengths, batch, max_len, softmax_scale, out));
  if (act != MLA_BF16) return MLA_ERR_UNSUPPORTED;
  if (opts && opts->append) return MLA_ERR_UNSUPPORTED;
  if (d_model <= 0 || d_model % 64 != 0) return MLA_ERR_INVALID_ARG;
  if (batch == 0) return MLA_OK;
  if (block_table) {
    if (block_size <= 0 || block_size % TILE != 0 || max_blocks <= 0 ||
        (int64_t)max_blocks * block_size < max_len || rows < block_size)
      return MLA_ERR_INVALID_ARG;
  } else {
    if (seq_capacity < max_len || seq_capacity < 1 || (int64_t)batch * seq_capacity > rows)
      return MLA_ERR_INVALID_ARG;
  }
  const int B = batch, H = dims->heads, D = d_model;
  const Plan pl = decode_plan(B, H, max_len, MLA_BF16, cdt, block_table, block_size, opts);
  const FusedWs fw = fused_ws(B, H, D, pl);
  if (!workspace || workspace_bytes < fw.total || ((uintptr_t)workspace & 255) != 0)
    return MLA_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  if (softmax_scale == 0.f) softmax_scale = 1.0f / std::sqrt((float)(D_N + D_R));
  (void)hipGetLastError();
  bf16* q = (bf16*)(ws + fw.dec.q_off);
  float* qpart = (float*)(ws + fw.qpart);
  bf16* olat = (bf16*)(ws + fw.olat);
  float* opart = (float*)(ws + fw.opart);
  // 1. q_lat = W_QK[h] x for every head: [B, D] x [512 H, D]^T
  SkinnyParams sq{(const bf16*)x, (const bf16*)w_qk, qpart, D, D, B, H * D_C, D, fw.qp.S,
                  fw.qp.cps};
  launch_skinny(sq, fw.qp, stream);
  MLA_TRY(launch_status());
  const int64_t qpieces = (int64_t)B * H * 72;
  hipLaunchKernelGGL(mla_fused_q_finish_kernel, dim3((unsigned)ceil_div(qpieces, 256)), dim3(256),
                     0, stream, (const float*)qpart, fw.qp.S, (const bf16*)q_pe, q, B, H,
                     softmax_scale * LOG2E);
  MLA_TRY(launch_status());
  // 2. attention over the latent cache
  _Float16* part_h = (_Float16*)(ws + fw.dec.po_off);
  float* part_scale = (float*)(ws + fw.dec.ps_off);
  float* part_lse = (float*)(ws + fw.dec.pl_off);
  const DecodeParams dp = decode_params(q, latent, ls, rope, rs, scales, rows, seq_capacity,
                                        block_table, max_blocks, block_size, lengths, max_len, B,
                                        H, pl, part_h, part_scale, part_lse);
  MLA_TRY(launch_attention(dp, pl, cdt == MLA_FP8_E4M3, opts, stream));
  // 3. merged latent rows, then y = o_lat [B, 512 H] x W_VO^T [D, 512 H]^T
  hipLaunchKernelGGL(mla_merge_latent_kernel, dim3(B * H), dim3(128), 0, stream,
                     (const _Float16*)part_h, (const float*)part_scale, (const float*)part_lse,
                     olat, lse, B, H, pl.S);
  MLA_TRY(launch_status());
  SkinnyParams so{olat, (const bf16*)w_vo, opart, (int64_t)H * D_C, (int64_t)H * D_C, B, D,
                  H * D_C, fw.op.S, fw.op.cps};
  launch_skinny(so, fw.op, stream);
  MLA_TRY(launch_status());
  hipLaunchKernelGGL(mla_fused_out_finish_kernel, dim3((unsigned)ceil_div((int64_t)B * D, 1024)),
                     dim3(256), 0, stream, (const float*)opart, fw.op.S, (bf16*)out, B, D);
  return launch_status();
}

mla_status mla_cache_append(const mla_dims* dims, const void* c_kv, const void* k_pe,
                            mla_dtype in_dtype, const int32_t* positions, int32_t batch,
                            void* latent, int64_t ls, void* rope, int64_t rs, void* scales,
                            mla_dtype cdt, int64_t rows, int64_t seq_capacity,
                            const int32_t* block_table, int32_t max_blocks, int32_t block_size,
                            float rope_theta, hipStream_t stream) {
  AppendParams p;
  MLA_TRY(check_append(dims, c_kv, k_pe, in_dtype, positions, batch, latent, ls, rope, rs,
                       scales, cdt, rows, seq_capacity, block_table, max_blocks, block_size,
                       rope_theta, &p));
  if (batch == 0) return MLA_OK;
  (void)hipGetLastError();
  hipLaunchKernelGGL(mla_append_kernel, dim3(batch), dim3(64), 0, stream, p);
  return launch_status();
}

size_t mla_project_workspace_size(int32_t batch, int32_t d_model) {
  if (batch < 0 || d_model <= 0 || d_model % PJ_CHUNK != 0) return 0;
  if (batch == 0) return 256;
  return project_ws_bytes(batch, d_model);
}

mla_status mla_project(const mla_dims* dims, const void* hidden, const void* w_dkv,
                       const void* w_kr, mla_dtype act, int32_t d_model, int32_t batch,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!dims || batch < 0) return MLA_ERR_INVALID_ARG;
  if (!dims_supported(dims)) return MLA_ERR_UNSUPPORTED;
  if (act != MLA_F32 && act != MLA_BF16) return MLA_ERR_UNSUPPORTED;
  if (d_model <= 0 || d_model % PJ_CHUNK != 0) return MLA_ERR_INVALID_ARG;
  if (batch == 0) return MLA_OK;
  if (!hidden || !w_dkv || !w_kr || !aligned16(hidden) || !aligned16(w_dkv) || !aligned16(w_kr))
    return MLA_ERR_INVALID_ARG;
  if (!workspace || !aligned16(workspace) || workspace_bytes < project_ws_bytes(batch, d_model))
    return MLA_ERR_WORKSPACE;
  const ProjPlan pl = project_plan(batch, d_model);
  ProjectParams pp;
  pp.h = hidden;
  pp.w_dkv = w_dkv;
  pp.w_kr = w_kr;
  pp.part = (float*)workspace;
  pp.B = batch;
  pp.D = d_model;
  pp.S = pl.S;
  pp.cps = pl.cps;
  (void)hipGetLastError();
  const int grid = PJ_NTILES * pl.S * pl.mgroups;
  if (act == MLA_BF16)
    launch_project<bf16>(pp, pl.msub, grid, stream);
  else
    launch_project<float>(pp, pl.msub, grid, stream);
  return launch_status();
}

mla_status mla_project_append(const mla_dims* dims, const void* hidden, const void* w_dkv,
                              const void* w_kr, mla_dtype act, int32_t d_model,
                              const int32_t* positions, int32_t batch, void* latent, int64_t ls,
                              void* rope, int64_t rs, void* scales, mla_dtype cdt, int64_t rows,
                              int64_t seq_capacity, const int32_t* block_table,
                              int32_t max_blocks, int32_t block_size, float rope_theta,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  AppendParams a;
  // the append's own checks (the hidden state stands in for its inputs)
  MLA_TRY(check_append(dims, hidden, hidden, act, positions, batch, latent, ls, rope, rs, scales,
                       cdt, rows, seq_capacity, block_table, max_blocks, block_size, rope_theta,
                       &a));
  if (d_model <= 0 || d_model % PJ_CHUNK != 0) return MLA_ERR_INVALID_ARG;
  if (batch == 0) return MLA_OK;
  if (!w_dkv || !w_kr || !aligned16(hidden) || !aligned16(w_dkv) || !aligned16(w_kr))
    return MLA_ERR_INVALID_ARG;
  const ProjPlan pl = project_plan(batch, d_model);
  if (!workspace || !aligned16(workspace) || workspace_bytes < project_ws_bytes(batch, d_model))
    return MLA_ERR_WORKSPACE;
  a.c_kv = nullptr;
  a.k_pe = nullptr;
  ProjectParams pp;
  pp.h = hidden;
  pp.w_dkv = w_dkv;
  pp.w_kr = w_kr;
  pp.part = (float*)workspace;
  pp.B = batch;
  pp.D = d_model;
  pp.S = pl.S;
  pp.cps = pl.cps;
  const int grid = PJ_NTILES * pl.S * pl.mgroups;
  (void)hipGetLastError();
  if (act == MLA_BF16)
    launch_project<bf16>(pp, pl.msub, grid, stream);
  else
    launch_project<float>(pp, pl.msub, grid, stream);
  hipLaunchKernelGGL(mla_project_append_kernel, dim3(batch), dim3(256), 0, stream,
                     (const float*)workspace, pl.S, batch, a);
  return launch_status();
}

}  // extern "C"
