// C ABI of the MLA decode library: argument validation, split planning and
// kernel launches on the caller's stream. See include/mla.h for the contract.
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>

#include <hip/hip_ext.h>

#include "mla.h"
#include "append.hpp"
#include "decode_mfma.hpp"
#include "fp32_path.hpp"
#include "kv_project.hpp"
#include "project_mfma.hpp"

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
};

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

Plan make_plan(int B, int H, int max_len, mla_dtype act, const mla_decode_options* opts) {
  Plan pl;
  const int cus = device_cu_count();
  const int len = max_len > 0 ? max_len : 1;
  int S;
  if (act == MLA_F32) {
    pl.NW = 0;
    pl.G = 1;
    const int min_tok = 128;
    S = std::max(ceil_div(len, F32_MAX_SPLIT),
                 std::min(ceil_div(cus, (int64_t)B * H), ceil_div(len, min_tok)));
  } else {
    const int hw = H / 32;
    pl.NW = (hw % 4 == 0) ? 4 : (hw % 2 == 0) ? 2 : 1;
    pl.G = hw / pl.NW;
    // one resident workgroup per CU; splits no shorter than 256 tokens
    const int groups = B * pl.G;
    S = std::min(ceil_div(cus, groups), ceil_div(len, 256));
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

// Workspace: absorbed queries [B, H, 576] (activation dtype), split partials
// [B, S, H, 512] (fp32 on the fp32 path; fp16 relative to a per-row fp32
// scale [B, S, H] otherwise), split lse [B, S, H] fp32.
struct WsLayout {
  size_t q_off, po_off, ps_off, pl_off, total;
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
  w.total = align_up(w.pl_off + rows * 4, 256);
  return w;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

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
  const size_t ae = elem_size(act);
  if (((uintptr_t)q_nope | (uintptr_t)q_pe | (uintptr_t)w_uk | (uintptr_t)w_uv | (uintptr_t)out) %
          16 != 0 &&
      ae == 2)
    return MLA_ERR_INVALID_ARG;
  return MLA_OK;
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
  const Plan pl = make_plan(B, H, max_len, act, opts);
  const WsLayout wl = ws_layout(B, H, pl, act);
  if (!workspace || workspace_bytes < wl.total || ((uintptr_t)workspace & 255) != 0)
    return MLA_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  float* part_o = (float*)(ws + wl.po_off);           // fp32 path
  _Float16* part_h = (_Float16*)(ws + wl.po_off);     // bf16 path
  float* part_scale = (float*)(ws + wl.ps_off);
  float* part_lse = (float*)(ws + wl.pl_off);
  const float c = softmax_scale * LOG2E;
  (void)hipGetLastError();  // start from a clean launch-error state

  if (act == MLA_F32) {
    if (do_append) {
      hipLaunchKernelGGL(mla_append_kernel, dim3(B), dim3(64), 0, stream, app);
      MLA_TRY(launch_status());
    }
    float* q = (float*)(ws + wl.q_off);
    hipLaunchKernelGGL(mla_absorb_f32_kernel, dim3(B * H), dim3(256), 0, stream,
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
    hipLaunchKernelGGL(mla_combine_f32_kernel, dim3(B * H), dim3(128), 0, stream, part_o,
                       part_lse, (const float*)w_uv, (float*)out, lse, H, pl.S);
    return launch_status();
  }

  bf16* q = (bf16*)(ws + wl.q_off);
  const int nbc = ceil_div(B, 32);
  AbsorbParams ap{(const bf16*)q_nope, (const bf16*)q_pe, (const bf16*)w_uk, q, B, H, nbc, c};
  const int absorb_blocks = ceil_div(H, 32) * 128;
  if (do_append)
    hipLaunchKernelGGL(mla_absorb_append_kernel, dim3(append_blocks(B) + absorb_blocks), dim3(256),
                       0, stream, ap, app);
  else
    hipLaunchKernelGGL(mla_absorb_kernel, dim3(absorb_blocks), dim3(256), 0, stream, ap);
  MLA_TRY(launch_status());

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
  dp.part_o = part_h;
  dp.part_scale = part_scale;
  dp.part_lse = part_lse;
  const int nq = B * pl.S;
  const dim3 grid(ceil_div(nq, 8) * 8 * pl.G);
  // with timing events, the launch itself records the kernel's start and end
  // (the dispatch's own timestamps, not those of separate event packets)
  hipEvent_t ev0 = opts ? opts->attn_begin : nullptr, ev1 = opts ? opts->attn_end : nullptr;
  auto launch = [&](auto kern, int threads) {
    if (ev0 || ev1)
      hipExtLaunchKernelGGL(kern, grid, dim3(threads), 0, stream, ev0, ev1, 0, dp);
    else
      hipLaunchKernelGGL(kern, grid, dim3(threads), 0, stream, dp);
  };
  const bool fp8 = (cdt == MLA_FP8_E4M3);
  switch (pl.NW * 2 + (fp8 ? 1 : 0)) {
    case 8: launch(mla_decode_bf16_kernel<4>, 256); break;
    case 9: launch(mla_decode_fp8_kernel<4>, 256); break;
    case 4: launch(mla_decode_bf16_kernel<2>, 128); break;
    case 5: launch(mla_decode_fp8_kernel<2>, 128); break;
    case 2: launch(mla_decode_bf16_kernel<1>, 64); break;
    case 3: launch(mla_decode_fp8_kernel<1>, 64); break;
    default: return MLA_ERR_UNSUPPORTED;
  }
  MLA_TRY(launch_status());

  CombineParams cp{part_h, part_scale, part_lse, (const bf16*)w_uv, (bf16*)out, lse, B, H, pl.S, nbc};
  hipLaunchKernelGGL(pl.S <= CB_G ? mla_combine_s4_kernel : mla_combine_kernel,
                     dim3(ceil_div(H, 8) * 8 * nbc), dim3(CB_THREADS), 0, stream, cp);
  return launch_status();
}

}  // namespace

extern "C" {

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
  (void)cdt;
  if (batch == 0) return 256;
  const Plan pl = make_plan(batch, dims->heads, max_len, act, opts);
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
