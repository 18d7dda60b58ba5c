/*
 * mla.h: C ABI of an MI355X (gfx950) library for Multi-Head Latent Attention
 * (MLA) decode over a compressed KV cache.
 *
 * The method (sources cited by page title and section):
 *   - "How DeepSeek Rewrote the Transformer [MLA]" (linuxpro, English
 *     edition), section "MLA: compress the pair, not the heads": each cached
 *     token is a 512-wide latent c_KV plus a 64-wide decoupled RoPE key k^R
 *     (576 numbers per token per layer, independent of the head count); the
 *     heads rebuild K and V from the latent; by associativity
 *     Q K^T = (Q W_UK^T) c^T, so W_UK is absorbed into the query and W_UV is
 *     applied after attention, and attention runs on the latent cache.
 *   - same page, section "Classic attention and the cost of the KV cache":
 *     softmax(Q K^T / sqrt(d_k) + M) V with a causal mask M; the new token
 *     appends its own K/V row and reads the whole history.
 *   - "DeepSeek AI efficiency, architecture, benchmarks" (technova-ai),
 *     section "Architectural Innovations: MLA": c_KV = W_DKV h_t,
 *     K = W_UK c_KV, V = W_UV c_KV.
 *
 * Shapes used throughout (the only ones supported): d_c = 512 (latent),
 * d_rope = 64 (RoPE key), d_nope = 128 (no-RoPE query/key), d_v = 128.
 *
 * Conventions
 *   - All pointers are DEVICE pointers unless stated; the caller owns every
 *     buffer. The library never allocates or frees device memory.
 *   - Calls are asynchronous on the given HIP stream; none synchronizes.
 *   - Host-visible arguments are validated before anything is launched: an
 *     invalid call returns an error status, launches nothing and leaves all
 *     outputs untouched. Launch failures return MLA_ERR_HIP.
 *   - Device-resident integers (lengths, positions, block tables) cannot be
 *     checked without a sync. Preconditions: 0 <= lengths[b] <= max_len,
 *     every block id read is in [0, cache_rows / block_size), positions are
 *     within the cache. Kernels clamp out-of-range values to stay inside the
 *     buffers (no fault), but the result of such a call is unspecified.
 *   - Strides are in ELEMENTS. Rows of the latent and RoPE arrays must start
 *     16-byte aligned (stride * element size a multiple of 16, pointers
 *     16-byte aligned). A packed 576-wide row (latent | RoPE key) is passed as
 *     latent = base, rope = base + 512, both with stride 576. The decode calls
 *     also need stride * element size below 2^24 bytes (MLA_ERR_UNSUPPORTED
 *     otherwise).
 *   - The library is stateless apart from a per-device cache of the compute
 *     unit count; all entry points are thread-safe. Calls that share a
 *     workspace must be ordered by the caller (same stream).
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1,  /* null pointer, bad size, misalignment */
  MLA_ERR_UNSUPPORTED = 2,  /* valid request outside what is implemented */
  MLA_ERR_WORKSPACE = 3,    /* workspace missing or too small */
  MLA_ERR_HIP = 4           /* a HIP call or kernel launch failed */
} mla_status;

typedef enum {
  MLA_F32 = 0,       /* IEEE binary32 */
  MLA_BF16 = 1,      /* bfloat16 */
  MLA_FP8_E4M3 = 2   /* OCP fp8 e4m3fn codes (cache only), one bf16 scale per row */
} mla_dtype;

/* Head count and per-head widths. Supported: d_c = 512, d_rope = 64,
 * d_nope = 128, d_v = 128; heads >= 1 for the f32 path, heads a multiple of
 * 32 for the bf16 / fp8-cache path. */
typedef struct {
  int32_t heads, d_c, d_rope, d_nope, d_v;
} mla_dims;

/* The arguments of mla_cache_append that a decode call does not already
 * carry (see mla_decode_options.append). */
typedef struct mla_append_args {
  const void* c_kv;           /* [batch, d_c] new latent rows, in_dtype */
  const void* k_pe;           /* [batch, d_rope] new RoPE keys, not yet rotated */
  mla_dtype in_dtype;         /* MLA_F32 or MLA_BF16 */
  const int32_t* positions;   /* [batch] 0-based position of each new token */
  float rope_theta;           /* RoPE base (10000 in the DeepSeek-V3 setting) */
  /* If non-NULL, c_kv, k_pe and in_dtype are ignored: the rows are those of
   * a preceding mla_project call on the same stream with the same batch and
   * d_model, whose workspace this is (the sums of its partial products).
   * The cache then receives exactly what mla_project_append would write.
   * projected_bytes must be at least mla_project_workspace_size(batch,
   * d_model), and [projected, projected + projected_bytes) must not overlap
   * the decode call's own workspace (the absorbed queries are written while
   * the append still reads the sums); either violation returns
   * MLA_ERR_WORKSPACE and launches nothing. */
  const void* projected;
  int32_t d_model;            /* with projected: its hidden width */
  size_t projected_bytes;     /* with projected: size of that buffer in bytes */
} mla_append_args;

/* Optional tuning and instrumentation for the decode calls (pass NULL for the
 * defaults). Zero fields mean "choose automatically".
 *   num_splits     number of token ranges each sequence is cut into (split-KV).
 *   length_aware   non-zero: on the bf16 cache, cut the sequences by their
 *                  actual lengths (read on the device) instead of by max_len:
 *                  the launch keeps its number of workgroups, and a split
 *                  length between half and all of the default one is chosen so
 *                  that the work items cover every sequence; long sequences
 *                  then get more splits than short ones (up to twice the
 *                  default count), so every workgroup has about the same
 *                  number of tokens. For batches of unequal lengths. Costs
 *                  one small planning launch; the workspace holds twice the
 *                  default split slots (query mla_decode_workspace_size with
 *                  the same options). Ignored for the f32 and fp8 caches,
 *                  by mla_decode_fused, and where the default plan has a
 *                  single split per sequence.
 *   attn_begin/end if non-NULL, HIP events that record the start and the end
 *                  of the split attention kernel on `stream` (bf16 / fp8
 *                  path: taken from the kernel's own dispatch; f32 path:
 *                  recorded immediately before and after it), for timing it. */
typedef struct {
  int32_t num_splits;
  int32_t length_aware;
  hipEvent_t attn_begin;
  hipEvent_t attn_end;
  /* If non-NULL, the call first writes the new tokens' rows into the cache,
   * with exactly the effect of mla_cache_append on the same cache arrays,
   * strides, scales and block table (which must then be writable), before
   * any of it is read. On the bf16 / fp8-cache path the append runs in the
   * same launch as the query absorption, saving a kernel launch per step.
   * Errors of the append arguments are those of mla_cache_append. */
  const mla_append_args* append;
} mla_decode_options;

/* Text for a status code (static storage; never NULL). */
const char* mla_status_string(mla_status status);

/* Bytes of cache per token per layer: 576 * element size, plus 2 bytes of
 * scale for the fp8 cache (1152 for bf16, 2304 for f32, 578 for fp8). This is
 * the MLA row of "How DeepSeek Rewrote the Transformer [MLA]", section
 * "MLA: compress the pair, not the heads" (576 numbers per token per layer).
 * Returns 0 for an unknown dtype or non-positive widths. */
size_t mla_cache_bytes_per_token(mla_dtype cache_dtype, int32_t d_c, int32_t d_rope);

/*
 * mla_cache_append: write the new token of every sequence into the cache.
 *
 * For each b in [0, batch): the latent c_kv[b, 0:512] is stored as is
 * (converted to the cache type with round-to-nearest-even), and the RoPE key
 * k_pe[b, 0:64] is rotated by its position p = positions[b] and stored:
 * interleaved pairs (x[2i], x[2i+1]) turn by angle p * rope_theta^(-2i/64),
 * p 0-based; the angle and its sine/cosine are computed in double precision,
 * the rotation is rounded to fp32, then to the cache type. (Source: the
 * decoupled RoPE key of "How DeepSeek Rewrote the Transformer [MLA]",
 * section "MLA: compress the pair, not the heads", cached beside the latent;
 * the pages name RoPE but give no formula, so this standard form is a
 * documented reading.)
 *
 * fp8 cache: the 576 values of the row (latent and rotated key, in fp32) get
 * one scale s = bf16_rne(amax / 448) (s = 1 if amax == 0; s = 2^-126 if
 * amax / 448 is below 2^-126), written to scales[row], and each value x is
 * stored as the e4m3fn code of x / s (fp32 division), rounded to nearest
 * even and saturated to +-448.
 *
 * Arguments
 *   c_kv       [batch, 512] in in_dtype (MLA_F32 or MLA_BF16), row stride 512
 *   k_pe       [batch, 64]  in in_dtype, un-rotated, row stride 64
 *   positions  [batch] int32 (device): 0-based position of the new token
 *   latent/rope/scales, strides: the cache arrays (scales: fp8 only, else NULL)
 *   cache_rows total rows of the cache arrays (bounds for the kernel)
 *   contiguous cache (block_table == NULL): row = b * seq_capacity + p
 *   paged cache: row = block_table[b * max_blocks_per_seq + p / block_size]
 *                * block_size + p % block_size
 *   rope_theta the RoPE base (10000 for the workloads here)
 * Errors: INVALID_ARG for null/misaligned pointers or bad sizes,
 * UNSUPPORTED for other dims/dtypes, HIP on launch failure. batch == 0 is a
 * valid no-op.
 */
mla_status mla_cache_append(const mla_dims* dims, const void* c_kv, const void* k_pe,
                            mla_dtype in_dtype, const int32_t* positions, int32_t batch,
                            void* latent, int64_t latent_stride, void* rope,
                            int64_t rope_stride, void* scales, mla_dtype cache_dtype,
                            int64_t cache_rows, int64_t seq_capacity,
                            const int32_t* block_table, int32_t max_blocks_per_seq,
                            int32_t block_size, float rope_theta, hipStream_t stream);

/*
 * mla_project_append: compute the new tokens' cache rows from their hidden
 * states and append them (the step before mla_cache_append, fused with it).
 *
 * For each b in [0, batch): c = W_DKV h[b] (the latent, 512 values) and
 * k = W_KR h[b] (the un-rotated RoPE key, 64 values), then the row is
 * stored exactly as mla_cache_append stores (c, k) at position positions[b]
 * (RoPE, rounding or fp8 quantisation, addressing). (Sources: the equation
 * c_KV = W_DKV h_t of "DeepSeek AI efficiency, architecture, benchmarks",
 * section "Architectural Innovations: Multi-Head Latent Attention (MLA)";
 * the diagram of "How DeepSeek Rewrote the Transformer [MLA]", section
 * "MLA: compress the pair, not the heads", where the input h_t yields both
 * the latent and the RoPE key. The pages name no bias and no normalisation
 * of c, so there is none.) The products are accumulated in fp32 (bf16 or
 * fp32 operands); the fp32 sums are the values handed to the append.
 *
 * Arguments
 *   hidden     [batch, d_model] in act_dtype (MLA_BF16 or MLA_F32), row stride
 *              d_model, 16-byte aligned
 *   w_dkv      [512, d_model] in act_dtype, row-major (row n gives latent n)
 *   w_kr       [64, d_model]  in act_dtype, row-major (row n gives key n)
 *   d_model    hidden width: a positive multiple of 64 (7168 in the
 *              DeepSeek-V3 setting)
 *   positions .. rope_theta: as for mla_cache_append
 *   workspace  device scratch of at least mla_project_workspace_size(batch,
 *              d_model) bytes, 16-byte aligned (fp32 partial sums); its
 *              contents on entry do not matter
 * Errors: those of mla_cache_append; INVALID_ARG for a d_model that is not a
 * positive multiple of 64 or null/misaligned weights; WORKSPACE for a
 * missing, misaligned or small workspace. batch == 0 is a valid no-op.
 * Two launches on `stream`; the result does not depend on timing (fixed
 * summation order).
 */
mla_status mla_project_append(const mla_dims* dims, const void* hidden, const void* w_dkv,
                              const void* w_kr, mla_dtype act_dtype, int32_t d_model,
                              const int32_t* positions, int32_t batch, void* latent,
                              int64_t latent_stride, void* rope, int64_t rope_stride,
                              void* scales, mla_dtype cache_dtype, int64_t cache_rows,
                              int64_t seq_capacity, const int32_t* block_table,
                              int32_t max_blocks_per_seq, int32_t block_size, float rope_theta,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mla_project: the first half of mla_project_append alone. It leaves the
 * new rows' products, as partial sums, in `workspace` for the append of a
 * following decode call (mla_append_args.projected), so a decode step runs
 * the down-projection, the append, the absorption and the attention in
 * four launches without a launch of its own for the append. Arguments,
 * sizes and errors as for mla_project_append (the same workspace size).
 */
mla_status mla_project(const mla_dims* dims, const void* hidden, const void* w_dkv,
                       const void* w_kr, mla_dtype act_dtype, int32_t d_model, int32_t batch,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes needed by mla_project_append and mla_project (0 on invalid
 * sizes). */
size_t mla_project_workspace_size(int32_t batch, int32_t d_model);

/* Workspace bytes needed by mla_decode / mla_decode_paged for these sizes
 * (absorbed queries, split partials). 0 on invalid arguments. The split plan
 * depends on the current device's compute-unit count, so query it on the
 * device that will run the decode, with the same options. */
size_t mla_decode_workspace_size(const mla_dims* dims, int32_t batch, int32_t max_len,
                                 mla_dtype act_dtype, mla_dtype cache_dtype,
                                 const mla_decode_options* opts);

/*
 * mla_decode: one decode step of MLA attention for `batch` sequences over a
 * contiguous cache (sequence b owns rows [b*seq_capacity, b*seq_capacity +
 * lengths[b])). (Sources: "How DeepSeek Rewrote the Transformer [MLA]",
 * section "MLA: compress the pair, not the heads": the query absorbs W_UK,
 * every head scores against and mixes the shared latent rows, W_UV is
 * applied after attention; section "Classic attention and the cost of the
 * KV cache": softmax attention of the new token over the cached rows, the
 * causal mask being the length mask for a single query.)
 *
 * For every sequence b and head h, with N = lengths[b] (the causal length,
 * counting the current token once it has been appended):
 *   q_lat        = q_nope[b,h,:] . W_UK[h]                  (absorbed query)
 *   s_t          = softmax_scale * (q_lat . c_t + q_pe[b,h,:] . k^R_t), t < N
 *   out[b,h,:]   = (sum_t softmax(s)_t c_t) . W_UV[h]
 *   lse[b,h]     = ln sum_t exp(s_t)
 * which equals softmax attention with keys W_UK[h] c_t | k^R_t and values
 * c_t W_UV[h] (the non-absorbed form) up to rounding. N == 0 gives out = 0
 * and lse = -inf.
 *
 * Arguments
 *   q_nope [batch, H, 128], q_pe [batch, H, 64] (already rotated): act_dtype
 *   w_uk   [H, 128, 512], w_uv [H, 512, 128]: act_dtype, row-major
 *   act_dtype   MLA_F32 (requires an MLA_F32 cache) or MLA_BF16 (bf16 or fp8
 *               cache); bf16 math uses bf16 MFMA operands, fp32 accumulation;
 *               an fp8 cache goes to the fp8 matrix cores as stored, with the
 *               query and the softmax weights split into two e4m3 parts (hi
 *               and lo, power-of-two scales per 32-wide block)
 *   latent, rope, strides, scales (fp8 only), cache_dtype: the cache
 *   cache_rows  total rows of the cache arrays, at most 2^31 - 1
 *               (MLA_ERR_UNSUPPORTED otherwise)
 *   lengths     [batch] int32 (device)
 *   max_len     host upper bound of lengths (sizes the split plan)
 *   softmax_scale  the factor on every score; 0 selects the scale of the
 *               "Classic attention and the cost of the KV cache" section,
 *               1/sqrt(d_k) with d_k = d_nope + d_rope (the key width);
 *               non-finite values are INVALID_ARG
 *   out    [batch, H, 128] act_dtype;  lse [batch, H] fp32 or NULL
 *   workspace   device buffer of at least mla_decode_workspace_size(...)
 *               bytes (256-byte aligned)
 *   opts   NULL or tuning/timing options
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP (see above). batch == 0 is
 * a valid no-op.
 */
mla_status mla_decode(const mla_dims* dims, const void* q_nope, const void* q_pe,
                      const void* w_uk, const void* w_uv, mla_dtype act_dtype,
                      const void* latent, int64_t latent_stride, const void* rope,
                      int64_t rope_stride, const void* scales, mla_dtype cache_dtype,
                      int64_t cache_rows, int64_t seq_capacity, const int32_t* lengths,
                      int32_t batch, int32_t max_len, float softmax_scale, void* out,
                      float* lse, void* workspace, size_t workspace_bytes,
                      const mla_decode_options* opts, hipStream_t stream);

/*
 * mla_decode_paged: as mla_decode (same sources), over a paged cache. Token t
 * of sequence b lives in row block_table[b * max_blocks_per_seq +
 * t / block_size] * block_size + t % block_size. block_size must be a
 * positive multiple of 32 (the kernel's token tile; fp8 caches with blocks
 * that are not multiples of 64 take the widening kernel). Block-table
 * indexing is exact: the result equals mla_decode on the same rows laid out
 * contiguously. (The pages give no paging scheme; the paged layout is the
 * one of the batched ragged workload this library is measured on.)
 */
mla_status mla_decode_paged(const mla_dims* dims, const void* q_nope, const void* q_pe,
                            const void* w_uk, const void* w_uv, mla_dtype act_dtype,
                            const void* latent, int64_t latent_stride, const void* rope,
                            int64_t rope_stride, const void* scales, mla_dtype cache_dtype,
                            int64_t cache_rows, const int32_t* block_table,
                            int32_t max_blocks_per_seq, int32_t block_size,
                            const int32_t* lengths, int32_t batch, int32_t max_len,
                            float softmax_scale, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, const mla_decode_options* opts,
                            hipStream_t stream);

/* Optional timing events of mla_prefill (pass NULL for none): if non-NULL,
 * attn_begin / attn_end record the start and end of the causal attention
 * kernel, expand_begin / expand_end those of the key/value decompression,
 * on `stream`. */
typedef struct {
  hipEvent_t attn_begin;
  hipEvent_t attn_end;
  hipEvent_t expand_begin;
  hipEvent_t expand_end;
} mla_prefill_options;

/* Workspace bytes needed by mla_prefill (0 on invalid sizes): W_UV
 * transposed, and the decompressed keys and values of every head for
 * max_len tokens of each sequence (256 bytes per token and head, plus 128
 * bytes per token for the RoPE keys). */
size_t mla_prefill_workspace_size(const mla_dims* dims, int32_t batch, int32_t max_len);

/*
 * mla_prefill: attention of a chunk of new tokens (a prompt, or a chunk of
 * one) over their sequence's cache, in the recompute mode.
 *
 * The chunk's `chunk` tokens of sequence b are the last rows of its cache:
 * the cache holds lengths[b] rows, and query i (0 <= i < chunk) sits at
 * position p = lengths[b] - chunk + i and attends to rows 0 .. p (the causal
 * mask of "How DeepSeek Rewrote the Transformer [MLA]", section "Classic
 * attention and the cost of the KV cache"; the cache rows of the chunk are
 * written beforehand, e.g. by mla_cache_append). Queries with p < 0 see no
 * row: out = 0 and lse = -inf. For every head h, with keys
 * k_t = [W_UK[h] c_t | k^R_t] and values v_t = c_t W_UV[h] decompressed from
 * the latent rows ("DeepSeek AI efficiency, architecture, benchmarks",
 * section "Architectural Innovations: Multi-Head Latent Attention (MLA)",
 * equations for K and V; "Como a MLA da DeepSeek cortou 93% da memoria",
 * section "O preco da economia: mais contas": with many queries the
 * recompute of K and V is cheaper than absorbing every query):
 *   s_t        = softmax_scale * (q_nope . W_UK[h] c_t + q_pe . k^R_t),  t <= p
 *   out[b,i,h] = sum_t softmax(s)_t c_t W_UV[h]
 *   lse[b,i,h] = ln sum_t exp(s_t)
 * This equals mla_decode of each query over its own prefix.
 *
 * Arguments
 *   q_nope [batch, chunk, H, 128], q_pe [batch, chunk, H, 64] (already
 *               rotated): bf16, row-major
 *   w_uk [H, 128, 512], w_uv [H, 512, 128]: bf16
 *   act_dtype   MLA_BF16: bf16 queries, weights and output. The
 *               decompression runs on bf16 MFMA with fp32 accumulation; the
 *               attention products take the queries, keys, values and
 *               softmax weights in fp16 (fp32 accumulation), so queries and
 *               decompressed keys and values beyond +-65504 saturate
 *   latent, rope, strides, cache_dtype (MLA_BF16), cache_rows: the cache
 *   block_table NULL: contiguous cache, sequence b at rows
 *               [b*seq_capacity, b*seq_capacity + lengths[b]);
 *               otherwise paged as in mla_decode_paged (block_size a
 *               positive multiple of 32)
 *   lengths     [batch] int32 (device): rows of each sequence, chunk included
 *   chunk       queries per sequence (>= 1)
 *   max_len     host upper bound of lengths (sizes the workspace)
 *   softmax_scale  as for mla_decode (0 selects 1/sqrt(d_nope + d_rope))
 *   out [batch, chunk, H, 128] bf16;  lse [batch, chunk, H] fp32 or NULL
 *   workspace   at least mla_prefill_workspace_size(dims, batch, max_len)
 *               bytes, 256-byte aligned
 * Errors: INVALID_ARG, UNSUPPORTED (dtypes other than bf16, heads not a
 * multiple of 32), WORKSPACE, HIP, as for mla_decode. batch == 0 is a valid
 * no-op. Three launches on `stream`.
 */
mla_status mla_prefill(const mla_dims* dims, const void* q_nope, const void* q_pe,
                       const void* w_uk, const void* w_uv, mla_dtype act_dtype,
                       const void* latent, int64_t latent_stride, const void* rope,
                       int64_t rope_stride, mla_dtype cache_dtype, int64_t cache_rows,
                       int64_t seq_capacity, const int32_t* block_table,
                       int32_t max_blocks_per_seq, int32_t block_size, const int32_t* lengths,
                       int32_t batch, int32_t chunk, int32_t max_len, float softmax_scale,
                       void* out, float* lse, void* workspace, size_t workspace_bytes,
                       const mla_prefill_options* opts, hipStream_t stream);

/*
 * mla_fuse_weights: the offline absorption of "How DeepSeek Rewrote the
 * Transformer [MLA]", section "MLA: compress the pair, not the heads" (W_UK
 * absorbed into the query matrix, W_UV into the output matrix W_O before
 * serving). For every head h, with the query projection q_nope[h] = W_Q[h] x
 * and the output y = sum_h o[h] W_O[h] of a model of width d_model:
 *   w_qk[h]                  = W_UK[h]^T W_Q[h]        [H, 512, d_model]
 *   w_vo[n][512 h + c]       = (W_UV[h] W_O[h])[c][n]  [d_model, 512 H]
 * (each fused weight is stored with its contraction index contiguous, the
 * layout mla_decode_fused streams). fp32 accumulation, one bf16 rounding.
 *   w_q [H, 128, d_model], w_uk [H, 128, 512], w_uv [H, 512, 128],
 *   w_o [H, 128, d_model]: bf16, row-major; act_dtype MLA_BF16.
 * d_model: a positive multiple of 64. Errors as for mla_decode.
 */
mla_status mla_fuse_weights(const mla_dims* dims, int32_t d_model, const void* w_q,
                            const void* w_uk, const void* w_uv, const void* w_o,
                            mla_dtype act_dtype, void* w_qk, void* w_vo, hipStream_t stream);

/* Workspace bytes needed by mla_decode_fused (0 on invalid sizes). */
size_t mla_decode_fused_workspace_size(const mla_dims* dims, int32_t batch, int32_t max_len,
                                       int32_t d_model, const mla_decode_options* opts);

/*
 * mla_decode_fused: one decode step from each token's model-width input x to
 * its model-width attention output, with the weights fused offline by
 * mla_fuse_weights:
 *   q_lat[b,h] = w_qk[h] x[b];  s_t = softmax_scale (q_lat . c_t + q_pe[b,h] . k^R_t)
 *   y[b]       = sum_h (sum_t softmax(s)_t c_t) W_VO[h];  lse[b,h] = ln sum_t exp(s_t)
 * which equals the unfused y = sum_h o[b,h] W_O[h] of mla_decode with
 * q_nope[b,h] = W_Q[h] x[b], up to rounding (the identity the absorption
 * rests on).
 *   x [batch, d_model], q_pe [batch, H, 64] (already rotated): bf16
 *   w_qk, w_vo: as written by mla_fuse_weights; act_dtype MLA_BF16
 *   cache arguments, lengths, max_len, softmax_scale, lse, opts: as for
 *   mla_decode (the cache bf16 or fp8); block_table NULL selects the
 *   contiguous layout of mla_decode (seq_capacity), otherwise the paged
 *   layout of mla_decode_paged
 *   out [batch, d_model] bf16
 *   workspace   at least mla_decode_fused_workspace_size(...) bytes,
 *               256-byte aligned
 * opts->append is not supported here (MLA_ERR_UNSUPPORTED): append with
 * mla_cache_append first. Errors as for mla_decode.
 */
mla_status mla_decode_fused(const mla_dims* dims, const void* x, const void* q_pe,
                            const void* w_qk, const void* w_vo, int32_t d_model,
                            mla_dtype act_dtype, const void* latent, int64_t latent_stride,
                            const void* rope, int64_t rope_stride, const void* scales,
                            mla_dtype cache_dtype, int64_t cache_rows, int64_t seq_capacity,
                            const int32_t* block_table, int32_t max_blocks_per_seq,
                            int32_t block_size, const int32_t* lengths, int32_t batch,
                            int32_t max_len, float softmax_scale, void* out, float* lse,
                            void* workspace, size_t workspace_bytes,
                            const mla_decode_options* opts, hipStream_t stream);

/*
 * mla_decode_paged_noalloc: mla_decode_paged without a workspace argument,
 * for callers that cannot allocate device memory or pass a buffer of their
 * own around: code captured into a HIP graph, serving loops that must not
 * call hipMalloc, harnesses that forbid allocation. It calls no allocating
 * routine; the absorbed queries and split partials go to a scratch array
 * inside the library, of MLA_NOALLOC_SCRATCH_BYTES bytes per device (one
 * copy per GPU the library runs on, held until the process ends; its device
 * address is looked up once per device on the first call there).
 *
 * Arguments, results and errors are those of mla_decode_paged. A call whose
 * plan needs more than MLA_NOALLOC_SCRATCH_BYTES (mla_decode_workspace_size
 * with the same arguments) returns MLA_ERR_WORKSPACE and launches nothing;
 * 80 MiB covers, for example, 64 sequences of 4096 tokens or 32 of 32768 at
 * 128 heads. Every call on one GPU uses the same scratch, which keeps the
 * last call's contents (nothing in it needs clearing: each call writes every
 * byte it reads). Calls that can overlap on one GPU (other streams, other
 * host threads) race on it: order them on one stream, or use
 * mla_decode_paged with separate workspaces.
 */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)80 << 20)

mla_status mla_decode_paged_noalloc(const mla_dims* dims, const void* q_nope, const void* q_pe,
                                    const void* w_uk, const void* w_uv, mla_dtype act_dtype,
                                    const void* latent, int64_t latent_stride, const void* rope,
                                    int64_t rope_stride, const void* scales,
                                    mla_dtype cache_dtype, int64_t cache_rows,
                                    const int32_t* block_table, int32_t max_blocks_per_seq,
                                    int32_t block_size, const int32_t* lengths, int32_t batch,
                                    int32_t max_len, float softmax_scale, void* out, float* lse,
                                    const mla_decode_options* opts, hipStream_t stream);

/* Debug checks of the device-resident integers (the preconditions the host
 * cannot check without a synchronisation): lengths[b] within [0, max_len],
 * every block-table entry a decode split reads (rows t < lengths[b]) within
 * [0, cache_rows / block_size), every cache row that the append, the
 * fp32 decode and the prefill address within the cache arrays, and every append
 * position within its sequence's capacity (seq_capacity, or max_blocks_per_seq
 * * block_size when paged). In every build the kernels clamp such values
 * (a length to [0, max_len], an out-of-range row to row 0, an out-of-range
 * append is dropped), so they never access memory outside the arrays; the
 * library built with MLA_DEBUG_CHECKS=1 also records each violation as a bit
 * in a per-device error word: */
#define MLA_DEBUG_LENGTH 1u     /* a length outside [0, max_len] */
#define MLA_DEBUG_BLOCK 2u      /* a block-table entry or cache row outside the cache */
#define MLA_DEBUG_POSITION 4u   /* an append position outside the capacity */

/* Waits for `stream`, then stores the current device's error word in *word
 * (a host pointer) and clears it. The word collects the violations of every
 * call on that device since the last read (from any stream). Returns
 * MLA_ERR_UNSUPPORTED (and *word = 0) from a library built without the
 * checks, MLA_ERR_INVALID_ARG for a null `word`, MLA_ERR_HIP if a HIP call
 * fails. Not for use under graph capture (it synchronizes). */
mla_status mla_debug_errors(uint32_t* word, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
