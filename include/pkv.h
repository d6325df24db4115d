/*
 * pkv.h -- C ABI of the paged-KV GQA + RoPE attention library for AMD MI355X (gfx950).
 *
 * One step of one attention layer over an in-flight batch:
 *   1. pkv_append_rope: rotate the new tokens' q and k (RoPE), write the
 *      rotated q to q_out and scatter the rotated k and the raw v into the paged
 *      KV pool through the per-request block table (pkv_append_qknorm_rope: the
 *      same with each q and k head normalised first);
 *   2. pkv_attention_forward: causal attention for context-phase rows and for
 *      generation-phase rows (one token, or a token and its draft tokens), reading
 *      K/V through the block table.
 *
 * Sources (secondary descriptions of TensorRT-LLM; cited by page title and section):
 *   [REPORT]   "TensorRT-LLM source analysis report" (adg.csdn.net):
 *              1.1 attention parameters, 1.2 KV cache parameters, 1.3 in-flight batching.
 *   [NOTES]    "TensorRT-LLM 1.0 study notes" (openharmonycrossplatform.csdn.net):
 *              二.2 KVCacheManager, 三.3.2 MicroBatchScheduler, 五.5.3 kernels and streams,
 *              六.6.1-6.3 FlashAttention / paged attention, 6.4 INT8 KV cache quantisation.
 *   [TEARDOWN] "TensorRT-LLM source teardown part 1: architecture overview"
 *              (pinghaoyang.com.cn): KV cache manager interfaces, AttentionMetadata
 *              fields, AttentionBackend.forward signature, attention backend lifecycle.
 *
 * Conventions for every entry point:
 *   - All device work is enqueued asynchronously on `stream` (a hipStream_t; NULL is
 *     the null stream).  Nothing synchronises the host, nothing allocates memory, and
 *     no host-to-device copy happens inside a call, so calls are capturable in a HIP
 *     graph (the teardown's lifecycle section: metadata tensors are allocated once).
 *     Calls on one stream run in order, so an attention call sees the K/V that an
 *     earlier append call on the same stream wrote ([NOTES] 五.5.3, one stream is FIFO).
 *   - The caller owns every buffer.  Pointers documented "device" must be device
 *     memory of the current device; "host" pointers are read during the call only.
 *   - Every argument is validated on the host before any launch.  On error nothing
 *     is launched, no output is touched, the call returns a negative pkv_status and
 *     pkv_last_error() describes the problem.  A HIP launch failure returns
 *     PKV_ERR_HIP; faults of already-launched kernels surface at the caller's next
 *     synchronisation.
 *   - Device copies of lengths and the block table must hold the same values as
 *     the host copies.  Kernels re-check every index they derive from device data
 *     (block IDs against num_pool_blocks, rows against num_tokens) and skip what is
 *     out of range instead of faulting.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 1
/* bytes of the per-GPU scratch array of pkv_attention_forward_noalloc */
#define PKV_SCRATCH_BYTES ((size_t)64 << 20)

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = -1,  /* null pointer, inconsistent sizes, misaligned buffer    */
  PKV_ERR_UNSUPPORTED = -2,  /* valid request this library does not implement          */
  PKV_ERR_ORDER = -3,        /* a context request after a generation request ([REPORT] 1.3) */
  PKV_ERR_CHUNK_ALIGN = -4,  /* context request whose cached length is not a multiple of
                                tokens_per_block: only the last chunk of a prompt may be
                                ragged ([REPORT] 1.3, chunked context)                  */
  PKV_ERR_BUDGET = -5,       /* num_tokens > max_num_tokens ([REPORT] 1.3; [NOTES] 三.3.2) */
  PKV_ERR_BLOCK_RANGE = -6,  /* block table too narrow, or a block ID outside the pool   */
  PKV_ERR_WORKSPACE = -7,    /* workspace missing or smaller than required               */
  PKV_ERR_HIP = -8           /* a HIP runtime call failed                                */
} pkv_status;

/* element formats */
enum { PKV_FP32 = 0, PKV_BF16 = 1, PKV_FP8_E4M3 = 2 /* OCP E4M3: bias 7, max 448, no inf */,
       PKV_INT8 = 3 /* two's-complement int8 codes, -128 .. 127 */ };
/* host_request_types values ([REPORT] 1.1: context vs generation phase) */
enum { PKV_REQ_CONTEXT = 0, PKV_REQ_GENERATION = 1 };
/* rotary embedding styles ([REPORT] 1.1 names GPT-NeoX among the RoPE variants) */
enum { PKV_ROPE_NONE = 0, PKV_ROPE_NEOX = 1, PKV_ROPE_GPTJ = 2 };

/*
 * Per-layer attention description ([REPORT] 1.1 attention parameters; [TEARDOWN]
 * AttentionBackend.forward).
 *   num_heads, num_kv_heads : H and Hkv; H % Hkv == 0.  Query head h reads KV head
 *                             h / (H / Hkv) (GQA as contiguous head groups).
 *   head_dim                : D, 64 or 128.
 *   tokens_per_block        : T, tokens per KV block: 16, 32, 64, 128 or 256.
 *   io_dtype                : q, k, v, q_out and out: PKV_FP32 or PKV_BF16.
 *   kv_dtype                : KV pool: PKV_FP32, PKV_BF16, PKV_FP8_E4M3 or PKV_INT8.
 *   rope_style, rotary_dim  : PKV_ROPE_NEOX rotates pairs (j, j + R/2), j < R/2, of
 *                             each q and new k head by angle pos * theta_j, where R =
 *                             rotary_dim (0 means head_dim; otherwise a multiple of 16,
 *                             <= head_dim) and the table gives cos/sin; dims >= R are
 *                             copied.  PKV_ROPE_GPTJ rotates the interleaved pairs
 *                             (2j, 2j + 1), j < R/2, by the same angles (same table);
 *                             the source analysis report, 1.1, lists the RoPE variants
 *                             (GPT-NeoX, ChatGLM, CogVLM) that differ in this pairing
 *                             and in R.  PKV_ROPE_NONE stores k as given.
 *   softmax_scale           : <= 0 means 1/sqrt(head_dim).
 *   k_scale_quant_orig,
 *   v_scale_quant_orig      : fp8 and int8 caches only: real value = scale * stored
 *                             value (the e4m3 value, or the integer code).  The append
 *                             quantises with 1/scale (computed in fp64) and rounds to
 *                             nearest-even, saturating to +-448 (fp8) or to -128 .. 127
 *                             (int8; NaN stores 0) ([NOTES] 6.4: kv_scale_orig_quant on
 *                             write, kv_scale_quant_orig on read, the INT8 KV cache
 *                             compressing only the stored format).
 *   max_num_tokens          : token budget of one batch (8192 by default, [REPORT] 1.3).
 */
typedef struct pkv_attn_desc {
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t tokens_per_block;
  int32_t io_dtype;
  int32_t kv_dtype;
  int32_t rope_style;
  int32_t rotary_dim;
  float softmax_scale;
  float k_scale_quant_orig;
  float v_scale_quant_orig;
  int32_t max_num_tokens;
} pkv_attn_desc;

/*
 * One in-flight batch ([REPORT] 1.1-1.3; [TEARDOWN] AttentionMetadata fields, which keep
 * host lengths and a device copy side by side so no host-to-device copy sits in the
 * hot path).
 *   num_requests            : B >= 0.  All context requests come first ([REPORT] 1.3).
 *   num_tokens              : N = sum of host_context_lengths; packed rows, no padding.
 *   max_context_length      : >= every context request's host_context_lengths entry.
 *   host_request_types      : host [B], PKV_REQ_CONTEXT or PKV_REQ_GENERATION.
 *   host_context_lengths    : host [B], n_r = tokens request r brings to this step
 *                             (a prompt or chunk length for a context request; for a
 *                             generation request 1, or 1 + k draft tokens to verify, at
 *                             most 64 -- the generation lengths of [REPORT] 1.4; token i
 *                             of the request sits at position S_r - n_r + i, i.e. the
 *                             position offsets are 0 .. n_r - 1 and the drafts form one
 *                             chain, causal among themselves).
 *   host_sequence_lengths   : host [B], S_r = cached tokens before the step + n_r.  The
 *                             new tokens occupy cache positions S_r - n_r .. S_r - 1.
 *   context_lengths,
 *   sequence_lengths        : device [B] copies of the two host arrays.
 *   kv_cache_block_offsets  : device int32 [B, max_blocks_per_seq]: physical block IDs of
 *                             request r's logical blocks 0 .. ceil(S_r/T)-1 ([REPORT] 1.2;
 *                             [TEARDOWN] get_batch_cache_indices).  Cache position t of
 *                             request r is slot t % T of block [r][t / T].
 *   host_kv_cache_block_offsets : optional host copy (NULL allowed); when given, every
 *                             used entry is range-checked on the host.
 *   num_pool_blocks         : blocks in the pool; valid IDs are 0 .. num_pool_blocks-1.
 */
typedef struct pkv_batch_desc {
  int32_t num_requests;
  int32_t num_tokens;
  int32_t max_context_length;
  int32_t max_blocks_per_seq;
  const int32_t* host_request_types;
  const int32_t* host_context_lengths;
  const int32_t* host_sequence_lengths;
  const int32_t* context_lengths;
  const int32_t* sequence_lengths;
  const int32_t* kv_cache_block_offsets;
  const int32_t* host_kv_cache_block_offsets;
  int64_t num_pool_blocks;
} pkv_batch_desc;

/* PKV_ABI_VERSION of the loaded library. */
int32_t pkv_abi_version(void);

/* Message of the last non-OK return on the calling thread ("" if none). */
const char* pkv_last_error(void);

/*
 * Upper bound of the workspace pkv_attention_forward needs for any batch with at most
 * max_num_requests requests and sequence lengths <= max_seq_len ([NOTES] 五: the
 * plugin pattern of a size query before enqueue).  0 on invalid arguments.
 */
size_t pkv_workspace_size(const pkv_attn_desc* desc, int32_t max_num_requests, int32_t max_seq_len);

/* Exact workspace bytes pkv_attention_forward needs for this batch; 0 on invalid arguments. */
size_t pkv_workspace_size_for_batch(const pkv_attn_desc* desc, const pkv_batch_desc* batch);

/*
 * Fill the GPT-NeoX rotary table ([REPORT] 1.1 rotary_embedding):
 *   cos_sin[pos][j][0] = cos(pos * theta_j), cos_sin[pos][j][1] = sin(pos * theta_j),
 *   theta_j = base^(-2j / rotary_dim), pos < max_pos, j < rotary_dim / 2, all fp64.
 * cos_sin: device, max_pos * rotary_dim fp64 values, written asynchronously on stream.
 */
int32_t pkv_rope_cos_sin(double base, int32_t rotary_dim, int32_t max_pos, double* cos_sin,
                         void* stream);

/*
 * RoPE + KV append ([NOTES] 二.2: the attention op itself writes each request's new K/V
 * into the blocks the block table names; [TEARDOWN] KV cache manager: pool layout
 * [num_blocks, 2, tokens_per_block, num_kv_heads, head_dim] with K at index 0 and V at 1).
 *   q        : device, N rows of H*D io elements, row r at q + r*q_row_stride; may be NULL
 *              together with q_out (then only K/V are written).
 *   k, v     : device, N rows of Hkv*D io elements each, row stride kv_row_stride.  For a
 *              fused QKV buffer pass three pointers into it and its row stride
 *              ([TEARDOWN] fused QKV input).  Strides are in elements; every row start
 *              must be 16-byte aligned.
 *   rope_cos_sin, rope_max_pos : device table as written by pkv_rope_cos_sin; required for
 *              PKV_ROPE_NEOX, every new position must be < rope_max_pos.  Ignored for NONE.
 *   q_out    : device [N, H*D] io dtype, dense: the rotated q rounded to the io format.
 *   kv_pool  : device [num_pool_blocks, 2, T, Hkv, D] kv dtype.  Only the slots of the new
 *              positions are written; each is the fp64 result rounded once to the cache
 *              format (nearest-even).
 * Per element the rotation is two fp64 products and one fp64 add/subtract, no fused
 * multiply-add, so the written bits are a function of the inputs and the table alone.
 */
int32_t pkv_append_rope(const pkv_attn_desc* desc, const pkv_batch_desc* batch,
                        const void* q, int64_t q_row_stride,
                        const void* k, const void* v, int64_t kv_row_stride,
                        const double* rope_cos_sin, int32_t rope_max_pos,
                        void* q_out, void* kv_pool, void* stream);

/* kinds of per-head q/k normalisation (see pkv_append_qknorm_rope) */
enum { PKV_NORM_NONE = 0, PKV_NORM_RMS = 1, PKV_NORM_LAYER = 2 };

/*
 * Per-head normalisation of queries and keys before the rotation.  [REPORT] 1.1 lists
 * "QK LayerNorm" (layer normalisation of the queries and keys) among the attention
 * features; [TEARDOWN]'s listing of the kernel directory names a fused QK-norm + RoPE
 * kernel next to grouped RMSNorm kernels.  Over the D elements x_j of one q head or one
 * new k head, in fp64, in this order, sums in index order j = 0 .. D-1, no fused
 * multiply-add:
 *   PKV_NORM_RMS  : mu = 0;                 PKV_NORM_LAYER: mu = (sum_j x_j) / D;
 *   d_j = x_j - mu,  var = (sum_j d_j * d_j) / D,  inv = 1 / sqrt(var + eps),
 *   y_j = (d_j * inv) * w_j          (RMS)      y_j = (d_j * inv) * w_j + b_j   (LAYER).
 *   kind             : PKV_NORM_RMS or PKV_NORM_LAYER (PKV_NORM_NONE: no normalisation).
 *   eps              : finite, >= 0.
 *   q_weight, k_weight : device fp32 [head_dim], 16-byte aligned, one vector for all query
 *                      heads and one for all key heads; q_weight may be NULL when q is.
 *   q_bias, k_bias   : device fp32 [head_dim], 16-byte aligned; PKV_NORM_LAYER only
 *                      (NULL means zero).
 */
typedef struct pkv_qk_norm {
  int32_t kind;
  float eps;
  const float* q_weight;
  const float* k_weight;
  const float* q_bias;
  const float* k_bias;
} pkv_qk_norm;

/*
 * pkv_append_rope with each q head and each new k head normalised first: y as defined
 * for pkv_qk_norm replaces x in the rotation (and in the dimensions past rotary_dim), and
 * the stored value is y rotated and rounded once.  v is stored as given.  norm == NULL or
 * kind PKV_NORM_NONE is exactly pkv_append_rope.  Arguments and errors as for
 * pkv_append_rope; additionally PKV_ERR_INVALID_ARG for an unknown kind, a negative or
 * non-finite eps or a missing or misaligned weight, and PKV_ERR_UNSUPPORTED when
 * num_heads + num_kv_heads > 256.
 */
int32_t pkv_append_qknorm_rope(const pkv_attn_desc* desc, const pkv_batch_desc* batch, const pkv_qk_norm* norm,
                               const void* q, int64_t q_row_stride,
                               const void* k, const void* v, int64_t kv_row_stride,
                               const double* rope_cos_sin, int32_t rope_max_pos,
                               void* q_out, void* kv_pool, void* stream);

/*
 * Attention over the paged cache ([NOTES] 六.6.1-6.3; [TEARDOWN] AttentionBackend.forward).
 * For request r, new row i at position m = S_r - n_r + i and query head h, with
 * g = h / (H/Hkv):  out[row][h] = sum_{t <= m} softmax_t(scale * <q[row][h], K_g[t]>) V_g[t].
 * Context rows are therefore causal over the cached prefix plus the chunk; a one-token
 * generation row attends to all S_r cached positions, its own appended token included,
 * and the draft tokens of a generation request are causal among themselves.
 *   q        : device, N rows of H*D io elements (normally q_out of the append), row
 *              stride q_row_stride elements, 16-byte aligned rows.
 *   kv_pool  : device pool as above, already holding positions 0 .. S_r-1 of every request.
 *   out      : device [N, H*D] io dtype, dense; rows in q's packed order.
 *   workspace: device scratch of at least pkv_workspace_size_for_batch() bytes (256-byte
 *              aligned); may be NULL when that size is 0.  Contents need no initialisation.
 * Accumulation is fp32; outputs are rounded to nearest-even.  For a fixed batch the result
 * is bitwise reproducible (no floating-point atomics).
 */
int32_t pkv_attention_forward(const pkv_attn_desc* desc, const pkv_batch_desc* batch,
                              const void* q, int64_t q_row_stride, const void* kv_pool,
                              void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_attention_forward with the result written as fp8 by the attention kernels themselves
 * ([TEARDOWN], attention backends: the default backend's FP8 output, which fuses the
 * quantisation into the attention computation instead of a separate quantisation kernel
 * between attention and the next GEMM).
 *   out_scale_quant_orig : real value = scale * stored value (the convention of the KV
 *              scales); finite, > 0, with a finite reciprocal.
 *   out      : device [N, H*D] bytes, dense, OCP E4M3 codes: the fp32 attention result
 *              times 1/out_scale_quant_orig (the reciprocal computed in fp64, rounded to
 *              fp32), rounded once to nearest-even, saturating to +-448; NaN stays NaN.
 * Everything else as for pkv_attention_forward.
 */
int32_t pkv_attention_forward_fp8_out(const pkv_attn_desc* desc, const pkv_batch_desc* batch,
                                      const void* q, int64_t q_row_stride, const void* kv_pool,
                                      float out_scale_quant_orig, void* out,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_attention_forward for callers that cannot allocate or pass a workspace: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.  The split-KV
 * partial results go to the library's own device scratch array instead of a caller
 * workspace: one array of PKV_SCRATCH_BYTES (64 MiB) per GPU, held from the
 * library's first use on that GPU until the process ends.  Nothing is allocated; the
 * array's device address is looked up once per device.  Arguments, results and errors
 * as for pkv_attention_forward, and additionally PKV_ERR_WORKSPACE (nothing launched)
 * when the batch needs more scratch than the array holds (pkv_workspace_size_for_batch
 * gives the need).  Nothing in the array has to start at zero (every partial result a
 * call reads was written earlier in the same call).  Every call on one GPU shares that
 * GPU's array: calls that may overlap on one GPU (several streams, or several threads)
 * race and must be serialised by the caller.
 */
int32_t pkv_attention_forward_noalloc(const pkv_attn_desc* desc, const pkv_batch_desc* batch,
                                      const void* q, int64_t q_row_stride, const void* kv_pool,
                                      void* out, void* stream);

/*
 * Draft tokens verified as a tree ([REPORT] 1.4: spec_decoding_position_offsets and
 * spec_decoding_packed_mask; a Medusa-style candidate tree checked in one forward pass,
 * [TEARDOWN] speculative decoding).  For every packed row of a generation request with
 * n tokens (the row of its token i):
 *   position offset o_i : 0 <= o_i < n.  The row's q and k are rotated at position
 *              S_r - n + o_i; its K/V still go to cache position S_r - n + i (the offsets
 *              move the rotation, not the slot).
 *   packed mask M_i    : two 32-bit words, bit j of word j / 32 at bit j % 32 set when the
 *              row attends to new token j's key (cache position S_r - n + j).  Bit i must
 *              be set and no bit j >= n.  Every row also attends to all S_r - n cached
 *              positions.
 * Offsets 0 .. n-1 with M_i = bits 0 .. i give the chain that the entry points without
 * a tree compute.  Context rows' entries are ignored.
 *   host_position_offsets, position_offsets : host and device int32 [N], packed row order.
 *   host_packed_mask, packed_mask           : host and device uint32 [N][2].
 * The host copies are validated (PKV_ERR_INVALID_ARG names the first bad row); the
 * kernels read the device copies, which must hold the same values.
 */
typedef struct pkv_spec_tree {
  const int32_t* host_position_offsets;
  const int32_t* position_offsets;
  const uint32_t* host_packed_mask;
  const uint32_t* packed_mask;
} pkv_spec_tree;

/* pkv_append_rope with generation rows rotated at S_r - n_r + o_i (pkv_spec_tree). */
int32_t pkv_append_rope_tree(const pkv_attn_desc* desc, const pkv_batch_desc* batch, const pkv_spec_tree* tree,
                             const void* q, int64_t q_row_stride,
                             const void* k, const void* v, int64_t kv_row_stride,
                             const double* rope_cos_sin, int32_t rope_max_pos,
                             void* q_out, void* kv_pool, void* stream);

/* pkv_attention_forward with generation rows attending to the cached positions and the
 * new tokens their packed masks name (pkv_spec_tree). */
int32_t pkv_attention_forward_tree(const pkv_attn_desc* desc, const pkv_batch_desc* batch, const pkv_spec_tree* tree,
                                   const void* q, int64_t q_row_stride, const void* kv_pool,
                                   void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Opt-in timing for measurement tools.  pkv_kernel_timing_enable(1) times every kernel
 * launch, pkv_kernel_timing_enable(2) every phase instead: the append, the context
 * attention, and the generation attention (named "decode": the split pass and its
 * combine as one span, with no events between them); 0 switches timing off.  Enabling
 * creates a pool of 8192 HIP events (once; they are reused) and clears the record; while
 * enabled, each timed launch or phase is bracketed by two events of the pool recorded on
 * its stream (no synchronisation, no allocation inside the entry points).  Once the pool
 * is used up, further launches are not timed.  pkv_kernel_timings() synchronises on the
 * recorded events, writes up to max_entries names (static strings) and durations in
 * milliseconds, returns the number of entries recorded since timing was last enabled,
 * sets pkv_last_error() to the number of untimed launches if any, and may be called only
 * from the thread that launched.  Not graph-capturable.
 */
int32_t pkv_kernel_timing_enable(int32_t on);
int32_t pkv_kernel_timings(const char** names, float* milliseconds, int32_t max_entries);

/*
 * Tuning and testing control of the generation (decode) split pass, which shares the
 * batch's 32-key tiles among a fixed number of workgroups: by default two per compute unit
 * of the device (at most 1024), never more than the batch has tiles.  n > 0 caps that
 * number at n for later calls from any thread of the process; n = 0 restores the default;
 * n < 0 only queries.  Returns the setting in force before the call.  Results stay within
 * the documented accuracy for every setting; they are bitwise reproducible for a fixed
 * setting and device.
 */
int32_t pkv_set_decode_workgroups(int32_t n);

/*
 * Mixed batches (context and generation requests in one call; "TensorRT-LLM source
 * analysis report", 1.3, mixed-phase processing): by default, when both parts take the
 * fast kernels (at most 256 context requests, generation requests of one token over KV
 * heads in fours, tokens_per_block >= 16), one launch runs the context attention on some
 * compute units and the generation split pass on the others, sized by estimated time;
 * the combine follows.  With the decode workgroup cap above set (n > 0), the split pass
 * gets that many workgroups (one per compute unit) and the context part the rest.
 * on = 0 runs the two parts one after the other, on = 1 restores the default, on < 0 only
 * queries.  Returns the setting in force before the call (process-wide).  Results stay
 * within the documented accuracy either way.
 */
int32_t pkv_set_coschedule(int32_t on);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
