// Validation rules and the decode split plan.
//
// Batch rules follow "TensorRT-LLM source analysis report", section 1.3 (in-flight
// batching): context requests precede generation requests, every chunk but a prompt's
// last is a multiple of the KV block size, and a batch holds at most max_num_tokens
// tokens (also "TensorRT-LLM 1.0 study notes", 三.3.2: batchNumTokens + reqTokens >
// maxNumTokens stops the batch).
#include "plan.h"

#include <algorithm>
#include <cmath>
#include <cstdio>

namespace pkv {

namespace {

int fail(std::string& err, int code, const char* fmt, long long a = 0, long long b = 0, long long c = 0) {
  char buf[256];
  std::snprintf(buf, sizeof buf, fmt, a, b, c);
  err = buf;
  return code;
}

bool pow2_in(int32_t x, int32_t lo, int32_t hi) { return x >= lo && x <= hi && (x & (x - 1)) == 0; }

}  // namespace

int validate_desc(const pkv_attn_desc* d, std::string& err) {
  if (!d) return fail(err, PKV_ERR_INVALID_ARG, "desc is NULL");
  if (d->num_heads < 1 || d->num_kv_heads < 1)
    return fail(err, PKV_ERR_INVALID_ARG, "num_heads=%lld num_kv_heads=%lld must be >= 1", d->num_heads, d->num_kv_heads);
  if (d->num_heads % d->num_kv_heads)
    return fail(err, PKV_ERR_INVALID_ARG, "num_heads=%lld is not a multiple of num_kv_heads=%lld", d->num_heads, d->num_kv_heads);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(err, PKV_ERR_UNSUPPORTED, "head_dim=%lld (supported: 64, 128)", d->head_dim);
  if (!pow2_in(d->tokens_per_block, 16, 256))
    return fail(err, PKV_ERR_UNSUPPORTED, "tokens_per_block=%lld (supported: 16, 32, 64, 128, 256)", d->tokens_per_block);
  if (d->io_dtype != PKV_FP32 && d->io_dtype != PKV_BF16)
    return fail(err, PKV_ERR_UNSUPPORTED, "io_dtype=%lld (supported: FP32, BF16)", d->io_dtype);
  if (d->kv_dtype != PKV_FP32 && d->kv_dtype != PKV_BF16 && d->kv_dtype != PKV_FP8_E4M3 && d->kv_dtype != PKV_INT8)
    return fail(err, PKV_ERR_UNSUPPORTED, "kv_dtype=%lld (supported: FP32, BF16, FP8_E4M3, INT8)", d->kv_dtype);
  if (d->rope_style != PKV_ROPE_NONE && d->rope_style != PKV_ROPE_NEOX && d->rope_style != PKV_ROPE_GPTJ)
    return fail(err, PKV_ERR_UNSUPPORTED, "rope_style=%lld (supported: NONE, NEOX, GPTJ)", d->rope_style);
  if (d->rotary_dim < 0 || d->rotary_dim > d->head_dim)
    return fail(err, PKV_ERR_INVALID_ARG, "rotary_dim=%lld outside [0, head_dim=%lld]", d->rotary_dim, d->head_dim);
  if (d->rotary_dim % 16)
    return fail(err, PKV_ERR_UNSUPPORTED, "rotary_dim=%lld is not a multiple of 16", d->rotary_dim);
  if (!std::isfinite(d->softmax_scale))
    return fail(err, PKV_ERR_INVALID_ARG, "softmax_scale is not finite");
  if (d->kv_dtype == PKV_FP8_E4M3 || d->kv_dtype == PKV_INT8) {
    if (!(std::isfinite(d->k_scale_quant_orig) && d->k_scale_quant_orig > 0.f &&
          std::isfinite(d->v_scale_quant_orig) && d->v_scale_quant_orig > 0.f))
      return fail(err, PKV_ERR_INVALID_ARG, "fp8 / int8 cache needs finite positive k/v scales");
  }
  if (d->max_num_tokens < 0) return fail(err, PKV_ERR_INVALID_ARG, "max_num_tokens=%lld < 0", d->max_num_tokens);
  return PKV_OK;
}

bool desc_fast_decode(const pkv_attn_desc& d) {
  if (!kHaveFastDecode) return false;
  const int32_t G = d.num_heads / d.num_kv_heads;
  return d.io_dtype == PKV_BF16 && (d.kv_dtype == PKV_BF16 || d.kv_dtype == PKV_FP8_E4M3 || d.kv_dtype == PKV_INT8) &&
         G <= 16 &&
         (d.head_dim == 128 || d.head_dim == 64);
}

bool desc_fast_prefill(const pkv_attn_desc& d) {
  if (!kHaveFastPrefill) return false;
  const int32_t G = d.num_heads / d.num_kv_heads;
  return d.io_dtype == PKV_BF16 && d.kv_dtype == PKV_BF16 && d.head_dim == 128 &&
         (G == 1 || G == 2 || G == 4 || G == 8);
}

int validate_batch(const pkv_attn_desc* d, const pkv_batch_desc* b, BatchPlan* plan, std::string& err) {
  if (!b) return fail(err, PKV_ERR_INVALID_ARG, "batch is NULL");
  const int32_t B = b->num_requests;
  if (B < 0) return fail(err, PKV_ERR_INVALID_ARG, "num_requests=%lld < 0", B);
  if (b->num_tokens < 0) return fail(err, PKV_ERR_INVALID_ARG, "num_tokens=%lld < 0", b->num_tokens);
  BatchPlan p;
  p.B = B;
  p.N = b->num_tokens;
  if (B == 0) {
    if (b->num_tokens != 0) return fail(err, PKV_ERR_INVALID_ARG, "num_tokens=%lld with no requests", b->num_tokens);
    if (plan) *plan = p;
    return PKV_OK;
  }
  if (!b->host_request_types || !b->host_context_lengths || !b->host_sequence_lengths)
    return fail(err, PKV_ERR_INVALID_ARG, "host length arrays must not be NULL");
  if (!b->context_lengths || !b->sequence_lengths || !b->kv_cache_block_offsets)
    return fail(err, PKV_ERR_INVALID_ARG, "device length arrays and kv_cache_block_offsets must not be NULL");
  if (b->max_blocks_per_seq < 1) return fail(err, PKV_ERR_INVALID_ARG, "max_blocks_per_seq=%lld < 1", b->max_blocks_per_seq);
  if (b->num_pool_blocks < 1) return fail(err, PKV_ERR_INVALID_ARG, "num_pool_blocks=%lld < 1", b->num_pool_blocks);
  const int32_t T = d->tokens_per_block;
  int64_t sum_n = 0;
  bool seen_gen = false;
  for (int32_t r = 0; r < B; ++r) {
    const int32_t ty = b->host_request_types[r];
    const int32_t n = b->host_context_lengths[r];
    const int32_t S = b->host_sequence_lengths[r];
    if (ty != PKV_REQ_CONTEXT && ty != PKV_REQ_GENERATION)
      return fail(err, PKV_ERR_INVALID_ARG, "request %lld: request type %lld", r, ty);
    if (ty == PKV_REQ_CONTEXT && seen_gen)
      return fail(err, PKV_ERR_ORDER, "request %lld: context request after a generation request", r);
    if (n < 1) return fail(err, PKV_ERR_INVALID_ARG, "request %lld: context length %lld < 1", r, n);
    if (ty == PKV_REQ_GENERATION && n > kMaxGenTokens)
      return fail(err, PKV_ERR_UNSUPPORTED, "request %lld: generation request with %lld new tokens (at most %lld)", r, n,
                  static_cast<int64_t>(kMaxGenTokens));
    if (S < n) return fail(err, PKV_ERR_INVALID_ARG, "request %lld: sequence length %lld < context length %lld", r, S, n);
    if (ty == PKV_REQ_CONTEXT && (S - n) % T)
      return fail(err, PKV_ERR_CHUNK_ALIGN, "request %lld: cached length %lld is not a multiple of tokens_per_block %lld",
                  r, S - n, T);
    const int64_t need = (static_cast<int64_t>(S) + T - 1) / T;
    if (need > b->max_blocks_per_seq)
      return fail(err, PKV_ERR_BLOCK_RANGE, "request %lld needs %lld blocks, table has %lld", r, need, b->max_blocks_per_seq);
    if (b->host_kv_cache_block_offsets) {
      const int32_t* row = b->host_kv_cache_block_offsets + static_cast<int64_t>(r) * b->max_blocks_per_seq;
      for (int64_t j = 0; j < need; ++j)
        if (row[j] < 0 || row[j] >= b->num_pool_blocks)
          return fail(err, PKV_ERR_BLOCK_RANGE, "request %lld logical block %lld: block id %lld outside the pool", r, j, row[j]);
    }
    sum_n += n;
    if (ty == PKV_REQ_CONTEXT) {
      p.num_ctx++;
      p.ctx_tokens += n;
      p.max_ctx_n = std::max(p.max_ctx_n, n);
      const int64_t past = S - n;
      p.ctx_pairs += static_cast<int64_t>(n) * past + static_cast<int64_t>(n) * (n + 1) / 2;
    } else {
      seen_gen = true;
      p.num_gen++;
      p.max_S_gen = std::max(p.max_S_gen, S);
      p.gen_keys += S;
      p.gen_tokens += n;
      p.max_gen_n = std::max(p.max_gen_n, n);
    }
    p.max_n = std::max(p.max_n, n);
    p.max_S = std::max(p.max_S, S);
  }
  if (sum_n != b->num_tokens)
    return fail(err, PKV_ERR_INVALID_ARG, "num_tokens=%lld but context lengths sum to %lld", b->num_tokens, sum_n);
  if (b->num_tokens > d->max_num_tokens)
    return fail(err, PKV_ERR_BUDGET, "num_tokens=%lld exceeds max_num_tokens=%lld", b->num_tokens, d->max_num_tokens);
  if (p.max_ctx_n > b->max_context_length)
    return fail(err, PKV_ERR_INVALID_ARG, "max_context_length=%lld < longest context chunk %lld", b->max_context_length, p.max_ctx_n);
  if (plan) {
    plan_decode(*d, *b, &p);
    *plan = p;
  }
  return PKV_OK;
}

void plan_decode(const pkv_attn_desc& d, const pkv_batch_desc& b, BatchPlan* p) {
  const int32_t G = d.num_heads / d.num_kv_heads;
  p->fast_decode = p->num_gen > 0 && desc_fast_decode(d) && G * p->max_gen_n <= kMaxDecodeCols;
  p->col_blocks = (G * p->max_gen_n + 15) / 16;
  p->fast_prefill = p->num_ctx > 0 && desc_fast_prefill(d);
  p->dec_heads = p->dec_cols = 0;
  p->dec_units = p->dec_segments = p->dec_max_wgs = 0;
  p->ws_pre_off = p->ws_ml_off = p->ws_o_off = p->ws_bytes = 0;
  if (!p->fast_decode) return;
  // Work units of the balanced split pass: request r has ceil(S_r / 32) tiles in each of its
  // (head group, column block) segments, with ceil(G * n_r / 16) column blocks of its own.
  // The kernel derives the same count from the device lengths.
  p->dec_cbw = decode_column_waves(d.num_kv_heads, p->col_blocks);
  p->dec_allcols = p->dec_cbw > 1;
  p->dec_heads = p->dec_cbw > 1 ? 4 / p->dec_cbw : decode_heads_per_wg(d.num_kv_heads);
  const int64_t hgs = d.num_kv_heads / p->dec_heads;
  int64_t units = 0;
  for (int32_t r = p->num_ctx; r < p->B; ++r) {
    const int64_t n = b.host_context_lengths[r];
    const int64_t S = std::max<int64_t>(b.host_sequence_lengths[r], n);
    units += (S - 1) / kDecodeTile + 1;
  }
  p->dec_units = units;
  p->dec_lane_cbs = p->dec_allcols ? 1 : p->col_blocks;
  p->dec_lanes = static_cast<int32_t>(hgs * p->dec_lane_cbs);
  p->dec_segments = static_cast<int64_t>(p->num_gen) * p->dec_lanes;
  p->dec_max_wgs = p->dec_lanes * std::min<int64_t>(std::max<int64_t>(1, kDecodeMaxWGs / p->dec_lanes), units);
  p->dec_cols = p->dec_allcols ? G * p->max_gen_n : std::min(16, G * p->max_gen_n);
  const int64_t entries = (p->dec_segments + p->dec_max_wgs) * p->dec_heads * p->dec_cols;
  auto up = [](size_t x) { return ((x + 255) / 256) * 256; };
  p->ws_pre_off = 0;
  p->ws_ml_off = up(static_cast<size_t>(p->num_gen + 1) * 2 * sizeof(int64_t));   // first units, first rows
  p->ws_o_off = p->ws_ml_off + up(static_cast<size_t>(entries) * 2 * sizeof(float));
  p->ws_bytes = p->ws_o_off + static_cast<size_t>(entries) * d.head_dim * sizeof(float);
}

size_t workspace_upper_bound(const pkv_attn_desc& d, int32_t max_num_requests, int32_t max_seq_len) {
  if (max_num_requests <= 0 || max_seq_len <= 0) return 0;
  if (!desc_fast_decode(d)) return 0;
  // Worst case over the batches of at most max_num_requests generation requests of at
  // most max_seq_len keys: every request with the most column blocks, and per slot 16
  // columns of 4 KV heads (one head per segment has Hkv segments per column block, four
  // heads have Hkv / 4 and a single column block).
  const int64_t G = d.num_heads / d.num_kv_heads;
  const int64_t R = max_num_requests;
  const int64_t cbmax = (std::min<int64_t>(G * kMaxGenTokens, kMaxDecodeCols) + 15) / 16;
  const int64_t tiles = (static_cast<int64_t>(max_seq_len) - 1) / kDecodeTile + 1;
  const int64_t W = std::max<int64_t>(kDecodeMaxWGs, d.num_kv_heads * cbmax);   // workgroups, at most
  // segments carrying all column blocks: at most Hkv segments per request, at most 4 heads
  // x G * kMaxGenTokens columns per slot
  const int64_t all_cols = std::min<int64_t>(G * kMaxGenTokens, kMaxDecodeCols);
  const int64_t entries = std::max((R * d.num_kv_heads * cbmax + 4 * W) * 16, (R * d.num_kv_heads + 4 * W) * all_cols);
  auto up = [](size_t x) { return ((x + 255) / 256) * 256; };
  return up(static_cast<size_t>(R + 1) * 2 * sizeof(int64_t)) + up(static_cast<size_t>(entries) * 2 * sizeof(float)) +
         static_cast<size_t>(entries) * d.head_dim * sizeof(float);
}

int validate_tree(const pkv_batch_desc* b, const BatchPlan& plan, const pkv_spec_tree* t, std::string& err) {
  if (!t) return fail(err, PKV_ERR_INVALID_ARG, "spec tree is NULL");
  if (!t->host_position_offsets || !t->position_offsets || !t->host_packed_mask || !t->packed_mask)
    return fail(err, PKV_ERR_INVALID_ARG, "spec tree: host and device position offsets and packed masks are all required");
  if ((reinterpret_cast<uintptr_t>(t->position_offsets) & 3u) || (reinterpret_cast<uintptr_t>(t->packed_mask) & 7u))
    return fail(err, PKV_ERR_INVALID_ARG, "spec tree: position offsets must be 4-byte and packed masks 8-byte aligned");
  int64_t row = plan.ctx_tokens;
  for (int32_t r = plan.num_ctx; r < plan.B; ++r) {
    const int32_t n = b->host_context_lengths[r];
    for (int32_t i = 0; i < n; ++i, ++row) {
      const int32_t o = t->host_position_offsets[row];
      if (o < 0 || o >= n)
        return fail(err, PKV_ERR_INVALID_ARG, "spec tree: row %lld has position offset %lld outside 0 .. n-1 (n = %lld)",
                    row, o, n);
      const uint64_t m = static_cast<uint64_t>(t->host_packed_mask[2 * row]) |
                         (static_cast<uint64_t>(t->host_packed_mask[2 * row + 1]) << 32);
      if (!((m >> i) & 1u))
        return fail(err, PKV_ERR_INVALID_ARG, "spec tree: row %lld (token %lld of its request) lacks its own mask bit", row, i);
      if (n < 64 && (m >> n) != 0)
        return fail(err, PKV_ERR_INVALID_ARG, "spec tree: row %lld names a token at or past n = %lld in its mask", row, n);
    }
  }
  return PKV_OK;
}

}  // namespace pkv
