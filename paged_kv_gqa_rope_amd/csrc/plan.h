// Host-side validation and launch planning.  No HIP types here, so this part of the
// library is ordinary C++ and its rules can be exercised without a GPU.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "pkv.h"

namespace pkv {

// Derived facts about one batch, computed on the host from the host copies.
struct BatchPlan {
  int32_t B = 0, N = 0;
  int32_t num_ctx = 0, num_gen = 0;
  int32_t ctx_tokens = 0;     // packed rows owned by context requests (they come first)
  int32_t max_ctx_n = 0;      // longest context chunk
  int32_t max_n = 0;          // largest n_r over all requests
  int32_t max_S = 0;          // largest S_r over all requests
  int32_t max_S_gen = 0;      // largest S_r over generation requests
  int64_t ctx_pairs = 0;      // causal (query, key) pairs of context rows
  int64_t gen_keys = 0;       // sum of S_r over generation requests
  int32_t gen_tokens = 0;     // packed rows owned by generation requests
  int32_t max_gen_n = 0;      // most new tokens of one generation request (1 + draft tokens)
  // split-KV decode policy (generation rows on the MFMA decode path)
  bool fast_decode = false;
  bool fast_prefill = false;
  int32_t chunk = 0;          // keys per split, a multiple of tokens_per_block
  int32_t max_splits = 0;     // max over generation requests of ceil(S_r / chunk)
  int64_t decode_items = 0;   // (request, kv head, split) work items
  int32_t col_blocks = 0;     // blocks of 16 (token, query head) columns per (request, kv head)
  // workspace layout (bytes)
  size_t ws_ml_off = 0, ws_o_off = 0, ws_bytes = 0;
};

// Numeric limits of the split policy.
constexpr int32_t kMaxSplits = 128;       // splits per generation request
constexpr int32_t kMaxChunk = 2048;        // keys per split, at most
constexpr int64_t kMinDecodeItems = 1408;  // (request, kv head, split) items, at least: 5.5 per CU
// Generation requests carry 1 .. kMaxGenTokens new tokens (a token and its draft tokens).
constexpr int32_t kMaxGenTokens = 64;
// The split pass takes (token, query head) columns of one KV head in blocks of 16; with
// more than kMaxDecodeCols columns per request the generic kernel takes the batch.
constexpr int32_t kMaxDecodeCols = 64;
// The persistent context kernel orders up to kPrefillMaxReqs requests per launch (larger
// batches take several launches).
constexpr int32_t kPrefillMaxReqs = 512;
// The split pass gives a workgroup 4 neighbouring KV heads, one wave each, when the KV
// heads come in fours and either the cache is one byte per element (fp8 / int8) or it is
// bf16 with groups of at least 8 query heads and one block of 16 columns; otherwise one
// head, its waves streaming alternate tiles.  Measured on MI355X at 2048-key splits (split
// pass): 16 fp8 requests of 16K..32K keys 143 us against 161 with one-head workgroups (150
// at 1024-key splits); 128 bf16 GQA-8 requests of 256..4096 keys 203 against 219; but 64
// bf16 MHA requests 397 against 370, and the GQA-8 requests with 4 draft tokens each (two
// column blocks) 492 against 415, so those keep one head per workgroup.
inline int32_t decode_heads_per_wg(int32_t kv_bytes, int32_t num_kv_heads, int32_t group, int32_t col_blocks) {
  if (num_kv_heads % 4 != 0) return 1;
  if (kv_bytes == 1) return 4;
  return kv_bytes == 2 && group >= 8 && col_blocks == 1 ? 4 : 1;
}
// Which specialised kernels this build dispatches to (the generic kernel covers the rest).
constexpr bool kHaveFastDecode = true;
constexpr bool kHaveFastPrefill = true;

int validate_desc(const pkv_attn_desc* d, std::string& err);
int validate_batch(const pkv_attn_desc* d, const pkv_batch_desc* b, BatchPlan* plan, std::string& err);

// Kernel selection for a validated desc (pure function of the desc).
bool desc_fast_decode(const pkv_attn_desc& d);
bool desc_fast_prefill(const pkv_attn_desc& d);

// Decode split policy + workspace layout for a validated batch.
void plan_decode(const pkv_attn_desc& d, const pkv_batch_desc& b, BatchPlan* plan);
size_t workspace_upper_bound(const pkv_attn_desc& d, int32_t max_num_requests, int32_t max_seq_len);

inline int32_t io_bytes(int32_t dt) { return dt == PKV_FP32 ? 4 : dt == PKV_BF16 ? 2 : 1; }
inline int32_t rot_dim(const pkv_attn_desc& d) { return d.rotary_dim ? d.rotary_dim : d.head_dim; }

}  // namespace pkv
