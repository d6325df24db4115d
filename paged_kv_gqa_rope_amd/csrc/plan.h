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
  int32_t col_blocks = 0;     // blocks of 16 (token, query head) columns per (request, kv head)
  int32_t dec_heads = 0;      // KV heads per segment (decode_heads_per_wg)
  int32_t dec_cols = 0;       // columns stored per (piece, KV head): min(16, G * max_gen_n)
  int64_t dec_units = 0;      // 32-key tiles summed over all (request, head group, column block) segments
  int64_t dec_segments = 0;   // generation requests x head groups x col_blocks
  int64_t dec_max_wgs = 0;    // split-pass workgroups the workspace has room for: min(kDecodeMaxWGs, units)
  // workspace layout (bytes)
  size_t ws_pre_off = 0, ws_ml_off = 0, ws_o_off = 0, ws_bytes = 0;
};

// The persistent split pass runs kDecodeWGsPerCU workgroups per CU (all resident at
// once), at most kDecodeMaxWGs, and never more than the batch has 32-key tile units.
constexpr int32_t kDecodeWGsPerCU = 2;
constexpr int32_t kDecodeMaxWGs = 1024;
constexpr int32_t kDecodeTile = 32;        // keys per work unit
// Generation requests carry 1 .. kMaxGenTokens new tokens (a token and its draft tokens).
constexpr int32_t kMaxGenTokens = 64;
// The split pass takes (token, query head) columns of one KV head in blocks of 16; with
// more than kMaxDecodeCols columns per request the generic kernel takes the batch.
constexpr int32_t kMaxDecodeCols = 64;
// The persistent context kernel orders up to kPrefillMaxReqs requests per launch (larger
// batches take several launches).
constexpr int32_t kPrefillMaxReqs = 512;
// The split pass gives a segment 4 neighbouring KV heads, one wave each, when the KV heads
// come in fours and either the cache is one byte per element (fp8 / int8) or it is bf16
// with groups of at least 8 query heads and one block of 16 columns; otherwise one head,
// its waves sharing the tiles.  Four waves reading the neighbouring heads' pieces of the
// same cache rows at about the same time are served faster by HBM; one-head segments win
// where a segment has few query columns per KV head and bf16 rows (MHA, draft tokens with
// several column blocks), measured on MI355X.
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
