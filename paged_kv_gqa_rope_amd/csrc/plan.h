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
  int32_t dec_heads = 0;      // KV heads per segment
  int32_t dec_cbw = 1;        // waves per head, one column block each
  bool dec_allcols = false;   // segments (request, head group) carry all column blocks
  int32_t dec_cols = 0;       // columns stored per (piece, KV head): min(16, G * max_gen_n), or G * max_gen_n
                              // when segments carry all column blocks
  int64_t dec_units = 0;      // 32-key tiles summed over the generation requests
  int32_t dec_lane_cbs = 1;   // column blocks with a lane of their own (one-head segments with drafts)
  int32_t dec_lanes = 0;      // lanes: head groups x dec_lane_cbs; each range of tiles runs on one per lane
  int64_t dec_segments = 0;   // generation requests x lanes
  int64_t dec_max_wgs = 0;    // split-pass workgroups the workspace has room for: a multiple of the lanes,
                              // at most max(kDecodeMaxWGs, lanes), at most units x lanes
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
// come in fours; otherwise one head, its waves sharing the tiles.  Four waves reading the
// neighbouring heads' pieces of the same cache rows at about the same time are served
// faster by HBM.  Measured on MI355X with the balanced split pass (split pass, us, four
// heads against one): 64 bf16 MHA requests of 528..4022 keys 344 / 348; 128 GQA-8
// requests with 4 draft tokens each (two column blocks) 365 / 402; 128 GQA-8 requests
// 179 / 180; 16 fp8 requests of 16K..32K keys 142 / 141.
inline int32_t decode_heads_per_wg(int32_t num_kv_heads) { return num_kv_heads % 4 == 0 ? 4 : 1; }
// With several column blocks (draft tokens) and KV heads in fours, a segment carries all
// column blocks of 4 / cbw heads, one wave per (head, column block), cbw = 2 or 4: the
// waves of one head load the same tiles at about the same time, HBM serving them once.
// Measured (128 GQA-8 requests with 4 draft tokens, two column blocks, split pass): 244 us
// against 363 with one segment per column block, and 294 for a pass that streams the
// tiles of 4 heads through an LDS ring shared by all column blocks (its in-flight bytes
// are bounded by LDS).
inline int32_t decode_column_waves(int32_t num_kv_heads, int32_t col_blocks) {
  if (num_kv_heads % 4 != 0 || col_blocks <= 1) return 1;
  return col_blocks == 2 ? 2 : 4;
}
// Which specialised kernels this build dispatches to (the generic kernel covers the rest).
constexpr bool kHaveFastDecode = true;
constexpr bool kHaveFastPrefill = true;

int validate_desc(const pkv_attn_desc* d, std::string& err);
int validate_batch(const pkv_attn_desc* d, const pkv_batch_desc* b, BatchPlan* plan, std::string& err);
// Host check of a draft tree for a validated batch: every generation row's position
// offset in 0 .. n-1, its own mask bit set and no bit at or past n; pointers given and
// aligned.
int validate_tree(const pkv_batch_desc* b, const BatchPlan& plan, const pkv_spec_tree* t, std::string& err);

// Kernel selection for a validated desc (pure function of the desc).
bool desc_fast_decode(const pkv_attn_desc& d);
bool desc_fast_prefill(const pkv_attn_desc& d);

// Decode split policy + workspace layout for a validated batch.
void plan_decode(const pkv_attn_desc& d, const pkv_batch_desc& b, BatchPlan* plan);
size_t workspace_upper_bound(const pkv_attn_desc& d, int32_t max_num_requests, int32_t max_seq_len);

inline int32_t io_bytes(int32_t dt) { return dt == PKV_FP32 ? 4 : dt == PKV_BF16 ? 2 : 1; }
inline int32_t rot_dim(const pkv_attn_desc& d) { return d.rotary_dim ? d.rotary_dim : d.head_dim; }

}  // namespace pkv
