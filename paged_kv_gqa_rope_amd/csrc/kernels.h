// Internal launch interface between the C ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"
#include "plan.h"

namespace pkv {

// element formats of io tensors and the KV pool
enum : int { F_FP32 = 0, F_BF16 = 1, F_FP8 = 2, F_INT8 = 3 };
// rotary pairing of the append: none, (j, j + R/2), (2j, 2j + 1)
enum : int { kRopeNone = 0, kRopeNeox = 1, kRopeGptj = 2 };
// per-head normalisation of q and k in the append
enum : int { kNormNone = 0, kNormRms = 1, kNormLayer = 2 };
constexpr int kMaxNormHeads = 256;   // q heads + k heads per token with a norm

struct AppendArgs {
  const void* q;            // may be null (then q_out is null)
  const void* k;
  const void* v;
  int64_t q_stride, kv_stride;   // elements
  const double* cos_sin;    // [max_pos][R/2][2]
  int32_t max_pos;
  void* q_out;
  void* pool;
  const int32_t* ctx_len;   // device n_r
  const int32_t* seq_len;   // device S_r
  const int32_t* table;     // device [B][mbps]
  int32_t B, N, H, Hkv, D, T, R, mbps;
  int64_t num_blocks;
  double inv_k_scale, inv_v_scale;   // fp8 / int8 cache: 1/scale; otherwise 1
  int32_t io_fmt, kv_fmt, rope;   // rope: kRopeNone / kRopeNeox / kRopeGptj
  int32_t max_n;            // largest n_r (grid extent)
  // per-head q/k normalisation before the rotation
  int32_t norm;             // kNormNone / kNormRms / kNormLayer
  double norm_eps;
  const float* qn_w;        // [D] weights for query heads (may be null without q)
  const float* kn_w;        // [D] weights for key heads
  const float* qn_b;        // [D] biases (layer form; may be null: zero)
  const float* kn_b;
  // draft tokens as a tree: rows from gen_row on (generation requests) are rotated at
  // S - n + pos_off[row] instead of S - n + i; null: the chain
  const int32_t* pos_off;
  int32_t gen_row;
};

struct AttnArgs {
  const void* q;
  int64_t q_stride;         // elements
  const void* pool;
  void* out;
  const int32_t* ctx_len;
  const int32_t* seq_len;
  const int32_t* table;
  int32_t B, N, H, Hkv, D, T, mbps;
  int32_t tshift;                // log2(T)
  int64_t num_blocks;
  float scale_log2;         // softmax scale * log2(e)
  float k_scale, v_scale;   // dequantisation scales (1 unless fp8 / int8)
  int32_t io_fmt, kv_fmt;
  int32_t out_fmt;               // io_fmt, or F_FP8: out = e4m3(O * out_mul)
  float out_mul;                 // 1 / out_scale_quant_orig for an fp8 output
  int32_t req_begin, req_end;    // requests [begin, end) handled by this launch
  int32_t row_begin;             // packed row of request req_begin
  int32_t max_n;                 // largest n_r among the handled requests
  // split-KV decode (persistent, balanced split pass)
  int32_t col_blocks;            // blocks of 16 (token, query head) columns per (request, kv head)
  int32_t dec_heads;             // KV heads per segment (1, 2 or 4)
  int32_t dec_cbw;               // waves per head, one column block each (1, 2 or 4)
  int32_t dec_allcols;           // 1: segments (request, head group) carry all column blocks
  int32_t dec_lanes;             // workgroups per range of tiles (head groups x dec_lane_cbs)
  int32_t dec_lane_cbs;          // column blocks with a lane of their own (1 unless one-head segments
                                 // hold one column block each)
  int32_t dec_cols;              // columns stored per (piece, KV head): min(16, G * max_n), or G * max_n (dec_allcols)
  int32_t dec_wgs;               // workgroups of the split pass (ranges x dec_lanes)
  int64_t* ws_pre;               // [generation requests + 1] first tile of each request, total last
  int64_t* ws_row;               // [generation requests + 1] first packed row of each request
  float* ws_ml;                  // [slots][dec_heads][dec_cols][2]  (m, l) per piece; slot (r + range) * lanes + lane
  float* ws_o;                   // [slots][dec_heads][dec_cols][D]  o per piece
  int32_t num_cus;               // compute units of the device
  // draft tokens as a tree (generation launches only): packed row's two mask words, bit j
  // set when the row sees new token j of its request; null: the chain (token i sees 0..i)
  const uint32_t* spec_mask;
};

// Bytes of the library's device scratch array (one per GPU) used by the entry point that
// allocates nothing.
constexpr size_t kScratchBytes = PKV_SCRATCH_BYTES;
// Device address of this device's scratch array (looked up once per device).
hipError_t scratch_device_pointer(void** out);

hipError_t launch_rope_table(double base, int32_t rot, int32_t max_pos, double* cos_sin, hipStream_t s);
hipError_t launch_append(const AppendArgs& a, hipStream_t s);
hipError_t launch_attn_generic(const AttnArgs& a, hipStream_t s);
hipError_t launch_decode_split(const AttnArgs& a, hipStream_t s);
hipError_t launch_decode_combine(const AttnArgs& a, hipStream_t s);
// Mixed batch in one launch: the context requests of ac on ctx_wgs workgroups' worth of
// the persistent context schedule, and the generation split pass of ad (its dec_wgs
// ranges) on the rest of the grid; the combine follows separately.
bool mixed_supported(const AttnArgs& ad, int num_ctx, int G);
hipError_t launch_mixed(const AttnArgs& ac, const int32_t* host_ctx_len, const int32_t* host_seq_len,
                        const AttnArgs& ad, int ctx_wgs, hipStream_t s);
// Persistent context kernel: one launch per kPrefillMaxReqs context requests.
struct PrefillSched {
  int32_t nreq;        // requests of this launch
  int32_t groups;      // 8: KV head g runs in the group of XCD g % 8; 1: one group
  int32_t hpg;         // KV heads per group
  uint16_t rank[kPrefillMaxReqs];   // place of request req_begin + i in the work order (most tiles first)
};
// host_ctx_len, host_seq_len: host copies of n_r and S_r, indexed by request
hipError_t launch_prefill(const AttnArgs& a, const int32_t* host_ctx_len, const int32_t* host_seq_len,
                          hipStream_t s);

}  // namespace pkv
