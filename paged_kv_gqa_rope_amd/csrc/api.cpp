// The extern "C" entry points declared in include/pkv.h: validate on the host, then
// enqueue the kernels of one step on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"
#include "pkv.h"
#include "plan.h"

namespace {

thread_local std::string g_err;

int set_err(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

// ---------------------------------------------------------------- per-device facts
// Looked up once per device (the first call that launches on it), then read from here.
constexpr int kMaxDevices = 64;
struct DeviceInfo {
  int cus = 0;   // compute units
};
std::mutex g_dev_mu;
DeviceInfo g_dev[kMaxDevices];
bool g_dev_ready[kMaxDevices] = {};

hipError_t device_info(DeviceInfo* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (!g_dev_ready[dev]) {
    DeviceInfo info;
    e = hipDeviceGetAttribute(&info.cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    g_dev[dev] = info;
    g_dev_ready[dev] = true;
  }
  *out = g_dev[dev];
  return hipSuccess;
}

// ---------------------------------------------------------------- opt-in kernel timing
// pkv_kernel_timing_enable(1) creates the events up front (kTimingEvents of them, kept for
// reuse); a launch while timing is on takes two from that pool and records them on its
// stream, so entry points never create events.  When the pool runs dry, later launches are
// not timed (pkv_kernel_timings reports how many were dropped through pkv_last_error).
// Cap on the decode split pass's workgroups (0: the default, kDecodeWGsPerCU per CU).
std::atomic<int32_t> g_decode_wgs{0};
// Mixed batches: context and generation parts in one launch (1) or one after the other (0).
std::atomic<int32_t> g_cosched{1};
// Per-CU rates that size the two parts of a mixed launch: the context kernel's matrix
// throughput and the split pass's streaming rate on a CU when few CUs stream.
constexpr double kCtxFlopsPerCU = 3.6e12;
constexpr double kGenBytesPerCU = 40e9;

constexpr size_t kTimingEvents = 8192;
struct TimingRec {
  const char* name;
  hipEvent_t beg, end;
};
std::mutex g_tmu;
// 0: off; 1: one record per kernel launch; 2: one record per phase (the append, the
// context attention, the generation attention: split pass and combine as one span)
int g_timing = 0;
enum TimeLevel { kLaunch = 1, kPhase = 2 };
std::vector<TimingRec> g_recs;
std::vector<hipEvent_t> g_spare;
size_t g_events = 0;        // events created so far (all in g_spare or g_recs)
size_t g_dropped = 0;       // launches not timed because the pool was empty

// Record the launches `launch` makes under `name` when timing is at `level`.
// The lock is never held while `launch` runs (it may time launches of its own).
template <class F>
hipError_t timed_at(int level, const char* name, hipStream_t s, F&& launch) {
  hipEvent_t b = nullptr, e = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_tmu);
    if (g_timing == level) {
      if (g_spare.size() >= 2) {
        e = g_spare.back();
        g_spare.pop_back();
        b = g_spare.back();
        g_spare.pop_back();
      } else {
        ++g_dropped;
      }
    }
  }
  if (!b) return launch();
  (void)hipEventRecord(b, s);
  const hipError_t err = launch();
  (void)hipEventRecord(e, s);
  std::lock_guard<std::mutex> lk(g_tmu);
  g_recs.push_back({name, b, e});
  return err;
}
// One kernel that is also a phase of its own.
template <class F>
hipError_t timed(const char* name, hipStream_t s, F&& launch) {
  return timed_at(kPhase, name, s, [&] { return timed_at(kLaunch, name, s, launch); });
}

int hip_fail(hipError_t e, const char* what) {
  return set_err(PKV_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int fmt_of(int32_t dt) {
  return dt == PKV_FP32 ? pkv::F_FP32 : dt == PKV_BF16 ? pkv::F_BF16 : dt == PKV_INT8 ? pkv::F_INT8 : pkv::F_FP8;
}
bool scaled_cache(int32_t dt) { return dt == PKV_FP8_E4M3 || dt == PKV_INT8; }

int check_rows(const void* p, int64_t stride, int64_t min_elems, int32_t dtype, const char* name) {
  if (stride < min_elems)
    return set_err(PKV_ERR_INVALID_ARG, std::string(name) + ": row stride shorter than one row");
  if (!aligned16(p) || (stride * pkv::io_bytes(dtype)) % 16)
    return set_err(PKV_ERR_INVALID_ARG, std::string(name) + ": rows must start on 16-byte boundaries");
  return PKV_OK;
}

}  // namespace

extern "C" {

int32_t pkv_abi_version(void) { return PKV_ABI_VERSION; }

const char* pkv_last_error(void) { return g_err.c_str(); }

size_t pkv_workspace_size(const pkv_attn_desc* desc, int32_t max_num_requests, int32_t max_seq_len) {
  std::string err;
  if (pkv::validate_desc(desc, err) != PKV_OK) {
    g_err = err;
    return 0;
  }
  return pkv::workspace_upper_bound(*desc, max_num_requests, max_seq_len);
}

size_t pkv_workspace_size_for_batch(const pkv_attn_desc* desc, const pkv_batch_desc* batch) {
  std::string err;
  pkv::BatchPlan plan;
  if (pkv::validate_desc(desc, err) != PKV_OK || pkv::validate_batch(desc, batch, &plan, err) != PKV_OK) {
    g_err = err;
    return 0;
  }
  return plan.ws_bytes;
}

int32_t pkv_rope_cos_sin(double base, int32_t rotary_dim, int32_t max_pos, double* cos_sin, void* stream) {
  if (!(std::isfinite(base) && base > 0.0)) return set_err(PKV_ERR_INVALID_ARG, "rope base must be finite and > 0");
  if (rotary_dim < 2 || rotary_dim % 2) return set_err(PKV_ERR_INVALID_ARG, "rotary_dim must be even and >= 2");
  if (max_pos < 0) return set_err(PKV_ERR_INVALID_ARG, "max_pos < 0");
  if (max_pos == 0) return PKV_OK;
  if (!cos_sin) return set_err(PKV_ERR_INVALID_ARG, "cos_sin is NULL");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e =
      timed("rope_table", s, [&] { return pkv::launch_rope_table(base, rotary_dim, max_pos, cos_sin, s); });
  if (e != hipSuccess) return hip_fail(e, "rope table launch");
  return PKV_OK;
}

static int32_t append_impl(const pkv_attn_desc* desc, const pkv_batch_desc* batch, const pkv_qk_norm* norm,
                           const void* q, int64_t q_row_stride, const void* k, const void* v, int64_t kv_row_stride,
                           const double* rope_cos_sin, int32_t rope_max_pos, void* q_out, void* kv_pool,
                           void* stream, const pkv_spec_tree* tree = nullptr, bool with_tree = false) {
  std::string err;
  int rc = pkv::validate_desc(desc, err);
  if (rc != PKV_OK) return set_err(rc, err);
  pkv::BatchPlan plan;
  rc = pkv::validate_batch(desc, batch, &plan, err);
  if (rc != PKV_OK) return set_err(rc, err);
  if (with_tree && (rc = pkv::validate_tree(batch, plan, tree, err)) != PKV_OK) return set_err(rc, err);
  if (plan.N == 0) return PKV_OK;
  const int32_t H = desc->num_heads, Hkv = desc->num_kv_heads, D = desc->head_dim;
  if ((q == nullptr) != (q_out == nullptr)) return set_err(PKV_ERR_INVALID_ARG, "q and q_out must both be given or both NULL");
  if (!k || !v || !kv_pool) return set_err(PKV_ERR_INVALID_ARG, "k, v and kv_pool must not be NULL");
  if (q) {
    if ((rc = check_rows(q, q_row_stride, static_cast<int64_t>(H) * D, desc->io_dtype, "q")) != PKV_OK) return rc;
    if (!aligned16(q_out)) return set_err(PKV_ERR_INVALID_ARG, "q_out must be 16-byte aligned");
  }
  if ((rc = check_rows(k, kv_row_stride, static_cast<int64_t>(Hkv) * D, desc->io_dtype, "k")) != PKV_OK) return rc;
  if ((rc = check_rows(v, kv_row_stride, static_cast<int64_t>(Hkv) * D, desc->io_dtype, "v")) != PKV_OK) return rc;
  if (!aligned16(kv_pool)) return set_err(PKV_ERR_INVALID_ARG, "kv_pool must be 16-byte aligned");
  if (desc->rope_style != PKV_ROPE_NONE) {
    if (!rope_cos_sin) return set_err(PKV_ERR_INVALID_ARG, "rope_cos_sin is NULL");
    if (!aligned16(rope_cos_sin)) return set_err(PKV_ERR_INVALID_ARG, "rope_cos_sin must be 16-byte aligned");
    if (rope_max_pos < plan.max_S)
      return set_err(PKV_ERR_INVALID_ARG, "rope_max_pos=" + std::to_string(rope_max_pos) +
                                              " does not cover position " + std::to_string(plan.max_S - 1));
  }
  const int32_t nkind = norm ? norm->kind : PKV_NORM_NONE;
  if (nkind != PKV_NORM_NONE) {
    if (nkind != PKV_NORM_RMS && nkind != PKV_NORM_LAYER)
      return set_err(PKV_ERR_INVALID_ARG, "unknown qk norm kind " + std::to_string(nkind));
    if (!(norm->eps >= 0.f) || !std::isfinite(norm->eps))
      return set_err(PKV_ERR_INVALID_ARG, "qk norm eps must be finite and >= 0");
    if (!norm->k_weight || !aligned16(norm->k_weight) || (q && (!norm->q_weight || !aligned16(norm->q_weight))))
      return set_err(PKV_ERR_INVALID_ARG, "qk norm weights missing or not 16-byte aligned");
    if (nkind == PKV_NORM_LAYER && ((norm->q_bias && !aligned16(norm->q_bias)) || (norm->k_bias && !aligned16(norm->k_bias))))
      return set_err(PKV_ERR_INVALID_ARG, "qk norm biases must be 16-byte aligned");
    if ((q ? H : 0) + Hkv > pkv::kMaxNormHeads)
      return set_err(PKV_ERR_UNSUPPORTED, "qk norm supports at most " + std::to_string(pkv::kMaxNormHeads) +
                                              " q + k heads per token");
  }
  pkv::AppendArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.q_stride = q_row_stride;
  a.kv_stride = kv_row_stride;
  a.cos_sin = rope_cos_sin;
  a.max_pos = rope_max_pos;
  a.q_out = q_out;
  a.pool = kv_pool;
  a.ctx_len = batch->context_lengths;
  a.seq_len = batch->sequence_lengths;
  a.table = batch->kv_cache_block_offsets;
  a.B = plan.B;
  a.N = plan.N;
  a.H = H;
  a.Hkv = Hkv;
  a.D = D;
  a.T = desc->tokens_per_block;
  a.R = pkv::rot_dim(*desc);
  a.mbps = batch->max_blocks_per_seq;
  a.num_blocks = batch->num_pool_blocks;
  const bool quant = scaled_cache(desc->kv_dtype);
  a.inv_k_scale = quant ? 1.0 / static_cast<double>(desc->k_scale_quant_orig) : 1.0;
  a.inv_v_scale = quant ? 1.0 / static_cast<double>(desc->v_scale_quant_orig) : 1.0;
  a.io_fmt = fmt_of(desc->io_dtype);
  a.kv_fmt = fmt_of(desc->kv_dtype);
  a.rope = desc->rope_style == PKV_ROPE_NEOX ? pkv::kRopeNeox
           : desc->rope_style == PKV_ROPE_GPTJ ? pkv::kRopeGptj : pkv::kRopeNone;
  a.max_n = plan.max_n;
  a.pos_off = with_tree ? tree->position_offsets : nullptr;
  a.gen_row = plan.ctx_tokens;
  a.norm = nkind == PKV_NORM_RMS ? pkv::kNormRms : nkind == PKV_NORM_LAYER ? pkv::kNormLayer : pkv::kNormNone;
  if (a.norm != pkv::kNormNone) {
    a.norm_eps = static_cast<double>(norm->eps);
    a.qn_w = norm->q_weight;
    a.kn_w = norm->k_weight;
    a.qn_b = a.norm == pkv::kNormLayer ? norm->q_bias : nullptr;
    a.kn_b = a.norm == pkv::kNormLayer ? norm->k_bias : nullptr;
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = timed("append_rope", s, [&] { return pkv::launch_append(a, s); });
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return PKV_OK;
}

int32_t pkv_append_rope(const pkv_attn_desc* desc, const pkv_batch_desc* batch, const void* q, int64_t q_row_stride,
                        const void* k, const void* v, int64_t kv_row_stride, const double* rope_cos_sin,
                        int32_t rope_max_pos, void* q_out, void* kv_pool, void* stream) {
  return append_impl(desc, batch, nullptr, q, q_row_stride, k, v, kv_row_stride, rope_cos_sin, rope_max_pos, q_out,
                     kv_pool, stream);
}

int32_t pkv_append_qknorm_rope(const pkv_attn_desc* desc, const pkv_batch_desc* batch, const pkv_qk_norm* norm,
                               const void* q, int64_t q_row_stride, const void* k, const void* v,
                               int64_t kv_row_stride, const double* rope_cos_sin, int32_t rope_max_pos,
                               void* q_out, void* kv_pool, void* stream) {
  return append_impl(desc, batch, norm, q, q_row_stride, k, v, kv_row_stride, rope_cos_sin, rope_max_pos, q_out,
                     kv_pool, stream);
}

int32_t pkv_append_rope_tree(const pkv_attn_desc* desc, const pkv_batch_desc* batch, const pkv_spec_tree* tree,
                             const void* q, int64_t q_row_stride, const void* k, const void* v,
                             int64_t kv_row_stride, const double* rope_cos_sin, int32_t rope_max_pos, void* q_out,
                             void* kv_pool, void* stream) {
  return append_impl(desc, batch, nullptr, q, q_row_stride, k, v, kv_row_stride, rope_cos_sin, rope_max_pos, q_out,
                     kv_pool, stream, tree, true);
}

// use_scratch: the split-KV partials go to the library's scratch array instead of the
// caller's workspace (workspace and workspace_bytes are then ignored).
static int32_t attention_impl(const pkv_attn_desc* desc, const pkv_batch_desc* batch, const void* q,
                              int64_t q_row_stride, const void* kv_pool, void* out, bool fp8_out, float out_scale,
                              void* workspace, size_t workspace_bytes, void* stream, bool use_scratch = false,
                              const pkv_spec_tree* tree = nullptr, bool with_tree = false) {
  std::string err;
  int rc = pkv::validate_desc(desc, err);
  if (rc != PKV_OK) return set_err(rc, err);
  pkv::BatchPlan plan;
  rc = pkv::validate_batch(desc, batch, &plan, err);
  if (rc != PKV_OK) return set_err(rc, err);
  if (with_tree && (rc = pkv::validate_tree(batch, plan, tree, err)) != PKV_OK) return set_err(rc, err);
  if (plan.N == 0) return PKV_OK;
  const int32_t H = desc->num_heads, D = desc->head_dim;
  if (!q || !kv_pool || !out) return set_err(PKV_ERR_INVALID_ARG, "q, kv_pool and out must not be NULL");
  if ((rc = check_rows(q, q_row_stride, static_cast<int64_t>(H) * D, desc->io_dtype, "q")) != PKV_OK) return rc;
  if (!aligned16(out) || !aligned16(kv_pool)) return set_err(PKV_ERR_INVALID_ARG, "out and kv_pool must be 16-byte aligned");
  if (fp8_out && !(std::isfinite(out_scale) && out_scale > 0.f && std::isfinite(1.0f / out_scale)))
    return set_err(PKV_ERR_INVALID_ARG, "out_scale_quant_orig must be finite and > 0 (with a finite reciprocal)");
  if (use_scratch) {
    if (plan.ws_bytes > pkv::kScratchBytes)
      return set_err(PKV_ERR_WORKSPACE, "this batch needs " + std::to_string(plan.ws_bytes) +
                                            " bytes of scratch; the library's scratch array holds " +
                                            std::to_string(pkv::kScratchBytes));
    workspace = nullptr;
    workspace_bytes = 0;
    if (plan.ws_bytes > 0) {
      const hipError_t se = pkv::scratch_device_pointer(&workspace);
      if (se != hipSuccess) return hip_fail(se, "scratch symbol lookup");
      workspace_bytes = pkv::kScratchBytes;
    }
  }
  if (plan.ws_bytes > 0) {
    if (!workspace || workspace_bytes < plan.ws_bytes)
      return set_err(PKV_ERR_WORKSPACE, "workspace of " + std::to_string(plan.ws_bytes) + " bytes required, " +
                                            std::to_string(workspace ? workspace_bytes : 0) + " given");
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
      return set_err(PKV_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  }
  pkv::AttnArgs a{};
  a.q = q;
  a.q_stride = q_row_stride;
  a.pool = kv_pool;
  a.out = out;
  a.ctx_len = batch->context_lengths;
  a.seq_len = batch->sequence_lengths;
  a.table = batch->kv_cache_block_offsets;
  a.B = plan.B;
  a.N = plan.N;
  a.H = H;
  a.Hkv = desc->num_kv_heads;
  a.D = D;
  a.T = desc->tokens_per_block;
  a.tshift = 0;
  while ((1 << a.tshift) < a.T) ++a.tshift;
  a.mbps = batch->max_blocks_per_seq;
  a.num_blocks = batch->num_pool_blocks;
  const double scale = desc->softmax_scale > 0.f ? desc->softmax_scale : 1.0 / std::sqrt(static_cast<double>(D));
  a.scale_log2 = static_cast<float>(scale * 1.4426950408889634);
  const bool quant = scaled_cache(desc->kv_dtype);
  a.k_scale = quant ? desc->k_scale_quant_orig : 1.f;
  a.v_scale = quant ? desc->v_scale_quant_orig : 1.f;
  a.io_fmt = fmt_of(desc->io_dtype);
  a.kv_fmt = fmt_of(desc->kv_dtype);
  a.out_fmt = fp8_out ? pkv::F_FP8 : a.io_fmt;
  a.out_mul = fp8_out ? static_cast<float>(1.0 / static_cast<double>(out_scale)) : 1.f;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  DeviceInfo dev;
  hipError_t e = device_info(&dev);
  if (e != hipSuccess) return hip_fail(e, "device query");
  a.num_cus = dev.cus;
  // generation part's arguments (the context part's are set below)
  pkv::AttnArgs ad = a;
  ad.spec_mask = with_tree ? tree->packed_mask : nullptr;
  if (plan.num_gen > 0) {
    ad.req_begin = plan.num_ctx;
    ad.req_end = plan.B;
    ad.row_begin = plan.ctx_tokens;
    ad.max_n = plan.max_gen_n;
    ad.col_blocks = plan.col_blocks;
    if (plan.fast_decode) {
      ad.dec_heads = plan.dec_heads;
      ad.dec_cbw = plan.dec_cbw;
      ad.dec_allcols = plan.dec_allcols ? 1 : 0;
      ad.dec_cols = plan.dec_cols;
      ad.dec_lanes = plan.dec_lanes;
      ad.dec_lane_cbs = plan.dec_lane_cbs;
      ad.ws_pre = reinterpret_cast<int64_t*>(static_cast<char*>(workspace) + plan.ws_pre_off);
      ad.ws_row = ad.ws_pre + (plan.num_gen + 1);
      ad.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.ws_ml_off);
      ad.ws_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.ws_o_off);
    }
  }
  // ranges of tiles of the split pass, each on one workgroup per lane, for a target count
  auto set_ranges = [&](int64_t target) {
    const int64_t lanes = std::max(plan.dec_lanes, 1);
    const int64_t ranges = std::max<int64_t>(1, std::min(target, plan.dec_max_wgs) / lanes);
    ad.dec_wgs = static_cast<int32_t>(ranges * lanes);
  };
  const int32_t cap = g_decode_wgs.load(std::memory_order_relaxed);
  a.req_begin = 0;
  a.req_end = plan.num_ctx;
  a.row_begin = 0;
  a.max_n = plan.max_ctx_n;
  const int G = H / desc->num_kv_heads;
  const bool mixed = g_cosched.load(std::memory_order_relaxed) != 0 && plan.num_ctx > 0 && plan.num_gen > 0 &&
                     plan.fast_prefill && plan.fast_decode && dev.cus >= 16 && pkv::mixed_supported(ad, plan.num_ctx, G);
  if (mixed) {
    // CUs for the generation part in proportion to its estimated time: context flops at
    // the context kernel's per-CU rate against generation bytes at a per-CU streaming rate
    double flops = 0.0, bytes = 0.0;
    for (int32_t r = 0; r < plan.B; ++r) {
      const double n = batch->host_context_lengths[r], S = batch->host_sequence_lengths[r];
      if (r < plan.num_ctx) flops += 4.0 * H * D * (n * (S - n) + n * (n + 1) / 2);
      else bytes += 2.0 * S * desc->num_kv_heads * D * (desc->kv_dtype == PKV_FP32 ? 4 : desc->kv_dtype == PKV_BF16 ? 2 : 1);
    }
    const double tc = flops / kCtxFlopsPerCU, tg = bytes / kGenBytesPerCU;
    int64_t gen_cus = cap > 0 ? cap : static_cast<int64_t>(std::llround(dev.cus * tg / std::max(tc + tg, 1e-30)));
    gen_cus = std::min<int64_t>(std::max<int64_t>(gen_cus / 8 * 8, 8), dev.cus - 8);
    set_ranges(gen_cus);
    const int ctx_wgs = std::max(8, (dev.cus - ad.dec_wgs) / 8 * 8);
    const char* failed = nullptr;
    e = timed_at(kPhase, "mixed", s, [&] {
      hipError_t le = timed_at(kLaunch, "mixed", s, [&] {
        return pkv::launch_mixed(a, batch->host_context_lengths, batch->host_sequence_lengths, ad, ctx_wgs, s);
      });
      if (le != hipSuccess) {
        failed = "mixed launch";
        return le;
      }
      le = timed_at(kLaunch, "decode_combine", s, [&] { return pkv::launch_decode_combine(ad, s); });
      if (le != hipSuccess) failed = "decode combine launch";
      return le;
    });
    if (e != hipSuccess) return hip_fail(e, failed ? failed : "mixed launch");
    return PKV_OK;
  }
  if (plan.num_ctx > 0) {
    if (plan.fast_prefill)
      e = timed("prefill_mfma", s, [&] { return pkv::launch_prefill(a, batch->host_context_lengths, batch->host_sequence_lengths, s); });
    else
      e = timed("attn_generic_ctx", s, [&] { return pkv::launch_attn_generic(a, s); });
    if (e != hipSuccess) return hip_fail(e, "context attention launch");
  }
  if (plan.num_gen > 0) {
    if (plan.fast_decode) {
      set_ranges(cap > 0 ? cap : static_cast<int64_t>(pkv::kDecodeWGsPerCU) * std::max(dev.cus, 1));
      const char* failed = nullptr;
      e = timed_at(kPhase, "decode", s, [&] {
        hipError_t le = timed_at(kLaunch, "decode_split", s, [&] { return pkv::launch_decode_split(ad, s); });
        if (le != hipSuccess) {
          failed = "decode launch";
          return le;
        }
        le = timed_at(kLaunch, "decode_combine", s, [&] { return pkv::launch_decode_combine(ad, s); });
        if (le != hipSuccess) failed = "decode combine launch";
        return le;
      });
      if (e != hipSuccess) return hip_fail(e, failed ? failed : "decode launch");
    } else {
      e = timed("attn_generic_gen", s, [&] { return pkv::launch_attn_generic(ad, s); });
      if (e != hipSuccess) return hip_fail(e, "generation attention launch");
    }
  }
  return PKV_OK;
}

int32_t pkv_attention_forward(const pkv_attn_desc* desc, const pkv_batch_desc* batch, const void* q,
                              int64_t q_row_stride, const void* kv_pool, void* out, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return attention_impl(desc, batch, q, q_row_stride, kv_pool, out, false, 1.f, workspace, workspace_bytes, stream);
}

int32_t pkv_attention_forward_fp8_out(const pkv_attn_desc* desc, const pkv_batch_desc* batch, const void* q,
                                      int64_t q_row_stride, const void* kv_pool, float out_scale_quant_orig,
                                      void* out, void* workspace, size_t workspace_bytes, void* stream) {
  return attention_impl(desc, batch, q, q_row_stride, kv_pool, out, true, out_scale_quant_orig, workspace,
                        workspace_bytes, stream);
}

int32_t pkv_attention_forward_tree(const pkv_attn_desc* desc, const pkv_batch_desc* batch, const pkv_spec_tree* tree,
                                   const void* q, int64_t q_row_stride, const void* kv_pool, void* out,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  return attention_impl(desc, batch, q, q_row_stride, kv_pool, out, false, 1.f, workspace, workspace_bytes, stream,
                        false, tree, true);
}

int32_t pkv_attention_forward_noalloc(const pkv_attn_desc* desc, const pkv_batch_desc* batch, const void* q,
                                      int64_t q_row_stride, const void* kv_pool, void* out, void* stream) {
  return attention_impl(desc, batch, q, q_row_stride, kv_pool, out, false, 1.f, nullptr, 0, stream, true);
}

int32_t pkv_set_coschedule(int32_t on) {
  if (on < 0) return g_cosched.load();
  return g_cosched.exchange(on ? 1 : 0);
}

int32_t pkv_set_decode_workgroups(int32_t n) {
  if (n < 0) return g_decode_wgs.load();
  return g_decode_wgs.exchange(n);
}

int32_t pkv_kernel_timing_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_tmu);
  for (auto& r : g_recs) {
    g_spare.push_back(r.beg);
    g_spare.push_back(r.end);
  }
  g_recs.clear();
  g_dropped = 0;
  if (on) {
    while (g_events < kTimingEvents) {
      hipEvent_t e = nullptr;
      if (hipEventCreate(&e) != hipSuccess) return set_err(PKV_ERR_HIP, "event create failed");
      g_spare.push_back(e);
      ++g_events;
    }
  }
  g_timing = on == 2 ? kPhase : on ? kLaunch : 0;
  return PKV_OK;
}

int32_t pkv_kernel_timings(const char** names, float* milliseconds, int32_t max_entries) {
  std::lock_guard<std::mutex> lk(g_tmu);
  const int32_t n = static_cast<int32_t>(g_recs.size());
  for (int32_t i = 0; i < n && i < max_entries; ++i) {
    if (hipEventSynchronize(g_recs[i].end) != hipSuccess) return set_err(PKV_ERR_HIP, "event synchronize failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, g_recs[i].beg, g_recs[i].end) != hipSuccess)
      return set_err(PKV_ERR_HIP, "event elapsed time failed");
    if (names) names[i] = g_recs[i].name;
    if (milliseconds) milliseconds[i] = ms;
  }
  if (g_dropped) g_err = std::to_string(g_dropped) + " launches were not timed (event pool exhausted)";
  return n;
}

}  // extern "C"
