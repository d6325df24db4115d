// Host driver for the batch validation and split planning (plan.cpp), built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_plan_sanitized.py.
// It prints one "case <name> <status>" line per fixed case, then checks random batches:
// every accepted batch's plan is consistent and its workspace fits the upper bound.
#include <cstdio>
#include <algorithm>
#include <array>
#include <cstdlib>
#include <random>
#include <string>
#include <vector>

#include "plan.h"

namespace {

pkv_attn_desc base_desc() {
  pkv_attn_desc d{};
  d.num_heads = 32;
  d.num_kv_heads = 8;
  d.head_dim = 128;
  d.tokens_per_block = 64;
  d.io_dtype = PKV_BF16;
  d.kv_dtype = PKV_BF16;
  d.rope_style = PKV_ROPE_NEOX;
  d.rotary_dim = 0;
  d.softmax_scale = 0.f;
  d.k_scale_quant_orig = 1.f;
  d.v_scale_quant_orig = 1.f;
  d.max_num_tokens = 8192;
  return d;
}

// A batch with its own host arrays; the "device" pointers point at the same host memory
// (validation only checks that they are given).
struct Batch {
  std::vector<int32_t> types, n, S, table;
  int32_t width = 1;
  pkv_batch_desc desc{};
  void build(int64_t pool, bool host_table = true) {
    desc = pkv_batch_desc{};
    desc.num_requests = static_cast<int32_t>(types.size());
    int32_t tot = 0, mctx = 0;
    for (size_t r = 0; r < types.size(); ++r) {
      tot += n[r];
      if (types[r] == PKV_REQ_CONTEXT && n[r] > mctx) mctx = n[r];
    }
    desc.num_tokens = tot;
    desc.max_context_length = mctx;
    desc.max_blocks_per_seq = width;
    desc.host_request_types = types.data();
    desc.host_context_lengths = n.data();
    desc.host_sequence_lengths = S.data();
    desc.context_lengths = n.data();
    desc.sequence_lengths = S.data();
    desc.kv_cache_block_offsets = table.data();
    desc.host_kv_cache_block_offsets = host_table ? table.data() : nullptr;
    desc.num_pool_blocks = pool;
  }
};

// requests (type, n, S) with consecutive block IDs; returns the pool size used
int64_t fill(Batch& b, const std::vector<std::array<int32_t, 3>>& reqs, int32_t T) {
  b.types.clear();
  b.n.clear();
  b.S.clear();
  int32_t width = 1;
  for (auto& q : reqs) {
    b.types.push_back(q[0]);
    b.n.push_back(q[1]);
    b.S.push_back(q[2]);
    width = std::max(width, (q[2] + T - 1) / T);
  }
  b.width = width;
  b.table.assign(reqs.size() * width, -1);
  int64_t next = 0;
  for (size_t r = 0; r < reqs.size(); ++r)
    for (int32_t j = 0; j < (reqs[r][2] + T - 1) / T; ++j) b.table[r * width + j] = static_cast<int32_t>(next++);
  return std::max<int64_t>(next, 1);
}

int run(const char* name, const pkv_attn_desc* d, const pkv_batch_desc* b) {
  std::string err;
  int rc = pkv::validate_desc(d, err);
  if (rc == PKV_OK && b) {
    pkv::BatchPlan p;
    rc = pkv::validate_batch(d, b, &p, err);
  }
  std::printf("case %s %d\n", name, rc);
  return rc;
}

// A draft tree's host and "device" arrays for a batch (the device pointers alias the
// host arrays, 8-byte aligned; validation reads only the host copies).
struct Tree {
  std::vector<int32_t> off;
  std::vector<uint64_t> mask64;                      // two 32-bit words per row
  pkv_spec_tree t{};
  // a valid tree per generation request: parent of token i drawn from 0 .. i-1
  void random(const Batch& b, std::mt19937_64& rng) {
    off.assign(b.desc.num_tokens, 0);
    mask64.assign(b.desc.num_tokens, 0);
    int64_t row = 0;
    for (size_t r = 0; r < b.types.size(); ++r) {
      const int32_t n = b.n[r];
      if (b.types[r] == PKV_REQ_GENERATION) {
        std::vector<int32_t> depth(n, 0);
        for (int32_t i = 0; i < n; ++i) {
          uint64_t m = 1ull << i;
          if (i > 0) {
            const int32_t par = static_cast<int32_t>(rng() % static_cast<uint64_t>(i));
            depth[i] = depth[par] + 1;
            m |= mask64[row + par];
          }
          off[row + i] = depth[i];
          mask64[row + i] = m;
        }
      }
      row += n;
    }
    point();
  }
  void point() {
    t.host_position_offsets = off.data();
    t.position_offsets = off.data();
    t.host_packed_mask = reinterpret_cast<const uint32_t*>(mask64.data());
    t.packed_mask = reinterpret_cast<const uint32_t*>(mask64.data());
  }
};

int run_tree(const char* name, const pkv_attn_desc* d, const pkv_batch_desc* b, const pkv_spec_tree* t) {
  std::string err;
  int rc = pkv::validate_desc(d, err);
  pkv::BatchPlan p;
  if (rc == PKV_OK) rc = pkv::validate_batch(d, b, &p, err);
  if (rc == PKV_OK) rc = pkv::validate_tree(b, p, t, err);
  std::printf("case %s %d\n", name, rc);
  return rc;
}

}  // namespace

int main(int argc, char** argv) {
  const int fuzz = argc > 1 ? std::atoi(argv[1]) : 2000;
  const int C = PKV_REQ_CONTEXT, G = PKV_REQ_GENERATION;
  pkv_attn_desc d = base_desc();
  Batch b;

  // ---- descriptors
  run("desc_null", nullptr, nullptr);
  { auto x = d; x.head_dim = 96; run("head_dim_96", &x, nullptr); }
  { auto x = d; x.tokens_per_block = 48; run("tokens_per_block_48", &x, nullptr); }
  { auto x = d; x.num_heads = 30; run("heads_not_multiple", &x, nullptr); }
  { auto x = d; x.rotary_dim = 24; run("rotary_dim_24", &x, nullptr); }
  { auto x = d; x.rotary_dim = 256; run("rotary_dim_gt_head_dim", &x, nullptr); }
  { auto x = d; x.kv_dtype = PKV_FP8_E4M3; x.k_scale_quant_orig = 0.f; run("fp8_zero_scale", &x, nullptr); }
  { auto x = d; x.io_dtype = PKV_FP8_E4M3; run("io_fp8", &x, nullptr); }
  { auto x = d; x.softmax_scale = 1.f / 0.f; run("softmax_scale_inf", &x, nullptr); }

  // ---- batches
  int64_t pool = fill(b, {{C, 100, 100}, {G, 1, 300}}, 64);
  b.build(pool);
  run("ok_mixed", &d, &b.desc);
  pool = fill(b, {{G, 1, 300}, {C, 100, 100}}, 64);
  b.build(pool);
  run("order", &d, &b.desc);
  pool = fill(b, {{C, 100, 132}}, 64);
  b.build(pool);
  run("chunk_align", &d, &b.desc);
  pool = fill(b, {{C, 8000, 8000}, {C, 300, 300}}, 64);
  b.build(pool);
  run("budget", &d, &b.desc);
  pool = fill(b, {{C, 100, 100}, {G, 1, 300}}, 64);
  b.build(pool - 1);
  run("block_id_outside_pool", &d, &b.desc);
  pool = fill(b, {{C, 100, 100}, {G, 1, 300}}, 64);
  b.width = 2;
  b.build(pool);
  run("table_too_narrow", &d, &b.desc);
  pool = fill(b, {{G, 65, 300}}, 64);
  b.build(pool);
  run("too_many_draft_tokens", &d, &b.desc);
  pool = fill(b, {{G, 5, 3}}, 64);
  b.build(pool);
  run("sequence_shorter_than_chunk", &d, &b.desc);
  pool = fill(b, {{C, 100, 100}, {G, 1, 300}}, 64);
  b.build(pool);
  b.desc.num_tokens = 7;
  run("num_tokens_mismatch", &d, &b.desc);
  b.build(pool);
  b.desc.max_context_length = 99;
  run("max_context_length_short", &d, &b.desc);
  b.build(pool);
  b.desc.host_sequence_lengths = nullptr;
  run("host_lengths_null", &d, &b.desc);
  b.build(pool);
  b.types[1] = 7;
  run("bad_request_type", &d, &b.desc);
  b.types[1] = G;
  b.build(pool);
  b.n[0] = 0;
  b.S[0] = 0;
  run("zero_context_length", &d, &b.desc);
  pkv_batch_desc empty{};
  run("empty", &d, &empty);

  // ---- draft trees (one context request, then two generation requests with 3 and 5 tokens)
  {
    std::mt19937_64 trng(7);
    pool = fill(b, {{C, 64, 64}, {G, 3, 300}, {G, 5, 90}}, 64);
    b.build(pool);
    Tree t;
    t.random(b, trng);
    run_tree("tree_ok", &d, &b.desc, &t.t);
    t.off[64 + 2] = 3;                               // offset past n - 1 = 2
    run_tree("tree_offset_past_n", &d, &b.desc, &t.t);
    t.random(b, trng);
    t.mask64[64 + 3 + 4] &= ~(1ull << 4);            // last token lacks its own bit
    run_tree("tree_own_bit_missing", &d, &b.desc, &t.t);
    t.random(b, trng);
    t.mask64[64 + 1] |= 1ull << 40;                  // a bit in the high word, past n = 3
    run_tree("tree_bit_past_n", &d, &b.desc, &t.t);
    run_tree("tree_null", &d, &b.desc, nullptr);
  }

  // ---- random batches: accepted ones plan consistently and fit the workspace bound
  std::mt19937_64 rng(12345);
  auto U = [&](int lo, int hi) { return static_cast<int32_t>(std::uniform_int_distribution<int>(lo, hi)(rng)); };
  const int heads[][2] = {{32, 32}, {32, 8}, {64, 8}, {16, 4}, {8, 1}, {40, 8}};
  const int dts[] = {PKV_BF16, PKV_FP8_E4M3, PKV_INT8, PKV_FP32};
  int accepted = 0;
  for (int it = 0; it < fuzz; ++it) {
    pkv_attn_desc x = base_desc();
    const auto& hh = heads[U(0, 5)];
    x.num_heads = hh[0];
    x.num_kv_heads = hh[1];
    x.tokens_per_block = 16 << U(0, 4);
    x.kv_dtype = dts[U(0, 3)];
    x.io_dtype = x.kv_dtype == PKV_FP32 || U(0, 4) == 0 ? PKV_FP32 : PKV_BF16;
    x.head_dim = U(0, 3) == 0 ? 64 : 128;
    x.max_num_tokens = U(1, 20000);
    const int T = x.tokens_per_block;
    std::vector<std::array<int32_t, 3>> reqs;
    const int nc = U(0, 6), ng = U(0, 40);
    for (int i = 0; i < nc; ++i) {
      int32_t past = T * U(0, 40);
      if (U(0, 20) == 0) past += U(1, T - 1);          // sometimes misaligned
      const int32_t n = U(1, 3000);
      reqs.push_back({C, n, past + n});
    }
    for (int i = 0; i < ng; ++i) {
      const int32_t n = U(0, 10) == 0 ? U(1, 70) : 1;
      reqs.push_back({G, n, U(0, 40000) + n});
    }
    if (U(0, 30) == 0 && reqs.size() > 1) std::swap(reqs.front(), reqs.back());
    pool = fill(b, reqs, T);
    if (U(0, 30) == 0 && !b.table.empty()) b.table[U(0, static_cast<int>(b.table.size()) - 1)] = U(-3, static_cast<int>(pool) + 3);
    b.build(pool);
    std::string err;
    pkv::BatchPlan p;
    if (pkv::validate_desc(&x, err) != PKV_OK) continue;
    if (pkv::validate_batch(&x, &b.desc, &p, err) != PKV_OK) {
      if (err.empty()) { std::printf("FAIL empty error message\n"); return 1; }
      continue;
    }
    ++accepted;
    int32_t maxS = 1;
    for (int32_t s : b.S) maxS = std::max(maxS, s);
    const size_t bound = pkv::workspace_upper_bound(x, b.desc.num_requests, maxS);
    if (p.ws_bytes > bound) {
      std::printf("FAIL workspace %zu > bound %zu (iteration %d)\n", p.ws_bytes, bound, it);
      return 1;
    }
    if (p.fast_decode) {
      // work units recounted from the lengths: ceil(S/32) tiles per (head group, column block)
      const int64_t Gq = x.num_heads / x.num_kv_heads, hgs = x.num_kv_heads / p.dec_heads;
      const bool all = p.dec_allcols;
      int64_t units = 0;
      for (size_t r = p.num_ctx; r < b.S.size(); ++r) units += (b.S[r] + 31) / 32;
      const int64_t lanes = hgs * (all ? 1 : p.col_blocks);
      // heads x column waves fill the 4 waves (or one head whose waves share the tiles)
      const bool heads_ok = (p.dec_heads == 1 && p.dec_cbw == 1) || p.dec_heads * p.dec_cbw == 4;
      const bool waves_ok = p.dec_cbw == 1 || (x.num_kv_heads % 4 == 0 && p.dec_cbw >= p.col_blocks && all);
      const int64_t cols = all ? Gq * p.max_gen_n : std::min<int64_t>(16, Gq * p.max_gen_n);
      const int64_t max_wgs = lanes * std::min<int64_t>(std::max<int64_t>(1, pkv::kDecodeMaxWGs / lanes), units);
      if (!waves_ok || x.num_kv_heads % p.dec_heads != 0 || units != p.dec_units || !heads_ok ||
          p.dec_lanes != lanes || p.dec_max_wgs != max_wgs || p.dec_cols != cols ||
          p.dec_segments != static_cast<int64_t>(p.num_gen) * lanes) {
        std::printf("FAIL split plan (iteration %d)\n", it);
        return 1;
      }
    }
    if (p.num_ctx + p.num_gen != p.B || p.N != b.desc.num_tokens) {
      std::printf("FAIL plan counts (iteration %d)\n", it);
      return 1;
    }
    // a random valid tree is accepted; the same tree with one planted fault is not
    if (p.num_gen > 0 && p.N > 0) {
      Tree t;
      t.random(b, rng);
      if (pkv::validate_tree(&b.desc, p, &t.t, err) != PKV_OK) {
        std::printf("FAIL valid tree rejected: %s (iteration %d)\n", err.c_str(), it);
        return 1;
      }
      const int32_t r = U(p.num_ctx, p.B - 1);
      int64_t row = 0;
      for (int32_t j = 0; j < r; ++j) row += b.n[j];
      const int32_t i = U(0, b.n[r] - 1);
      if (U(0, 1)) t.off[row + i] = b.n[r] + U(0, 3);
      else t.mask64[row + i] &= ~(1ull << i);
      if (pkv::validate_tree(&b.desc, p, &t.t, err) == PKV_OK) {
        std::printf("FAIL planted tree fault accepted (iteration %d)\n", it);
        return 1;
      }
    }
  }
  std::printf("fuzz %d accepted %d\n", fuzz, accepted);
  return 0;
}
