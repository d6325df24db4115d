// RoPE table and RoPE + KV-append kernels for gfx950.
//
// The append is the write half of the paged KV cache: "TensorRT-LLM 1.0 study notes",
// 二.2 (KVCacheManager): the attention op writes each request's new K/V into the blocks
// its block table names.  Pool layout [num_blocks, 2, T, Hkv, D], K at index 0 and V at
// index 1: "TensorRT-LLM source teardown part 1", KV cache manager interfaces
// (get_buffers).  RoPE is the GPT-NeoX variant named in "TensorRT-LLM source analysis
// report", 1.1; rotation of pairs (j, j + R/2) is the reading documented in pkv.h.
//
// Memory-bound: each workgroup owns a few consecutive packed rows (tokens) and spreads
// the (head, 8-element group) tasks of those tokens over its 256 threads, so every
// load and store is a 16-byte access and neighbouring lanes touch neighbouring bytes.
// Arithmetic is fp64 with contraction off and one rounding per stored element, so the
// stored bits depend only on the inputs and the table.  With a per-head q/k norm
// ("TensorRT-LLM source analysis report", 1.1, QK LayerNorm; the teardown's kernel
// directory lists a fused QK-norm + RoPE kernel), a pre-pass computes each head's mean
// and inverse deviation into LDS and the tasks normalise their elements before rotating.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace pkv {
namespace {

constexpr int kAppendThreads = 256;
constexpr int kMaxTokensPerWg = 8;
constexpr int kFlatMaxRequests = 4096;

// Streaming accesses: every input element is read once and every output element written
// once per step, so stores, and loads of inputs nothing reads again, carry the
// nontemporal hint.  (With a q/k norm the statistics pass reads q and k first; their
// second read then comes from the caches, so those loads stay ordinary.)
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
template <bool NT>
__device__ __forceinline__ uint4 ld16(const void* p) {
  if constexpr (NT) {
    const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  } else {
    return *static_cast<const uint4*>(p);
  }
}
__device__ __forceinline__ void st16(void* p, uint4 u) {
  __builtin_nontemporal_store(u32x4_t{u.x, u.y, u.z, u.w}, static_cast<u32x4_t*>(p));
}
__device__ __forceinline__ void st8(void* p, uint2 u) {
  __builtin_nontemporal_store(u32x2_t{u.x, u.y}, static_cast<u32x2_t*>(p));
}

// 8 raw io elements as loaded (bf16: one 16-byte vector; fp32: two)
struct Raw8 {
  uint4 a, b;
};

template <int F, bool NT = false>
__device__ __forceinline__ Raw8 load_raw8(const void* base, int64_t off) {
  Raw8 r;
  if constexpr (F == F_BF16) {
    r.a = ld16<NT>(static_cast<const uint16_t*>(base) + off);
    r.b = make_uint4(0, 0, 0, 0);
  } else {
    const float* p = static_cast<const float*>(base) + off;
    r.a = ld16<NT>(p);
    r.b = ld16<NT>(p + 4);
  }
  return r;
}

template <int F>
__device__ __forceinline__ void widen8(const Raw8& r, double (&x)[8]) {
  if constexpr (F == F_BF16) {
    const uint32_t w[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = static_cast<double>(bf16_to_f32(w[i] & 0xFFFFu));
      x[2 * i + 1] = static_cast<double>(bf16_to_f32(w[i] >> 16));
    }
  } else {
    const uint32_t w[8] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = static_cast<double>(__uint_as_float(w[i]));
  }
}

template <int F, bool NT = false>
__device__ __forceinline__ void load8(const void* base, int64_t off, double (&x)[8]) {
  widen8<F>(load_raw8<F, NT>(base, off), x);
}

// Round y (times `mul` for fp8 and int8) once to format F and store 8 elements at base+off.
template <int F>
__device__ __forceinline__ void store8(void* base, int64_t off, const double (&y)[8], double mul) {
  if constexpr (F == F_FP32) {
    float* p = static_cast<float*>(base) + off;
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = __float_as_uint(static_cast<float>(y[i]));
    st16(p, make_uint4(w[0], w[1], w[2], w[3]));
    st16(p + 4, make_uint4(w[4], w[5], w[6], w[7]));
  } else if constexpr (F == F_BF16) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = f64x2_to_bf16x2(y[2 * i], y[2 * i + 1]);
    st16(static_cast<uint16_t*>(base) + off, make_uint4(w[0], w[1], w[2], w[3]));
  } else {
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i)
      w[i / 4] |= (F == F_INT8 ? f64_to_int8(y[i] * mul) : f64_to_e4m3(y[i] * mul)) << (8 * (i % 4));
    st8(static_cast<uint8_t*>(base) + off, make_uint2(w[0], w[1]));
  }
}

// y1 = x1*c - x2*s, y2 = x2*c + x1*s: two fp64 products and one add/subtract each.
__device__ __forceinline__ void rotate8(const double (&x1)[8], const double (&x2)[8], const double2 (&cs)[8],
                                        double (&y1)[8], double (&y2)[8]) {
#pragma clang fp contract(off)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const double2 t = cs[i];
    const double a = x1[i] * t.x;
    const double b = x2[i] * t.y;
    const double e = x2[i] * t.x;
    const double f = x1[i] * t.y;
    y1[i] = a - b;
    y2[i] = e + f;
  }
}

// Per-head normalisation of 8 elements at dims dim0 .. dim0+7 of one q or k head:
// y = ((x - mean) * inv) * w (+ b), fp64, with (mean, inv) of the head from the pre-pass.
__device__ __forceinline__ void norm8(double (&x)[8], int dim0, double2 st, const float* __restrict__ w,
                                      const float* __restrict__ b) {
#pragma clang fp contract(off)
  const float4 w0 = *reinterpret_cast<const float4*>(w + dim0), w1 = *reinterpret_cast<const float4*>(w + dim0 + 4);
  const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  float bv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (b) {
    const float4 b0 = *reinterpret_cast<const float4*>(b + dim0), b1 = *reinterpret_cast<const float4*>(b + dim0 + 4);
    bv[0] = b0.x; bv[1] = b0.y; bv[2] = b0.z; bv[3] = b0.w;
    bv[4] = b1.x; bv[5] = b1.y; bv[6] = b1.z; bv[7] = b1.w;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const double d = x[i] - st.x;
    const double y = (d * st.y) * static_cast<double>(wv[i]);
    x[i] = b ? y + static_cast<double>(bv[i]) : y;
  }
}

// Where one token goes: its packed row, request, absolute position and pool slot.
struct TokenSlot {
  int64_t row;
  int32_t r, m, blk, slot;      // blk < 0: table entry out of range (skip the K/V store)
};

// One (token, task) unit of work.  Tasks of a token: rotation groups of 8 pairs for
// every q and k head, pass-through groups of 8 dims past the rotary part, and groups of
// 8 v dims.  Loads of a task are issued before any of its arithmetic.
constexpr int kHeadsPerRotTask = 4;

// One (token, task) unit of work.  Tasks of a token, in order: rotation tasks (one
// group of 8 pairs for up to kHeadsPerRotTask q/k heads, so the table slice is read
// once for all of them), pass-through groups of 8 dims past the rotary part, and
// groups of 8 v dims.  A task's loads are all issued before its arithmetic.
template <int IO, int KV, int RS, bool NORM>
__device__ __forceinline__ void append_task(const AppendArgs& a, const TokenSlot& tk, int t, int Hq,
                                            const void* __restrict__ q, const void* __restrict__ k,
                                            const void* __restrict__ v, const double* __restrict__ cs_base,
                                            void* __restrict__ q_out, void* __restrict__ pool,
                                            const double2* __restrict__ stat) {
  constexpr bool NTQK = !NORM;               // q/k read only here (no norm statistics pass)
  const int R = RS != kRopeNone ? a.R : 0;
  const int half = R / 2;
  const int rg = R / 16, pg = (a.D - R) / 8, vg = a.D / 8;
  // element offsets of a task's 8 pairs: rotate-half -> first elements at j0, partners
  // at j0 + R/2; interleaved -> 16 consecutive elements from 2*j0 (pairs (2j, 2j+1))
  auto off_a = [&](int j0) { return RS == kRopeGptj ? 2 * j0 : j0; };
  auto off_b = [&](int j0) { return RS == kRopeGptj ? 2 * j0 + 8 : j0 + half; };
  const int qk = Hq + a.Hkv;
  const int nhc = (qk + kHeadsPerRotTask - 1) / kHeadsPerRotTask;
  auto pool_off = [&](int which, int g) {
    return ((static_cast<int64_t>(tk.blk) * 2 + which) * a.T + tk.slot) * static_cast<int64_t>(a.Hkv) * a.D +
           static_cast<int64_t>(g) * a.D;
  };
  // normalise a widened group of head `head` (NORM only); (mean, inv) come from stat[head]
  auto normalise = [&](double (&x)[8], int head, int dim0) {
    if constexpr (NORM) {
      const bool isq = head < Hq;
      norm8(x, dim0, stat[head], isq ? a.qn_w : a.kn_w, isq ? a.qn_b : a.kn_b);
    }
  };
  auto head_src = [&](int head, const void*& src, int64_t& off) {
    const bool isq = head < Hq;
    src = isq ? q : k;
    off = isq ? tk.row * a.q_stride + static_cast<int64_t>(head) * a.D
              : tk.row * a.kv_stride + static_cast<int64_t>(head - Hq) * a.D;
  };
  if (t < nhc * rg) {                                       // rotated pair groups
    if (tk.m >= a.max_pos) return;
    const int hc = t / max(rg, 1), j0 = (t % max(rg, 1)) * 8;
    const int h0 = hc * kHeadsPerRotTask;
    const int nh = min(kHeadsPerRotTask, qk - h0);
    Raw8 r1[kHeadsPerRotTask], r2[kHeadsPerRotTask];
#pragma unroll
    for (int u = 0; u < kHeadsPerRotTask; ++u) {
      if (u < nh) {
        const void* src;
        int64_t off;
        head_src(h0 + u, src, off);
        r1[u] = load_raw8<IO, NTQK>(src, off + off_a(j0));
        r2[u] = load_raw8<IO, NTQK>(src, off + off_b(j0));
      }
    }
    const double2* cs = reinterpret_cast<const double2*>(cs_base) + static_cast<int64_t>(tk.m) * half + j0;
    double2 c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = cs[i];
#pragma unroll
    for (int u = 0; u < kHeadsPerRotTask; ++u) {
      if (u >= nh) break;
      const int head = h0 + u;
      double x1[8], x2[8], y1[8], y2[8];
      if constexpr (RS == kRopeGptj) {                    // de-interleave the 16 elements
        double e0[8], e1[8];
        widen8<IO>(r1[u], e0);
        widen8<IO>(r2[u], e1);
        normalise(e0, head, off_a(j0));
        normalise(e1, head, off_b(j0));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x1[i] = e0[2 * i];
          x2[i] = e0[2 * i + 1];
          x1[i + 4] = e1[2 * i];
          x2[i + 4] = e1[2 * i + 1];
        }
      } else {
        widen8<IO>(r1[u], x1);
        widen8<IO>(r2[u], x2);
        normalise(x1, head, off_a(j0));
        normalise(x2, head, off_b(j0));
      }
      rotate8(x1, x2, c, y1, y2);
      double s1[8], s2[8];                                // the two stored groups of 8
      if constexpr (RS == kRopeGptj) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s1[2 * i] = y1[i];
          s1[2 * i + 1] = y2[i];
          s2[2 * i] = y1[i + 4];
          s2[2 * i + 1] = y2[i + 4];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          s1[i] = y1[i];
          s2[i] = y2[i];
        }
      }
      if (head < Hq) {
        const int64_t o = tk.row * a.H * a.D + static_cast<int64_t>(head) * a.D;
        store8<IO>(q_out, o + off_a(j0), s1, 1.0);
        store8<IO>(q_out, o + off_b(j0), s2, 1.0);
      } else if (tk.blk >= 0) {
        const int64_t o = pool_off(0, head - Hq);
        store8<KV>(pool, o + off_a(j0), s1, a.inv_k_scale);
        store8<KV>(pool, o + off_b(j0), s2, a.inv_k_scale);
      }
    }
  } else if (t < nhc * rg + qk * pg) {                      // dimensions past the rotary part
    t -= nhc * rg;
    const int head = t / pg, j = R + (t % pg) * 8;
    const void* src;
    int64_t off;
    head_src(head, src, off);
    double x[8];
    load8<IO, NTQK>(src, off + j, x);
    normalise(x, head, j);
    if (head < Hq)
      store8<IO>(q_out, tk.row * a.H * a.D + static_cast<int64_t>(head) * a.D + j, x, 1.0);
    else if (tk.blk >= 0)
      store8<KV>(pool, pool_off(0, head - Hq) + j, x, a.inv_k_scale);
  } else {                                                  // values, not rotated
    t -= nhc * rg + qk * pg;
    const int g = t / vg, j = (t % vg) * 8;
    double x[8];
    load8<IO, true>(v, tk.row * a.kv_stride + static_cast<int64_t>(g) * a.D + j, x);
    if (tk.blk >= 0) store8<KV>(pool, pool_off(1, g) + j, x, a.inv_v_scale);
  }
}

// (mean, 1/sqrt(var + eps)) of one head's D elements: fp64 sums in index order.  The
// row's loads are issued together (all of a bf16 row, half of an fp32 row of 128 at a
// time) so that one memory latency covers them, and a bf16 row loaded for the mean is
// reused for the variance.
template <int IO, int D>
__device__ __forceinline__ void row_stats(const void* src, int64_t off, bool layer, double eps, double& mean,
                                          double& inv) {
  constexpr int NG = D / 8;                       // groups of 8 elements
  constexpr int BATCH = IO == F_BF16 ? NG : 8;    // groups held in registers at once
  Raw8 r[BATCH];
  auto fetch = [&](int g0) __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < BATCH; ++b) r[b] = load_raw8<IO>(src, off + static_cast<int64_t>(g0 + b) * 8);
  };
  mean = 0.0;
  if (layer) {
    double s = 0.0;
#pragma unroll
    for (int g0 = 0; g0 < NG; g0 += BATCH) {
      fetch(g0);
#pragma unroll
      for (int b = 0; b < BATCH; ++b) {
        double x[8];
        widen8<IO>(r[b], x);
#pragma unroll
        for (int i = 0; i < 8; ++i) s += x[i];
      }
    }
    mean = s / static_cast<double>(D);
  }
  double ss = 0.0;
#pragma unroll
  for (int g0 = 0; g0 < NG; g0 += BATCH) {
    if (!(layer && BATCH == NG)) fetch(g0);      // a whole bf16 row is still in r
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      double x[8];
      widen8<IO>(r[b], x);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const double d = x[i] - mean;
        ss += d * d;
      }
    }
  }
  inv = 1.0 / __builtin_sqrt(ss / static_cast<double>(D) + eps);
}

__device__ __forceinline__ TokenSlot make_slot(const AppendArgs& a, int64_t row, int r, int i) {
  TokenSlot tk;
  tk.row = row;
  tk.r = r;
  tk.m = a.seq_len[r] - a.ctx_len[r] + i;
  const int64_t lblk = tk.m / a.T;
  int32_t blk = (tk.m >= 0 && lblk < a.mbps) ? a.table[static_cast<int64_t>(r) * a.mbps + lblk] : -1;
  tk.blk = (blk >= 0 && blk < a.num_blocks) ? blk : -1;
  tk.slot = tk.m % a.T;
  return tk;
}

// FLAT: the grid walks the packed rows, tokens_per_wg consecutive rows per workgroup,
// and each workgroup finds the rows' requests through an LDS prefix scan of the
// context lengths (batches of at most kFlatMaxRequests requests).  Otherwise the grid
// is (row tile, request), for any batch size.
template <int IO, int KV, int RS, bool FLAT, bool NORM>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a, int tokens_per_wg) {
  __shared__ int32_t s_cu[kFlatMaxRequests + 1];
  __shared__ TokenSlot s_tok[kMaxTokensPerWg];
  const int Hq = a.q ? a.H : 0;
  int ntok;
  if constexpr (FLAT) {
    const int64_t row0 = static_cast<int64_t>(blockIdx.x) * tokens_per_wg;
    if (row0 >= a.N) return;                               // uniform
    ntok = static_cast<int>(min<int64_t>(tokens_per_wg, a.N - row0));
    // inclusive scan of ctx_len into s_cu[1..B] (s_cu[0] = 0), chunked per thread
    const int B = a.B;
    const int per = (B + kAppendThreads - 1) / kAppendThreads;
    const int b0 = threadIdx.x * per, b1 = min(b0 + per, B);
    int32_t local = 0;
    for (int b = b0; b < b1; ++b) local += a.ctx_len[b];
    // exclusive prefix of `local` over the threads: a shuffle scan inside each wave, then
    // the totals of the waves before
    const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
    int32_t incl = local;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int32_t y = __shfl_up(incl, d, kWave);
      if (lane >= d) incl += y;
    }
    __shared__ int32_t s_wave[kAppendThreads / kWave];
    if (lane == kWave - 1) s_wave[wv] = incl;
    if (threadIdx.x == 0) s_cu[0] = 0;
    __syncthreads();
    int32_t run = incl - local;
    for (int w = 0; w < wv; ++w) run += s_wave[w];
    for (int b = b0; b < b1; ++b) {
      run += a.ctx_len[b];
      s_cu[b + 1] = run;
    }
    __syncthreads();
    if (threadIdx.x < ntok) {
      const int64_t row = row0 + threadIdx.x;
      int lo = 0, hi = B - 1;                              // request r: s_cu[r] <= row < s_cu[r+1]
      while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (s_cu[mid] <= row) lo = mid; else hi = mid - 1;
      }
      s_tok[threadIdx.x] = make_slot(a, row, lo, static_cast<int>(row - s_cu[lo]));
    }
  } else {
    const int r = blockIdx.y;
    const int n = a.ctx_len[r];
    const int tok0 = blockIdx.x * tokens_per_wg;
    if (tok0 >= n) return;                                 // uniform
    const int64_t rowr = block_prefix(a.ctx_len, r);
    ntok = min(tokens_per_wg, n - tok0);
    if (threadIdx.x < ntok)
      s_tok[threadIdx.x] = make_slot(a, rowr + tok0 + threadIdx.x, r, tok0 + threadIdx.x);
  }
  __syncthreads();
  // NORM: (mean, 1/sqrt(var + eps)) of every q and k head of the workgroup's tokens, one
  // thread per (token, head), fp64 sums in index order (as the oracle and pkv.h state)
  const double2* stat = nullptr;
  if constexpr (NORM) {
    __shared__ double2 s_stat[kMaxTokensPerWg * kMaxNormHeads];
    const int nh = Hq + a.Hkv;
    const bool layer = a.norm == kNormLayer;
    for (int u = threadIdx.x; u < ntok * nh; u += kAppendThreads) {
      const int it = u / nh, head = u - it * nh;
      const TokenSlot tk = s_tok[it];
      double mean = 0.0, inv = 0.0;
      if (tk.row < a.N && tk.m >= 0) {
        const bool isq = head < Hq;
        const void* src = isq ? a.q : a.k;
        const int64_t off = isq ? tk.row * a.q_stride + static_cast<int64_t>(head) * a.D
                                : tk.row * a.kv_stride + static_cast<int64_t>(head - Hq) * a.D;
        if (a.D == 128) row_stats<IO, 128>(src, off, layer, a.norm_eps, mean, inv);
        else row_stats<IO, 64>(src, off, layer, a.norm_eps, mean, inv);
      }
      s_stat[u] = make_double2(mean, inv);
    }
    __syncthreads();
    stat = s_stat;
  }
  const int R = RS != kRopeNone ? a.R : 0;
  const int per_tok = ((Hq + a.Hkv + kHeadsPerRotTask - 1) / kHeadsPerRotTask) * (R / 16) +
                      (Hq + a.Hkv) * ((a.D - R) / 8) + a.Hkv * (a.D / 8);
  const int total = ntok * per_tok;
  const void* __restrict__ q = a.q;
  const void* __restrict__ k = a.k;
  const void* __restrict__ v = a.v;
  const double* __restrict__ cs = a.cos_sin;
  void* __restrict__ q_out = a.q_out;
  void* __restrict__ pool = a.pool;
  for (int task = threadIdx.x; task < total; task += kAppendThreads) {
    const int it = task / per_tok;
    const TokenSlot tk = s_tok[it];
    if (tk.row >= a.N || tk.m < 0) continue;
    append_task<IO, KV, RS, NORM>(a, tk, task - it * per_tok, Hq, q, k, v, cs, q_out, pool,
                                  NORM ? stat + it * (Hq + a.Hkv) : nullptr);
  }
}

// cos_sin[m][j] = (cos(m*theta_j), sin(m*theta_j)), theta_j = base^(-2j/R), fp64.
__global__ void rope_table_kernel(double base, int R, int max_pos, double* __restrict__ cs) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int half = R / 2;
  if (idx >= static_cast<int64_t>(max_pos) * half) return;
  const int j = static_cast<int>(idx % half);
  const int64_t m = idx / half;
  const double inv_freq = pow(base, -(2.0 * j) / static_cast<double>(R));
  const double ang = static_cast<double>(m) * inv_freq;
  double s, c;
  sincos(ang, &s, &c);
  cs[2 * idx] = c;
  cs[2 * idx + 1] = s;
}

template <int IO, int KV>
hipError_t launch_append_t(const AppendArgs& a, hipStream_t s) {
  // enough workgroups to fill the chip: about N / 512 tokens each, at most 8
  int64_t want = a.N / 512;
  const int tpw = static_cast<int>(want < 1 ? 1 : want > kMaxTokensPerWg ? kMaxTokensPerWg : want);
  auto go2 = [&](auto rs, auto nrm) {
    constexpr int RS = decltype(rs)::value;
    constexpr bool NORM = decltype(nrm)::value;
    if (a.B <= kFlatMaxRequests) {
      const dim3 grid(static_cast<unsigned>((a.N + tpw - 1) / tpw));
      hipLaunchKernelGGL((append_kernel<IO, KV, RS, true, NORM>), grid, dim3(kAppendThreads), 0, s, a, tpw);
    } else {
      const dim3 grid((a.max_n + tpw - 1) / tpw, a.B);
      hipLaunchKernelGGL((append_kernel<IO, KV, RS, false, NORM>), grid, dim3(kAppendThreads), 0, s, a, tpw);
    }
  };
  auto go = [&](auto rs) {
    if (a.norm != kNormNone) go2(rs, std::true_type());
    else go2(rs, std::false_type());
  };
  if (a.rope == kRopeNeox) go(std::integral_constant<int, kRopeNeox>());
  else if (a.rope == kRopeGptj) go(std::integral_constant<int, kRopeGptj>());
  else go(std::integral_constant<int, kRopeNone>());
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  if (a.io_fmt == F_BF16) {
    if (a.kv_fmt == F_BF16) return launch_append_t<F_BF16, F_BF16>(a, s);
    if (a.kv_fmt == F_FP8) return launch_append_t<F_BF16, F_FP8>(a, s);
    if (a.kv_fmt == F_INT8) return launch_append_t<F_BF16, F_INT8>(a, s);
    return launch_append_t<F_BF16, F_FP32>(a, s);
  }
  if (a.kv_fmt == F_BF16) return launch_append_t<F_FP32, F_BF16>(a, s);
  if (a.kv_fmt == F_FP8) return launch_append_t<F_FP32, F_FP8>(a, s);
  if (a.kv_fmt == F_INT8) return launch_append_t<F_FP32, F_INT8>(a, s);
  return launch_append_t<F_FP32, F_FP32>(a, s);
}

hipError_t launch_rope_table(double base, int32_t rot, int32_t max_pos, double* cos_sin, hipStream_t s) {
  const int64_t total = static_cast<int64_t>(max_pos) * (rot / 2);
  const int threads = 256;
  const dim3 grid(static_cast<unsigned>((total + threads - 1) / threads));
  hipLaunchKernelGGL(rope_table_kernel, grid, dim3(threads), 0, s, base, rot, max_pos, cos_sin);
  return hipGetLastError();
}

}  // namespace pkv
