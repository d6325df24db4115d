// RoPE table and RoPE + KV-append kernels for gfx950.
//
// The append is the write half of the paged KV cache: "TensorRT-LLM 1.0 study notes",
// 二.2 (KVCacheManager): the attention op writes each request's new K/V into the blocks
// its block table names.  Pool layout [num_blocks, 2, T, Hkv, D], K at index 0 and V at
// index 1: "TensorRT-LLM source teardown part 1", KV cache manager interfaces
// (get_buffers).  RoPE is the GPT-NeoX variant named in "TensorRT-LLM source analysis
// report", 1.1; rotation of pairs (j, j + R/2) is the reading documented in pkv.h.
//
// Memory-bound: each workgroup owns kAppendTokens tokens of one request and spreads
// the (head, 8-element group) tasks of those tokens over its 256 threads, so every
// load and store is a 16-byte access and neighbouring lanes touch neighbouring bytes.
// Arithmetic is fp64 with contraction off and one rounding per stored element, so the
// stored bits depend only on the inputs and the table.
#include "device_common.h"
#include "kernels.h"

namespace pkv {
namespace {

constexpr int kAppendThreads = 256;
constexpr int kAppendTokens = 4;

template <int F>
__device__ __forceinline__ void load8(const void* base, int64_t off, double (&x)[8]) {
  if constexpr (F == F_BF16) {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = static_cast<double>(bf16_to_f32(w[i] & 0xFFFFu));
      x[2 * i + 1] = static_cast<double>(bf16_to_f32(w[i] >> 16));
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    const float4 a = p[0], b = p[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

// Round y (times `mul` for fp8) once to format F and store 8 elements at base+off.
template <int F>
__device__ __forceinline__ void store8(void* base, int64_t off, const double (&y)[8], double mul) {
  if constexpr (F == F_FP32) {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + off);
    p[0] = make_float4(static_cast<float>(y[0]), static_cast<float>(y[1]), static_cast<float>(y[2]),
                       static_cast<float>(y[3]));
    p[1] = make_float4(static_cast<float>(y[4]), static_cast<float>(y[5]), static_cast<float>(y[6]),
                       static_cast<float>(y[7]));
  } else if constexpr (F == F_BF16) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = f64_to_bf16(y[2 * i]) | (f64_to_bf16(y[2 * i + 1]) << 16);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + off) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i / 4] |= f64_to_e4m3(y[i] * mul) << (8 * (i % 4));
    *reinterpret_cast<uint2*>(static_cast<uint8_t*>(base) + off) = make_uint2(w[0], w[1]);
  }
}

// y1 = x1*c - x2*s, y2 = x2*c + x1*s: two fp64 products and one add/subtract each.
__device__ __forceinline__ void rotate8(const double (&x1)[8], const double (&x2)[8],
                                        const double2* __restrict__ cs, double (&y1)[8], double (&y2)[8]) {
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

__device__ __forceinline__ int64_t pool_off(const AppendArgs& a, int32_t blk, int which, int slot, int g) {
  return ((static_cast<int64_t>(blk) * 2 + which) * a.T + slot) * static_cast<int64_t>(a.Hkv) * a.D +
         static_cast<int64_t>(g) * a.D;
}

template <int IO, int KV, bool ROPE>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a) {
  const int r = blockIdx.y;
  const int n = a.ctx_len[r];
  const int tok0 = blockIdx.x * kAppendTokens;
  if (tok0 >= n) return;                                   // uniform over the block
  const int64_t row0 = block_prefix(a.ctx_len, r);
  const int past = a.seq_len[r] - n;
  const int Hq = a.q ? a.H : 0;
  const int R = ROPE ? a.R : 0;
  const int half = R / 2;
  const int rg = R / 16;                                   // rotation tasks per q/k head
  const int pg = (a.D - R) / 8;                            // pass-through tasks per q/k head
  const int vg = a.D / 8;                                  // tasks per v head
  const int qk = Hq + a.Hkv;
  const int per_tok = qk * (rg + pg) + a.Hkv * vg;
  const int ntok = min(kAppendTokens, n - tok0);
  for (int task = threadIdx.x; task < ntok * per_tok; task += kAppendThreads) {
    const int it = task / per_tok;
    int t = task - it * per_tok;
    const int i = tok0 + it;
    const int64_t row = row0 + i;
    const int m = past + i;
    if (row >= a.N || m < 0) continue;
    const int64_t lblk = m / a.T;
    const int slot = m % a.T;
    const int32_t blk = lblk < a.mbps ? a.table[static_cast<int64_t>(r) * a.mbps + lblk] : -1;
    const bool blk_ok = blk >= 0 && blk < a.num_blocks;
    double x1[8], x2[8], y1[8], y2[8];
    if (t < qk * rg) {                                      // rotated pair group
      const int head = t / rg, j0 = (t % rg) * 8;
      const bool isq = head < Hq;
      const void* src = isq ? a.q : a.k;
      const int64_t off = isq ? row * a.q_stride + static_cast<int64_t>(head) * a.D
                              : row * a.kv_stride + static_cast<int64_t>(head - Hq) * a.D;
      if (m >= a.max_pos) continue;
      load8<IO>(src, off + j0, x1);
      load8<IO>(src, off + j0 + half, x2);
      const double2* cs = reinterpret_cast<const double2*>(a.cos_sin) + static_cast<int64_t>(m) * half + j0;
      rotate8(x1, x2, cs, y1, y2);
      if (isq) {
        const int64_t o = row * a.H * a.D + static_cast<int64_t>(head) * a.D;
        store8<IO>(a.q_out, o + j0, y1, 1.0);
        store8<IO>(a.q_out, o + j0 + half, y2, 1.0);
      } else if (blk_ok) {
        const int64_t o = pool_off(a, blk, 0, slot, head - Hq);
        store8<KV>(a.pool, o + j0, y1, a.inv_k_scale);
        store8<KV>(a.pool, o + j0 + half, y2, a.inv_k_scale);
      }
    } else if (t < qk * (rg + pg)) {                        // dimensions past the rotary part
      t -= qk * rg;
      const int head = t / pg, j = R + (t % pg) * 8;
      const bool isq = head < Hq;
      const void* src = isq ? a.q : a.k;
      const int64_t off = isq ? row * a.q_stride + static_cast<int64_t>(head) * a.D
                              : row * a.kv_stride + static_cast<int64_t>(head - Hq) * a.D;
      load8<IO>(src, off + j, x1);
      if (isq) {
        store8<IO>(a.q_out, row * a.H * a.D + static_cast<int64_t>(head) * a.D + j, x1, 1.0);
      } else if (blk_ok) {
        store8<KV>(a.pool, pool_off(a, blk, 0, slot, head - Hq) + j, x1, a.inv_k_scale);
      }
    } else {                                                // values, not rotated
      t -= qk * (rg + pg);
      const int g = t / vg, j = (t % vg) * 8;
      load8<IO>(a.v, row * a.kv_stride + static_cast<int64_t>(g) * a.D + j, x1);
      if (blk_ok) store8<KV>(a.pool, pool_off(a, blk, 1, slot, g) + j, x1, a.inv_v_scale);
    }
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
  const dim3 grid((a.max_n + kAppendTokens - 1) / kAppendTokens, a.B);
  if (a.rope)
    hipLaunchKernelGGL((append_kernel<IO, KV, true>), grid, dim3(kAppendThreads), 0, s, a);
  else
    hipLaunchKernelGGL((append_kernel<IO, KV, false>), grid, dim3(kAppendThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  if (a.io_fmt == F_BF16) {
    if (a.kv_fmt == F_BF16) return launch_append_t<F_BF16, F_BF16>(a, s);
    if (a.kv_fmt == F_FP8) return launch_append_t<F_BF16, F_FP8>(a, s);
    return launch_append_t<F_BF16, F_FP32>(a, s);
  }
  if (a.kv_fmt == F_BF16) return launch_append_t<F_FP32, F_BF16>(a, s);
  if (a.kv_fmt == F_FP8) return launch_append_t<F_FP32, F_FP8>(a, s);
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
