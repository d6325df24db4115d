// Generic paged attention on the vector ALUs: any io/cache format, any head grouping.
//
// It serves the fp32 configurations and every shape the MFMA kernels do not take.
// One wave owns one query row and a chunk of query heads that share one KV head
// (GQA read as contiguous groups, "TensorRT-LLM source analysis report", 1.1).  The
// row walks its visible keys 64 at a time ("TensorRT-LLM 1.0 study notes", 6.3: loop
// over the KV blocks through the block table): lane t scores key c0+t against every
// head of the chunk, the wave keeps an online softmax (running max and sum, 6.2), and
// then every lane accumulates its share of head_dim over the chunk's value rows.
#include <math.h>

#include "device_common.h"
#include "kernels.h"

namespace pkv {
namespace {

constexpr int kMaxHeadsPerWave = 8;

template <int F>
__device__ __forceinline__ float load_elem(const void* base, int64_t off) {
  if constexpr (F == F_FP32) return static_cast<const float*>(base)[off];
  else if constexpr (F == F_BF16) return bf16_to_f32(static_cast<const uint16_t*>(base)[off]);
  else if constexpr (F == F_INT8) return static_cast<float>(static_cast<const int8_t*>(base)[off]);
  else return e4m3x2_to_f32(static_cast<const uint8_t*>(base)[off]).x;
}

template <int F>
__device__ __forceinline__ void store_elem(void* base, int64_t off, float v) {
  if constexpr (F == F_FP32) static_cast<float*>(base)[off] = v;
  else static_cast<uint16_t*>(base)[off] = static_cast<uint16_t>(f32_to_bf16(v));
}

__device__ __forceinline__ int64_t kv_off(const AttnArgs& a, int32_t blk, int which, int slot, int g) {
  return ((static_cast<int64_t>(blk) * 2 + which) * a.T + slot) * static_cast<int64_t>(a.Hkv) * a.D +
         static_cast<int64_t>(g) * a.D;
}

template <int IO, int KV>
__global__ __launch_bounds__(kWave) void attn_generic_kernel(AttnArgs a, int hc) {
  const int r = a.req_begin + blockIdx.z;
  const int n = a.ctx_len[r];
  const int i = blockIdx.x;
  if (i >= n) return;
  const int lane = threadIdx.x;
  const int64_t row = wave_prefix(a.ctx_len, r) + i;
  if (row >= a.N) return;
  // keys 0..m: m is this row's position (a chain), or the request's last key when its
  // draft tokens form a tree (the row's mask then selects among the new keys)
  const int base = a.seq_len[r] - n;
  const bool tree = a.spec_mask != nullptr;
  const int m = tree ? a.seq_len[r] - 1 : base + i;
  const int L = m + 1;
  uint32_t vm_lo = 0, vm_hi = 0;
  if (tree) {
    vm_lo = a.spec_mask[row * 2];
    vm_hi = a.spec_mask[row * 2 + 1];
  }
  const int G = a.H / a.Hkv;
  const int h0 = blockIdx.y * hc;
  const int g = h0 / G;

  __shared__ float qs[kMaxHeadsPerWave][128];
  __shared__ float ps[kMaxHeadsPerWave][kWave];
  __shared__ int32_t blks[kWave];
  for (int e = lane; e < hc * a.D; e += kWave) {
    const int hh = e / a.D, d = e % a.D;
    qs[hh][d] = load_elem<IO>(a.q, row * a.q_stride + static_cast<int64_t>(h0 + hh) * a.D + d);
  }
  __syncthreads();

  float mrun[kMaxHeadsPerWave], lrun[kMaxHeadsPerWave], acc[kMaxHeadsPerWave][2];
#pragma unroll
  for (int hh = 0; hh < kMaxHeadsPerWave; ++hh) {
    mrun[hh] = -INFINITY;
    lrun[hh] = 0.f;
    acc[hh][0] = acc[hh][1] = 0.f;
  }
  const float kscale = a.scale_log2 * a.k_scale;
  for (int c0 = 0; c0 < L; c0 += kWave) {
    const int t = c0 + lane;
    int32_t blk = -1;
    const int j = t - base;                              // new key j (tree masks)
    const bool vis = !tree || j < 0 || (((j < 32 ? vm_lo : vm_hi) >> (j & 31)) & 1u);
    if (t < L && vis) {
      const int64_t lb = t / a.T;
      blk = lb < a.mbps ? a.table[static_cast<int64_t>(r) * a.mbps + lb] : -1;
      if (blk >= a.num_blocks) blk = -1;
    }
    float s[kMaxHeadsPerWave];
#pragma unroll
    for (int hh = 0; hh < kMaxHeadsPerWave; ++hh) s[hh] = 0.f;
    if (blk >= 0) {
      const int64_t ko = kv_off(a, blk, 0, t % a.T, g);
      for (int d = 0; d < a.D; ++d) {
        const float kd = load_elem<KV>(a.pool, ko + d);
#pragma unroll
        for (int hh = 0; hh < kMaxHeadsPerWave; ++hh)
          if (hh < hc) s[hh] += qs[hh][d] * kd;
      }
    }
    blks[lane] = blk;
#pragma unroll
    for (int hh = 0; hh < kMaxHeadsPerWave; ++hh) {
      if (hh >= hc) break;
      const float x = blk >= 0 ? s[hh] * kscale : -INFINITY;
      const float mnew = fmaxf(mrun[hh], wave_max(x));
      const float alpha = mrun[hh] == -INFINITY ? 0.f : exp2f(mrun[hh] - mnew);
      const float p = x == -INFINITY ? 0.f : exp2f(x - mnew);
      lrun[hh] = lrun[hh] * alpha + wave_sum(p);
      mrun[hh] = mnew;
      ps[hh][lane] = p;
      acc[hh][0] *= alpha;
      acc[hh][1] *= alpha;
    }
    __syncthreads();
    const int cnt = min(kWave, L - c0);
    for (int tt = 0; tt < cnt; ++tt) {
      const int32_t b = blks[tt];
      if (b < 0) continue;
      const int64_t vo = kv_off(a, b, 1, (c0 + tt) % a.T, g);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int d = lane + kWave * j;
        if (d >= a.D) break;
        const float v = load_elem<KV>(a.pool, vo + d) * a.v_scale;
#pragma unroll
        for (int hh = 0; hh < kMaxHeadsPerWave; ++hh)
          if (hh < hc) acc[hh][j] += ps[hh][tt] * v;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int hh = 0; hh < kMaxHeadsPerWave; ++hh) {
    if (hh >= hc) break;
    const float inv = 1.f / lrun[hh];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int d = lane + kWave * j;
      if (d >= a.D) break;
      const int64_t o = row * a.H * a.D + static_cast<int64_t>(h0 + hh) * a.D + d;
      if (a.out_fmt == F_FP8)
        static_cast<uint8_t*>(a.out)[o] = static_cast<uint8_t>(f32_to_e4m3((acc[hh][j] * inv) * a.out_mul));
      else
        store_elem<IO>(a.out, o, acc[hh][j] * inv);
    }
  }
}

int gcd_int(int x, int y) {
  while (y) {
    const int t = x % y;
    x = y;
    y = t;
  }
  return x;
}

template <int IO, int KV>
hipError_t launch_t(const AttnArgs& a, hipStream_t s) {
  const int G = a.H / a.Hkv;
  const int hc = gcd_int(G, kMaxHeadsPerWave);
  const dim3 grid(a.max_n, a.H / hc, a.req_end - a.req_begin);
  hipLaunchKernelGGL((attn_generic_kernel<IO, KV>), grid, dim3(kWave), 0, s, a, hc);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_generic(const AttnArgs& a, hipStream_t s) {
  if (a.io_fmt == F_BF16) {
    if (a.kv_fmt == F_BF16) return launch_t<F_BF16, F_BF16>(a, s);
    if (a.kv_fmt == F_FP8) return launch_t<F_BF16, F_FP8>(a, s);
    if (a.kv_fmt == F_INT8) return launch_t<F_BF16, F_INT8>(a, s);
    return launch_t<F_BF16, F_FP32>(a, s);
  }
  if (a.kv_fmt == F_BF16) return launch_t<F_FP32, F_BF16>(a, s);
  if (a.kv_fmt == F_FP8) return launch_t<F_FP32, F_FP8>(a, s);
  if (a.kv_fmt == F_INT8) return launch_t<F_FP32, F_INT8>(a, s);
  return launch_t<F_FP32, F_FP32>(a, s);
}

}  // namespace pkv
