// Device helpers shared by the gfx950 kernels: element formats, reductions, index math.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace pkv {

constexpr int kWave = 64;

// ---------------------------------------------------------------- element formats
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// fp32 -> bf16, nearest-even; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// fp64 -> bf16 in one rounding (nearest-even), over the whole range: subnormal results,
// overflow to infinity, NaN.  Works on the binary64 bit pattern: the kept part is the
// sign, 11-bit exponent and top 7 fraction bits; the dropped 45 bits decide the rounding.
__device__ __forceinline__ uint32_t f64_to_bf16(double x) {
  const uint64_t b = static_cast<uint64_t>(__double_as_longlong(x));
  const uint32_t sign = static_cast<uint32_t>(b >> 48) & 0x8000u;
  const uint64_t a = b & 0x7FFFFFFFFFFFFFFFull;
  if (a > 0x7FF0000000000000ull) return sign | 0x7FC0u;               // NaN
  const uint32_t E = static_cast<uint32_t>(a >> 52);                   // biased binary64 exponent
  if (E >= 897u) {                                                     // result is normal (or overflows)
    const uint64_t r = (a + 0xFFFFFFFFFFFull + ((a >> 45) & 1ull)) >> 45;   // exponent:fraction7, rounded
    if (r >= (static_cast<uint64_t>(896 + 255) << 7)) return sign | 0x7F80u;
    return sign | static_cast<uint32_t>(r - (896ull << 7));
  }
  // subnormal (or zero) bf16: value / 2^-133 rounded to an integer q <= 128
  const uint64_t m = E ? ((a & 0xFFFFFFFFFFFFFull) | (1ull << 52)) : (a & 0xFFFFFFFFFFFFFull);
  const uint32_t s = 942u - (E ? E : 1u);                              // >= 46
  if (s >= 54u) return sign;                                           // below half the smallest subnormal
  const uint64_t q = (m + ((1ull << (s - 1)) - 1ull) + ((m >> s) & 1ull)) >> s;
  return sign | static_cast<uint32_t>(q);
}

// fp64 -> bf16, the same rounding as f64_to_bf16 by another route: round to fp32 with
// round-to-odd (truncate, then set the lowest bit if anything was dropped) and round
// that to bf16 to nearest-even in hardware.  fp32 keeps 16 more bits than bf16 (>= 2
// are needed), so the two roundings compose to a single nearest-even rounding
// (Boldo and Melquiond, "Emulation of FMA and correctly rounded sums: proved
// algorithms using rounding to odd").  Returns a pair packed as lo | hi << 16.
__device__ __forceinline__ float f64_to_f32_odd(double x) {
  const float f = static_cast<float>(x);                    // nearest-even
  const double back = static_cast<double>(f);
  uint32_t b = __float_as_uint(f);
  if (back != x) {                                          // inexact (or NaN)
    if (fabs(back) > fabs(x)) b -= 1;                       // step back toward zero: truncation
    b |= 1u;                                                // sticky bit
  }
  return __uint_as_float(b);
}

typedef float pkv_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 pkv_bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f64x2_to_bf16x2(double lo, double hi) {
  const pkv_f32x2 v = {f64_to_f32_odd(lo), f64_to_f32_odd(hi)};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, pkv_bf16x2));
}

// fp64 -> OCP E4M3 in one rounding (nearest-even), saturating finite overflow and
// infinities to +-448.  Kept part: exponent and top 3 fraction bits; 49 bits dropped.
__device__ __forceinline__ uint32_t f64_to_e4m3(double x) {
  const uint64_t b = static_cast<uint64_t>(__double_as_longlong(x));
  const uint32_t sign = static_cast<uint32_t>(b >> 56) & 0x80u;
  const uint64_t a = b & 0x7FFFFFFFFFFFFFFFull;
  if (a > 0x7FF0000000000000ull) return sign | 0x7Fu;                  // NaN
  const uint32_t E = static_cast<uint32_t>(a >> 52);
  if (E >= 1017u) {                                                    // normal e4m3 range or above
    const uint64_t r = (a + 0xFFFFFFFFFFFFull + ((a >> 49) & 1ull)) >> 49;
    const uint64_t code = r - (1016ull << 3);
    return sign | static_cast<uint32_t>(code > 0x7Eull ? 0x7Eull : code);
  }
  const uint64_t m = E ? ((a & 0xFFFFFFFFFFFFFull) | (1ull << 52)) : (a & 0xFFFFFFFFFFFFFull);
  const uint32_t s = 1066u - (E ? E : 1u);                             // >= 50
  if (s >= 54u) return sign;
  const uint64_t q = (m + ((1ull << (s - 1)) - 1ull) + ((m >> s) & 1ull)) >> s;
  return sign | static_cast<uint32_t>(q);
}

// fp32 -> OCP E4M3 code in one rounding (nearest-even), saturating finite overflow and
// infinities to +-448; NaN -> 0x7F with the sign.  Normal results keep the exponent and the
// top 3 fraction bits (20 bits dropped); results below 2^-6 are multiples of 2^-9, so they
// are |f| * 2^9 (exact) rounded to an integer with ties to even.
__device__ __forceinline__ uint32_t f32_to_e4m3(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  // all three candidates, then a select (no divergent branches)
  const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;          // exponent:fraction3, rounded
  const uint32_t nrm = min(r - (120u << 3), 0x7Eu);                     // rebias 127 -> 7, saturate
  const uint32_t sub = static_cast<uint32_t>(__builtin_rintf(__uint_as_float(min(a, 121u << 23)) * 512.0f));
  const uint32_t code = a > 0x7F800000u ? 0x7Fu : a >= (121u << 23) ? nrm : sub;   // NaN / |f| >= 2^-6 / below
  return sign | code;
}

// fp64 -> int8 code: round to the nearest integer (ties to even, v_rndne_f64), saturate
// to -128 .. 127 (infinities included); NaN stores 0.  Returns the code's low byte.
__device__ __forceinline__ uint32_t f64_to_int8(double x) {
  if (x != x) return 0u;
  const double r = fmin(fmax(__builtin_rint(x), -128.0), 127.0);
  return static_cast<uint32_t>(static_cast<int32_t>(r)) & 0xFFu;
}

// OCP E4M3 -> fp32 for two codes (bytes 0 and 1 of `packed`), hardware conversion.
__device__ __forceinline__ float2 e4m3x2_to_f32(uint32_t packed) {
  auto v = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(packed), false);
  return make_float2(v[0], v[1]);
}
// bytes 2 and 3
__device__ __forceinline__ float2 e4m3x2_hi_to_f32(uint32_t packed) {
  auto v = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(packed), true);
  return make_float2(v[0], v[1]);
}

// ---------------------------------------------------------------- wave reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ int64_t wave_sum_i64(int64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Combine each lane with lane l ^ 16 (ROWS = 16) or l ^ 32 (ROWS = 32) through the VALU
// lane swaps of gfx950 (no LDS round trip); both lanes of a pair get op(x_l, x_partner).
template <int ROWS>
__device__ __forceinline__ void lane_swap(float v, float& a, float& b) {
  const uint32_t u = __float_as_uint(v);
  if constexpr (ROWS == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  } else {
    static_assert(ROWS == 32, "row pairs of 16 or 32 lanes");
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  }
}
template <int ROWS>
__device__ __forceinline__ float xor_max(float v) {
  float a, b;
  lane_swap<ROWS>(v, a, b);
  return fmaxf(a, b);
}
template <int ROWS>
__device__ __forceinline__ float xor_sum(float v) {
  float a, b;
  lane_swap<ROWS>(v, a, b);
  return a + b;
}

// Sum of len[0 .. r-1] over one wave (every lane gets the result).
__device__ __forceinline__ int64_t wave_prefix(const int32_t* __restrict__ len, int r) {
  int64_t s = 0;
  for (int j = threadIdx.x % kWave; j < r; j += kWave) s += len[j];
  return wave_sum_i64(s);
}

// Same over a whole block (blockDim.x a multiple of 64, <= 1024); every thread gets it.
__device__ __forceinline__ int64_t block_prefix(const int32_t* __restrict__ len, int r) {
  __shared__ int64_t part[16];
  int64_t s = 0;
  for (int j = threadIdx.x; j < r; j += blockDim.x) s += len[j];
  s = wave_sum_i64(s);
  const int w = threadIdx.x / kWave, nw = blockDim.x / kWave;
  __syncthreads();
  if (threadIdx.x % kWave == 0) part[w] = s;
  __syncthreads();
  int64_t t = 0;
  for (int i = 0; i < nw; ++i) t += part[i];
  return t;
}

}  // namespace pkv
