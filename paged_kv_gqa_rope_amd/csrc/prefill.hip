// Context-phase (prefill / chunked prefill) attention on bf16 MFMA for gfx950.
//
// "TensorRT-LLM 1.0 study notes", 6.1-6.2: the context phase runs FlashAttention --
// an outer loop over query tiles, an inner loop over key/value tiles staged in on-chip
// memory, S = Q K^T and O += P V on the matrix units with fp32 accumulation, and an
// online softmax that rescales the running output whenever the running maximum grows.
// Rows are causal over the request's cached prefix plus its chunk ("TensorRT-LLM source
// analysis report", 1.3, chunked context); K/V come from the paged pool through the
// block table ("TensorRT-LLM source teardown part 1", KV cache manager interfaces).
//
// CDNA4 mapping:
//  * one workgroup = one KV head's whole GQA group (G = 1, 2, 4 or 8) for a block of
//    query positions: 4 waves (8 when G = 8), each owning 32 query rows of one query
//    head, so every K/V tile staged in LDS feeds all G heads that share it; two
//    workgroups share a CU so one's softmax overlaps the other's MFMAs;
//  * the transposed products keep the softmax in-lane: S^T = K Q^T on
//    v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 dims of K from LDS, B = Q^T held in
//    registers), so lane l owns query l%32 and 16 keys per 32-key block, and the row
//    max/sum need one cross-lane step (lanes l and l^32);
//  * O^T = V^T P^T: B = P^T straight from the score accumulators (converted to bf16),
//    A = V^T read from LDS with ds_read_b64_tr_b16;
//  * 64-key tiles are double-buffered in LDS (global loads for tile t+1 are in flight
//    while tile t is computed), block IDs are fetched two tiles ahead;
//  * only tiles that cross the diagonal are masked, fully masked tiles are skipped, and
//    the output rescale is skipped when no lane's running maximum moved.
#include <math.h>

#include "device_common.h"
#include "kernels.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kD = 128;
constexpr int kTileK = 64;                 // keys per LDS tile
constexpr int kKStride = 136;              // LDS row stride of K (272 B: b128 reads conflict-free)
constexpr int kVStride = 160;              // LDS row stride of V (320 B: the 4 rows of a transposed read hit disjoint banks)
constexpr int kKBuf = kTileK * kKStride;
constexpr float kLazyLog2 = 8.f;           // rescale only when the maximum grows by > 2^8
constexpr int kXcds = 8;                   // MI355X accelerator complex dies
constexpr int kVBuf = kTileK * kVStride;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

template <int NW, int G>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_kernel(AttnArgs a) {
  constexpr int RB = NW / G;               // 32-row blocks per workgroup
  constexpr int ROWS = RB * 32;            // query positions per workgroup
  constexpr int NT = NW * kWave;
  // XCD-aware placement: workgroups go to the 8 XCDs round-robin by linear ID, so when
  // the (request, KV head) pairs split evenly, linear ID L runs on XCD L % 8 and takes
  // that XCD's (L / 8)-th item; all query tiles of one pair then share one L2.
  const int nq = a.max_n > 0 ? (a.max_n + ROWS - 1) / ROWS : 1;   // query tiles of the longest chunk
  const int np = a.Hkv * (a.req_end - a.req_begin);                 // (request, KV head) pairs
  const int L = blockIdx.x;
  int pair, qt;
  if (np % kXcds == 0) {
    const int j = L / kXcds;
    pair = (j / nq) * kXcds + L % kXcds;
    qt = j % nq;
  } else {
    pair = L / nq;
    qt = L % nq;
  }
  const int g = pair % a.Hkv;
  const int r = a.req_begin + pair / a.Hkv;
  const int n = a.ctx_len[r];
  const int ntq = (n + ROWS - 1) / ROWS;
  if (qt >= ntq) return;                                            // uniform
  const int qtile = ntq - 1 - qt;                                   // heaviest tiles first
  const int S = a.seq_len[r];
  const int past = S - n;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int l32 = lane % 32, lh = lane / 32;
  const int h = g * G + wave % G;
  const int q0 = qtile * ROWS + (wave / G) * 32;                        // first row of this wave
  const bool wave_active = q0 < n;
  const int qlast = min(q0 + 31, n - 1);                                // last valid row
  const int wave_max_pos = past + qlast;
  const int tile_rows_end = min(qtile * ROWS + ROWS, n);               // rows of the workgroup
  const int kv_end = past + tile_rows_end;                              // keys 0 .. kv_end-1
  const int ntiles = (kv_end + kTileK - 1) / kTileK;
  const int64_t row0 = wave_prefix(a.ctx_len, r);                       // packed row of request r
  const int tshift = a.tshift, tmask = a.T - 1;
  const int64_t kv_row = static_cast<int64_t>(a.Hkv) * kD;
  const int64_t blk_elems = 2 * static_cast<int64_t>(a.T) * kv_row;
  const int32_t* table = a.table + static_cast<int64_t>(r) * a.mbps;
  const int last_blk = (S - 1) >> tshift;

  __shared__ __attribute__((aligned(16))) uint16_t kbuf[2][kKBuf];
  __shared__ __attribute__((aligned(16))) uint16_t vbuf[2][kVBuf];

  // ---- Q^T (B operand): query q0 + l32, dims lh*64 + ks*8 + j for ks = 0..7
  bf16x8 qf[8];
  {
    const int qi = min(q0 + l32, n - 1);
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (row0 + qi) * a.q_stride +
                         static_cast<int64_t>(h) * kD + lh * 64;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(qp + ks * 8));
  }
  const int my_pos = past + min(q0 + l32, n - 1);                       // this lane's query position
  const float c = a.scale_log2;

  // ---- cooperative tile loads: thread t moves the 16-byte chunk t%16 of K and V rows
  //      t/16 + u*NT/16 of the tile
  constexpr int KCH = (kTileK * 16) / NT;              // 16-byte chunks of K (and of V) per thread
  static_assert(KCH == 2 || KCH == 4, "4 or 8 waves per workgroup");
  const int ccol = (threadIdx.x % 16) * 8;
  const int crow0 = threadIdx.x / 16;                  // chunk u covers tile row crow0 + u*NT/16
  // Two register stages (tiles t+1 and t+2 in flight) and the block IDs of the tile
  // after those, all in named registers (indexable arrays here end up in scratch).
  struct Stage {
    u32x4 k0, k1, k2, k3, v0, v1, v2, v3;
  };
  Stage st0, st1;
  int32_t in0 = 0, in1 = 0, in2 = 0, in3 = 0;
  auto key_of = [&](int tile, int u) __attribute__((always_inline)) { return min(tile * kTileK + crow0 + u * (NT / 16), S - 1); };
  auto id_of = [&](int tile, int u) __attribute__((always_inline)) { return table[min(key_of(tile, u) >> tshift, last_blk)]; };
  auto fetch_ids = [&](int tile) __attribute__((always_inline)) {
    in0 = id_of(tile, 0);
    in1 = id_of(tile, 1);
    if constexpr (KCH == 4) {
      in2 = id_of(tile, 2);
      in3 = id_of(tile, 3);
    }
  };
  auto chunk_ptr = [&](int tile, int u, int32_t id) __attribute__((always_inline)) {  // K chunk; its V chunk is T rows later
    id = (id >= 0 && id < a.num_blocks) ? id : 0;       // clamped key: never an unwritten slot
    return static_cast<const uint16_t*>(a.pool) + static_cast<int64_t>(id) * blk_elems +
           static_cast<int64_t>(key_of(tile, u) & tmask) * kv_row + static_cast<int64_t>(g) * kD + ccol;
  };
  const int64_t vofs = static_cast<int64_t>(a.T) * kv_row;
  auto issue = [&](int tile, Stage& q) __attribute__((always_inline)) {
    const uint16_t* p0 = chunk_ptr(tile, 0, in0);
    const uint16_t* p1 = chunk_ptr(tile, 1, in1);
    q.k0 = *reinterpret_cast<const u32x4*>(p0);
    q.k1 = *reinterpret_cast<const u32x4*>(p1);
    q.v0 = *reinterpret_cast<const u32x4*>(p0 + vofs);
    q.v1 = *reinterpret_cast<const u32x4*>(p1 + vofs);
    if constexpr (KCH == 4) {
      const uint16_t* p2 = chunk_ptr(tile, 2, in2);
      const uint16_t* p3 = chunk_ptr(tile, 3, in3);
      q.k2 = *reinterpret_cast<const u32x4*>(p2);
      q.k3 = *reinterpret_cast<const u32x4*>(p3);
      q.v2 = *reinterpret_cast<const u32x4*>(p2 + vofs);
      q.v3 = *reinterpret_cast<const u32x4*>(p3 + vofs);
    }
  };
  auto commit = [&](int buf, const Stage& q) __attribute__((always_inline)) {
    constexpr int RS = NT / 16;                         // rows between chunks
    *reinterpret_cast<u32x4*>(&kbuf[buf][crow0 * kKStride + ccol]) = q.k0;
    *reinterpret_cast<u32x4*>(&kbuf[buf][(crow0 + RS) * kKStride + ccol]) = q.k1;
    *reinterpret_cast<u32x4*>(&vbuf[buf][crow0 * kVStride + ccol]) = q.v0;
    *reinterpret_cast<u32x4*>(&vbuf[buf][(crow0 + RS) * kVStride + ccol]) = q.v1;
    if constexpr (KCH == 4) {
      *reinterpret_cast<u32x4*>(&kbuf[buf][(crow0 + 2 * RS) * kKStride + ccol]) = q.k2;
      *reinterpret_cast<u32x4*>(&kbuf[buf][(crow0 + 3 * RS) * kKStride + ccol]) = q.k3;
      *reinterpret_cast<u32x4*>(&vbuf[buf][(crow0 + 2 * RS) * kVStride + ccol]) = q.v2;
      *reinterpret_cast<u32x4*>(&vbuf[buf][(crow0 + 3 * RS) * kVStride + ccol]) = q.v3;
    }
  };

  float m_run = -INFINITY, l_run = 0.f;      // raw-score max of query l32; this lane's partial sum
  f32x16 o[4];                               // O^T[dim blk*32 + (i/4)*8 + lh*4 + i%4][query l32]
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[b][i] = 0.f;

  // Tile t is computed from LDS buffer t%2 while tiles t+1 and t+2 are in flight in
  // the two register stages; the loop is unrolled by two so each half uses fixed
  // stages (tile t+1 sits in the stage the other half filled).
#define PKV_PREFILL_TILE(T_, BUF_) \
  do { \
    const int kb0 = (T_) * kTileK; \
    if (wave_active && kb0 <= wave_max_pos) { \
      const uint16_t* kt = kbuf[BUF_]; \
      const uint16_t* vt = vbuf[BUF_]; \
      /* ---- S^T = K Q^T: two 32-key blocks, their MFMA chains interleaved and the K */ \
      /* operands read from LDS one step ahead */ \
      f32x16 s[2]; \
_Pragma("unroll") \
      for (int i = 0; i < 16; ++i) s[0][i] = s[1][i] = 0.f; \
      const uint16_t* kr0 = kt + l32 * kKStride + lh * 64; \
      const uint16_t* kr1 = kr0 + 32 * kKStride; \
      bf16x8 ka = as_bf16x8(*reinterpret_cast<const uint4*>(kr0)); \
      bf16x8 kc = as_bf16x8(*reinterpret_cast<const uint4*>(kr1)); \
_Pragma("unroll") \
      for (int ks = 0; ks < 8; ++ks) { \
        bf16x8 na = ka, nc = kc; \
        if (ks < 7) { \
          na = as_bf16x8(*reinterpret_cast<const uint4*>(kr0 + (ks + 1) * 8)); \
          nc = as_bf16x8(*reinterpret_cast<const uint4*>(kr1 + (ks + 1) * 8)); \
        } \
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s[0], 0, 0, 0); \
        s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kc, qf[ks], s[1], 0, 0, 0); \
        ka = na; \
        kc = nc; \
      } \
      /* ---- causal mask on tiles that cross this wave's diagonal (or the end of the keys) */ \
      if (kb0 + kTileK - 1 > past + q0) { \
        const int lim = my_pos - kb0 - lh * 4;                 /* key offset kb*32+(i/4)*8+i%4 <= lim */ \
_Pragma("unroll") \
        for (int kb = 0; kb < 2; ++kb) \
_Pragma("unroll") \
          for (int i = 0; i < 16; ++i) \
            s[kb][i] = (kb * 32 + (i / 4) * 8 + (i % 4) <= lim) ? s[kb][i] : -INFINITY; \
      } \
      /* ---- online softmax (raw-score domain; exp2 of (s - m) * c) */ \
      float tmax = -INFINITY; \
_Pragma("unroll") \
      for (int kb = 0; kb < 2; ++kb) \
_Pragma("unroll") \
        for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[kb][i]); \
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave)); \
      /* Lazy rescaling: the running maximum used as the exponent offset only moves when a */ \
      /* score exceeds it by more than 2^8 in exp2 units, so P stays <= 256 (exact enough */ \
      /* in fp32 sums and bf16 products) and most tiles skip the rescale of O.  The first */ \
      /* tile always sets it (m_run starts at -inf). */ \
      if (__any((tmax - m_run) * c > kLazyLog2)) { \
        const float m_new = fmaxf(m_run, tmax); \
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c); \
        l_run *= alpha; \
_Pragma("unroll") \
        for (int b = 0; b < 4; ++b) \
_Pragma("unroll") \
          for (int i = 0; i < 16; ++i) o[b][i] *= alpha; \
        m_run = m_new; \
      } \
      const float mc = m_run * c; \
      /* P^T as four B operands (16 keys each): slot j of step ks2 is s[ks2/2][(ks2%2)*8 + j] */ \
      bf16x8 pb[4]; \
_Pragma("unroll") \
      for (int ks2 = 0; ks2 < 4; ++ks2) { \
        const int kb = ks2 / 2, i0 = (ks2 % 2) * 8; \
        float p[8]; \
_Pragma("unroll") \
        for (int j = 0; j < 8; ++j) { \
          p[j] = __builtin_amdgcn_exp2f(fmaf(s[kb][i0 + j], c, -mc)); \
          l_run += p[j]; \
        } \
        pb[ks2] = as_bf16x8(make_uint4(pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]), \
                                       pack_bf16(p[6], p[7]))); \
      } \
      /* ---- O^T += V^T P^T over four 16-key steps */ \
_Pragma("unroll") \
      for (int ks2 = 0; ks2 < 4; ++ks2) { \
        /* source rows for the transposed read: keys ks2*16 + lh*4 + (lane%16)/4 (+8) */ \
        const int krow = ks2 * 16 + lh * 4 + (lane % 16) / 4; \
_Pragma("unroll") \
        for (int b = 0; b < 4; ++b) { \
          const int dcol = b * 32 + ((lane / 16) % 2) * 16 + 4 * (lane % 4); \
          const uint16_t* src = vt + krow * kVStride + dcol; \
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(src)); \
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(src + 8 * kVStride)); \
          const uint4 u = make_uint4(__builtin_bit_cast(uint2, lo).x, __builtin_bit_cast(uint2, lo).y, \
                                     __builtin_bit_cast(uint2, hi).x, __builtin_bit_cast(uint2, hi).y); \
          o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(u), pb[ks2], o[b], 0, 0, 0); \
        } \
      } \
    } \
  } while (0)
  fetch_ids(0);
  issue(0, st0);
  if (ntiles > 1) {
    fetch_ids(1);
    issue(1, st1);
  }
  if (ntiles > 2) fetch_ids(2);
  commit(0, st0);
  __syncthreads();
  for (int t = 0; t < ntiles; t += 2) {
    if (t + 2 < ntiles) {                     // even tile: st0 free, st1 holds tile t+1
      issue(t + 2, st0);
      if (t + 3 < ntiles) fetch_ids(t + 3);
    }
    PKV_PREFILL_TILE(t, 0);
    if (t + 1 < ntiles) commit(1, st1);
    __syncthreads();
    if (t + 1 >= ntiles) break;
    if (t + 3 < ntiles) {                     // odd tile: st1 free, st0 holds tile t+2
      issue(t + 3, st1);
      if (t + 4 < ntiles) fetch_ids(t + 4);
    }
    PKV_PREFILL_TILE(t + 1, 1);
    if (t + 2 < ntiles) commit(0, st0);
    __syncthreads();
  }
#undef PKV_PREFILL_TILE

  // ---- normalise and store: lane owns query l32 and dims blk*32 + (i/4)*8 + lh*4 + i%4
  if (!wave_active) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  const float inv = 1.f / l_tot;
  const int qi = q0 + l32;
  if (qi >= n) return;
  uint16_t* op = static_cast<uint16_t*>(a.out) + (row0 + qi) * static_cast<int64_t>(a.H) * kD +
                 static_cast<int64_t>(h) * kD;
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d = b * 32 + i4 * 8 + lh * 4;
      const uint32_t w0 = pack_bf16(o[b][i4 * 4 + 0] * inv, o[b][i4 * 4 + 1] * inv);
      const uint32_t w1 = pack_bf16(o[b][i4 * 4 + 2] * inv, o[b][i4 * 4 + 3] * inv);
      *reinterpret_cast<uint2*>(op + d) = make_uint2(w0, w1);
    }
}

template <int NW, int G>
hipError_t launch_t(const AttnArgs& a, hipStream_t s) {
  static_assert(NW % G == 0, "a workgroup holds whole query groups");
  constexpr int ROWS = (NW / G) * 32;
  const int nq = (a.max_n + ROWS - 1) / ROWS;
  const dim3 grid(nq * a.Hkv * (a.req_end - a.req_begin));
  hipLaunchKernelGGL((prefill_kernel<NW, G>), grid, dim3(NW * kWave), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const AttnArgs& a, hipStream_t s) {
  switch (a.H / a.Hkv) {
    case 1: return launch_t<4, 1>(a, s);
    case 2: return launch_t<4, 2>(a, s);
    case 4: return launch_t<4, 4>(a, s);
    case 8: return launch_t<8, 8>(a, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace pkv
