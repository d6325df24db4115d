// Generation-phase (decode) attention over the paged cache: split-KV pass + combine.
//
// "TensorRT-LLM 1.0 study notes", 6.3: a generation request has one query token that
// attends to every cached token, reached block by block through the block table; the
// phase is bound by HBM bandwidth.  This design splits each request's keys into
// chunks so that even a handful of long requests fills all 256 CUs, and merges the
// per-chunk partial results (running max m, sum l, unnormalised output o) in a
// second pass with the same rescaling identity FlashAttention uses to merge tiles
// (study notes 6.2, update of acc_o by the new running max).
//
// Pass 1, 4 waves per workgroup.  A workgroup takes one (generation request, KV head,
// chunk) and its waves stream alternate tiles of the chunk, their states merged in LDS at
// the end -- or, with the KV heads in fours and a one-byte cache (fp8 / int8), or a bf16
// cache read by GQA groups of 8 or more query heads in one block of columns (see
// decode_heads_per_wg), 4 neighbouring KV heads, one wave each, every wave streaming all
// tiles of the chunk for its head: the four waves then read the neighbouring pieces of the
// same cache rows at about the same time, which HBM serves faster than one head's pieces
// alone.  Per wave and tile:
//   * S^T = K Q^T on MFMA 16x16x32 bf16: A = 16 keys x 32 dims of K, loaded straight
//     from HBM in operand layout; B = the G query heads of the KV head (GQA group,
//     G <= 16, padded with zero heads), kept in registers for the whole chunk.
//   * online softmax per head on the accumulators (lanes l, l^16, l^32, l^48 hold the
//     same head), exp2 with the log2(e) factor folded into the scale.
//   * O += P V on MFMA: A = P (heads x 32 keys) straight from the score registers,
//     B = V read transposed from an LDS copy of the tile with ds_read_b64_tr_b16.
//   * an fp8 or int8 cache is dequantised to bf16 on load (exact: every e4m3 value
//     and every integer -128 .. 127 is a bf16 value); k_scale folds into the softmax
//     scale and v_scale into the combine, so the pass works on raw codes times one.
// Pass 2, one workgroup per (request, query head): M = max m_s, L = sum 2^(m_s-M) l_s,
// O = sum 2^(m_s-M) o_s / L in a fixed order (no atomics: bitwise reproducible).
#include <math.h>

#include "device_common.h"
#include "kernels.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kTile = 32;          // keys per wave iteration
constexpr int kD = 128;            // head_dim handled here
constexpr int kVStride = 136;      // LDS row stride (bf16 elements) of a staged V tile

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// 16 bytes of the cache, streamed.  Every K/V byte is read once per step and every load
// instruction covers whole rows (whole 128-byte lines), so the loads carry the
// nontemporal hint: lines are not kept for reuse that will not come.
__device__ __forceinline__ uint4 load_kv(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
// K tile in LDS: 16-byte chunk c of key row r sits at chunk position c ^ (r & 15), so the
// 16 rows one MFMA operand read touches at one chunk fall on 16 distinct bank groups.
__device__ __forceinline__ int kpos(int r, int c) { return c ^ (r & 15); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// two fp32 -> packed bf16, round to nearest-even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
// 8 e4m3 codes (two dwords) -> 8 bf16 values, exactly (every e4m3 value is a bf16 value):
// v_cvt_scalef32_pk_bf16_fp8 with scale 1 converts two codes per instruction.
__device__ __forceinline__ uint4 e4m3x8_to_bf16x8(uint2 c) {
  auto lo = [](uint32_t w) { return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)); };
  auto hi = [](uint32_t w) { return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)); };
  return make_uint4(lo(c.x), hi(c.x), lo(c.y), hi(c.y));
}

// 8 int8 codes (two dwords) -> 8 bf16 values, exactly: each byte is sign-extended and
// converted to fp32 (one SDWA v_cvt_f32_i32 per code); an integer of magnitude <= 128
// has at most 8 significant bits, so the upper half of its fp32 pattern is its bf16
// pattern, and v_perm_b32 packs two of them per dword.
__device__ __forceinline__ uint4 int8x8_to_bf16x8(uint2 c) {
  auto cv = [](uint32_t w, int byte) { return __float_as_uint(static_cast<float>(static_cast<int8_t>(w >> (8 * byte)))); };
  auto pk = [](uint32_t lo, uint32_t hi) { return __builtin_amdgcn_perm(hi, lo, 0x07060302u); };
  return make_uint4(pk(cv(c.x, 0), cv(c.x, 1)), pk(cv(c.x, 2), cv(c.x, 3)), pk(cv(c.y, 0), cv(c.y, 1)),
                    pk(cv(c.y, 2), cv(c.y, 3)));
}
// One-byte cache codes -> bf16 for the cache format KV.
template <int KV>
__device__ __forceinline__ uint4 codes8_to_bf16x8(uint2 c) {
  if constexpr (KV == F_INT8) return int8x8_to_bf16x8(c);
  else return e4m3x8_to_bf16x8(c);
}

__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Registers of one 32-key tile in flight: K and V rows as loaded (16 lanes per bf16
// row, 8 lanes per fp8 / int8 row), copied to LDS at compute time.
template <int KV>
struct TileRegs {
  uint4 k[KV == F_BF16 ? 8 : 4];
  uint4 v[KV == F_BF16 ? 8 : 4];
};

// B: KV heads per workgroup (1, or kWaves: one per wave).
template <int KV, int B>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_split_kernel(AttnArgs a) {
  static_assert(B == 1 || B == kWaves, "one head per workgroup, or one per wave");
  // KV head (group) fastest: the workgroups of every head of one (request, chunk) run
  // side by side.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wave-uniform
  const int hgs = a.Hkv / B;                                   // head groups
  const int g = (blockIdx.x % hgs) * B + (B == 1 ? 0 : wave);  // this wave's KV head
  const int cb = blockIdx.x / hgs, split = blockIdx.y, rg = blockIdx.z;
  const int r = a.req_begin + rg;
  // device lengths, kept to n >= 1 and S >= n whatever they hold
  const int n = max(a.ctx_len[r], 1);                          // 1, or 1 + draft tokens
  const int S = max(a.seq_len[r], n);
  const int G = a.H / a.Hkv;
  const int k0 = split * a.chunk;
  if (k0 >= S || split >= a.max_splits || cb * 16 >= G * n) return;   // uniform over the block
  const int kend = min(k0 + a.chunk, S);
  const int lane = threadIdx.x % kWave;
  const int li = lane % 16, lg = lane / 16;
  // Columns of the score tile: (token, query head) pairs, 16 per column block.  Lane
  // column li is token tok = gc / G of the request (position S - n + tok; it sees keys up
  // to that position: causal among a request's draft tokens) and head g*G + gc % G.
  const int gc = cb * 16 + li, tok = gc / G;
  const bool col_ok = tok < n;
  const int key_lim = col_ok ? S - n + tok : -1;               // keys 0 .. key_lim
  const int64_t row0 = a.max_n == 1 ? static_cast<int64_t>(a.row_begin) + rg : wave_prefix(a.ctx_len, r);
  if (row0 < a.row_begin || row0 + n > a.N) return;             // rows outside the generation rows: skip
  const int64_t row = row0 + min(tok, n - 1);
  const int64_t kv_row = static_cast<int64_t>(a.Hkv) * kD;     // elements per (block, K|V, slot)
  // The block table is read-only here: reading it through the constant address space
  // keeps its (wave-uniform) reads on the scalar unit, out of the vector-load queue.
  const __attribute__((address_space(4))) int32_t* table =
      (const __attribute__((address_space(4))) int32_t*)(a.table + static_cast<int64_t>(r) * a.mbps);

  __shared__ __attribute__((aligned(16))) uint16_t vtile[kWaves][kTile * kVStride];
  __shared__ __attribute__((aligned(16))) uint16_t ktile[kWaves][kTile * kD];

  // B operand Q^T: column li, dims ks*32 + lg*8 + j (the dim order inside a
  // contraction is free as long as K uses the same one).
  bf16x8 qf[4];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + row * a.q_stride +
                         static_cast<int64_t>(g * G + gc % G) * kD + lg * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint4 u = *reinterpret_cast<const uint4*>(qp + ks * 32);
      if (!col_ok) u = make_uint4(0, 0, 0, 0);
      qf[ks] = as_bf16x8(u);
    }
  }
  const float xscale = a.scale_log2 * a.k_scale;
  float m_run = -INFINITY, l_run = 0.f;                         // for column li
  f32x4 o[8];                                                   // O[column lg*4+i][dim nb*16+li]
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ntiles = (kend - k0 + kTile - 1) / kTile;
  const int tshift = a.tshift, tmask = a.T - 1;
  const int last_blk = min((kend - 1) >> tshift, a.mbps - 1);
  const int64_t blk_bytes = 2 * static_cast<int64_t>(a.T) * kv_row * (KV == F_BF16 ? 2 : 1);   // K and V of T slots
  uint16_t* vt = vtile[wave];
  uint16_t* kt = ktile[wave];
  // Load `it` of a tile covers rows it*kRows + lane/kLanes at byte column (lane%kLanes)*16
  // (16 lanes per 256-byte bf16 row, 8 per 128-byte fp8 / int8 row).
  constexpr int kEB = KV == F_BF16 ? 2 : 1;                    // cache element bytes
  constexpr int kLoads = KV == F_BF16 ? 8 : 4;
  constexpr int kRows = kWave * 16 / (kD * kEB);               // rows per load instruction
  constexpr int kLanes = kWave / kRows;                        // lanes per row
  const uint32_t row_bytes = static_cast<uint32_t>(kv_row) * kEB;
  uint32_t lane_off[kLoads];                                   // byte offset inside a tile
#pragma unroll
  for (int it = 0; it < kLoads; ++it)
    lane_off[it] = static_cast<uint32_t>(it * kRows + lane / kLanes) * row_bytes + (lane % kLanes) * 16u;
  // A tile needs no masking when it lies inside the chunk and inside the causal range of
  // every valid column of the block (the lowest of them is token cb*16 / G).
  const int lim_all = S - n + (cb * 16) / G;

  // Block IDs of a tile: tiles are 32-aligned and T is a power of two >= 16, so a tile
  // lies in one block (T >= 32) or covers two (T = 16).  Read two tiles ahead.
  auto fetch_ids = [&](int tile, int32_t (&raw)[2]) {
    const int kb0 = __builtin_amdgcn_readfirstlane((k0 + tile * kTile) >> tshift);
    raw[0] = __builtin_amdgcn_readfirstlane(table[min(kb0, last_blk)]);
    raw[1] = __builtin_amdgcn_readfirstlane(table[min(kb0 + 1, last_blk)]);
  };
  // Issue every load of tile `tile` (ids already resolved) into `R`.  Loads it < kLoads/2
  // cover tile rows 0..15, the others rows 16..31, so every load has one scalar base: B0
  // (the tile's block at the tile's first slot) or B1 (the block of rows 16..31; the
  // same block unless T = 16).  Rows past the chunk end are still slots of an allocated
  // block (in bounds); their scores are masked and their V rows zeroed in compute.
  auto issue = [&](int tile, const int32_t (&rawid)[2], TileRegs<KV>& R) {
    const int tb = k0 + tile * kTile;
    int32_t id0 = __builtin_amdgcn_readfirstlane(rawid[0]);
    int32_t id1 = __builtin_amdgcn_readfirstlane(rawid[1]);
    id0 = (id0 >= 0 && id0 < a.num_blocks) ? id0 : 0;
    id1 = (id1 >= 0 && id1 < a.num_blocks) ? id1 : 0;
    const char* head = static_cast<const char*>(a.pool) + g * (kD * kEB);
    const char* b0 = head + static_cast<int64_t>(id0) * blk_bytes + static_cast<int64_t>(tb & tmask) * row_bytes;
    const char* b1 = a.T >= kTile ? b0 : head + static_cast<int64_t>(id1) * blk_bytes - 16 * static_cast<int64_t>(row_bytes);
    const int64_t vofs = static_cast<int64_t>(a.T) * row_bytes;
#pragma unroll
    for (int it = 0; it < kLoads; ++it) R.k[it] = load_kv((it < kLoads / 2 ? b0 : b1) + lane_off[it]);
#pragma unroll
    for (int it = 0; it < kLoads; ++it) R.v[it] = load_kv((it < kLoads / 2 ? b0 : b1) + vofs + lane_off[it]);
  };
  // Online-softmax update and O += P V for tile `tile` held in `R`.
  auto compute = [&](int tile, const TileRegs<KV>& R) {
    const int tb = k0 + tile * kTile;
    // K and V rows into this wave's LDS tiles (bf16; an fp8 / int8 cache is dequantised here)
    wave_lds_fence();
    if constexpr (KV == F_BF16) {
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int row = it * 4 + lg;
        *reinterpret_cast<uint4*>(kt + row * kD + kpos(row, li) * 8) = R.k[it];
        *reinterpret_cast<uint4*>(vt + row * kVStride + li * 8) = R.v[it];
      }
    } else {
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int row = it * 8 + lane / 8, c0 = (lane % 8) * 2;
        *reinterpret_cast<uint4*>(kt + row * kD + kpos(row, c0) * 8) =
            codes8_to_bf16x8<KV>(make_uint2(R.k[it].x, R.k[it].y));
        *reinterpret_cast<uint4*>(kt + row * kD + kpos(row, c0 + 1) * 8) =
            codes8_to_bf16x8<KV>(make_uint2(R.k[it].z, R.k[it].w));
        uint16_t* d = vt + row * kVStride + (lane % 8) * 16;
        *reinterpret_cast<uint4*>(d) = codes8_to_bf16x8<KV>(make_uint2(R.v[it].x, R.v[it].y));
        *reinterpret_cast<uint4*>(d + 8) = codes8_to_bf16x8<KV>(make_uint2(R.v[it].z, R.v[it].w));
      }
    }
    if (tb + kTile > kend) {
      // wave-uniform, last tile of a chunk only: rows at or past the chunk end were read
      // from unwritten slots; zero their V so that P = 0 times them stays 0
#pragma unroll
      for (int it = 0; it < kLoads; ++it) {
        const int row = it * kRows + lane / kLanes;
        if (tb + row >= kend) {
          uint16_t* d = vt + row * kVStride + (lane % kLanes) * (kD / kLanes);
#pragma unroll
          for (int j = 0; j < kD / kLanes; j += 8) *reinterpret_cast<uint4*>(d + j) = make_uint4(0, 0, 0, 0);
        }
      }
    }
    wave_lds_fence();
    // A operand K: lane (li, lg) of step ks holds key kb*16 + li, dims ks*32 + lg*8 .. +7
    bf16x8 kf[2][4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int row = kb * 16 + li;
        kf[kb][ks] = as_bf16x8(*reinterpret_cast<const uint4*>(kt + row * kD + kpos(row, ks * 4 + lg) * 8));
      }
    // scores S^T[key][head]: lane holds head li, keys tb + kb*16 + lg*4 + i
    f32x4 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kb][ks], qf[ks], sacc[kb], 0, 0, 0);
    }
    float x[8];
    float tmax = -INFINITY;
    if (tb + kTile <= kend && tb + kTile - 1 <= lim_all) {      // wave-uniform: no masking
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = sacc[e / 4][e % 4] * xscale;
        tmax = fmaxf(tmax, x[e]);
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = tb + kb * 16 + lg * 4 + i;
          x[kb * 4 + i] = key < kend && key <= key_lim ? sacc[kb][i] * xscale : -INFINITY;
          tmax = fmaxf(tmax, x[kb * 4 + i]);
        }
    }
    tmax = xor_max<32>(xor_max<16>(tmax));
    // Lazy rescale: the reference m_run moves only when some column's tile max exceeds it
    // by more than 8 (log2 units); otherwise the tile's terms are taken against the old
    // reference (each at most 2^8) and O needs no rescaling.  (m, l, o) stay consistent
    // for the combine, whatever the reference.
    if (__builtin_amdgcn_ballot_w64(tmax > m_run + 8.f)) {
      const float m_new = fmaxf(m_run, tmax);
      // -inf while a draft column has seen no key of its causal range yet: offset 0 then
      // (every term is exp2(-inf) = 0), never -inf - -inf
      const float alpha = __builtin_amdgcn_exp2f(m_run - (m_new == -INFINITY ? 0.f : m_new));
      l_run *= alpha;
      m_run = m_new;
      // rescale O rows: lane's O rows are columns lg*4+i; their alpha lives in lane lg*4+i
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ah = __shfl(alpha, lg * 4 + i, kWave);
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) o[nb][i] *= ah;
      }
    }
    const float m_off = m_run == -INFINITY ? 0.f : m_run;
    float lsum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] = __builtin_amdgcn_exp2f(x[e] - m_off);
      lsum += x[e];
    }
    lsum = xor_sum<32>(xor_sum<16>(lsum));
    l_run += lsum;
    // P as the A operand: row = column li, k-slot j <-> key (j/4)*16 + lg*4 + j%4
    uint4 pu;
    pu.x = pack_bf16(x[0], x[1]);
    pu.y = pack_bf16(x[2], x[3]);
    pu.z = pack_bf16(x[4], x[5]);
    pu.w = pack_bf16(x[6], x[7]);
    const bf16x8 pa = as_bf16x8(pu);
    // O += P V: B operand = V[keys][dims nb*16 .. +15] read transposed
    const int krow = lg * 4 + li / 4;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const uint16_t* src = vt + krow * kVStride + nb * 16 + 4 * (li % 4);
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(src));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(src + 16 * kVStride));
      const uint4 u = make_uint4(__builtin_bit_cast(uint2, lo).x, __builtin_bit_cast(uint2, lo).y,
                                 __builtin_bit_cast(uint2, hi).x, __builtin_bit_cast(uint2, hi).y);
      o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, as_bf16x8(u), o[nb], 0, 0, 0);
    }
  };

  // Software pipeline: the wave's next tile is in flight while a tile is computed (B = 1:
  // the wave's tiles are w, w + 4, ...; B = 4: every tile).  Loads and ID fetches run
  // unconditionally (past the wave's last tile they repeat the chunk's last tile), so
  // every path has the same loads in flight and the compiler's wait before a tile's
  // compute covers that tile only, not the one issued after it.
  constexpr int TS = B == 1 ? kWaves : 1;                      // tile stride of a wave
  TileRegs<KV> ra, rb;
  int32_t ids_a[2], ids_b[2];
  const int tl = ntiles - 1;
  int t = B == 1 ? wave : 0;
  fetch_ids(min(t, tl), ids_a);
  issue(min(t, tl), ids_a, ra);
  fetch_ids(min(t + TS, tl), ids_b);
  for (; t < ntiles; t += 2 * TS) {
    issue(min(t + TS, tl), ids_b, rb);
    fetch_ids(min(t + 2 * TS, tl), ids_a);
    compute(t, ra);
    issue(min(t + 2 * TS, tl), ids_a, ra);
    fetch_ids(min(t + 3 * TS, tl), ids_b);
    if (t + TS < ntiles) compute(t + TS, rb);
  }
  const int ncol = min(16, G * n - cb * 16);                     // valid columns of the block
  if constexpr (B > 1) {
    // ---- this wave alone holds its head's state for the chunk: write (m, l, o) as they are
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = lg * 4 + i, cc = cb * 16 + c;
      if (c < ncol) {
        const int64_t part = ((row0 - a.row_begin + cc / G) * a.H + g * G + cc % G) * a.max_splits + split;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) a.ws_o[part * kD + nb * 16 + li] = o[nb][i];
      }
    }
    if (lg == 0 && li < ncol) {
      const int cc = cb * 16 + li;
      const int64_t part = ((row0 - a.row_begin + cc / G) * a.H + g * G + cc % G) * a.max_splits + split;
      a.ws_ml[part * 2] = m_run;
      a.ws_ml[part * 2 + 1] = l_run;
    }
    return;
  }

  // ---- merge the 4 waves' partial states, then write the chunk's (m, l, o)
  __syncthreads();
  float* red = reinterpret_cast<float*>(&vtile[0][0]);          // [wave][16 heads][kD]
  __shared__ float ml[kWaves][16][2];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wave * 16 + lg * 4 + i) * kD + nb * 16 + li] = o[nb][i];
  if (lg == 0) {
    ml[wave][li][0] = m_run;
    ml[wave][li][1] = l_run;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < ncol * kD; e += kThreads) {
    const int c = e / kD, d = e % kD;
    const int cc = cb * 16 + c;                                 // (token cc / G, head g*G + cc % G)
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, ml[w][c][0]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float s = ml[w][c][0] == -INFINITY ? 0.f : exp2f(ml[w][c][0] - M);
      L += s * ml[w][c][1];
      O += s * red[(w * 16 + c) * kD + d];
    }
    const int64_t tok_row = row0 - a.row_begin + cc / G;        // generation row of the token
    const int64_t part = (tok_row * a.H + g * G + cc % G) * a.max_splits + split;
    a.ws_o[part * kD + d] = O;
    if (d == 0) {
      a.ws_ml[part * 2] = M;
      a.ws_ml[part * 2 + 1] = L;
    }
  }
}

// One workgroup of kD threads per (generation token, query head).  Thread s < ns
// first loads split s's (m, l); a fixed-shape tree gives M = max m and L = sum 2^(m-M) l;
// then thread d sums 2^(m_s-M) o_s[d] over the splits in order, eight loads in flight.
// Splits past a draft token's position hold m = -inf and weigh nothing; split 0 always
// holds key 0, so M is finite.
__global__ __launch_bounds__(kD) void decode_combine_kernel(AttnArgs a) {
  static_assert(kD >= 128, "one thread per split needs kD >= kMaxSplits");
  const int h = blockIdx.x, rg = blockIdx.y, tok = blockIdx.z, t = threadIdx.x;
  const int r = a.req_begin + rg;
  if (tok >= a.ctx_len[r]) return;                                  // uniform
  const int S = a.seq_len[r];
  const int ns = min((S + a.chunk - 1) / a.chunk, a.max_splits);
  const int64_t row = (a.max_n == 1 ? static_cast<int64_t>(a.row_begin) + rg : wave_prefix(a.ctx_len, r)) + tok;
  if (row < a.row_begin || row >= a.N) return;                      // uniform: outside the generation rows
  const int64_t base = ((row - a.row_begin) * a.H + h) * a.max_splits;
  __shared__ float s_w[kD];
  __shared__ float s_red[kD / kWave];
  const float m_t = t < ns ? a.ws_ml[(base + t) * 2] : -INFINITY;
  const float l_t = t < ns ? a.ws_ml[(base + t) * 2 + 1] : 0.f;   // 0 wherever m_t = -inf
  float M = wave_max(m_t);
  if (t % kWave == 0) s_red[t / kWave] = M;
  __syncthreads();
  M = s_red[0];
#pragma unroll
  for (int w = 1; w < kD / kWave; ++w) M = fmaxf(M, s_red[w]);
  const float w_t = t < ns && m_t != -INFINITY ? exp2f(m_t - M) : 0.f;
  s_w[t] = w_t;
  float L = wave_sum(w_t * l_t);
  __syncthreads();
  if (t % kWave == 0) s_red[t / kWave] = L;
  __syncthreads();
  L = s_red[0];
#pragma unroll
  for (int w = 1; w < kD / kWave; ++w) L += s_red[w];
  float o = 0.f;
  const float* op = a.ws_o + base * kD + t;
  int s = 0;
  for (; s + 8 <= ns; s += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = op[static_cast<int64_t>(s + u) * kD];
#pragma unroll
    for (int u = 0; u < 8; ++u) o += s_w[s + u] * v[u];
  }
  for (; s < ns; ++s) o += s_w[s] * op[static_cast<int64_t>(s) * kD];
  const float val = o * (a.v_scale / L);
  const int64_t oi = row * a.H * kD + static_cast<int64_t>(h) * kD + t;
  if (a.out_fmt == F_FP8)
    static_cast<uint8_t*>(a.out)[oi] = static_cast<uint8_t>(f32_to_e4m3(val * a.out_mul));
  else
    static_cast<uint16_t*>(a.out)[oi] = static_cast<uint16_t>(f32_to_bf16(val));
}

}  // namespace

hipError_t launch_decode_split(const AttnArgs& a, hipStream_t s) {
  const int kv_bytes = a.kv_fmt == F_FP8 || a.kv_fmt == F_INT8 ? 1 : a.kv_fmt == F_BF16 ? 2 : 4;
  const int B = decode_heads_per_wg(kv_bytes, a.Hkv, a.H / a.Hkv, a.col_blocks);
  const dim3 grid(a.Hkv / B * a.col_blocks, a.max_splits, a.req_end - a.req_begin);
  if (a.kv_fmt == F_FP8) {
    if (B == kWaves) hipLaunchKernelGGL((decode_split_kernel<F_FP8, kWaves>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((decode_split_kernel<F_FP8, 1>), grid, dim3(kThreads), 0, s, a);
  } else if (a.kv_fmt == F_INT8) {
    if (B == kWaves) hipLaunchKernelGGL((decode_split_kernel<F_INT8, kWaves>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((decode_split_kernel<F_INT8, 1>), grid, dim3(kThreads), 0, s, a);
  } else {
    if (B == kWaves) hipLaunchKernelGGL((decode_split_kernel<F_BF16, kWaves>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((decode_split_kernel<F_BF16, 1>), grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_decode_combine(const AttnArgs& a, hipStream_t s) {
  const dim3 grid(a.H, a.req_end - a.req_begin, a.max_n);
  hipLaunchKernelGGL(decode_combine_kernel, grid, dim3(kD), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
