// Device code of the context-phase attention (see prefill.hip for the design), shared
// by the context kernel and the mixed-batch kernel.
#pragma once
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace pkv {
namespace {
namespace pf {


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kD = 128;
constexpr int kTileK = 64;                     // keys per LDS tile
constexpr int kRowBytes = kD * 2;              // one key's K (or V) row of one KV head
constexpr int kTileBytes = kTileK * kRowBytes; // 16 KB
constexpr int kStageBytes = 2 * kTileBytes;    // K tile, then V tile
constexpr int kChunksPerStage = kStageBytes / 1024;   // 1 KB per wave-wide 16-byte load
constexpr float kLazyLog2 = 8.f;               // rescale only when the maximum grows by > 2^8
constexpr int kXcds = 8;                       // MI355X accelerator complex dies

// LDS swizzles: 16-byte chunk c of tile row r sits at chunk position c ^ f(r).
//  K is read with ds_read_b128, 16 lanes per phase on 16 rows at one chunk: f = r & 15
//  spreads them over all 64 banks.  V is read with ds_read_b64_tr_b16, each phase on 4
//  rows x 4 neighbouring chunks: f = (r & 3) << 2 puts the 4 rows in different chunk groups.
__device__ __forceinline__ int swz_k(int r) { return r & 15; }
__device__ __forceinline__ int swz_v(int r) { return (r & 3) << 2; }

// s_waitcnt immediate for vmcnt(n) that leaves the other counters unconstrained
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }
// two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
// ds_read_b64_tr_b16 issued as inline asm: the compiler would otherwise wait for every
// outstanding global-to-LDS tile load before it (it cannot tell the stages apart).  The
// results are only valid after an lgkm wait has been passed them.
template <int OFF>
__device__ __forceinline__ s16x4 tr_read(uint32_t addr) {
  s16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
template <int N>
__device__ __forceinline__ void lgkm_wait2(s16x4& v0, s16x4& v1) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(v0), "+v"(v1) : "i"(N));
}
// ds_read_b128 issued as inline asm (same reason as tr_read)
template <int OFF>
__device__ __forceinline__ u32x4 k_read(uint32_t addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
// wait until at most N LDS operations of this wave are outstanding; the operands tie the
// values of the reads that must have completed to the wait
template <int N>
__device__ __forceinline__ void lgkm_wait(u32x4& k0, u32x4& k1) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(k0), "+v"(k1) : "i"(N));
}
// 16-byte global load issued as inline asm into a register the caller keeps in place
// ("+v"): the compiler would otherwise wait for it, and with it for every tile load in
// flight, at its first use.  The value is only valid after a vmcnt wait that covers it.
template <int OFF>
__device__ __forceinline__ void g_load16(u32x4& r, const void* p) {
  asm volatile("global_load_dwordx4 %0, %1, off offset:%2" : "+v"(r) : "v"(p), "i"(OFF));
}
template <int I>
using ic = std::integral_constant<int, I>;
// f(ic<I>()) for I = B .. E-1, unrolled at compile time
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(ic<B>());
    static_for<B + 1, E>(f);
  }
}

// Block-wide exclusive prefix sum of one int per thread (blockDim.x = NT, a multiple of
// 64); part[] holds NT / 64 wave totals.  Every thread calls it (it synchronises).
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* part) {
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  int x = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(x, d, kWave);
    if (lane >= d) x += y;
  }
  if (lane == kWave - 1) part[w] = x;
  __syncthreads();
  int off = 0;
  for (int i = 0; i < w; ++i) off += part[i];
  __syncthreads();
  return off + x - v;
}

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Persistent schedule.  An item is (request, KV head, query tile); its cost is its number
// of 64-key tiles, largest for the last query tile of a chunk.  A group's items are
// numbered request by request in the order the host gives (most tiles first), KV head by
// KV head within a request, and heaviest query tile first within a (request, KV head):
// s = (items of earlier requests) + (KV head within the group) * ntq + k, with ntq the
// request's query tiles and k = 0 its last one.  Workgroup w of the W in its group takes
// the items s = j * W + (j even ? w : W - 1 - w), j = 0, 1, ...: every round of W items is
// dealt out in alternating direction, so the sums of the costs even out, and the W
// workgroups of a round mostly share one (request, KV head), whose K/V then stays in L2.
// Groups: when the KV heads split evenly over the 8 XCDs (workgroups go to the XCDs
// round-robin by linear ID), group x = ID % 8 holds the KV heads h = x (mod 8) of every
// request and runs on XCD x; otherwise one group holds everything.
//
// BT: a cache block holds a whole number of 64-key tiles (tokens_per_block >= 64), so a
// tile sits in one block and its address is scalar.  Otherwise a tile spans 64/T <= 4
// blocks and each lane picks its row's block among the tile's (scalar) block IDs.
// LDS bytes of prefill_body: NS stages of the ring, the request table and the scan
// scratch of one workgroup of NW waves.
template <int NS>
__host__ __device__ constexpr int prefill_lds_bytes() {
  return NS * kStageBytes + 16 * kPrefillMaxReqs + 4 * (kPrefillMaxReqs + 1) + 4 * 8;
}

template <int NW, int G, int NS, bool BT>
__device__ __forceinline__ void prefill_body(const AttnArgs& a, const PrefillSched& sc, int bid, int nbid,
                                             unsigned char* lds) {
  constexpr int RB = NW / G;               // 32-row blocks per workgroup
  constexpr int ROWS = RB * 32;            // query positions per item
  constexpr int NT = NW * kWave;
  constexpr int LPW = kChunksPerStage / NW;   // 1 KB loads per wave per tile
  static_assert(kChunksPerStage % NW == 0, "whole loads per wave");
  static_assert(NS >= 2, "at least double buffering");
  static_assert(NT >= kPrefillMaxReqs, "one request per thread when the table is built");

  // LDS (prefill_lds_bytes<NS>() bytes, 1 KB aligned): the tile ring, then the request table
  unsigned char* const ring = lds;
  int4* const s_req = reinterpret_cast<int4*>(lds + NS * kStageBytes);   // {n, S, first packed row, request}
  int32_t* const s_pre = reinterpret_cast<int32_t*>(s_req + kPrefillMaxReqs);   // a group's items before each request
  int32_t* const s_part = s_pre + kPrefillMaxReqs + 1;

  const int tid = threadIdx.x;
  const int wave = uni(tid / kWave);
  const int lane = tid % kWave;
  const int l32 = lane % 32, lh = lane / 32;
  const int nreq = sc.nreq, hpg = sc.hpg;

  // ---- request table: lengths and first packed rows in the host's order, then the
  //      running count of a group's items over that order
  {
    const int64_t base = block_prefix(a.ctx_len, a.req_begin);
    int n = 0, S = 0;
    if (tid < nreq) {      // device lengths, kept to n >= 1 and S >= n whatever they hold
      n = max(a.ctx_len[a.req_begin + tid], 1);
      S = max(a.seq_len[a.req_begin + tid], n);
    }
    const int ex = block_excl_scan<NT>(n, s_part);
    if (tid < nreq) {
      const int at = sc.rank[tid];
      s_req[at] = make_int4(n, S, static_cast<int>(base + ex), a.req_begin + tid);
      s_pre[at] = hpg * ((n + ROWS - 1) / ROWS);
    }
  }
  __syncthreads();
  {
    const int v = tid < nreq ? s_pre[tid] : 0;
    const int ex = block_excl_scan<NT>(v, s_part);
    if (tid < nreq) s_pre[tid] = ex;
    if (tid == nreq - 1) s_pre[nreq] = ex + v;
  }
  __syncthreads();

  const int groups = sc.groups;
  const int x = bid % groups;
  const int w = bid / groups;
  const int W = nbid / groups;
  const int Mg = uni(s_pre[nreq]);
  const int full = Mg / W, rem = Mg - full * W;
  const int J = full + (((full & 1) ? W - 1 - w : w) < rem ? 1 : 0);   // this workgroup's items
  if (J == 0) return;                                                  // uniform

  struct Item {
    int r, g, qtile, n, S, row0, ntiles;
  };
  auto item = [&](int j) __attribute__((always_inline)) {
    const int s = j * W + ((j & 1) ? W - 1 - w : w);
    int lo = 0, hi = nreq - 1;                                         // last request i with s_pre[i] <= s
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (uni(s_pre[mid]) <= s) lo = mid;
      else hi = mid - 1;
    }
    const int4 q = s_req[lo];
    Item it;
    it.n = uni(q.x);
    it.S = uni(q.y);
    it.row0 = uni(q.z);
    it.r = uni(q.w);
    const int ntq = (it.n + ROWS - 1) / ROWS;
    const int off = s - uni(s_pre[lo]);
    const int gl = off / ntq, k = off - gl * ntq;
    it.g = gl * groups + x;
    it.qtile = max(ntq - 1 - k, 0);
    const int kv_end = (it.S - it.n) + min(it.qtile * ROWS + ROWS, it.n);
    it.ntiles = max((kv_end + kTileK - 1) / kTileK, 1);
    return it;
  };

  const uint32_t ring_b = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) unsigned char*)(ring)));
  const float c = a.scale_log2;

  // ---- tile loads: wave w moves the 1 KB chunks q = w*LPW + j of a stage (K tile: q < 16,
  //      V tile: q >= 16); chunk q holds tile rows 4*(q%16) .. +3 and lane i lands at row
  //      4*(q%16) + i/16, chunk position i%16, so it fetches that row's chunk (i%16) ^ f(row).
  const uint32_t kvrb = static_cast<uint32_t>(a.Hkv) * kRowBytes;   // bytes per token row
  const uint32_t vofs = static_cast<uint32_t>(a.T) * kvrb;          // V half of a block
  const int64_t blk_bytes = 2 * static_cast<int64_t>(vofs);
  const int tshift = a.tshift, tmask = a.T - 1;
  auto ld_row = [&](int j) __attribute__((always_inline)) { return 4 * ((wave * LPW + j) % 16) + lane / 16; };
  auto ld_isv = [&](int j) __attribute__((always_inline)) { return wave * LPW + j >= 16; };   // uniform
  auto ld_col = [&](int j) __attribute__((always_inline)) {                                   // byte column
    const int rr = ld_row(j);
    return static_cast<uint32_t>(((lane % 16) ^ (ld_isv(j) ? swz_v(rr) : swz_k(rr))) * 16);
  };
  auto ld_dst = [&](int j) __attribute__((always_inline)) {                                   // uniform
    const int qc = wave * LPW + j;
    return (qc >= 16 ? kTileBytes : 0) + (qc % 16) * 1024;
  };
  // full-tile byte offsets inside a block (BT) -- constant across tiles
  uint32_t off[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) off[j] = (ld_isv(j) ? vofs : 0u) + ld_row(j) * kvrb + ld_col(j);

  struct Ids {
    int32_t i0, i1, i2, i3;
  };
  // The block table is read-only here: reading it through the constant address space keeps
  // its uniform reads on the scalar unit although the tile loads write memory (LDS).
  auto table_of = [&](int r) __attribute__((always_inline)) {
    return (const __attribute__((address_space(4))) int32_t*)(a.table + static_cast<int64_t>(r) * a.mbps);
  };
  // block IDs of tile `tile` of item `it`: BT -> its one block; else its 64/T blocks
  // (clamped to the request's last block)
  auto fetch = [&](const Item& it, int tile, Ids& xi) __attribute__((always_inline)) {
    const auto table = table_of(it.r);
    const int last_blk = min((it.S - 1) >> tshift, a.mbps - 1);
    const int b0 = uni((tile * kTileK) >> tshift);
    xi.i0 = uni(table[min(b0, last_blk)]);
    if constexpr (!BT) {
      xi.i1 = uni(table[min(b0 + 1, last_blk)]);
      xi.i2 = uni(table[min(b0 + 2, last_blk)]);
      xi.i3 = uni(table[min(b0 + 3, last_blk)]);
    }
  };
  auto valid_id = [&](int32_t id) __attribute__((always_inline)) { return (id >= 0 && id < a.num_blocks) ? id : 0; };
  // Keys past S-1 (only in the tile that holds key S-1) are fetched from key S-1 instead:
  // never an unwritten slot, and their scores are masked anyway.
  auto issue = [&](const Item& it, int tile, int slot, const Ids& xi) __attribute__((always_inline)) {
    unsigned char* st = ring + slot * kStageBytes;
    const char* pool_g = static_cast<const char*>(a.pool) + static_cast<int64_t>(it.g) * kRowBytes;
    const int lim = it.S - 1 - tile * kTileK;                          // last tile row with a key
    if constexpr (BT) {
      const char* base = pool_g + static_cast<int64_t>(valid_id(xi.i0)) * blk_bytes +
                         static_cast<int64_t>((tile * kTileK) & tmask) * kvrb;
      if (lim >= kTileK - 1) {
#pragma unroll
        for (int j = 0; j < LPW; ++j) {
          const char* p = base + off[j];
          __builtin_amdgcn_global_load_lds(p, (lds_void*)(st + ld_dst(j)), 16, 0, 0);
        }
      } else {
#pragma unroll
        for (int j = 0; j < LPW; ++j) {
          const uint32_t o = (ld_isv(j) ? vofs : 0u) + min(ld_row(j), lim) * kvrb + ld_col(j);
          const char* p = base + o;
          __builtin_amdgcn_global_load_lds(p, (lds_void*)(st + ld_dst(j)), 16, 0, 0);
        }
      }
    } else {
      const int b0 = (tile * kTileK) >> tshift;
#pragma unroll
      for (int j = 0; j < LPW; ++j) {
        const int key = min(tile * kTileK + ld_row(j), it.S - 1);
        const int sb = (key >> tshift) - b0;                          // 0 .. 64/T - 1
        const int32_t id = valid_id(sb == 0 ? xi.i0 : sb == 1 ? xi.i1 : sb == 2 ? xi.i2 : xi.i3);
        const char* p = pool_g + static_cast<int64_t>(id) * blk_bytes + (ld_isv(j) ? vofs : 0u) +
                        static_cast<uint32_t>(key & tmask) * kvrb + ld_col(j);
        __builtin_amdgcn_global_load_lds(p, (lds_void*)(st + ld_dst(j)), 16, 0, 0);
      }
    }
  };

  // ---- LDS read addresses (bytes, relative to a stage), constant across tiles
  //  K: lane reads row kb*32 + l32, chunk lh*8 + ks -> position (lh*8 ^ f(l32)) ^ ks
  uint32_t kofs[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) kofs[ks] = l32 * kRowBytes + (((lh * 8) ^ swz_k(l32)) ^ ks) * 16;
  //  V^T: lane reads 8 bytes at row ks2*16 + hi*8 + lh*4 + (lane%16)/4, dims b*32 +
  //  ((lane/16)%2)*16 + 4*(lane%4): chunk b*4 + cl, stored at position ((b ^ xv) * 4) + cl
  uint32_t vrd[4];
  {
    const int xv = (lane % 16) / 4;                                     // row & 3, so f = xv << 2
    const int cl = ((lane / 16) % 2) * 2 + (lane % 4) / 2;
    const uint32_t lp = kTileBytes + (lh * 4 + xv) * kRowBytes + cl * 16 + (lane % 2) * 8;
#pragma unroll
    for (int b = 0; b < 4; ++b) vrd[b] = lp + ((b ^ xv) * 4) * 16;
  }

  // ---- Q^T (B operand) of an item: query q0 + l32 of this wave's head, dims lh*64 + ks*8 + j
  //      for ks = 0..7; rows past the chunk repeat its last row
  //      (asynchronous: see g_load16)
  auto load_q = [&](const Item& it, u32x4 (&dst)[8]) __attribute__((always_inline)) {
    const int hh = it.g * G + wave % G;
    const int qq0 = it.qtile * ROWS + (wave / G) * 32;
    const int64_t row = min<int64_t>(it.row0 + min(qq0 + l32, it.n - 1), a.N - 1);
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + row * a.q_stride + static_cast<int64_t>(hh) * kD + lh * 64;
    static_for<0, 8>([&](auto KSc) __attribute__((always_inline)) {
      constexpr int ks = decltype(KSc)::value;
      g_load16<ks * 16>(dst[ks], qp);
    });
  };

  // ---- the compute side's item: this wave's head, rows and causal limits
  Item C = item(0);
  int h, q0, past, wave_max_pos, my_pos;
  bool wave_active;
  auto enter = [&](const Item& it) __attribute__((always_inline)) {
    past = it.S - it.n;
    h = it.g * G + wave % G;
    q0 = it.qtile * ROWS + (wave / G) * 32;
    wave_active = q0 < it.n;
    wave_max_pos = past + min(q0 + 31, it.n - 1);
    my_pos = past + min(q0 + l32, it.n - 1);
  };
  // Q of the compute side's item, loaded in place (see g_load16): the first before the
  // ring's first tiles, so the first iteration's wait covers it; each later one in the last
  // tile of the item before, once that tile's QK products have read the old Q, and then the
  // next iteration waits for every load of this wave (the Q loads are its newest).
  u32x4 qf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) qf[ks] = u32x4{0u, 0u, 0u, 0u};
  load_q(C, qf);
  enter(C);
  Item Cn = C;                               // the compute side's next item
  if (J > 1) Cn = item(1);
  bool q_next = false;                       // this iteration loads the next item's Q
  bool q_wait = false;                       // this iteration waits for all loads

  float m_run = -INFINITY, l_run = 0.f;      // raw-score max of query l32; this lane's partial sum
  f32x16 o[4];                               // O^T[dim blk*32 + (i/4)*8 + lh*4 + i%4][query l32]
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[b][i] = 0.f;

  auto compute = [&](int t, int slot) __attribute__((always_inline)) {
    const int kb0 = t * kTileK;
    const bool act = wave_active && kb0 <= wave_max_pos;   // uniform
    const uint32_t sbase = ring_b + static_cast<uint32_t>(slot * kStageBytes);
    // ---- S^T = K Q^T: two 32-key blocks, their MFMA chains interleaved and the K operands
    //      read RA steps ahead
    f32x16 s[2];
    if (act) {
    uint32_t ka_[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) ka_[ks] = sbase + kofs[ks];
#pragma unroll
    for (int i = 0; i < 16; ++i) s[0][i] = s[1][i] = 0.f;
    constexpr int RA = 3;                    // steps of K operands in flight ahead of the MFMAs
    u32x4 kr[RA + 1][2];
    auto kread = [&](auto KSc) __attribute__((always_inline)) {
      constexpr int ks = decltype(KSc)::value;
      kr[ks % (RA + 1)][0] = k_read<0>(ka_[ks]);
      kr[ks % (RA + 1)][1] = k_read<32 * kRowBytes>(ka_[ks]);
    };
    static_for<0, RA>([&](auto KSc) __attribute__((always_inline)) { kread(KSc); });
    static_for<0, 8>([&](auto KSc) __attribute__((always_inline)) {
      constexpr int ks = decltype(KSc)::value;
      if constexpr (ks + RA < 8) kread(ic<ks + RA>());
      auto& xk = kr[ks % (RA + 1)];
      lgkm_wait<2 * (ks + RA < 8 ? RA : 7 - ks)>(xk[0], xk[1]);
      s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(xk[0]), as_bf16x8(qf[ks]), s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(xk[1]), as_bf16x8(qf[ks]), s[1], 0, 0, 0);
    });
    }
    // The last tile of an item: the next item's Q replaces this one's (one program point
    // for every wave, so the registers the loads write are the ones the products read).
    if (q_next) load_q(Cn, qf);
    if (!act) return;
    // ---- causal mask on tiles that cross this wave's diagonal (or the end of the keys)
    if (kb0 + kTileK - 1 > past + q0) {
      const int lim = my_pos - kb0 - lh * 4;                 // key offset kb*32+(i/4)*8+i%4 <= lim
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = (kb * 32 + (i / 4) * 8 + (i % 4) <= lim) ? s[kb][i] : -INFINITY;
    }
    // ---- online softmax (raw-score domain; exp2 of (s - m) * c)
    // row max: four independent chains over the lane's 32 scores, then across the lane
    // halves (lanes l and l^32 hold the same query) with a VALU lane swap
    float m4[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      m4[k] = s[k / 2][(k % 2) * 8];
#pragma unroll
      for (int j = 1; j < 8; ++j) m4[k] = fmaxf(m4[k], s[k / 2][(k % 2) * 8 + j]);
    }
    const float tmax = xor_max<32>(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
    // Lazy rescaling: the running maximum used as the exponent offset only moves when a
    // score exceeds it by more than 2^8 in exp2 units, so P stays <= 256 (exact enough in
    // fp32 sums and bf16 products) and most tiles skip the rescale of O.  The first tile
    // of an item always sets it (m_run starts at -inf).
    if (__any((tmax - m_run) * c > kLazyLog2)) {
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[b][i] *= alpha;
      m_run = m_new;
    }
    const float mc = m_run * c;
    // P^T as four B operands (16 keys each): slot j of step ks2 is s[ks2/2][(ks2%2)*8 + j]
    bf16x8 pb[4];
    float l4[4];                             // partial row sums, one per B operand
#pragma unroll
    for (int ks2 = 0; ks2 < 4; ++ks2) {
      const int kb = ks2 / 2, i0 = (ks2 % 2) * 8;
      float p[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) p[j] = __builtin_amdgcn_exp2f(fmaf(s[kb][i0 + j], c, -mc));
      const uint32_t w0 = pack_bf16(p[0], p[1]), w1 = pack_bf16(p[2], p[3]), w2 = pack_bf16(p[4], p[5]),
                     w3 = pack_bf16(p[6], p[7]);
      // Row sums in plain fp32 adds of the unrounded P (the normaliser then differs from
      // the sum of the bf16-rounded P by at most 2^-9 relative).  v_dot2c_f32_bf16 would sum
      // the rounded values, but on gfx950 it waits for the matrix core, so the other wave's
      // MFMAs in flight stall it; adds issue beside them.
      l4[ks2] = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      pb[ks2] = as_bf16x8(u32x4{w0, w1, w2, w3});
    }
    l_run += (l4[0] + l4[1]) + (l4[2] + l4[3]);
    // ---- O^T += V^T P^T: 16 MFMAs (step ks2 = R/4 of 16 keys, dim block b = R%4), the
    //      V^T operands of each read RV MFMAs ahead
    uint32_t va_[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) va_[b] = sbase + vrd[b];
    constexpr int RV = 4;
    s16x4 vr[RV + 1][2];
    auto vread = [&](auto Rc) __attribute__((always_inline)) {
      constexpr int R = decltype(Rc)::value;
      constexpr int base = (R / 4) * 16 * kRowBytes;
      vr[R % (RV + 1)][0] = tr_read<base>(va_[R % 4]);
      vr[R % (RV + 1)][1] = tr_read<base + 8 * kRowBytes>(va_[R % 4]);
    };
    static_for<0, RV>([&](auto Rc) __attribute__((always_inline)) { vread(Rc); });
    static_for<0, 16>([&](auto Rc) __attribute__((always_inline)) {
      constexpr int R = decltype(Rc)::value;
      if constexpr (R + RV < 16) vread(ic<R + RV>());
      auto& d = vr[R % (RV + 1)];
      lgkm_wait2<2 * (R + RV < 16 ? RV : 15 - R)>(d[0], d[1]);
      const u32x4 u = {__builtin_bit_cast(uint2, d[0]).x, __builtin_bit_cast(uint2, d[0]).y,
                       __builtin_bit_cast(uint2, d[1]).x, __builtin_bit_cast(uint2, d[1]).y};
      o[R % 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(u), pb[R / 4], o[R % 4], 0, 0, 0);
    });
  };

  // ---- normalise and store the compute side's item: lane owns query l32 and dims
  //      blk*32 + (i/4)*8 + lh*4 + i%4
  //      (st_*: the finished item's rows, kept until the next iteration stores them)
  int st_n = 0, st_row0 = 0, st_h = 0, st_q0 = 0;
  bool st_active = false;
  auto store = [&]() __attribute__((always_inline)) {
    if (!st_active) return;
    const float inv = 1.f / xor_sum<32>(l_run);
    const int qi = st_q0 + l32;
    const int64_t row = st_row0 + static_cast<int64_t>(qi);
    if (qi >= st_n || row >= a.N) return;
    const int64_t oe = row * static_cast<int64_t>(a.H) * kD + static_cast<int64_t>(st_h) * kD;
    if (a.out_fmt == F_FP8) {                                  // four e4m3 codes per store
      uint8_t* op = static_cast<uint8_t*>(a.out) + oe;
      const float m = a.out_mul;
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d = b * 32 + i4 * 8 + lh * 4;
          uint32_t wd = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) wd |= f32_to_e4m3((o[b][i4 * 4 + e] * inv) * m) << (8 * e);
          *reinterpret_cast<uint32_t*>(op + d) = wd;
        }
    } else {
      uint16_t* op = static_cast<uint16_t*>(a.out) + oe;
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
  };

  // ---- the ring: this workgroup's items form one stream of tiles, and stream tile t lives
  //      in stage t % NS.  Iteration t waits for this wave's loads of tile t (the NS-2 later
  //      tiles may stay in flight), meets the other waves at the barrier -- after which tile
  //      t is complete in LDS and stage (t-1) % NS is no longer read -- refills that stage
  //      with stream tile t+NS-1 and computes tile t.  The loads run NS-1 tiles ahead across
  //      item boundaries; past the stream's last tile they repeat it, so every iteration
  //      has the same loads in flight.
  Item L = C;                                // the loader's item and tile
  int jl = 0, ul = 0;
  auto advance = [&]() __attribute__((always_inline)) {
    if (ul + 1 < L.ntiles) {
      ++ul;
    } else if (jl + 1 < J) {
      ++jl;
      ul = 0;
      L = item(jl);
    }
  };
  Ids nx;
  {
    // the first NS-1 tiles: all block-ID fetches first (one wait for their latency), then
    // the loads
    Item lp[NS - 1];
    int up[NS - 1];
    Ids xp[NS - 1];
#pragma unroll
    for (int u = 0; u < NS - 1; ++u) {
      lp[u] = L;
      up[u] = ul;
      fetch(L, ul, xp[u]);
      advance();
    }
#pragma unroll
    for (int u = 0; u < NS - 1; ++u) issue(lp[u], up[u], u, xp[u]);
  }
  fetch(L, ul, nx);
  int slot = 0, fill = NS - 1, tc = 0, jc = 0;
  bool st_pending = false;
  for (;;) {
    if (q_wait) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * LPW));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (st_pending) {                        // the previous item's output, then a fresh state
      store();
      st_pending = false;
      m_run = -INFINITY;
      l_run = 0.f;
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[b][i] = 0.f;
    }
    q_wait = false;
    issue(L, ul, fill, nx);
    advance();
    fetch(L, ul, nx);
    q_next = tc + 1 == C.ntiles && jc + 1 < J;
    compute(tc, slot);
    slot = slot == NS - 1 ? 0 : slot + 1;
    fill = fill == NS - 1 ? 0 : fill + 1;
    if (++tc == C.ntiles) {                  // item done: its output is stored next iteration
      st_n = C.n;
      st_row0 = C.row0;
      st_h = h;
      st_q0 = q0;
      st_active = wave_active;
      if (++jc == J) break;
      st_pending = true;
      q_wait = true;
      C = Cn;
      enter(C);
      tc = 0;
      if (jc + 1 < J) Cn = item(jc + 1);
    }
  }
  store();
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // no load may still target this workgroup's LDS at exit
}


// The persistent schedule's host half for one launch of at most kPrefillMaxReqs context
// requests [a.req_begin, a.req_end): work order (most tiles first), XCD groups, and W
// workgroups per group for a grid of at most `wgs` workgroups.  Returns the grid size.
inline int64_t prefill_sched(const AttnArgs& a, const int32_t* host_n, const int32_t* host_S, int rows, int wgs,
                             PrefillSched& sc) {
  const int groups = a.Hkv % kXcds == 0 ? kXcds : 1;
  sc = PrefillSched{};
  sc.nreq = a.req_end - a.req_begin;
  sc.groups = groups;
  sc.hpg = a.Hkv / groups;
  // requests with the most 64-key tiles first (a close bound: ntq query tiles over
  // past + rows/2 * (ntq + 1) keys on average)
  int order[kPrefillMaxReqs];
  int64_t cost[kPrefillMaxReqs];
  int64_t tiles = 0;                                 // query tiles of all requests
  for (int i = 0; i < sc.nreq; ++i) {
    order[i] = i;
    const int64_t n = host_n[a.req_begin + i], past = host_S[a.req_begin + i] - n, ntq = (n + rows - 1) / rows;
    cost[i] = ntq * (2 * past + rows * (ntq + 1));
    tiles += ntq;
  }
  std::stable_sort(order, order + sc.nreq, [&](int i, int j) { return cost[i] > cost[j]; });
  for (int p = 0; p < sc.nreq; ++p) sc.rank[order[p]] = static_cast<uint16_t>(p);
  const int64_t per_group = tiles * sc.hpg;
  const int64_t W = std::max<int64_t>(1, std::min<int64_t>(per_group, std::max(1, wgs / groups)));
  return W * groups;
}

}  // namespace pf
}  // namespace
}  // namespace pkv
