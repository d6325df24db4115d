// Device code of the generation-phase split pass (see decode.hip for the design),
// shared by the split kernel and the mixed-batch kernel.
#pragma once
#include <math.h>

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace pkv {
namespace {
namespace dc {


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kTile = 32;          // keys per wave iteration
// The split pass handles head_dim DH = 64 or 128 (a template parameter): a staged V row
// is padded by 8 elements, and a K row holds DH / 8 16-byte chunks.
template <int DH>
constexpr int v_stride() { return DH + 8; }        // LDS row stride (bf16 elements) of a staged V tile
constexpr int kXcds = 8;           // XCDs of the chip, each with its own L2
constexpr int kPieceBatch = 32;    // pieces listed at a time by the split pass
constexpr int kCombHeads = 4;      // query heads (one wave each) per combine workgroup

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// 16 bytes of the cache.  Where every K/V byte is read once per step (one column block, or
// several sharing one staged tile) and every load instruction covers whole rows (whole
// 128-byte lines), the loads carry the nontemporal hint (NT): lines are not kept for reuse
// that will not come.
template <bool NT>
__device__ __forceinline__ uint4 load_kv(const void* p) {
  if constexpr (NT) {
    const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  } else {
    return *static_cast<const uint4*>(p);
  }
}
// K tile in LDS: 16-byte chunk c of key row r sits at chunk position c ^ (r & (DH/8 - 1)),
// so the rows one MFMA operand read touches at one chunk fall on distinct bank groups.
template <int DH>
__device__ __forceinline__ int kpos(int r, int c) { return c ^ (r & (DH / 8 - 1)); }

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
// Workgroup barrier for LDS data: this wave's LDS writes complete (lgkmcnt(0)), then
// s_barrier; global loads in flight stay in flight (no vmcnt wait).  The empty asm
// statements keep the compiler from moving LDS accesses across it.
constexpr int kLgkm0 = 15 | (7 << 4) | (0 << 8) | (3 << 14);   // vmcnt and expcnt unconstrained
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kLgkm0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Registers of one 32-key tile in flight: K and V rows as loaded (DH / 8 lanes per bf16
// row, DH / 16 per fp8 / int8 row), copied to LDS at compute time.
template <int KV, int DH>
struct TileRegs {
  uint4 k[kTile * DH * (KV == F_BF16 ? 2 : 1) / 1024];
  uint4 v[kTile * DH * (KV == F_BF16 ? 2 : 1) / 1024];
};

__device__ __forceinline__ int64_t min64(int64_t x, int64_t y) { return x < y ? x : y; }
__device__ __forceinline__ int64_t max64(int64_t x, int64_t y) { return x > y ? x : y; }
// End key of tiles [.., t_end) of a request with S keys: min(t_end * 32, S), without
// forming t_end * 32 when it is past S.
__device__ __forceinline__ int tiles_end(int t_end, int S) { return t_end > (S - 1) / kTile ? S : t_end * kTile; }

// Generation request r as the split pass sees it (device lengths, kept to n >= 1 and
// S >= n whatever they hold): n new tokens, S keys, `tiles` 32-key tiles, and `cbs` blocks
// of 16 (token, query head) columns per KV head.  Its work units are its 32-key tiles.
struct ReqGeom {
  int n, S, tiles, cbs;
};
__device__ __forceinline__ ReqGeom req_geom(const AttnArgs& a, int r, int G) {
  ReqGeom q;
  q.n = max(a.ctx_len[r], 1);
  q.S = max(a.seq_len[r], q.n);
  q.tiles = (q.S - 1) / kTile + 1;
  q.cbs = static_cast<int>(min64((static_cast<int64_t>(G) * q.n + 15) / 16, a.col_blocks));
  return q;
}

// Exclusive prefix sum of v over the workgroup's kThreads threads; *total gets the sum.
__device__ __forceinline__ int64_t block_exclusive_scan(int64_t v, int64_t* total, int64_t* part) {
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  int64_t x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int64_t y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) part[w] = x;
  __syncthreads();
  int64_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    before += i < w ? part[i] : 0;
    tot += part[i];
  }
  *total = tot;
  return before + x - v;
}


// Pieces of a workgroup's range, as listed in LDS: (request, head group, column block,
// first tile) and (tiles, n, S, packed row of the request's first token).
struct Piece {
  int r, hg, cb, t0, nt, n, S, row0;
};
__device__ __forceinline__ Piece read_piece(const int4* pa, const int4* pb, int p) {
  const int4 x = pa[p], y = pb[p];
  Piece q;
  q.r = __builtin_amdgcn_readfirstlane(x.x);
  q.hg = __builtin_amdgcn_readfirstlane(x.y);
  q.cb = __builtin_amdgcn_readfirstlane(x.z);
  q.t0 = __builtin_amdgcn_readfirstlane(x.w);
  q.nt = __builtin_amdgcn_readfirstlane(y.x);
  q.n = __builtin_amdgcn_readfirstlane(y.y);
  q.S = __builtin_amdgcn_readfirstlane(y.z);
  q.row0 = __builtin_amdgcn_readfirstlane(y.w);
  return q;
}

// The np listed pieces as one tile stream per wave.  B: KV heads per segment (1, or
// kWaves: one per wave).  With B = kWaves a wave's items are all tiles of every piece for
// its head; with B = 1 the waves share a piece's tiles (wave w takes tiles w, w + 4, ...),
// every wave having ceil(tiles / 4) items per piece (items past the piece's tiles load its
// last tile again and compute nothing), so that all waves reach a piece's end, where their
// states are merged in LDS, at the same item.  Loads run two items ahead of the compute
// across piece boundaries: a new piece starts with its first tiles already in flight, and
// only the softmax state and Q are reset.  Each piece leaves one partial state in its slot.
// NT: stream the cache with the nontemporal hint (every byte read once) or keep its lines
// in L2 (segments of one column block each read the same keys).  TREE: draft tokens
// verified as a tree; a column sees the cached keys and the new keys its mask row names.
template <int KV, int HPS, int CBW, bool NT, bool TREE, int DH>
__device__ __forceinline__ void decode_stream(const AttnArgs& a, const int np, const int k, const int plane, const int4* pla,
                                              const int4* plb, uint16_t (*vtile)[kTile * v_stride<DH>()],
                                              uint16_t (*ktile)[kTile * DH], float (*ml)[16][2]) {
  constexpr int kD = DH;
  constexpr int kVStride = v_stride<DH>();
  constexpr int kKS = DH / 32;                                 // contraction steps of S^T = K Q^T
  constexpr int kNB = DH / 16;                                 // 16-dim blocks of O
  // ALT: one KV head per segment, its waves sharing the tiles; otherwise every wave streams
  // all tiles for its own (KV head, column block): HPS heads x CBW column blocks.
  constexpr bool ALT = HPS == 1 && CBW == 1;
  static_assert(ALT || HPS * CBW == kWaves, "a workgroup's waves cover its heads and column blocks");
  // The thread index passes through an empty asm statement so that nothing derived from
  // it is hoisted out of the batch loop and kept live across it (registers are tight).
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform
  const int lane = tid % kWave;
  const int li = lane % 16, lg = lane / 16;
  const int G = a.H / a.Hkv;
  constexpr int TS = ALT ? kWaves : 1;                         // tile stride of a wave's items
  const int base = ALT ? wave : 0;                              // first tile of a wave's items
  const int wh = ALT ? 0 : wave / CBW;                          // the wave's head in the segment
  const int wcb = CBW > 1 ? wave % CBW : 0;                     // the wave's column block (CBW > 1)
  const int64_t kv_row = static_cast<int64_t>(a.Hkv) * kD;     // elements per (block, K|V, slot)
  const int tshift = a.tshift, tmask = a.T - 1;
  const int64_t blk_bytes = 2 * static_cast<int64_t>(a.T) * kv_row * (KV == F_BF16 ? 2 : 1);   // K and V of T slots
  uint16_t* vt = vtile[wave];
  uint16_t* kt = ktile[wave];
  // Load `it` of a tile covers rows it*kRows + lane/kLanes at byte column (lane%kLanes)*16
  // (16 lanes per 256-byte bf16 row, 8 per 128-byte fp8 / int8 row).
  constexpr int kEB = KV == F_BF16 ? 2 : 1;                    // cache element bytes
  constexpr int kLoads = kTile * kD * kEB / 1024;              // 1 KB load instructions per K (or V) tile
  constexpr int kRows = kWave * 16 / (kD * kEB);               // rows per load instruction
  constexpr int kLanes = kWave / kRows;                        // lanes per row
  const uint32_t row_bytes = static_cast<uint32_t>(kv_row) * kEB;
  // byte offset of the lane inside load 0 of a tile; load `it` adds it*kRows rows to the
  // (scalar) base, so one register serves every load
  const uint32_t lane_off = static_cast<uint32_t>(lane / kLanes) * row_bytes + (lane % kLanes) * 16u;
  const float xscale = a.scale_log2 * a.k_scale;
  // SHARE (several column blocks per head): the CBW waves of one head split each tile's
  // loads (with two waves one loads the K rows and the other the V rows; with four, each
  // loads 16 rows of K or of V), stage them in one LDS tile of the head and meet at a
  // workgroup barrier before the math, so every cache byte leaves HBM once.  Two LDS tiles per head alternate between items: a wave
  // writes tile s of item i + 2 only after the barrier of item i + 1, which every wave
  // passes after its reads of item i are complete.
  constexpr bool SHARE = CBW > 1;
  constexpr int kPart = SHARE ? 2 * kLoads / CBW : 1;          // loads of a wave's share
  const int s_kind = SHARE ? wcb / (CBW / 2 > 0 ? CBW / 2 : 1) : 0;   // 0: K rows, 1: V rows
  const int s_it0 = SHARE ? (wcb % (CBW / 2 > 0 ? CBW / 2 : 1)) * kPart : 0;   // first load
  struct Share {
    uint4 r[kPart];
  };
  using Regs = typename std::conditional<SHARE, Share, TileRegs<KV, DH>>::type;
  int stg = 0;                                                  // LDS tile of the next item

  // ---- fetch cursor (wave-uniform): item f_k of piece f_p, with the piece's facts kept in
  // scalars (the LDS list is read only when the cursor moves to another piece)
  int f_p = 0, f_k = 0, f_cnt, f_t0, f_nt, f_r, f_hg, f_last;
  auto fetch_piece = [&](int p) {
    const Piece q = read_piece(pla, plb, p);
    f_cnt = (q.nt + TS - 1) / TS;
    f_t0 = q.t0;
    f_nt = q.nt;
    f_r = q.r;
    f_hg = q.hg;
    f_last = min((tiles_end(q.t0 + q.nt, q.S) - 1) >> tshift, a.mbps - 1);
  };
  // A ticket carries one item to its loads: the block IDs of its tile, its first key and
  // the wave's KV head.  Tiles are 32-aligned and T is a power of two >= 16, so a tile lies
  // in one block (T >= 32) or covers two (T = 16).  The block table is read-only here:
  // reading it through the constant address space keeps its (wave-uniform) reads on the
  // scalar unit, out of the vector-load queue.  Past the stream's last item the cursor
  // stays on it (its loads repeat).
  struct Ticket {
    int32_t id0, id1;
    int tb, g;
  };
  auto fetch = [&](Ticket& t) {
    const int tile = f_t0 + min(base + f_k * TS, f_nt - 1);
    const int kb0 = (tile * kTile) >> tshift;
    const __attribute__((address_space(4))) int32_t* table =
        (const __attribute__((address_space(4))) int32_t*)(a.table + static_cast<int64_t>(f_r) * a.mbps);
    t.id0 = table[min(kb0, f_last)];
    t.id1 = table[min(kb0 + 1, f_last)];
    t.tb = tile * kTile;
    t.g = f_hg * HPS + wh;
    if (f_k + 1 < f_cnt) {
      ++f_k;
    } else if (f_p + 1 < np) {
      ++f_p;
      f_k = 0;
      fetch_piece(f_p);
    }
  };
  // Issue every load of a ticket's tile into `R`.  Loads it < kLoads/2 cover tile rows
  // 0..15, the others rows 16..31, so every load has one scalar base: B0 (the tile's block
  // at the tile's first slot) or B1 (the block of rows 16..31; the same block unless
  // T = 16).  Rows past the piece end are still slots of an allocated block (in bounds);
  // their scores are masked and their V rows zeroed in compute.
  auto issue = [&](const Ticket& t, Regs& R) {
    int32_t id0 = __builtin_amdgcn_readfirstlane(t.id0);
    int32_t id1 = __builtin_amdgcn_readfirstlane(t.id1);
    id0 = (id0 >= 0 && id0 < a.num_blocks) ? id0 : 0;
    id1 = (id1 >= 0 && id1 < a.num_blocks) ? id1 : 0;
    const char* head = static_cast<const char*>(a.pool) + t.g * (kD * kEB);
    const char* b0 = head + static_cast<int64_t>(id0) * blk_bytes + static_cast<int64_t>(t.tb & tmask) * row_bytes;
    const char* b1 = a.T >= kTile ? b0 : head + static_cast<int64_t>(id1) * blk_bytes - 16 * static_cast<int64_t>(row_bytes);
    const int64_t vofs = static_cast<int64_t>(a.T) * row_bytes;
    if constexpr (SHARE) {
      const char* bk = s_kind ? b0 + vofs : b0;
      const char* bh = s_kind ? b1 + vofs : b1;
#pragma unroll
      for (int j = 0; j < kPart; ++j) {
        const int it = s_it0 + j;
        R.r[j] = load_kv<NT>((it < kLoads / 2 ? bk : bh) + static_cast<int64_t>(it * kRows) * row_bytes + lane_off);
      }
    } else {
#pragma unroll
      for (int it = 0; it < kLoads; ++it)
        R.k[it] = load_kv<NT>((it < kLoads / 2 ? b0 : b1) + static_cast<int64_t>(it * kRows) * row_bytes + lane_off);
#pragma unroll
      for (int it = 0; it < kLoads; ++it)
        R.v[it] = load_kv<NT>((it < kLoads / 2 ? b0 : b1) + vofs + static_cast<int64_t>(it * kRows) * row_bytes + lane_off);
    }
  };

  // ---- state of the piece being computed
  bf16x8 qf[kKS];
  float m_run, l_run;                                           // for column li
  f32x4 o[kNB];                                                 // O[column lg*4+i][dim nb*16+li]
  int key_lim;                                                  // keys 0 .. key_lim for column li
  uint32_t vm_lo = 0, vm_hi = 0;                                // TREE: column li's mask over the new keys
  int c_base = 0;                                               // TREE: first new key of the request
  int c_t0, c_nt, c_cnt, c_kend, c_lim, c_ncol, c_valid, c_g, c_cb;
  int64_t c_slot;
  auto start_piece = [&](int p) {
    const Piece q = read_piece(pla, plb, p);
    const int n = q.n, S = q.S;
    c_t0 = q.t0;
    c_nt = q.nt;
    c_cnt = (q.nt + TS - 1) / TS;
    c_cb = CBW > 1 ? wcb : q.cb;
    c_g = q.hg * HPS + wh;                                      // this wave's KV head
    c_kend = tiles_end(q.t0 + q.nt, S);
    // A tile needs no masking when it lies inside the piece and inside the causal range
    // of every valid column of the block (the lowest of them is token cb*16 / G; with a
    // tree, every column sees the cached keys only for sure).
    c_lim = TREE ? S - n - 1 : S - n + (c_cb * 16) / G;
    c_base = S - n;
    c_ncol = min(16, G * n - c_cb * 16);                        // valid columns of the block
    if (CBW == 1) c_ncol = min(c_ncol, a.dec_cols);
    c_slot = static_cast<int64_t>(q.r - a.req_begin + k) * a.dec_lanes + plane;
    // Columns of the score tile: (token, query head) pairs, 16 per column block.  Lane
    // column li is token tok = gc / G of the request (position S - n + tok; it sees keys
    // up to that position: causal among a request's draft tokens) and head g*G + gc % G.
    const int gc = c_cb * 16 + li, tok = gc / G;
    const bool col_ok = tok < n;
    key_lim = col_ok ? (TREE ? S - 1 : S - n + tok) : -1;
    const int64_t row0 = q.row0;
    // rows outside the generation rows, or a column block the request does not have: no output
    c_valid = row0 >= a.row_begin && row0 + n <= a.N && c_ncol > 0;
    const int64_t row = c_valid ? row0 + min(tok, n - 1) : a.row_begin;
    if constexpr (TREE) {
      const uint2 mw = col_ok && c_valid ? *reinterpret_cast<const uint2*>(a.spec_mask + row * 2) : make_uint2(0, 0);
      vm_lo = mw.x;
      vm_hi = mw.y;
    }
    // B operand Q^T: column li, dims ks*32 + lg*8 + j (the dim order inside a
    // contraction is free as long as K uses the same one).
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + row * a.q_stride +
                         static_cast<int64_t>(c_g * G + gc % G) * kD + lg * 8;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      uint4 u = *reinterpret_cast<const uint4*>(qp + ks * 32);
      if (!col_ok) u = make_uint4(0, 0, 0, 0);
      qf[ks] = as_bf16x8(u);
    }
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  // Write the piece's partial state (m, l, o) to its slot.
  auto end_piece = [&]() {
    const int ncol = c_ncol;
    if constexpr (!ALT) {
      // this wave alone holds its (head, column block) state for the piece
      if (c_valid) {
        const int64_t e0 = (c_slot * HPS + wh) * a.dec_cols + (CBW > 1 ? c_cb * 16 : 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = lg * 4 + i;
          if (c < ncol) {
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb) a.ws_o[(e0 + c) * kD + nb * 16 + li] = o[nb][i];
          }
        }
        if (lg == 0 && li < ncol) {
          a.ws_ml[(e0 + li) * 2] = m_run;
          a.ws_ml[(e0 + li) * 2 + 1] = l_run;
        }
      }
    } else {
      // merge the 4 waves' states in LDS, then write the piece's (m, l, o)
      __syncthreads();
      float* red = reinterpret_cast<float*>(&vtile[0][0]);      // [wave][16 columns][kD]
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[(wave * 16 + lg * 4 + i) * kD + nb * 16 + li] = o[nb][i];
      if (lg == 0) {
        ml[wave][li][0] = m_run;
        ml[wave][li][1] = l_run;
      }
      __syncthreads();
      if (c_valid) {
        const int64_t e0 = c_slot * a.dec_cols;
        for (int e = tid; e < ncol * kD; e += kThreads) {
          const int c = e / kD, d = e % kD;
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
          a.ws_o[(e0 + c) * kD + d] = O;
          if (d == 0) {
            a.ws_ml[(e0 + c) * 2] = M;
            a.ws_ml[(e0 + c) * 2 + 1] = L;
          }
        }
      }
      __syncthreads();                                          // LDS free for the next tiles
    }
  };
  // The tile's math from LDS tiles kt (K) and vt (V): scores, online softmax, O += P V.
  auto tile_math = [&](const uint16_t* kt, const uint16_t* vt, const int tb, const int kend, const int lim_all) {
    // A operand K: lane (li, lg) of step ks holds key kb*16 + li, dims ks*32 + lg*8 .. +7
    bf16x8 kf[2][kKS];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        const int row = kb * 16 + li;
        kf[kb][ks] = as_bf16x8(*reinterpret_cast<const uint4*>(kt + row * kD + kpos<DH>(row, ks * 4 + lg) * 8));
      }
    // scores S^T[key][head]: lane holds head li, keys tb + kb*16 + lg*4 + i
    f32x4 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks)
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
          bool vis = key < kend && key <= key_lim;
          if constexpr (TREE) {
            // new key j = key - c_base (0 <= j < n <= 64) is seen when bit j of the mask is set
            const int j = key - c_base;
            vis = vis && (j < 0 || (((j < 32 ? vm_lo : vm_hi) >> (j & 31)) & 1u));
          }
          x[kb * 4 + i] = vis ? sacc[kb][i] * xscale : -INFINITY;
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
        for (int nb = 0; nb < kNB; ++nb) o[nb][i] *= ah;
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
    for (int nb = 0; nb < kNB; ++nb) {
      const uint16_t* src = vt + krow * kVStride + nb * 16 + 4 * (li % 4);
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(src));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(src + 16 * kVStride));
      const uint4 u = make_uint4(__builtin_bit_cast(uint2, lo).x, __builtin_bit_cast(uint2, lo).y,
                                 __builtin_bit_cast(uint2, hi).x, __builtin_bit_cast(uint2, hi).y);
      o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, as_bf16x8(u), o[nb], 0, 0, 0);
    }
  };

  // This wave's share of a tile into the head's LDS tile (SHARE); V rows at or past the
  // piece end are written as zeros (P = 0 times them stays 0).
  auto stage_share = [&](uint16_t* kt, uint16_t* vt, const int tb, const int kend, const Regs& R) {
    if constexpr (SHARE) {
      // the row and byte column of load `it` as in `issue`
      auto row_of = [&](int it) { return it * kRows + lane / kLanes; };
      if (s_kind == 0) {                                        // K rows (wave-uniform)
#pragma unroll
        for (int j = 0; j < kPart; ++j) {
          const int row = row_of(s_it0 + j);
          if constexpr (KV == F_BF16) {
            *reinterpret_cast<uint4*>(kt + row * kD + kpos<DH>(row, lane % kLanes) * 8) = R.r[j];
          } else {
            const int c0 = (lane % kLanes) * 2;
            *reinterpret_cast<uint4*>(kt + row * kD + kpos<DH>(row, c0) * 8) = codes8_to_bf16x8<KV>(make_uint2(R.r[j].x, R.r[j].y));
            *reinterpret_cast<uint4*>(kt + row * kD + kpos<DH>(row, c0 + 1) * 8) = codes8_to_bf16x8<KV>(make_uint2(R.r[j].z, R.r[j].w));
          }
        }
      } else {                                                  // V rows
        const int lim = tb + kTile > kend ? kend - tb : kTile;  // rows from lim on are zeroed
#pragma unroll
        for (int j = 0; j < kPart; ++j) {
          const int row = row_of(s_it0 + j);
          const bool keep = row < lim;
          if constexpr (KV == F_BF16) {
            const uint4 u = R.r[j];
            *reinterpret_cast<uint4*>(vt + row * kVStride + (lane % kLanes) * 8) =
                make_uint4(keep ? u.x : 0u, keep ? u.y : 0u, keep ? u.z : 0u, keep ? u.w : 0u);
          } else {
            const uint4 lo = codes8_to_bf16x8<KV>(make_uint2(R.r[j].x, R.r[j].y));
            const uint4 hi = codes8_to_bf16x8<KV>(make_uint2(R.r[j].z, R.r[j].w));
            uint16_t* d = vt + row * kVStride + (lane % kLanes) * 16;
            *reinterpret_cast<uint4*>(d) = make_uint4(keep ? lo.x : 0u, keep ? lo.y : 0u, keep ? lo.z : 0u, keep ? lo.w : 0u);
            *reinterpret_cast<uint4*>(d + 8) = make_uint4(keep ? hi.x : 0u, keep ? hi.y : 0u, keep ? hi.z : 0u, keep ? hi.w : 0u);
          }
        }
      }
    }
  };
  // K and V rows of a whole tile into this wave's LDS tiles (bf16; an fp8 / int8 cache is
  // dequantised here), then the tile's math.
  auto compute = [&](const int tb, const int kend, const int lim_all, const TileRegs<KV, DH>& R) {
    wave_lds_fence();
    if constexpr (KV == F_BF16) {
#pragma unroll
      for (int it = 0; it < kLoads; ++it) {
        const int row = it * kRows + lane / kLanes, ch = lane % kLanes;
        *reinterpret_cast<uint4*>(kt + row * kD + kpos<DH>(row, ch) * 8) = R.k[it];
        *reinterpret_cast<uint4*>(vt + row * kVStride + ch * 8) = R.v[it];
      }
    } else {
#pragma unroll
      for (int it = 0; it < kLoads; ++it) {
        const int row = it * kRows + lane / kLanes, c0 = (lane % kLanes) * 2;
        *reinterpret_cast<uint4*>(kt + row * kD + kpos<DH>(row, c0) * 8) =
            codes8_to_bf16x8<KV>(make_uint2(R.k[it].x, R.k[it].y));
        *reinterpret_cast<uint4*>(kt + row * kD + kpos<DH>(row, c0 + 1) * 8) =
            codes8_to_bf16x8<KV>(make_uint2(R.k[it].z, R.k[it].w));
        uint16_t* d = vt + row * kVStride + (lane % kLanes) * 16;
        *reinterpret_cast<uint4*>(d) = codes8_to_bf16x8<KV>(make_uint2(R.v[it].x, R.v[it].y));
        *reinterpret_cast<uint4*>(d + 8) = codes8_to_bf16x8<KV>(make_uint2(R.v[it].z, R.v[it].w));
      }
    }
    if (tb + kTile > kend) {
      // wave-uniform, last tile of a piece only: rows at or past the piece end were read
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
    tile_math(kt, vt, tb, kend, lim_all);
  };
  // Compute item k of the current piece from R (nothing for an item past its tiles).  With
  // SHARE every wave stages its share and meets the others at the barrier, whether or not
  // the piece has its column block.
  auto compute_item = [&](int k, const Regs& R) {
    const int tile = base + k * TS;
    if constexpr (SHARE) {
      uint16_t* skt = ktile[wh * 2 + stg];
      uint16_t* svt = vtile[wh * 2 + stg];
      stg ^= 1;
      const int tb = (c_t0 + tile) * kTile;
      stage_share(skt, svt, tb, c_kend, R);
      lds_barrier();
      if (tile < c_nt && c_valid) tile_math(skt, svt, tb, c_kend, c_lim);
    } else {
      if (tile < c_nt && c_valid) compute((c_t0 + tile) * kTile, c_kend, c_lim, R);
    }
  };

  // Software pipeline over the stream: the next item's loads are in flight while an item
  // is computed and its block IDs are read one item further ahead; every path has the same
  // loads in flight, so the compiler's wait before an item's compute covers that item only.
  Regs ra, rb;
  Ticket ta, tb;
  fetch_piece(0);
  fetch(ta);
  issue(ta, ra);                                                // item 0
  fetch(tb);                                                    // item 1
  int cp = 0, ck = 0;                                           // item in compute
  start_piece(0);
  while (true) {
    issue(tb, rb);
    fetch(ta);
    compute_item(ck, ra);
    if (ck + 1 == c_cnt) {
      end_piece();
      if (cp + 1 >= np) break;
      ++cp;
      ck = 0;
      start_piece(cp);
    } else {
      ++ck;
    }
    issue(ta, ra);
    fetch(tb);
    compute_item(ck, rb);
    if (ck + 1 == c_cnt) {
      end_piece();
      if (cp + 1 >= np) break;
      ++cp;
      ck = 0;
      start_piece(cp);
    } else {
      ++ck;
    }
  }
}

// ---- range bookkeeping of the split pass
//
// The batch's work is its generation requests' 32-key tiles, in request order (U units).
// NL lanes (a.dec_lanes) run in lockstep: a lane is a head group (times a column block
// where one head's segment holds a single block), and each of the Wr = W / NL
// ranges of about U / Wr consecutive units goes to NL workgroups, one per lane, which
// stream the same tiles for their lanes' heads at about the same time: the neighbouring
// head groups' pieces of a request's cache rows then leave HBM together.  Launched
// workgroup w runs on XCD w % 8 (round-robin dispatch); it takes logical index
// lw = (w % 8) * (W / 8) + w / 8, range lw / NL and lane lw % NL, so the lanes of a range
// share an XCD and each XCD works through one contiguous eighth.  A range cuts the
// requests it touches into pieces; the piece of request r (r-th generation request) and
// range k on lane l leaves its partial state in slot (r + k) * NL + l, unique because
// r + k grows along the units.
struct RangeLds {
  int64_t part[2 * kWaves];
  int64_t start[3], walk[4];
  int4 pla[kPieceBatch], plb[kPieceBatch];
  int pcount;
};
// Prefix sums of the tiles (and of the rows) over the requests, this workgroup's range
// and where it starts; workgroup 0 also records every request's first unit (and the
// total) and first packed row for the combine.  Returns false for an empty range.
__device__ __forceinline__ bool range_begin(const AttnArgs& a, RangeLds& L, int bid, int nbid, int& k, int& lane) {
  const int G = a.H / a.Hkv;
  const int R = a.req_end - a.req_begin;
  const int per = (R + kThreads - 1) / kThreads;
  const int i0 = min(static_cast<int>(threadIdx.x) * per, R), i1 = min(i0 + per, R);
  int64_t mine = 0, mrows = 0;
  for (int i = i0; i < i1; ++i) {
    mine += req_geom(a, a.req_begin + i, G).tiles;
    mrows += a.ctx_len[a.req_begin + i];
  }
  int64_t U, rows_total;
  const int64_t before = block_exclusive_scan(mine, &U, L.part);
  const int64_t rows_before = block_exclusive_scan(mrows, &rows_total, L.part + kWaves);
  const int W = nbid, w = bid, NL = max(a.dec_lanes, 1);
  const int Wr = max(W / NL, 1);
  const int lw = W % kXcds == 0 ? (w % kXcds) * (W / kXcds) + w / kXcds : w;
  k = lw / NL;
  lane = lw % NL;
  const int kk = min(k, Wr - 1);
  const int64_t u0 = static_cast<int64_t>(kk) * U / Wr, u1 = k < Wr ? static_cast<int64_t>(kk + 1) * U / Wr : u0;
  // The thread whose run holds unit u0 records its request, offset and first row.  Rows:
  // the generation rows follow each other in request order.
  if ((u0 >= before && u0 < before + mine) || w == 0) {
    int64_t acc = before, racc = a.row_begin + rows_before;
    for (int i = i0; i < i1; ++i) {
      const int64_t units = req_geom(a, a.req_begin + i, G).tiles;
      if (w == 0) {
        a.ws_pre[i] = acc;
        a.ws_row[i] = racc;
      }
      if (u0 >= acc && u0 < acc + units) {
        L.start[0] = i;
        L.start[1] = u0 - acc;
        L.start[2] = racc;
      }
      acc += units;
      racc += a.ctx_len[a.req_begin + i];
    }
    if (w == 0 && threadIdx.x == 0) {
      a.ws_pre[R] = U;
      a.ws_row[R] = a.row_begin + rows_total;
    }
  }
  __syncthreads();
  if (u0 >= u1) return false;                                   // empty range (uniform)
  if (threadIdx.x == 0) {
    L.walk[0] = L.start[0];
    L.walk[1] = L.start[1];
    L.walk[2] = u1 - u0;
    L.walk[3] = L.start[2];
  }
  return true;
}
// Thread 0 cuts the next part of the range into at most kPieceBatch pieces for `lane`,
// listed in LDS as (request, head group, column block, first tile) and (tiles, n, S,
// first row); every thread gets their number (0: the range is done).  A lane's column
// block that a request does not have gets no piece.
__device__ __forceinline__ int list_pieces(const AttnArgs& a, const int lane, RangeLds& L) {
  const int G = a.H / a.Hkv;
  const int ncb = max(a.dec_lane_cbs, 1);
  const int hg = lane / ncb, cb = lane % ncb;
  if (threadIdx.x == 0) {
    int r = a.req_begin + static_cast<int>(L.walk[0]);
    int64_t off = L.walk[1], left = L.walk[2], row0 = L.walk[3];
    int np = 0;
    while (left > 0 && r < a.req_end && np < kPieceBatch) {
      const ReqGeom q = req_geom(a, r, G);
      if (off < q.tiles) {
        const int t0 = static_cast<int>(off);
        const int take = static_cast<int>(min64(q.tiles - t0, left));
        if (cb < q.cbs) {
          L.pla[np] = make_int4(r, hg, cb, t0);
          L.plb[np] = make_int4(take, q.n, q.S, static_cast<int>(min64(max64(row0, -1), a.N)));
          ++np;
        }
        left -= take;
        off += take;
      }
      if (off >= q.tiles) {
        row0 += a.ctx_len[r];
        ++r;
        off = 0;
      }
    }
    L.walk[0] = r - a.req_begin;
    L.walk[1] = off;
    L.walk[2] = left;
    L.walk[3] = row0;
    L.pcount = np;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(L.pcount);
}
// LDS bytes of decode_split_body: the staged V and K tiles of the four waves, their
// softmax states and the range's bookkeeping.
template <int DH>
__host__ __device__ constexpr int decode_lds_bytes() {
  return (kWaves * kTile * v_stride<DH>() + kWaves * kTile * DH) * 2 + kWaves * 16 * 2 * 4 + static_cast<int>(sizeof(RangeLds));
}


// Split pass with register-staged tiles (any KV head count, any cache format).  With
// CBW > 1 a segment carries all column blocks of its heads, and the waves of one head
// share each staged tile (every tile leaves HBM once).
template <int KV, int HPS, int CBW, bool NT, bool TREE, int DH>
__device__ __forceinline__ void decode_split_body(const AttnArgs& a, int bid, int nbid, unsigned char* lds) {
  constexpr int kVStride = v_stride<DH>(), kD = DH;
  auto& vtile = *reinterpret_cast<uint16_t (*)[kWaves][kTile * kVStride]>(lds);
  auto& ktile = *reinterpret_cast<uint16_t (*)[kWaves][kTile * kD]>(lds + kWaves * kTile * kVStride * 2);
  auto& ml = *reinterpret_cast<float (*)[kWaves][16][2]>(lds + (kWaves * kTile * kVStride + kWaves * kTile * kD) * 2);
  RangeLds& L = *reinterpret_cast<RangeLds*>(lds + (kWaves * kTile * kVStride + kWaves * kTile * kD) * 2 +
                                             kWaves * 16 * 2 * 4);
  int k, lane;
  if (!range_begin(a, L, bid, nbid, k, lane)) return;
  while (true) {
    const int np = list_pieces(a, lane, L);
    if (np == 0) return;                                        // uniform
    decode_stream<KV, HPS, CBW, NT, TREE, DH>(a, np, k, lane, L.pla, L.plb, vtile, ktile, ml);
    __syncthreads();                                            // the list is read before it is refilled
  }
}

}  // namespace dc
}  // namespace
}  // namespace pkv
