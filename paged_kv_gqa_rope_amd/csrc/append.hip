// RoPE table and RoPE + KV-append kernels for gfx950.
//
// The append is the write half of the paged KV cache: "TensorRT-LLM 1.0 study notes",
// 二.2 (KVCacheManager): the attention op writes each request's new K/V into the blocks
// its block table names.  Pool layout [num_blocks, 2, T, Hkv, D], K at index 0 and V at
// index 1: "TensorRT-LLM source teardown part 1", KV cache manager interfaces
// (get_buffers).  RoPE is the GPT-NeoX variant named in "TensorRT-LLM source analysis
// report", 1.1; rotation of pairs (j, j + R/2) is the reading documented in pkv.h.
//
// Memory-bound: each wave takes one token at a time and streams its q, k and v rows in
// 1 KB instructions (64 lanes x one 8-element chunk), so every load and store is
// coalesced and a lane's chunk sits at the same place in every head it visits.  A
// rotate-half pair's partner chunk is in the same instruction, R/16 lanes away, and comes
// over a lane shuffle; interleaved pairs sit inside one chunk.  A wave issues the loads
// of a whole batch of instructions before any of their arithmetic.  Arithmetic is fp64
// with contraction off and one rounding per stored element, so the stored bits depend
// only on the inputs and the table.  With a per-head q/k norm ("TensorRT-LLM source
// analysis report", 1.1, QK LayerNorm; the teardown's kernel directory lists a fused
// QK-norm + RoPE kernel), the wave copies the batch's q and k rows into LDS, one lane
// per head sums its row in index order, and each lane normalises its chunk and its
// partner's before rotating.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "device_common.h"
#include "kernels.h"

namespace pkv {
namespace {

constexpr int kAppendWaves = 4;
constexpr int kAppendThreads = kAppendWaves * kWave;
constexpr int kMaxTokensPerWg = 64;
constexpr int kFlatMaxRequests = 4096;
constexpr int kAppendWGs = 2048;         // about eight workgroups per CU: many tokens in flight
constexpr size_t kMaxDynamicLds = 64 * 1024;

// chunk instructions whose loads a wave holds at once (bf16 chunks are 16 bytes, fp32 32)
template <int IO, bool NORM>
__host__ __device__ constexpr int append_batch() {
  return IO == F_BF16 ? 6 : (NORM ? 5 : 4);
}
// per-wave LDS of the norm: the batch's q/k rows (padded by 16 bytes) and their statistics
template <int IO, bool NORM>
__host__ __device__ constexpr int norm_rows(int D) {
  return NORM ? append_batch<IO, NORM>() * (kWave * 8 / D) : 0;
}
template <int IO>
__host__ __device__ constexpr int norm_row_bytes(int D) {
  return D * (IO == F_BF16 ? 2 : 4) + 16;
}
template <int IO, bool NORM>
__host__ __device__ constexpr int norm_wave_bytes(int D) {
  return norm_rows<IO, NORM>(D) * (norm_row_bytes<IO>(D) + 16);
}

// Streaming accesses: every input element is read once and every output element written
// once per step, so loads and stores of q, k, v and their outputs carry the nontemporal
// hint; the table and the norm weights stay ordinary (shared by many lanes).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
// 8 raw io elements as loaded (bf16: one 16-byte vector; fp32: two)
struct Raw8 {
  uint4 a, b;
};

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

// Per-head normalisation of 8 elements at dims dim0 .. dim0+7 of one q or k head:
// y = ((x - mean) * inv) * w (+ b), fp64, with (mean, inv) of the head.  The RMS form has
// mean 0 and no bias (x - 0 is x, so the subtraction is left out).  w and b are the
// weights and biases widened to fp64 (exactly) in LDS.
template <bool LAYER>
__device__ __forceinline__ void norm8(double (&x)[8], int dim0, double2 st, const double* w, const double* b) {
#pragma clang fp contract(off)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const double d = LAYER ? x[i] - st.x : x[i];
    const double y = (d * st.y) * w[dim0 + i];
    x[i] = LAYER ? y + b[dim0 + i] : y;
  }
}

// Where one token goes: its packed row, request, cache position, rotation position and
// pool slot.
struct TokenSlot {
  int64_t row;
  int32_t r, m, p, blk, slot;   // blk < 0: table entry out of range (skip the K/V store)
};

__device__ __forceinline__ TokenSlot make_slot(const AppendArgs& a, int64_t row, int r, int i) {
  TokenSlot tk;
  tk.row = row;
  tk.r = r;
  const int n = a.ctx_len[r], base = a.seq_len[r] - n;
  tk.m = base + i;
  // a draft tree's token rotates at base + its position offset (checked on the host to
  // lie in 0 .. n-1; kept there whatever the device copy holds)
  tk.p = tk.m;
  if (a.pos_off != nullptr && row >= a.gen_row && row < a.N) tk.p = base + min(max(a.pos_off[row], 0), max(n - 1, 0));
  const int64_t lblk = tk.m / a.T;
  int32_t blk = (tk.m >= 0 && lblk < a.mbps) ? a.table[static_cast<int64_t>(r) * a.mbps + lblk] : -1;
  tk.blk = (blk >= 0 && blk < a.num_blocks) ? blk : -1;
  tk.slot = tk.m % a.T;
  return tk;
}

// A token read from LDS lands in vector registers; its fields are the same in every
// lane, and saying so keeps the buffer descriptors built from them in scalar registers.
__device__ __forceinline__ TokenSlot uniform_slot(const TokenSlot& t) {
  TokenSlot u;
  const uint64_t row = static_cast<uint64_t>(t.row);
  u.row = static_cast<int64_t>((static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(row >> 32))) << 32) |
                               static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(row))));
  u.r = __builtin_amdgcn_readfirstlane(t.r);
  u.m = __builtin_amdgcn_readfirstlane(t.m);
  u.p = __builtin_amdgcn_readfirstlane(t.p);
  u.blk = __builtin_amdgcn_readfirstlane(t.blk);
  u.slot = __builtin_amdgcn_readfirstlane(t.slot);
  return u;
}

// Intra-wave LDS hand-over: the wave's stores are visible to its own later loads.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint4 shfl16(uint4 v, int src) {
  return make_uint4(__shfl(v.x, src), __shfl(v.y, src), __shfl(v.z, src), __shfl(v.w, src));
}

// A token's q, k and v rows are walked as 8-element chunks, 64 per instruction:
// instructions [0, nq) cover q, then nk of k, then nk of v.  D / 8 chunks make a head and
// divide 64, so lane l always holds chunk l % (D/8) of some head.
struct RowGeom {
  int cph, nqc, nkc, nq, nk, nqk, ntot;
  __device__ RowGeom(const AppendArgs& a, int Hq) {
    cph = a.D / 8;
    nqc = Hq * cph;
    nkc = a.Hkv * cph;
    nq = (nqc + kWave - 1) / kWave;
    nk = (nkc + kWave - 1) / kWave;
    nqk = nq + nk;
    ntot = nqk + nk;
  }
};

// Raw buffer accesses (gfx9-family descriptor: stride 0, 32-bit data format, range
// checked per access).  A lane whose chunk is not stored or loaded gets an offset past
// every range: its load returns zeros and its store is dropped.  Every chunk instruction
// thus issues the same memory operations whatever its lanes' roles, so the compiler's
// wait counts stay exact instead of falling back to draining all outstanding accesses.
constexpr int kBufWord3 = 0x00020000;
constexpr int kBufNT = 2;                        // nontemporal cache policy (loads of inputs read once)
constexpr uint32_t kOff = 0x80000000u;           // past every range
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kBufWord3);
}
__device__ __forceinline__ uint4 bload16(Rsrc r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, kBufNT);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void bstore16(Rsrc r, uint32_t off, uint4 u) {
  __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{u.x, u.y, u.z, u.w}, r, static_cast<int>(off), 0, 0);
}
__device__ __forceinline__ void bstore8(Rsrc r, uint32_t off, uint2 u) {
  __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{u.x, u.y}, r, static_cast<int>(off), 0, 0);
}
template <int F>
__host__ __device__ constexpr int fmt_bytes() {
  return F == F_FP32 ? 4 : F == F_BF16 ? 2 : 1;
}

// y (times `mul` for fp8 and int8) rounded once to format F: 8 elements as stored
// (bf16 in .a, fp32 in .a and .b, fp8 and int8 in .a.x and .a.y).
template <int F>
__device__ __forceinline__ Raw8 pack8(const double (&y)[8], double mul) {
  Raw8 o;
  o.b = make_uint4(0, 0, 0, 0);
  if constexpr (F == F_FP32) {
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = __float_as_uint(static_cast<float>(y[i]));
    o.a = make_uint4(w[0], w[1], w[2], w[3]);
    o.b = make_uint4(w[4], w[5], w[6], w[7]);
  } else if constexpr (F == F_BF16) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = f64x2_to_bf16x2(y[2 * i], y[2 * i + 1]);
    o.a = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i)
      w[i / 4] |= (F == F_INT8 ? f64_to_int8(y[i] * mul) : f64_to_e4m3(y[i] * mul)) << (8 * (i % 4));
    o.a = make_uint4(w[0], w[1], 0, 0);
  }
  return o;
}
// One chunk of format F at off: exactly one or two buffer stores whatever the lane.
template <int F>
__device__ __forceinline__ void store8(Rsrc r, uint32_t off, const Raw8& o) {
  if constexpr (F == F_FP32) {
    bstore16(r, off, o.a);
    bstore16(r, off + 16, o.b);
  } else if constexpr (F == F_BF16) {
    bstore16(r, off, o.a);
  } else {
    bstore8(r, off, make_uint2(o.a.x, o.a.y));
  }
}
__device__ __forceinline__ Raw8 select8(bool c, const Raw8& p, const Raw8& q) {
  Raw8 o;
  o.a = make_uint4(c ? p.a.x : q.a.x, c ? p.a.y : q.a.y, c ? p.a.z : q.a.z, c ? p.a.w : q.a.w);
  o.b = make_uint4(c ? p.b.x : q.b.x, c ? p.b.y : q.b.y, c ? p.b.z : q.b.z, c ? p.b.w : q.b.w);
  return o;
}

// Loads of instructions [b0, b0 + NB) of one token (lanes past a row's end get zeros).
template <int IO, int NB>
__device__ __forceinline__ void append_load(const AppendArgs& a, const RowGeom& g, const TokenSlot& tk, int lane,
                                            int b0, bool live, Raw8 (&r)[NB]) {
  constexpr int CB = 8 * fmt_bytes<IO>();        // bytes of one chunk
  const unsigned char* qb = static_cast<const unsigned char*>(a.q) + tk.row * a.q_stride * fmt_bytes<IO>();
  const unsigned char* kb = static_cast<const unsigned char*>(a.k) + tk.row * a.kv_stride * fmt_bytes<IO>();
  const unsigned char* vb = static_cast<const unsigned char*>(a.v) + tk.row * a.kv_stride * fmt_bytes<IO>();
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    const int i = b0 + u;
    const bool isq = i < g.nq, isk = i < g.nqk;
    const Rsrc rs = rsrc(isq ? qb : isk ? kb : vb, static_cast<int64_t>(isq ? g.nqc : g.nkc) * CB);
    const int ch = (isq ? i : isk ? i - g.nq : i - g.nqk) * kWave + lane;
    const uint32_t off = live && i < g.ntot ? static_cast<uint32_t>(ch) * CB : kOff;
    r[u].a = bload16(rs, off);
    r[u].b = IO == F_FP32 ? bload16(rs, off + 16) : make_uint4(0, 0, 0, 0);
  }
}

// Rotation role of a lane's chunk (dims e0 .. e0+7), the same in every instruction:
// 1 rotate-half first half (partner R/16 lanes up), 2 second half (partner R/16 lanes
// down), 3 interleaved pairs inside the chunk, 0 none (dims past the rotary part).
struct Role {
  int role, jt, poff;
};
// Rotate-half over whole 128-dim bf16 heads: a head is one 16-lane DPP row and partner
// chunks are 8 lanes apart, so the exchange is a row rotation (no LDS traffic).
constexpr int kRopeNeoxRow = 3;
template <int RS>
__host__ __device__ constexpr bool neox() {
  return RS == kRopeNeox || RS == kRopeNeoxRow;
}
__device__ __forceinline__ uint4 row_ror8(uint4 v) {
  return make_uint4(__builtin_amdgcn_mov_dpp(v.x, 0x128, 0xF, 0xF, false),
                    __builtin_amdgcn_mov_dpp(v.y, 0x128, 0xF, 0xF, false),
                    __builtin_amdgcn_mov_dpp(v.z, 0x128, 0xF, 0xF, false),
                    __builtin_amdgcn_mov_dpp(v.w, 0x128, 0xF, 0xF, false));
}
template <int RS>
__device__ __forceinline__ Role chunk_role(int e0, int R) {
  const int half = R / 2;
  Role r{0, 0, 0};
  if constexpr (neox<RS>()) {
    if (e0 < half) r = Role{1, e0, half / 8};
    else if (e0 < R) r = Role{2, e0 - half, -(half / 8)};
  } else if constexpr (RS == kRopeGptj) {
    if (e0 < R) r = Role{3, e0 / 2, 0};
  }
  return r;
}
// (cos, sin) of the lane's pairs at the token's position (row 0 where nothing rotates)
template <int RS>
__device__ __forceinline__ void load_table(const AppendArgs& a, const TokenSlot& tk, const Role& rl,
                                           double2 (&cs)[8]) {
  if constexpr (RS != kRopeNone) {
    const double2* t = reinterpret_cast<const double2*>(a.cos_sin) +
                       (rl.role != 0 && tk.p < a.max_pos ? static_cast<int64_t>(tk.p) * (a.R / 2) + rl.jt : 0);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      cs[k] = t[RS == kRopeGptj ? k % 4 : k];
      // rotate-half first half: y = x1*cos + x2*(-sin), which rounds as x1*cos - x2*sin
      if (rl.role == 1) cs[k].y = -cs[k].y;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) cs[k] = make_double2(0.0, 0.0);
  }
}

// Arithmetic and stores of instructions [b0, b0 + NB) of one token.  Rotation roles of a
// lane's chunk (dims e0 .. e0+7): rotate-half first half (partner R/16 lanes up), second
// half (partner R/16 lanes down), interleaved (pairs inside the chunk), or none (dims
// past the rotary part).
template <int IO, int KV, int RS, int NK, int NB>
__device__ __forceinline__ void append_compute(const AppendArgs& a, const RowGeom& g, const TokenSlot& tk,
                                               const Role& rl, const double2 (&cs)[8], int lane, int b0,
                                               const Raw8 (&r)[NB], unsigned char* __restrict__ stage,
                                               const double* __restrict__ wts) {
#pragma clang fp contract(off)
  constexpr bool NORM = NK != kNormNone, LAYER = NK == kNormLayer;
  constexpr int kRaw = IO == F_BF16 ? 0 : 1;     // fp32 chunks are two 16-byte halves
  constexpr int CB = 8 * fmt_bytes<IO>(), KB = 8 * fmt_bytes<KV>();
  const int D = a.D;
  const int cph = g.cph, hpi = kWave / cph;
  const int c = lane % cph, e0 = c * 8;
  const int role = rl.role, poff = rl.poff;
  // positions past the table (rejected by the host) leave the rotated dims unwritten
  const bool rot_ok = tk.p < a.max_pos;
  const bool kv_ok = tk.blk >= 0;
  const int64_t kdst = ((static_cast<int64_t>(tk.blk) * 2) * a.T + tk.slot) * static_cast<int64_t>(a.Hkv) * D;
  // descriptors are built where they are used (from scalar bases and sizes), so they stay
  // in scalar registers
  unsigned char* const qo = static_cast<unsigned char*>(a.q_out) + tk.row * static_cast<int64_t>(a.H) * D * fmt_bytes<IO>();
  unsigned char* const ko = static_cast<unsigned char*>(a.pool) + (kv_ok ? kdst * fmt_bytes<KV>() : 0);
  unsigned char* const vo = ko + (kv_ok ? static_cast<int64_t>(a.T) * a.Hkv * D * fmt_bytes<KV>() : 0);
  const int64_t qo_bytes = static_cast<int64_t>(g.nqc) * CB, kv_bytes = kv_ok ? static_cast<int64_t>(g.nkc) * KB : 0;
  const int rowb = norm_row_bytes<IO>(D);
  double2* stat = reinterpret_cast<double2*>(stage + norm_rows<IO, NORM>(D) * rowb);
  const int poff_lane = lane + poff;
  const int nq = g.nq, nqk = g.nqk, ntot = g.ntot;

  if constexpr (NORM) {
    // this batch's q/k rows into LDS, then one lane per row: (mean, 1/sqrt(var + eps)),
    // fp64 sums in index order (as the oracle and pkv.h state)
    const int nqk_b = min(NB, max(nqk - b0, 0));
    wave_sync();                                  // earlier readers of the staging rows are done
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      if (u < nqk_b) {
        unsigned char* dst = stage + (u * hpi + lane / cph) * rowb + c * CB;
        *reinterpret_cast<uint4*>(dst) = r[u].a;
        if constexpr (kRaw) *reinterpret_cast<uint4*>(dst + 16) = r[u].b;
      }
    }
    wave_sync();
    constexpr bool layer = LAYER;
    // A row's chunks are read kStatAhead at a time (cph = D / 8 is 8 or 16), so one LDS
    // latency covers several chunks; the sums still run in index order.
    constexpr int kStatAhead = 8;
    for (int h = lane; h < nqk_b * hpi; h += kWave) {
      const unsigned char* row = stage + h * rowb;
      double s = 0.0;
      if (layer) {
        for (int q0 = 0; q0 < cph; q0 += kStatAhead) {
          Raw8 q8[kStatAhead];
#pragma unroll
          for (int j = 0; j < kStatAhead; ++j) {
            q8[j].a = *reinterpret_cast<const uint4*>(row + (q0 + j) * CB);
            q8[j].b = kRaw ? *reinterpret_cast<const uint4*>(row + (q0 + j) * CB + 16) : make_uint4(0, 0, 0, 0);
          }
#pragma unroll
          for (int j = 0; j < kStatAhead; ++j) {
            double x[8];
            widen8<IO>(q8[j], x);
#pragma unroll
            for (int e = 0; e < 8; ++e) s += x[e];
          }
        }
      }
      const double mean = layer ? s / static_cast<double>(D) : 0.0;
      double ss = 0.0;
      for (int q0 = 0; q0 < cph; q0 += kStatAhead) {
        Raw8 q8[kStatAhead];
#pragma unroll
        for (int j = 0; j < kStatAhead; ++j) {
          q8[j].a = *reinterpret_cast<const uint4*>(row + (q0 + j) * CB);
          q8[j].b = kRaw ? *reinterpret_cast<const uint4*>(row + (q0 + j) * CB + 16) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < kStatAhead; ++j) {
          double x[8];
          widen8<IO>(q8[j], x);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            if (layer) {
              const double d = x[e] - mean;
              ss += d * d;
            } else {
              // x widens a bf16 or fp32 value (at most 24 significant bits), so x * x is
              // exact in fp64 and the fused form rounds once, as ss + x * x does
              ss = __builtin_fma(x[e], x[e], ss);
            }
          }
        }
      }
      stat[h] = make_double2(mean, 1.0 / __builtin_sqrt(ss / static_cast<double>(D) + a.norm_eps));
    }
    wave_sync();
  }
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    const int i = b0 + u;
    const bool isq = i < nq, isk = i < nqk;
    const int kind = isq ? 0 : isk ? 1 : 2;
    const int ch = (isq ? i : isk ? i - nq : i - nqk) * kWave + lane;
    const bool live = i < ntot;
    if (kind == 2) {                                 // values: not rotated
      const uint32_t off = live ? static_cast<uint32_t>(ch) * KB : kOff;
      if constexpr (KV == IO) {
        store8<KV>(rsrc(vo, kv_bytes), off, r[u]);
      } else {
        double x[8];
        widen8<IO>(r[u], x);
        store8<KV>(rsrc(vo, kv_bytes), off, pack8<KV>(x, a.inv_v_scale));
      }
      continue;
    }
    Raw8 pr = r[u];
    if constexpr (RS == kRopeNeoxRow && !NORM) {
      pr.a = row_ror8(r[u].a);
    } else if constexpr (RS == kRopeNeox) {          // every lane takes part in the shuffle
      pr.a = shfl16(r[u].a, poff_lane);
      if constexpr (kRaw) pr.b = shfl16(r[u].b, poff_lane);
    }
    double x[8], y[8];
    widen8<IO>(r[u], x);
    if constexpr (NORM) {
      const bool isq = kind == 0;
      norm8<LAYER>(x, e0, stat[u * hpi + lane / cph], wts + (isq ? 0 : D), wts + (isq ? 2 : 3) * D);
    }
    // every lane computes its rotation; the role then selects (no divergent branches)
    if constexpr (RS == kRopeGptj) {                 // pairs (2k, 2k+1) inside the chunk
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const double2 t = cs[k];
        const double x1 = x[2 * k], x2 = x[2 * k + 1];
        const double p = x1 * t.x, q = x2 * t.y, e = x2 * t.x, f = x1 * t.y;
        const double y1 = p - q, y2 = e + f;
        y[2 * k] = role == 3 ? y1 : x1;
        y[2 * k + 1] = role == 3 ? y2 : x2;
      }
    } else if constexpr (neox<RS>()) {
      double pv[8];
      if constexpr (NORM && RS == kRopeNeoxRow) {
        // the partner's normalised values over the row rotation (the same fp64 values
        // its own lane computed)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const uint64_t bits = __builtin_bit_cast(uint64_t, x[k]);
          const uint32_t lo = __builtin_amdgcn_mov_dpp(static_cast<int>(bits), 0x128, 0xF, 0xF, false);
          const uint32_t hi = __builtin_amdgcn_mov_dpp(static_cast<int>(bits >> 32), 0x128, 0xF, 0xF, false);
          pv[k] = __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
        }
      } else {
        widen8<IO>(pr, pv);
        if constexpr (NORM) {
          const bool isq = kind == 0;
          norm8<LAYER>(pv, e0 + poff * 8, stat[u * hpi + lane / cph], wts + (isq ? 0 : D), wts + (isq ? 2 : 3) * D);
        }
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const double2 t = cs[k];
        // first half: y = x1*cos - x2*sin with x1 own (the sine arrives negated: a + (-b)
        // rounds as a - b); second half: y = x2*cos + x1*sin with x2 own
        const double own = x[k] * t.x, other = pv[k] * t.y;
        const double sum = own + other;
        y[k] = RS == kRopeNeoxRow || role != 0 ? sum : x[k];
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) y[k] = x[k];
    }
    const bool skip = !live || (role != 0 && !rot_ok);
    // dims past the rotary part keep their input bits when nothing changes them
    const bool raw = !NORM && RS != kRopeNeoxRow && role == 0;
    if (kind == 0) {
      const uint32_t off = skip ? kOff : static_cast<uint32_t>(ch) * CB;
      store8<IO>(rsrc(qo, qo_bytes), off, select8(raw, r[u], pack8<IO>(y, 1.0)));
    } else {
      const uint32_t off = skip ? kOff : static_cast<uint32_t>(ch) * KB;
      if constexpr (KV == IO) store8<KV>(rsrc(ko, kv_bytes), off, select8(raw, r[u], pack8<KV>(y, a.inv_k_scale)));
      else store8<KV>(rsrc(ko, kv_bytes), off, pack8<KV>(y, a.inv_k_scale));
    }
  }
}

// FLAT: the grid walks the packed rows, tokens_per_wg consecutive rows per workgroup,
// and each workgroup finds the rows' requests through an LDS prefix scan of the
// context lengths (batches of at most kFlatMaxRequests requests).  Otherwise the grid
// is (row tile, request), for any batch size.  Each wave then takes every fourth token
// of the workgroup.
template <int IO, int KV, int RS, bool FLAT, int NK>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a, int tokens_per_wg) {
  constexpr bool NORM = NK != kNormNone;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ TokenSlot s_tok[kMaxTokensPerWg];
  const int Hq = a.q ? a.H : 0;
  const int cu_bytes = FLAT ? ((a.B + 1) * 4 + 15) / 16 * 16 : 0;
  int ntok;
  if constexpr (FLAT) {
    int32_t* s_cu = reinterpret_cast<int32_t*>(smem);
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
    __shared__ int32_t s_wave[kAppendWaves];
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
  // the norm's weights and biases in LDS, widened to fp64: q weights, k weights, q
  // biases, k biases
  double* wts = reinterpret_cast<double*>(smem + cu_bytes);
  if constexpr (NORM) {
    for (int d = threadIdx.x; d < a.D; d += kAppendThreads) {
      wts[d] = a.qn_w ? static_cast<double>(a.qn_w[d]) : 0.0;
      wts[a.D + d] = static_cast<double>(a.kn_w[d]);
      wts[2 * a.D + d] = a.qn_b ? static_cast<double>(a.qn_b[d]) : 0.0;
      wts[3 * a.D + d] = a.kn_b ? static_cast<double>(a.kn_b[d]) : 0.0;
    }
  }
  __syncthreads();
  // the wave index is the same in every lane; saying so keeps the token walk scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  unsigned char* stage = smem + cu_bytes + (NORM ? 32 * a.D : 0) + wave * norm_wave_bytes<IO, NORM>(a.D);
  // The workgroup's (token, batch) items, token-major; wave w takes items w, w + 4, ...
  // The table and the loads of a wave's next item are issued before the arithmetic of
  // its current one.
  constexpr int NB = append_batch<IO, NORM>();
  const RowGeom g(a, Hq);
  const int nb = (g.ntot + NB - 1) / NB;
  const int nitems = ntok * nb;
  const Role rl = chunk_role<RS>((lane % g.cph) * 8, RS != kRopeNone ? a.R : 0);
  auto next_item = [&](int j) {
    while (j < nitems) {
      const TokenSlot tk = uniform_slot(s_tok[j / nb]);
      if (tk.row < a.N && tk.m >= 0) break;
      j += kAppendWaves;
    }
    return j;
  };
  int j = next_item(wave);
  if (j >= nitems) return;
  Raw8 cur[NB];
  append_load<IO, NB>(a, g, uniform_slot(s_tok[j / nb]), lane, (j % nb) * NB, true, cur);
  for (;;) {
    const int jn = next_item(j + kAppendWaves);
    const bool more = jn < nitems;
    const TokenSlot tk = uniform_slot(s_tok[j / nb]);
    double2 cs[8];
    load_table<RS>(a, tk, rl, cs);
    Raw8 nxt[NB];
    // issued on every pass (all lanes out of range on the last) so that the loads and
    // stores of an item do not depend on a branch
    const int jl = more ? jn : j;
    append_load<IO, NB>(a, g, uniform_slot(s_tok[jl / nb]), lane, (jl % nb) * NB, more, nxt);
    append_compute<IO, KV, RS, NK, NB>(a, g, tk, rl, cs, lane, (j % nb) * NB, cur, stage, wts);
    if (!more) break;
    j = jn;
#pragma unroll
    for (int u = 0; u < NB; ++u) cur[u] = nxt[u];
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
  auto go2 = [&](auto rs, auto nrm) {
    constexpr int RS = decltype(rs)::value;
    constexpr int NK = decltype(nrm)::value;
    constexpr bool NORM = NK != kNormNone;
    // items of a token (batches of NB chunk instructions), as the kernel counts them
    const int64_t cph = a.D / 8, Hq = a.q ? a.H : 0;
    const int64_t ntot = (Hq * cph + kWave - 1) / kWave + 2 * ((a.Hkv * cph + kWave - 1) / kWave);
    const int64_t nb = (ntot + append_batch<IO, NORM>() - 1) / append_batch<IO, NORM>();
    // about kAppendWGs workgroups: items per wave, then whole tokens per workgroup
    const int64_t ipw = (a.N * nb + kAppendWGs * kAppendWaves - 1) / (kAppendWGs * kAppendWaves);
    const int tpw = static_cast<int>(std::min<int64_t>(kMaxTokensPerWg, std::max<int64_t>(1, (ipw * kAppendWaves + nb - 1) / nb)));
    const size_t stage = (NORM ? 32 * static_cast<size_t>(a.D) : 0) + static_cast<size_t>(kAppendWaves) * norm_wave_bytes<IO, NORM>(a.D);
    const size_t lds = (static_cast<size_t>(a.B + 1) * 4 + 15) / 16 * 16 + stage;
    if (a.B <= kFlatMaxRequests && lds <= kMaxDynamicLds) {
      const dim3 grid(static_cast<unsigned>((a.N + tpw - 1) / tpw));
      hipLaunchKernelGGL((append_kernel<IO, KV, RS, true, NK>), grid, dim3(kAppendThreads), lds, s, a, tpw);
    } else {
      const dim3 grid((a.max_n + tpw - 1) / tpw, a.B);
      hipLaunchKernelGGL((append_kernel<IO, KV, RS, false, NK>), grid, dim3(kAppendThreads), stage, s, a, tpw);
    }
  };
  auto go = [&](auto rs) {
    if (a.norm == kNormRms) go2(rs, std::integral_constant<int, kNormRms>());
    else if (a.norm == kNormLayer) go2(rs, std::integral_constant<int, kNormLayer>());
    else go2(rs, std::integral_constant<int, kNormNone>());
  };
  if (a.rope == kRopeNeox && IO == F_BF16 && a.D == 128 && a.R == 128) go(std::integral_constant<int, kRopeNeoxRow>());
  else if (a.rope == kRopeNeox) go(std::integral_constant<int, kRopeNeox>());
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
