// Generation-phase (decode) attention over the paged cache: split-KV pass + combine.
//
// "TensorRT-LLM 1.0 study notes", 6.3: a generation request has one query token that
// attends to every cached token, reached block by block through the block table; the
// phase is bound by HBM bandwidth.  This design cuts the batch's keys into pieces so that
// even a handful of long requests fills all 256 CUs, and merges the per-piece partial
// results (running max m, sum l, unnormalised output o) in a second pass with the same
// rescaling identity FlashAttention uses to merge tiles (study notes 6.2, update of acc_o
// by the new running max).
//
// Pass 1 is persistent and balanced: a fixed number of workgroups (two per CU) share the
// batch's 32-key tiles of every segment in equal contiguous ranges, so each streams the
// same number of bytes whatever the mix of lengths, and each XCD takes one contiguous
// eighth of them.  A workgroup has 4 waves.  When the KV heads come in fours, every wave
// streams all tiles of a piece for its own (KV head, block of 16 query columns): with one
// column block a segment is (request, 4 neighbouring KV heads, column block), and the four
// waves read the neighbouring heads' pieces of the same cache rows at about the same time,
// which HBM serves faster than one head's pieces alone; with 2 (or 3-4) column blocks
// (draft tokens) a segment is (request, 2 (or 1) KV heads) with all column blocks, and the
// 2 (or 4) waves of one head each load a share of every tile (K or V, or half of either),
// stage it in one LDS tile of the head and meet at a barrier, so each tile leaves HBM
// once.  Otherwise a segment is (request, one KV head, column block),
// its waves sharing the tiles and merging their states in LDS at the end of each piece.
// Per wave and tile:
//   * S^T = K Q^T on MFMA 16x16x32 bf16: A = 16 keys x 32 dims of K, read in operand
//     layout from an LDS copy of the tile (XOR-swizzled 16-byte chunks); B = the G query
//     heads of the KV head (GQA group, G <= 16, padded with zero heads), kept in
//     registers for the whole piece.
//   * online softmax per head on the accumulators (lanes l, l^16, l^32, l^48 hold the
//     same head), exp2 with the log2(e) factor folded into the scale.
//   * O += P V on MFMA: A = P (heads x 32 keys) straight from the score registers,
//     B = V read transposed from an LDS copy of the tile with ds_read_b64_tr_b16.
//   * an fp8 or int8 cache is dequantised to bf16 on load (exact: every e4m3 value
//     and every integer -128 .. 127 is a bf16 value); k_scale folds into the softmax
//     scale and v_scale into the combine, so the pass works on raw codes times one.
// Pass 2, one wave per (generation token, query head): M = max m_p, L = sum 2^(m_p-M) l_p,
// O = sum 2^(m_p-M) o_p / L over the segment's pieces in a fixed order (no atomics:
// bitwise reproducible).
#include "decode_dev.h"

namespace pkv {
namespace {
using namespace dc;

// The split pass on its own: one workgroup of four waves per range.
template <int KV, int HPS, int CBW, bool NT, bool TREE, int DH>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_split_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[decode_lds_bytes<DH>()];
  decode_split_body<KV, HPS, CBW, NT, TREE, DH>(a, blockIdx.x, gridDim.x, lds);
}

// One wave per (generation token, query head) -- or per TPW tokens of one request and query
// head, when requests carry draft tokens -- kCombHeads query heads per workgroup, two
// dimensions per lane.  The pieces of the token's (request, lane) are the ranges that meet
// the request's tiles (found from the recorded first tiles and the same range
// arithmetic).  M = max m_p and L = sum 2^(m_p-M) l_p over them, then lane d sums
// 2^(m_p-M) o_p[2d, 2d+1] over the pieces in order.  64 pieces at a time: lane p holds
// piece p's (m, l), butterfly reductions give M and L in a fixed order, and the o_p are
// loaded kPre (then eight) at a time.  Every metadata load is issued before the first use,
// and the loads of a wave's TPW tokens are all in flight together; at most 64 VGPRs keep
// 8 waves per SIMD resident (one round of waves for most batches).  Pieces past a draft
// token's position hold m = -inf and weigh nothing; the piece holding key 0 makes M finite.
// The sums run in the same order for every TPW (bitwise the same output).  Head size DH:
// lane d holds dimensions 2d and 2d + 1, so with DH = 64 lanes 32 .. 63 hold no
// dimensions (they still hold pieces' (m, l)).
template <int TPW, int DH>
__global__ __launch_bounds__(kCombHeads * kWave) __attribute__((amdgpu_waves_per_eu(8, 8))) void decode_combine_kernel(AttnArgs a) {
  constexpr int kPre = TPW == 1 ? 8 : 4;                             // o_p loads issued with the (m, l) loads
  constexpr int kD = DH;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int h = blockIdx.x * kCombHeads + wave, rg = blockIdx.y, tok0 = blockIdx.z * TPW;
  const int r = a.req_begin + rg;
  const int R = a.req_end - a.req_begin, W = a.dec_wgs;
  const int n_dev = a.ctx_len[r], s_dev = a.seq_len[r];
  const int64_t P = a.ws_pre[rg], U = a.ws_pre[R], row0 = a.ws_row[rg];
  if (h >= a.H || tok0 >= n_dev || U <= 0 || W <= 0) return;      // wave-uniform
  const int G = a.H / a.Hkv, B = a.dec_heads;
  const int n = max(n_dev, 1), S = max(s_dev, n);                   // as the split pass keeps them
  const int tiles = (S - 1) / kTile + 1;
  const int cbs = static_cast<int>(min64((static_cast<int64_t>(G) * n + 15) / 16, a.col_blocks));
  const int g = h / G, hg = g / B, wv = g % B;
  const bool all = a.dec_allcols != 0;
  const int ncb = max(a.dec_lane_cbs, 1), NL = max(a.dec_lanes, 1);
  const int Wr = max(W / NL, 1);
  // the ranges that meet the request's tiles [P, P + tiles): its pieces, range k in slot (rg + k) * NL + pl
  const int64_t f = ((P + 1) * Wr - 1) / U, l = ((P + tiles) * Wr - 1) / U;
  const int kf = static_cast<int>(min64(max64(f, 0), Wr - 1));
  const int np = static_cast<int>(min64(max64(l, kf), Wr - 1)) - kf + 1;
  const int64_t stride = static_cast<int64_t>(NL) * B * a.dec_cols;          // entries between pieces
  // Per token: its output row and the first piece's entry.  A token outside the
  // generation rows, or whose column the split pass did not compute, gets no output.
  bool ok[TPW];
  int64_t row[TPW];
  const float* ob[TPW];                                             // the first piece's o (wave-uniform)
  const float* mlp[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int tok = tok0 + t;
    row[t] = row0 + tok;
    // segment and stored column of (token, head): (request, head group, column block) and
    // the column within its block, or, when segments carry all column blocks, (request,
    // head group) and the column
    const int c = tok * G + h % G, cb = all ? 0 : c / 16, col = all ? c : c % 16;
    const int pl = hg * ncb + (ncb > 1 ? cb : 0);                   // the split-pass lane that computed it
    ok[t] = tok < n_dev && row[t] >= a.row_begin && row[t] < a.N && !(!all && cb >= cbs) && col < a.dec_cols;
    const int64_t e0 = ok[t] ? ((static_cast<int64_t>(rg + kf) * NL + pl) * B + wv) * a.dec_cols + col : 0;
    ob[t] = a.ws_o + e0 * kD;
    mlp[t] = a.ws_ml + e0 * 2;
  }
  // o_p of piece p for this lane
  const int64_t ps = stride * kD;                                   // floats between pieces
  const int dl = DH == 128 ? lane : min(lane, DH / 2 - 1);           // this lane's dimension pair
  auto o_at = [&](int t, int p) { return *reinterpret_cast<const float2*>(ob[t] + p * ps + 2 * dl); };
  float L[TPW], ox[TPW], oy[TPW];
  if (np <= kWave) {
    // One memory round trip: every lane loads one piece's (m, l) while the first kPre
    // pieces' o are loaded (issued after the (m, l) loads, so waiting for those does not
    // wait for these); the weights follow from the maximum.
    float2 mlv[TPW], u0[TPW][kPre];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
      mlv[t] = ok[t] ? *reinterpret_cast<const float2*>(mlp[t] + min(lane, np - 1) * stride * 2) : make_float2(0.f, 0.f);
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int e = 0; e < kPre; ++e)                                // weight 0 past the last piece
        u0[t][e] = ok[t] ? o_at(t, min(e, np - 1)) : make_float2(0.f, 0.f);
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const float M = wave_max(lane < np ? mlv[t].x : -INFINITY);
      const float wt = lane < np && mlv[t].x != -INFINITY ? exp2f(mlv[t].x - M) : 0.f;
      L[t] = wave_sum(wt * (lane < np ? mlv[t].y : 0.f));
      ox[t] = oy[t] = 0.f;
#pragma unroll
      for (int e = 0; e < kPre; ++e) {
        const float w = __shfl(wt, e, kWave);
        ox[t] += w * u0[t][e].x;
        oy[t] += w * u0[t][e].y;
      }
      for (int k = kPre; k < np && ok[t]; k += 8) {               // eight loads in flight
        float2 u[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] = o_at(t, min(k + e, np - 1));
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // 0 past the last piece (lanes >= np hold weight 0; pieces past lane 63 do not exist)
          const float w = k + e < kWave ? __shfl(wt, k + e, kWave) : 0.f;
          ox[t] += w * u[e].x;
          oy[t] += w * u[e].y;
        }
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      L[t] = ox[t] = oy[t] = 0.f;
      if (!ok[t]) continue;
      float M = -INFINITY;
      for (int pb = 0; pb < np; pb += kWave) {
        const int p = pb + lane;
        M = fmaxf(M, wave_max(p < np ? mlp[t][p * stride * 2] : -INFINITY));
      }
      for (int pb = 0; pb < np; pb += kWave) {
        const int p = pb + lane;
        float wt = 0.f, lp = 0.f;
        if (p < np) {
          const float2 v = *reinterpret_cast<const float2*>(mlp[t] + p * stride * 2);
          wt = v.x == -INFINITY ? 0.f : exp2f(v.x - M);
          lp = v.y;
        }
        L[t] += wave_sum(wt * lp);
        const int cnt = min(kWave, np - pb);
        for (int k = 0; k < cnt; k += 8) {                         // eight loads in flight
          float2 u[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) u[e] = k + e < cnt ? o_at(t, pb + k + e) : make_float2(0.f, 0.f);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float w = __shfl(wt, k + e, kWave);              // u[e] = 0 past the last piece
            ox[t] += w * u[e].x;
            oy[t] += w * u[e].y;
          }
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    if (!ok[t] || 2 * lane >= DH) continue;
    const float sc = a.v_scale / L[t];
    const int64_t oi = (row[t] * a.H + h) * kD + 2 * lane;
    if (a.out_fmt == F_FP8) {
      const uint32_t lo = f32_to_e4m3(ox[t] * sc * a.out_mul), hi = f32_to_e4m3(oy[t] * sc * a.out_mul);
      *reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(a.out) + oi) = static_cast<uint16_t>(lo | (hi << 8));
    } else {
      const uint32_t lo = f32_to_bf16(ox[t] * sc), hi = f32_to_bf16(oy[t] * sc);
      *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.out) + oi) = lo | (hi << 16);
    }
  }
}

}  // namespace

template <int KV, bool TREE, int DH>
void launch_split_t(const AttnArgs& a, hipStream_t s) {
  const dim3 grid(a.dec_wgs), block(kThreads);
  if (a.dec_cbw == 4) hipLaunchKernelGGL((decode_split_kernel<KV, 1, 4, true, TREE, DH>), grid, block, 0, s, a);
  else if (a.dec_cbw == 2) hipLaunchKernelGGL((decode_split_kernel<KV, 2, 2, true, TREE, DH>), grid, block, 0, s, a);
  else if (a.dec_heads == kWaves) hipLaunchKernelGGL((decode_split_kernel<KV, 4, 1, true, TREE, DH>), grid, block, 0, s, a);
  else if (a.col_blocks == 1) hipLaunchKernelGGL((decode_split_kernel<KV, 1, 1, true, TREE, DH>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((decode_split_kernel<KV, 1, 1, false, TREE, DH>), grid, block, 0, s, a);
}

template <bool TREE, int DH>
void launch_split_kv(const AttnArgs& a, hipStream_t s) {
  if (a.kv_fmt == F_FP8) launch_split_t<F_FP8, TREE, DH>(a, s);
  else if (a.kv_fmt == F_INT8) launch_split_t<F_INT8, TREE, DH>(a, s);
  else launch_split_t<F_BF16, TREE, DH>(a, s);
}

hipError_t launch_decode_split(const AttnArgs& a, hipStream_t s) {
  if (a.D != 64 && a.D != 128) return hipErrorInvalidValue;
  if (a.spec_mask != nullptr) {
    if (a.D == 64) launch_split_kv<true, 64>(a, s);
    else launch_split_kv<true, 128>(a, s);
  } else {
    if (a.D == 64) launch_split_kv<false, 64>(a, s);
    else launch_split_kv<false, 128>(a, s);
  }
  return hipGetLastError();
}

template <int DH>
void launch_combine_t(const AttnArgs& a, hipStream_t s) {
  constexpr int kTpw = 2;                                            // tokens per wave with draft tokens
  const int hb = (a.H + kCombHeads - 1) / kCombHeads, R = a.req_end - a.req_begin;
  if (a.max_n > 1)
    hipLaunchKernelGGL((decode_combine_kernel<kTpw, DH>), dim3(hb, R, (a.max_n + kTpw - 1) / kTpw), dim3(kCombHeads * kWave), 0, s, a);
  else
    hipLaunchKernelGGL((decode_combine_kernel<1, DH>), dim3(hb, R, a.max_n), dim3(kCombHeads * kWave), 0, s, a);
}

hipError_t launch_decode_combine(const AttnArgs& a, hipStream_t s) {
  if (a.D == 64) launch_combine_t<64>(a, s);
  else if (a.D == 128) launch_combine_t<128>(a, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
