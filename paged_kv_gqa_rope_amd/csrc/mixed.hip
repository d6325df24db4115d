// Mixed in-flight batches (context requests and generation requests in one step) in one
// launch: "TensorRT-LLM source analysis report", 1.3 (mixed-phase processing: chunked
// context together with generation).  The context kernel is bound by the matrix cores
// and moves little memory; the generation split pass is bound by HBM and does little
// arithmetic.  Run one after the other they add up; here the first workgroups of the grid
// run the context kernel's persistent schedule and the rest run split-pass ranges, so
// both proceed at once on disjoint CUs (one workgroup per CU: the context role's LDS
// leaves no room for a second).  The host splits the CUs in proportion to the estimated
// time of each part (context flops at the context kernel's per-CU rate, generation bytes
// at a per-CU streaming rate).  A split-pass workgroup uses four of the eight waves;
// the other four end at once, and the barriers of the four that stay count only waves
// that have not ended.  The combine pass runs afterwards as usual.
#include "decode_dev.h"
#include "prefill_dev.h"

namespace pkv {
namespace {

constexpr int kMixedWaves = 8;
constexpr int kMixedLds = pf::prefill_lds_bytes<4>() > dc::decode_lds_bytes<128>() ? pf::prefill_lds_bytes<4>()
                                                                                  : dc::decode_lds_bytes<128>();

template <int G, bool BT, int KV, bool TREE>
__global__ __launch_bounds__(kMixedWaves * kWave) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mixed_kernel(AttnArgs ac, PrefillSched sc, AttnArgs ad, int nctx) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[kMixedLds];
  const int bid = static_cast<int>(blockIdx.x);
  if (bid < nctx) {
    pf::prefill_body<kMixedWaves, G, 4, BT>(ac, sc, bid, nctx, lds);
    return;
  }
  // waves 4-7 of a split-pass workgroup end here (a wave-uniform test)
  if (__builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x)) >= dc::kThreads) return;
  dc::decode_split_body<KV, 4, 1, true, TREE, 128>(ad, bid - nctx, static_cast<int>(gridDim.x) - nctx, lds);
}

template <int G, int KV, bool TREE>
hipError_t launch_mixed_t(const AttnArgs& ac, const int32_t* host_n, const int32_t* host_S, const AttnArgs& ad,
                          int ctx_wgs, hipStream_t s) {
  constexpr int ROWS = (kMixedWaves / G) * 32;
  PrefillSched sc;
  const int nctx = static_cast<int>(pf::prefill_sched(ac, host_n, host_S, ROWS, ctx_wgs, sc));
  const dim3 grid(static_cast<unsigned>(nctx + ad.dec_wgs));
  if (ac.T % pf::kTileK == 0)
    hipLaunchKernelGGL((mixed_kernel<G, true, KV, TREE>), grid, dim3(kMixedWaves * kWave), 0, s, ac, sc, ad, nctx);
  else
    hipLaunchKernelGGL((mixed_kernel<G, false, KV, TREE>), grid, dim3(kMixedWaves * kWave), 0, s, ac, sc, ad, nctx);
  return hipGetLastError();
}

// draft trees (a packed mask per generation row) or chains; the context kernel reads a
// bf16 cache, so that is the only cache format here
template <int G>
hipError_t launch_mixed_g(const AttnArgs& ac, const int32_t* host_n, const int32_t* host_S, const AttnArgs& ad,
                          int ctx_wgs, hipStream_t s) {
  if (ad.spec_mask != nullptr) return launch_mixed_t<G, F_BF16, true>(ac, host_n, host_S, ad, ctx_wgs, s);
  return launch_mixed_t<G, F_BF16, false>(ac, host_n, host_S, ad, ctx_wgs, s);
}

}  // namespace

bool mixed_supported(const AttnArgs& ad, int num_ctx, int G) {
  return num_ctx <= kPrefillMaxReqs && ad.dec_heads == 4 && ad.dec_cbw == 1 && ad.col_blocks == 1 &&
         (G == 1 || G == 2 || G == 4 || G == 8) && ad.T >= 16 && ad.D == 128 && ad.kv_fmt == F_BF16;
}

hipError_t launch_mixed(const AttnArgs& ac, const int32_t* host_ctx_len, const int32_t* host_seq_len,
                        const AttnArgs& ad, int ctx_wgs, hipStream_t s) {
  if (!host_ctx_len || !host_seq_len || ac.req_end <= ac.req_begin || ctx_wgs < 1 || ad.dec_wgs < 1)
    return hipErrorInvalidValue;
  if (ad.kv_fmt != F_BF16) return hipErrorNotSupported;
  switch (ac.H / ac.Hkv) {
    case 1: return launch_mixed_g<1>(ac, host_ctx_len, host_seq_len, ad, ctx_wgs, s);
    case 2: return launch_mixed_g<2>(ac, host_ctx_len, host_seq_len, ad, ctx_wgs, s);
    case 4: return launch_mixed_g<4>(ac, host_ctx_len, host_seq_len, ad, ctx_wgs, s);
    case 8: return launch_mixed_g<8>(ac, host_ctx_len, host_seq_len, ad, ctx_wgs, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace pkv
