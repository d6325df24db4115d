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
//  * one item = one KV head's whole GQA group (G = 1, 2, 4 or 8 query heads) for a block
//    of query positions of one request: NW waves, each owning 32 query rows of one query
//    head, so every K/V tile staged in LDS feeds NW waves (all G heads that share it);
//  * persistent workgroups, at most one per CU: each works through a fixed, balanced
//    list of items (see the schedule below) as one stream of tiles, so start-up, output
//    stores and the next item's loads overlap the tiles of the item before;
//  * K/V tiles (64 keys x 128 dims each) travel from the pool straight into LDS with
//    global_load_lds_dwordx4 (no register staging, no LDS store instructions) through
//    a ring of NS stages, so NS-1 tiles are in flight while one is computed; each
//    16-byte chunk is placed at an XOR-swizzled position so that the reads below are
//    free of bank conflicts without padding;
//  * the transposed products keep the softmax in-lane: S^T = K Q^T on
//    v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 dims of K from LDS, B = Q^T held in
//    registers), so lane l owns query l%32 and 16 keys per 32-key block, and the row
//    max/sum need one cross-lane step (lanes l and l^32);
//  * O^T = V^T P^T: B = P^T straight from the score accumulators (converted to bf16),
//    A = V^T read from LDS with ds_read_b64_tr_b16;
//  * only tiles that cross the diagonal are masked, fully masked tiles are skipped, and
//    the output rescale is skipped unless some lane's running maximum grew by > 2^8.
#include "prefill_dev.h"

namespace pkv {
namespace {
using namespace pf;

template <int NW, int G, int NS, bool BT>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_kernel(AttnArgs a, PrefillSched sc) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[prefill_lds_bytes<NS>()];
  prefill_body<NW, G, NS, BT>(a, sc, blockIdx.x, gridDim.x, lds);
}

template <int NW, int G, int NS>
hipError_t launch_t(const AttnArgs& a0, const int32_t* host_n, const int32_t* host_S, hipStream_t s) {
  static_assert(NW % G == 0, "a workgroup holds whole query groups");
  constexpr int ROWS = (NW / G) * 32;
  const int cus = std::max(a0.num_cus, 1);
  hipError_t e = hipSuccess;
  for (int b0 = a0.req_begin; b0 < a0.req_end; b0 += kPrefillMaxReqs) {
    AttnArgs a = a0;
    a.req_begin = b0;
    a.req_end = std::min(b0 + kPrefillMaxReqs, a0.req_end);
    PrefillSched sc;
    const dim3 grid(static_cast<unsigned>(prefill_sched(a, host_n, host_S, ROWS, cus, sc)));
    if (a.T % kTileK == 0)   // tokens_per_block is a power of two: whole tiles per block
      hipLaunchKernelGGL((prefill_kernel<NW, G, NS, true>), grid, dim3(NW * kWave), 0, s, a, sc);
    else
      hipLaunchKernelGGL((prefill_kernel<NW, G, NS, false>), grid, dim3(NW * kWave), 0, s, a, sc);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_prefill(const AttnArgs& a, const int32_t* host_ctx_len, const int32_t* host_seq_len,
                          hipStream_t s) {
  if (a.T < 16) return hipErrorNotSupported;   // a 64-key tile spans at most 4 blocks
  if (!host_ctx_len || !host_seq_len || a.req_end <= a.req_begin) return hipErrorInvalidValue;
  switch (a.H / a.Hkv) {
    case 1: return launch_t<8, 1, 4>(a, host_ctx_len, host_seq_len, s);
    case 2: return launch_t<8, 2, 4>(a, host_ctx_len, host_seq_len, s);
    case 4: return launch_t<8, 4, 4>(a, host_ctx_len, host_seq_len, s);
    case 8: return launch_t<8, 8, 4>(a, host_ctx_len, host_seq_len, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace pkv
