"""CPU oracle for paged-KV GQA attention with RoPE.  TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct statement of what the hot
path computes, in float64 numpy over a contiguous (unpaged) per-request KV
layout.  It is used only by ``tests/``, by ``__graft_entry__.smoke()`` and by
the ``cpu_baseline`` leg of ``bench.py``.  The product path (the HIP library
and its Python binding) never imports, calls or links anything here, and this
package imports nothing from the product; the two share only the seeded input
generators in ``workloads``.

Sources, by page (all pages are secondary descriptions of TensorRT-LLM):

* "TensorRT-LLM source analysis report" (adg.csdn.net), sections 1.1
  (attention parameters: sequence_length, context_lengths, host_request_types,
  max_context_length, rotary_embedding; GQA head grouping; GPT-NeoX RoPE),
  1.2 (KV cache parameters: kv_cache_block_offsets) and 1.3 (in-flight
  batching: context requests before generation requests, chunks that are
  multiples of the KV block size, the max_num_tokens budget).
* "TensorRT-LLM 1.0 study notes" (openharmonycrossplatform.csdn.net),
  section 6.1-6.3 (context phase with causal FlashAttention, generation phase
  of one query token over all cached K/V reached through block pointers) and
  the INT8 KV cache passage under 6.4 (quantise on write with
  kv_scale_orig_quant, dequantise on read with kv_scale_quant_orig).
* "TensorRT-LLM source teardown part 1: architecture overview"
  (pinghaoyang.com.cn), sections on the KV cache manager interfaces (pool
  layout [num_blocks, 2, tokens_per_block, num_kv_heads, head_dim] and the
  per-request block ID table), the AttentionMetadata fields and the
  AttentionBackend.forward signature (packed q [num_tokens, num_heads*head_dim]
  and k, v [num_tokens, num_kv_heads*head_dim]), and the kernel directory
  listing (a fused QK-norm + RoPE kernel).

No page writes down the formula of attention, RoPE, the GQA mapping or the
fp8 encoding; the readings taken here are listed in each function.

Parity status per function: every public function is pinned by tests in
``tests/test_oracle.py`` and ``tests/test_codecs.py`` (closed forms,
invariants, library special cases, exhaustive codec enumeration and a
pure-Python brute force); none is "parity unpinned".
"""
from . import codecs, rope, qknorm, attention, step  # noqa: F401
