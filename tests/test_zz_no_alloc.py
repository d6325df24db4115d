"""pkv_attention_forward_noalloc (the library's own scratch array instead of a caller
workspace) against pkv_attention_forward on the same inputs: two calls in a row, the
second with a smaller batch, each bitwise equal to the workspace entry point's output
(same kernels and split policy) and within the oracle's bars."""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import step as O
from parity_util import bits_of, compare_attention
from workloads import synth as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def H():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from paged_kv_gqa_rope_amd import _lib, harness
    _lib.lib()
    return harness


def _noalloc(H, st):
    from paged_kv_gqa_rope_amd import _lib as L
    return L.pkv_attention_forward_noalloc(st.desc, st.bdesc, st.q_out.data_ptr(), st.q_out.shape[1],
                                           st.pool.data_ptr(), st.out.data_ptr(), st.stream)


BATCHES = [
    # (label, batch): each pair runs big first, then smaller, so the second call finds the
    # first call's partial results in the scratch array
    ("mixed-gqa8", lambda: W.make_batch(W.SHAPES[4], ctx=[(128, 0), (64, 256)],
                                        gen_past=[300, 2500, 4000, 63, 1000, 700, 1500, 90], seed=5100)),
    ("mixed-gqa8-small", lambda: W.make_batch(W.SHAPES[4], gen_past=[200, 77], seed=5101)),
    ("fp8-drafts", lambda: W.fitted(W.make_batch(dataclasses.replace(W.SHAPES[5], max_num_tokens=1 << 12),
                                                 gen_past=[3000, 9000, 200], gen_new=[4, 2, 1], seed=5102))),
    ("fp8-small", lambda: W.fitted(W.make_batch(W.SHAPES[5], gen_past=[1500], seed=5103))),
]


@pytest.mark.parametrize("pair", [(0, 1), (2, 3)])
def test_noalloc_matches_the_workspace_entry_point(H, pair):
    for i in pair:
        label, make = BATCHES[i]
        b = make()
        print("CASE noalloc", label, b.shape.name, flush=True)
        st = H.PagedStep(b)
        assert st.ws_bytes > 0, "the case must use split-KV partial results"
        assert st.append() == 0
        assert st.forward() == 0
        torch.cuda.synchronize()
        want = bits_of(st.out_host()).copy()
        st.out.zero_()
        assert _noalloc(H, st) == 0
        torch.cuda.synchronize()
        got = bits_of(st.out_host())
        assert np.array_equal(got, want), f"{label}: scratch output differs from workspace output"
        compare_attention(st.out_host(), O.run(b)["out"], b.shape, label)
