"""The library's opt-in timing at both levels: one record per kernel launch, or one per
phase with the generation attention (split pass and combine) as a single span."""
import pytest
import torch

from workloads import synth as W

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cosched", [0, 1])
def test_timing_levels_record_launches_and_phases(cosched):
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from paged_kv_gqa_rope_amd import _lib as L
    from paged_kv_gqa_rope_amd.harness import PagedStep
    b = W.small_workload(4)                  # context chunks, then generation requests
    print("CASE timing levels", b.label, "co-scheduled" if cosched else "serial", flush=True)
    old = L.pkv_set_coschedule(cosched)
    try:
        _check_levels(L, PagedStep(b), cosched)
    finally:
        L.pkv_set_coschedule(old)


def _check_levels(L, st, cosched):
    st.step()
    torch.cuda.synchronize()
    if cosched:      # context and split pass in one launch, then the combine
        expect = {1: {"append_rope", "mixed", "decode_combine"}, 2: {"append_rope", "mixed"}}
    else:
        expect = {1: {"append_rope", "prefill_mfma", "decode_split", "decode_combine"},
                  2: {"append_rope", "prefill_mfma", "decode"}}
    spans = {}
    for level, names in expect.items():
        L.check(L.pkv_kernel_timing_enable(level))
        for _ in range(3):
            st.step()
        torch.cuda.synchronize()
        rec = L.pkv_kernel_timings()
        L.check(L.pkv_kernel_timing_enable(0))
        got = {}
        for name, ms in rec:
            assert ms > 0.0, (name, ms)
            got.setdefault(name, []).append(ms)
        assert set(got) == names, (level, sorted(got))
        assert all(len(v) == 3 for v in got.values()), {n: len(v) for n, v in got.items()}
        spans[level] = {n: sum(v) / len(v) for n, v in got.items()}
    print("per launch (ms)", spans[1], "per phase (ms)", spans[2])
    # nothing is recorded with timing off
    st.step()
    torch.cuda.synchronize()
    assert L.pkv_kernel_timings() == []
