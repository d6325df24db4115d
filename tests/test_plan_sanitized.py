"""The HIP-free host part of the library (batch validation, split plan, workspace
bound, draft-tree checks) built on its own with AddressSanitizer and
UndefinedBehaviorSanitizer, driven through every error case and a few thousand random
batches (each with a random valid tree and a planted tree fault)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_gqa_rope_amd", "csrc")

EXPECTED = {
    "desc_null": -1, "head_dim_96": -2, "tokens_per_block_48": -2, "heads_not_multiple": -1,
    "rotary_dim_24": -2, "rotary_dim_gt_head_dim": -1, "fp8_zero_scale": -1, "io_fp8": -2,
    "softmax_scale_inf": -1, "ok_mixed": 0, "order": -3, "chunk_align": -4, "budget": -5,
    "block_id_outside_pool": -6, "table_too_narrow": -6, "too_many_draft_tokens": -2,
    "sequence_shorter_than_chunk": -1, "num_tokens_mismatch": -1, "max_context_length_short": -1,
    "host_lengths_null": -1, "bad_request_type": -1, "zero_context_length": -1, "empty": 0,
    "tree_ok": 0, "tree_offset_past_n": -1, "tree_own_bit_missing": -1, "tree_bit_past_n": -1, "tree_null": -1,
}


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("g++ not found")
    out = str(tmp_path_factory.mktemp("plan") / "plan_check")
    flags = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
    srcs = [os.path.join(CSRC, "plan.cpp"), os.path.join(ROOT, "tests", "native", "plan_check.cpp")]
    res = subprocess.run([cxx] + flags + srcs + ["-o", out], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return out


def test_validation_cases_and_random_batches_under_sanitizers(driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    res = subprocess.run([driver, "3000"], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr[-4000:]
    got = {}
    for line in res.stdout.splitlines():
        if line.startswith("case "):
            _, name, rc = line.split()
            got[name] = int(rc)
    assert got == EXPECTED
    fuzz = [l for l in res.stdout.splitlines() if l.startswith("fuzz")][0].split()
    assert int(fuzz[3]) > 300, fuzz            # enough accepted batches to mean something
