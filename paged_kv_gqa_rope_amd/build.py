"""Compile the gfx950 kernels and the C ABI into ``paged_kv_gqa_rope_amd/libpkv.so``.

Every call compiles every source (no up-to-date checks): ``hipcc`` cross-compiles
for gfx950 without a GPU.  Objects go to ``_build/`` next to this file; the shared
library is written under a temporary name and renamed into place.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpkv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]
# Packed fp32 VALU forms stay disabled in all device code.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # private arrays stay in registers; LDS is laid out by hand
          "-mllvm", "-disable-promote-alloca-to-lds"]
PER_FILE = {
    # the append's bit-exact recipe: no fused multiply-add anywhere in that file
    "append.hip": ["-ffp-contract=off"],
    # scores are finite or -inf, never NaN: max needs no NaN canonicalisation
    "prefill.hip": ["-fno-honor-nans"],
    "mixed.hip": ["-fno-honor-nans"],
}


def sources() -> list[str]:
    return sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(name: str) -> str:
    src = os.path.join(CSRC, name)
    obj = os.path.join(BUILD, name + ".o")
    cmd = [HIPCC] + COMMON + DEVICE + PER_FILE.get(name, []) + ["-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    names = sources()
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(names)))) as ex:
        objs = list(ex.map(_compile, names))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(names)} sources", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
