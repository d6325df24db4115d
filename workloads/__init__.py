"""Seeded synthetic in-flight batches for paged-KV attention.

This package is the single source of inputs for both the CPU oracle and the
GPU path.  It holds no arithmetic of the method itself: it draws request
lengths, a physical block permutation and raw values, and nothing else.
RoPE, the storage codecs, the paged scatter and attention all live on the
two sides that are compared.
"""
from .synth import (  # noqa: F401
    FP32, BF16, FP8_E4M3, INT8, CONTEXT, GENERATION,
    Shape, Batch, make_batch, SHAPES, workload, small_workload, WORKLOADS, SMALL_WORKLOADS,
)
