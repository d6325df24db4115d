#!/usr/bin/env python3
"""Benchmark one step (RoPE + KV append, then attention) of the paged-KV GQA path.

Prints ONE JSON line.  ``value`` is the whole-step throughput of the decode
workload (64 generation requests, cached lengths 512..4096, 32 q heads = 32 KV
heads, head_dim 128, 64-token blocks, bf16): algorithmic bytes of the step per
second, inputs resident in HBM.  The prefill, mixed and fp8-decode workloads
are reported under ``workloads``.  ``ms_per_step`` comes from K steps timed with torch
events on the launch stream and no other instrumentation; per-kernel durations come from
K further steps with the library's own HIP events recorded around every launch on that
stream (the decode roofline takes the split pass plus its combine).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads 2,3,4,5]
                       [--no-cpu-baseline] [--copy-calibration]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode attn GB/s & % HBM peak; prefill attn TFLOP/s & % MFMA peak; tok/s"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
BF16_DENSE_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
BYTES = {"fp32": 4, "bf16": 2, "fp8_e4m3": 1, "int8": 1}
HEADLINE = 2


def algorithmic(batch) -> dict:
    """Algorithmic work of one step (see the formulas in the design notes)."""
    import numpy as np
    sh = batch.shape
    H, Hkv, D, T = sh.num_heads, sh.num_kv_heads, sh.head_dim, sh.tokens_per_block
    bio, bkv = BYTES[sh.io_dtype], BYTES[sh.kv_dtype]
    gen = batch.request_types == 1
    S = batch.sequence_lengths.astype(np.int64)
    n = batch.context_lengths.astype(np.int64)
    p = S - n
    decode_bytes = int(np.sum(S[gen] * Hkv * D * 2 * bkv + n[gen] * H * D * 2 * bio + 4 * ((S[gen] + T - 1) // T)))
    ctx = ~gen
    ctx_flops = int(4 * D * H * np.sum(n[ctx] * p[ctx] + n[ctx] * (n[ctx] + 1) // 2))
    N = int(n.sum())
    R = sh.rot_dim
    append_bytes = N * ((H + 2 * Hkv) * D * bio + H * D * bio + 2 * Hkv * D * bkv + (R // 2) * 16)
    return dict(decode_bytes=decode_bytes, ctx_flops=ctx_flops, append_bytes=append_bytes, tokens=N,
                gen_keys=int(S[gen].sum()), num_gen=int(gen.sum()), num_ctx=int(ctx.sum()))


def describe(batch) -> str:
    sh = batch.shape
    import numpy as np
    gen = batch.request_types == 1
    parts = []
    if (~gen).any():
        parts.append(f"{int((~gen).sum())} context requests (n={sorted(set(batch.context_lengths[~gen].tolist()))}, "
                     f"cached={sorted(set(batch.past_lengths[~gen].tolist()))})")
    if gen.any():
        parts.append(f"{int(gen.sum())} generation requests (cached {int(batch.past_lengths[gen].min())}.."
                     f"{int(batch.past_lengths[gen].max())}, sum S={int(batch.sequence_lengths[gen].sum())})")
    return (f"{sh.name}: " + " + ".join(parts) + f"; H={sh.num_heads} Hkv={sh.num_kv_heads} D={sh.head_dim} "
            f"T={sh.tokens_per_block} io={sh.io_dtype} kv={sh.kv_dtype} rope_base={sh.rope_theta:g}"
            + (f" rope={sh.rope_style} rotary_dim={sh.rot_dim}" if sh.rope_style != "neox" or sh.rot_dim != sh.head_dim
               else "")
            + (f" qk_norm={sh.qk_norm}" if sh.qk_norm != "none" else "")
            + (f" out=fp8(scale {sh.out_fp8_scale:g})" if sh.out_fp8_scale > 0 else "")
            + (" drafts=random trees" if getattr(batch, "tree", False) else ""))


def variant_batch(name: str):
    """Batches of the variant measurements: a workload at full size with one change."""
    import dataclasses

    from workloads import synth as W
    if name == "gptj3":          # workload 3 with RoPE on interleaved pairs over the whole head
        sh = dataclasses.replace(W.SHAPES[3], rope_style="gptj")
        return W.make_batch(sh, ctx=[(2048, 0)] * 8, seed=1003, label="w3-gptj")
    if name == "gptj3-half":     # interleaved pairs on the first half of each head (R = D/2)
        sh = dataclasses.replace(W.SHAPES[3], rope_style="gptj", rotary_dim=64)
        return W.make_batch(sh, ctx=[(2048, 0)] * 8, seed=1003, label="w3-gptj-half")
    if name == "spec4-gqa8":     # workload 4's 128 generation requests, each with 1 + 3 draft tokens
        sh = dataclasses.replace(W.SHAPES[4])
        past = W._uniform_pasts(1004, 128, 256, 4096)
        return W.make_batch(sh, gen_past=past, gen_new=[4] * 128, seed=1004, label="w4-spec4")
    if name == "tree4-gqa8":     # the same 128 requests with their 1 + 3 tokens as random draft trees
        sh = dataclasses.replace(W.SHAPES[4])
        past = W._uniform_pasts(1004, 128, 256, 4096)
        return W.make_batch(sh, gen_past=past, gen_new=[4] * 128, seed=1004, label="w4-tree4", tree=True)
    if name == "qknorm3":        # workload 3 with a per-head RMS norm of q and k before RoPE
        sh = dataclasses.replace(W.SHAPES[3], qk_norm="rms")
        return W.make_batch(sh, ctx=[(2048, 0)] * 8, seed=1003, label="w3-qknorm")
    if name == "fp8out3":        # workload 3 with the attention output written as fp8 (scale 2^-6)
        sh = dataclasses.replace(W.SHAPES[3], out_fp8_scale=2.0 ** -6)
        return W.make_batch(sh, ctx=[(2048, 0)] * 8, seed=1003, label="w3-fp8out")
    if name == "mha64-2":        # workload 2's 64 requests with 64-dim heads
        b = W.workload(2)
        sh = dataclasses.replace(b.shape, name="decode-mha-bf16-d64", head_dim=64)
        return dataclasses.replace(b, shape=sh, label="w2-d64")
    if name == "int8kv5":        # workload 5 with an int8 KV cache, K/V scales fitted to its values (amax/127)
        sk, sv = W.W5_INT8_SCALES
        sh = dataclasses.replace(W.SHAPES[5], name="longdecode-gqa4-int8kv", kv_dtype=W.INT8,
                                 k_scale=sk, v_scale=sv)
        b = W.workload(5)
        return dataclasses.replace(b, shape=sh, label="w5-int8kv")
    raise KeyError(name)


VARIANTS = ("gptj3", "gptj3-half", "qknorm3", "fp8out3", "spec4-gqa8", "tree4-gqa8", "int8kv5", "mha64-2")


def decode_us(res: dict) -> float:
    """Decode attention time: the split pass and its combine as one span (one event pair
    around both launches), else the sum of their own event pairs."""
    if "decode" in res.get("phases", {}):
        return res["phases"]["decode"]["avg_us"]
    kern = res["kernels"]
    return kern["decode_split"]["avg_us"] + kern.get("decode_combine", {"avg_us": 0.0})["avg_us"]


def _timed_pass(L, st, steps: int, level: int) -> dict:
    """K steps with the library's timing at `level` (1: launches, 2: phases); average per name."""
    import torch
    L.check(L.pkv_kernel_timing_enable(level))
    for _ in range(steps):
        st.step()
    torch.cuda.synchronize()
    timings = L.pkv_kernel_timings()
    L.check(L.pkv_kernel_timing_enable(0))
    per: dict[str, list[float]] = {}
    for name, ms in timings:
        per.setdefault(name, []).append(ms)
    return {n: dict(avg_us=1e3 * sum(v) / len(v), launches=len(v)) for n, v in per.items()}


def _step_ms(st, steps: int) -> float:
    """Average ms of K steps, one event pair around all of them (library timing off)."""
    import torch
    stream = torch.cuda.current_stream()
    beg, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    beg.record(stream)
    for _ in range(steps):
        st.step()
    end.record(stream)
    torch.cuda.synchronize()
    return beg.elapsed_time(end) / steps


def run_workload(k: int, steps: int, warmup: int, batch=None) -> dict:
    """Warm-up, then K timed steps with the library's timing off (ms_per_step), then K
    steps with an event pair around every launch (per-kernel durations) and K with one
    around every phase (the decode span: split pass and combine with nothing between).
    A mixed batch runs by default as one launch for its context and split-pass parts; its
    per-kernel durations (for the rooflines) come from the same passes repeated with the
    two parts launched one after the other, and `coscheduled` keeps the one-launch figures.
    K serial steps run before the one-launch timing, so neither mode is timed colder."""
    import torch

    from paged_kv_gqa_rope_amd import _lib as L
    from paged_kv_gqa_rope_amd.harness import PagedStep
    from workloads import synth as W

    if batch is None:
        batch = W.workload(k)
    t0 = time.time()
    st = PagedStep(batch, sentinel=False)
    torch.cuda.synchronize()
    setup_s = time.time() - t0
    for _ in range(warmup):
        st.step()
    torch.cuda.synchronize()
    mixed = "mixed" in _timed_pass(L, st, 1, 1)
    if mixed:
        # the serial launches run K steps first, so that both launch modes are timed
        # after the same number of steps (the first few dozen steps run slower)
        old = L.pkv_set_coschedule(0)
        try:
            _step_ms(st, steps)
        finally:
            L.pkv_set_coschedule(old)
    ms_per_step = _step_ms(st, steps)
    kern = _timed_pass(L, st, steps, 1)
    phases = _timed_pass(L, st, steps, 2)
    co = None
    if mixed:
        co = dict(ms_per_step=ms_per_step, kernels=kern, phases=phases)
        old = L.pkv_set_coschedule(0)
        try:
            ms_serial = _step_ms(st, steps)
            kern = _timed_pass(L, st, steps, 1)
            phases = _timed_pass(L, st, steps, 2)
        finally:
            L.pkv_set_coschedule(old)
        co["ms_per_step_serial"] = ms_serial
    w = algorithmic(batch)
    step_bytes = w["append_bytes"] + w["decode_bytes"]
    res = dict(workload=describe(batch), setup_s=round(setup_s, 2), ms_per_step=ms_per_step,
               tok_per_s=w["tokens"] / (ms_per_step * 1e-3), kernels=kern, phases=phases, work=w)
    if co is not None:
        res["coscheduled"] = co
    if "decode_split" in kern:
        span = decode_us(res) * 1e-6
        res["decode_GBps"] = w["decode_bytes"] / span / 1e9
        res["decode_split_GBps"] = w["decode_bytes"] / (kern["decode_split"]["avg_us"] * 1e-6) / 1e9
    for name in ("prefill_mfma", "attn_generic_ctx"):
        if name in kern:
            res["prefill_TFLOPs"] = w["ctx_flops"] / (kern[name]["avg_us"] * 1e-6) / 1e12
            res["prefill_kernel"] = name
    if "append_rope" in kern:
        res["append_GBps"] = w["append_bytes"] / (kern["append_rope"]["avg_us"] * 1e-6) / 1e9
    res["step_GBps"] = step_bytes / (ms_per_step * 1e-3) / 1e9
    del st
    torch.cuda.empty_cache()
    return res


def measured_traffic(kernel: str, k: int):
    """HBM bytes per launch measured with rocprofv3 counters (profiles/pmc_traffic.json),
    or None when absent or when the kernel's sources changed since the measurement."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    entry = json.load(open(path)).get("kernels", {}).get(f"{kernel}@{k}")
    if not entry:
        return None
    h = hashlib.sha256()
    for f in entry["sources"]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return entry["hbm_bytes_per_launch"] if h.hexdigest() == entry["sha256"] else None


# Targets: decode attention >= 70% of HBM peak, context attention >= 45% of dense bf16 peak.
TARGET_FRAC = {"hbm": 0.70, "mfma": 0.45}


def roofline_for(res: dict, k: int) -> dict:
    """Roofline of the dominant kernel.  Decode: algorithmic bytes over the split pass's
    average launch, and over the whole decode phase (split pass and combine, one event
    pair around both), the phase deciding the target; context: causal flops over the
    context kernel."""
    kern = res["kernels"]
    w = res["work"]
    if "decode_split" in kern and w["decode_bytes"] > 0 and w["ctx_flops"] == 0:
        split_us = kern["decode_split"]["avg_us"]
        ach = w["decode_bytes"] / (split_us * 1e-6) / 1e9
        phase_us = decode_us(res)
        phase = w["decode_bytes"] / (phase_us * 1e-6) / 1e9
        return dict(kernel="decode_split", bound="hbm", achieved=ach, peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=ach / HBM_PEAK_GBS, traffic=measured_traffic("decode_split", k), avg_us=split_us,
                    phase=dict(name="decode_split + decode_combine", avg_us=phase_us, achieved=phase,
                               frac=phase / HBM_PEAK_GBS),
                    target_frac=TARGET_FRAC["hbm"], meets_target=phase / HBM_PEAK_GBS >= TARGET_FRAC["hbm"])
    name = "prefill_mfma" if "prefill_mfma" in kern else "attn_generic_ctx"
    ach = w["ctx_flops"] / (kern[name]["avg_us"] * 1e-6) / 1e12
    return dict(kernel=name, bound="mfma", achieved=ach, peak=BF16_DENSE_PEAK_TFLOPS, unit="TFLOP/s",
                frac=ach / BF16_DENSE_PEAK_TFLOPS, traffic=measured_traffic(name, k), avg_us=kern[name]["avg_us"],
                target_frac=TARGET_FRAC["mfma"], meets_target=ach / BF16_DENSE_PEAK_TFLOPS >= TARGET_FRAC["mfma"])


def _blas_vendor() -> str:
    import numpy as np
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg["Build Dependencies"]["blas"]
        return f"{b.get('name')} {b.get('version', '')}".strip()
    except Exception:  # pragma: no cover
        return "unknown"


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        return 1


def _predrawn(batch):
    """The batch with its value draws memoised, so that drawing happens before the timer."""
    import dataclasses

    from workloads import synth as W

    class PreDrawn(W.Batch):
        def _draw(self, tag, r, rows, heads):
            key = (tag, r)
            if key not in self._memo:
                self._memo[key] = W.Batch._draw(self, tag, r, rows, heads)
            return self._memo[key]

    pb = PreDrawn(**{f.name: getattr(batch, f.name) for f in dataclasses.fields(batch)})
    pb._memo = {}
    return pb


def _oracle_request(O, b, r, tabs, hist, heads=None):
    """The oracle's step for request r: append of its new tokens (RoPE, rounding, cache
    codes), its cache read back, attention of its new rows.  ``hist`` is its stored history."""
    import numpy as np
    sh = b.shape
    q_out, k_new, v_new = O.append_request(b, r, tabs)
    K = O.codecs.decode(np.concatenate([hist[0], k_new]), sh.kv_dtype, sh.k_scale)
    V = O.codecs.decode(np.concatenate([hist[1], v_new]), sh.kv_dtype, sh.v_scale)
    q = O.io_decode(b, q_out)
    pos = int(b.past_lengths[r]) + np.arange(q.shape[0])
    return O.attend(q, K, V, pos, heads=heads)


def cpu_baseline(budget_s: float = 24.0) -> dict:
    """The oracle (fp64 numpy, untuned) on bounded samples of workloads 2-5, in the units of
    the GPU figures.  Per sampled request the timer covers the oracle's step (append of the
    new tokens, reading the cache, attention); drawing the values and encoding the history
    (the cache contents before the step) happen before it."""
    import numpy as np

    from oracle import step as O
    from workloads import synth as W
    plan = [(2, "gen", 0.2), (3, "ctx", 0.3), (4, "ctx", 0.2), (4, "gen", 0.1), (5, "gen", 0.2)]
    per = {}
    for k, part, share in plan:
        b = _predrawn(W.workload(k))
        sh = b.shape
        tabs = O.tables(b)
        gen = np.nonzero(b.request_types == 1)[0] if part == "gen" else np.nonzero(b.request_types == 0)[0]
        el, done, kv_bytes, flops, toks = 0.0, [], 0, 0, 0
        bio, bkv = BYTES[sh.io_dtype], BYTES[sh.kv_dtype]
        for r in gen:
            r = int(r)
            for f in ("new_q", "new_k", "new_v"):
                getattr(b, f)(r)
            hist = O.history_request(b, r)
            t0 = time.perf_counter()
            _oracle_request(O, b, r, tabs, hist)
            el += time.perf_counter() - t0
            n, S = int(b.context_lengths[r]), int(b.sequence_lengths[r])
            p = S - n
            kv_bytes += S * sh.num_kv_heads * sh.head_dim * 2 * bkv + n * sh.num_heads * sh.head_dim * 2 * bio
            flops += 4 * sh.head_dim * sh.num_heads * (n * p + n * (n + 1) // 2)
            toks += n
            done.append(r)
            b._memo.clear()
            if el >= share * budget_s:
                break
        key = f"workload_{k}" + ("_generation" if k == 4 and part == "gen" else "_context" if k == 4 else "")
        e = dict(seconds=round(el, 2), tok_per_s=toks / el,
                 sample=f"{part} requests {done[0]}..{done[-1]} ({len(done)} of {len(gen)}), all heads")
        if part == "gen":
            e["kv_GBps"] = kv_bytes / el / 1e9
        else:
            e["GFLOPs"] = flops / el / 1e9
        per[key] = e
    head = per[f"workload_{HEADLINE}"]
    return dict(value=head["kv_GBps"], unit="GB/s", cores=len(os.sched_getaffinity(0)), kind="oracle",
                sample=f"workload {HEADLINE}: {head['sample']}, {head['seconds']} s of oracle steps "
                       f"(append + cache read + attention per request; value draws and history encoding "
                       f"outside the timer)",
                blas=_blas_vendor(), blas_threads=_blas_threads(), per_config=per)


def copy_calibration(gib: float = 1.0, reps: int = 5):
    """A plain device copy of known size, for scaling HBM byte counters."""
    import torch
    n = int(gib * (1 << 30))
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "reps": reps}),
          file=sys.stderr)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workloads", default="2,3,4,5")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--variants", default=",".join(VARIANTS),
                    help="comma-separated variant measurements (empty for none): " + ", ".join(VARIANTS))
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.copy_calibration:
        copy_calibration()
    ks = [int(x) for x in args.workloads.split(",") if x]
    results = {}
    for k in ks:
        print(f"[bench] workload {k} ...", file=sys.stderr, flush=True)
        results[k] = run_workload(k, args.steps, args.warmup)
        print(f"[bench] workload {k}: {results[k]['ms_per_step']:.3f} ms/step "
              f"{ {n: round(v['avg_us'], 1) for n, v in results[k]['kernels'].items()} } phases "
              f"{ {n: round(v['avg_us'], 1) for n, v in results[k]['phases'].items()} }", file=sys.stderr, flush=True)
        co = results[k].get("coscheduled")
        if co:
            print(f"[bench] workload {k} one launch for context + split pass: {co['ms_per_step']:.3f} ms/step "
                  f"(serial {co['ms_per_step_serial']:.3f}) "
                  f"{ {n: round(v['avg_us'], 1) for n, v in co['kernels'].items()} } phases "
                  f"{ {n: round(v['avg_us'], 1) for n, v in co['phases'].items()} }", file=sys.stderr, flush=True)
    head_k = HEADLINE if HEADLINE in results else ks[0]
    head = results[head_k]
    line = {
        "metric": METRIC,
        "value": head["step_GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) values, seeded lengths and block permutation)",
        "config": {"workload": head["workload"], "tok_per_s": head["tok_per_s"],
                   "decode_GBps": head.get("decode_GBps"), "pct_hbm_peak": 100 * head.get("decode_GBps", 0) / HBM_PEAK_GBS,
                   "kernels_us": {n: round(v["avg_us"], 2) for n, v in head["kernels"].items()},
                   "phases_us": {n: round(v["avg_us"], 2) for n, v in head["phases"].items()}},
        "roofline": roofline_for(head, head_k),
    }
    others = {}
    for k, r in results.items():
        if k == head_k:
            continue
        o = dict(workload=r["workload"], ms_per_step=r["ms_per_step"], tok_per_s=r["tok_per_s"],
                 kernels_us={n: round(v["avg_us"], 2) for n, v in r["kernels"].items()},
                 phases_us={n: round(v["avg_us"], 2) for n, v in r["phases"].items()})
        for f in ("decode_GBps", "prefill_TFLOPs", "append_GBps", "prefill_kernel"):
            if f in r:
                o[f] = r[f]
        if "decode_GBps" in r:
            o["decode_pct_hbm_peak"] = 100 * r["decode_GBps"] / HBM_PEAK_GBS
        if "prefill_TFLOPs" in r:
            o["prefill_pct_bf16_peak"] = 100 * r["prefill_TFLOPs"] / BF16_DENSE_PEAK_TFLOPS
        o["roofline"] = roofline_for(r, k)
        co = r.get("coscheduled")
        if co:
            # the step above is one launch for the context and split-pass parts; the
            # per-kernel figures and rooflines come from the same batch launched serially
            o["ms_per_step_serial"] = co["ms_per_step_serial"]
            o["coscheduled_us"] = {n: round(v["avg_us"], 2) for n, v in co["kernels"].items()}
            o["coscheduled_phases_us"] = {n: round(v["avg_us"], 2) for n, v in co["phases"].items()}
        others[f"workload_{k}"] = o
    line["workloads"] = others
    variants = {}
    for name in [x for x in args.variants.split(",") if x]:
        print(f"[bench] variant {name} ...", file=sys.stderr, flush=True)
        r = run_workload(0, args.steps, args.warmup, batch=variant_batch(name))
        print(f"[bench] variant {name}: {r['ms_per_step']:.3f} ms/step "
              f"{ {n: round(v['avg_us'], 1) for n, v in r['kernels'].items()} } phases "
              f"{ {n: round(v['avg_us'], 1) for n, v in r['phases'].items()} }", file=sys.stderr, flush=True)
        o = dict(workload=r["workload"], ms_per_step=r["ms_per_step"], tok_per_s=r["tok_per_s"],
                 kernels_us={n: round(v["avg_us"], 2) for n, v in r["kernels"].items()},
                 phases_us={n: round(v["avg_us"], 2) for n, v in r["phases"].items()})
        for f in ("decode_GBps", "prefill_TFLOPs", "append_GBps", "prefill_kernel"):
            if f in r:
                o[f] = r[f]
        variants[name] = o
    if variants:
        line["variants"] = variants
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
