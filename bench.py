#!/usr/bin/env python3
"""Benchmark of the learned-relative GQA attention forward on one MI355X.

One step = one whole forward over the workload: the scheduler pre-pass
(``attn_plan``), the fp16 value copy (``attn_stage_values``) and the attention
kernel (``attn_fwd_planned``), inputs already resident in HBM.  Prints ONE JSON line:

* ``value``: effective attention TFLOP/s, counting 4*D flops per unmasked
  (query, key, head) pair (2*D for q.k, 2*D for p.v) over the step's wall time;
* ``roofline``: the attention kernel's algorithmic flops per launch divided by
  its average duration, timed with HIP events on the stream it runs on,
  against the dense MFMA peak (bf16 and fp16 share it);
* ``cpu_baseline``: the fp64 oracle timed on this host's cores over a bounded
  sample of the same workload's rows.

Default workload: the S=8192 full-causal GQA shape (B=1, S=8192, Hq=32, Hkv=8,
D=128, E=1024, no window), the long full-causal shape the MFMA-utilisation
target is stated for.  ``--workload`` selects another.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 / fp16 MFMA
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E
DEFAULT_WORKLOAD = "full_causal_8k"
MALL_FLUSH_BYTES = 512 << 20  # twice the MI355X's 256 MB MALL


class MallFlush:
    """Evicts the step's inputs from the 256 MB MALL before every timed step.

    ``read``: a reduction reads a 512 MiB buffer, which leaves the MALL full of
    clean lines.  ``write``: a fill writes it, which leaves the MALL full of
    dirty lines that the timed kernels then write back to HBM as they evict
    them (traffic that is not theirs).
    """

    def __init__(self, mode, dev):
        import torch
        self.mode = mode
        self.buf = torch.ones(MALL_FLUSH_BYTES, dtype=torch.uint8, device=dev)
        self.sink = None

    def __call__(self):
        if self.mode == "read":
            self.sink = self.buf.sum()
        else:
            self.buf.fill_(1)

    def describe(self):
        return f"a {MALL_FLUSH_BYTES >> 20} MiB {self.mode}"
# the forward kernel's sources: its traffic record holds their combined sha256
KERNEL_SRCS = [os.path.join(ROOT, "transformer_attention_03_amd", "csrc", f) for f in ("inkattn.hip", "common.h")]


def kernel_source_sha256() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def allowed_counts(x) -> np.ndarray:
    """Allowed keys per query row from the workload's structure (closed form).

    Documents are contiguous column ranges starting where positions restart, real
    tokens form one prefix span per row, so row i sees the real keys in
    [max(doc_start(i), i - W + 1), i].
    """
    valid = x["valid"].numpy().astype(np.int64)
    pos = x["positions"].numpy().astype(np.int64)
    B, S = valid.shape
    W = x["window"] if x["window"] else S
    cols = np.arange(S)
    lo = np.maximum(cols - pos, cols - W + 1)
    pref = np.concatenate([np.zeros((B, 1), np.int64), np.cumsum(valid, axis=1)], axis=1)
    n = pref[:, cols + 1] - pref[np.arange(B)[:, None], lo]
    return np.where(valid > 0, n, 0)


def used_profile_entries(x, E=None) -> int:
    """Profile elements the method reads: allowed pairs with distance below E (per head)."""
    valid = x["valid"].numpy().astype(np.int64)
    pos = x["positions"].numpy().astype(np.int64)
    B, S = valid.shape
    E = x["profiles"].shape[-1] if E is None else E
    W = x["window"] if x["window"] else S
    cols = np.arange(S)
    lo = np.maximum(np.maximum(cols - pos, cols - W + 1), cols - E + 1)
    pref = np.concatenate([np.zeros((B, 1), np.int64), np.cumsum(valid, axis=1)], axis=1)
    n = pref[:, cols + 1] - pref[np.arange(B)[:, None], lo]
    return int(np.where(valid > 0, n, 0).sum())


def algorithmic_work(x):
    w = x["workload"]
    cnt = allowed_counts(x)
    pairs = int(cnt.sum()) * w.Hq
    flops = 4.0 * w.D * pairs
    valid_rows = int(x["valid"].sum())
    pe = 2 if w.profiles_dtype.itemsize == 2 else 4
    nbytes = (valid_rows * w.Hq * w.D * 2                 # q (real rows)
              + valid_rows * w.Hkv * w.D * 2 * 2          # k, v (real keys)
              + used_profile_entries(x) * w.Hq * pe       # profile entries read
              + valid_rows * w.Hq * 4                     # sink
              + w.B * w.S * w.Hq * (w.D + 1) * 4          # out + lse (all rows)
              + w.B * w.S * (1 + 4))                      # valid + positions
    return cnt, pairs, flops, nbytes


def flex_allowed_counts(x) -> np.ndarray:
    """Allowed keys per query row of a generic flex workload (closed form): the row
    sees the keys from the start of its block (after the last EOS before it, or a
    fixed-block start) up to itself, within the window."""
    w = x["workload"]
    S = w.S
    cnt = np.zeros((w.B, S), dtype=np.int64)
    for b in range(w.B):
        ends = set(x["doc_ends"][b]) if x["tokens"] is not None else set()
        start = 0
        for i in range(S):
            st = start
            if x["fixed_block_size"]:
                st = max(st, (i // x["fixed_block_size"]) * x["fixed_block_size"])
            if x["sliding_window"]:
                st = max(st, i - x["sliding_window"] + 1)
            cnt[b, i] = i - st + 1
            if i in ends:
                start = i + 1
    return cnt


def flex_algorithmic_work(x):
    w = x["workload"]
    cnt = flex_allowed_counts(x)
    pairs = int(cnt.sum()) * w.Hq
    flops = 4.0 * w.D * pairs
    nbytes = (w.B * w.S * w.Hq * w.D * 2            # q
              + 2 * w.B * w.S * w.Hkv * w.D * 2     # k, v
              + w.B * w.S * w.Hq * w.D * 2          # out (bf16)
              + w.B * w.S * w.Hq * 4                # lse
              + w.B * w.S * 4 + w.Hq * 4)           # tokens, sink weights
    return cnt, pairs, flops, nbytes


def traffic_from_profiles(workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if still current."""
    path = os.path.join(ROOT, "profiles", f"traffic_attn_fwd_kernel_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha256") != kernel_source_sha256():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(x, target_s: float, seed: int = 11):
    """The oracle as it stands, on a bounded random sample of the workload's rows.

    The sample grows by 4x from 64 rows until one timing is long enough to
    extrapolate from, then is sized to about ``target_s`` seconds.
    """
    import torch
    import oracle
    from transformer_attention_03_amd import workloads as W
    w = x["workload"]
    total = w.B * w.S
    n = min(64, total)
    while True:
        t, _ = oracle.timed_fwd(x, W.sample_rows(w.B, w.S, n, seed))
        if t >= target_s / 8 or n >= total:
            break
        n = min(total, n * 4)
    if n < total and t < 0.75 * target_s:
        n = int(min(total, max(n, n * target_s / max(t, 1e-9))))
    rows = torch.arange(total) if n >= total else W.sample_rows(w.B, w.S, n, seed + 1)
    t, _ = oracle.timed_fwd(x, rows)
    cnt = allowed_counts(x).reshape(-1)
    pairs = int(cnt[rows.numpy()].sum()) * w.Hq
    flops = 4.0 * w.D * pairs
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"{rows.numel()} {'(all)' if n >= total else 'random'} query rows of {total} (all {w.Hq} heads), {pairs} unmasked pairs, "
                      f"{t:.1f} s wall, fp64"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mall-flush", action="store_true",
                    help="do not flush the 256 MB MALL between timed steps (then ms_per_step is wall clock)")
    ap.add_argument("--mall-flush", choices=("read", "write"), default="write",
                    help="how the MALL is flushed before each timed step: a 512 MiB read or write")
    ap.add_argument("--backward", action="store_true",
                    help="time the gradients (attn_bwd) of the workload instead of the forward")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB mebibytes (calibrates HBM counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        src = torch.empty(args.copy_calibration << 20, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": src.numel()}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only (asked for --gpus {args.gpus}); "
              "a multi-GPU forward would shard by head group or by query range, which is not implemented.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from transformer_attention_03_amd import binding
    from transformer_attention_03_amd import workloads as W

    if args.workload in W.FLEX_WORKLOADS:
        return bench_flex(args)
    if args.workload in W.RELPROJ_WORKLOADS:
        return bench_relproj(args)
    if args.workload not in W.WORKLOADS:
        sys.exit(f"unknown workload {args.workload!r}; choose from {sorted(W.WORKLOADS) + sorted(W.FLEX_WORKLOADS)}")
    w = W.WORKLOADS[args.workload]
    x = W.generate(w)
    if args.backward:
        return bench_backward(args, w, x)
    cnt, pairs, flops, nbytes = algorithmic_work(x)

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    d = {k: (x[k].to(dev) if isinstance(x.get(k), torch.Tensor) else None)
         for k in ("q", "k", "v", "profiles", "sink", "valid", "positions")}
    out = torch.empty((w.B, w.S, w.Hq, w.D), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.S, w.Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(max(16, binding.attn_fwd_workspace_size(w.B, w.S, w.S, w.Hkv, w.D)), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream(dev)

    # the mask counts the kernels use must equal the closed form above
    dc = binding.attn_debug_counts(d["valid"], positions=d["positions"], window=w.window).cpu().numpy()
    if not np.array_equal(dc, cnt):
        sys.exit("allowed-key counts of the library and of the workload structure disagree")

    # The arguments are marshalled once: every step then launches the three
    # kernels with one C call each, so the host stays ahead of the GPU and the
    # events around the attention kernel time the kernel, not Python.
    plan, stage_values, attention, out, lse = binding.planned_forward_launchers(
        d["q"], d["k"], d["v"], d["profiles"], d["sink"], d["valid"], positions=d["positions"],
        window=w.window, out=out, lse=lse, workspace=ws, stream=stream)

    # The 256 MB MALL (last-level cache) would otherwise keep inputs of one step
    # for the next: a 512 MiB read or write before every step, outside the
    # step's events.
    flush = None if args.no_mall_flush else MallFlush(args.mall_flush, dev)

    def step(evs=None):
        if flush is not None:
            flush()
        if evs is not None:
            evs[0].record(stream)
        plan()
        stage_values()
        if evs is not None:
            evs[1].record(stream)
        attention()
        if evs is not None:
            evs[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3 / args.steps
    step_ms = float(np.mean([e[0].elapsed_time(e[2]) for e in evs]))
    # with the flush, a step's time is its own events' span (the flush is not the step's work)
    ms_step = step_ms if flush is not None else wall_ms
    kern_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    if not torch.isfinite(out).all():
        sys.exit("non-finite output")

    valid_tokens = int(x["valid"].sum())
    achieved = flops / (kern_ms * 1e-3) / 1e12
    line = {
        "metric": "fwd attention TFLOP/s (unmasked pairs) + % MFMA peak, 1 GPU; tokens/s",
        "value": flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B={w.B} S={w.S} Hq={w.Hq} Hkv={w.Hkv} D={w.D} E={w.E} "
                               f"window={w.window} profiles={str(w.profiles_dtype).replace('torch.', '')}",
                   "global_batch": w.B, "seq_len": w.S, "parallelism": "none (1 GPU)",
                   "qk_mfma": "bf16", "pv_mfma": "fp16", "accumulate": "fp32"},
        "timing": ("per-step HIP events (pre-pass, value copy, attention kernel); the MALL is flushed by "
                   f"{flush.describe() if flush is not None else ''} before each step, outside the events; wall clock over the "
                   f"{args.steps} steps, flushes included: {wall_ms:.4f} ms/step") if flush is not None else
                  "wall clock over the timed steps, no cache flush between them",
        "tokens_per_s": valid_tokens / (ms_step * 1e-3),
        "mfma_frac_step": flops / (ms_step * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS,
        "unmasked_pairs": pairs,
        "hbm_gbs_algorithmic": nbytes / (kern_ms * 1e-3) / 1e9,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / MFMA_PEAK_TFLOPS, "traffic": traffic_from_profiles(w.name),
                     "kernel": "attn_fwd_kernel", "kernel_ms": kern_ms,
                     "algorithmic_flops_per_launch": flops, "algorithmic_bytes_per_launch": nbytes},
    }
    if w.window:
        # window-bound shapes: the HBM roofline is the binding one
        gbs = nbytes / (kern_ms * 1e-3) / 1e9
        line["roofline"].update({"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": gbs / HBM_PEAK_GBS})
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(x, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def backward_work(x):
    """Algorithmic work of the gradients: 10 D flops per unmasked pair (q.k, dout.v, P^T dout,
    dS k and dS^T q, 2 D each); bytes: q, k, v (bf16), the profile entries the forward used,
    sink, out, lse, dout, dlse (fp32) read once; dq, dk, dv (fp32), the whole profile gradient
    (dtype of profiles) and dsink written once."""
    w = x["workload"]
    cnt, pairs, _, _ = algorithmic_work(x)
    flops = 10.0 * w.D * pairs
    pb = 2 if str(w.profiles_dtype).endswith("bfloat16") else 4
    rows = w.B * w.S * w.Hq
    nbytes = (2 * rows * w.D + 2 * 2 * w.B * w.S * w.Hkv * w.D + used_profile_entries(x) * w.Hq * pb
              + rows * 4 * (1 + w.D + 1 + w.D + 1)
              + 4 * rows * w.D + 2 * 4 * w.B * w.S * w.Hkv * w.D + rows * w.E * pb + 4 * rows)
    return cnt, pairs, flops, nbytes


def backward_cpu_baseline(x, dout, dlse, target_s: float):
    """The backward oracle as it stands, on the last rows of each sequence (the oracle's row
    range), grown until the run takes about ``target_s`` seconds."""
    import oracle
    w = x["workload"]
    cnt = allowed_counts(x)

    def timed(n):
        t0 = time.perf_counter()
        oracle.attn_bwd(x["q"], x["k"], x["v"], x["profiles"], x["sink"], x["valid"], dout, dlse,
                        positions=x["positions"], window=x["window"], row_lo=w.S - n)
        return time.perf_counter() - t0

    n = 8
    t = timed(n)
    while t < target_s / 8 and n < w.S:
        n = min(w.S, n * 4)
        t = timed(n)
    if n < w.S and t < 0.75 * target_s:
        n = int(min(w.S, max(n, n * target_s / max(t, 1e-9))))
        t = timed(n)
    pairs = int(cnt[:, w.S - n:].sum()) * w.Hq
    return {"value": 10.0 * w.D * pairs / t / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"last {n} query rows of each of {w.B} sequence(s) (all {w.Hq} heads), {pairs} unmasked "
                      f"pairs, {t:.1f} s wall, fp64, one thread"}


def bench_backward(args, w, x):
    """Gradients of the forward on workload ``w``: one step = one attn_bwd call (pre-pass, row
    statistics and transposed copies, the dQ / profile-gradient kernel and the dK / dV kernel),
    with the forward's out / lse and seeded upstream gradients already resident in HBM."""
    import torch
    from transformer_attention_03_amd import binding

    cnt, pairs, flops, nbytes = backward_work(x)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    d = {k: (x[k].to(dev) if isinstance(x.get(k), torch.Tensor) else None)
         for k in ("q", "k", "v", "profiles", "sink", "valid", "positions")}
    gen = torch.Generator().manual_seed(4242)
    dout_h = torch.randn(w.B, w.S, w.Hq, w.D, generator=gen)
    dlse_h = torch.randn(w.B, w.S, w.Hq, generator=gen)
    dout, dlse = dout_h.to(dev), dlse_h.to(dev)
    out, lse = binding.attn_fwd(d["q"], d["k"], d["v"], d["profiles"], d["sink"], d["valid"],
                                positions=d["positions"], window=w.window)
    grads = (torch.empty((w.B, w.S, w.Hq, w.D), dtype=torch.float32, device=dev),
             torch.empty((w.B, w.S, w.Hkv, w.D), dtype=torch.float32, device=dev),
             torch.empty((w.B, w.S, w.Hkv, w.D), dtype=torch.float32, device=dev),
             torch.empty((w.B, w.Hq, w.S, w.E), dtype=w.profiles_dtype, device=dev),
             torch.empty((w.B, w.S, w.Hq), dtype=torch.float32, device=dev))
    ws = torch.empty(max(16, binding.attn_bwd_workspace_size(w.B, w.S, w.S, w.Hq, w.Hkv, w.D)), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        binding.attn_bwd(d["q"], d["k"], d["v"], d["profiles"], d["sink"], d["valid"], out, lse, dout, dlse,
                         positions=d["positions"], window=w.window, grads=grads, workspace=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    call_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    if not all(bool(torch.isfinite(g.float()).all()) for g in grads):
        sys.exit("non-finite gradient")
    achieved = flops / (call_ms * 1e-3) / 1e12
    line = {
        "metric": "bwd attention TFLOP/s (unmasked pairs, 10*D flops per pair) + % MFMA peak, 1 GPU",
        "value": flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name} backward: B={w.B} S={w.S} Hq={w.Hq} Hkv={w.Hkv} D={w.D} E={w.E} "
                               f"window={w.window} profiles={str(w.profiles_dtype).replace('torch.', '')}",
                   "global_batch": w.B, "seq_len": w.S, "parallelism": "none (1 GPU)",
                   "mfma": "bf16", "accumulate": "fp32"},
        "unmasked_pairs": pairs,
        "hbm_gbs_algorithmic": nbytes / (call_ms * 1e-3) / 1e9,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / MFMA_PEAK_TFLOPS, "traffic": None,
                     "kernel": "attn_bwd call (pre-pass, prep, bwd_dq_kernel, bwd_dkdv_kernel)",
                     "kernel_ms": call_ms, "algorithmic_flops_per_launch": flops,
                     "algorithmic_bytes_per_launch": nbytes},
    }
    if w.window:
        # window-bound shapes (about 120 flops per algorithmic byte, under the 312 at which
        # the two peaks meet): the HBM roofline is the binding one, as for the forward
        gbs = nbytes / (call_ms * 1e-3) / 1e9
        line["roofline"].update({"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": gbs / HBM_PEAK_GBS})
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = backward_cpu_baseline(x, dout_h.double(), dlse_h.double(), args.cpu_seconds)
    print(json.dumps(line), flush=True)


def flex_cpu_baseline(x, target_s: float, seed: int = 11):
    """The generic flex oracle as it stands, on a bounded random sample of rows."""
    import torch
    import oracle
    from transformer_attention_03_amd import workloads as W
    w = x["workload"]
    total = w.B * w.S

    def timed(rows):
        t0 = time.perf_counter()
        oracle.flex_fwd(x["q"], x["k"], x["v"], x["sink_weights"], x["tokens"], x["eos_id"],
                        x["fixed_block_size"], x["sliding_window"], x["scale"], rows=rows)
        return time.perf_counter() - t0

    n = min(64, total)
    while True:
        t = timed(W.sample_rows(w.B, w.S, n, seed))
        if t >= target_s / 8 or n >= total:
            break
        n = min(total, n * 4)
    if n < total and t < 0.75 * target_s:
        n = int(min(total, max(n, n * target_s / max(t, 1e-9))))
    rows = torch.arange(total) if n >= total else W.sample_rows(w.B, w.S, n, seed + 1)
    t = timed(rows)
    cnt = flex_allowed_counts(x).reshape(-1)
    pairs = int(cnt[rows.numpy()].sum()) * w.Hq
    return {"value": 4.0 * w.D * pairs / t / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"{rows.numel()} {'(all)' if n >= total else 'random'} query rows of {total} "
                      f"(all {w.Hq} heads), {pairs} unmasked pairs, {t:.1f} s wall, fp64"}


def bench_flex(args):
    """The generic flex-attention forward (no relative term): one step = one
    flex_attn_fwd call (positions, pre-pass, value copy and attention kernel)."""
    import torch
    from transformer_attention_03_amd import binding
    from transformer_attention_03_amd import workloads as W

    w = W.FLEX_WORKLOADS[args.workload]
    x = W.generate_flex(w)
    cnt, pairs, flops, nbytes = flex_algorithmic_work(x)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    q, k, v = x["q"].to(dev), x["k"].to(dev), x["v"].to(dev)
    sw = None if x["sink_weights"] is None else x["sink_weights"].to(dev)
    tok = None if x["tokens"] is None else x["tokens"].to(dev)
    out = torch.empty((w.B, w.Hq, w.S, w.D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device=dev)
    ws = torch.empty(max(16, binding.flex_attn_workspace_size(w.B, w.S, w.S, w.Hkv, w.D)), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream(dev)

    # (arguments marshalled once: each step is one C call)
    step, out, lse = binding.flex_forward_launcher(q, k, v, sw, tok, x["eos_id"], x["fixed_block_size"],
                                                   x["sliding_window"], x["scale"], out=out, lse=lse,
                                                   workspace=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    call_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    if not torch.isfinite(out.float()).all():
        sys.exit("non-finite output")
    achieved = flops / (call_ms * 1e-3) / 1e12
    line = {
        "metric": "fwd attention TFLOP/s (unmasked pairs) + % MFMA peak, 1 GPU; tokens/s",
        "value": flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: generic flex forward, B={w.B} S={w.S} Hq={w.Hq} Hkv={w.Hkv} "
                               f"D={w.D} mask={w.mask} docs U{{{w.doc_min}..{w.doc_max}}} per-head sinks, "
                               f"bf16 output",
                   "global_batch": w.B, "seq_len": w.S, "parallelism": "none (1 GPU)",
                   "qk_mfma": "bf16", "pv_mfma": "fp16", "accumulate": "fp32"},
        "tokens_per_s": w.B * w.S / (ms_step * 1e-3),
        "mfma_frac_step": flops / (ms_step * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS,
        "unmasked_pairs": pairs,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / MFMA_PEAK_TFLOPS, "traffic": traffic_from_profiles(w.name),
                     "kernel": "flex_attn_fwd call (positions, pre-pass, value copy, attn_fwd_kernel)",
                     "kernel_ms": call_ms, "algorithmic_flops_per_launch": flops,
                     "algorithmic_bytes_per_launch": nbytes},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = flex_cpu_baseline(x, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def relproj_algorithmic_work(y):
    """Attention flops as for the profile workloads (4 D per unmasked pair); bytes with the
    relative features (d_rel bf16 per real row and head) and the table in place of the profile
    entries.  The producer's own flops (2 d_rel per profile entry used) are reported apart."""
    w = y["workload"]
    cnt = allowed_counts(y)
    pairs = int(cnt.sum()) * w.Hq
    flops = 4.0 * w.D * pairs
    valid_rows = int(y["valid"].sum())
    used = used_profile_entries(y, E=y["E"])
    nbytes = (valid_rows * w.Hq * w.D * 2 + valid_rows * w.Hkv * w.D * 2 * 2
              + valid_rows * w.Hq * y["d_rel"] * 2 + y["table"].numel() * 2
              + valid_rows * w.Hq * 4 + w.B * w.S * w.Hq * (w.D + 1) * 4 + w.B * w.S * (1 + 4))
    return cnt, pairs, flops, nbytes, 2.0 * y["d_rel"] * used * w.Hq


def bench_relproj(args):
    """The forward with its profile rows formed in the kernel (attn_fwd_relproj): one step = one
    call (pre-pass, value copy, attention kernel forming the rows from relative features)."""
    import torch
    from transformer_attention_03_amd import binding
    from transformer_attention_03_amd import workloads as W

    y = W.generate_relproj(args.workload)
    w = y["workload"]
    cnt, pairs, flops, nbytes, prod_flops = relproj_algorithmic_work(y)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    d = {k: y[k].to(dev) for k in ("q", "k", "v", "rfeat", "table", "sink", "valid", "positions")}
    out = torch.empty((w.B, w.S, w.Hq, w.D), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.S, w.Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(max(16, binding.attn_fwd_workspace_size(w.B, w.S, w.S, w.Hkv, w.D)), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        binding.attn_fwd_relproj(d["q"], d["k"], d["v"], d["rfeat"], d["table"], d["sink"], d["valid"],
                                 positions=d["positions"], window=w.window, out=out, lse=lse, workspace=ws,
                                 stream=stream)

    flush = None if args.no_mall_flush else MallFlush(args.mall_flush, dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in evs:
        if flush is not None:
            flush()
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    call_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    ms_step = call_ms if flush is not None else (t1 - t0) * 1e3 / args.steps
    if not torch.isfinite(out).all():
        sys.exit("non-finite output")
    gbs = nbytes / (call_ms * 1e-3) / 1e9
    tf = flops / (call_ms * 1e-3) / 1e12
    line = {
        "metric": "fwd attention TFLOP/s (unmasked pairs) + % MFMA peak, 1 GPU; tokens/s",
        "value": flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: B={w.B} S={w.S} Hq={w.Hq} Hkv={w.Hkv} D={w.D} E={w.E} "
                               f"window={w.window} profile rows formed in-kernel from d_rel={y['d_rel']} "
                               f"relative features and a table of {y['table'].shape[0]} slice(s)",
                   "global_batch": w.B, "seq_len": w.S, "parallelism": "none (1 GPU)",
                   "qk_mfma": "bf16", "pv_mfma": "fp16", "profile_mfma": "bf16", "accumulate": "fp32"},
        "tokens_per_s": int(y["valid"].sum()) / (ms_step * 1e-3),
        "unmasked_pairs": pairs,
        "producer_tflops": prod_flops / (call_ms * 1e-3) / 1e12,
        "hbm_gbs_algorithmic": gbs,
        "roofline": {"bound": "mfma", "achieved": tf, "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / MFMA_PEAK_TFLOPS, "traffic": None,
                     "kernel": "attn_fwd_relproj call (pre-pass, value copy, attn_fwd_kernel forming profile rows)",
                     "kernel_ms": call_ms, "algorithmic_flops_per_launch": flops,
                     "algorithmic_bytes_per_launch": nbytes,
                     "mfma_frac_with_producer": (flops + prod_flops) / (call_ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
