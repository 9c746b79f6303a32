#!/usr/bin/env python3
"""Fused-group HBM throughput on one MI355X.

One step = the AdamW step over the Llama-style parameter tree (145 leaves,
887 685 120 parameters, bf16 theta/g, f32 m/v, one launch for every leaf)
followed by the causal row softmax over f32 scores [8,16,1024,1024]
(131 072 rows x 1024: scale, causal mask, row max, subtract, exp, row sum,
divide; one launch).  Inputs are seeded synthetic tensors, resident in HBM
before timing starts.

`value` is the step's algorithmic bytes (AdamW: 22 B per parameter;
softmax: allowed scores read once + every output written once) divided by
the measured time per step, in GB/s.  The roofline object is for the
dominant kernel (AdamW), timed with HIP events on the stream it runs on.
Every other workload (the step's two kernels alone, the clipped cosine
AdamW, a 22-layer tree, the tiny-GPT tree cold, warm and graph-replayed,
the tree-mapped SGD and AdamW groups, RMSNorm+GELU with and without h
stored, LayerNorm with its statistics, the byte-mask, bf16 and wide
softmaxes (exact and online), the 64-node chain, torch's device copy and
an emitted copy) is timed on its own with the cache flushed between calls and reported under
"groups" (median, min, max of --reps calls).  The CPU baseline runs the
oracle single-threaded on the same step (inputs drawn on the host).

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=16, help="Llama-style tree depth (16: the explicit leaf list)")
    ap.add_argument("--reps", type=int, default=21, help="calls per workload in the per-group timing")
    ap.add_argument("--no-groups", action="store_true", help="skip the per-group timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=float, default=1.0, help="fraction of the step the oracle times")
    ap.add_argument("--profile-step", action="store_true",
                    help="run warmup + K steps only (for rocprofv3 runs), no per-group timing, no CPU leg")
    ap.add_argument("--pmc-calib", action="store_true",
                    help="first run one 1 GiB device copy, a known-size reference for the HBM byte counters")
    ap.add_argument("--profile-all", action="store_true",
                    help="with --profile-step: after the steps run each other workload twice (for rocprofv3)")
    return ap.parse_args()


def gb(nbytes, ms):
    return nbytes / (ms * 1e-3) / 1e9


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: each GPU would run the same kernels on "
                                   "its own share of rows, elements or leaves, with no exchange inside the step, "
                                   "so no multi-GPU figure is produced",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0 or args.reps < 1 or not (0.0 < args.cpu_sample <= 1.0):
        print(json.dumps({"error": "--steps and --reps must be at least 1, --warmup at least 0, "
                                   "--cpu-sample in (0, 1]"}))
        sys.exit(2)

    import torch
    import elementwise_reduction_groups_amd as P
    from synth import configs

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    HP = configs.ADAMW_HP
    hp = (HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"], HP["t"])

    # ---------------------------------------------------------------- inputs
    shapes = [s for _, s in configs.llama_leaves(L=args.layers)]
    n_params = sum(math.prod(s) for s in shapes)
    state = configs.adamw_state(shapes, theta_dtype=torch.bfloat16, grad_dtype=torch.bfloat16,
                                mv_dtype=torch.float32, device=dev, seed=configs.SEED_BASE + 2)
    tree = P.Tree([[s["theta"], s["grad"], s["m"], s["v"]] for s in state])
    adamw_bytes = n_params * (2 + 2 + 4 + 4 + 2 + 4 + 4)

    R, C = 131072, 1024
    scores = configs.softmax_scores(R, C, device=dev)
    probs = torch.empty_like(scores)
    softmax = P.Group(configs.softmax_causal_dag(0.125, 1024), [((R, C), "f32")], (R, C), "f32")
    allowed = sum(min(r % 1024, C - 1) + 1 for r in range(1024)) * (R // 1024)
    softmax_bytes = allowed * 4 + R * C * 4
    step_bytes = adamw_bytes + softmax_bytes
    torch.cuda.synchronize()
    if args.pmc_calib:
        # 2^28 f32 = 1 GiB read and 1 GiB written by one torch copy kernel
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        tree.adamw_step(*hp, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        softmax.run([scores], probs, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    ms_per_step = wall_ms / args.steps
    adamw_ms = [e[0].elapsed_time(e[1]) for e in events]
    softmax_ms = [e[1].elapsed_time(e[2]) for e in events]
    adamw_avg = statistics.fmean(adamw_ms)
    value = gb(step_bytes, ms_per_step)

    result = {
        "metric": "fused-group HBM GB/s (AdamW tree step, row softmax) and % of MI355X peak",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 arithmetic; bf16/f32 storage",
        "data": "synthetic (seeded), resident in HBM",
        "config": {
            "workload": "AdamW step over a Llama-style tree (16 layers, D=2048, FFN 5632, vocab 32000: 145 leaves, "
                        "887685120 params; bf16 theta/g, f32 m/v) + causal row softmax f32 [8,16,1024,1024]",
            "params": n_params, "leaves": len(shapes), "softmax_rows": R, "softmax_cols": C,
            "step_bytes": step_bytes, "adamw_bytes": adamw_bytes, "softmax_bytes": softmax_bytes,
        },
        "frac_of_peak": round(value / HBM_PEAK_GBS, 4),
        "roofline": {
            "kernel": "adamw_tree_kernel<bf16,bf16,f32>",
            "bound": "hbm",
            "achieved": round(gb(adamw_bytes, adamw_avg), 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gb(adamw_bytes, adamw_avg) / HBM_PEAK_GBS, 4),
            "traffic": None,
            "avg_ms": round(adamw_avg, 4),
            "bytes_per_launch": adamw_bytes,
        },
        "env": {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None),
                "numpy": __import__("numpy").__version__, "device": torch.cuda.get_device_name(dev),
                "library_version": P.psk_version()},
        "kernels": {
            "adamw_ms_median": round(statistics.median(adamw_ms), 4),
            "softmax_ms_median": round(statistics.median(softmax_ms), 4),
            "softmax_GBps": round(gb(softmax_bytes, statistics.median(softmax_ms)), 1),
        },
    }
    traffic = committed_traffic()
    if traffic is not None:
        result["roofline"]["traffic"] = traffic
    if args.profile_step:
        if args.profile_all:
            profile_others(P, configs, torch, dev, stream, hp, state)
        print(json.dumps(result), flush=True)
        return

    # ----------------------------------------------------- per-group timing
    if not args.no_groups:
        result["groups"] = time_groups(args, P, configs, torch, dev, stream, tree, softmax, scores, probs,
                                       adamw_bytes, softmax_bytes, hp, state)
        # each HBM-bound group against the emitted r1:w1 copy measured in the
        # same run (a practical streaming rate, not the published peak)
        ref = result["groups"].get("copy_emitted", {}).get("GBps")
        if ref:
            for name, g in result["groups"].items():
                if name not in ("copy_emitted", "copy_ceiling", "chain64_f32", "adamw_tiny_gpt_f32"):
                    g["frac_of_emitted_copy"] = round(g["GBps"] / ref, 3)

    # ------------------------------------------------ static dispatch counts
    result["dispatch"] = dispatch_report(P, configs)

    # ------------------------------------------------------------ CPU leg
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, configs, n_params, shapes, R, C, step_bytes)

    print(json.dumps(result), flush=True)


ADAMW_COUNTERS = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                              "adamw_tree_kernel_llama16_bf16.txt")
ADAMW_SOURCES = ["elementwise_reduction_groups_amd/csrc/adamw.hip", "elementwise_reduction_groups_amd/csrc/psk_internal.h"]


def kernel_source_sha(paths):
    """SHA-256 of the AdamW kernel's source: adamw.hip whole, and of the
    shared header only its AdamW section (the structures the kernel reads)."""
    import hashlib
    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    for rel in paths:
        with open(os.path.join(root, rel), "rb") as f:
            data = f.read()
        if rel.endswith(".h"):
            text = data.decode()
            a = text.index("// ------------------------------------------------------------------ AdamW")
            b = text.index("// --------------------------------------------------------------- counters")
            data = text[a:b].encode()
        h.update(data)
    return h.hexdigest()


def committed_traffic():
    """HBM bytes per AdamW launch from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, calibrated on a copy kernel), or None when the
    kernel source has changed since the counters were taken."""
    try:
        kv = {}
        for line in open(ADAMW_COUNTERS):
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
        if kv.get("kernel_source_sha256") != kernel_source_sha(ADAMW_SOURCES):
            return None
        return int(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def tree_sgd(P, configs, torch, dev, state):
    """theta' = theta - lr * g as a generic tree-mapped group over the theta
    and g buffers of the Llama tree (in place; 6 bytes per parameter)."""
    tree = P.Tree([[s["theta"], s["grad"]] for s in state])
    group = P.Group(configs.tree_sgd_dag(), [((1,), "bf16"), ((1,), "bf16"), ((), "f32")], (1,), "bf16", tree=True)
    return tree, group, torch.tensor(1e-4, dtype=torch.float32, device=dev)


def dispatch_report(P, configs):
    """Launches and bytes of a synthetic GPT forward (the corpus GPT's sizes)
    before and after the partition, with reductions ending groups and with
    rows fused; and of the AdamW step over the tiny GPT's tree."""
    from synth.body import gpt_forward
    b = gpt_forward(V=92, D=64, H=2, L=2, B=2, T=32)
    out = {"gpt_forward_V92_D64_H2_L2_B2_T32": {
        "reductions_end_groups": P.psk_dispatch_count(b.nodes, b.types, b.outputs),
        "rows_fused": P.psk_dispatch_count(b.nodes, b.types, b.outputs, rows=True)}}
    dag = configs.adamw_group_dag()
    lets = sum(1 for n in dag if n.op not in ("input", "const"))
    leaves = len(configs.tiny_gpt_leaves())
    out["adamw_tiny_gpt_tree"] = {"leaves": leaves, "lets_per_leaf": lets,
                                  "launches_unfused": lets * leaves, "launches_one_per_leaf": leaves,
                                  "launches_one_per_tree": 1}
    return out


def layernorm_group(P, configs):
    R, C = 16384, 4096
    return P.Group(configs.layernorm_dag(configs.f32(1e-5)), [((R, C), "bf16"), ((C,), "bf16"), ((C,), "bf16")],
                   (R, C), "bf16", root=configs.LAYERNORM_ROOT,
                   extras=[(configs.LAYERNORM_MEAN, (R, 1), "f32"), (configs.LAYERNORM_RSTD, (R, 1), "f32")])


def adamw_group(P, configs, torch, dev, state, hp):
    """The AdamW step written as a group (m', v' stored, theta' the root),
    mapped over the Llama tree in place; the nine f32 step scalars are
    formed on the host in f64 and rounded once, as the library does."""
    import numpy as np
    b1, b2, t = hp[1], hp[2], hp[5]
    sc = np.array([b1, b2, 1 - b1, 1 - b2, 1 - b1 ** t, 1 - b2 ** t, hp[0], hp[3], hp[4]], np.float64)
    scal = torch.from_numpy(sc.astype(np.float32)).to(dev)
    grp = P.Group(configs.adamw_group_dag(), [((1,), "bf16"), ((1,), "bf16"), ((1,), "f32"), ((1,), "f32")] +
                  [((), "f32")] * 9, (1,), "bf16", tree=True,
                  extras=[(configs.ADAMW_GROUP_M, (1,), "f32"), (configs.ADAMW_GROUP_V, (1,), "f32")])
    tree = P.Tree([[s["theta"], s["grad"], s["m"], s["v"]] for s in state])
    args = (tree, [0, 1, 2, 3] + [-1] * 9, [0, 2, 3], [None] * 4 + [scal[i] for i in range(9)])
    grp._keep = (tree, scal)
    return grp, args


def profile_others(P, configs, torch, dev, stream, hp, state):
    tiny_shapes = [s for _, s in configs.tiny_gpt_leaves()]
    tiny = configs.adamw_state(tiny_shapes, device=dev, seed=configs.SEED_BASE)
    tiny_tree = P.Tree([[s["theta"], s["grad"], s["m"], s["v"]] for s in tiny])
    x, r, g = configs.rmsnorm_inputs(16384, 4096, device=dev)
    y = torch.empty_like(x)
    rms = P.Group(configs.rmsnorm_gelu_dag(configs.f32(1e-5)),
                  [((16384, 4096), "bf16"), ((16384, 4096), "bf16"), ((4096,), "bf16")], (16384, 4096), "bf16")
    A, B, Cc = configs.chain_inputs(16384, 16384, device=dev)
    Z = torch.empty_like(A)
    chain = P.Group(configs.chain64_dag(), [((16384, 16384), "f32"), ((16384, 1), "f32"), ((1, 16384), "f32")],
                    (16384, 16384), "f32")
    sgd_tree, sgd, lr = tree_sgd(P, configs, torch, dev, state)
    xl, gl, bl = configs.layernorm_inputs(16384, 4096, device=dev)
    yl = torch.empty_like(xl)
    ml = torch.empty((16384, 1), device=dev)
    rl = torch.empty((16384, 1), device=dev)
    ln = layernorm_group(P, configs)
    adamw_g, adamw_args = adamw_group(P, configs, torch, dev, state, hp)
    xs = configs.softmax_scores(131072, 1024, device=dev)
    ys = torch.empty_like(xs)
    mask = configs.causal_mask_bytes(1024, device=dev)
    masked = P.Group(configs.softmax_masked_dag(0.125), [((8, 16, 1024, 1024), "f32"), ((1024, 1024), "u8")],
                     (8, 16, 1024, 1024), "f32")
    sb = xs.to(torch.bfloat16)
    pb = torch.empty_like(sb)
    soft_bf16 = P.Group(configs.softmax_causal_dag(0.125, 1024), [((131072, 1024), "bf16")], (131072, 1024), "bf16")
    xw = configs.softmax_scores(8192, 131072, device=dev)
    yw = torch.empty_like(xw)
    wide = P.Group(configs.softmax_dag(0.125), [((8192, 131072), "f32")], (8192, 131072), "f32")
    wide_online = P.Group(configs.softmax_dag(0.125), [((8192, 131072), "f32")], (8192, 131072), "f32", online=True)
    rms_h = P.Group(configs.rmsnorm_gelu_dag(configs.f32(1e-5)),
                    [((16384, 4096), "bf16"), ((16384, 4096), "bf16"), ((4096,), "bf16")], (16384, 4096), "bf16",
                    extras=[(configs.RMSNORM_H, (16384, 4096), "bf16")])
    rh = r.clone()
    torch.cuda.synchronize()
    for _ in range(2):
        rms_h.run([x, rh, g], y, stream=stream, extra_outs=[rh])
        sgd.run_tree(sgd_tree, [0, 1, -1], 0, [None, None, lr], stream=stream)
        ln.run([xl, gl, bl], yl, stream=stream, extra_outs=[ml, rl])
        adamw_g.run_tree(*adamw_args, stream=stream)
        masked.run([xs.view(8, 16, 1024, 1024), mask], ys.view(8, 16, 1024, 1024), stream=stream)
        soft_bf16.run([sb], pb, stream=stream)
        wide.run([xw], yw, stream=stream)
        wide_online.run([xw], yw, stream=stream)
        tiny_tree.adamw_step(*hp, stream=stream)
        rms.run([x, r, g], y, stream=stream)
        chain.run([A, B, Cc], Z, stream=stream)
    torch.cuda.synchronize()


def time_groups(args, P, configs, torch, dev, stream, tree, softmax, scores, probs, adamw_bytes, softmax_bytes, hp,
                state):
    """Each workload alone: a 1 GiB write between calls evicts the 256 MB
    last-level cache; HIP events around each call; median of --reps."""
    R, C = scores.shape
    allowed = sum(min(r % 1024, C - 1) + 1 for r in range(1024)) * (R // 1024)
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)

    def timed(fn, reps):
        ms = []
        for _ in range(reps + 2):
            flush.zero_()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            ms.append(a.elapsed_time(b))
        ms = ms[2:]
        return statistics.median(ms), min(ms), max(ms)

    out = {}

    def add(name, nbytes, fn, note=None):
        med, lo, hi = timed(fn, args.reps)
        out[name] = {"ms_median": round(med, 4), "ms_min": round(lo, 4), "ms_max": round(hi, 4),
                     "bytes": nbytes, "GBps": round(gb(nbytes, med), 1),
                     "frac_of_peak": round(gb(nbytes, med) / HBM_PEAK_GBS, 4)}
        if note:
            out[name]["note"] = note

    add("adamw_llama_bf16", adamw_bytes, lambda: tree.adamw_step(*hp, stream=stream))
    # depth sensitivity: the same architecture at 22 layers (199 leaves, 1 195 991 040 params)
    if args.layers != 22:
        shapes22 = [s for _, s in configs.llama_leaves(L=22)]
        n22 = sum(math.prod(s) for s in shapes22)
        st22 = configs.adamw_state(shapes22, theta_dtype=torch.bfloat16, grad_dtype=torch.bfloat16,
                                   mv_dtype=torch.float32, device=dev, seed=configs.SEED_BASE + 12)
        tree22 = P.Tree([[s["theta"], s["grad"], s["m"], s["v"]] for s in st22])
        add("adamw_llama22_bf16", 22 * n22, lambda: tree22.adamw_step(*hp, stream=stream),
            note=f"22 layers: {len(shapes22)} leaves, {n22} params")
        del tree22, st22
        torch.cuda.empty_cache()
    add("softmax_causal_f32", softmax_bytes, lambda: softmax.run([scores], probs, stream=stream))
    # the same tree with global-norm clipping and a cosine schedule: a
    # sum-of-squares pass over g (2 B/param more) and the step
    n_params = adamw_bytes // 22
    add("adamw_llama_bf16_clip_cosine", adamw_bytes + 2 * n_params,
        lambda: tree.adamw_step(*hp, stream=stream, total=1000, warmup=100, schedule="cosine", grad_clip=1.0),
        note="three launches: per-chunk sums of squares (f64), a one-workgroup combine, the clipped step")

    # a generic group mapped over the same tree: plain SGD on theta (bf16)
    sgd_tree, sgd, lr = tree_sgd(P, configs, torch, dev, state)
    add("tree_sgd_llama_bf16", 6 * n_params, lambda: sgd.run_tree(sgd_tree, [0, 1, -1], 0, [None, None, lr],
                                                                   stream=stream),
        note="emitted tree-mapped group: theta' = theta - lr * g, lr a device scalar")

    # tiny GPT tree, f32
    tiny_shapes = [s for _, s in configs.tiny_gpt_leaves()]
    tiny = configs.adamw_state(tiny_shapes, device=dev, seed=configs.SEED_BASE)
    tiny_tree = P.Tree([[s["theta"], s["grad"], s["m"], s["v"]] for s in tiny])
    n_tiny = sum(math.prod(s) for s in tiny_shapes)
    add("adamw_tiny_gpt_f32", n_tiny * 28, lambda: tiny_tree.adamw_step(*hp, stream=stream),
        note="3 MB: launch-latency bound, no HBM target; ms_* cold (cache flushed), us_warm_median back to back, "
             "us_per_step_graph_of_20: 20 steps captured in one HIP graph")
    warm = []
    for k in range(args.reps + 2):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        tiny_tree.adamw_step(*hp, stream=stream)
        b.record(stream)
        b.synchronize()
        if k >= 2:
            warm.append(a.elapsed_time(b))
    out["adamw_tiny_gpt_f32"]["us_warm_median"] = round(statistics.median(warm) * 1e3, 2)
    # launch-bound: 20 steps captured in one HIP graph, replayed back to back
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(20):
            tiny_tree.adamw_step(*hp)
    torch.cuda.synchronize()
    per_step = []
    for k in range(args.reps + 2):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        graph.replay()
        b.record()
        b.synchronize()
        if k >= 2:
            per_step.append(a.elapsed_time(b) / 20)
    out["adamw_tiny_gpt_f32"]["us_per_step_graph_of_20"] = round(statistics.median(per_step) * 1e3, 2)

    # add + RMSNorm + gamma + GELU, bf16 [16384, 4096]
    x, r, g = configs.rmsnorm_inputs(16384, 4096, device=dev)
    y = torch.empty_like(x)
    rms = P.Group(configs.rmsnorm_gelu_dag(configs.f32(1e-5)),
                  [((16384, 4096), "bf16"), ((16384, 4096), "bf16"), ((4096,), "bf16")], (16384, 4096), "bf16")
    add("rmsnorm_gelu_bf16", rms.info.algorithmic_bytes, lambda: rms.run([x, r, g], y, stream=stream))

    # softmax variants over [8, 16, 1024, 1024] scores: a [1024, 1024] byte
    # mask (causal pattern) read from memory, and bf16 scores and probabilities
    xs4 = scores.view(8, 16, 1024, 1024)
    mask = configs.causal_mask_bytes(1024, device=dev)
    masked = P.Group(configs.softmax_masked_dag(0.125), [((8, 16, 1024, 1024), "f32"), ((1024, 1024), "u8")],
                     (8, 16, 1024, 1024), "f32")
    add("softmax_mask_buffer_f32", allowed * 4 + R * C * 4 + 1024 * 1024,
        lambda: masked.run([xs4, mask], probs.view(8, 16, 1024, 1024), stream=stream),
        note="the scores the mask allows read (vectors it refuses are not loaded), the mask once, "
             "probabilities written")
    sb = scores.to(torch.bfloat16)
    pb = torch.empty_like(sb)
    soft_bf16 = P.Group(configs.softmax_causal_dag(0.125, 1024), [((R, C), "bf16")], (R, C), "bf16")
    add("softmax_causal_bf16", allowed * 2 + R * C * 2, lambda: soft_bf16.run([sb], pb, stream=stream))
    del sb, pb
    # wide rows: the tiled kernel re-reads the row in each phase
    xw = configs.softmax_scores(8192, 131072, device=dev)
    yw = torch.empty_like(xw)
    wide = P.Group(configs.softmax_dag(0.125), [((8192, 131072), "f32")], (8192, 131072), "f32")
    add("softmax_wide_8192x131072_f32", 2 * xw.numel() * 4, lambda: wide.run([xw], yw, stream=stream),
        note="tiled kernel, 512 lanes a row: 3 phases walk it, the leading tiles from registers, the rest re-read; bytes counted once")
    wide_online = P.Group(configs.softmax_dag(0.125), [((8192, 131072), "f32")], (8192, 131072), "f32", online=True)
    add("softmax_wide_8192x131072_f32_online", 2 * xw.numel() * 4, lambda: wide_online.run([xw], yw, stream=stream),
        note="PSK_GROUP_ONLINE: the sum taken in the maximum's pass (2 phases); its rounding differs from the exact "
             "sum (declared differs, within the f32 tolerance)")
    del xw, yw

    # layer normalization with its row statistics, bf16 [16384, 4096]: one
    # kernel, two reduction phases, three outputs
    xl, gl, bl = configs.layernorm_inputs(16384, 4096, device=dev)
    yl = torch.empty_like(xl)
    ml = torch.empty((16384, 1), device=dev)
    rl = torch.empty((16384, 1), device=dev)
    ln = layernorm_group(P, configs)
    add("layernorm_stats_bf16", ln.info.algorithmic_bytes,
        lambda: ln.run([xl, gl, bl], yl, stream=stream, extra_outs=[ml, rl]),
        note="mean, x - mean read twice, variance, normalise; mean and rstd stored per row")

    # add + RMSNorm + gamma + GELU that also stores h = x + res in place over res
    rms_h = P.Group(configs.rmsnorm_gelu_dag(configs.f32(1e-5)),
                    [((16384, 4096), "bf16"), ((16384, 4096), "bf16"), ((4096,), "bf16")], (16384, 4096), "bf16",
                    extras=[(configs.RMSNORM_H, (16384, 4096), "bf16")])
    add("add_rmsnorm_gelu_store_h_bf16", rms_h.info.algorithmic_bytes,
        lambda: rms_h.run([x, r, g], y, stream=stream, extra_outs=[r]), note="h written in place over the residual")

    # the AdamW step as an emitted three-output tree-mapped group
    adamw_g, adamw_args = adamw_group(P, configs, torch, dev, state, hp)
    add("adamw_llama_bf16_emitted_group", adamw_bytes, lambda: adamw_g.run_tree(*adamw_args, stream=stream),
        note="the generic tree-mapped group path; bit-identical to the hand-written kernel")

    # 64-node chain over [16384, 16384]
    A, B, Cc = configs.chain_inputs(16384, 16384, device=dev)
    Z = torch.empty_like(A)
    chain = P.Group(configs.chain64_dag(), [((16384, 16384), "f32"), ((16384, 1), "f32"), ((1, 16384), "f32")],
                    (16384, 16384), "f32")
    add("chain64_f32", chain.info.algorithmic_bytes, lambda: chain.run([A, B, Cc], Z, stream=stream),
        note="ALU-bound: 64 node evaluations per element")
    out["chain64_f32"]["node_evals_per_s"] = round(64 * 16384 * 16384 / (out["chain64_f32"]["ms_median"] * 1e-3), 1)

    # streaming copies of 1 GiB read + 1 GiB written: torch's device copy, and
    # the emitted pointwise kernel of y = -(-x) (bit-exact copy; nontemporal
    # 16-byte accesses), the plain r1:w1 stream of this library's kernels
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    add("copy_ceiling", 2 * src.numel() * 4, lambda: dst.copy_(src), note="torch device copy, read+write")
    from synth.dag import parse_dag
    copy = P.Group(parse_dag("%0 = input 0\n%1 = neg %0\n%2 = neg %1\n"), [((src.numel(),), "f32")],
                   (src.numel(),), "f32")
    add("copy_emitted", 2 * src.numel() * 4, lambda: copy.run([src], dst, stream=stream),
        note="emitted pointwise y = -(-x): the r1:w1 streaming rate of an emitted kernel")
    del flush, src, dst
    return out


def cpu_baseline(args, configs, n_params, shapes, R, C, step_bytes):
    """The oracle, single-threaded, on a fixed fraction of the step's work:
    the first leaves of the same tree up to that fraction of its parameters
    (drawn on the host with the same distributions) and that fraction of the
    softmax rows.  Reported as GB/s of the same algorithmic-bytes count."""
    import numpy as np
    import torch
    import oracle

    torch.set_num_threads(max(1, os.cpu_count() or 1))
    f = args.cpu_sample
    target = int(n_params * f)
    take, tot = [], 0
    for s in shapes:
        if tot >= target:
            break
        take.append(s)
        tot += math.prod(s)
    st = configs.adamw_state(take, theta_dtype=torch.bfloat16, grad_dtype=torch.bfloat16, mv_dtype=torch.float32,
                             device="cpu", seed=configs.SEED_BASE + 2)
    u16 = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    HP = configs.ADAMW_HP
    t0 = time.perf_counter()
    for s in st:
        oracle.adamw(u16(s["theta"]), u16(s["grad"]), s["m"].numpy(), s["v"].numpy(), HP["lr"], HP["beta1"],
                     HP["beta2"], HP["eps"], HP["weight_decay"], HP["t"])
    t_adamw = time.perf_counter() - t0
    rows = max(1024, int(R * f) // 1024 * 1024)
    x = configs.softmax_scores(rows, C).numpy()
    t0 = time.perf_counter()
    oracle.softmax_causal(x, 1024, 0.125)
    t_soft = time.perf_counter() - t0
    adamw_b = tot * 22
    soft_b = (rows // 1024) * sum(min(q, C - 1) + 1 for q in range(1024)) * 4 + rows * C * 4
    secs = t_adamw + t_soft
    return {"value": round((adamw_b + soft_b) / secs / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{tot} of {n_params} AdamW parameters ({len(take)} leaves) + {rows} of {R} softmax rows; "
                      f"{secs:.1f} s single-threaded",
            "seconds": round(secs, 2), "cpu_model": _cpu_model(), "host_cpus": os.cpu_count()}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
