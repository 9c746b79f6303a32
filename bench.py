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

Every workload of the registry (build_workloads) is also timed on its own,
with the last-level cache flushed between calls, and reported under
"groups": the median of --reps calls in each of --procs processes (this
one and --procs - 1 children run one after another), with the median of
the processes' medians, the extremes over all calls, and each process's
median.  The CPU baseline times the oracle over every workload on one
host thread and on all of them (at most 16, a GPU machine's share), on the GPU
run's own inputs copied to the host.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--procs P]

Measurement helpers (the commands that made the summaries in profiles/):
    python bench.py --profile-step --profile-all ...   under rocprofv3
    python bench.py --summarize-profiles DIR           writes profiles/*.txt
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import subprocess
import sys
import time

HBM_PEAK_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=16, help="Llama-style tree depth (16: the explicit leaf list)")
    ap.add_argument("--reps", type=int, default=21, help="calls per workload in the per-group timing")
    ap.add_argument("--procs", type=int, default=3, help="processes the per-group timing runs in")
    ap.add_argument("--no-groups", action="store_true", help="skip the per-group timing")
    ap.add_argument("--only", default="", help="comma-separated workload names to time (default: all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=16, help="most host threads the CPU leg uses")
    ap.add_argument("--profile-step", action="store_true",
                    help="run warmup + K steps only (for rocprofv3 runs), no per-group timing, no CPU leg")
    ap.add_argument("--pmc-calib", action="store_true",
                    help="first run one 1 GiB device copy, a known-size reference for the HBM byte counters")
    ap.add_argument("--profile-all", action="store_true",
                    help="with --profile-step: after the steps run each workload of the registry twice")
    ap.add_argument("--groups-only", metavar="JSON", default="",
                    help="(child process) time the workloads only and write their timings to this file")
    ap.add_argument("--summarize-profiles", metavar="DIR", default="",
                    help="write profiles/*.txt from the rocprofv3 output under DIR (no GPU needed)")
    return ap.parse_args(argv)


def gb(nbytes, ms):
    return nbytes / (ms * 1e-3) / 1e9


def allowed_causal(R, C, T=1024):
    """Scores a causal mask of period T allows in an [R, C] view."""
    return sum(min(r % T, C - 1) + 1 for r in range(T)) * (R // T) + \
        sum(min(r % T, C - 1) + 1 for r in range(R % T))


# ---------------------------------------------------------------- registry
class Workload:
    """One workload timed on its own.  `group` builds the emitted group (no
    GPU needed: its kernel name is what the profiler shows), or `kernel`
    names the hand-written kernel; `setup(ctx)` allocates its inputs on the
    device and returns the call to time.  Bytes are algorithmic: each input
    read once at its own size, each output written once."""

    def __init__(self, name, profile, read, write, setup, group=None, kernel=None, note=None, hbm=True,
                 node_evals=0, size_copy=None):
        self.name, self.profile, self.read, self.write = name, profile, read, write
        self.setup, self.group, self.kernel, self.note, self.hbm = setup, group, kernel, note, hbm
        self.node_evals = node_evals
        self.size_copy = size_copy      # an emitted copy moving about the same bytes, timed alongside

    @property
    def bytes(self):
        return self.read + self.write


class Ctx:
    """What the workloads share: the library, the generators, the device,
    the stream, the step's AdamW state and hyperparameters."""

    def __init__(self, P, configs, torch, dev, stream, hp, state=None, layers=16):
        self.P, self.configs, self.torch, self.dev, self.stream, self.hp = P, configs, torch, dev, stream, hp
        self.state, self.layers = state, layers

    def llama_state(self):
        if self.state is None:
            C, torch = self.configs, self.torch
            shapes = [s for _, s in C.llama_leaves(L=self.layers)]
            self.state = C.adamw_state(shapes, theta_dtype=torch.bfloat16, grad_dtype=torch.bfloat16,
                                       mv_dtype=torch.float32, device=self.dev, seed=C.SEED_BASE + 2)
        return self.state


def _llama_n(configs, L=16):
    return sum(math.prod(s) for _, s in configs.llama_leaves(L=L))


def _tiny_n(configs):
    return sum(math.prod(s) for _, s in configs.tiny_gpt_leaves())


# the hand-written AdamW kernels as the kernel trace names them (mangled or
# demangled): any of the alternatives identifies the kernel
BF16_ADAMW = ("adamw_tree_kernelIDF16bDF16bfLb0E", "adamw_tree_kernel<__bf16, __bf16, float, false>")
F32_ADAMW = ("adamw_tree_kernelIfffLb0E", "adamw_tree_kernel<float, float, float, false>")


def build_workloads(P, configs, layers=16):
    C = configs
    eps = C.f32(1e-5)
    n = _llama_n(C, layers)
    n22 = _llama_n(C, 22)
    R1, C1 = 131072, 1024
    a1 = allowed_causal(R1, C1)
    R3, C3 = 16384, 4096
    N4 = 16384
    RW, CW = 8192, 131072
    W = []

    def tree_of(ctx, state):
        return ctx.P.Tree([[s["theta"], s["grad"], s["m"], s["v"]] for s in state])

    # -- AdamW, hand-written tree kernel
    def s_adamw(ctx):
        tree = tree_of(ctx, ctx.llama_state())
        return lambda: tree.adamw_step(*ctx.hp, stream=ctx.stream)
    W.append(Workload("adamw_llama_bf16", "adamw_tree_kernel_llama16_bf16", 12 * n, 10 * n, s_adamw,
                      kernel=BF16_ADAMW))

    def s_adamw22(ctx):
        shapes = [s for _, s in ctx.configs.llama_leaves(L=22)]
        st = ctx.configs.adamw_state(shapes, theta_dtype=ctx.torch.bfloat16, grad_dtype=ctx.torch.bfloat16,
                                     mv_dtype=ctx.torch.float32, device=ctx.dev, seed=ctx.configs.SEED_BASE + 12)
        tree = tree_of(ctx, st)
        return lambda: tree.adamw_step(*ctx.hp, stream=ctx.stream)
    W.append(Workload("adamw_llama22_bf16", None, 12 * n22, 10 * n22, s_adamw22,
                      kernel=BF16_ADAMW,
                      note=f"22 layers: 199 leaves, {n22} params (depth sensitivity)"))

    def s_clip(ctx):
        tree = tree_of(ctx, ctx.llama_state())
        return lambda: tree.adamw_step(*ctx.hp, stream=ctx.stream, total=1000, warmup=100, schedule="cosine",
                                       grad_clip=1.0)
    W.append(Workload("adamw_llama_bf16_clip_cosine", None, 14 * n, 10 * n, s_clip,
                      note="three launches: per-chunk sums of squares (f64), a one-workgroup combine, the "
                           "clipped step"))

    def g_sgd():
        return P.Group(C.tree_sgd_dag(), [((1,), "bf16"), ((1,), "bf16"), ((), "f32")], (1,), "bf16", tree=True)

    def s_sgd(ctx):
        st = ctx.llama_state()
        tree = ctx.P.Tree([[s["theta"], s["grad"]] for s in st])
        grp = g_sgd()
        lr = ctx.torch.tensor(1e-4, dtype=ctx.torch.float32, device=ctx.dev)
        return lambda: grp.run_tree(tree, [0, 1, -1], 0, [None, None, lr], stream=ctx.stream)
    W.append(Workload("tree_sgd_llama_bf16", "psk_tree_sgd_llama16_bf16", 4 * n, 2 * n, s_sgd, group=g_sgd,
                      note="emitted tree-mapped group: theta' = theta - lr * g, lr a device scalar"))

    def g_adamw_group():
        return P.Group(C.adamw_group_dag(), [((1,), "bf16"), ((1,), "bf16"), ((1,), "f32"), ((1,), "f32")] +
                       [((), "f32")] * 9, (1,), "bf16", tree=True,
                       extras=[(C.ADAMW_GROUP_M, (1,), "f32"), (C.ADAMW_GROUP_V, (1,), "f32")])

    def s_adamw_group(ctx):
        import numpy as np
        hp = ctx.hp
        b1, b2, t = hp[1], hp[2], hp[5]
        sc = np.array([b1, b2, 1 - b1, 1 - b2, 1 - b1 ** t, 1 - b2 ** t, hp[0], hp[3], hp[4]], np.float64)
        scal = ctx.torch.from_numpy(sc.astype(np.float32)).to(ctx.dev)
        grp = g_adamw_group()
        tree = tree_of(ctx, ctx.llama_state())
        scalars = [None] * 4 + [scal[i] for i in range(9)]
        return lambda: grp.run_tree(tree, [0, 1, 2, 3] + [-1] * 9, [0, 2, 3], scalars, stream=ctx.stream)
    W.append(Workload("adamw_llama_bf16_emitted_group", "psk_tree_adamw_group_llama16_bf16", 12 * n, 10 * n,
                      s_adamw_group, group=g_adamw_group,
                      note="the AdamW let-list as an emitted three-output tree group; bit-identical to the "
                           "hand-written kernel"))

    def s_tiny(ctx):
        shapes = [s for _, s in ctx.configs.tiny_gpt_leaves()]
        st = ctx.configs.adamw_state(shapes, device=ctx.dev, seed=ctx.configs.SEED_BASE)
        tree = tree_of(ctx, st)
        return lambda: tree.adamw_step(*ctx.hp, stream=ctx.stream)
    nt = _tiny_n(C)
    W.append(Workload("adamw_tiny_gpt_f32", "adamw_tree_kernel_tiny_gpt_f32", 16 * nt, 12 * nt, s_tiny,
                      kernel=F32_ADAMW, hbm=False,
                      note="3 MB: launch-latency bound, no HBM target; ms_* cold (cache flushed), us_warm_median "
                           "back to back, us_per_step_graph_of_20: 20 steps captured in one HIP graph"))

    # -- row groups
    def g_softmax():
        return P.Group(C.softmax_causal_dag(0.125, 1024), [((R1, C1), "f32")], (R1, C1), "f32")

    def s_softmax(ctx):
        x = ctx.configs.softmax_scores(R1, C1, device=ctx.dev)
        y = ctx.torch.empty_like(x)
        grp = g_softmax()
        return lambda: grp.run([x], y, stream=ctx.stream)
    W.append(Workload("softmax_causal_f32", "psk_row_softmax_causal_131072x1024_f32", 4 * a1, 4 * R1 * C1,
                      s_softmax, group=g_softmax))

    def g_rms():
        return P.Group(C.rmsnorm_gelu_dag(eps), [((R3, C3), "bf16"), ((R3, C3), "bf16"), ((C3,), "bf16")],
                       (R3, C3), "bf16")

    def s_rms(ctx):
        x, r, g = ctx.configs.rmsnorm_inputs(R3, C3, device=ctx.dev)
        y = ctx.torch.empty_like(x)
        grp = g_rms()
        return lambda: grp.run([x, r, g], y, stream=ctx.stream)
    W.append(Workload("rmsnorm_gelu_bf16", "psk_row_rmsnorm_gelu_16384x4096_bf16", 4 * R3 * C3 + 2 * C3,
                      2 * R3 * C3, s_rms, group=g_rms))

    def g_rms_h():
        return P.Group(C.rmsnorm_gelu_dag(eps), [((R3, C3), "bf16"), ((R3, C3), "bf16"), ((C3,), "bf16")],
                       (R3, C3), "bf16", extras=[(C.RMSNORM_H, (R3, C3), "bf16")])

    def s_rms_h(ctx):
        x, r, g = ctx.configs.rmsnorm_inputs(R3, C3, device=ctx.dev)
        y = ctx.torch.empty_like(x)
        grp = g_rms_h()
        return lambda: grp.run([x, r, g], y, stream=ctx.stream, extra_outs=[r])
    W.append(Workload("add_rmsnorm_gelu_store_h_bf16", "psk_row_add_rmsnorm_gelu_store_h_16384x4096_bf16",
                      4 * R3 * C3 + 2 * C3, 4 * R3 * C3, s_rms_h, group=g_rms_h,
                      note="h written in place over the residual"))

    def g_ln():
        return P.Group(C.layernorm_dag(eps), [((R3, C3), "bf16"), ((C3,), "bf16"), ((C3,), "bf16")], (R3, C3),
                       "bf16", root=C.LAYERNORM_ROOT,
                       extras=[(C.LAYERNORM_MEAN, (R3, 1), "f32"), (C.LAYERNORM_RSTD, (R3, 1), "f32")])

    def s_ln(ctx):
        x, g, b = ctx.configs.layernorm_inputs(R3, C3, device=ctx.dev)
        y = ctx.torch.empty_like(x)
        m = ctx.torch.empty((R3, 1), device=ctx.dev)
        r = ctx.torch.empty((R3, 1), device=ctx.dev)
        grp = g_ln()
        return lambda: grp.run([x, g, b], y, stream=ctx.stream, extra_outs=[m, r])
    W.append(Workload("layernorm_stats_bf16", "psk_row_layernorm_stats_16384x4096_bf16", 2 * R3 * C3 + 4 * C3,
                      2 * R3 * C3 + 8 * R3, s_ln, group=g_ln,
                      note="mean, x - mean read twice, variance, normalise; mean and rstd stored per row",
                      size_copy="copy_emitted_16384x4096_bf16"))

    def g_masked():
        return P.Group(C.softmax_masked_dag(0.125), [((8, 16, 1024, 1024), "f32"), ((1024, 1024), "u8")],
                       (8, 16, 1024, 1024), "f32")

    def s_masked(ctx):
        x = ctx.configs.softmax_scores(R1, C1, device=ctx.dev).view(8, 16, 1024, 1024)
        y = ctx.torch.empty_like(x)
        m = ctx.configs.causal_mask_bytes(1024, device=ctx.dev)
        grp = g_masked()
        return lambda: grp.run([x, m], y, stream=ctx.stream)
    W.append(Workload("softmax_mask_buffer_f32", "psk_row_softmax_mask_buffer_8x16x1024x1024_f32",
                      4 * a1 + 1024 * 1024, 4 * R1 * C1, s_masked, group=g_masked,
                      note="the scores the mask allows read (vectors it refuses are not loaded), the mask once, "
                           "probabilities written"))

    def g_soft_bf16():
        return P.Group(C.softmax_causal_dag(0.125, 1024), [((R1, C1), "bf16")], (R1, C1), "bf16")

    def s_soft_bf16(ctx):
        x = ctx.configs.softmax_scores(R1, C1, device=ctx.dev).to(ctx.torch.bfloat16)
        y = ctx.torch.empty_like(x)
        grp = g_soft_bf16()
        return lambda: grp.run([x], y, stream=ctx.stream)
    W.append(Workload("softmax_causal_bf16", "psk_row_softmax_causal_131072x1024_bf16", 2 * a1, 2 * R1 * C1,
                      s_soft_bf16, group=g_soft_bf16))

    def g_wide(online=False):
        return lambda: P.Group(C.softmax_dag(0.125), [((RW, CW), "f32")], (RW, CW), "f32", online=online)

    def s_wide(online):
        def setup(ctx):
            x = ctx.configs.softmax_scores(RW, CW, device=ctx.dev)
            y = ctx.torch.empty_like(x)
            grp = g_wide(online)()
            return lambda: grp.run([x], y, stream=ctx.stream)
        return setup
    W.append(Workload("softmax_wide_8192x131072_f32", "psk_rows_softmax_wide_8192x131072_f32", 4 * RW * CW,
                      4 * RW * CW, s_wide(False), group=g_wide(False),
                      note="rows too wide for one workgroup's registers and LDS; bytes counted once"))
    W.append(Workload("softmax_wide_8192x131072_f32_online", "psk_rows_softmax_wide_online_8192x131072_f32",
                      4 * RW * CW, 4 * RW * CW, s_wide(True), group=g_wide(True),
                      note="PSK_GROUP_ONLINE: the sum taken in the maximum's pass; its rounding differs from the "
                           "exact sum (declared differs, within the f32 tolerance)"))

    # -- pointwise groups
    def g_chain():
        return P.Group(C.chain64_dag(), [((N4, N4), "f32"), ((N4, 1), "f32"), ((1, N4), "f32")], (N4, N4), "f32")

    def s_chain(ctx):
        A, B, Cc = ctx.configs.chain_inputs(N4, N4, device=ctx.dev)
        Z = ctx.torch.empty_like(A)
        grp = g_chain()
        return lambda: grp.run([A, B, Cc], Z, stream=ctx.stream)
    W.append(Workload("chain64_f32", "psk_pw_chain64_16384x16384_f32", 4 * N4 * N4 + 8 * N4, 4 * N4 * N4, s_chain,
                      group=g_chain, hbm=False, node_evals=64 * N4 * N4,
                      note="VALU-bound: 64 node evaluations per element"))

    def g_valu():
        return P.Group(C.valu_ceiling_dag(), [((N4, 1), "f32"), ((1, N4), "f32")], (N4, N4), "bf16")

    def s_valu(ctx):
        B = ctx.configs.chain_inputs(N4, 1, device=ctx.dev)[1]       # [N, 1]
        Cc = ctx.configs.chain_inputs(1, N4, device=ctx.dev)[2]      # [1, N]
        Z = ctx.torch.empty((N4, N4), dtype=ctx.torch.bfloat16, device=ctx.dev)
        grp = g_valu()
        return lambda: grp.run([B, Cc], Z, stream=ctx.stream)
    W.append(Workload("valu_ceiling_f32", "psk_pw_valu_ceiling_16384x16384_bf16", 8 * N4, 2 * N4 * N4, s_valu,
                      group=g_valu, hbm=False, node_evals=64 * N4 * N4,
                      note="64 f32 add/mul members in 8 independent chains over broadcast [R,1] and [1,N] inputs: "
                           "one vector instruction per member and 2 bytes of output (bf16) per 64: the VALU rate "
                           "an emitted kernel sustains (with an f32 output its 1 GiB of writes held it 16% lower)"))

    # -- streaming references
    def s_copy_torch(ctx):
        src = ctx.torch.empty(1 << 28, dtype=ctx.torch.float32, device=ctx.dev)
        dst = ctx.torch.empty_like(src)
        return lambda: dst.copy_(src)
    W.append(Workload("copy_ceiling", None, 1 << 30, 1 << 30, s_copy_torch, note="torch device copy, read+write"))

    def g_copy():
        from synth.dag import parse_dag
        return P.Group(parse_dag("%0 = input 0\n%1 = neg %0\n%2 = neg %1\n"), [((1 << 28,), "f32")], (1 << 28,),
                       "f32")

    def s_copy(ctx):
        src = ctx.torch.empty(1 << 28, dtype=ctx.torch.float32, device=ctx.dev)
        dst = ctx.torch.empty_like(src)
        grp = g_copy()
        return lambda: grp.run([src], dst, stream=ctx.stream)
    W.append(Workload("copy_emitted", "psk_pw_copy_1GiB_f32", 1 << 30, 1 << 30, s_copy, group=g_copy,
                      note="emitted pointwise y = -(-x): the r1:w1 streaming rate of an emitted kernel"))

    # the same copy at LayerNorm's size (256 MiB moved): a launch this short
    # streams below the 1 GiB rate (ramp-up and drain weigh more)
    def g_copy_ln():
        from synth.dag import parse_dag
        return P.Group(parse_dag("%0 = input 0\n%1 = neg %0\n%2 = neg %1\n"), [((R3, C3), "bf16")], (R3, C3),
                       "bf16")

    def s_copy_ln(ctx):
        src = ctx.torch.empty((R3, C3), dtype=ctx.torch.bfloat16, device=ctx.dev)
        dst = ctx.torch.empty_like(src)
        grp = g_copy_ln()
        return lambda: grp.run([src], dst, stream=ctx.stream)
    W.append(Workload("copy_emitted_16384x4096_bf16", "psk_pw_copy_16384x4096_bf16", 2 * R3 * C3, 2 * R3 * C3,
                      s_copy_ln, group=g_copy_ln,
                      note="emitted y = -(-x) over LayerNorm's [16384,4096] bf16 rows: the r1:w1 rate at its size"))
    return W


# ------------------------------------------------------------- GPU timing
def time_workloads(ctx, reps, only=()):
    """Each workload alone: a 1 GiB write between calls evicts the 256 MB
    last-level cache; HIP events around each call on the library's stream;
    median, min and max of `reps` calls (after 2 discarded)."""
    torch = ctx.torch
    flush = torch.empty(1 << 28, dtype=torch.float32, device=ctx.dev)
    out = {}
    for w in build_workloads(ctx.P, ctx.configs, ctx.layers):
        if only and w.name not in only:
            continue
        fn = w.setup(ctx)
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps + 2):
            flush.zero_()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(ctx.stream)
            fn()
            b.record(ctx.stream)
            b.synchronize()
            ms.append(a.elapsed_time(b))
        ms = ms[2:]
        rec = {"ms_median": statistics.median(ms), "ms_min": min(ms), "ms_max": max(ms), "bytes": w.bytes}
        if w.note:
            rec["note"] = w.note
        if w.name == "adamw_tiny_gpt_f32":
            rec.update(_tiny_extras(ctx, fn, reps))
        out[w.name] = rec
        del fn
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    del flush
    return out


def _tiny_extras(ctx, fn, reps):
    """The launch-bound tiny tree: back to back, and 20 steps replayed from
    one HIP graph."""
    torch = ctx.torch
    warm = []
    for k in range(reps + 2):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(ctx.stream)
        fn()
        b.record(ctx.stream)
        b.synchronize()
        if k >= 2:
            warm.append(a.elapsed_time(b))
    shapes = [s for _, s in ctx.configs.tiny_gpt_leaves()]
    st = ctx.configs.adamw_state(shapes, device=ctx.dev, seed=ctx.configs.SEED_BASE)
    tree = ctx.P.Tree([[s["theta"], s["grad"], s["m"], s["v"]] for s in st])
    tree.adamw_step(*ctx.hp)             # the first run on a device loads the code object
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(20):
            tree.adamw_step(*ctx.hp)
    torch.cuda.synchronize()
    per = []
    for k in range(reps + 2):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        graph.replay()
        b.record()
        b.synchronize()
        if k >= 2:
            per.append(a.elapsed_time(b) / 20)
    return {"us_warm_median": round(statistics.median(warm) * 1e3, 2),
            "us_per_step_graph_of_20": round(statistics.median(per) * 1e3, 2)}


def combine_processes(runs, workloads):
    """Per workload: the median of the processes' medians, the extremes over
    every call, and each process's median."""
    by = {w.name: w for w in workloads}
    out = {}
    for name in runs[0]:
        recs = [r[name] for r in runs if name in r]
        med = statistics.median(r["ms_median"] for r in recs)
        w = by[name]
        g = {"ms_median": round(med, 4), "ms_min": round(min(r["ms_min"] for r in recs), 4),
             "ms_max": round(max(r["ms_max"] for r in recs), 4),
             "ms_median_per_process": [round(r["ms_median"], 4) for r in recs], "bytes": w.bytes,
             "GBps": round(gb(w.bytes, med), 1), "frac_of_peak": round(gb(w.bytes, med) / HBM_PEAK_GBS, 4)}
        for k, v in recs[0].items():
            if k not in ("ms_median", "ms_min", "ms_max", "bytes"):
                g[k] = v
        if w.node_evals:
            g["node_evals_per_s"] = float(f"{w.node_evals / (med * 1e-3):.4g}")
        out[name] = g
    # each HBM-bound workload against the emitted r1:w1 copy of the same run
    ref = out.get("copy_emitted", {}).get("GBps")
    for w in workloads:
        if ref and w.name in out and w.hbm and not w.name.startswith("copy_"):
            out[w.name]["frac_of_emitted_copy"] = round(out[w.name]["GBps"] / ref, 3)
        if w.size_copy and w.name in out and w.size_copy in out:
            out[w.name]["frac_of_same_size_copy"] = round(out[w.name]["GBps"] / out[w.size_copy]["GBps"], 3)
    # the 64-node chain against the measured VALU rate of add/mul members
    if "chain64_f32" in out and "valu_ceiling_f32" in out:
        out["chain64_f32"]["frac_of_valu_ceiling_node_evals"] = round(
            out["chain64_f32"]["node_evals_per_s"] / out["valu_ceiling_f32"]["node_evals_per_s"], 4)
    return out


def run_children(args, n):
    """n more processes, one after another, each timing every workload."""
    runs = []
    for k in range(n):
        path = os.path.join("/tmp", f"psk_bench_groups_{os.getpid()}_{k}.json")
        cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--groups-only", path, "--reps", str(args.reps),
               "--layers", str(args.layers)]
        if args.only:
            cmd += ["--only", args.only]
        r = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"per-group timing process {k + 1} failed ({r.returncode}):\n{r.stderr[-3000:]}")
        with open(path) as f:
            runs.append(json.load(f))
        os.remove(path)
    return runs


# ------------------------------------------------------------ CPU baseline
def cpu_baseline(args, ctx, scores):
    """The oracle over every workload, on one host thread and on all of them
    (oracle.parallel: blocks of rows, elements or leaves; bit for bit the
    single-threaded result, checked), on the GPU run's own inputs copied to
    the host.  Configs 0-3 whole; the 64-node chain on a sample of its rows.
    Rates are the same algorithmic bytes per second as the GPU's."""
    import numpy as np
    import oracle
    import oracle.parallel as OP
    torch, C = ctx.torch, ctx.configs
    threads = OP.host_threads(args.cpu_threads)

    def host(t):
        t = t.detach().contiguous().cpu()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    def timed(fn):
        t0 = time.perf_counter()
        r = fn()
        return time.perf_counter() - t0, r

    def same(a, b):
        if isinstance(a, (list, tuple)):
            return all(same(x, y) for x, y in zip(a, b))
        return np.array_equal(a.view(np.uint8), b.view(np.uint8))

    per = {}

    def record(name, nbytes, sample, f1, fn):
        t1, r1 = timed(f1)
        tn, rn = timed(fn)
        per[name] = {"bytes": nbytes, "sample": sample, "s_1_thread": round(t1, 3), f"s_{threads}_threads": round(tn, 3),
                     "GBps_1_thread": round(nbytes / t1 / 1e9, 3), "GBps_all_threads": round(nbytes / tn / 1e9, 3),
                     "threads_bit_identical": bool(same(r1, rn))}
        return t1, tn

    HP = C.ADAMW_HP
    hp = (HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"], HP["t"])
    # 0: the tiny GPT tree, f32 (repeated so the time is measurable)
    tiny = C.adamw_state([s for _, s in C.tiny_gpt_leaves()], device=ctx.dev, seed=C.SEED_BASE)
    tl = [tuple(host(s[k]).reshape(-1) for k in ("theta", "grad", "m", "v")) for s in tiny]
    nt = sum(l[0].size for l in tl)
    reps = 50
    record("0_adamw_tiny_gpt_f32", 28 * nt * reps, f"the whole tree ({nt} params), {reps} steps",
           lambda: [OP.adamw_leaves(tl, hp, 1) for _ in range(reps)][-1],
           lambda: [OP.adamw_leaves(tl, hp, threads) for _ in range(reps)][-1])
    # 1: causal softmax, every row
    xs = host(scores)
    R1, C1 = xs.shape
    b1 = 4 * allowed_causal(R1, C1) + 4 * R1 * C1
    s1 = record("1_softmax_causal_f32", b1, f"all {R1} rows",
                lambda: OP.softmax_causal(xs, 1024, 0.125, 1), lambda: OP.softmax_causal(xs, 1024, 0.125, threads))
    del xs
    # 2: AdamW over the Llama tree, every leaf (the GPU run's state as it stands)
    ll = [tuple(host(s[k]).reshape(-1) for k in ("theta", "grad", "m", "v")) for s in ctx.llama_state()]
    n2 = sum(l[0].size for l in ll)
    s2 = record("2_adamw_llama_bf16", 22 * n2, f"all {len(ll)} leaves, {n2} params",
                lambda: OP.adamw_leaves(ll, hp, 1), lambda: OP.adamw_leaves(ll, hp, threads))
    del ll
    # 3: add + RMSNorm + gamma + GELU, every row
    x, r, g = (host(t) for t in C.rmsnorm_inputs(16384, 4096, device=ctx.dev))
    eps = C.f32(1e-5)
    record("3_rmsnorm_gelu_bf16", 6 * x.size + 2 * g.size, f"all {x.shape[0]} rows",
           lambda: OP.rmsnorm_gelu(x, r, g, eps, 1), lambda: OP.rmsnorm_gelu(x, r, g, eps, threads))
    # 4: the 64-node chain on its first rows
    rows = 1024
    A, B, Cc = C.chain_inputs(16384, 16384, device=ctx.dev)
    ins = [host(A[:rows]), host(B[:rows]), host(Cc)]
    del A, B, Cc
    nodes = C.chain64_dag()
    record("4_chain64_f32", 8 * rows * 16384 + 4 * rows + 4 * 16384, f"{rows} of 16384 rows",
           lambda: OP.eval_group(nodes, ins, (rows, 16384), 0, 1),
           lambda: OP.eval_group(nodes, ins, (rows, 16384), 0, threads))
    per["4_chain64_f32"]["node_evals_per_s_all_threads"] = float(
        f"{64 * rows * 16384 / per['4_chain64_f32'][f's_{threads}_threads']:.4g}")
    step_bytes = per["1_softmax_causal_f32"]["bytes"] + per["2_adamw_llama_bf16"]["bytes"]
    t1 = s1[0] + s2[0]
    tn = s1[1] + s2[1]
    return {"value": round(step_bytes / tn / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole step (AdamW over all {n2} Llama params + all {R1} softmax rows) on {threads} host "
                      f"threads, the GPU run's own inputs",
            "value_1_thread": round(step_bytes / t1 / 1e9, 3), "seconds_all_threads": round(tn, 2),
            "seconds_1_thread": round(t1, 2), "per_config": per, "cpu_model": _cpu_model(),
            "host_cpus": os.cpu_count()}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ------------------------------------------------------ profile summaries
ADAMW_COUNTERS = os.path.join(ROOT, "profiles", "adamw_tree_kernel_llama16_bf16.txt")
ADAMW_SOURCES = ["elementwise_reduction_groups_amd/csrc/adamw.hip", "elementwise_reduction_groups_amd/csrc/psk_internal.h"]
PROFILE_RUNS = {
    # subdirectory, output prefix, rocprofv3 arguments (each its own run; counters never with tracing)
    "kt": ("p_kt", "kt", "--kernel-trace --stats", "--steps 10 --warmup 3"),
    "fetch": ("p_fetch", "f", "--pmc FETCH_SIZE", "--pmc-calib --steps 2 --warmup 1"),
    "write": ("p_write", "w", "--pmc WRITE_SIZE", "--pmc-calib --steps 2 --warmup 1"),
    "valu": ("p_valu", "v", "--pmc SQ_INSTS_VALU SQ_WAVES", "--steps 2 --warmup 1"),
    "tcc": ("p_tcc", "t", "--pmc TCC_HIT_sum TCC_MISS_sum", "--steps 2 --warmup 1"),
}


# The SQ counters behind the LayerNorm diagnosis (one pass of 8 SQ counters,
# the two row groups only), summarized into profiles/SQ_SUMMARY.
SQ_RUN = ("p_sq", "sq", "--pmc SQ_WAIT_ANY SQ_WAVE_CYCLES SQ_INST_LEVEL_VMEM SQ_INSTS_VMEM SQ_ACTIVE_INST_ANY "
          "SQ_INSTS_VALU SQ_WAVES SQ_BUSY_CYCLES", "--only layernorm_stats_bf16,rmsnorm_gelu_bf16 --steps 1 --warmup 0")
SQ_SUMMARY = "sq_counters_layernorm_rmsnorm_16384x4096_bf16.txt"


def profile_command(key, base="gpurun_out"):
    sub, pre, prof, extra = SQ_RUN if key == "sq" else PROFILE_RUNS[key]
    return (f"rocprofv3 {prof} --output-format csv -d {base}/{sub} -o {pre} -- python3 bench.py --profile-step "
            f"--profile-all {extra}")


def summarize_sq(base, P, configs):
    """profiles/SQ_SUMMARY from the SQ counter run: per-dispatch means for the
    LayerNorm and RMSNorm+GELU kernels, with the ratios the diagnosis uses."""
    import csv
    import collections
    path = os.path.join(base, SQ_RUN[0], SQ_RUN[1] + "_counter_collection.csv")
    if not os.path.exists(path):
        return None
    ws = {w.name: w for w in build_workloads(P, configs)}
    names = {ws[n].group().info.kernel.decode(): n for n in ("layernorm_stats_bf16", "rmsnorm_gelu_bf16")}
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(path)):
        for kn, n in names.items():
            if kn in r["Kernel_Name"]:
                agg[n][r["Counter_Name"]].append(float(r["Counter_Value"]))
    lines = ["# SQ counters: LayerNorm + mean + rstd (persistent rows) and add + RMSNorm + gamma + GELU (one row a "
             "workgroup), both [16384,4096] bf16, on one MI355X (gfx950)",
             "# commands (from the repository root, TMPDIR=/tmp):",
             f"#   {profile_command('sq')}",
             f"#   python3 bench.py --summarize-profiles {base}",
             "# per-dispatch means; SQ_WAVE_CYCLES, SQ_WAIT_ANY and SQ_ACTIVE_INST_ANY are wave-cycles (quad-cycle "
             "units) summed over waves"]
    for n in ("layernorm_stats_bf16", "rmsnorm_gelu_bf16"):
        if n not in agg:
            continue
        m = {c: statistics.fmean(v) for c, v in agg[n].items()}
        lines.append(f"[{n}]   dispatches {len(next(iter(agg[n].values())))}")
        for c in sorted(m):
            lines.append(f"{c} = {m[c]:.0f}")
        wc = m.get("SQ_WAVE_CYCLES", 0.0)
        if wc:
            lines.append(f"wait_fraction = {m['SQ_WAIT_ANY'] / wc:.3f}          # SQ_WAIT_ANY / SQ_WAVE_CYCLES")
            lines.append(f"issue_fraction = {m['SQ_ACTIVE_INST_ANY'] / wc:.3f}         # SQ_ACTIVE_INST_ANY / SQ_WAVE_CYCLES")
        if m.get("SQ_BUSY_CYCLES"):
            lines.append(f"vmem_in_flight_per_busy_cycle = {m['SQ_INST_LEVEL_VMEM'] / m['SQ_BUSY_CYCLES']:.2f}")
        if m.get("SQ_WAVES"):
            lines.append(f"valu_per_wave = {m['SQ_INSTS_VALU'] / m['SQ_WAVES']:.0f}")
    with open(os.path.join(ROOT, "profiles", SQ_SUMMARY), "w") as f:
        f.write("\n".join(lines) + "\n")
    return SQ_SUMMARY


def kernel_source_sha(paths):
    """SHA-256 of the AdamW kernel's source: adamw.hip whole, and of the
    shared header only its AdamW section (the structures the kernel reads)."""
    import hashlib
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
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
                kv[k.strip()] = v.split("#", 1)[0].strip()
        if kv.get("kernel_source_sha256") != kernel_source_sha(ADAMW_SOURCES):
            return None
        return int(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def summarize_profiles(base):
    """profiles/<workload>.txt from the rocprofv3 runs under `base` (the five
    runs of PROFILE_RUNS): kernel time from the kernel trace; FETCH_SIZE and
    WRITE_SIZE in KiB per dispatch, each scaled by what the same counter
    reads for the 1 GiB device copy the counter runs start with (a known
    read of 1 GiB and write of 1 GiB); VALU instructions and waves; L2 hits."""
    import csv
    import collections
    sys.path.insert(0, ROOT)
    import elementwise_reduction_groups_amd as P
    from synth import configs

    def rows(key, suffix):
        sub, pre = PROFILE_RUNS[key][:2]
        path = os.path.join(base, sub, f"{pre}_{suffix}.csv")
        return list(csv.DictReader(open(path))) if os.path.exists(path) else []

    workloads = [w for w in build_workloads(P, configs) if w.profile]
    names = []
    for w in workloads:
        for k in ((w.group().info.kernel.decode(),) if w.group else w.kernel):
            names.append((k, w))

    def which(kernel_name):
        if "rocclr_copyBuffer" in kernel_name:
            return "copy"
        for k, w in names:
            if k in kernel_name:
                return w.profile
        return None

    stats = {}
    for r in rows("kt", "kernel_stats"):
        k = which(r["Name"])
        if k:
            stats[k] = r

    def counters(key, cname):
        d = collections.defaultdict(list)
        for r in rows(key, "counter_collection"):
            k = which(r["Kernel_Name"])
            if k and r["Counter_Name"] == cname:
                d[k].append((float(r["Counter_Value"]), int(r["Grid_Size"]), r))
        return d

    F, Wr = counters("fetch", "FETCH_SIZE"), counters("write", "WRITE_SIZE")
    V, WV = counters("valu", "SQ_INSTS_VALU"), counters("valu", "SQ_WAVES")
    TH, TM = counters("tcc", "TCC_HIT_sum"), counters("tcc", "TCC_MISS_sum")
    copy_f = max(F["copy"], key=lambda x: x[1])
    copy_w = max(Wr["copy"], key=lambda x: x[1])
    ff, fw = 1048576.0 / copy_f[0], 1048576.0 / copy_w[0]
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    written = []
    for w in workloads:
        k = w.profile
        if k not in stats or k not in F or k not in Wr:
            continue
        st = stats[k]
        fk = statistics.fmean(x[0] for x in F[k])
        wk = statistics.fmean(x[0] for x in Wr[k])
        fetch_b, write_b = int(round(fk * 1024 * ff)), int(round(wk * 1024 * fw))
        avg_ns = float(st["AverageNs"])
        r0 = F[k][0][2]
        lines = [f"# {k}: rocprofv3 summary on one MI355X (gfx950)",
                 f"# kernel: {w.group().info.kernel.decode() if w.group else 'psk::' + w.kernel[-1]}",
                 "# commands (from the repository root, TMPDIR=/tmp):"] + \
                [f"#   {profile_command(key)}" for key in PROFILE_RUNS] + \
                [f"#   python3 bench.py --summarize-profiles gpurun_out",
                 f"calls = {st['Calls']}", f"average_duration_ns = {avg_ns:.0f}",
                 f"min_duration_ns = {st['MinNs']}", f"max_duration_ns = {st['MaxNs']}",
                 f"grid_threads = {F[k][0][1]}", f"workgroup = {r0['Workgroup_Size']}",
                 f"vgpr = {r0.get('VGPR_Count', r0.get('Arch_VGPR_Count', '?'))}", f"sgpr = {r0['SGPR_Count']}",
                 f"lds_bytes = {r0['LDS_Block_Size']}", f"scratch_bytes = {r0['Scratch_Size']}",
                 f"fetch_size_kib_per_dispatch = {fk:.1f}", f"write_size_kib_per_dispatch = {wk:.1f}",
                 f"fetch_calibration = {ff:.5f}   # 1 GiB device copy: FETCH_SIZE read {copy_f[0]:.1f} KiB",
                 f"write_calibration = {fw:.5f}   # same copy: WRITE_SIZE read {copy_w[0]:.1f} KiB",
                 f"fetch_bytes_per_launch = {fetch_b}", f"write_bytes_per_launch = {write_b}",
                 f"traffic_bytes_per_launch = {fetch_b + write_b}",
                 f"algorithmic_bytes_per_launch = {w.bytes}   # read {w.read} + write {w.write}",
                 f"traffic_over_algorithmic = {(fetch_b + write_b) / w.bytes:.4f}",
                 f"achieved_GBps_from_average = {w.bytes / avg_ns:.1f}",
                 f"frac_of_8TBps = {w.bytes / avg_ns / 8000:.4f}"]
        if k in V and k in WV:
            valu, waves = V[k][0][0], WV[k][0][0]
            lines += [f"sq_insts_valu_per_dispatch = {valu:.0f}", f"sq_waves_per_dispatch = {waves:.0f}",
                      f"valu_lane_instr_per_s = {valu * 64 / (avg_ns * 1e-9):.4g}"]
            if w.node_evals:
                lines += [f"node_evals_per_s = {w.node_evals / (avg_ns * 1e-9):.4g}",
                          f"valu_lane_instr_per_node_eval = {valu * 64 / w.node_evals:.3f}"]
        if k in TH and k in TM:
            h, m = TH[k][0][0], TM[k][0][0]
            lines += [f"tcc_hit_per_dispatch = {h:.0f}", f"tcc_miss_per_dispatch = {m:.0f}",
                      f"tcc_hit_rate = {h / max(h + m, 1):.4f}"]
        if k == "adamw_tree_kernel_llama16_bf16":
            lines.append("kernel_source_sha256 = " + kernel_source_sha(ADAMW_SOURCES))
        with open(os.path.join(ROOT, "profiles", k + ".txt"), "w") as f:
            f.write("\n".join(lines) + "\n")
        written.append((k, avg_ns, (fetch_b + write_b) / w.bytes))
    for k, avg, ratio in written:
        print(f"{k}: average {avg / 1e3:.1f} us, traffic / algorithmic {ratio:.4f}")
    sq = summarize_sq(base, P, configs)
    if sq:
        print(f"{sq}: written")
    return written


# -------------------------------------------------------------------- main
def main():
    args = parse()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: each GPU would run the same kernels on "
                                   "its own share of rows, elements or leaves, with no exchange inside the step, "
                                   "so no multi-GPU figure is produced",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0 or args.reps < 1 or args.procs < 1 or args.cpu_threads < 1:
        print(json.dumps({"error": "--steps, --reps, --procs and --cpu-threads must be at least 1, --warmup at "
                                   "least 0"}))
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
    only = tuple(s for s in args.only.split(",") if s)

    if args.groups_only:
        ctx = Ctx(P, configs, torch, dev, stream, hp, layers=args.layers)
        with open(args.groups_only, "w") as f:
            json.dump(time_workloads(ctx, args.reps, only), f)
        return

    # ---------------------------------------------------------------- inputs
    shapes = [s for _, s in configs.llama_leaves(L=args.layers)]
    n_params = sum(math.prod(s) for s in shapes)
    state = configs.adamw_state(shapes, theta_dtype=torch.bfloat16, grad_dtype=torch.bfloat16,
                                mv_dtype=torch.float32, device=dev, seed=configs.SEED_BASE + 2)
    ctx = Ctx(P, configs, torch, dev, stream, hp, state=state, layers=args.layers)
    tree = P.Tree([[s["theta"], s["grad"], s["m"], s["v"]] for s in state])
    adamw_bytes = n_params * (2 + 2 + 4 + 4 + 2 + 4 + 4)

    R, C = 131072, 1024
    scores = configs.softmax_scores(R, C, device=dev)
    probs = torch.empty_like(scores)
    softmax = P.Group(configs.softmax_causal_dag(0.125, 1024), [((R, C), "f32")], (R, C), "f32")
    softmax_bytes = allowed_causal(R, C) * 4 + R * C * 4
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
        "dtype": "f32",
        "storage": "bf16 theta/g, f32 m/v (AdamW); f32 scores and probabilities (softmax)",
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
            "traffic": committed_traffic(),
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
    if args.profile_step:
        if args.profile_all:
            # only the workloads with a summary: another workload launching
            # the same kernel (the 22-layer tree) would mix into its counters
            for w in build_workloads(P, configs, args.layers):
                if (only and w.name not in only) or not w.profile:
                    continue
                fn = w.setup(ctx)
                for _ in range(6):      # the first call touches freshly allocated memory; 6 keep it to a sixth
                    fn()
                torch.cuda.synchronize()
                del fn
                torch.cuda.empty_cache()
        print(json.dumps(result), flush=True)
        return

    # ----------------------------------------------------- per-group timing
    if not args.no_groups:
        workloads = build_workloads(P, configs, args.layers)
        runs = [time_workloads(ctx, args.reps, only)]
        if args.procs > 1:
            runs += run_children(args, args.procs - 1)
        result["groups"] = combine_processes(runs, workloads)
        result["groups_protocol"] = (f"median of {args.reps} calls per process (2 discarded first), cache flushed "
                                     f"between calls, in {args.procs} processes; ms_median is the median of the "
                                     f"processes' medians, ms_min/ms_max the extremes over all calls")

    # ------------------------------------------------ static dispatch counts
    result["dispatch"] = dispatch_report(P, configs)

    # ------------------------------------------------------------ CPU leg
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, ctx, scores)

    print(json.dumps(result), flush=True)


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


if __name__ == "__main__":
    main()
