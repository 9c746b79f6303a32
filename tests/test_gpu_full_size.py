"""Every output element of the full-size workloads against the oracle, in
the launch layouts the benchmark times.

The GPU's inputs are copied to the host and the oracle runs over them on
the host's threads (oracle.parallel: blocks of rows, leaves or elements;
bit for bit the single-threaded oracle).  Each test asserts that the count
of elements compared equals the output's size:

  * AdamW over the Llama-style tree (145 leaves, 887 685 120 parameters,
    bf16 theta and g, f32 m and v): theta', m', v' of every leaf bit for bit;
  * causal softmax, f32 [131072, 1024]: all 134M outputs within
    1e-7 + 2e-6 |ref|;
  * add + RMSNorm + gamma + GELU, bf16 [16384, 4096]: all 67M outputs within
    one bf16 ulp;
  * the 64-node chain, f32 [16384, 16384]: all 268M outputs within
    1e-7 + 2e-6 |ref|;
  * and the other timed workloads at their sizes: the wide softmax
    [8192, 131072] f32 (split rows), LayerNorm with its statistics, the
    byte-mask softmax and the bf16 causal softmax.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle.parallel as OP
from synth import configs
from tests.gpu_util import compare_all, to_np

P = pytest.importorskip("elementwise_reduction_groups_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
THREADS = OP.host_threads(16)
EPS = configs.f32(1e-5)


def say(msg):
    print(f"[full size] {msg}", file=sys.stderr, flush=True)


def test_adamw_llama_tree_every_element():
    shapes = [s for _, s in configs.llama_leaves()]
    state = configs.adamw_state(shapes, theta_dtype=torch.bfloat16, grad_dtype=torch.bfloat16,
                                mv_dtype=torch.float32, device=DEV, seed=configs.SEED_BASE + 2)
    n = sum(math.prod(s) for s in shapes)
    assert len(shapes) == 145 and n == 887685120
    say("AdamW Llama tree: inputs to host")
    host = [tuple(to_np(s[k]).reshape(-1) for k in ("theta", "grad", "m", "v")) for s in state]
    tree = P.Tree([[s["theta"], s["grad"], s["m"], s["v"]] for s in state])
    HP = configs.ADAMW_HP
    hp = (HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"], HP["t"])
    say("AdamW Llama tree: one step on the GPU")
    tree.adamw_step(*hp)
    torch.cuda.synchronize()
    say(f"AdamW Llama tree: oracle on {THREADS} host threads")
    ref = OP.adamw_leaves(host, hp, THREADS)
    compared = 0
    for leaf, (s, r) in enumerate(zip(state, ref)):
        for k, name, rr in zip(("theta", "m", "v"), ("theta'", "m'", "v'"), r):
            compared += compare_all(to_np(s[k]), rr, "bits", f"leaf {leaf} {name}")
    assert compared == 3 * n


def test_causal_softmax_every_element():
    R, C = 131072, 1024
    x = configs.softmax_scores(R, C, device=DEV)
    g = P.Group(configs.softmax_causal_dag(0.125, 1024), [((R, C), "f32")], (R, C), "f32")
    out = torch.full_like(x, float("nan"))
    say("causal softmax [131072, 1024] f32 on the GPU")
    g.run([x], out)
    torch.cuda.synchronize()
    say(f"causal softmax: oracle on {THREADS} host threads")
    ref = OP.softmax_causal(to_np(x), 1024, 0.125, THREADS)
    assert compare_all(to_np(out), ref, "f32", "causal softmax") == R * C


def test_rmsnorm_gelu_every_element():
    R, C = 16384, 4096
    x, r, gm = configs.rmsnorm_inputs(R, C, device=DEV)
    g = P.Group(configs.rmsnorm_gelu_dag(EPS), [((R, C), "bf16"), ((R, C), "bf16"), ((C,), "bf16")], (R, C), "bf16")
    out = torch.full_like(x, float("nan"))
    say("add + RMSNorm + gamma + GELU [16384, 4096] bf16 on the GPU")
    g.run([x, r, gm], out)
    torch.cuda.synchronize()
    say(f"RMSNorm + GELU: oracle on {THREADS} host threads")
    ref = OP.rmsnorm_gelu(to_np(x), to_np(r), to_np(gm), EPS, THREADS)
    assert compare_all(to_np(out), ref, "bf16", "RMSNorm + GELU") == R * C


def test_chain64_every_element():
    N = 16384
    nodes = configs.chain64_dag()
    A, B, C = configs.chain_inputs(N, N, device=DEV)
    g = P.Group(nodes, [((N, N), "f32"), ((N, 1), "f32"), ((1, N), "f32")], (N, N), "f32")
    out = torch.full_like(A, float("nan"))
    say("64-node chain [16384, 16384] f32 on the GPU")
    g.run([A, B, C], out)
    torch.cuda.synchronize()
    say(f"64-node chain: oracle on {THREADS} host threads")
    ref = OP.eval_group(nodes, [to_np(A), to_np(B), to_np(C)], (N, N), 0, THREADS)
    assert compare_all(to_np(out), ref, "f32", "chain64") == N * N


def test_wide_softmax_every_element():
    """The [8192, 131072] f32 softmax (rows split over workgroups): all 1.07e9
    outputs within 1e-7 + 2e-6 |ref|."""
    R, C = 8192, 131072
    x = configs.softmax_scores(R, C, device=DEV)
    g = P.Group(configs.softmax_dag(0.125), [((R, C), "f32")], (R, C), "f32")
    out = torch.full_like(x, float("nan"))
    say("wide softmax [8192, 131072] f32 on the GPU")
    g.run([x], out)
    torch.cuda.synchronize()
    g.check()
    say(f"wide softmax: oracle on {THREADS} host threads")
    ref = OP.eval_group(configs.softmax_dag(0.125), [to_np(x)], (R, C), 0, THREADS)
    assert compare_all(to_np(out), ref, "f32", "wide softmax") == R * C


def test_layernorm_stats_every_element():
    """LayerNorm storing mean and rstd, bf16 [16384, 4096] (persistent rows):
    all 67M outputs within one bf16 ulp or the derived bound near a
    cancellation (y * gamma + beta), every row's statistics within the
    bound of its own summation tree."""
    from tests.test_gpu_multi import assert_layernorm_close, check_stats, layernorm_group
    R, C = 16384, 4096
    x, gm, bt = configs.layernorm_inputs(R, C, device=DEV)
    g = layernorm_group(R, C)
    out = torch.full_like(x, float("nan"))
    mean = torch.full((R, 1), float("nan"), device=DEV)
    rstd = torch.full((R, 1), float("nan"), device=DEV)
    say("LayerNorm + statistics [16384, 4096] bf16 on the GPU")
    g.run([x, gm, bt], out, extra_outs=[mean, rstd])
    torch.cuda.synchronize()
    say(f"LayerNorm: oracle on {THREADS} host threads")
    ref = OP.eval_group(configs.layernorm_dag(EPS), [to_np(x), to_np(gm), to_np(bt)], (R, C), 1, THREADS,
                        root=configs.LAYERNORM_ROOT)
    got = to_np(out)
    assert got.size == ref.size == R * C
    assert_layernorm_close(got, ref, x, gm, bt, C, "LayerNorm full size")
    check_stats(g.info, x, mean, rstd, C, "LayerNorm full size")


def test_byte_mask_softmax_every_element():
    """Softmax with a [1024, 1024] causal byte mask broadcast over 8 x 16
    heads, f32: all 134M outputs within 1e-7 + 2e-6 |ref| (refused
    positions +0)."""
    shape = (8, 16, 1024, 1024)
    x = configs.softmax_scores(8 * 16 * 1024, 1024, device=DEV).view(shape)
    m = configs.causal_mask_bytes(1024, device=DEV)
    dag = configs.softmax_masked_dag(0.125)
    g = P.Group(dag, [(shape, "f32"), ((1024, 1024), "u8")], shape, "f32")
    out = torch.full_like(x, float("nan"))
    say("byte-mask softmax [8, 16, 1024, 1024] f32 on the GPU")
    g.run([x, m], out)
    torch.cuda.synchronize()
    say(f"byte-mask softmax: oracle on {THREADS} host threads")
    ref = OP.eval_group(dag, [to_np(x), m.cpu().numpy().view(np.uint8)], shape, 0, THREADS)
    assert compare_all(to_np(out), ref, "f32", "byte-mask softmax") == math.prod(shape)
    refused = ~m.cpu().numpy()
    assert np.all(to_np(out).reshape(-1, 1024, 1024)[:, refused].view(np.uint32) == 0)


def test_causal_softmax_bf16_every_element():
    """Causal softmax with bf16 scores and probabilities [131072, 1024]: all
    134M outputs within one bf16 ulp."""
    R, C = 131072, 1024
    x = configs.softmax_scores(R, C, device=DEV).to(torch.bfloat16)
    dag = configs.softmax_causal_dag(0.125, 1024)
    g = P.Group(dag, [((R, C), "bf16")], (R, C), "bf16")
    out = torch.empty_like(x)
    say("causal softmax [131072, 1024] bf16 on the GPU")
    g.run([x], out)
    torch.cuda.synchronize()
    say(f"bf16 causal softmax: oracle on {THREADS} host threads")
    ref = OP.eval_group(dag, [to_np(x)], (R, C), 1, THREADS)
    assert compare_all(to_np(out), ref, "bf16", "bf16 causal softmax") == R * C
