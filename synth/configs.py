"""The five synthetic workloads and their seeded generators.

Workloads (sizes as measured):
  0. AdamW step over a tiny GPT parameter tree, f32 (V=92, D=64, L=2):
     28 leaves, 108 032 parameters.
  1. Causal row softmax, f32 scores [8,16,1024,1024] viewed as 131 072 rows x 1024.
  2. AdamW step over a Llama-style tree (16 layers, D=2048, FFN 5632,
     vocab 32000): 145 leaves, 887 685 120 parameters; bf16 param and grad,
     f32 moments.
  3. Residual add + RMSNorm + gamma + GELU, bf16 [16384, 4096].
  4. Seeded random 64-node elementwise chain over A [16384,16384],
     B [16384,1], C [1,16384], all f32.

Distributions: N(0, s) means standard deviation s (presk language reference,
section "Initializers").  bf16 tensors are drawn in f32 and rounded to nearest even
(presk native chapter, "The realization").  Every tensor, or leaf slot, gets a
generator of its own derived from (seed, index), so a leaf's values do not
depend on how many leaves precede it.

No function here computes anything a fusion group computes.
"""
from __future__ import annotations

import math
import os
from typing import Dict, List, Sequence, Tuple

import torch

from .dag import Node, parse_dag, random_chain_dag

SEED_BASE = 1000

ADAMW_HP = dict(lr=3e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, t=10)


def _gen(device, seed: int, *idx: int) -> torch.Generator:
    g = torch.Generator(device=device)
    s = seed
    for k in idx:
        s = (s * 1_000_003 + k + 1) % (2**63 - 1)
    g.manual_seed(s)
    return g


# ---------------------------------------------------------------- param trees
def tiny_gpt_leaves(V: int = 92, D: int = 64, L: int = 2, T: int = 32) -> List[Tuple[str, Tuple[int, ...]]]:
    leaves = [("tok_emb", (V, D)), ("pos_emb", (T, D))]
    for l in range(L):
        p = f"blocks.{l}."
        leaves += [
            (p + "ln1.g", (D,)), (p + "ln1.b", (D,)),
            (p + "attn.Wqkv", (D, 3 * D)), (p + "attn.bqkv", (3 * D,)),
            (p + "attn.Wo", (D, D)), (p + "attn.bo", (D,)),
            (p + "ln2.g", (D,)), (p + "ln2.b", (D,)),
            (p + "ff.W1", (D, 4 * D)), (p + "ff.b1", (4 * D,)),
            (p + "ff.W2", (4 * D, D)), (p + "ff.b2", (D,)),
        ]
    leaves += [("lnf.g", (D,)), ("lnf.b", (D,))]
    return leaves


def llama_leaves(L: int = 16, D: int = 2048, F: int = 5632, V: int = 32000) -> List[Tuple[str, Tuple[int, ...]]]:
    leaves = [("embedding", (V, D))]
    for l in range(L):
        p = f"layers.{l}."
        leaves += [
            (p + "Wq", (D, D)), (p + "Wk", (D, D)), (p + "Wv", (D, D)), (p + "Wo", (D, D)),
            (p + "W_gate", (D, F)), (p + "W_up", (D, F)), (p + "W_down", (F, D)),
            (p + "norm1", (D,)), (p + "norm2", (D,)),
        ]
    return leaves


def numel(shape: Sequence[int]) -> int:
    return int(math.prod(shape))


def adamw_state(shapes: Sequence[Sequence[int]], theta_dtype=torch.float32, grad_dtype=torch.float32,
                mv_dtype=torch.float32, device="cpu", seed: int = SEED_BASE) -> List[Dict[str, torch.Tensor]]:
    """theta N(0,0.02), grad N(0,1e-2), m N(0,1e-3), v |N(0,1e-4)|; one
    generator per (leaf, slot).  Each leaf slot is its own allocation."""
    out = []
    for i, shp in enumerate(shapes):
        n = numel(shp)
        d = {}
        for slot, (name, std, dt, absval) in enumerate((
                ("theta", 0.02, theta_dtype, False), ("grad", 1e-2, grad_dtype, False),
                ("m", 1e-3, mv_dtype, False), ("v", 1e-4, mv_dtype, True))):
            x = torch.randn(n, generator=_gen(device, seed, i, slot), device=device, dtype=torch.float32)
            if absval:
                x.abs_()
            x.mul_(std)
            d[name] = x.to(dt) if dt != torch.float32 else x
        out.append(d)
    return out


# ------------------------------------------------------------ row workloads
def softmax_scores(rows: int, cols: int, device="cpu", seed: int = SEED_BASE + 1, std: float = 3.0) -> torch.Tensor:
    x = torch.randn(rows, cols, generator=_gen(device, seed, 0), device=device, dtype=torch.float32)
    return x.mul_(std)


def rmsnorm_inputs(rows: int, cols: int, device="cpu", seed: int = SEED_BASE + 3):
    x = torch.randn(rows, cols, generator=_gen(device, seed, 0), device=device).to(torch.bfloat16)
    r = torch.randn(rows, cols, generator=_gen(device, seed, 1), device=device).to(torch.bfloat16)
    g = torch.randn(cols, generator=_gen(device, seed, 2), device=device).mul_(0.1).add_(1.0).to(torch.bfloat16)
    return x, r, g


def chain_inputs(rows: int, cols: int, device="cpu", seed: int = SEED_BASE + 4):
    """A [rows, cols], B [rows, 1], C [1, cols], all U(-1, 1) f32."""
    def u(shape, k):
        t = torch.rand(*shape, generator=_gen(device, seed, k), device=device, dtype=torch.float32)
        return t.mul_(2.0).sub_(1.0)
    return u((rows, cols), 0), u((rows, 1), 1), u((1, cols), 2)


# ------------------------------------------------------------- group DAGs
def softmax_causal_dag(scale: float = 0.125, period: int = 1024) -> List[Node]:
    """scale, causal mask (refused positions become -inf), row max, subtract,
    exp, row sum, divide."""
    return parse_dag(f"""
        %0 = input 0
        %1 = const {float(scale).hex()}
        %2 = mul %0 %1
        %3 = causal_mask %2 {period}
        %4 = row_max %3
        %5 = sub %3 %4
        %6 = exp %5
        %7 = row_sum %6
        %8 = div %6 %7
    """)


def rmsnorm_gelu_dag(eps_f32: float) -> List[Node]:
    """h = x + res; y = h / sqrt(mean(h*h) + eps) * gamma; gelu(y)."""
    return parse_dag(f"""
        %0 = input 0
        %1 = input 1
        %2 = input 2
        %3 = add %0 %1
        %4 = pow2 %3
        %5 = row_mean %4
        %6 = const {float(eps_f32).hex()}
        %7 = add %5 %6
        %8 = sqrt %7
        %9 = div %3 %8
        %10 = mul %9 %2
        %11 = gelu %10
    """)


def f32(x: float) -> float:
    """Round a Python float to the nearest f32 value (an input conversion)."""
    return float(torch.tensor(x, dtype=torch.float32).item())


CHAIN_DAG_SEED = SEED_BASE + 4


def chain_dag_candidate(seed: int = CHAIN_DAG_SEED) -> List[Node]:
    return random_chain_dag(seed)


CHAIN64_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                            "tests", "golden", "chain64_dag.txt")


def chain64_dag() -> List[Node]:
    """The accepted 64-node chain (written by tests/golden/make_chain64_dag.py)."""
    with open(CHAIN64_PATH) as f:
        return parse_dag(f.read())


# ---------------------------------------------------------------------------
# Groups mapped over a parameter tree (one value per leaf element; rank-0
# inputs are one value for the whole tree).
def tree_sgd_dag() -> List[Node]:
    """theta' = theta - lr * g; input 2 (lr) is rank 0."""
    return parse_dag("""
        %0 = input 0
        %1 = input 1
        %2 = input 2
        %3 = mul %2 %1
        %4 = sub %0 %3
    """)


def tree_mixed_dag() -> List[Node]:
    """tanh(x) * exp(-|y|) + gelu(x) * s, with s rank 0: transcendental
    members, a bf16 and an f32 per-element input."""
    return parse_dag("""
        %0 = input 0
        %1 = input 1
        %2 = input 2
        %3 = tanh %0
        %4 = abs %1
        %5 = neg %4
        %6 = exp %5
        %7 = mul %3 %6
        %8 = gelu %0
        %9 = mul %8 %2
        %10 = add %7 %9
    """)


def tree_leaf_values(shapes: Sequence[Sequence[int]], dtype, device="cpu", seed: int = SEED_BASE + 5,
                     std: float = 1.0) -> List[torch.Tensor]:
    """One normal(0, std) tensor per leaf shape, in the given storage type."""
    out = []
    for i, s in enumerate(shapes):
        g = _gen("cpu", seed, i)
        out.append((torch.randn(numel(s), generator=g) * std).to(dtype).to(device))
    return out


# ---------------------------------------------------------------------------
# Multi-output groups.
def layernorm_dag(eps_f32: float) -> List[Node]:
    """(x - mean) / sqrt(mean((x - mean)^2) + eps) * gamma + beta, plus
    rstd = 1 / sqrt(var + eps).  Node 12 is the normalised output (the
    root), node 3 the row mean, node 14 rstd (both one value per row)."""
    return parse_dag(f"""
        %0 = input 0
        %1 = input 1
        %2 = input 2
        %3 = row_mean %0
        %4 = sub %0 %3
        %5 = pow2 %4
        %6 = row_mean %5
        %7 = const {float(eps_f32).hex()}
        %8 = add %6 %7
        %9 = sqrt %8
        %10 = div %4 %9
        %11 = mul %10 %1
        %12 = add %11 %2
        %13 = const 1.0
        %14 = div %13 %9
    """)


LAYERNORM_ROOT, LAYERNORM_MEAN, LAYERNORM_RSTD = 12, 3, 14
RMSNORM_H = 3   # h = x + res in rmsnorm_gelu_dag


def layernorm_inputs(rows: int, cols: int, device="cpu", seed: int = SEED_BASE + 6):
    """x ~ N(1, 2) (rows with a non-zero mean), gamma ~ N(1, 0.1), beta ~
    N(0, 0.1), all bf16."""
    g = _gen("cpu", seed, 0)
    x = (torch.randn(rows, cols, generator=g) * 2.0 + 1.0).to(torch.bfloat16)
    gamma = (torch.randn(cols, generator=g) * 0.1 + 1.0).to(torch.bfloat16)
    beta = (torch.randn(cols, generator=g) * 0.1).to(torch.bfloat16)
    return x.to(device), gamma.to(device), beta.to(device)


def adamw_group_dag() -> List[Node]:
    """The AdamW step as a group over a parameter tree: inputs 0..3 are
    theta, g, m, v (per element), 4..12 the f32 step scalars b1, b2, 1-b1,
    1-b2, 1-b1^t, 1-b2^t, lr, eps, wd (per tree).  Node 15 is m', node 19
    v' (stored: extra outputs), node 28 theta' (the root)."""
    return parse_dag("""
        %0 = input 0
        %1 = input 1
        %2 = input 2
        %3 = input 3
        %4 = input 4
        %5 = input 5
        %6 = input 6
        %7 = input 7
        %8 = input 8
        %9 = input 9
        %10 = input 10
        %11 = input 11
        %12 = input 12
        %13 = mul %4 %2
        %14 = mul %6 %1
        %15 = add %13 %14
        %16 = mul %5 %3
        %17 = mul %1 %1
        %18 = mul %7 %17
        %19 = add %16 %18
        %20 = div %15 %8
        %21 = div %19 %9
        %22 = sqrt %21
        %23 = add %22 %11
        %24 = div %20 %23
        %25 = mul %12 %0
        %26 = add %24 %25
        %27 = mul %10 %26
        %28 = sub %0 %27
    """)


ADAMW_GROUP_M, ADAMW_GROUP_V, ADAMW_GROUP_THETA = 15, 19, 28


# ---------------------------------------------------------------------------
# Softmax variants: a mask read from a byte buffer, wide rows, bf16 storage.
def softmax_masked_dag(scale: float = 0.125) -> List[Node]:
    """Input 0 the scores, input 1 a mask (u8, broadcast into the scores):
    scale, -inf where the mask refuses, row max, subtract, exp, row sum,
    divide, then 0 where the mask refuses (so a row it empties is zeros)."""
    return parse_dag(f"""
        %0 = input 0
        %1 = input 1
        %2 = const {float(scale).hex()}
        %3 = mul %0 %2
        %4 = where %1 %3 -inf
        %5 = row_max %4
        %6 = sub %4 %5
        %7 = exp %6
        %8 = row_sum %7
        %9 = div %7 %8
        %10 = where %1 %9 0.0
    """)


def causal_mask_bytes(T: int, device="cpu") -> torch.Tensor:
    """[T, T] bool, true where column <= row (the causal_mask op's pattern)."""
    return torch.ones(T, T, dtype=torch.bool, device=device).tril()


def padding_mask(lengths: Sequence[int], T: int, device="cpu") -> torch.Tensor:
    """[B, 1, 1, T] bool key-padding mask: row b allows its first lengths[b]
    columns (broadcast over heads and query positions)."""
    m = torch.arange(T)[None, :] < torch.tensor(list(lengths))[:, None]
    return m[:, None, None, :].to(device)


def random_mask(rows: int, cols: int, p_keep: float = 0.5, empty_rows: Sequence[int] = (), device="cpu",
                seed: int = SEED_BASE + 7) -> torch.Tensor:
    """[rows, cols] bool, each position allowed with probability p_keep; the
    listed rows refuse everything."""
    g = _gen("cpu", seed, 0)
    m = torch.rand(rows, cols, generator=g) < p_keep
    for r in empty_rows:
        m[r] = False
    return m.to(device)


def softmax_dag(scale: float = 0.125) -> List[Node]:
    """The plain row softmax (no mask): scale, row max, subtract, exp, row
    sum, divide."""
    return parse_dag(f"""
        %0 = input 0
        %1 = const {float(scale).hex()}
        %2 = mul %0 %1
        %3 = row_max %2
        %4 = sub %2 %3
        %5 = exp %4
        %6 = row_sum %5
        %7 = div %5 %6
    """)


# ---------------------------------------------------------------------------
# A measurement workload: the VALU rate an emitted pointwise kernel sustains.
def valu_ceiling_dag(chains: int = 8, depth: int = 7) -> List[Node]:
    """64 members of add and mul only: x = B + C over a [R, 1] and a [1, N]
    input (so the output's bytes are the only HBM traffic an element costs),
    then `chains` independent chains of `depth` alternating
    multiplications and additions by constants starting from x (values stay
    within a few units: each chain contracts towards a fixed point), summed
    pairwise at the end.  Every member is one f32 operation, so it is one
    vector instruction of the emitted kernel."""
    lines = ["%0 = input 0", "%1 = input 1", "%2 = add %0 %1"]
    consts = {}

    def const(v):
        if v not in consts:
            consts[v] = len(lines)
            lines.append(f"%{len(lines)} = const {float(v).hex()}")
        return consts[v]

    ends = []
    for c in range(chains):
        cur = 2
        for d in range(depth):
            if d % 2 == 0:
                k = const(0.5 + 0.0625 * ((c + d) % 7))
                lines.append(f"%{len(lines)} = mul %{cur} %{k}")
            else:
                k = const(-0.375 + 0.125 * ((c * 3 + d) % 7))
                lines.append(f"%{len(lines)} = add %{cur} %{k}")
            cur = len(lines) - 1
        ends.append(cur)
    while len(ends) > 1:
        nxt = []
        for a, b in zip(ends[0::2], ends[1::2]):
            lines.append(f"%{len(lines)} = add %{a} %{b}")
            nxt.append(len(lines) - 1)
        if len(ends) % 2:
            nxt.append(ends[-1])
        ends = nxt
    return parse_dag("\n".join(lines) + "\n")
