"""Neutral form of a fusion group's op DAG: a let-list in static single assignment.

A group is written as a first-order let-list, one binding per line, each
operand naming an earlier binding (the shape of PSK-Core's ANF, presk
language reference, section "PSK-Core").  Text form::

    %0 = input 0          # group input slot 0
    %1 = const 0x1p-3     # an f32 immediate (hex or decimal)
    %2 = mul %0 %1
    %3 = causal_mask %2 1024
    %4 = row_max %3

Nothing here evaluates a node: the oracle and the GPU library each map these
names to their own op codes.
"""
from __future__ import annotations

import dataclasses
import random
from typing import List, Optional, Sequence, Tuple

# name -> (arity, kind).  kind: "leaf" (input/const), "ew" (elementwise),
# "row" (last-axis keepdim reduction), "nonew" (a boundary: only the
# partition reads it).
OPS = {
    "input": (0, "leaf"),
    "const": (0, "leaf"),
    "add": (2, "ew"), "sub": (2, "ew"), "mul": (2, "ew"), "div": (2, "ew"),
    "max": (2, "ew"), "min": (2, "ew"),
    "neg": (1, "ew"), "abs": (1, "ew"), "exp": (1, "ew"), "log": (1, "ew"),
    "sqrt": (1, "ew"), "tanh": (1, "ew"), "erf": (1, "ew"), "gelu": (1, "ew"),
    "sqrtabs": (1, "ew"), "pow2": (1, "ew"), "pown": (1, "ew"),
    "select": (3, "ew"), "causal_mask": (1, "ew"), "where": (2, "ew"),
    "row_max": (1, "row"), "row_sum": (1, "row"), "row_mean": (1, "row"),
    # boundaries, only meaningful to the partition
    "reduce": (1, "nonew"), "matmul": (2, "nonew"), "cast": (1, "nonew"),
    "opaque": (-1, "nonew"),
}

# ops that carry an integer parameter after their operands
_IPARAM_OPS = {"input", "pown", "causal_mask"}
# ops that carry a float immediate after their operands
_IMM_OPS = {"const", "where"}


@dataclasses.dataclass(frozen=True)
class Node:
    op: str
    args: Tuple[int, ...] = ()
    imm: Optional[float] = None      # const value (already an f32 value); where's fill value
    iparam: Optional[int] = None     # input slot, pown exponent, causal period

    def __post_init__(self):
        if self.op not in OPS:
            raise ValueError(f"unknown op {self.op!r}")
        arity = OPS[self.op][0]
        if arity >= 0 and len(self.args) != arity:
            raise ValueError(f"{self.op} takes {arity} operands, got {len(self.args)}")


def _fmt_imm(x: float) -> str:
    return float(x).hex()


def format_dag(nodes: Sequence[Node]) -> str:
    lines = []
    for i, n in enumerate(nodes):
        parts = [f"%{i} =", n.op]
        parts += [f"%{a}" for a in n.args]
        if n.op in _IMM_OPS:
            parts.append(_fmt_imm(n.imm))
        if n.op in _IPARAM_OPS:
            parts.append(str(int(n.iparam)))
        lines.append(" ".join(parts))
    return "\n".join(lines) + "\n"


def parse_dag(text: str) -> List[Node]:
    nodes: List[Node] = []
    for raw in text.splitlines():
        line = raw.split("#", 1)[0].strip()
        if not line:
            continue
        lhs, rhs = [s.strip() for s in line.split("=", 1)]
        if lhs != f"%{len(nodes)}":
            raise ValueError(f"bindings must be numbered in order: got {lhs!r}")
        toks = rhs.split()
        op, rest = toks[0], toks[1:]
        args = tuple(int(t[1:]) for t in rest if t.startswith("%"))
        extra = [t for t in rest if not t.startswith("%")]
        imm = iparam = None
        if op in _IMM_OPS:
            s = extra.pop(0)
            imm = float.fromhex(s) if "0x" in s.lower() else float(s)
        if op in _IPARAM_OPS:
            iparam = int(extra.pop(0))
        if extra:
            raise ValueError(f"trailing tokens in {raw!r}")
        nodes.append(Node(op, args, imm, iparam))
    return nodes


def member_count(nodes: Sequence[Node]) -> int:
    return sum(1 for n in nodes if OPS[n.op][1] != "leaf")


# ---------------------------------------------------------------------------
# Random 64-node chain (the generic pointwise workload).
# Structure only: op kinds and wiring.  Whether a drawn DAG is numerically
# well posed is decided by a separate acceptance step on the oracle side.
# ---------------------------------------------------------------------------
CHAIN_OPS = ("add", "mul", "exp", "gelu", "sqrtabs", "tanh", "pow2")


def random_chain_dag(seed: int, n_members: int = 64, n_inputs: int = 3,
                     reread_target: Tuple[int, int] = (12, 14),
                     p_reread: float = 0.5, max_tries: int = 10000) -> List[Node]:
    """Draw a connected DAG of ``n_members`` elementwise nodes over
    ``n_inputs`` inputs, a single root and no dead value.

    Contract: op kinds uniform over CHAIN_OPS (binary ops are forced near the
    end when more than one value is still unread); each operand is taken from
    the values nobody has read yet, except that a binary node's second
    operand re-reads an already-read value with probability ``p_reread`` (a
    value is read at most twice); the DAG is kept only when the number of
    values read exactly twice lies in ``reread_target``.  Deterministic in
    ``seed``.
    """
    for attempt in range(max_tries):
        rng = random.Random(seed * 1_000_003 + attempt)
        nodes: List[Node] = [Node("input", (), None, k) for k in range(n_inputs)]
        reads = [0] * n_inputs
        unread = list(range(n_inputs))
        ok = True
        for i in range(n_members):
            left = n_members - i
            # binary nodes that consume two unread values are the only way to
            # shrink the unread pool; force them when the pool is too large
            must_merge = len(unread) - 1 >= left
            op = rng.choice(("add", "mul")) if must_merge else rng.choice(CHAIN_OPS)
            if OPS[op][0] == 1:
                a = unread.pop(rng.randrange(len(unread)))
                args = (a,)
            else:
                a = unread.pop(rng.randrange(len(unread)))
                once = [v for v in range(len(nodes)) if reads[v] == 1 and v != a]
                if (not must_merge and once and rng.random() < p_reread) or not unread:
                    if not once:
                        ok = False
                        break
                    b = rng.choice(once)
                else:
                    b = unread.pop(rng.randrange(len(unread)))
                args = (a, b)
            for v in args:
                reads[v] += 1
            nodes.append(Node(op, args))
            reads.append(0)
            unread.append(len(nodes) - 1)
        if not ok or len(unread) != 1 or unread[0] != len(nodes) - 1:
            continue
        twice = sum(1 for r in reads if r == 2)
        if reread_target[0] <= twice <= reread_target[1]:
            return nodes
    raise RuntimeError("no DAG met the structural contract")
