"""Seeded random pointwise groups made of IEEE-exact operations (add, sub,
mul, div, max, min, neg, abs, sqrt, pow2, select, where): any output rank,
broadcast inputs of every kind, bf16 and f32 storage, byte masks, extra
stored values.  Both the GPU path and the oracle compute such a group
exactly (one rounding per op, the same rounding of stored values), so the
two must agree bit for bit.  Test infrastructure only: it builds
descriptions and inputs, it evaluates nothing."""
import math
import random
from typing import List, Tuple

from synth.dag import Node

BINARY = ["add", "sub", "mul", "div", "max", "min"]
UNARY = ["neg", "abs", "sqrt", "pow2"]


def _input_shape(rng, out_shape):
    kind = rng.choice(["full", "full", "bcast", "scalar", "col", "rowconst"])
    r = len(out_shape)
    if kind == "full":
        return tuple(out_shape)
    if kind == "scalar":
        return ()
    if kind == "col":
        return (out_shape[-1],)
    if kind == "rowconst":
        return tuple(out_shape[:-1]) + (1,) if r > 1 else (1,)
    k = rng.randint(1, r)                      # right-aligned, some axes broadcast
    return tuple(d if rng.random() < 0.6 else 1 for d in out_shape[r - k:])


def random_group(rng: random.Random):
    """(nodes, inputs [(shape, dtype)], out_shape, out_dtype, extras [(node, dtype)])"""
    rank = rng.randint(1, 4)
    lead = [rng.choice([1, 2, 3, 5, 7, 16, 33]) for _ in range(rank - 1)]
    out_shape = tuple(lead + [rng.choice([1, 3, 8, 12, 64, 100, 129, 256, 1000])])
    out_dtype = rng.choice(["f32", "bf16"])
    inputs, nodes, is_row = [], [], []
    for k in range(rng.randint(1, 4)):
        shape = _input_shape(rng, out_shape) if k else tuple(out_shape)   # input 0 spans the output
        inputs.append((shape, rng.choice(["f32", "bf16"])))
        nodes.append(Node("input", (), None, k))
        is_row.append(len(shape) == 0 or shape[-1] == 1)       # one value per row (or per tensor)
    mask = None
    if rng.random() < 0.35:
        mask = len(nodes)
        mshape = _input_shape(rng, out_shape) or (1,)
        inputs.append((mshape, "u8"))
        nodes.append(Node("input", (), None, len(inputs) - 1))
        is_row.append(mshape[-1] == 1)
    if rng.random() < 0.5:
        nodes.append(Node("const", (), float(rng.choice([0.5, -3.0, 1.25, 0.0, 7.0]))))
        is_row.append(True)
    values = [i for i in range(len(nodes)) if i != mask]
    unread = set(values)
    members = []

    def pick():
        if unread and rng.random() < 0.6:
            return rng.choice(sorted(unread))
        return rng.choice(values)

    def add(op, args, imm=None):
        idx = len(nodes)
        nodes.append(Node(op, tuple(args), imm))
        is_row.append(all(is_row[a] for a in args))
        for a in args:
            unread.discard(a)
        unread.add(idx)
        values.append(idx)
        members.append(idx)
        return idx

    for _ in range(rng.randint(1, 14)):
        r = rng.random()
        if mask is not None and r < 0.15:
            add("where", [mask, pick()], float(rng.choice([0.0, -math.inf, 2.5])))
        elif r < 0.25:
            add("select", [pick(), pick(), pick()])
        elif r < 0.5:
            add(rng.choice(UNARY), [pick()])
        else:
            add(rng.choice(BINARY), [pick(), pick()])
    if mask is not None and not any(nodes[m].op == "where" for m in members):
        add("where", [mask, members[-1]], 0.0)
    # every value read: fold what is unread into the root
    while len(unread) > 1:
        a, b = sorted(unread)[:2]
        add(rng.choice(["add", "mul", "max"]), [a, b])
    root = len(nodes) - 1
    if root not in members or is_row[root]:
        root = add("add", [root, 0])            # input 0 spans the output
    extras = []
    cand = [m for m in members if m != root and not is_row[m]]
    rng.shuffle(cand)
    for m in cand[:rng.randint(0, 2)]:
        extras.append((m, rng.choice(["f32", "bf16"])))
    return nodes, inputs, out_shape, out_dtype, extras


def random_tree_group(rng: random.Random):
    """A random group of the same operations to map over a parameter tree:
    rank-1 inputs (one element per leaf element, f32 or bf16) and rank-0
    inputs (one value for the tree, f32).  (nodes, inputs, out_dtype,
    extras [(node, dtype)])"""
    inputs, nodes, per_tree = [], [], []
    n_el = rng.randint(1, 3)
    for k in range(n_el + rng.randint(0, 2)):
        inputs.append(((1,), rng.choice(["f32", "bf16"])) if k < n_el else ((), "f32"))
        nodes.append(Node("input", (), None, k))
        per_tree.append(k >= n_el)              # one value for the whole tree
    values = list(range(len(nodes)))
    unread = set(values)
    members = []

    def pick():
        if unread and rng.random() < 0.6:
            return rng.choice(sorted(unread))
        return rng.choice(values)

    def add(op, args):
        idx = len(nodes)
        nodes.append(Node(op, tuple(args)))
        per_tree.append(all(per_tree[a] for a in args))
        for a in args:
            unread.discard(a)
        unread.add(idx)
        values.append(idx)
        members.append(idx)
        return idx

    for _ in range(rng.randint(1, 12)):
        r = rng.random()
        if r < 0.1:
            add("select", [pick(), pick(), pick()])
        elif r < 0.4:
            add(rng.choice(UNARY), [pick()])
        else:
            add(rng.choice(BINARY), [pick(), pick()])
    while len(unread) > 1:
        a, b = sorted(unread)[:2]
        add(rng.choice(["add", "mul", "max"]), [a, b])
    if len(nodes) - 1 not in members or per_tree[-1]:
        add("add", [len(nodes) - 1, 0])         # input 0 is per element
    cand = [m for m in members if m != len(nodes) - 1 and not per_tree[m]]
    rng.shuffle(cand)
    extras = [(m, rng.choice(["f32", "bf16"])) for m in cand[:rng.randint(0, 2)]]
    return nodes, inputs, rng.choice(["f32", "bf16"]), extras


def random_row_group(rng: random.Random, masks: bool = False):
    """A random row group: the exact element operations (sqrt of a magnitude
    instead of sqrt, no difference of a value with itself, so that no NaN
    and no signed zero decides a maximum) and row maxima, whose result does
    not depend on the order the lanes combine in.  Row values feed later
    members (one or more reduction phases); stored extras may be element
    values or row values.  With `masks`, the first input passes through one
    causal mask or one byte mask (a u8 input read only by its WHERE), so
    that the kernels skip refused vectors.  (nodes, inputs, out_shape,
    out_dtype, extras [(node, shape, dtype)])"""
    rank = rng.randint(1, 3)
    cols = rng.choice([3, 64, 100, 129, 1000, 4096, 40000])
    lead = [rng.choice([1, 2, 5, 17]) for _ in range(rank - 1)]
    out_shape = tuple(lead + [cols])
    row_shape = tuple(lead + [1])
    out_dtype = rng.choice(["f32", "bf16"])
    inputs, nodes, is_row = [], [], []
    for k in range(rng.randint(1, 3)):
        shape = _input_shape(rng, out_shape) if k else tuple(out_shape)
        inputs.append((shape, rng.choice(["f32", "bf16"])))
        nodes.append(Node("input", (), None, k))
        is_row.append(len(shape) == 0 or shape[-1] == 1)
    if rng.random() < 0.5:
        nodes.append(Node("const", (), float(rng.choice([0.5, -3.0, 1.25, 7.0]))))
        is_row.append(True)
    values = list(range(len(nodes)))
    unread = set(values)
    members = []

    def pick(elem=False):
        pool = [v for v in (sorted(unread) if unread and rng.random() < 0.6 else values) if not elem or not is_row[v]]
        return rng.choice(pool or [0])

    def add(op, args):
        idx = len(nodes)
        nodes.append(Node(op, tuple(args)))
        is_row.append(op == "row_max" or all(is_row[a] for a in args))
        for a in args:
            unread.discard(a)
        unread.add(idx)
        values.append(idx)
        members.append(idx)
        return idx

    if masks:
        if rng.random() < 0.5:
            nodes.append(Node("causal_mask", (0,), None, rng.choice([1, 3, 64, cols])))
        else:
            inputs.append((rng.choice([out_shape, (cols,)]), "u8"))
            nodes.append(Node("input", (), None, len(inputs) - 1))     # read by the WHERE only
            is_row.append(False)
            nodes.append(Node("where", (len(nodes) - 1, 0), rng.choice([float("-inf"), 0.0, 1.5])))
        is_row.append(False)
        unread.discard(0)
        unread.add(len(nodes) - 1)
        values.append(len(nodes) - 1)
        members.append(len(nodes) - 1)
    for _ in range(rng.randint(2, 14)):
        r = rng.random()
        if r < 0.2:
            add("row_max", [pick(elem=True)])
        elif r < 0.3:
            add("select", [pick(), pick(), pick()])
        elif r < 0.5:
            add(rng.choice(["neg", "abs", "sqrtabs", "pow2"]), [pick()])
        else:
            a = pick()
            b = pick()
            op = rng.choice(BINARY)
            if a == b and op == "sub":
                op = "add"
            add(op, [a, b])
    while len(unread) > 1:
        a, b = sorted(unread)[:2]
        add(rng.choice(["add", "mul", "max"]), [a, b])
    root = len(nodes) - 1
    if root not in members or is_row[root]:
        root = add("add", [root, 0])
    extras = []
    cand = [m for m in members if m != root]
    rng.shuffle(cand)
    for m in cand[:rng.randint(0, 2)]:
        extras.append((m, row_shape if is_row[m] else out_shape, rng.choice(["f32", "bf16"])))
    return nodes, inputs, out_shape, out_dtype, extras


def random_online_group(rng: random.Random):
    """A random group holding the online normalizer's pattern: y a random
    chain of element operations over the inputs (sometimes under a causal
    mask, or a byte mask whose refused positions become -inf), then
    m = row_max(y), d = y - m, e = exp(d), s = row_sum(e) and a root from
    e / s (times a further input, or zeroed where the byte mask refuses).
    Extras: members of y's chain in either storage type, and m, d, e or s
    stored as f32 (stored as bf16 they would not pair).  (nodes, inputs,
    out_shape, out_dtype, extras [(node, shape, dtype)])"""
    cols = rng.choice([3, 64, 100, 1000, 1023, 4096, 40000, 70000, 300000])
    lead = [rng.choice([1, 2, 5, 17] if cols < 40000 else [1, 2, 3]) for _ in range(rng.randint(0, 2))]
    out_shape = tuple(lead + [cols])
    row_shape = tuple(lead + [1])
    out_dtype = rng.choice(["f32", "bf16"])
    inputs = [(out_shape, rng.choice(["f32", "bf16"]))]
    nodes = [Node("input", (), None, 0)]
    is_row = [False]
    for k in range(1, rng.randint(1, 3)):
        shape = _input_shape(rng, out_shape)
        inputs.append((shape, rng.choice(["f32", "bf16"])))
        nodes.append(Node("input", (), None, k))
        is_row.append(len(shape) == 0 or shape[-1] == 1)
    if rng.random() < 0.5:
        nodes.append(Node("const", (), float(rng.choice([0.125, -0.5, 1.5, 3.0]))))
        is_row.append(True)

    def add(op, args, imm=None, iparam=None):
        nodes.append(Node(op, tuple(args), imm, iparam))
        is_row.append(op in ("row_max", "row_sum") or all(is_row[a] for a in args))
        return len(nodes) - 1

    chain = []
    y = 0
    unread = set(range(1, len(nodes)))
    for _ in range(rng.randint(0, 4)):
        other = rng.randrange(len(nodes))
        if rng.random() < 0.3:
            y = add(rng.choice(["neg", "abs", "pow2"]), [y])
        else:
            y = add(rng.choice(["add", "sub", "mul", "max", "min"]), [y, other] if rng.random() < 0.5 else [other, y])
            unread.discard(other)
        chain.append(y)
    for leaf in sorted(unread):                  # every input and constant is read
        y = add(rng.choice(["add", "mul"]), [y, leaf])
        chain.append(y)
    if is_row[y]:
        y = add("add", [y, 0])
        chain.append(y)
    mask = None
    r = rng.random()
    if r < 0.25:
        y = add("causal_mask", [y], None, rng.choice([1, 7, 64, cols]))
    elif r < 0.5:
        mshape = rng.choice([out_shape, (cols,), out_shape[-2:]])
        inputs.append((tuple(mshape), "u8"))
        mask = add("input", [], None, len(inputs) - 1)
        is_row[mask] = False
        y = add("where", [mask, y], float("-inf"))
    m = add("row_max", [y])
    d = add("sub", [y, m])
    e = add("exp", [d])
    s = add("row_sum", [e])
    root = add("div", [e, s])
    if rng.random() < 0.3:
        root = add("mul", [root, rng.randrange(len(inputs) - (mask is not None))])
    if mask is not None and rng.random() < 0.6:
        root = add("where", [mask, root], 0.0)
    extras = []
    for node in rng.sample([m, d, e, s] + chain, k=min(rng.randint(0, 2), 4 + len(chain))):
        if node == root:
            continue
        shape = row_shape if is_row[node] else out_shape
        extras.append((node, shape, "f32" if node in (m, d, e, s) else rng.choice(["f32", "bf16"])))
    return nodes, inputs, out_shape, out_dtype, extras
