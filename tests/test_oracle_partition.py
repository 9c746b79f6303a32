"""Pins for the oracle's fusion-group partition (PSK-Realize, "What a group is").

The pages give the conditions a group satisfies, not a procedure.  The
oracle's greedy scan is checked against exhaustive enumeration of every
partition of small random bodies: the greedy result must satisfy the
conditions, and no valid partition may have fewer groups.
"""
import random

import numpy as np
import pytest

from synth.dag import Node, OPS


def set_partitions(items):
    if not items:
        yield []
        return
    first, rest = items[0], items[1:]
    for part in set_partitions(rest):
        for i in range(len(part)):
            yield part[:i] + [[first] + part[i]] + part[i + 1:]
        yield [[first]] + part


def node_class(nd):
    k = OPS[nd.op][1]
    if k == "leaf":
        return "leaf"
    if k == "ew" and not (nd.op == "pown" and nd.iparam > 2):
        return "ew"
    return "boundary"


def valid(nodes, types, is_output, groups, cap=64):
    """The three membership conditions, one root per group, the cap, and
    boundaries (reductions, pow n>2, ...) alone."""
    readers = [[] for _ in nodes]
    for j, nd in enumerate(nodes):
        for a in nd.args:
            readers[a].append(j)
    gid = {}
    for k, g in enumerate(groups):
        for i in g:
            gid[i] = k
    for g in groups:
        if len(g) > cap:
            return False
        cls = [node_class(nodes[i]) for i in g]
        if len(g) > 1 and any(c != "ew" for c in cls):
            return False
        if len({types[i] for i in g}) != 1:
            return False
        roots = [i for i in g if is_output[i] or not readers[i]
                 or any(gid.get(r) != gid[i] for r in readers[i])]
        if len(roots) != 1:
            return False
    return True


def random_body(rng, n):
    nodes, types, outs = [], [], []
    n_leaves = rng.randint(1, 2)
    for i in range(n_leaves):
        nodes.append(Node("input", (), None, i))
        types.append(0)
        outs.append(False)
    while len(nodes) < n:
        r = rng.random()
        if r < 0.12:
            op = "row_sum"
        elif r < 0.18:
            op = None
        else:
            op = rng.choice(["add", "mul", "exp", "tanh", "sub"])
        i = len(nodes)
        if op is None:
            a = rng.randrange(i)
            nodes.append(Node("pown", (a,), None, 3))
        elif OPS[op][0] == 1:
            nodes.append(Node(op, (rng.randrange(i),)))
        else:
            nodes.append(Node(op, (rng.randrange(i), rng.randrange(i))))
        types.append(0 if rng.random() < 0.8 else 1)
        outs.append(rng.random() < 0.15)
    outs[-1] = True
    return nodes, types, outs


def groups_from(group_of):
    gs = {}
    for i, g in enumerate(group_of):
        if g >= 0:
            gs.setdefault(int(g), []).append(i)
    return [gs[k] for k in sorted(gs)]


@pytest.mark.parametrize("n", [3, 4, 5, 6, 7, 8])
def test_greedy_is_valid_and_minimal(orc, n):
    rng = random.Random(100 + n)
    n_bodies = 150 if n <= 6 else 40
    for _ in range(n_bodies):
        nodes, types, outs = random_body(rng, n)
        g, r = orc.partition(nodes, types, outs)
        greedy = groups_from(g)
        assert valid(nodes, types, outs, greedy)
        members = [i for i, nd in enumerate(nodes) if node_class(nd) != "leaf"]
        best = min(len(p) for p in set_partitions(members) if valid(nodes, types, outs, p))
        assert len(greedy) == best
        # roots flagged are exactly one per group, the group's last member
        for grp in greedy:
            assert [i for i in grp if r[i]] == [max(grp)]
        # groups are numbered by their root's position
        assert [max(grp) for grp in greedy] == sorted(max(grp) for grp in greedy)


@pytest.mark.parametrize("length,sizes", [(63, [63]), (64, [64]), (65, [1, 64]), (129, [1, 64, 64])])
def test_cap_on_chains(orc, length, sizes):
    # past sixty-four nodes the group stops growing
    nodes = [Node("input", (), None, 0)] + [Node("exp", (i,)) for i in range(length)]
    types = [0] * len(nodes)
    outs = [False] * len(nodes)
    outs[-1] = True
    g, r = orc.partition(nodes, types, outs)
    assert [len(x) for x in groups_from(g)] == sizes
    assert g[0] == -1


def test_conditions_each_cut_a_group(orc):
    # x - mu read by two consumers on both sides of a reduction cannot be
    # interior (PSK-Realize, "What it removes": layer normalization)
    text = [Node("input", (), None, 0),        # 0 x
            Node("row_mean", (0,)),            # 1 mu (boundary)
            Node("sub", (0, 1)),               # 2 x - mu
            Node("pow2", (2,)),                # 3
            Node("row_mean", (3,)),            # 4 var (boundary)
            Node("sqrt", (4,)),                # 5
            Node("div", (2, 5))]               # 6
    types = [0] * 7
    outs = [False] * 6 + [True]
    g, r = orc.partition(text, types, outs)
    gs = groups_from(g)
    # {mu} {x-mu} {pow2} {var} {sqrt, div}: x-mu is read by pow2 (cut by the
    # reduction that reads pow2) and by div
    assert gs == [[1], [2], [3], [4], [5, 6]]
    # an output cannot be interior; a type change cuts the chain; pow 3 stays alone
    nodes = [Node("input", (), None, 0), Node("exp", (0,)), Node("tanh", (1,)), Node("pown", (2,), None, 3),
             Node("exp", (3,)), Node("mul", (4, 4))]
    g, _ = orc.partition(nodes, [0, 0, 0, 0, 0, 0], [False, False, True, False, False, True])
    assert groups_from(g) == [[1, 2], [3], [4, 5]]
    g, _ = orc.partition(nodes, [0, 0, 1, 1, 1, 1], [False] * 5 + [True])
    assert groups_from(g) == [[1], [2], [3], [4, 5]]


# ---------------------------------------------------- partition with rows fused
# The pages name reduction fusion as future work (PSK-Realize, "Not in this
# version") and poot fuses reduction-rooted regions ("Fusion and Planning",
# "Reduction-rooted regions").  The reading taken: a last-axis row reduction
# and a value of the group's rows (the root's shape with a last axis of 1,
# any storage type) join a group under the same reader rule as an element
# member, a reduction only when it reduces a value of the root's shape.
# valid_rows states these conditions directly; the oracle's greedy scan is
# checked against every partition of small random bodies.
def valid_rows(nodes, types, is_output, groups, cap=64):
    readers = [[] for _ in nodes]
    for j, nd in enumerate(nodes):
        for a in nd.args:
            readers[a].append(j)
    gid = {i: k for k, g in enumerate(groups) for i in g}
    for g in groups:
        if len(g) > cap:
            return False
        roots = [i for i in g if is_output[i] or not readers[i] or any(gid.get(r) != gid[i] for r in readers[i])]
        if len(roots) != 1:
            return False
        if len(g) == 1:
            continue                               # any let alone is a group
        root_shape, root_dt = types[roots[0]]
        row_shape = root_shape[:-1] + (1,) if root_shape and root_shape[-1] > 1 else None
        for i in g:
            nd = nodes[i]
            kind = OPS[nd.op][1]
            if kind == "row":
                # a reduction over a value of the group's shape, its value
                # one per row of the group's rows
                if row_shape is None or types[nd.args[0]][0] != root_shape or types[i][0] != row_shape:
                    return False
            elif kind == "ew" and not (nd.op == "pown" and nd.iparam > 2):
                shape, dt = types[i]
                if (shape, dt) != (root_shape, root_dt) and not (row_shape is not None and shape == row_shape):
                    return False
            else:
                return False                       # contractions, casts, pow n > 2: alone
    return True


RB, CB = 4, 8
SHAPES = [(RB, CB), (RB, 1), (CB,), ()]


def _bcast(a, b):
    n = max(len(a), len(b))
    a, b = (1,) * (n - len(a)) + a, (1,) * (n - len(b)) + b
    return tuple(max(x, y) for x, y in zip(a, b))


def random_row_body(rng, n):
    """Inputs of element, row, column-vector and scalar shapes; elementwise
    lets (their shape the broadcast of their operands'), row reductions of
    any value, a matmul or pow 3 now and then; storage types f32 or bf16."""
    nodes, types, outs = [], [], []
    for k, shape in enumerate([(RB, CB), rng.choice(SHAPES[1:])]):
        nodes.append(Node("input", (), None, k))
        types.append((shape, "f32"))
        outs.append(False)
    while len(nodes) < n:
        i = len(nodes)
        r = rng.random()
        dt = "bf16" if rng.random() < 0.12 else "f32"
        if r < 0.22:
            # mostly over element values, the reductions the row kernels run
            elem = [j for j in range(i) if types[j][0] == (RB, CB)]
            a = rng.choice(elem) if elem and rng.random() < 0.85 else rng.randrange(i)
            nodes.append(Node(rng.choice(["row_max", "row_sum", "row_mean"]), (a,)))
            sh = types[a][0]
            types.append(((sh[:-1] + (1,)) if sh else (), dt))
        elif r < 0.25:
            nodes.append(Node("matmul", (rng.randrange(i), rng.randrange(i))))
            types.append(((RB, CB), dt))
        elif r < 0.27:
            a = rng.randrange(i)
            nodes.append(Node("pown", (a,), None, 3))
            types.append((types[a][0], dt))
        elif r < 0.65:
            # mostly an element value against a row value (x - max x, e / sum e)
            elem = [j for j in range(i) if types[j][0] == (RB, CB)]
            rowv = [j for j in range(i) if types[j][0] == (RB, 1)]
            a = rng.choice(elem) if elem and rng.random() < 0.7 else rng.randrange(i)
            b = rng.choice(rowv) if rowv and rng.random() < 0.5 else rng.randrange(i)
            nodes.append(Node(rng.choice(["add", "mul", "sub", "div"]), (a, b)))
            types.append((_bcast(types[a][0], types[b][0]), dt))
        else:
            a = rng.randrange(i)
            nodes.append(Node(rng.choice(["exp", "tanh", "sqrtabs", "neg"]), (a,)))
            types.append((types[a][0], dt))
        outs.append(rng.random() < 0.08)
    outs[-1] = True
    return nodes, types, outs


@pytest.mark.parametrize("n", [3, 4, 5, 6, 7, 8, 9, 10])
def test_row_fused_greedy_is_valid_and_minimal(orc, n):
    """With rows fused the greedy partition satisfies the conditions and no
    valid partition has fewer groups (bodies of up to 8 lets, every set
    partition of the lets enumerated)."""
    rng = random.Random(700 + n)
    n_bodies = 200 if n <= 7 else (60 if n <= 9 else 25)
    fused_somewhere = 0
    for _ in range(n_bodies):
        nodes, types, outs = random_row_body(rng, n)
        g, r = orc.partition(nodes, types, outs, rows=True)
        greedy = groups_from(g)
        assert valid_rows(nodes, types, outs, greedy), (nodes, types, outs, greedy)
        members = [i for i, nd in enumerate(nodes) if node_class(nd) != "leaf"]
        best = min(len(p) for p in set_partitions(members) if valid_rows(nodes, types, outs, p))
        assert len(greedy) == best, (nodes, types, outs, greedy)
        for grp in greedy:
            assert [i for i in grp if r[i]] == [max(grp)]
        fused_somewhere += any(OPS[nodes[i].op][1] == "row" for grp in greedy if len(grp) > 1 for i in grp)
    # the bodies exercise the row rule: some reduction joins a larger group
    if n >= 5:
        assert fused_somewhere >= n_bodies // 10, fused_somewhere


def test_valid_rows_rejects_each_violation():
    """Each condition of valid_rows on its own, on a softmax-shaped body."""
    E, Rw = ((RB, CB), "f32"), ((RB, 1), "f32")
    nodes = [Node("input", (), None, 0), Node("row_max", (0,)), Node("sub", (0, 1)), Node("exp", (2,)),
             Node("row_sum", (3,)), Node("div", (3, 4))]
    types = [E, Rw, E, E, Rw, E]
    outs = [False] * 5 + [True]
    assert valid_rows(nodes, types, outs, [[1, 2, 3, 4, 5]])
    assert not valid_rows(nodes, types, outs, [[1, 2, 3, 4, 5]], cap=4)               # the cap
    assert not valid_rows(nodes, types, [False, False, False, True, False, True],
                          [[1, 2, 3, 4, 5]])                                              # an output inside
    assert valid_rows(nodes, types, outs, [[1, 2], [3, 4, 5]])                            # two valid groups
    assert not valid_rows(nodes, types, outs, [[1, 2, 3, 5], [4]])                        # exp read outside
    assert not valid_rows(nodes, [E, Rw, E, ((RB, CB), "bf16"), Rw, E], outs, [[1, 2, 3, 4, 5]])  # a type
    assert not valid_rows(nodes, [E, Rw, E, E, ((RB, 2), "f32"), E], outs, [[1, 2, 3, 4, 5]])     # a shape
    # a reduction of a row value does not join
    n2 = nodes + [Node("row_sum", (4,)), Node("mul", (5, 6))]
    t2 = types + [Rw, E]
    assert not valid_rows(n2, t2, [False] * 7 + [True], [[1, 2, 3, 4, 5, 6, 7]])
    assert valid_rows(n2, t2, [False] * 7 + [True], [[1, 2, 3], [4], [5, 7], [6]])
    # a matmul never shares a group
    n3 = [Node("input", (), None, 0), Node("matmul", (0, 0)), Node("exp", (1,))]
    assert not valid_rows(n3, [E, E, E], [False, False, True], [[1, 2]])
