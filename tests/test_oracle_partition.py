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
