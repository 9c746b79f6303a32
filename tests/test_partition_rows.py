"""The partition with fused row reductions and the dispatch-count report
(host logic, no GPU): the library against the oracle's own partition on
random bodies, every fused group accepted by the group validator, and
hand-counted bodies (a layer normalization, a softmax)."""
import random

import numpy as np
import pytest

from synth import configs
from synth.dag import Node, parse_dag

P = pytest.importorskip("elementwise_reduction_groups_amd")

R, C = 16, 64
ELEM, ROW = ((R, C), "f32"), ((R, 1), "f32")


@pytest.fixture(scope="module")
def lib():
    return P.lib()


def layernorm_body():
    nodes = parse_dag(f"""
        %0 = input 0
        %1 = input 1
        %2 = input 2
        %3 = row_mean %0
        %4 = sub %0 %3
        %5 = pow2 %4
        %6 = row_mean %5
        %7 = const {configs.f32(1e-5).hex()}
        %8 = add %6 %7
        %9 = sqrt %8
        %10 = div %4 %9
        %11 = mul %10 %1
        %12 = add %11 %2
    """)
    types = [ELEM, ((C,), "f32"), ((C,), "f32"), ROW, ELEM, ELEM, ROW, ((), "f32"), ROW, ROW, ELEM, ELEM, ELEM]
    outs = [False] * 12 + [True]
    return nodes, types, outs


def test_layernorm_splits_at_each_mean_unless_rows_fuse(lib):
    nodes, types, outs = layernorm_body()
    g, r, ng = P.psk_partition(nodes, types, outs)
    # the mean, x - mean (read by the variance and the division), its square,
    # the variance, +eps and sqrt, then divide, scale and shift
    assert ng == 6
    assert len({g[4], g[5], g[10]}) == 3 and g[8] == g[9] and g[10] == g[11] == g[12]
    rep = P.psk_dispatch_count(nodes, types, outs)
    assert rep["lets"] == 9 and rep["launches_unfused"] == 9 and rep["launches_fused"] == 6
    assert rep["fused_groups"] == 2
    g2, r2, ng2 = P.psk_partition(nodes, types, outs, rows=True)
    assert ng2 == 1 and set(g2[3:7].tolist() + g2[8:].tolist()) == {0}
    rep2 = P.psk_dispatch_count(nodes, types, outs, rows=True)
    assert rep2["launches_fused"] == 1
    # one launch reads x, gamma, beta, eps once and writes the output
    e, row, vec = R * C * 4, R * 4, C * 4
    assert rep2["bytes_fused"] == e + 2 * vec + 4 + e
    # unfused: each let writes its value and reads its operands
    assert rep["bytes_unfused"] == (row + e) + (e + e + row) + (e + e) + (row + e) + (row + row + 4) + \
        (row + row) + (e + e + row) + (e + e + vec) + (e + e + vec)


def test_softmax_body_fuses_to_one_launch(lib):
    nodes = configs.softmax_causal_dag(0.125, C)
    types = [ELEM, ((), "f32"), ELEM, ELEM, ROW, ELEM, ELEM, ROW, ELEM]
    outs = [False] * 8 + [True]
    _, _, ng = P.psk_partition(nodes, types, outs)
    # {mul, mask}, max, {sub, exp}, sum, div: the mask's and exp's values are
    # read by a reduction and by a member, so they end their groups
    assert ng == 5
    _, _, ng2 = P.psk_partition(nodes, types, outs, rows=True)
    assert ng2 == 1


def _random_body(rng, n):
    nodes, types, outs = [Node("input", (), None, 0)], [ELEM], [False]
    nodes.append(Node("input", (), None, 1))
    types.append(ROW)
    outs.append(False)
    for i in range(2, n):
        r = rng.random()
        if r < 0.15:
            a = rng.randrange(i)
            nodes.append(Node(rng.choice(["row_max", "row_sum", "row_mean"]), (a,)))
            types.append(ROW)
        elif r < 0.2:
            nodes.append(Node("matmul", (rng.randrange(i), rng.randrange(i))))
            types.append(ELEM)
        elif r < 0.6:
            a, b = rng.randrange(i), rng.randrange(i)
            nodes.append(Node(rng.choice(["add", "mul", "sub"]), (a, b)))
            types.append(ELEM if (R, C) in (types[a][0], types[b][0]) else ROW)
        else:
            a = rng.randrange(i)
            nodes.append(Node(rng.choice(["exp", "tanh", "sqrtabs"]), (a,)))
            bf = types[a][0] == (R, C) and rng.random() < 0.1      # a bf16 value of the same shape
            types.append(((R, C), "bf16") if bf else types[a])
        outs.append(rng.random() < 0.08)
    outs[-1] = True
    return nodes, types, outs


def test_rows_partition_matches_oracle(lib, orc):
    rng = random.Random(11)
    for trial in range(1500):
        nodes, types, outs = _random_body(rng, rng.randint(3, 70))
        for rows in (False, True):
            g, r, ng = P.psk_partition(nodes, types, outs, rows=rows)
            og, orr = orc.partition(nodes, types, outs, rows=rows)
            np.testing.assert_array_equal(g, og)
            np.testing.assert_array_equal(r, orr)
        # fusing reductions never needs more launches
        assert P.psk_partition(nodes, types, outs, rows=True)[2] <= P.psk_partition(nodes, types, outs)[2]


def _group_desc(nodes, types, g, members, root):
    """The descriptor of one group: its members in order, every value from
    outside it an input."""
    index, out_nodes, inputs = {}, [], []
    for i in members:
        nd = nodes[i]
        args = []
        for a in nd.args:
            if a not in index:
                index[a] = len(out_nodes)
                out_nodes.append(Node("input", (), None, len(inputs)))
                inputs.append(types[a])
            args.append(index[a])
        index[i] = len(out_nodes)
        out_nodes.append(Node(nd.op, tuple(args), nd.imm, nd.iparam))
    return P.GroupDesc(out_nodes, inputs, types[root][0], types[root][1], root=index[root])


def test_every_fused_row_group_is_a_valid_group(lib):
    rng = random.Random(12)
    checked = 0
    for trial in range(600):
        nodes, types, outs = _random_body(rng, rng.randint(3, 50))
        g, r, ng = P.psk_partition(nodes, types, outs, rows=True)
        for gi in range(ng):
            members = [i for i in range(len(nodes)) if g[i] == gi]
            root = [i for i in members if r[i]][0]
            if any(nodes[i].op == "matmul" for i in members):
                assert len(members) == 1
                continue
            if nodes[root].op.startswith("row_") and types[root] == ROW:
                continue       # a reduction alone is a reduction launch, not a row group
            desc = _group_desc(nodes, types, g, members, root)
            assert P.psk_group_source(desc)
            checked += 1
    assert checked > 1000


def test_dispatch_count_refusals(lib):
    with pytest.raises(P.PskError) as ei:
        P.psk_dispatch_count([Node("input", (), None, 0), Node("exp", (1,))], [ELEM, ELEM], [False, True])
    assert ei.value.status == P.PSK_E_ORDER


def test_gpt_body_dispatch_counts(lib, orc):
    """The synthetic GPT forward (V=92, D=64, H=2, L=2, B=2, T=32): the
    library's and the oracle's partitions agree in both modes, and fusing
    reductions removes the launches that the mean and the softmax cut."""
    from synth.body import gpt_forward
    b = gpt_forward()
    for rows in (False, True):
        g, r, ng = P.psk_partition(b.nodes, b.types, b.outputs, rows=rows)
        og, orr = orc.partition(b.nodes, b.types, b.outputs, rows=rows)
        np.testing.assert_array_equal(g, og)
        np.testing.assert_array_equal(r, orr)
    plain = P.psk_dispatch_count(b.nodes, b.types, b.outputs)
    fused = P.psk_dispatch_count(b.nodes, b.types, b.outputs, rows=True)
    assert plain["launches_unfused"] == fused["launches_unfused"] == 103
    # a layer normalization is 6 launches in the presk-style partition and 1
    # with rows fused, the causal softmax 5 and 1 (five of the one and two of
    # the other in this body)
    assert plain["launches_fused"] == 75 and fused["launches_fused"] == 41
    assert fused["bytes_fused"] < plain["bytes_fused"] < plain["bytes_unfused"]
