"""Host-side robustness of the group validator and emitter (no GPU): seeded
random pointwise groups are accepted and emitted; the same descriptors with
random damage (operand indices, op codes, root, shapes, dtypes, extras) are
refused with a status, never a crash, and a refusal creates nothing."""
import copy
import random

import pytest

from synth.dag import Node
from tests.random_groups import random_group

P = pytest.importorskip("elementwise_reduction_groups_amd")


@pytest.fixture(scope="module")
def lib():
    return P.lib()


def test_random_groups_are_accepted_and_emitted(lib):
    rng = random.Random(2024)
    accepted = 0
    for _ in range(400):
        nodes, inputs, shape, dt, extras = random_group(rng)
        d = P.GroupDesc(nodes, inputs, shape, dt, root=len(nodes) - 1,
                        extras=[(m, shape, xdt) for m, xdt in extras])
        src = P.psk_group_source(d)
        assert 'extern "C" __global__' in src
        accepted += 1
    assert accepted == 400


def test_damaged_descriptors_are_refused_not_crashed(lib):
    rng = random.Random(7)
    statuses = set()
    for trial in range(1500):
        nodes, inputs, shape, dt, extras = random_group(rng)
        nodes = list(nodes)
        inputs = list(inputs)
        extras = [(m, shape, xdt) for m, xdt in extras]
        root = len(nodes) - 1
        what = rng.randrange(7)
        if what == 0 and len(nodes) > 1:            # an operand pointing forward or out of range
            i = rng.randrange(len(nodes))
            nd = nodes[i]
            if nd.args:
                args = list(nd.args)
                args[rng.randrange(len(args))] = rng.choice([i, i + 1, len(nodes) + 3, -1, -7])
                nodes[i] = Node(nd.op, tuple(args), nd.imm, nd.iparam)
        elif what == 1:                              # the root not the last unread member
            root = rng.randrange(len(nodes))
        elif what == 2:                              # an input widening the output
            k = rng.randrange(len(inputs))
            s, t = inputs[k]
            inputs[k] = (tuple(s) + (3,) if s else (2, 2), t)
        elif what == 3:                              # an input slot that does not exist
            nodes.append(Node("input", (), None, len(inputs) + 2))
        elif what == 4 and extras:                   # an extra on the root, or twice the same node
            extras.append(rng.choice([(root, shape, "f32"), extras[0]]))
        elif what == 5:                              # a wrong extra shape
            extras.append((rng.randrange(len(nodes)), tuple(shape) + (2,), "f32"))
        else:                                        # a mask read by an arithmetic op
            inputs.append((tuple(shape), "u8"))
            nodes.insert(0, Node("input", (), None, len(inputs) - 1))
            nodes = [nodes[0]] + [Node(n.op, tuple(a + 1 for a in n.args), n.imm, n.iparam) for n in nodes[1:]]
            nodes.append(Node("add", (0, len(nodes) - 1)))
            root = len(nodes) - 1
            extras = [(m + 1, s, t) for m, s, t in extras]
        try:
            d = P.GroupDesc(nodes, inputs, shape, dt, root=root, extras=extras)
        except (ValueError, IndexError):
            continue                                 # the binding's own argument checks
        try:
            P.psk_group_source(d)
            statuses.add("ok")
        except P.PskError as e:
            assert 0 < e.status < len(P.STATUS_NAMES)
            statuses.add(e.status)
            with pytest.raises(P.PskError):
                P.psk_group_create(d)
    assert len(statuses) >= 5
