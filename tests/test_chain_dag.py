"""The committed 64-node chain: structure and well-posedness, judged on the oracle."""
import re

import numpy as np

from synth import configs
from synth.dag import CHAIN_OPS, member_count, random_chain_dag


def test_chain64_structure():
    nodes = configs.chain64_dag()
    assert member_count(nodes) == 64
    assert sum(1 for n in nodes if n.op == "input") == 3
    reads = [0] * len(nodes)
    for n in nodes:
        for a in n.args:
            reads[a] += 1
    assert all(r >= 1 for r in reads[:-1]) and reads[-1] == 0      # one root, nothing dead
    assert 12 <= sum(1 for r in reads if r == 2) <= 14              # about a fifth read twice
    assert {n.op for n in nodes if n.op != "input"} <= set(CHAIN_OPS)
    # reproducible from the seed recorded in the header
    seed = int(re.search(r"seed=(\d+)", open(configs.CHAIN64_PATH).read()).group(1))
    assert random_chain_dag(seed) == nodes


def test_chain64_interval_bound(orc):
    bounds = orc.interval_bounds(configs.chain64_dag(), [(-1.0, 1.0)] * 3)
    assert max(max(abs(lo), abs(hi)) for lo, hi in bounds) <= 1e4


def test_chain64_f32_oracle_near_f64(orc):
    nodes = configs.chain64_dag()
    A, B, C = configs.chain_inputs(64, 4096, seed=77)
    A, B, C = A.numpy(), B.numpy(), C.numpy()
    got = orc.eval_group(nodes, [A, B, C], A.shape).astype(np.float64)
    ref = orc.eval_group_f64(nodes, [A, B, C], A.shape)
    assert np.all(np.abs(got - ref) <= 0.25 * (1e-7 + 2e-6 * np.abs(ref)))
