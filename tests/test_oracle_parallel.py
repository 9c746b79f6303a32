"""The threaded oracle driver gives the single-threaded oracle's bits: rows,
elements and leaves are independent in every function it drives."""
import numpy as np
import torch

import oracle
import oracle.parallel as OP
from synth import configs


def same(a, b):
    return np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_ranges_cover_exactly():
    for n in (0, 1, 7, 100, 1001):
        for parts in (1, 3, 16, 2000):
            rs = OP.ranges(n, parts)
            assert sum(b - a for a, b in rs) == n
            assert all(rs[k][1] == rs[k + 1][0] for k in range(len(rs) - 1))


def test_row_groups_threaded_equal_single():
    x = configs.softmax_scores(3 * 257, 300, seed=3).numpy()
    assert same(OP.softmax_causal(x, 257, 0.125, 5), oracle.softmax_causal(x, 257, 0.125))
    xr, rr, g = configs.rmsnorm_inputs(123, 520, seed=4)
    u16 = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    eps = configs.f32(1e-5)
    assert same(OP.rmsnorm_gelu(u16(xr), u16(rr), u16(g), eps, 7), oracle.rmsnorm_gelu(u16(xr), u16(rr), u16(g), eps))
    A, B, C = configs.chain_inputs(45, 333, seed=5)
    ins = [A.numpy(), B.numpy(), C.numpy()]
    nodes = configs.chain64_dag()
    assert same(OP.eval_group(nodes, ins, (45, 333), 0, 6), oracle.eval_group(nodes, ins, (45, 333)))


def test_adamw_threaded_equal_single():
    st = configs.adamw_state([(300, 33), (77,), (5000,)], theta_dtype=torch.bfloat16, grad_dtype=torch.bfloat16,
                             mv_dtype=torch.float32, seed=6)
    u16 = lambda t: t.view(torch.int16).numpy().view(np.uint16).reshape(-1)
    leaves = [(u16(s["theta"]), u16(s["grad"]), s["m"].numpy().reshape(-1), s["v"].numpy().reshape(-1)) for s in st]
    HP = configs.ADAMW_HP
    hp = (HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"], HP["t"])
    got = OP.adamw_leaves(leaves, hp, 4, block=1024)     # leaves split across blocks
    for leaf, outs in zip(leaves, got):
        for a, b in zip(outs, oracle.adamw(*leaf, *hp)):
            assert same(a, b)
