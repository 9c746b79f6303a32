"""GPU parity of generic tree-mapped groups (psk_group_run_tree: one launch
maps a group over every leaf of a parameter tree) against the oracle's
per-leaf evaluation.  Groups of IEEE operations only (add, sub, mul, bf16
rounding) are compared bit for bit; groups with transcendental members to
the f32 / bf16 bars of the other group tests."""
import numpy as np
import pytest
import torch

import oracle
from synth import configs
from tests.gpu_util import assert_bf16_close, assert_bits, assert_f32_close, to_np

P = pytest.importorskip("elementwise_reduction_groups_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
F32, BF16 = P.PSK_F32, P.PSK_BF16
TDT = {torch.float32: "f32", torch.bfloat16: "bf16"}
RAGGED = [(1,), (3,), (7,), (9,), (511,), (513,), (4095,), (4096,), (4097,), ((1 << 18) + 5,), (64, 3)]


def sgd_group(theta_dt, grad_dt, lr_dt=torch.float32):
    return P.Group(configs.tree_sgd_dag(), [((1,), TDT[theta_dt]), ((1,), TDT[grad_dt]), ((), TDT[lr_dt])],
                   (1,), TDT[theta_dt], tree=True)


def mixed_group(out_dt):
    return P.Group(configs.tree_mixed_dag(), [((1,), "f32"), ((1,), "bf16"), ((), "f32")], (1,), TDT[out_dt],
                   tree=True)


def scalar(v, dt=torch.float32):
    return torch.tensor(v, dtype=dt, device=DEV)


@pytest.mark.parametrize("theta_dt,grad_dt", [(torch.bfloat16, torch.bfloat16), (torch.float32, torch.bfloat16),
                                              (torch.float32, torch.float32), (torch.bfloat16, torch.float32)])
def test_sgd_in_place_ragged_bit_exact(theta_dt, grad_dt):
    theta = configs.tree_leaf_values(RAGGED, theta_dt, DEV, seed=31)
    grad = configs.tree_leaf_values(RAGGED, grad_dt, DEV, seed=32, std=0.1)
    lr = scalar(0.0123)
    t_np, g_np = [to_np(t) for t in theta], [to_np(g) for g in grad]
    g = sgd_group(theta_dt, grad_dt)
    assert g.info.kind == 2
    tree = P.Tree([[t, gr] for t, gr in zip(theta, grad)])
    g.run_tree(tree, [0, 1, -1], 0, [None, None, lr])
    torch.cuda.synchronize()
    ref = oracle.tree_map_group(configs.tree_sgd_dag(), [[t, gr, None] for t, gr in zip(t_np, g_np)],
                                [None, None, np.float32(0.0123)], F32 if theta_dt == torch.float32 else BF16)
    for i, (t, r) in enumerate(zip(theta, ref)):
        assert_bits(to_np(t), r, f"leaf {i} theta'")
    for i, (gr, r) in enumerate(zip(grad, g_np)):
        assert_bits(to_np(gr), r, f"leaf {i} g changed")


def test_sgd_bf16_scalar_and_repeat_launches():
    # lr stored as bf16; three launches in a row apply the step three times
    theta = configs.tree_leaf_values(RAGGED[:6], torch.float32, DEV, seed=33)
    grad = configs.tree_leaf_values(RAGGED[:6], torch.float32, DEV, seed=34)
    lr = scalar(0.5, torch.bfloat16)
    g = sgd_group(torch.float32, torch.float32, torch.bfloat16)
    tree = P.Tree([[t, gr] for t, gr in zip(theta, grad)])
    ref = [to_np(t) for t in theta]
    g_np = [to_np(x) for x in grad]
    for _ in range(3):
        g.run_tree(tree, [0, 1, -1], 0, [None, None, lr])
        ref = oracle.tree_map_group(configs.tree_sgd_dag(), [[t, gr, None] for t, gr in zip(ref, g_np)],
                                    [None, None, np.uint16(0x3F00)], F32)
    torch.cuda.synchronize()
    for i, (t, r) in enumerate(zip(theta, ref)):
        assert_bits(to_np(t), r, f"leaf {i} after three steps")


@pytest.mark.parametrize("out_dt", [torch.float32, torch.bfloat16])
def test_mixed_out_of_place_misaligned_poisoned(out_dt):
    # leaves carved from flat buffers at odd element offsets (scalar path)
    # and 16-byte aligned ones (vector path); the output slot is pre-filled
    # with NaN so a skipped element stays NaN
    sizes = [1000, 4097, 17, 8192, 5, 12288, 1]
    total = sum(sizes) + 64
    fx = configs.tree_leaf_values([(total,)], torch.float32, DEV, seed=35, std=2.0)[0]
    fy = configs.tree_leaf_values([(total,)], torch.bfloat16, DEV, seed=36, std=2.0)[0]
    fo = torch.full((total,), float("nan"), dtype=out_dt, device=DEV)
    slots, off = [], 1
    for i, n in enumerate(sizes):
        o = off if i % 2 == 0 else (off + 7) // 8 * 8
        slots.append([fx[o:o + n], fy[o:o + n], fo[o:o + n]])
        off = o + n
    xs, ys = [to_np(s[0]) for s in slots], [to_np(s[1]) for s in slots]
    s = scalar(-0.75)
    tree = P.Tree(slots)
    assert 0 < tree.info.vector_leaves < len(sizes)
    mixed_group(out_dt).run_tree(tree, [0, 1, -1], 2, [None, None, s])
    torch.cuda.synchronize()
    ref = oracle.tree_map_group(configs.tree_mixed_dag(), [[x, y, None] for x, y in zip(xs, ys)],
                                [None, None, np.float32(-0.75)], F32 if out_dt == torch.float32 else BF16)
    for i, (sl, r) in enumerate(zip(slots, ref)):
        got = to_np(sl[2])
        if out_dt == torch.float32:
            assert_f32_close(got, r, f"leaf {i}")
        else:
            assert_bf16_close(got, r, f"leaf {i}")
        assert_bits(to_np(sl[0]), xs[i], f"leaf {i} x changed")
    # the padding around the leaves is never written
    used = torch.zeros(total, dtype=torch.bool)
    off = 1
    for i, n in enumerate(sizes):
        o = off if i % 2 == 0 else (off + 7) // 8 * 8
        used[o:o + n] = True
        off = o + n
    assert torch.isnan(fo.float().cpu()[~used]).all()


def test_special_values():
    # x = +-0 gives tanh 0 and gelu 0, so the result is 0 whatever y; exp of
    # -inf is 0; a NaN in either input gives NaN
    x = torch.tensor([0.0, 0.0, -0.0, float("nan"), 1.0, 3.0, -2.0, 0.5], device=DEV)
    y = torch.tensor([5.0, float("inf"), -float("inf"), 0.0, float("nan"), -float("inf"), float("inf"), 0.0],
                     dtype=torch.bfloat16, device=DEV)
    out = torch.empty(8, device=DEV)
    tree = P.Tree([[x, y, out]])
    mixed_group(torch.float32).run_tree(tree, [0, 1, -1], 2, [None, None, scalar(2.0)])
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = oracle.tree_map_group(configs.tree_mixed_dag(), [[to_np(x), to_np(y), None]],
                                [None, None, np.float32(2.0)], F32)[0]
    assert (got[:3] == 0).all() and (ref[:3] == 0).all()
    assert np.isnan(ref[3]) and np.isnan(ref[4])
    assert_f32_close(got, ref, "special values")


def test_llama_tree_sgd_full_size_sampled():
    """theta' = theta - lr * g over the 145-leaf, 887M-parameter tree (bf16),
    one launch, checked bit for bit on the first and last 64 and 4096 random
    elements of every leaf."""
    shapes = [s for _, s in configs.llama_leaves()]
    theta = configs.tree_leaf_values(shapes, torch.bfloat16, DEV, seed=41)
    grad = configs.tree_leaf_values(shapes, torch.bfloat16, DEV, seed=42, std=0.05)
    gen = torch.Generator(device="cpu").manual_seed(7)
    idx = []
    for t in theta:
        n = t.numel()
        r = torch.randint(0, n, (4096,), generator=gen)
        idx.append(torch.unique(torch.cat([torch.arange(64), torch.arange(n - 64, n), r])).to(DEV))
    before = [(to_np(t[i]), to_np(g[i])) for t, g, i in zip(theta, grad, idx)]
    tree = P.Tree([[t, g] for t, g in zip(theta, grad)])
    assert tree.info.total_numel == 887685120
    sgd_group(torch.bfloat16, torch.bfloat16).run_tree(tree, [0, 1, -1], 0, [None, None, scalar(3e-4)])
    torch.cuda.synchronize()
    ref = oracle.tree_map_group(configs.tree_sgd_dag(), [[t, g, None] for t, g in before],
                                [None, None, np.float32(3e-4)], BF16)
    for leaf, (t, i, r) in enumerate(zip(theta, idx, ref)):
        assert_bits(to_np(t[i]), r, f"leaf {leaf} theta'")


def test_empty_leaves_and_empty_tree():
    theta = [torch.zeros(0, device=DEV), torch.ones(5, device=DEV), torch.zeros(0, device=DEV)]
    grad = [torch.zeros(0, device=DEV), torch.full((5,), 2.0, device=DEV), torch.zeros(0, device=DEV)]
    g = sgd_group(torch.float32, torch.float32)
    g.run_tree(P.Tree([[t, gr] for t, gr in zip(theta, grad)]), [0, 1, -1], 0, [None, None, scalar(0.25)])
    torch.cuda.synchronize()
    assert theta[1].tolist() == [0.5] * 5
    empty = P.Tree([], n_slots=2)
    g.run_tree(empty, [0, 1, -1], 0, [None, None, scalar(0.25)])


def test_refusals_on_device():
    t, gr = torch.ones(16, device=DEV), torch.ones(16, device=DEV)
    tb = torch.ones(16, dtype=torch.bfloat16, device=DEV)
    tree = P.Tree([[t, gr]])
    g = sgd_group(torch.float32, torch.float32)

    def refused(status, fn):
        with pytest.raises(P.PskError) as ei:
            fn()
        assert ei.value.status == status, ei.value.name

    refused(P.PSK_E_SHAPE, lambda: g.run_tree(tree, [0, 2, -1], 0, [None, None, scalar(1.0)]))   # slot 2 of 2
    refused(P.PSK_E_SHAPE, lambda: g.run_tree(tree, [0, 1, -1], 5, [None, None, scalar(1.0)]))
    refused(P.PSK_E_NULL, lambda: g.run_tree(tree, [0, 1, -1], 0, [None, None, None]))
    refused(P.PSK_E_ALIAS, lambda: g.run_tree(tree, [0, 1, -1], 0, [None, None, t[3]]))   # lr inside theta'
    g.run_tree(tree, [0, 1, -1], 0, [None, None, gr[3]])   # lr inside g, which is only read: fine
    torch.cuda.synchronize()
    assert t.tolist() == [0.0] * 16
    refused(P.PSK_E_TYPE, lambda: g.run_tree(P.Tree([[tb, gr]]), [0, 1, -1], 0, [None, None, scalar(1.0)]))
    refused(P.PSK_E_UNSUPPORTED, lambda: g.run([t, gr, scalar(1.0)], t))          # tree groups run on trees
    plain = P.Group(configs.tree_sgd_dag(), [((16,), "f32"), ((16,), "f32"), ((), "f32")], (16,), "f32")
    refused(P.PSK_E_UNSUPPORTED, lambda: plain.run_tree(tree, [0, 1, -1], 0, [None, None, scalar(1.0)]))
