"""Launch-configuration independence on the GPU: the same group gives the
same bits under every launch layout that changes no reduction bracketing
(workgroup size, XCD mapping, nontemporal accesses, elements per thread in
tree kernels, rows per workgroup), and out-of-place runs leave their inputs
unchanged."""
import numpy as np
import pytest
import torch

from synth import configs
from tests.gpu_util import assert_bits, to_np

P = pytest.importorskip("elementwise_reduction_groups_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
EPS = configs.f32(1e-5)


def run_layouts(make, layouts, monkeypatch):
    results = []
    for lay in layouts:
        monkeypatch.setenv("PSK_LAYOUT", lay)
        results.append(make())
    for lay, r in zip(layouts[1:], results[1:]):
        for a, b in zip(results[0], r):
            assert_bits(a, b, f"layout {lay!r} vs {layouts[0]!r}")


def test_pointwise_chain_layouts(monkeypatch):
    A, B, C = configs.chain_inputs(257, 1029, device=DEV)
    before = [to_np(t) for t in (A, B, C)]

    def make():
        g = P.Group(configs.chain64_dag(), [((257, 1029), "f32"), ((257, 1), "f32"), ((1, 1029), "f32")], (257, 1029),
                    "f32")
        out = torch.full((257, 1029), float("nan"), device=DEV)
        g.run([A, B, C], out)
        torch.cuda.synchronize()
        return [to_np(out)]
    run_layouts(make, ["", "block=64", "block=1024", "xcd=0", "xcd=1", "nt=0", "block=128,xcd=0,nt=0"], monkeypatch)
    for t, b in zip((A, B, C), before):
        assert_bits(to_np(t), b, "inputs unchanged")


def test_tree_group_layouts(monkeypatch):
    sizes = [(1,), (7,), (4095,), (4097,), (20000,)]
    theta = configs.tree_leaf_values(sizes, torch.bfloat16, DEV, seed=61)
    grad = configs.tree_leaf_values(sizes, torch.float32, DEV, seed=62)
    lr = torch.tensor(0.01, device=DEV)
    before = [to_np(t) for t in theta + grad]

    def make():
        g = P.Group(configs.tree_mixed_dag(), [((1,), "f32"), ((1,), "bf16"), ((), "f32")], (1,), "bf16", tree=True)
        outs = [torch.full_like(t, float("nan")) for t in theta]
        tree = P.Tree([[gr, t, o] for gr, t, o in zip(grad, theta, outs)])
        g.run_tree(tree, [0, 1, -1], 2, [None, None, lr])
        torch.cuda.synchronize()
        return [to_np(o) for o in outs]
    run_layouts(make, ["", "tper=4", "tper=8", "tper=16", "block=128", "block=256", "xcd=1", "xcd=1,block=128",
                       "nt=0", "sc1=1", "sc1=0", "tper=2,sc1=1"], monkeypatch)
    for t, b in zip(theta + grad, before):
        assert_bits(to_np(t), b, "inputs unchanged")


def test_row_group_rows_per_workgroup(monkeypatch):
    # 16-lane rows: the workgroup size decides how many rows share it
    R, C = 333, 100
    x, r, gm = configs.rmsnorm_inputs(R, C, device=DEV, seed=63)
    before = [to_np(t) for t in (x, r, gm)]

    def make():
        g = P.Group(configs.rmsnorm_gelu_dag(EPS), [((R, C), "bf16"), ((R, C), "bf16"), ((C,), "bf16")], (R, C),
                    "bf16")
        out = torch.full((R, C), float("nan"), dtype=torch.bfloat16, device=DEV)
        g.run([x, r, gm], out)
        torch.cuda.synchronize()
        return [to_np(out)]
    run_layouts(make, ["", "block=64", "block=512", "block=1024", "xcd=1", "nt=0"], monkeypatch)
    for t, b in zip((x, r, gm), before):
        assert_bits(to_np(t), b, "inputs unchanged")


def test_adamw_kernel_block_orders(monkeypatch):
    """The hand-written AdamW kernel with workgroups in round-robin order
    (the default) and with each XCD taking a contiguous eighth of the
    chunks: the same bits, every leaf of a ragged tree."""
    sizes = [(1,), (7,), (4095,), (4097,), (20000,), (70000,)]
    init = [configs.tree_leaf_values(sizes, dt, DEV, seed=71 + k)
            for k, dt in enumerate([torch.bfloat16, torch.bfloat16, torch.float32, torch.float32])]
    results = []
    for lay in ["", "axcd=1"]:
        monkeypatch.setenv("PSK_LAYOUT", lay)
        th, g, m, v = [[t.clone() for t in ts] for ts in init]
        v = [t.abs() for t in v]
        tree = P.Tree([list(x) for x in zip(th, g, m, v)])
        tree.adamw_step(3e-4, 0.9, 0.999, 1e-8, 0.01, 10)
        torch.cuda.synchronize()
        results.append([to_np(t) for t in th + m + v])
    for a, b in zip(*results):
        assert_bits(a, b, "AdamW: round-robin against XCD-contiguous blocks")
