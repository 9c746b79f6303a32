"""GPU parity past 2^31 elements: the emitted pointwise, row and tiled row
kernels index with 64 bits once an output reaches 2^31 - 4096 elements, and
the tree kernels take 64-bit chunk starts.  Outputs are compared on samples
the oracle computes one by one (the first and last elements, those around
2^31, and random ones); every group here is elementwise per sample (or per
row), so the samples' inputs alone determine them."""
import numpy as np
import pytest
import torch

import oracle
from synth import configs
from synth.dag import parse_dag
from tests.gpu_util import assert_bits, assert_f32_close, to_np

P = pytest.importorskip("elementwise_reduction_groups_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
F32, BF16 = P.PSK_F32, P.PSK_BF16
N31 = 1 << 31


def flat_samples(n, seed, k=6000):
    rng = np.random.default_rng(seed)
    idx = np.concatenate([np.arange(64), np.arange(n - 4096, n), np.arange(N31 - 2048, min(n, N31 + 2048)),
                          rng.integers(0, n, k)])
    return torch.from_numpy(np.unique(idx[(idx >= 0) & (idx < n)])).to(DEV)


def free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_pointwise_broadcast_past_2_31():
    R, C = (1 << 21) + 3, 1028               # 2 155 875 340 elements, f32
    dag = parse_dag("%0 = input 0\n%1 = input 1\n%2 = input 2\n%3 = mul %0 %1\n%4 = add %3 %2\n")
    x = torch.randn(R, C, device=DEV, generator=torch.Generator(DEV).manual_seed(1))
    b = torch.randn(C, device=DEV, generator=torch.Generator(DEV).manual_seed(2))
    c = torch.randn(R, 1, device=DEV, generator=torch.Generator(DEV).manual_seed(3))
    out = torch.empty_like(x)
    g = P.Group(dag, [((R, C), "f32"), ((C,), "f32"), ((R, 1), "f32")], (R, C), "f32")
    g.run([x, b, c], out)
    torch.cuda.synchronize()
    idx = flat_samples(R * C, 4)
    r, cc = idx // C, idx % C
    ref = oracle.eval_group(dag, [to_np(x.view(-1)[idx]), to_np(b[cc]), to_np(c[r, 0])], (len(idx),), F32)
    assert_bits(to_np(out.view(-1)[idx]), ref, "pointwise past 2^31")
    del x, out, b, c
    free()


def test_softmax_rows_past_2_31():
    R, C = (1 << 21) + 5, 1024               # 2 147 488 768 elements, f32
    x = configs.softmax_scores(R, C, device=DEV, seed=5)
    out = torch.empty_like(x)
    g = P.Group(configs.softmax_dag(0.125), [((R, C), "f32")], (R, C), "f32")
    assert g.info.kind == 1
    g.run([x], out)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([[0, 1], np.arange(R - 40, R), np.arange((1 << 21) - 8, (1 << 21) + 5),
                                     rng.integers(0, R, 200)]))
    ri = torch.from_numpy(rows).to(DEV)
    ref = oracle.eval_group(configs.softmax_dag(0.125), [to_np(x[ri])], (len(rows), C), F32)
    assert_f32_close(to_np(out[ri]), ref, "softmax rows past 2^31")
    del x, out
    free()


@pytest.mark.parametrize("layout,kind", [("", 4), ("tiled=1", 3)])
def test_wide_rows_past_2_31(layout, kind, monkeypatch):
    """Rows split over workgroups (the default) and the tiled kernel (forced)
    over 2^31 + elements: 64-bit offsets."""
    if layout:
        monkeypatch.setenv("PSK_LAYOUT", layout)
    R, C = 16385, 131072                     # 2 147 614 720 elements, bf16
    x = configs.softmax_scores(R, C, device=DEV, seed=7).to(torch.bfloat16)
    out = torch.empty_like(x)
    g = P.Group(configs.softmax_dag(0.125), [((R, C), "bf16")], (R, C), "bf16")
    assert g.info.kind == kind
    g.run([x], out)
    torch.cuda.synchronize()
    g.check()
    rows = np.array([0, 1, 16382, 16383, 16384])
    ri = torch.from_numpy(rows).to(DEV)
    ref = oracle.eval_group(configs.softmax_dag(0.125), [to_np(x[ri])], (len(rows), C), BF16)
    from tests.gpu_util import assert_bf16_close
    assert_bf16_close(to_np(out[ri]), ref, "tiled rows past 2^31")
    del x, out
    free()


def test_tree_leaf_past_2_31_sgd_and_adamw():
    n = N31 + 100
    theta = [torch.randn(5, device=DEV).to(torch.bfloat16),
             (torch.randn(n, device=DEV, generator=torch.Generator(DEV).manual_seed(8)) * 0.02).to(torch.bfloat16)]
    grad = [torch.randn(5, device=DEV).to(torch.bfloat16),
            (torch.randn(n, device=DEV, generator=torch.Generator(DEV).manual_seed(9)) * 0.01).to(torch.bfloat16)]
    idx = flat_samples(n, 10)
    t0, g0 = to_np(theta[1][idx]), to_np(grad[1][idx])
    lr = torch.tensor(0.0123, device=DEV)
    sgd = P.Group(configs.tree_sgd_dag(), [((1,), "bf16"), ((1,), "bf16"), ((), "f32")], (1,), "bf16", tree=True)
    tree = P.Tree([[t, gr] for t, gr in zip(theta, grad)])
    sgd.run_tree(tree, [0, 1, -1], 0, [None, None, lr])
    torch.cuda.synchronize()
    ref = oracle.eval_group(configs.tree_sgd_dag(), [t0, g0, np.float32(0.0123)], (len(idx),), BF16)
    assert_bits(to_np(theta[1][idx]), ref, "tree SGD past 2^31")
    del tree
    # the hand-written AdamW kernel on the same leaf (theta, g bf16; m, v f32)
    m = [torch.zeros(5, device=DEV), torch.randn(n, device=DEV, generator=torch.Generator(DEV).manual_seed(11)) * 1e-3]
    v = [torch.zeros(5, device=DEV),
         (torch.randn(n, device=DEV, generator=torch.Generator(DEV).manual_seed(12)) * 1e-4).abs_()]
    t0, g0, m0, v0 = to_np(theta[1][idx]), to_np(grad[1][idx]), to_np(m[1][idx]), to_np(v[1][idx])
    HP = configs.ADAMW_HP
    hp = (HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"], HP["t"])
    tree = P.Tree([[theta[k], grad[k], m[k], v[k]] for k in range(2)])
    tree.adamw_step(*hp)
    torch.cuda.synchronize()
    rt, rm, rv = oracle.adamw(t0, g0, m0, v0, *hp)
    assert_bits(to_np(theta[1][idx]), rt, "AdamW theta' past 2^31")
    assert_bits(to_np(m[1][idx]), rm, "AdamW m' past 2^31")
    assert_bits(to_np(v[1][idx]), rv, "AdamW v' past 2^31")
    del tree, theta, grad, m, v
    free()
