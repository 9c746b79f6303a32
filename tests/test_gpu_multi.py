"""GPU parity of multi-output groups (extra stored values) against the
oracle, through the C ABI: layer normalization with its row statistics in
one kernel, add + RMSNorm + GELU that also stores h, a pointwise group with
two extra outputs, and the AdamW step written as a tree-mapped group (three
outputs) against both the oracle and the hand-written AdamW kernel."""
import math

import numpy as np
import pytest
import torch

import oracle
from synth import configs
from synth.dag import parse_dag
from tests.gpu_util import assert_bf16_close, assert_bits, to_np

P = pytest.importorskip("elementwise_reduction_groups_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
EPS = configs.f32(1e-5)
U = 2.0 ** -24
F32, BF16 = P.PSK_F32, P.PSK_BF16


def layernorm_group(R, C):
    return P.Group(configs.layernorm_dag(EPS), [((R, C), "bf16"), ((C,), "bf16"), ((C,), "bf16")], (R, C), "bf16",
                   root=configs.LAYERNORM_ROOT,
                   extras=[(configs.LAYERNORM_MEAN, (R, 1), "f32"), (configs.LAYERNORM_RSTD, (R, 1), "f32")])


def assert_layernorm_close(got, ref, x, gm, bt, C, what):
    """bf16 outputs at most one bf16 ulp apart, or apart by no more than the
    two f32 values may differ: the statistics come from sums in different
    orders, each within (C + 16) u of exact, and the output adds y*gamma to
    beta, so near a cancellation the bound is on the terms' magnitudes."""
    d = bf16_ulps_np(got, ref)
    if d.max() <= 1:
        return
    x64 = x.double().cpu()
    y = (x64 - x64.mean(dim=1, keepdim=True)) * torch.rsqrt(x64.var(dim=1, unbiased=False, keepdim=True) + EPS)
    terms = (y * gm.double().cpu()).abs() + bt.double().cpu().abs()
    g = torch.from_numpy((got.astype(np.uint32) << 16).view(np.float32)).double()
    r = torch.from_numpy((ref.astype(np.uint32) << 16).view(np.float32)).double()
    ok = (g - r).abs() <= 2.0 ** -7 * r.abs() + 2 * (C + 16) * U * terms
    assert bool(ok.all()), f"{what}: {int((~ok).sum())} elements outside the bound"


def bf16_ulps_np(a, b):
    def ordered(u):
        s = u.astype(np.int32)
        return np.where(s & 0x8000, -(s & 0x7FFF), s & 0x7FFF)
    return np.abs(ordered(a) - ordered(b))


def reduction_path(info, C):
    """Longest chain of f32 additions from an element to a row sum in the
    row kernel: the lane's own elements in order, the butterfly across the
    lanes of a wave (or a 16-lane row), then the waves one after another."""
    L, V = info.lanes_per_row, info.vec
    per_lane = math.ceil(C / (L * V)) * V
    return per_lane + int(math.log2(min(L, 64))) + max(L // 64 - 1, 0)


def check_stats(info, x, mean, rstd, C, what):
    """GPU statistics against float64, each within the bound its own
    summation tree gives: a sum of C terms along a path of k additions is
    within k u sum|x| of the exact sum (one more rounding for the mean);
    the variance adds the rounding of each deviation and its square, and
    rstd three roundings (add eps, sqrt, divide) and half the variance's."""
    k = reduction_path(info, C)
    x64 = x.double().cpu()
    m64 = x64.mean(dim=1)
    bound = k * U * x64.abs().mean(dim=1) + U * m64.abs() + 1e-30
    dm = (mean.double().cpu()[:, 0] - m64).abs()
    assert torch.all(dm <= bound), f"{what}: mean off by {float((dm / bound).max()):.2f} bounds"
    r64 = 1.0 / torch.sqrt(x64.var(dim=1, unbiased=False) + EPS)
    rel = (rstd.double().cpu()[:, 0] - r64).abs() / r64
    assert rel.max() <= (k + 8) * U, f"{what}: rstd relative error {float(rel.max()):.3g}"


@pytest.mark.parametrize("R,C", [(37, 1000), (5, 64), (130, 4096), (3, 12345), (64, 2048), (9, 100)])
def test_layernorm_with_statistics_small(R, C):
    x, gm, bt = configs.layernorm_inputs(R, C, device=DEV, seed=R + C)
    g = layernorm_group(R, C)
    info = g.info
    assert info.kind == 1 and info.phases == 2
    out = torch.full((R, C), float("nan"), dtype=torch.bfloat16, device=DEV)
    mean = torch.full((R, 1), float("nan"), device=DEV)
    rstd = torch.full((R, 1), float("nan"), device=DEV)
    g.run([x, gm, bt], out, extra_outs=[mean, rstd])
    torch.cuda.synchronize()
    rm, rr = np.zeros((R, 1), np.float32), np.zeros((R, 1), np.float32)
    ref = oracle.eval_group(configs.layernorm_dag(EPS), [to_np(x), to_np(gm), to_np(bt)], (R, C), BF16,
                            root=configs.LAYERNORM_ROOT,
                            extras=[(configs.LAYERNORM_MEAN, rm), (configs.LAYERNORM_RSTD, rr)])
    assert_layernorm_close(to_np(out), ref, x, gm, bt, C, f"layernorm {R}x{C}")
    check_stats(info, x, mean, rstd, C, f"layernorm {R}x{C}")
    # the oracle's statistics satisfy the sequential bound (C - 1 additions)
    assert np.all(np.abs(rm[:, 0].astype(np.float64) - x.double().cpu().mean(dim=1).numpy()) <=
                  C * U * x.double().cpu().abs().mean(dim=1).numpy() + 1e-30)


def test_layernorm_full_size_sampled_rows():
    R, C = 16384, 4096
    x, gm, bt = configs.layernorm_inputs(R, C, device=DEV)
    g = layernorm_group(R, C)
    out = torch.empty((R, C), dtype=torch.bfloat16, device=DEV)
    mean = torch.empty((R, 1), device=DEV)
    rstd = torch.empty((R, 1), device=DEV)
    g.run([x, gm, bt], out, extra_outs=[mean, rstd])
    torch.cuda.synchronize()
    assert g.info.algorithmic_bytes == R * C * 4 + 2 * C * 2 + 2 * R * 4
    check_stats(g.info, x, mean, rstd, C, "layernorm full size")
    rows = np.unique(np.concatenate([[0, 1, R - 1], np.random.default_rng(8).integers(0, R, 300)]))
    idx = torch.from_numpy(rows).to(DEV)
    xs = to_np(x[idx])
    ref = oracle.eval_group(configs.layernorm_dag(EPS), [xs, to_np(gm), to_np(bt)], (len(rows), C), BF16,
                            root=configs.LAYERNORM_ROOT)
    assert_layernorm_close(to_np(out[idx]), ref, x[idx], gm, bt, C, "layernorm sampled rows")


@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("R,C", [(33, 4096), (7, 1000), (260, 512)])
def test_add_rmsnorm_gelu_storing_h(R, C, in_place):
    x, res, gm = configs.rmsnorm_inputs(R, C, device=DEV, seed=R * C + 1)
    xn, rn, gn = to_np(x), to_np(res), to_np(gm)
    g = P.Group(configs.rmsnorm_gelu_dag(EPS), [((R, C), "bf16"), ((R, C), "bf16"), ((C,), "bf16")], (R, C), "bf16",
                extras=[(configs.RMSNORM_H, (R, C), "bf16")])
    out = torch.full((R, C), float("nan"), dtype=torch.bfloat16, device=DEV)
    h = res if in_place else torch.full((R, C), float("nan"), dtype=torch.bfloat16, device=DEV)
    g.run([x, res, gm], out, extra_outs=[h])
    torch.cuda.synchronize()
    rh = np.zeros((R, C), np.uint16)
    ref = oracle.eval_group(configs.rmsnorm_gelu_dag(EPS), [xn, rn, gn], (R, C), BF16,
                            extras=[(configs.RMSNORM_H, rh)])
    assert_bits(to_np(h), rh, f"h {R}x{C}")
    assert_bf16_close(to_np(out), ref, f"out {R}x{C}")
    if not in_place:
        assert_bits(to_np(res), rn, "res untouched")


def test_add_rmsnorm_gelu_storing_h_in_f32():
    # an f32 stored value under a bf16 root (8 f32 per lane vector); readers
    # see the f32 value, so the output is the single-output group's up to
    # the forms each takes (an f32 result keeps the f32 gelu and exact
    # division): within one bf16 ulp of it and of the oracle
    R, C = 48, 4096
    x, res, gm = configs.rmsnorm_inputs(R, C, device=DEV, seed=77)
    g = P.Group(configs.rmsnorm_gelu_dag(EPS), [((R, C), "bf16"), ((R, C), "bf16"), ((C,), "bf16")], (R, C), "bf16",
                extras=[(configs.RMSNORM_H, (R, C), "f32")])
    out = torch.full((R, C), float("nan"), dtype=torch.bfloat16, device=DEV)
    h = torch.full((R, C), float("nan"), device=DEV)
    g.run([x, res, gm], out, extra_outs=[h])
    single = P.Group(configs.rmsnorm_gelu_dag(EPS), [((R, C), "bf16"), ((R, C), "bf16"), ((C,), "bf16")], (R, C),
                     "bf16")
    out1 = torch.empty_like(out)
    single.run([x, res, gm], out1)
    torch.cuda.synchronize()
    assert torch.equal(h, x.float() + res.float())
    assert_bf16_close(to_np(out), to_np(out1), "f32 h vs single output")
    ref = oracle.eval_group(configs.rmsnorm_gelu_dag(EPS), [to_np(x), to_np(res), to_np(gm)], (R, C), BF16)
    assert_bf16_close(to_np(out), ref, "f32 h vs oracle")


def test_pointwise_two_extra_outputs_bit_exact():
    # a = x*y stored bf16 (read rounded), b = a + x stored f32, root b*b - a;
    # a ragged shape (element path) and a 16-byte one (vector path)
    nodes = parse_dag("%0 = input 0\n%1 = input 1\n%2 = mul %0 %1\n%3 = add %2 %0\n%4 = mul %3 %3\n%5 = sub %4 %2\n")
    for R, C in [(1000, 333), (64, 4096)]:
        gen = torch.Generator(device="cpu").manual_seed(R)
        x = torch.randn(R, C, generator=gen).to(DEV)
        y = torch.randn(C, generator=gen).to(DEV)
        g = P.Group(nodes, [((R, C), "f32"), ((C,), "f32")], (R, C), "f32",
                    extras=[(2, (R, C), "bf16"), (3, (R, C), "f32")])
        out = torch.full((R, C), float("nan"), device=DEV)
        a = torch.full((R, C), float("nan"), dtype=torch.bfloat16, device=DEV)
        b = torch.full((R, C), float("nan"), device=DEV)
        g.run([x, y], out, extra_outs=[a, b])
        torch.cuda.synchronize()
        ra, rb = np.zeros((R, C), np.uint16), np.zeros((R, C), np.float32)
        ref = oracle.eval_group(nodes, [to_np(x), to_np(y)], (R, C), F32, extras=[(2, ra), (3, rb)])
        assert_bits(to_np(a), ra, f"a {R}x{C}")
        assert_bits(to_np(b), rb, f"b {R}x{C}")
        assert_bits(to_np(out), ref, f"out {R}x{C}")


def test_multi_output_refusals_on_device():
    nodes = parse_dag("%0 = input 0\n%1 = exp %0\n%2 = tanh %1\n")
    g = P.Group(nodes, [((64,), "f32")], (64,), "f32", extras=[(1, (64,), "f32")])
    x = torch.randn(64, device=DEV)
    out, e = torch.empty(64, device=DEV), torch.empty(64, device=DEV)

    def refused(status, fn):
        with pytest.raises(P.PskError) as ei:
            fn()
        assert ei.value.status == status, ei.value.name

    refused(P.PSK_E_UNSUPPORTED, lambda: g.run([x], out))             # extra outputs need run_multi
    refused(P.PSK_E_ALIAS, lambda: g.run([x], out, extra_outs=[out]))  # two outputs, one buffer
    big = torch.empty(128, device=DEV)
    refused(P.PSK_E_ALIAS, lambda: g.run([x], big[:64], extra_outs=[big[32:96]]))
    g.run([x], x, extra_outs=[e])                                      # root in place over x: allowed
    torch.cuda.synchronize()


# --------------------------------------------------------- AdamW as a group
def adamw_tree_group(theta_dt, grad_dt, mv_dt):
    t = {torch.float32: "f32", torch.bfloat16: "bf16"}
    ins = [((1,), t[theta_dt]), ((1,), t[grad_dt]), ((1,), t[mv_dt]), ((1,), t[mv_dt])] + [((), "f32")] * 9
    return P.Group(configs.adamw_group_dag(), ins, (1,), t[theta_dt], tree=True,
                   extras=[(configs.ADAMW_GROUP_M, (1,), t[mv_dt]), (configs.ADAMW_GROUP_V, (1,), t[mv_dt])])


def adamw_scalar_tensor(hp):
    s = oracle.adamw_scalars(*hp)          # b1 b2 1-b1 1-b2 1-b1^t 1-b2^t lr eps wd, each rounded once to f32
    return torch.from_numpy(s.copy()).to(DEV)


HPA = (configs.ADAMW_HP["lr"], configs.ADAMW_HP["beta1"], configs.ADAMW_HP["beta2"], configs.ADAMW_HP["eps"],
       configs.ADAMW_HP["weight_decay"], configs.ADAMW_HP["t"])


@pytest.mark.parametrize("dt", [(torch.bfloat16, torch.bfloat16, torch.float32),
                                (torch.float32, torch.float32, torch.float32),
                                (torch.float32, torch.bfloat16, torch.bfloat16)])
def test_adamw_as_tree_group_matches_oracle_and_hand_written_kernel(dt):
    shapes = [(1,), (3,), (7,), (1023,), (4096,), (4097,), ((1 << 16) + 5,), (64, 3)]
    a = configs.adamw_state(shapes, theta_dtype=dt[0], grad_dtype=dt[1], mv_dtype=dt[2], device=DEV, seed=51)
    b = [{k: v.clone() for k, v in s.items()} for s in a]
    before = [{k: to_np(v) for k, v in s.items()} for s in a]
    sc = adamw_scalar_tensor(HPA)
    grp = adamw_tree_group(*dt)
    tree = P.Tree([[s["theta"], s["grad"], s["m"], s["v"]] for s in a])
    # in place: theta' -> slot 0, m' -> slot 2, v' -> slot 3
    grp.run_tree(tree, [0, 1, 2, 3] + [-1] * 9, [0, 2, 3], [None] * 4 + [sc[i] for i in range(9)])
    P.Tree([[s["theta"], s["grad"], s["m"], s["v"]] for s in b]).adamw_step(*HPA)
    torch.cuda.synchronize()
    for i, (s, r, h) in enumerate(zip(a, before, b)):
        rt, rm, rv = oracle.adamw(r["theta"], r["grad"], r["m"], r["v"], *HPA)
        assert_bits(to_np(s["theta"]), rt, f"leaf {i} theta'")
        assert_bits(to_np(s["m"]), rm, f"leaf {i} m'")
        assert_bits(to_np(s["v"]), rv, f"leaf {i} v'")
        for k in ("theta", "m", "v"):
            assert torch.equal(s[k].view(torch.int16) if s[k].dtype == torch.bfloat16 else s[k].view(torch.int32),
                               h[k].view(torch.int16) if h[k].dtype == torch.bfloat16 else h[k].view(torch.int32))


def test_adamw_as_tree_group_full_llama_tree_equals_hand_written():
    """The 145-leaf, 887M-parameter tree: the emitted three-output group and
    the hand-written kernel, each on its own copy of the state, agree bit for
    bit on every element; sampled elements against the oracle."""
    shapes = [s for _, s in configs.llama_leaves()]
    a = configs.adamw_state(shapes, theta_dtype=torch.bfloat16, grad_dtype=torch.bfloat16, mv_dtype=torch.float32,
                            device=DEV, seed=configs.SEED_BASE + 2)
    gen = torch.Generator(device="cpu").manual_seed(17)
    idx = []
    for s in a:
        n = s["theta"].numel()
        idx.append(torch.unique(torch.cat([torch.arange(64), torch.arange(n - 64, n),
                                           torch.randint(0, n, (2048,), generator=gen)])).to(DEV))
    before = [{k: to_np(s[k][i]) for k in s} for s, i in zip(a, idx)]
    sc = adamw_scalar_tensor(HPA)
    grp = adamw_tree_group(torch.bfloat16, torch.bfloat16, torch.float32)
    outs = [[torch.empty_like(s["theta"]), torch.empty_like(s["m"]), torch.empty_like(s["v"])] for s in a]
    tree = P.Tree([[s["theta"], s["grad"], s["m"], s["v"], *o] for s, o in zip(a, outs)])
    grp.run_tree(tree, [0, 1, 2, 3] + [-1] * 9, [4, 5, 6], [None] * 4 + [sc[i] for i in range(9)])
    P.Tree([[s["theta"], s["grad"], s["m"], s["v"]] for s in a]).adamw_step(*HPA)   # in place on the inputs
    torch.cuda.synchronize()
    for leaf, (s, o) in enumerate(zip(a, outs)):
        assert torch.equal(o[0].view(torch.int16), s["theta"].view(torch.int16)), f"leaf {leaf} theta'"
        assert torch.equal(o[1].view(torch.int32), s["m"].view(torch.int32)), f"leaf {leaf} m'"
        assert torch.equal(o[2].view(torch.int32), s["v"].view(torch.int32)), f"leaf {leaf} v'"
    for leaf, (o, r, i) in enumerate(zip(outs, before, idx)):
        rt, rm, rv = oracle.adamw(r["theta"], r["grad"], r["m"], r["v"], *HPA)
        assert_bits(to_np(o[0][i]), rt, f"leaf {leaf} theta' vs oracle")
        assert_bits(to_np(o[1][i]), rm, f"leaf {leaf} m' vs oracle")


def test_tree_multi_output_refusals_on_device():
    s = configs.adamw_state([(16,)], device=DEV, seed=4)[0]
    grp = adamw_tree_group(torch.float32, torch.float32, torch.float32)
    sc = adamw_scalar_tensor(HPA)
    tree = P.Tree([[s["theta"], s["grad"], s["m"], s["v"]]])
    scal = [None] * 4 + [sc[i] for i in range(9)]

    def refused(status, fn):
        with pytest.raises(P.PskError) as ei:
            fn()
        assert ei.value.status == status, ei.value.name

    refused(P.PSK_E_ALIAS, lambda: grp.run_tree(tree, [0, 1, 2, 3] + [-1] * 9, [0, 2, 2], scal))   # one slot twice
    refused(P.PSK_E_UNSUPPORTED, lambda: grp.run_tree(tree, [0, 1, 2, 3] + [-1] * 9, 0, scal))     # single-output call
    refused(P.PSK_E_SHAPE, lambda: grp.run_tree(tree, [0, 1, 2, 3] + [-1] * 9, [0, 2, 9], scal))
    # a scalar inside an output slot's buffer (m) is refused; inside g (read only) it is fine
    bad = list(scal)
    bad[10] = s["m"][5]
    refused(P.PSK_E_ALIAS, lambda: grp.run_tree(tree, [0, 1, 2, 3] + [-1] * 9, [0, 2, 3], bad))
    # two slots of one leaf holding one buffer cannot both be outputs
    tree2 = P.Tree([[s["theta"], s["grad"], s["m"], s["v"], s["m"]]])
    refused(P.PSK_E_ALIAS, lambda: grp.run_tree(tree2, [0, 1, 2, 3] + [-1] * 9, [0, 2, 4], scal))


def test_add_rmsnorm_gelu_storing_h_in_place_full_size_sampled_rows():
    """[16384, 4096] bf16, h written in place over the residual, as timed."""
    R, C = 16384, 4096
    x, res, gm = configs.rmsnorm_inputs(R, C, device=DEV, seed=91)
    rows = np.unique(np.concatenate([[0, 1, R - 1], np.random.default_rng(92).integers(0, R, 300)]))
    idx = torch.from_numpy(rows).to(DEV)
    xs, rs, gn = to_np(x[idx]), to_np(res[idx]), to_np(gm)
    g = P.Group(configs.rmsnorm_gelu_dag(EPS), [((R, C), "bf16"), ((R, C), "bf16"), ((C,), "bf16")], (R, C), "bf16",
                extras=[(configs.RMSNORM_H, (R, C), "bf16")])
    out = torch.full((R, C), float("nan"), dtype=torch.bfloat16, device=DEV)
    g.run([x, res, gm], out, extra_outs=[res])
    torch.cuda.synchronize()
    rh = np.zeros((len(rows), C), np.uint16)
    ref = oracle.eval_group(configs.rmsnorm_gelu_dag(EPS), [xs, rs, gn], (len(rows), C), BF16,
                            extras=[(configs.RMSNORM_H, rh)])
    assert_bits(to_np(res[idx]), rh, "h full size")
    assert_bf16_close(to_np(out[idx]), ref, "out full size")
