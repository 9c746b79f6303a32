"""Pins for the oracle's multi-output groups (extra stored values).

A multi-output group computes what the partitioned program computes: each
stored value ends a group, and the next group reads it from memory.  These
tests evaluate that partitioned program with separate single-output calls
and compare bit for bit, and pin the layer normalization against PyTorch's
float64 layer_norm and closed forms."""
import math

import numpy as np
import pytest
import torch

from synth import configs
from synth.dag import parse_dag

F32, BF16 = 0, 1
U = 2.0 ** -24


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _widen(u: np.ndarray) -> np.ndarray:
    return (u.astype(np.uint32) << 16).view(np.float32)


def test_add_rmsnorm_storing_h_equals_the_partitioned_program(orc):
    eps = configs.f32(1e-5)
    x, r, g = configs.rmsnorm_inputs(24, 512, seed=3)
    x, r, g = _bits(x), _bits(r), _bits(g)
    h = np.zeros((24, 512), np.uint16)
    out = orc.eval_group(configs.rmsnorm_gelu_dag(eps), [x, r, g], (24, 512), BF16,
                         extras=[(configs.RMSNORM_H, h)])
    # group 1: h = bf16(x + res); group 2 reads the stored h
    h2 = orc.eval_group(parse_dag("%0 = input 0\n%1 = input 1\n%2 = add %0 %1\n"), [x, r], (24, 512), BF16)
    norm = parse_dag(f"""
        %0 = input 0
        %1 = input 1
        %2 = pow2 %0
        %3 = row_mean %2
        %4 = const {eps.hex()}
        %5 = add %3 %4
        %6 = sqrt %5
        %7 = div %0 %6
        %8 = mul %7 %1
        %9 = gelu %8
    """)
    out2 = orc.eval_group(norm, [h2, g], (24, 512), BF16)
    np.testing.assert_array_equal(h, h2)
    np.testing.assert_array_equal(out, out2)
    # h itself: one rounding of the f32 sum, as torch rounds it
    ht = (torch.from_numpy(_widen(x)) + torch.from_numpy(_widen(r))).to(torch.bfloat16)
    np.testing.assert_array_equal(h, _bits(ht))
    # and the value read inside the group is the rounded one: storing h in
    # f32 instead changes the output somewhere
    hf = np.zeros((24, 512), np.float32)
    out3 = orc.eval_group(configs.rmsnorm_gelu_dag(eps), [x, r, g], (24, 512), BF16,
                          extras=[(configs.RMSNORM_H, hf)])
    assert not np.array_equal(out3, out)
    np.testing.assert_array_equal(out3, orc.eval_group(configs.rmsnorm_gelu_dag(eps), [x, r, g], (24, 512), BF16))


def _layernorm(orc, x, gm, bt, eps, R, C):
    mean = np.zeros((R, 1), np.float32)
    rstd = np.zeros((R, 1), np.float32)
    out = orc.eval_group(configs.layernorm_dag(eps), [x, gm, bt], (R, C), BF16, root=configs.LAYERNORM_ROOT,
                         extras=[(configs.LAYERNORM_MEAN, mean), (configs.LAYERNORM_RSTD, rstd)])
    return out, mean, rstd


def test_layernorm_stats_equal_their_own_groups(orc):
    eps = configs.f32(1e-5)
    R, C = 16, 1000
    x, gm, bt = (_bits(t) for t in configs.layernorm_inputs(R, C, seed=4))
    out, mean, rstd = _layernorm(orc, x, gm, bt, eps, R, C)
    # the root alone (no extra outputs): f32 statistics change nothing
    alone = orc.eval_group(configs.layernorm_dag(eps)[:13], [x, gm, bt], (R, C), BF16)
    np.testing.assert_array_equal(out, alone)
    # the mean as a group of its own (a row value broadcast along the row)
    m2 = orc.eval_group(parse_dag("%0 = input 0\n%1 = row_mean %0\n"), [x], (R, C), F32)
    np.testing.assert_array_equal(mean[:, 0], m2[:, 0])


def test_layernorm_against_torch_float64(orc):
    eps = configs.f32(1e-5)
    R, C = 64, 4096
    xt, gt, bt_ = configs.layernorm_inputs(R, C, seed=5)
    x, gm, bt = _bits(xt), _bits(gt), _bits(bt_)
    out, mean, rstd = _layernorm(orc, x, gm, bt, eps, R, C)
    x64 = xt.double()
    ref = torch.nn.functional.layer_norm(x64, (C,), gt.double(), bt_.double(), eps)
    # bf16 output: one rounding to bf16 (relative 2^-8) of a value whose f32
    # error is bounded by the sums' (C + 16) u on the terms' magnitudes
    got = torch.from_numpy(_widen(out)).double()
    yg = ((x64 - x64.mean(dim=1, keepdim=True)) * torch.rsqrt(x64.var(dim=1, unbiased=False, keepdim=True) + eps)
          * gt.double()).abs()
    err = (C + 16) * U * (yg + bt_.double().abs())
    assert torch.all((got - ref).abs() <= 2.0 ** -8 * ref.abs() + 2 * err)
    # statistics: a sequential f32 sum of C terms is within (C - 1) u sum|x|
    # of the exact sum; the mean adds one rounding
    m64 = x64.mean(dim=1)
    bound = (C - 1) * U * x64.abs().mean(dim=1) + U * m64.abs()
    assert torch.all((torch.from_numpy(mean[:, 0]).double() - m64).abs() <= bound)
    r64 = 1.0 / torch.sqrt(x64.var(dim=1, unbiased=False) + eps)
    rel = (torch.from_numpy(rstd[:, 0]).double() - r64).abs() / r64
    assert rel.max() <= (C + 8) * U


def _ulps(a, b):
    def ordered(u):
        s = u.astype(np.int32)
        return np.where(s & 0x8000, -(s & 0x7FFF), s & 0x7FFF)
    return np.abs(ordered(a) - ordered(b))


def test_layernorm_closed_forms(orc):
    eps = configs.f32(1e-5)
    C = 256
    # a constant row: x - mean = 0 exactly, so the output is beta, bit for bit
    x = _bits(torch.full((3, C), 2.5).to(torch.bfloat16))
    gm = _bits(torch.linspace(0.5, 1.5, C).to(torch.bfloat16))
    bt = _bits(torch.linspace(-1, 1, C).to(torch.bfloat16))
    out, mean, rstd = _layernorm(orc, x, gm, bt, eps, 3, C)
    np.testing.assert_array_equal(out, np.broadcast_to(bt, (3, C)))
    assert (mean == 2.5).all()
    assert np.all(rstd == np.float32(1.0) / np.sqrt(np.float32(eps)))
    # a row of +a and -a: mean 0, variance a^2 exactly (a power of two)
    a = 0.5
    row = np.where(np.arange(C) % 2 == 0, a, -a).astype(np.float32)
    x = _bits(torch.from_numpy(np.tile(row, (2, 1))).to(torch.bfloat16))
    ones = _bits(torch.ones(C).to(torch.bfloat16))
    zeros = _bits(torch.zeros(C).to(torch.bfloat16))
    out, mean, rstd = _layernorm(orc, x, ones, zeros, eps, 2, C)
    assert (mean == 0).all()
    want = np.float32(a) / np.sqrt(np.float32(a * a) + np.float32(eps))
    np.testing.assert_array_equal(_widen(out), np.tile(np.where(row > 0, 1, -1) * _widen(_bits(
        torch.tensor(float(want)).to(torch.bfloat16))), (2, 1)))


def test_pointwise_multi_output_bits(orc):
    # a = x*y (stored bf16, read rounded), b = a + x (stored f32), root b*b - a
    nodes = parse_dag("%0 = input 0\n%1 = input 1\n%2 = mul %0 %1\n%3 = add %2 %0\n%4 = mul %3 %3\n%5 = sub %4 %2\n")
    rng = np.random.default_rng(6)
    x = rng.standard_normal((7, 33)).astype(np.float32)
    y = rng.standard_normal(33).astype(np.float32)
    a = np.zeros((7, 33), np.uint16)
    b = np.zeros((7, 33), np.float32)
    out = orc.eval_group(nodes, [x, y], (7, 33), F32, extras=[(2, a), (3, b)])
    at = torch.from_numpy(x * y).to(torch.bfloat16)
    np.testing.assert_array_equal(a, _bits(at))
    ar = at.float().numpy()
    np.testing.assert_array_equal(b.view(np.uint32), (ar + x).view(np.uint32))
    np.testing.assert_array_equal(out.view(np.uint32), ((ar + x) * (ar + x) - ar).view(np.uint32))


def test_adamw_group_dag_equals_the_dedicated_oracle_step(orc):
    # the AdamW step written as a let-list (m', v' stored, theta' the root),
    # evaluated by the generic evaluator, is the dedicated coding bit for bit
    hp = configs.ADAMW_HP
    args = (hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"], hp["t"])
    sc = orc.adamw_scalars(*args)
    for dts in [(torch.bfloat16, torch.bfloat16, torch.float32), (torch.float32, torch.float32, torch.bfloat16)]:
        st = configs.adamw_state([(3000,)], theta_dtype=dts[0], grad_dtype=dts[1], mv_dtype=dts[2], seed=12)[0]
        th, g, m, v = (_bits(st[k]) if st[k].dtype == torch.bfloat16 else st[k].numpy() for k in
                       ("theta", "grad", "m", "v"))
        rt, rm, rv = orc.adamw(th, g, m, v, *args)
        m2, v2 = np.zeros_like(m), np.zeros_like(v)
        ins = [th, g, m, v] + [np.asarray(sc[i]) for i in range(9)]
        out = orc.eval_group(configs.adamw_group_dag(), ins, (3000,), BF16 if th.dtype == np.uint16 else F32,
                             extras=[(configs.ADAMW_GROUP_M, m2), (configs.ADAMW_GROUP_V, v2)])
        np.testing.assert_array_equal(out, rt)
        np.testing.assert_array_equal(m2, rm)
        np.testing.assert_array_equal(v2, rv)
