"""Pins for the oracle's AdamW step (presk language reference, section "Configuration blocks", the optimizer)."""
import math

import numpy as np
import pytest
import torch

from synth import configs

HP = configs.ADAMW_HP
TOL_REL, TOL_ABS = 2e-6, 1e-7


def close(got, ref):
    got = got.astype(np.float64)
    ref = ref.astype(np.float64)
    return np.abs(got - ref) <= TOL_ABS + TOL_REL * np.abs(ref)


def _state(n, seed=0, dt=np.float32):
    st = configs.adamw_state([(n,)], seed=seed)[0]
    return [st[k].numpy().astype(dt) for k in ("theta", "grad", "m", "v")]


def test_scalars_closed_form(orc):
    # t = 10: 1 - 0.9^10 = 0.6513215599, 1 - 0.999^10 = 0.00995511979...
    s = orc.adamw_scalars(3e-4, 0.9, 0.999, 1e-8, 0.01, 10)
    assert s[4] == np.float32(0.6513215599)
    assert s[5] == np.float32(1.0 - 0.999 ** 10)
    # 1 - beta is formed in f64 and rounded once: f32(1 - 0.999) differs from
    # f32(1) - f32(0.999) by 1.3e-5 relative
    assert s[3] == np.float32(1.0 - 0.999)
    assert s[3] != np.float32(1.0) - np.float32(0.999)


def test_first_step_closed_form(orc):
    # t = 1, m = v = 0: mh = g and vh = g^2 exactly over the reals, so
    # theta' = theta - lr * (g / (|g| + eps) + wd * theta)
    r = np.random.default_rng(0)
    th = (r.standard_normal(4096) * 0.02).astype(np.float32)
    g = (r.standard_normal(4096) * 0.01).astype(np.float32)
    z = np.zeros_like(th)
    lr, wd, eps = 1e-3, 0.01, 1e-8
    to, mo, vo = orc.adamw(th, g, z, z, lr, 0.9, 0.999, eps, wd, 1)
    thd, gd = th.astype(np.float64), g.astype(np.float64)
    ref = thd - lr * (gd / (np.abs(gd) + eps) + wd * thd)
    assert np.all(close(to, ref))
    assert np.all(close(mo, 0.1 * gd)) and np.all(close(vo, 0.001 * gd * gd))


def test_exact_special_cases_preserve_leaf_patterns(orc):
    # every element carries a distinct pattern; in the special cases below
    # the step reproduces it exactly, so no element may move
    n = 1000
    pat = (np.arange(n, dtype=np.float32) * 1e-3 + 1.0).astype(np.float32)
    g = (np.arange(n, dtype=np.float32) * -2e-3 + 0.5).astype(np.float32)
    m = np.full(n, 0.25, np.float32)
    v = np.full(n, 0.125, np.float32)
    # lr = 0 -> theta' = theta
    to, _, _ = orc.adamw(pat, g, m, v, 0.0, 0.9, 0.999, 1e-8, 0.01, 3)
    np.testing.assert_array_equal(to.view(np.uint32), pat.view(np.uint32))
    # beta1 = 0 -> m' = g ; beta2 = 0 -> v' = g * g
    _, mo, vo = orc.adamw(pat, g, m, v, 1e-3, 0.0, 0.0, 1e-8, 0.01, 3)
    np.testing.assert_array_equal(mo.view(np.uint32), g.view(np.uint32))
    np.testing.assert_array_equal(vo.view(np.uint32), (g * g).view(np.uint32))
    # g = 0, m = v = 0, wd = 0 -> theta' = theta
    z = np.zeros(n, np.float32)
    to, mo, vo = orc.adamw(pat, z, z, z, 1e-3, 0.9, 0.999, 1e-8, 0.0, 7)
    np.testing.assert_array_equal(to.view(np.uint32), pat.view(np.uint32))
    assert not mo.any() and not vo.any()


def test_vs_torch_adamw(orc):
    # torch.optim.AdamW is what the language reference checks the step
    # against; it orders the operations differently, so compare within
    # tolerance
    n = 50_000
    th, g, m, v = _state(n, seed=3)
    t = HP["t"]
    to, mo, vo = orc.adamw(th, g, m, v, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"], t)
    p = torch.nn.Parameter(torch.from_numpy(th.copy()))
    opt = torch.optim.AdamW([p], lr=HP["lr"], betas=(HP["beta1"], HP["beta2"]), eps=HP["eps"],
                            weight_decay=HP["weight_decay"], foreach=False)
    p.grad = torch.from_numpy(g.copy())
    opt.state[p] = {"step": torch.tensor(float(t - 1)), "exp_avg": torch.from_numpy(m.copy()),
                    "exp_avg_sq": torch.from_numpy(v.copy())}
    opt.step()
    assert np.all(close(to, p.detach().numpy()))
    assert np.all(close(mo, opt.state[p]["exp_avg"].numpy()))
    assert np.all(close(vo, opt.state[p]["exp_avg_sq"].numpy()))


def test_vs_f64_step(orc):
    n = 20_000
    th, g, m, v = _state(n, seed=4)
    lr, b1, b2, eps, wd, t = (HP[k] for k in ("lr", "beta1", "beta2", "eps", "weight_decay", "t"))
    to, mo, vo = orc.adamw(th, g, m, v, lr, b1, b2, eps, wd, t)
    thd, gd, md, vd = (a.astype(np.float64) for a in (th, g, m, v))
    m2 = b1 * md + (1 - b1) * gd
    v2 = b2 * vd + (1 - b2) * gd * gd
    ref = thd - lr * ((m2 / (1 - b1 ** t)) / (np.sqrt(v2 / (1 - b2 ** t)) + eps) + wd * thd)
    assert np.all(close(to, ref)) and np.all(close(mo, m2)) and np.all(close(vo, v2))


def test_bf16_params_round_once(orc):
    # bf16 theta/grad: widened exactly, theta' rounded once from the f32 step
    n = 10_000
    st = configs.adamw_state([(n,)], theta_dtype=torch.bfloat16, grad_dtype=torch.bfloat16, seed=5)[0]
    u16 = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    th, g = u16(st["theta"]), u16(st["grad"])
    m, v = st["m"].numpy(), st["v"].numpy()
    args = (HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"], HP["t"])
    to, mo, vo = orc.adamw(th, g, m, v, *args)
    to32, mo32, vo32 = orc.adamw(orc.bf16_widen(th), orc.bf16_widen(g), m, v, *args)
    np.testing.assert_array_equal(to, orc.bf16_round(to32))
    np.testing.assert_array_equal(mo.view(np.uint32), mo32.view(np.uint32))
    np.testing.assert_array_equal(vo.view(np.uint32), vo32.view(np.uint32))


def test_bf16_moments_are_rounded_before_theta_reads_them(orc):
    # m', v' reach memory (they are outputs), so theta' reads their stored
    # values: with bf16 moments, theta' equals the f32 chain fed the rounded
    # moments
    n = 4096
    r = np.random.default_rng(6)
    th = (r.standard_normal(n) * 0.02).astype(np.float32)
    g = (r.standard_normal(n) * 0.01).astype(np.float32)
    m = orc.bf16_round((r.standard_normal(n) * 1e-3).astype(np.float32))
    v = orc.bf16_round((np.abs(r.standard_normal(n)) * 1e-4).astype(np.float32))
    lr, b1, b2, eps, wd, t = 1e-3, 0.9, 0.999, 1e-8, 0.01, 4
    to, mo, vo = orc.adamw(th, g, m, v, lr, b1, b2, eps, wd, t)
    s = orc.adamw_scalars(lr, b1, b2, eps, wd, t)
    mw, vw = orc.bf16_widen(mo), orc.bf16_widen(vo)
    mh = mw / s[4]
    vh = vw / s[5]
    ref = th - s[6] * (mh / (np.sqrt(vh) + s[7]) + s[8] * th)
    np.testing.assert_array_equal(to.view(np.uint32), ref.astype(np.float32).view(np.uint32))


# ------------------------------------------------- schedules and clipping
def test_schedules_closed_forms(orc):
    lr = 3e-4
    assert orc.lr_schedule("constant", lr, 7, 100, 10) == lr
    # warmup ramps linearly to lr at t = w, then decays to 0 at total
    for kind in ("linear", "cosine"):
        assert orc.lr_schedule(kind, lr, 5, 100, 10) == lr * 5 / 10
        assert orc.lr_schedule(kind, lr, 10, 100, 10) == lr
        assert abs(orc.lr_schedule(kind, lr, 100, 100, 10)) <= 1e-20
    # linear: halfway through the decay is half of lr
    assert abs(orc.lr_schedule("linear", lr, 55, 100, 10) - lr / 2) <= 1e-18
    # cosine: halfway is lr/2; at t = 32, lr (1 + cos(pi 22/90))/2
    assert abs(orc.lr_schedule("cosine", lr, 55, 100, 10) - lr / 2) <= 1e-18
    assert abs(orc.lr_schedule("cosine", lr, 32, 100, 10) -
               lr * 0.5 * (1 + math.cos(math.pi * 22 / 90))) <= 1e-18
    # no warmup: the decay starts at t = 0
    assert abs(orc.lr_schedule("linear", lr, 25, 100, 0) - lr * 0.75) <= 1e-18


def test_tree_sumsq_and_clip(orc):
    r = np.random.default_rng(8)
    leaves = [(r.standard_normal(n) * 0.01).astype(np.float32) for n in (1000, 17, 4096)]
    ss = orc.tree_sumsq(leaves)
    # math.fsum is the correctly rounded sum of the exact squares
    ref = math.fsum(float(x) ** 2 for g in leaves for x in g.astype(np.float64))
    assert abs(ss - ref) <= 2 * 2.0 ** -53 * ref
    # a long sum of small terms onto a large one, where plain summation stalls
    big = [np.array([4096.0], np.float32), np.full(1 << 16, 2.0 ** -20, np.float32)]
    assert orc.tree_sumsq(big) == 4096.0 ** 2 + (1 << 16) * 2.0 ** -40
    # bf16 leaves are widened exactly
    b = orc.bf16_round(leaves[0])
    assert orc.tree_sumsq([b]) == pytest.approx(float(np.sum(orc.bf16_widen(b).astype(np.float64) ** 2)), rel=1e-13)
    norm = math.sqrt(ref)
    assert orc.clip_factor(ref, 1e9) == np.float32(1.0)               # no clipping needed
    assert orc.clip_factor(ref, 0.5 * norm) == np.float32(0.5 * norm / (norm + 1e-6))


def test_clipped_step_vs_torch(orc):
    # clip_grad_norm_ over the whole tree, then AdamW: the pages define the
    # step as PyTorch does (within tolerance: different operation order)
    r = np.random.default_rng(9)
    shapes = (3000, 257)
    th = [(r.standard_normal(n) * 0.02).astype(np.float32) for n in shapes]
    g = [(r.standard_normal(n) * 0.5).astype(np.float32) for n in shapes]
    z = [np.zeros(n, np.float32) for n in shapes]
    c, lr = 1.0, 1e-3
    ss = orc.tree_sumsq(g)
    f = orc.clip_factor(ss, c)
    assert f < 1.0
    outs = [orc.adamw_scaled(a, b, m, v, lr, 0.9, 0.999, 1e-8, 0.01, 1, f) for a, b, m, v in zip(th, g, z, z)]
    ps = [torch.nn.Parameter(torch.from_numpy(a.copy())) for a in th]
    for p, gg in zip(ps, g):
        p.grad = torch.from_numpy(gg.copy())
    torch.nn.utils.clip_grad_norm_(ps, c)
    opt = torch.optim.AdamW(ps, lr=lr, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01, foreach=False)
    opt.step()
    for (to, mo, vo), p in zip(outs, ps):
        assert np.all(close(to, p.detach().numpy()))
        assert np.all(close(mo, opt.state[p]["exp_avg"].numpy()))
        assert np.all(close(vo, opt.state[p]["exp_avg_sq"].numpy()))


def test_scale_one_is_the_plain_step(orc):
    th, g, m, v = _state(5000, seed=10)
    args = (HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"], HP["t"])
    a = orc.adamw(th, g, m, v, *args)
    b = orc.adamw_scaled(th, g, m, v, *args, 1.0)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x.view(np.uint32), y.view(np.uint32))


def test_scaled_step_is_the_plain_step_on_the_scaled_gradient(orc):
    # the factor multiplies each gradient element once, in f32, before the moments
    th, g, m, v = _state(5000, seed=11)
    args = (HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"], HP["t"])
    f = np.float32(0.3713)
    a = orc.adamw_scaled(th, g, m, v, *args, f)
    b = orc.adamw(th, (g * f).astype(np.float32), m, v, *args)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x.view(np.uint32), y.view(np.uint32))
