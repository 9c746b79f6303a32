"""Pins for the oracle's elementwise evaluator and bf16 conversions.

Each test ties the oracle to something other than itself: numpy's IEEE f32
arithmetic, PyTorch's bf16 conversion, float64 evaluation, closed forms.
"""
import math

import numpy as np
import pytest
import torch

from synth.dag import Node, parse_dag

F32_ULP1 = 2.0 ** -23


def rng(seed=0):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------ bf16
def test_bf16_round_known_values(orc):
    # bf16 keeps the top 16 bits of binary32 (presk native chapter: storage
    # only, one round to nearest even on the way out)
    vals = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 0.0, -0.0, np.inf, -np.inf,
                     3.4028234663852886e38, 1e-45], np.float32)
    got = orc.bf16_round(vals)
    want = np.array([0x3F80, 0x3F80, 0x3F82, 0xC020, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x7F80, 0x0000], np.uint16)
    np.testing.assert_array_equal(got, want)
    nan = orc.bf16_round(np.array([np.nan, -np.nan], np.float32))
    assert all((int(b) & 0x7F80) == 0x7F80 and (int(b) & 0x7F) != 0 for b in nan)
    assert (int(nan[1]) & 0x8000) != 0


def test_bf16_round_matches_torch(orc):
    x = (rng(1).standard_normal(200_000) * np.exp(rng(2).uniform(-30, 30, 200_000))).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(orc.bf16_round(x), want)


def test_bf16_widen_is_exact(orc):
    b = np.arange(0, 65536, dtype=np.uint16)
    w = orc.bf16_widen(b)
    want = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    fin = np.isfinite(want)
    np.testing.assert_array_equal(w[fin].view(np.uint32), want[fin].view(np.uint32))
    assert np.all(np.isnan(w[~fin]) == np.isnan(want[~fin]))
    # widen then round is the identity on non-NaN bit patterns
    back = orc.bf16_round(w)
    nn = ~np.isnan(w)
    np.testing.assert_array_equal(back[nn], b[nn])


# ------------------------------------------------- single-op evaluations
def _eval1(orc, op, x, **kw):
    nodes = [Node("input", (), None, 0), Node(op, (0,), kw.get("imm"), kw.get("iparam"))]
    return orc.eval_group(nodes, [x], x.shape)


def _eval2(orc, op, x, y, out_shape=None):
    nodes = [Node("input", (), None, 0), Node("input", (), None, 1), Node(op, (0, 1))]
    return orc.eval_group(nodes, [x, y], out_shape or x.shape)


@pytest.mark.parametrize("op,npf", [("add", np.add), ("sub", np.subtract), ("mul", np.multiply),
                                    ("div", np.divide)])
def test_binary_ops_bit_exact_vs_numpy(orc, op, npf):
    r = rng(3)
    x = (r.standard_normal((37, 129)) * 10).astype(np.float32)
    y = (r.standard_normal((37, 129)) * 10).astype(np.float32)
    got = _eval2(orc, op, x, y)
    np.testing.assert_array_equal(got.view(np.uint32), npf(x, y).view(np.uint32))


def test_sqrt_abs_neg_bit_exact_vs_numpy(orc):
    x = (rng(4).standard_normal((5, 1001)) * 100).astype(np.float32)
    np.testing.assert_array_equal(_eval1(orc, "sqrtabs", x).view(np.uint32),
                                  np.sqrt(np.abs(x)).view(np.uint32))
    ax = np.abs(x)
    np.testing.assert_array_equal(_eval1(orc, "sqrt", ax).view(np.uint32), np.sqrt(ax).view(np.uint32))
    np.testing.assert_array_equal(_eval1(orc, "neg", x).view(np.uint32), (-x).view(np.uint32))
    np.testing.assert_array_equal(_eval1(orc, "abs", x).view(np.uint32), np.abs(x).view(np.uint32))
    np.testing.assert_array_equal(_eval1(orc, "pow2", x).view(np.uint32), (x * x).view(np.uint32))


@pytest.mark.parametrize("op,f64,lo,hi,ulps", [
    ("exp", np.exp, -80.0, 80.0, 2), ("log", np.log, 1e-30, 1e30, 2),
    ("tanh", np.tanh, -12.0, 12.0, 3), ("erf", None, -6.0, 6.0, 2)])
def test_transcendentals_within_ulps_of_f64(orc, op, f64, lo, hi, ulps):
    from scipy.special import erf
    f64 = f64 or erf
    r = rng(5)
    if op == "log":
        x = np.exp(r.uniform(np.log(lo), np.log(hi), 100_000)).astype(np.float32)
    else:
        x = r.uniform(lo, hi, 100_000).astype(np.float32)
    got = _eval1(orc, op, x).astype(np.float64)
    ref = f64(x.astype(np.float64))
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(got - ref) <= ulps * ulp + 1e-45)


def test_gelu_against_f64_definition(orc):
    # gelu(x) = x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)) (presk native chapter)
    from scipy.special import erfc
    x = rng(6).uniform(-8, 8, 200_000).astype(np.float32)
    x = np.concatenate([x, np.array([0.0, -0.0, 1.0, -1.0, 3.0], np.float32)])
    got = _eval1(orc, "gelu", x).astype(np.float64)
    xd = x.astype(np.float64)
    ref = 0.5 * xd * erfc(-xd / math.sqrt(2.0))
    # the complementary-error-function composition keeps a relative error of
    # a few f32 ulps plus the conditioning of erfc at the rounded argument
    # z = x/sqrt 2 (relative sensitivity 2 z^2 = x^2 for z >> 1), the far
    # negative tail included
    assert np.all(np.abs(got - ref) <= (16 + xd * xd) * 2.0 ** -24 * np.abs(ref) + 1e-44)
    # closed forms: gelu(0) = 0, gelu(1) = Phi(1) = 0.8413447460685429
    assert got[-5] == 0.0 and got[-4] == 0.0
    assert abs(got[-3] - 0.8413447460685429) <= 2 * 2.0 ** -24
    # gelu(-x) = gelu(x) - x
    assert abs(got[-2] - (got[-3] - 1.0)) <= 4 * 2.0 ** -24


def test_pown_and_select(orc):
    x = rng(7).uniform(-3, 3, 4096).astype(np.float32)
    p3 = _eval1(orc, "pown", x, iparam=3).astype(np.float64)
    assert np.all(np.abs(p3 - x.astype(np.float64) ** 3) <= 2 * np.spacing(np.abs(p3).astype(np.float32)))
    np.testing.assert_array_equal(_eval1(orc, "pown", x, iparam=0), np.ones_like(x))
    np.testing.assert_array_equal(_eval1(orc, "pown", x, iparam=1).view(np.uint32), x.view(np.uint32))
    # select moves bits: a NaN or inf in the branch not picked never reaches the result
    c = (np.arange(64) % 2).astype(np.float32)
    a = np.full(64, np.nan, np.float32)
    a[1::2] = 5.0
    b = np.full(64, 7.0, np.float32)
    b[1::2] = np.inf
    nodes = parse_dag("%0 = input 0\n%1 = input 1\n%2 = input 2\n%3 = select %0 %1 %2\n")
    got = orc.eval_group(nodes, [c, a, b], (64,))
    want = np.where(np.arange(64) % 2 == 1, 5.0, 7.0).astype(np.float32)
    np.testing.assert_array_equal(got, want)


def test_max_min_tie_gives_second_operand(orc):
    # presk language reference, section "Typing", builtins: at a tie max and min give their
    # second operand; +0 and -0 compare equal, so the sign bit shows which
    x = np.array([0.0, -0.0, 1.0, 2.0], np.float32)
    y = np.array([-0.0, 0.0, 2.0, 1.0], np.float32)
    mx = _eval2(orc, "max", x, y)
    mn = _eval2(orc, "min", x, y)
    np.testing.assert_array_equal(mx.view(np.uint32), np.array([0x80000000, 0, 0x40000000, 0x40000000], np.uint32))
    np.testing.assert_array_equal(mn.view(np.uint32), np.array([0x80000000, 0, 0x3F800000, 0x3F800000], np.uint32))


# ------------------------------------------------------------- broadcasting
@pytest.mark.parametrize("bshape", [(37, 1), (1, 129), (129,), (), (1, 1)])
def test_broadcast_add_bit_exact(orc, bshape):
    # inputs align from the last axis; a size-1 axis broadcasts
    r = rng(8)
    a = r.standard_normal((37, 129)).astype(np.float32)
    b = np.asarray(r.standard_normal(bshape), dtype=np.float32)
    got = _eval2(orc, "add", a, b, out_shape=(37, 129))
    np.testing.assert_array_equal(got.view(np.uint32), (a + b).view(np.uint32))


def test_broadcast_rank4(orc):
    r = rng(9)
    a = r.standard_normal((2, 3, 5, 7)).astype(np.float32)
    b = r.standard_normal((3, 1, 7)).astype(np.float32)
    c = r.standard_normal((2, 1, 5, 1)).astype(np.float32)
    nodes = parse_dag("%0 = input 0\n%1 = input 1\n%2 = input 2\n%3 = mul %0 %1\n%4 = sub %3 %2\n")
    got = orc.eval_group(nodes, [a, b, c], a.shape)
    np.testing.assert_array_equal(got.view(np.uint32), ((a * b) - c).view(np.uint32))


def test_bf16_root_rounds_once(orc):
    # A group keeps interior values in f32 and rounds only the root (presk
    # language reference, "Dead code after differentiation": under bf16 a
    # group changes bits).  Crafted: x = 1 + 2^-8 (exact in f32, a tie in
    # bf16), y = 2^-9.  Fused: bf16(x + y) = bf16(1 + 3*2^-9) -> 1 + 2^-7.
    # Unfused with a bf16 intermediate: bf16(x) = 1 (tie to even), then
    # bf16(1 + 2^-9) = 1.
    x = np.array([1.0 + 2**-8], np.float32)
    y = np.array([2.0**-9], np.float32)
    nodes = parse_dag("%0 = input 0\n%1 = input 1\n%2 = const 0x1p+0\n%3 = mul %0 %2\n%4 = add %3 %1\n")
    fused = orc.eval_group(nodes, [x, y], (1,), out_dtype=orc.BF16)
    assert int(fused[0]) == 0x3F81
    step1 = orc.eval_group(parse_dag("%0 = input 0\n%1 = const 0x1p+0\n%2 = mul %0 %1\n"), [x], (1,),
                           out_dtype=orc.BF16)
    unfused = orc.eval_group(parse_dag("%0 = input 0\n%1 = input 1\n%2 = add %0 %1\n"), [step1, y], (1,),
                             out_dtype=orc.BF16)
    assert int(unfused[0]) == 0x3F80


def test_uniform_f32_fused_equals_unfused(orc):
    # Under a uniform f32 realization a group changes no bit (PSK-Realize,
    # "What it buys, measured"; language reference, "Dead code after
    # differentiation"): evaluate a chain as one group, and as one group per
    # op with every intermediate stored in f32.
    r = rng(10)
    a = r.uniform(-1, 1, (16, 33)).astype(np.float32)
    b = r.uniform(-1, 1, (16, 1)).astype(np.float32)
    text = """%0 = input 0
%1 = input 1
%2 = mul %0 %1
%3 = exp %2
%4 = add %3 %0
%5 = tanh %4
%6 = gelu %5
%7 = sqrtabs %6
%8 = div %7 %3
"""
    nodes = parse_dag(text)
    fused = orc.eval_group(nodes, [a, b], a.shape)
    vals = {0: a, 1: b}
    for i in range(2, len(nodes)):
        nd = nodes[i]
        ins = [vals[j] for j in nd.args]
        sub = [Node("input", (), None, k) for k in range(len(ins))] + [Node(nd.op, tuple(range(len(ins))))]
        vals[i] = orc.eval_group(sub, ins, a.shape)
    np.testing.assert_array_equal(fused.view(np.uint32), vals[len(nodes) - 1].view(np.uint32))


def test_f32_evaluator_vs_f64_companion_random_chains(orc):
    # the C f32 evaluator and the numpy f64 evaluator are independent codes;
    # on well-conditioned random chains they agree to a few f32 ulps per node
    from synth.dag import random_chain_dag
    r = rng(11)
    checked = 0
    for seed in range(40):
        nodes = random_chain_dag(seed, n_members=12, reread_target=(1, 4))
        bounds = orc.interval_bounds(nodes, [(-1, 1)] * 3)
        if max(max(abs(lo), abs(hi)) for lo, hi in bounds) > 50:
            continue
        A = r.uniform(-1, 1, (8, 64)).astype(np.float32)
        B = r.uniform(-1, 1, (8, 1)).astype(np.float32)
        C = r.uniform(-1, 1, (1, 64)).astype(np.float32)
        got = orc.eval_group(nodes, [A, B, C], (8, 64)).astype(np.float64)
        ref = orc.eval_group_f64(nodes, [A, B, C], (8, 64))
        scale = max(1.0, max(max(abs(lo), abs(hi)) for lo, hi in bounds))
        assert np.all(np.abs(got - ref) <= 1e-5 * scale), seed
        checked += 1
    assert checked >= 10
