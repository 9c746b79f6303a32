"""Pins for the oracle's row groups: causal softmax and add+RMSNorm+gamma+GELU."""
import math

import numpy as np
import torch
import torch.nn.functional as F

from synth import configs

TOL_REL, TOL_ABS = 2e-6, 1e-7


def close_f32(got, ref):
    return np.abs(got.astype(np.float64) - ref.astype(np.float64)) <= TOL_ABS + TOL_REL * np.abs(ref.astype(np.float64))


def bf16_ulp_distance(a_u16, b_u16):
    """Distance in bf16 units in the last place, +0 and -0 equal."""
    def ordered(u):
        s = u.astype(np.int32)
        mag = s & 0x7FFF
        return np.where(s & 0x8000, -mag, mag)
    return np.abs(ordered(a_u16) - ordered(b_u16))


# -------------------------------------------------------------- softmax
def test_softmax_generic_equals_dedicated(orc):
    # two independent codings of the masked softmax: the let-list evaluated
    # with -inf at refused positions, and the direct definition (max and sum
    # over the allowed positions, 0 where refused) -- the presk native
    # chapter states they give the same bits
    x = configs.softmax_scores(3 * 64, 64, seed=5)
    x = x.numpy()
    nodes = configs.softmax_causal_dag(0.125, 64)
    a = orc.eval_group(nodes, [x], x.shape)
    b = orc.softmax_causal(x, 64, 0.125)
    np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))


def test_softmax_closed_forms(orc):
    T = 16
    x = np.random.default_rng(0).standard_normal((2 * T, 24)).astype(np.float32) * 3
    x[1, 0] = x[1, 1] = 2.5
    out = orc.softmax_causal(x, T, 0.125)
    # row 0: only column 0 allowed
    assert out[0, 0] == 1.0 and np.all(out[0, 1:].view(np.uint32) == 0)
    # row 1 with equal scores: exactly one half each
    assert out[1, 0] == 0.5 and out[1, 1] == 0.5
    # refused positions are +0 (bits)
    for r in range(2 * T):
        q = r % T
        assert np.all(out[r, q + 1:].view(np.uint32) == 0)
    # row T restarts the causal pattern (the mask has period T)
    assert out[T, 0] == 1.0
    # rows sum to 1 within (allowed count) * 2^-24 (sum of correctly rounded quotients)
    s = out.astype(np.float64).sum(axis=1)
    n_allowed = np.minimum(np.arange(2 * T) % T + 1, 24)
    assert np.all(np.abs(s - 1.0) <= (n_allowed + 2) * 2.0 ** -24)


def test_softmax_shift_invariance_bit_exact(orc):
    # on a dyadic grid, y + c is exact, so adding an integer to every score
    # leaves the max-subtracted exponents -- and so the output -- unchanged
    r = np.random.default_rng(1)
    x = (r.integers(-4096, 4096, (64, 64)) / 256.0).astype(np.float32)
    a = orc.softmax_causal(x, 64, 0.125)
    b = orc.softmax_causal(x + np.float32(8.0), 64, 0.125)   # 8 * 0.125 = 1 added to y
    np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))


def test_softmax_vs_torch_library(orc):
    # torch.softmax(x.masked_fill(~m, -inf)) is the export of a masked softmax
    # (presk language reference, "PyTorch export")
    T, C = 128, 128
    x = configs.softmax_scores(2 * T, C, seed=2)
    out = orc.softmax_causal(x.numpy(), T, 0.125)
    rows = torch.arange(2 * T)[:, None] % T
    allowed = torch.arange(C)[None, :] <= rows
    ref = torch.softmax((x * 0.125).masked_fill(~allowed, float("-inf")), dim=-1).numpy()
    assert np.all(close_f32(out, ref))


def test_softmax_vs_f64(orc):
    T, C = 96, 96
    x = configs.softmax_scores(T, C, seed=3).numpy()
    out = orc.softmax_causal(x, T, 0.125)
    ref = orc.eval_group_f64(configs.softmax_causal_dag(0.125, T), [x], x.shape)
    assert np.all(close_f32(out, ref))


def test_softmax_empty_row_gives_zeros(orc):
    # a row with no allowed position gives zeros (presk native chapter);
    # C = 0 columns allowed cannot happen with a causal mask, so feed a row
    # of width 0 through the direct definition
    x = np.zeros((2, 0), np.float32)
    out = orc.softmax_causal(x, 4, 0.125)
    assert out.shape == (2, 0)


# ---------------------------------------------------------------- RMSNorm
def _bf16(t):
    return t.view(torch.int16).numpy().view(np.uint16)


def test_rmsnorm_generic_equals_dedicated(orc):
    x, r, g = configs.rmsnorm_inputs(8, 256, seed=4)
    eps = configs.f32(1e-5)
    a = orc.eval_group(configs.rmsnorm_gelu_dag(eps), [_bf16(x), _bf16(r), _bf16(g)], (8, 256), out_dtype=orc.BF16)
    b = orc.rmsnorm_gelu(_bf16(x), _bf16(r), _bf16(g), eps)
    np.testing.assert_array_equal(a, b)


def test_rmsnorm_constant_row_closed_form(orc):
    # a constant row h = a with gamma = 1: y = a / sqrt(a^2 + eps), out = gelu(y)
    from scipy.special import erf
    C = 4096
    eps = configs.f32(1e-5)
    for a in (0.5, -1.25, 3.0, 2.0 ** -6):
        half = torch.full((1, C), a / 2, dtype=torch.bfloat16)
        g = torch.ones(C, dtype=torch.bfloat16)
        out = orc.rmsnorm_gelu(_bf16(half), _bf16(half), _bf16(g), eps)
        y = a / math.sqrt(a * a + eps)
        want = 0.5 * y * (1.0 + erf(y / math.sqrt(2.0)))
        want_bf16 = torch.tensor([want], dtype=torch.float32).to(torch.bfloat16)
        assert np.all(bf16_ulp_distance(out[0], np.repeat(_bf16(want_bf16), C)) <= 1), a


def test_rmsnorm_vs_torch_library(orc):
    x, r, g = configs.rmsnorm_inputs(64, 4096, seed=6)
    eps = configs.f32(1e-5)
    out = orc.rmsnorm_gelu(_bf16(x), _bf16(r), _bf16(g), eps)
    # the library routines in float64 (in f32 torch's gelu forms 1 + erf,
    # which cancels in the negative tail), rounded once to bf16
    h = x.double() + r.double()
    ref = F.gelu(F.rms_norm(h, (4096,), g.double(), eps), approximate="none").float().to(torch.bfloat16)
    d = bf16_ulp_distance(out, _bf16(ref))
    assert d.max() <= 1
    assert (d == 0).mean() > 0.98


def test_rmsnorm_vs_f64(orc):
    x, r, g = configs.rmsnorm_inputs(16, 1024, seed=7)
    eps = configs.f32(1e-5)
    out = orc.rmsnorm_gelu(_bf16(x), _bf16(r), _bf16(g), eps)
    ref = orc.eval_group_f64(configs.rmsnorm_gelu_dag(eps), [_bf16(x), _bf16(r), _bf16(g)], (16, 1024))
    ref_bf16 = _bf16(torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16))
    assert bf16_ulp_distance(out, ref_bf16).max() <= 1


# ------------------------------------------------------------ row maximum
def test_row_max_nan_and_ties(orc):
    """The row maximum against numpy's maximum, which returns NaN for a row
    holding a NaN wherever it stands; and signed zeros as IEEE 754-2019
    maximum orders them (+0 above -0, whatever the order in the row),
    checked on the sign bit."""
    from synth.dag import parse_dag
    nodes = parse_dag("%0 = input 0\n%1 = row_max %0\n%2 = sub %0 %1\n")
    rng = np.random.default_rng(11)
    x = rng.standard_normal((64, 37)).astype(np.float32)
    for r in range(0, 64, 3):                      # NaN at the first, last or an inner position
        x[r, [0, 36, r % 37][r % 3]] = np.nan
    x[5, :] = np.nan
    mx = np.zeros((64, 1), np.float32)
    orc.eval_group(nodes, [x], x.shape, extras=[(1, mx)])
    want = x.max(axis=1, keepdims=True)
    assert np.array_equal(np.isnan(mx), np.isnan(want))
    assert np.array_equal(mx[~np.isnan(want)], want[~np.isnan(want)])
    z = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0], [-1.0, -0.0, -0.0], [-0.0, -1.0, -2.0],
                  [-0.0, 0.0, -0.0]], np.float32)
    mz = np.zeros((5, 1), np.float32)
    orc.eval_group(nodes, [z], z.shape, extras=[(1, mz)])
    assert np.all(mz == 0) and list(np.signbit(mz[:, 0])) == [False, False, True, True, False]
    # any order of a row gives the same bits
    rng2 = np.random.default_rng(12)
    w = rng2.choice(np.array([-0.0, 0.0, -3.0, 2.0, np.nan, -np.inf], np.float32), size=(200, 6))
    m1 = np.zeros((200, 1), np.float32)
    m2 = np.zeros((200, 1), np.float32)
    orc.eval_group(nodes, [w], w.shape, extras=[(1, m1)])
    orc.eval_group(nodes, [np.ascontiguousarray(w[:, ::-1])], w.shape, extras=[(1, m2)])
    assert np.array_equal(np.isnan(m1), np.isnan(m2))
    fin = ~np.isnan(m1)
    assert np.array_equal(m1[fin].view(np.uint32), m2[fin].view(np.uint32))


def test_softmax_row_with_nan_is_nan(orc):
    """The dedicated causal softmax over a row holding a NaN among its
    allowed scores: every allowed output is NaN (the maximum is NaN); a
    NaN only in refused columns changes nothing."""
    T = 8
    x = np.random.default_rng(2).standard_normal((T, T)).astype(np.float32)
    y = x.copy()
    y[5, 2] = np.nan            # allowed in row 5 (columns 0..5)
    y[3, 6] = np.nan            # refused in row 3 (columns 0..3)
    a, b = orc.softmax_causal(x, T, 0.125), orc.softmax_causal(y, T, 0.125)
    assert np.isnan(b[5, :6]).all() and np.all(b[5, 6:] == 0)
    assert np.array_equal(a[3], b[3])
