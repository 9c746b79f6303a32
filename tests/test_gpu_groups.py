"""GPU parity of emitted group kernels (pointwise chains and row-reduction
groups) against the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from synth import configs
from synth.dag import parse_dag
from tests.gpu_util import assert_bf16_close, assert_bits, assert_f32_close, to_np

P = pytest.importorskip("elementwise_reduction_groups_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
EPS = configs.f32(1e-5)


def tdt(t):
    return "bf16" if t.dtype == torch.bfloat16 else "f32"


def run_group(nodes, inputs, out_shape, out_dtype, poison=True):
    g = P.Group(nodes, [(tuple(t.shape), tdt(t)) for t in inputs], out_shape, out_dtype)
    tdtype = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    out = torch.full(out_shape, float("nan"), dtype=tdtype, device=DEV) if poison else \
        torch.empty(out_shape, dtype=tdtype, device=DEV)
    g.run(inputs, out)
    torch.cuda.synchronize()
    return g, out


# ---------------------------------------------------------------- softmax
@pytest.mark.parametrize("rows,cols,period", [(300, 256, 256), (200, 1000, 200), (70, 1023, 64),
                                              (40, 4096, 4096), (33, 64, 64), (9, 12, 5)])
def test_causal_softmax_small(rows, cols, period):
    x = configs.softmax_scores(rows, cols, device=DEV, seed=rows + cols)
    nodes = configs.softmax_causal_dag(0.125, period)
    g, out = run_group(nodes, [x], (rows, cols), "f32")
    got = to_np(out)
    ref = oracle.softmax_causal(to_np(x), period, 0.125)
    assert_f32_close(got, ref, f"softmax {rows}x{cols}")
    # refused positions are exactly +0
    q = np.arange(rows)[:, None] % period
    masked = np.arange(cols)[None, :] > q
    assert np.all(got.view(np.uint32)[masked] == 0)
    # the generic oracle evaluator agrees too (same definition, other code)
    ref2 = oracle.eval_group(nodes, [to_np(x)], (rows, cols))
    assert_bits(ref, ref2, "oracle evaluators")


def test_causal_softmax_full_size_sampled_rows():
    R, C = 131072, 1024
    x = configs.softmax_scores(R, C, device=DEV)
    g, out = run_group(configs.softmax_causal_dag(0.125, 1024), [x], (R, C), "f32")
    info = g.info
    assert info.kind == 1 and info.lanes_per_row == 128 and info.vec == 4 and info.rows_per_block == 1
    rows = np.unique(np.concatenate([[0, 1, 2, 1023, 1024, 65535, R - 1],
                                     np.random.default_rng(5).integers(0, R, 600)]))
    xs = to_np(x[torch.from_numpy(rows).to(DEV)])
    got = to_np(out[torch.from_numpy(rows).to(DEV)])
    # the oracle row by row, each at its own causal position
    ref = np.stack([_softmax_row(xs[k], int(r) % 1024) for k, r in enumerate(rows)])
    assert_f32_close(got, ref, "softmax full size")
    assert not np.isnan(to_np(out)).any()


def _softmax_row(xrow, q):
    # one row at causal position q: a [q+1, C] block whose last row is the one
    # wanted, evaluated by the oracle with period q+1 so that row q is that row
    C = xrow.shape[0]
    block = np.zeros((q + 1, C), np.float32)
    block[q] = xrow
    out = oracle.softmax_causal(block, q + 1, 0.125, rows=(q, q + 1))
    return out[q]


# ---------------------------------------------------------------- RMSNorm
@pytest.mark.parametrize("rows,cols", [(37, 4096), (20, 4000), (19, 1000), (8, 64), (5, 8192), (3, 12)])
def test_rmsnorm_gelu_small(rows, cols):
    x, r, gm = configs.rmsnorm_inputs(rows, cols, device=DEV, seed=rows * cols)
    g, out = run_group(configs.rmsnorm_gelu_dag(EPS), [x, r, gm], (rows, cols), "bf16")
    ref = oracle.rmsnorm_gelu(to_np(x), to_np(r), to_np(gm), EPS)
    assert_bf16_close(to_np(out), ref, f"rmsnorm {rows}x{cols}")


def test_rmsnorm_gelu_full_size_sampled_rows():
    R, C = 16384, 4096
    x, r, gm = configs.rmsnorm_inputs(R, C, device=DEV)
    g, out = run_group(configs.rmsnorm_gelu_dag(EPS), [x, r, gm], (R, C), "bf16")
    info = g.info
    assert info.kind == 1 and info.lanes_per_row == 256 and info.vec == 8
    rows = torch.from_numpy(np.unique(np.concatenate([[0, 1, R - 1], np.random.default_rng(6).integers(0, R, 400)])))
    rows = rows.to(DEV)
    ref = oracle.rmsnorm_gelu(to_np(x[rows]), to_np(r[rows]), to_np(gm), EPS)
    assert_bf16_close(to_np(out[rows]), ref, "rmsnorm full size")
    o = to_np(out)
    assert not (((o & 0x7F80) == 0x7F80) & ((o & 0x7F) != 0)).any()


# ------------------------------------------------------------ 64-node chain
def test_chain64_small():
    nodes = configs.chain64_dag()
    A, B, C = configs.chain_inputs(96, 2048, device=DEV, seed=5)
    g, out = run_group(nodes, [A, B, C], (96, 2048), "f32")
    ref = oracle.eval_group(nodes, [to_np(A), to_np(B), to_np(C)], (96, 2048))
    assert_f32_close(to_np(out), ref, "chain64")


def test_chain64_full_size_sampled_rows():
    N = 16384
    nodes = configs.chain64_dag()
    A, B, C = configs.chain_inputs(N, N, device=DEV)
    g, out = run_group(nodes, [A, B, C], (N, N), "f32")
    assert g.info.kind == 0 and g.info.vec == 4 and g.info.members == 64
    rows = torch.from_numpy(np.unique(np.concatenate([[0, N - 1], np.random.default_rng(7).integers(0, N, 14)])))
    rows = rows.to(DEV)
    ref = oracle.eval_group(nodes, [to_np(A[rows]), to_np(B[rows]), to_np(C)], (len(rows), N))
    assert_f32_close(to_np(out[rows]), ref, "chain64 full size")
    assert not np.isnan(to_np(out)).any()


# -------------------------------------------------------- generic groups
def test_broadcast_indexing_bit_exact():
    # out[i, j] = A[i, j] + B[i] exactly: pins broadcast indexing
    A = torch.randn(1000, 333, device=DEV)
    B = torch.randn(1000, 1, device=DEV)
    _, out = run_group(parse_dag("%0 = input 0\n%1 = input 1\n%2 = add %0 %1\n"), [A, B], (1000, 333), "f32")
    assert_bits(to_np(out), to_np(A) + to_np(B), "A + Bcol")


def test_basic_ops_bit_exact_rank4():
    # add, mul, div, sqrt, max/min only: correctly rounded IEEE on both sides
    a = torch.randn(3, 5, 64, 48, device=DEV)
    b = torch.rand(5, 1, 48, device=DEV) + 0.5
    c = torch.randn(3, 1, 64, 1, device=DEV)
    nodes = parse_dag("""%0 = input 0
%1 = input 1
%2 = input 2
%3 = mul %0 %1
%4 = div %3 %1
%5 = sub %4 %2
%6 = abs %5
%7 = sqrt %6
%8 = max %7 %2
%9 = min %8 %1
%10 = const 0x1.8p+1
%11 = mul %9 %10
%12 = neg %11
%13 = pow2 %12
""")
    _, out = run_group(nodes, [a, b, c], (3, 5, 64, 48), "f32")
    ref = oracle.eval_group(nodes, [to_np(a), to_np(b), to_np(c)], (3, 5, 64, 48))
    assert_bits(to_np(out), ref, "basic ops")


def test_bf16_root_and_bf16_inputs():
    a = torch.randn(257, 136, device=DEV).to(torch.bfloat16)
    b = torch.randn(136, device=DEV)
    nodes = parse_dag("%0 = input 0\n%1 = input 1\n%2 = mul %0 %1\n%3 = tanh %2\n%4 = gelu %3\n%5 = exp %4\n")
    _, out = run_group(nodes, [a, b], (257, 136), "bf16")
    ref = oracle.eval_group(nodes, [to_np(a), to_np(b)], (257, 136), out_dtype=oracle.BF16)
    assert_bf16_close(to_np(out), ref, "bf16 chain")


def test_misaligned_views_take_the_element_path():
    base = torch.randn(1 + 64 * 100, device=DEV)
    x = base[1:].view(64, 100)                    # 4-byte aligned, not 16
    outb = torch.full((1 + 64 * 100,), float("nan"), device=DEV)
    out = outb[1:].view(64, 100)
    # a well-conditioned chain: sqrt(exp(x)) * x
    nodes = parse_dag("%0 = input 0\n%1 = exp %0\n%2 = sqrt %1\n%3 = mul %2 %0\n")
    g = P.Group(nodes, [((64, 100), "f32")], (64, 100), "f32")
    g.run([x], out)
    torch.cuda.synchronize()
    ref = oracle.eval_group(nodes, [to_np(x)], (64, 100))
    assert_f32_close(to_np(out), ref, "misaligned")
    assert np.isnan(to_np(outb[:1])).all()        # nothing written before the view


def test_in_place_and_alias_refusal():
    x = torch.randn(128, 1024, device=DEV)
    x0 = to_np(x)
    nodes = configs.softmax_causal_dag(0.125, 128)
    g = P.Group(nodes, [((128, 1024), "f32")], (128, 1024), "f32")
    g.run([x], x)                                   # in place
    torch.cuda.synchronize()
    assert_f32_close(to_np(x), oracle.softmax_causal(x0, 128, 0.125), "in place")
    y = torch.randn(64, 1, device=DEV)
    g2 = P.Group(parse_dag("%0 = input 0\n%1 = input 1\n%2 = add %0 %1\n"), [((64, 4), "f32"), ((64, 1), "f32")],
                 (64, 4), "f32")
    big = torch.zeros(64 * 4, device=DEV)
    with pytest.raises(P.PskError) as ei:
        g2.run([big.view(64, 4), big[:64].view(64, 1)], big.view(64, 4))
    assert ei.value.status == P.PSK_E_ALIAS


def test_binding_refuses_tensors_that_do_not_match_the_group():
    """The binding checks every tensor against the group's buffers (element
    count, storage type, device) before the launch: a short or mistyped
    tensor would otherwise be read or written past its end."""
    g = P.Group(parse_dag("%0 = input 0\n%1 = input 1\n%2 = add %0 %1\n"), [((64, 4), "f32"), ((64, 1), "f32")],
                (64, 4), "f32")
    x, y, out = torch.randn(64, 4, device=DEV), torch.randn(64, 1, device=DEV), torch.empty(64, 4, device=DEV)
    before = P.psk_get_stats().launches
    for ins, o, what in [([x, torch.randn(32, 1, device=DEV)], out, "elements"),
                         ([x, y], torch.empty(64, 3, device=DEV), "elements"),
                         ([x, y.to(torch.bfloat16)], out, "storage type"),
                         ([x, y], out.to(torch.bfloat16), "storage type"),
                         ([x], out, "inputs")]:
        with pytest.raises(ValueError, match=what):
            g.run(ins, o)
    with pytest.raises(ValueError, match="outputs"):
        g.run([x, y], out, extra_outs=[torch.empty(64, 4, device=DEV)])
    assert P.psk_get_stats().launches == before
    g.run([x.view(256), y.view(64)], out.view(16, 16))      # any view with the right count and type
    torch.cuda.synchronize()
    assert torch.equal(out, x + y)


def test_tree_binding_refuses_mixed_slot_types():
    """Every leaf's tensor in a slot must have that slot's storage type (the
    kernels size each leaf's accesses by it) and each leaf all the slots."""
    a = [torch.zeros(8, device=DEV) for _ in range(4)]
    b = [torch.zeros(8, device=DEV, dtype=torch.bfloat16)] + [torch.zeros(8, device=DEV) for _ in range(3)]
    with pytest.raises(ValueError, match="slot 0"):
        P.Tree([a, b])
    with pytest.raises(ValueError, match="slots"):
        P.Tree([a, a[:3]])


def test_empty_output_launches_nothing():
    g = P.Group(parse_dag("%0 = input 0\n%1 = exp %0\n"), [((0, 16), "f32")], (0, 16), "f32")
    before = P.psk_get_stats().launches
    g.run([torch.empty(0, 16, device=DEV)], torch.empty(0, 16, device=DEV))
    assert P.psk_get_stats().launches == before


def test_row_group_two_phase_max_sum_mean():
    # three reductions in two phases, a row-constant input and a scalar input
    x = torch.randn(150, 777, device=DEV)
    s = torch.rand(150, 1, device=DEV) + 0.5
    k = torch.tensor(0.75, device=DEV)
    nodes = parse_dag("""%0 = input 0
%1 = input 1
%2 = input 2
%3 = mul %0 %1
%4 = row_max %3
%5 = row_mean %3
%6 = sub %3 %4
%7 = exp %6
%8 = row_sum %7
%9 = div %7 %8
%10 = mul %9 %2
%11 = add %10 %5
""")
    _, out = run_group(nodes, [x, s, k], (150, 777), "f32")
    ref = oracle.eval_group(nodes, [to_np(x), to_np(s), to_np(k)], (150, 777))
    assert_f32_close(to_np(out), ref, "two-phase row group")


@pytest.mark.parametrize("C", [256, 1000, 40000])
def test_division_by_a_row_value_is_ieee_bit_exact(C):
    """x / row_max(|x| + d): the maximum is exact in any order, so the
    quotients must be IEEE's bit for bit: signed zeros, tiny and huge
    numerators (the path that falls back to IEEE division), negative and
    huge divisors (rows scaled by d), in the register and the tiled kernel."""
    R = 12
    gen = torch.Generator(device="cpu").manual_seed(C)
    x = torch.randn(R, C, generator=gen)
    x[0, ::3] = -0.0
    x[1, ::5] = 0.0
    x[2, ::7] = 1e-30                       # below 2^-86: the IEEE fallback
    x[3, ::11] = -3e38
    x[4] = x[4] * 1e-38                     # subnormal-range numerators
    x[5, 0] = 3.0                           # so that row 5's divisor is negative (below)
    x[5, 1::4] = 0.0                        # +0 / negative = -0, -0 / negative = +0
    x[5, 2::4] = -0.0
    d = torch.ones(R, 1)
    d[5] = -2.0                             # negative divisors after the negation below
    d[6] = 1e30
    d[7] = 1e-35
    nodes = parse_dag("""%0 = input 0
%1 = input 1
%2 = abs %0
%3 = add %2 %1
%4 = row_max %3
%5 = mul %4 %1
%6 = div %0 %5
""")
    _, out = run_group(nodes, [x.to(DEV), d.to(DEV)], (R, C), "f32")
    ref = oracle.eval_group(nodes, [x.numpy(), d.numpy()], (R, C))
    assert_bits(to_np(out), ref, f"x / row value, {C} columns")
    assert (to_np(out)[0, ::3].view(np.uint32) == 0x80000000).all()   # -0 / positive = -0
    assert (to_np(out)[5, 1::4].view(np.uint32) == 0x80000000).all()  # +0 / negative = -0
    assert (to_np(out)[5, 2::4].view(np.uint32) == 0).all()           # -0 / negative = +0
    # dividends the divisor does not depend on: infinities, both zeros, and
    # magnitudes on either side of 2^-86 and 2^87 mixed within every vector
    vals = torch.tensor([float("inf"), float("-inf"), 0.0, -0.0, 2.0 ** -86, -(2.0 ** -86) * (1 - 2 ** -24),
                         2.0 ** 87, -(2.0 ** 87) * (1 + 2 ** -23), 1e-40, 3.5, -1.25], dtype=torch.float32)
    xs = torch.randn(R, C, generator=gen)
    pick = torch.randint(0, 2 * vals.numel(), (R, C), generator=gen)
    xs = torch.where(pick < vals.numel(), vals[pick.clamp(max=vals.numel() - 1)], xs)
    xs[8] = torch.randn(C, generator=gen)             # a row with none of them
    ys = torch.randn(R, C, generator=gen) * torch.logspace(-30, 30, R).reshape(R, 1)
    nodes2 = parse_dag("%0 = input 0\n%1 = input 1\n%2 = abs %1\n%3 = row_max %2\n%4 = div %0 %3\n")
    _, out2 = run_group(nodes2, [xs.to(DEV), ys.to(DEV)], (R, C), "f32")
    ref2 = oracle.eval_group(nodes2, [xs.numpy(), ys.numpy()], (R, C))
    assert_bits(to_np(out2), ref2, f"special dividends / row value, {C} columns")
    # the same dividends over negative row values
    nodes3 = parse_dag("%0 = input 0\n%1 = input 1\n%2 = abs %1\n%3 = row_max %2\n%4 = neg %3\n%5 = div %0 %4\n")
    _, out3 = run_group(nodes3, [xs.to(DEV), ys.to(DEV)], (R, C), "f32")
    ref3 = oracle.eval_group(nodes3, [xs.numpy(), ys.numpy()], (R, C))
    assert_bits(to_np(out3), ref3, f"special dividends / negative row value, {C} columns")


def test_persistent_row_layout_is_bit_identical(monkeypatch):
    """The persistent row kernel (a layout switch: a few workgroups per CU
    walk the rows and load the next 1 to 4 ahead, the loop unrolled over
    its buffers) gives the one-row-per-workgroup kernel's bits: same
    reduction order, LDS halves alternating by row."""
    R, C = 3000, 4096
    x, r, g = configs.rmsnorm_inputs(R, C, device=DEV, seed=5)
    xl, gl, bl = configs.layernorm_inputs(R, C, device=DEV, seed=6)
    s = configs.softmax_scores(2048, 1024, device=DEV, seed=7)
    m = configs.random_mask(1024, 1024, 0.5, empty_rows=[3], device=DEV, seed=8)
    cases = [
        (configs.rmsnorm_gelu_dag(EPS), [((R, C), "bf16"), ((R, C), "bf16"), ((C,), "bf16")], (R, C), "bf16", {},
         [x, r, g], []),
        (configs.layernorm_dag(EPS), [((R, C), "bf16"), ((C,), "bf16"), ((C,), "bf16")], (R, C), "bf16",
         dict(root=configs.LAYERNORM_ROOT, extras=[(configs.LAYERNORM_MEAN, (R, 1), "f32"),
                                                  (configs.LAYERNORM_RSTD, (R, 1), "f32")]), [xl, gl, bl], [(R, 1), (R, 1)]),
        (configs.softmax_causal_dag(0.125, 1024), [((2048, 1024), "f32")], (2048, 1024), "f32", {}, [s], []),
        (configs.softmax_masked_dag(0.125), [((2, 1024, 1024), "f32"), ((1024, 1024), "u8")], (2, 1024, 1024), "f32",
         {}, [s.view(2, 1024, 1024), m], []),
    ]
    for nodes, ins, shape, dt, kw, tensors, xs in cases:
        outs = []
        for layout in ("persist=0", "persist=4", "persist=2", "persist=4,pf=2", "persist=3,pf=4", ""):
            monkeypatch.setenv("PSK_LAYOUT", layout)
            grp = P.Group(nodes, ins, shape, dt, **kw)
            out = torch.full(shape, float("nan"), dtype=torch.bfloat16 if dt == "bf16" else torch.float32, device=DEV)
            ex = [torch.full(sh, float("nan"), device=DEV) for sh in xs]
            grp.run(tensors, out, extra_outs=ex or None)
            torch.cuda.synchronize()
            outs.append([to_np(out)] + [to_np(e) for e in ex])
        for other in outs[1:]:
            for a, b in zip(outs[0], other):
                assert_bits(a, b, f"persistent layout, {shape}")


@pytest.mark.gpu
def test_layernorm_many_rows_two_a_workgroup(monkeypatch):
    """Past 32 rows a persistent workgroup the planner gives LayerNorm two
    rows a 512-thread workgroup (an odd row count leaves the last
    workgroup one row): the bits of one row a workgroup and of the
    persistent kernel, and every statistic and sampled rows against the
    oracle."""
    R, C = 32 * 1024 + 3, 4096
    xl, gl, bl = configs.layernorm_inputs(R, C, device=DEV, seed=11)
    nodes, ins = configs.layernorm_dag(EPS), [((R, C), "bf16"), ((C,), "bf16"), ((C,), "bf16")]
    kw = dict(root=configs.LAYERNORM_ROOT, extras=[(configs.LAYERNORM_MEAN, (R, 1), "f32"),
                                                   (configs.LAYERNORM_RSTD, (R, 1), "f32")])
    from tests.test_gpu_multi import assert_layernorm_close, check_stats
    outs, info = [], None
    for layout in ("", "persist=0,block=256", "persist=4"):
        monkeypatch.setenv("PSK_LAYOUT", layout)
        grp = P.Group(nodes, ins, (R, C), "bf16", **kw)
        if not layout:
            src = P.psk_group_source(grp.desc)
            assert "__launch_bounds__(512)" in src and "gridDim" not in src[src.index('extern "C"'):]
            info = grp.info
        out = torch.full((R, C), float("nan"), dtype=torch.bfloat16, device=DEV)
        ex = [torch.full((R, 1), float("nan"), device=DEV) for _ in range(2)]
        grp.run([xl, gl, bl], out, extra_outs=ex)
        torch.cuda.synchronize()
        outs.append((out, ex[0], ex[1]))
    for other in outs[1:]:
        for a, b in zip(outs[0], other):
            assert_bits(to_np(a), to_np(b), "LayerNorm, two rows a workgroup")
    rows = torch.tensor(np.r_[0:3, R // 2 - 1:R // 2 + 2, R - 3:R], device=DEV)
    xr = xl[rows].contiguous()
    ref = oracle.eval_group(nodes, [to_np(xr), to_np(gl), to_np(bl)], (rows.numel(), C), 1,
                            root=configs.LAYERNORM_ROOT)
    assert_layernorm_close(to_np(outs[0][0][rows]), ref, xr, gl, bl, C, "LayerNorm rows vs oracle")
    check_stats(info, xr, outs[0][1][rows], outs[0][2][rows], C, "LayerNorm statistics, two rows a workgroup")


def test_signed_zeros_through_fused_expressions():
    """0 - x is +0 for x = +0 also when another member reads it (the compiler
    must not turn it into -x), x + 0 is +0 for x = -0: every sign of zero the
    oracle gives, bit for bit, on both the vector and the element path."""
    nodes = parse_dag("""
        %0 = input 0
        %1 = input 1
        %2 = const 0x0p+0
        %3 = sub %2 %0
        %4 = mul %3 %1
        %5 = add %3 %1
        %6 = add %0 %2
        %7 = mul %6 %1
        %8 = sub %2 %1
        %9 = mul %8 %6
    """)
    vals = np.array([0.0, -0.0, 1.0, -1.0, 2.5], np.float32)
    xs, ys = np.meshgrid(vals, np.array([0.0, -0.0, 1.0, -1.0], np.float32))
    x = np.tile(xs.ravel(), 13)[:256].astype(np.float32)
    y = np.tile(ys.ravel(), 13)[:256].astype(np.float32)
    for offset in (0, 1):                       # aligned: vector path; offset by one element: element path
        bx = torch.zeros(257, device=DEV); by = torch.zeros(257, device=DEV)
        tx, ty = bx[offset:offset + 256], by[offset:offset + 256]
        tx.copy_(torch.from_numpy(x)); ty.copy_(torch.from_numpy(y))
        g = P.Group(nodes, [((256,), "f32"), ((256,), "f32")], (256,), "f32",
                    extras=[(4, (256,), "f32"), (5, (256,), "f32"), (7, (256,), "f32")])
        out = torch.full((256,), float("nan"), device=DEV)
        xo = [torch.full((256,), float("nan"), device=DEV) for _ in range(3)]
        g.run([tx, ty], out, extra_outs=xo)
        torch.cuda.synchronize()
        refx = [(m, np.zeros(256, np.float32)) for m in (4, 5, 7)]
        ref = oracle.eval_group(nodes, [x, y], (256,), P.PSK_F32, extras=refx)
        assert_bits(to_np(out), ref, f"(0 - y)(x + 0), offset {offset}")
        for (m, r), t in zip(refx, xo):
            assert_bits(to_np(t), r, f"member {m}, offset {offset}")


@pytest.mark.parametrize("layout", ["", "tiled=1,lanes=128,tn=1,rc=1,lc=1", "persist=2", "lanes=32"])
def test_row_max_signed_zeros_and_nan(layout, monkeypatch):
    """The row maximum over rows of signed zeros, NaNs, -inf and a few
    values, stored per row and subtracted from the row: IEEE 754-2019
    maximum (+0 above -0, NaN anywhere gives NaN) whatever the kernel's
    combining order, bit for bit against the oracle's sequential fold
    (NaN compared as NaN)."""
    if layout:
        monkeypatch.setenv("PSK_LAYOUT", layout)
    from synth.dag import parse_dag
    nodes = parse_dag("%0 = input 0\n%1 = row_max %0\n%2 = sub %0 %1\n")
    R, C = 96, 1000
    vals = np.array([-0.0, 0.0, -1.0, -2.5, -np.inf, np.nan, 3.5], np.float32)
    rng = np.random.default_rng(21)
    x = np.empty((R, C), np.float32)
    for r in range(R):
        pool = vals[: 2 + r % 5] if r % 7 else vals          # rows of only zeros, of zeros and negatives, ...
        x[r] = rng.choice(pool, size=C)
    x[3, :] = -0.0
    x[4, :] = 0.0
    x[5, ::2], x[5, 1::2] = -0.0, 0.0
    xt = torch.from_numpy(x).to(DEV)
    g = P.Group(nodes, [((R, C), "f32")], (R, C), "f32", extras=[(1, (R, 1), "f32")])
    out = torch.full((R, C), float("nan"), device=DEV)
    mx = torch.full((R, 1), float("nan"), device=DEV)
    g.run([xt], out, extra_outs=[mx])
    torch.cuda.synchronize()
    rmx = np.zeros((R, 1), np.float32)
    ref = oracle.eval_group(nodes, [x], (R, C), extras=[(1, rmx)])
    for name, got, r in (("row max", to_np(mx), rmx), ("x - row max", to_np(out), ref)):
        nan = np.isnan(r)
        assert np.array_equal(np.isnan(got), nan), f"{layout}: {name} NaN positions differ"
        assert_bits(got[~nan], r[~nan], f"{layout}: {name}")
    assert np.signbit(rmx[3, 0]) and not np.signbit(rmx[4, 0]) and not np.signbit(rmx[5, 0])


def test_split_product_exponential_within_three_ulps():
    """exp(x - max x) with f32 results takes the split-product exponential
    (2^t (1 + r ln 2), t = fl((x - m) log2 e)): against float64 exp of the
    same f32 differences, within 3 f32 ulps wherever the result is normal,
    and below 2^-126 where it is not; -inf gives 0."""
    from synth.dag import parse_dag
    nodes = parse_dag("%0 = input 0\n%1 = row_max %0\n%2 = sub %0 %1\n%3 = exp %2\n")
    R, C = 256, 4096
    rng = np.random.default_rng(31)
    x = (-rng.random((R, C)) * 104.0).astype(np.float32)
    x[:, 0] = 0.0                                            # the row maximum is 0: x - m is x
    x[:, 1] = -np.inf
    x[:, 2:40] = -(np.arange(38, dtype=np.float32) * 2.0 ** -20)   # tiny arguments
    g = P.Group(nodes, [((R, C), "f32")], (R, C), "f32")
    assert "psk_exp_np(" in P.psk_group_source(g.desc)
    out = torch.full((R, C), float("nan"), device=DEV)
    g.run([torch.from_numpy(x).to(DEV)], out)
    torch.cuda.synchronize()
    got = to_np(out).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    normal = ref >= 2.0 ** -126
    ulp = np.spacing(ref[normal].astype(np.float32)).astype(np.float64)
    err = np.abs(got[normal] - ref[normal]) / ulp
    assert err.max() <= 3.0, f"split-product exponential: {err.max():.2f} ulps"
    assert np.all(np.abs(got[~normal] - ref[~normal]) <= 2.0 ** -126)
    assert np.all(got[:, 1] == 0.0)


@pytest.mark.gpu
def test_emitted_tanh_within_three_ulps():
    """The emitted tanh (polynomial below |x| = 0.625, 1 - 2/(1 + e^{2|x|})
    above): against float64 tanh of the same f32 arguments, within 3 f32
    ulps wherever the result is normal (the f32 emulation with the hardware
    2^x and reciprocal off by an ulp gives 2.45), odd in x bit for bit, ±0
    kept, ±inf to ±1, NaN to NaN; subnormal results within 2^-126 (they
    may be flushed, as the f32 tolerance's absolute part allows)."""
    nodes = parse_dag("%0 = input 0\n%1 = tanh %0\n")
    rng = np.random.default_rng(47)
    n = 1 << 22
    x = np.concatenate([
        rng.uniform(-1.0, 1.0, n // 4), rng.uniform(-20.0, 20.0, n // 4),
        np.linspace(0.6, 0.65, n // 8), -np.linspace(0.6, 0.65, n // 8),      # either side of the split
        np.exp(rng.uniform(np.log(1e-30), np.log(1e-3), n // 4)) * rng.choice([-1.0, 1.0], n // 4)]).astype(np.float32)
    specials = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 0.625, -0.625, np.nextafter(np.float32(0.625), np.float32(0)),
                         1e-40, -1e-40, 9.0, 16.0, 17.0, 1e30, -1e30], dtype=np.float32)
    x = np.concatenate([x, specials])
    g = P.Group(nodes, [((x.size,), "f32")], (x.size,), "f32")
    assert "psk_tanh(" in P.psk_group_source(g.desc)
    out = torch.full((x.size,), float("nan"), device=DEV)
    g.run([torch.from_numpy(x).to(DEV)], out)
    torch.cuda.synchronize()
    got = to_np(out)
    ref = np.tanh(x.astype(np.float64))
    fin = np.isfinite(x)
    normal = fin & (np.abs(ref) >= 2.0 ** -126)
    ulp = np.spacing(np.abs(ref[normal]).astype(np.float32)).astype(np.float64)
    err = np.abs(got[normal].astype(np.float64) - ref[normal]) / ulp
    assert err.max() <= 3.0, f"tanh: {err.max():.2f} ulps at x = {x[normal][err.argmax()]!r}"
    sub = fin & ~normal                      # tanh(x) is x there; subnormals may be flushed
    assert np.all(np.abs(got[sub].astype(np.float64) - x[sub]) <= 2.0 ** -126)
    k = x.size - specials.size
    s = got[k:]
    assert s[0] == 0.0 and not np.signbit(s[0]) and s[1] == 0.0 and np.signbit(s[1])
    assert s[2] == 1.0 and s[3] == -1.0 and np.isnan(s[4])
    assert np.all(s[11:13] == 1.0) and s[13] == 1.0 and s[14] == -1.0
    # odd: tanh(-x) is -tanh(x) bit for bit
    h = k // 2
    neg = P.Group(nodes, [((h,), "f32")], (h,), "f32")
    o2 = torch.full((h,), float("nan"), device=DEV)
    neg.run([torch.from_numpy(-x[:h]).to(DEV)], o2)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(o2).view(np.uint32), (-got[:h]).view(np.uint32))


@pytest.mark.gpu
def test_emitted_gelu_within_its_bound():
    """The emitted f32 gelu (x Phi(x), Phi from the Chebyshev-fitted erfc,
    fractional error 1.2e-7, and a rounded exponent whose error grows with
    w^2): against x erfc(-w)/2 in float64, w = x/sqrt 2 rounded to f32 as the
    oracle rounds it, relative error below 2e-6 where |x| <= 4.3 (1.2e-6 in
    an f32 emulation with a correctly rounded 2^x and reciprocal; the
    hardware's add about an ulp each), and within the f32 tolerance (1e-7 +
    2e-6 |ref|) of the unrounded definition everywhere; ±0 keep their sign,
    +inf gives +inf, NaN gives NaN."""
    from scipy.special import erfc
    nodes = parse_dag("%0 = input 0\n%1 = gelu %0\n")
    rng = np.random.default_rng(53)
    n = 1 << 22
    x = np.concatenate([rng.uniform(-4.3, 4.3, n // 2), rng.uniform(-30.0, 30.0, n // 4),
                        rng.normal(0.0, 1.0, n // 4)]).astype(np.float32)
    specials = np.array([0.0, -0.0, np.inf, np.nan], dtype=np.float32)
    x = np.concatenate([x, specials])
    g = P.Group(nodes, [((x.size,), "f32")], (x.size,), "f32")
    assert "psk_gelu(" in P.psk_group_source(g.desc)
    out = torch.full((x.size,), float("nan"), device=DEV)
    g.run([torch.from_numpy(x).to(DEV)], out)
    torch.cuda.synchronize()
    got = to_np(out).astype(np.float64)
    xd = x.astype(np.float64)
    ref = 0.5 * xd * erfc(-xd / np.sqrt(2.0))
    fin = np.isfinite(x)
    assert np.all(np.abs(got[fin] - ref[fin]) <= 1e-7 + 2e-6 * np.abs(ref[fin]))
    w32 = (x * np.float32(0.70710678118654752440)).astype(np.float64)
    ref32 = 0.5 * xd * erfc(-w32)
    mid = fin & (np.abs(xd) <= 4.3) & (ref32 != 0)
    rel = np.abs(got[mid] - ref32[mid]) / np.abs(ref32[mid])
    assert rel.max() <= 2e-6, f"gelu: relative error {rel.max():.3g} at x = {x[mid][rel.argmax()]!r}"
    s = got[-4:]
    assert s[0] == 0.0 and not np.signbit(s[0]) and s[1] == 0.0 and np.signbit(s[1])
    assert s[2] == np.inf and np.isnan(s[3])
