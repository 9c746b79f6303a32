"""Strided inputs on the GPU, through the C ABI: views read in place (no
copy) against the oracle on a contiguous copy of the same view.

  * the causal softmax over scores.transpose(1, 2) (leading axes permuted,
    unit last-axis step: the vector path);
  * add + RMSNorm + gamma + GELU over a residual sliced from a wider
    tensor (row step twice the row length) and an x at an element offset;
  * the 64-node chain over a strided A (every second column: the element
    path) and a transposed A;
  * a [R, 1] value expanded along the rows (stride 0) equal to the [R, 1]
    input, bit for bit;
  * an output inside a strided input's span refused before any launch.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import configs
from tests.gpu_util import assert_bf16_close, assert_bits, assert_f32_close, to_np

P = pytest.importorskip("elementwise_reduction_groups_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
EPS = configs.f32(1e-5)


def spec(t, dt):
    return (tuple(t.shape), dt, tuple(t.stride()))


@pytest.mark.parametrize("B,H,T", [(2, 4, 256), (1, 3, 100)])
def test_causal_softmax_over_transposed_scores(B, H, T):
    x = configs.softmax_scores(B * H * T, T, device=DEV, seed=T).reshape(B, H, T, T)
    xt = x.transpose(1, 2)                                   # [B, T, H, T], strides (HTT, T, TT, 1)
    assert not xt.is_contiguous()
    before = to_np(x)
    g = P.Group(configs.softmax_causal_dag(0.125, T), [spec(xt, "f32")], tuple(xt.shape), "f32")
    assert g.info.vec == (4 if T % 4 == 0 else 1)
    out = torch.full(tuple(xt.shape), float("nan"), device=DEV)
    g.run([xt], out)
    torch.cuda.synchronize()
    ref = oracle.softmax_causal(to_np(xt.contiguous()).reshape(-1, T), T, 0.125).reshape(xt.shape)
    assert_f32_close(to_np(out), ref, f"softmax over scores.transpose(1, 2) {B}x{H}x{T}")
    assert_bits(to_np(x), before, "scores unchanged")
    # the dense group refuses the view (it was created for a dense input)
    dense = P.Group(configs.softmax_causal_dag(0.125, T), [(tuple(xt.shape), "f32")], tuple(xt.shape), "f32")
    with pytest.raises(ValueError):
        dense.run([xt], out)


@pytest.mark.parametrize("R,C", [(64, 4096), (37, 1000)])
def test_rmsnorm_over_sliced_residual(R, C):
    xg, rg, gm = configs.rmsnorm_inputs(R, 2 * C, device=DEV, seed=R + C)
    gm = gm[:C].contiguous()
    res = rg[:, :C]                                          # row step 2C
    x = xg[:, C:]                                            # row step 2C, first element at C
    g = P.Group(configs.rmsnorm_gelu_dag(EPS), [spec(x, "bf16"), spec(res, "bf16"), ((C,), "bf16")], (R, C),
                "bf16")
    assert g.info.vec == (8 if C % 8 == 0 else 1)
    out = torch.full((R, C), float("nan"), dtype=torch.bfloat16, device=DEV)
    g.run([x, res, gm], out)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm_gelu(to_np(x.contiguous()), to_np(res.contiguous()), to_np(gm), EPS)
    assert_bf16_close(to_np(out), ref, f"RMSNorm over a sliced residual {R}x{C}")


@pytest.mark.parametrize("view", ["every_second_column", "transposed"])
def test_chain64_over_strided_a(view):
    N = 1024
    nodes = configs.chain64_dag()
    Abig, B, Cc = configs.chain_inputs(N, 2 * N, device=DEV, seed=8)
    B = B.contiguous()
    Cc = Cc[:, :N].contiguous()
    A = Abig[:, ::2] if view == "every_second_column" else Abig[:, :N].t()
    g = P.Group(nodes, [spec(A, "f32"), ((N, 1), "f32"), ((1, N), "f32")], (N, N), "f32")
    assert g.info.vec == 1
    out = torch.full((N, N), float("nan"), device=DEV)
    g.run([A, B, Cc], out)
    torch.cuda.synchronize()
    ref = oracle.eval_group(nodes, [to_np(A.contiguous()), to_np(B), to_np(Cc)], (N, N))
    assert_f32_close(to_np(out), ref, f"chain64 over A {view}")


def test_expanded_row_value_equals_row_input():
    R, C = 96, 640
    from synth.dag import parse_dag
    nodes = parse_dag("%0 = input 0\n%1 = input 1\n%2 = mul %0 %1\n%3 = row_sum %2\n%4 = div %2 %3\n")
    x = configs.softmax_scores(R, C, device=DEV, seed=3)
    b = configs.softmax_scores(R, 1, device=DEV, seed=4)
    be = b.expand(R, C)                                      # strides (1, 0)
    g1 = P.Group(nodes, [((R, C), "f32"), ((R, 1), "f32")], (R, C), "f32")
    g2 = P.Group(nodes, [((R, C), "f32"), spec(be, "f32")], (R, C), "f32")
    o1 = torch.full((R, C), float("nan"), device=DEV)
    o2 = torch.full((R, C), float("nan"), device=DEV)
    g1.run([x, b], o1)
    g2.run([x, be], o2)
    torch.cuda.synchronize()
    assert_bits(to_np(o2), to_np(o1), "expanded row value")


def test_output_inside_a_strided_span_is_refused():
    R, C = 16, 64
    big = torch.zeros((R, 2 * C), device=DEV)
    view = big[:, C:]                                        # reaches from element C to the end of big
    out = big.view(-1)[:R * C].view(R, C)                    # dense, inside that span
    g = P.Group(configs.softmax_dag(0.125), [spec(view, "f32")], (R, C), "f32")
    with pytest.raises(P.PskError) as ei:
        g.run([view], out)
    assert ei.value.status == P.PSK_E_ALIAS
    torch.cuda.synchronize()
    assert not big.any().item(), "nothing was launched"


def _strided_copy(x, how, gen):
    """A view with x's values and shape over a larger buffer: rows padded
    (row step longer than the row, first element at an offset), every
    second element of the last axis, or the last two axes stored
    transposed."""
    S = tuple(x.shape)
    if how == "pad":
        off = int(torch.randint(0, 3, (1,), generator=gen))
        buf = torch.full(S[:-1] + (S[-1] + 5 + off,), 7.0, device=DEV).to(x.dtype)
        v = buf[..., off:off + S[-1]]
    elif how == "step":
        buf = torch.full(S[:-1] + (2 * S[-1],), 7.0, device=DEV).to(x.dtype)
        v = buf[..., ::2]
    else:
        buf = torch.full(S[:-2] + (S[-1], S[-2]), 7.0, device=DEV).to(x.dtype)
        v = buf.transpose(-1, -2)
    v.copy_(x)
    return v


@pytest.mark.parametrize("kind,chunk", [("pw", 0), ("pw", 1), ("row", 0), ("row", 1), ("masked", 0)])
def test_random_groups_over_strided_views(kind, chunk):
    """Seeded random groups of exact operations (tests/random_groups.py:
    pointwise, row, and row under a causal or byte mask) whose float inputs
    are given as strided views (padded rows at an offset, every second
    element, transposed storage), against the oracle on the contiguous
    inputs: bit for bit (bf16 row results within one ulp, as in the dense
    tests); the buffers around the views unchanged."""
    import random
    from tests.random_groups import random_group, random_row_group
    from tests.test_gpu_random_groups import make_input, same_bits
    rng = random.Random(6000 + 10 * chunk + len(kind))
    gen = torch.Generator().manual_seed(6100 + chunk)
    TD = {"f32": torch.float32, "bf16": torch.bfloat16}
    for trial in range(8):
        if kind == "pw":
            nodes, inputs, shape, dt, ex = random_group(rng)
            extras = [(m, shape, xdt) for m, xdt in ex]
        else:
            nodes, inputs, shape, dt, extras = random_row_group(rng, masks=kind == "masked")
        dense = [make_input(s, t, gen, False) for s, t in inputs]
        if kind != "pw":
            dense = [x if t == "u8" else torch.where(x == 0, torch.ones_like(x), x) for x, (_, t) in zip(dense, inputs)]
        specs, views = [], []
        for x, (s, t) in zip(dense, inputs):
            hows = ["pad", "step"] + (["transpose"] if len(s) >= 2 else [])
            if t == "u8" or len(s) == 0 or rng.random() < 0.3:
                specs.append((s, t)); views.append(x)
                continue
            v = _strided_copy(x, rng.choice(hows), gen)
            specs.append((s, t, tuple(v.stride()))); views.append(v)
        g = P.Group(nodes, specs, shape, dt, root=len(nodes) - 1, extras=extras)
        out = torch.full(shape, float("nan"), dtype=TD[dt], device=DEV)
        xs = [torch.full(xsh, float("nan"), dtype=TD[xdt], device=DEV) for _, xsh, xdt in extras]
        bufs = [to_np(v.as_strided((v.untyped_storage().nbytes() // v.element_size(),), (1,), 0))
                for v in views if not v.is_contiguous()]
        g.run(views, out, extra_outs=xs or None)
        torch.cuda.synchronize()
        ins = [x.cpu().numpy().view(np.uint8) if x.dtype == torch.uint8 else to_np(x) for x in dense]
        refx = [(m, np.zeros(xsh, np.float32 if xdt == "f32" else np.uint16)) for m, xsh, xdt in extras]
        ref = oracle.eval_group(nodes, ins, shape, P.PSK_F32 if dt == "f32" else P.PSK_BF16, root=len(nodes) - 1,
                                extras=refx)
        what = f"{kind} chunk {chunk} trial {trial}: kind {g.info.kind} shape {shape} {dt} specs {specs}"
        for name, got, r in [("root", to_np(out), ref)] + [(f"extra {m}", to_np(x), r) for (m, r), x in zip(refx, xs)]:
            if got.dtype == np.uint16 and kind != "pw":
                assert_bf16_close(got, r, f"{what}: {name}")
            else:
                ok = same_bits(got, r)
                assert ok.all(), f"{what}: {name} differs at {int((~ok).sum())} of {ok.size}"
        after = [to_np(v.as_strided((v.untyped_storage().nbytes() // v.element_size(),), (1,), 0))
                 for v in views if not v.is_contiguous()]
        for b, a in zip(bufs, after):
            assert_bits(a, b, f"{what}: buffer around a view unchanged")
