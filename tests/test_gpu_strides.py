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
