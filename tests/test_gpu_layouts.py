"""GPU parity of the row kernel's other launch layouts against the oracle:
32 lanes a row (the two 16-lane halves joined by a lane swizzle), one wave
a row holding up to 64 elements a lane, and the tiled kernel forced on rows
the register kernel would take.  The layout changes the reduction order, so
the bar is the tolerance, not the default layout's bits."""
import numpy as np
import pytest
import torch

import oracle
from synth import configs
from tests.gpu_util import assert_bf16_close, assert_f32_close, to_np

P = pytest.importorskip("elementwise_reduction_groups_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
F32, BF16 = P.PSK_F32, P.PSK_BF16
EPS = configs.f32(1e-5)

LAYOUTS = ["lanes=32", "lanes=32,block=64", "lanes=64,epmax=64", "tiled=1,rc=1"]


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("R,C,dt", [(70, 1024, "f32"), (33, 1000, "bf16"), (9, 700, "f32")])
def test_causal_softmax_layouts(layout, R, C, dt, monkeypatch):
    monkeypatch.setenv("PSK_LAYOUT", layout)
    x = configs.softmax_scores(R, C, device=DEV, seed=R * C)
    if dt == "bf16":
        x = x.to(torch.bfloat16)
    period = min(C, 64)
    g = P.Group(configs.softmax_causal_dag(0.125, period), [((R, C), dt)], (R, C), dt)
    if layout.startswith("lanes=32"):
        assert g.info.lanes_per_row == 32
    out = torch.full_like(x, float("nan"))
    g.run([x], out)
    torch.cuda.synchronize()
    ref = oracle.eval_group(configs.softmax_causal_dag(0.125, period), [to_np(x)], (R, C), F32 if dt == "f32" else BF16)
    (assert_f32_close if dt == "f32" else assert_bf16_close)(to_np(out), ref, f"{layout} softmax {R}x{C}")
    q = np.arange(R)[:, None] % period
    assert np.all(to_np(out)[np.arange(C)[None, :] > q] == 0)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_masked_softmax_with_emptied_rows_layouts(layout, monkeypatch):
    monkeypatch.setenv("PSK_LAYOUT", layout)
    R, C = 40, 1000
    x = configs.softmax_scores(R, C, device=DEV, seed=41)
    m = configs.random_mask(R, C, 0.3, empty_rows=[0, 13], device=DEV, seed=42)
    g = P.Group(configs.softmax_masked_dag(0.125), [((R, C), "f32"), ((R, C), "u8")], (R, C), "f32")
    out = torch.full_like(x, float("nan"))
    g.run([x, m], out)
    torch.cuda.synchronize()
    got = to_np(out)
    ref = oracle.eval_group(configs.softmax_masked_dag(0.125), [to_np(x), m.cpu().numpy().view(np.uint8)], (R, C), F32)
    assert_f32_close(got, ref, f"{layout} masked softmax")
    assert np.all(got[[0, 13]].view(np.uint32) == 0)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_rmsnorm_gelu_layouts(layout, monkeypatch):
    monkeypatch.setenv("PSK_LAYOUT", layout)
    R, C = 21, 1024
    x, r, gm = configs.rmsnorm_inputs(R, C, device=DEV, seed=43)
    g = P.Group(configs.rmsnorm_gelu_dag(EPS), [((R, C), "bf16"), ((R, C), "bf16"), ((C,), "bf16")], (R, C), "bf16")
    out = torch.full((R, C), float("nan"), dtype=torch.bfloat16, device=DEV)
    g.run([x, r, gm], out)
    torch.cuda.synchronize()
    ref = oracle.eval_group(configs.rmsnorm_gelu_dag(EPS), [to_np(x), to_np(r), to_np(gm)], (R, C), BF16)
    assert_bf16_close(to_np(out), ref, f"{layout} rmsnorm+gelu")
