"""GPU parity of the online normalizer (PSK_GROUP_ONLINE: a softmax's sum
taken in its maximum's pass, rescaled as the running maximum grows) against
the oracle's exact two-pass softmax.  The sum's rounding differs from the
exact one (declared differs), so the bar is the f32 tolerance (one bf16
ulp for bf16 results), and refused positions must still be +0 bits."""
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


def close(dt):
    return assert_f32_close if dt == "f32" else assert_bf16_close


@pytest.mark.parametrize("R,C,dt,period", [(8, 131072, "f32", None), (5, 33333, "f32", 3), (3, 300000, "f32", None),
                                           (3, 131072, "bf16", 7), (300, 1024, "f32", 1024), (70, 1023, "f32", 64),
                                           (33, 1000, "bf16", 1000), (9, 12, "f32", 5), (40, 4096, "f32", None)])
def test_online_softmax(R, C, dt, period):
    x = configs.softmax_scores(R, C, device=DEV, seed=R * 7 + C)
    if dt == "bf16":
        x = x.to(torch.bfloat16)
    dag = configs.softmax_dag(0.125) if period is None else configs.softmax_causal_dag(0.125, period)
    g = P.Group(dag, [((R, C), dt)], (R, C), dt, online=True)
    out = torch.full_like(x, float("nan"))
    g.run([x], out)
    torch.cuda.synchronize()
    got = to_np(out)
    ref = oracle.eval_group(dag, [to_np(x)], (R, C), F32 if dt == "f32" else BF16)
    close(dt)(got, ref, f"online softmax {R}x{C} {dt}")
    if period is not None:
        q = np.arange(R)[:, None] % period
        assert np.all(got[np.arange(C)[None, :] > q] == 0)


@pytest.mark.parametrize("layout", ["lanes=16", "lanes=32", "lanes=256", "tiled=1,rc=0,lc=0", "tiled=1,rc=1,lc=1"])
def test_online_softmax_layouts(layout, monkeypatch):
    monkeypatch.setenv("PSK_LAYOUT", layout)
    R, C = 37, 512
    x = configs.softmax_scores(R, C, device=DEV, seed=77)
    dag = configs.softmax_causal_dag(0.125, 100)
    g = P.Group(dag, [((R, C), "f32")], (R, C), "f32", online=True)
    out = torch.full_like(x, float("nan"))
    g.run([x], out)
    torch.cuda.synchronize()
    assert_f32_close(to_np(out), oracle.eval_group(dag, [to_np(x)], (R, C), F32), f"online {layout}")


@pytest.mark.parametrize("R,C", [(40, 1000), (6, 70000)])
def test_online_masked_softmax_with_emptied_rows(R, C):
    x = configs.softmax_scores(R, C, device=DEV, seed=R + C)
    m = configs.random_mask(R, C, 0.3, empty_rows=[0, R - 1], device=DEV, seed=R)
    dag = configs.softmax_masked_dag(0.125)
    g = P.Group(dag, [((R, C), "f32"), ((R, C), "u8")], (R, C), "f32", online=True)
    out = torch.full_like(x, float("nan"))
    g.run([x, m], out)
    torch.cuda.synchronize()
    got = to_np(out)
    ref = oracle.eval_group(dag, [to_np(x), m.cpu().numpy().view(np.uint8)], (R, C), F32)
    assert_f32_close(got, ref, f"online masked {R}x{C}")
    assert np.all(got[[0, R - 1]].view(np.uint32) == 0)
    assert np.all(got[~m.cpu().numpy()].view(np.uint32) == 0)


@pytest.mark.parametrize("layout,C,kind", [("split=0", 131072, 3), ("sept=32", 131072, 4), ("sept=16", 70000, 4),
                                           ("", 300000, 4)])
def test_online_wide_rows_split_and_tiled(layout, C, kind, monkeypatch):
    """The online normalizer over rows shared by several workgroups (each
    member's (maximum, sum) rescaled to the row's maximum when combined)
    and over the tiled kernel, against the exact oracle; rows whose maximum
    sits in different members, a rising row, and a masked row."""
    monkeypatch.setenv("PSK_LAYOUT", layout)
    R = 6
    x = configs.softmax_scores(R, C, device=DEV, seed=C + len(layout))
    x[1] = torch.linspace(-30.0, 30.0, C, device=DEV)          # maximum in the last member
    x[2] = torch.linspace(30.0, -30.0, C, device=DEV)          # in the first
    x[3, C // 2] = 40.0                                         # one spike in a middle member
    dag = configs.softmax_dag(0.125)
    g = P.Group(dag, [((R, C), "f32")], (R, C), "f32", online=True)
    assert g.info.kind == kind
    out = torch.full_like(x, float("nan"))
    g.run([x], out)
    torch.cuda.synchronize()
    assert_f32_close(to_np(out), oracle.eval_group(dag, [to_np(x)], (R, C), F32), f"online wide {layout} {C}")
    g.check()                                                    # no bounded wait ran out


@pytest.mark.parametrize("C", [1024, 131072])
def test_online_softmax_rising_rows(C):
    """Rows that rise from start to end: the running maximum grows in every
    tile a lane walks, the most rescaling the normalizer can see."""
    R = 4
    ramp = torch.linspace(-20.0, 20.0, C, device=DEV)
    x = torch.stack([ramp, ramp * 0.5, ramp * 0.01, ramp + torch.randn(C, device=DEV) * 0.1]) * 8.0
    dag = configs.softmax_dag(0.125)
    g = P.Group(dag, [((R, C), "f32")], (R, C), "f32", online=True)
    out = torch.full_like(x, float("nan"))
    g.run([x], out)
    torch.cuda.synchronize()
    assert_f32_close(to_np(out), oracle.eval_group(dag, [to_np(x)], (R, C), F32), f"online rising {C}")


def test_online_wide_full_size_sampled_rows():
    R, C = 8192, 131072
    x = configs.softmax_scores(R, C, device=DEV)
    dag = configs.softmax_dag(0.125)
    g = P.Group(dag, [((R, C), "f32")], (R, C), "f32", online=True)
    assert g.info.kind == 4 and g.info.split == 4      # split rows: (maximum, sum) pairs exchanged
    out = torch.empty_like(x)
    g.run([x], out)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, R - 1], np.random.default_rng(5).integers(0, R, 40)]))
    ri = torch.from_numpy(rows).to(DEV)
    assert_f32_close(to_np(out[ri]), oracle.eval_group(dag, [to_np(x[ri])], (len(rows), C), F32),
                     "online wide full size")
