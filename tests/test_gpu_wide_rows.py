"""GPU parity of the tiled row kernel (rows too wide to live in registers:
more than 32 elements per lane at 1024 lanes) against the oracle: each
reduction phase walks the row in tiles and re-reads what it needs."""
import numpy as np
import pytest
import torch

import oracle
from synth import configs
from tests.gpu_util import assert_bf16_close, assert_bits, assert_f32_close, to_np

P = pytest.importorskip("elementwise_reduction_groups_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
F32, BF16 = P.PSK_F32, P.PSK_BF16
EPS = configs.f32(1e-5)


# every wide-row test runs through both kernels for rows too wide for one
# workgroup's registers: rows split over workgroups (the default, kind 4)
# and the tiled kernel (kind 3, forced)
WIDE = pytest.mark.parametrize("layout,kind", [("", 4), ("tiled=1", 3)])


def _layout(monkeypatch, layout):
    if layout:
        monkeypatch.setenv("PSK_LAYOUT", layout)
    else:
        monkeypatch.delenv("PSK_LAYOUT", raising=False)


@WIDE
@pytest.mark.parametrize("R,C,dt", [(8, 40000, "f32"), (4, 65536, "f32"), (3, 131072, "bf16"), (5, 33333, "f32"),
                                    (2, 300000, "f32")])
def test_wide_softmax(R, C, dt, layout, kind, monkeypatch):
    _layout(monkeypatch, layout)
    x = configs.softmax_scores(R, C, device=DEV, seed=C)
    if dt == "bf16":
        x = x.to(torch.bfloat16)
    # a causal period shorter than the row count, so rows keep various prefixes;
    # and the unmasked softmax (period larger than every column index)
    for period in (3, C):
        g = P.Group(configs.softmax_causal_dag(0.125, period), [((R, C), dt)], (R, C), dt)
        info = g.info
        assert info.kind == kind and (info.tiles >= 2 or info.split >= 2)
        out = torch.full_like(x, float("nan"))
        g.run([x], out)
        torch.cuda.synchronize()
        g.check()
        ref = oracle.eval_group(configs.softmax_causal_dag(0.125, period), [to_np(x)], (R, C), F32 if dt == "f32"
                                else BF16)
        if dt == "f32":
            assert_f32_close(to_np(out), ref, f"wide softmax {R}x{C} period {period}")
        else:
            assert_bf16_close(to_np(out), ref, f"wide softmax {R}x{C} period {period}")


@WIDE
def test_wide_masked_softmax_with_emptied_rows(layout, kind, monkeypatch):
    _layout(monkeypatch, layout)
    R, C = 6, 70000
    x = configs.softmax_scores(R, C, device=DEV, seed=5)
    m = configs.random_mask(R, C, 0.2, empty_rows=[2], device=DEV, seed=6)
    g = P.Group(configs.softmax_masked_dag(0.125), [((R, C), "f32"), ((R, C), "u8")], (R, C), "f32")
    assert g.info.kind == kind
    out = torch.full_like(x, float("nan"))
    g.run([x, m], out)
    torch.cuda.synchronize()
    got = to_np(out)
    ref = oracle.eval_group(configs.softmax_masked_dag(0.125), [to_np(x), m.cpu().numpy().view(np.uint8)], (R, C),
                            F32)
    assert_f32_close(got, ref, "wide masked softmax")
    assert np.all(got[2].view(np.uint32) == 0)


@WIDE
def test_wide_layernorm_with_statistics(layout, kind, monkeypatch):
    _layout(monkeypatch, layout)
    R, C = 8, 50000
    x, gm, bt = configs.layernorm_inputs(R, C, device=DEV, seed=9)
    g = P.Group(configs.layernorm_dag(EPS), [((R, C), "bf16"), ((C,), "bf16"), ((C,), "bf16")], (R, C), "bf16",
                root=configs.LAYERNORM_ROOT,
                extras=[(configs.LAYERNORM_MEAN, (R, 1), "f32"), (configs.LAYERNORM_RSTD, (R, 1), "f32")])
    assert g.info.kind == kind
    out = torch.full((R, C), float("nan"), dtype=torch.bfloat16, device=DEV)
    mean = torch.full((R, 1), float("nan"), device=DEV)
    rstd = torch.full((R, 1), float("nan"), device=DEV)
    g.run([x, gm, bt], out, extra_outs=[mean, rstd])
    torch.cuda.synchronize()
    rm, rr = np.zeros((R, 1), np.float32), np.zeros((R, 1), np.float32)
    ref = oracle.eval_group(configs.layernorm_dag(EPS), [to_np(x), to_np(gm), to_np(bt)], (R, C), BF16,
                            root=configs.LAYERNORM_ROOT,
                            extras=[(configs.LAYERNORM_MEAN, rm), (configs.LAYERNORM_RSTD, rr)])
    # statistics: a lane sums its elements in order (tiled: tiles x vectors x vec per lane; split: its
    # segment's elements), then the wave butterfly, the waves, and (split) the workgroups of the row;
    # against float64 within that path's bound
    U = 2.0 ** -24
    if kind == 3:
        k = g.info.tiles * 2 * g.info.vec + 6 + 15
    else:
        k = -(-C // (g.info.split * g.info.block)) + g.info.vec + 6 + 7 + g.info.split
    x64 = x.double().cpu()
    m64 = x64.mean(dim=1)
    assert torch.all((mean.double().cpu()[:, 0] - m64).abs() <= k * U * x64.abs().mean(dim=1) + U * m64.abs())
    r64 = 1.0 / torch.sqrt(x64.var(dim=1, unbiased=False) + EPS)
    assert ((rstd.double().cpu()[:, 0] - r64).abs() / r64).max() <= (k + 8) * U
    d = np.abs(to_np(out).astype(np.int32) - ref.astype(np.int32))
    # away from cancellations the outputs are within one bf16 ulp
    big = np.abs((ref.astype(np.uint32) << 16).view(np.float32)) > 0.05
    assert d[big].max() <= 1


@WIDE
def test_wide_rms_norm_storing_h_in_place(layout, kind, monkeypatch):
    _layout(monkeypatch, layout)
    R, C = 4, 45000
    x, res, gm = configs.rmsnorm_inputs(R, C, device=DEV, seed=10)
    xn, rn, gn = to_np(x), to_np(res), to_np(gm)
    g = P.Group(configs.rmsnorm_gelu_dag(EPS), [((R, C), "bf16"), ((R, C), "bf16"), ((C,), "bf16")], (R, C), "bf16",
                extras=[(configs.RMSNORM_H, (R, C), "bf16")])
    assert g.info.kind == kind
    out = torch.full((R, C), float("nan"), dtype=torch.bfloat16, device=DEV)
    g.run([x, res, gm], out, extra_outs=[res])
    torch.cuda.synchronize()
    rh = np.zeros((R, C), np.uint16)
    ref = oracle.eval_group(configs.rmsnorm_gelu_dag(EPS), [xn, rn, gn], (R, C), BF16,
                            extras=[(configs.RMSNORM_H, rh)])
    np.testing.assert_array_equal(to_np(res), rh)
    assert_bf16_close(to_np(out), ref, "wide rmsnorm")


@pytest.mark.parametrize("case", ["softmax_f32", "softmax_bf16_ragged", "masked", "layernorm", "rmsnorm_h"])
def test_register_cache_changes_no_bit(case, monkeypatch):
    """Per-row inputs of the leading tiles kept in registers and of the next
    ones in LDS between phases (none, a few, every tile): the same
    arithmetic in the same order, so the same bits as re-reading them."""
    if case == "softmax_f32":
        R, C = 3, 131072
        ins = [configs.softmax_scores(R, C, device=DEV, seed=31)]
        args = (configs.softmax_dag(0.125), [((R, C), "f32")], (R, C), "f32")
        kw, xs = {}, []
    elif case == "softmax_bf16_ragged":
        R, C = 4, 70001
        ins = [configs.softmax_scores(R, C, device=DEV, seed=32).to(torch.bfloat16)]
        args = (configs.softmax_causal_dag(0.125, 50000), [((R, C), "bf16")], (R, C), "bf16")
        kw, xs = {}, []
    elif case == "masked":
        R, C = 4, 70000
        ins = [configs.softmax_scores(R, C, device=DEV, seed=33),
               configs.random_mask(R, C, 0.4, empty_rows=[1], device=DEV, seed=34)]
        args = (configs.softmax_masked_dag(0.125), [((R, C), "f32"), ((R, C), "u8")], (R, C), "f32")
        kw, xs = {}, []
    elif case == "layernorm":
        R, C = 4, 50000
        ins = list(configs.layernorm_inputs(R, C, device=DEV, seed=35))
        args = (configs.layernorm_dag(EPS), [((R, C), "bf16"), ((C,), "bf16"), ((C,), "bf16")], (R, C), "bf16")
        kw = dict(root=configs.LAYERNORM_ROOT,
                  extras=[(configs.LAYERNORM_MEAN, (R, 1), "f32"), (configs.LAYERNORM_RSTD, (R, 1), "f32")])
        xs = [((R, 1), torch.float32), ((R, 1), torch.float32)]
    else:
        R, C = 3, 45000
        ins = list(configs.rmsnorm_inputs(R, C, device=DEV, seed=36))
        args = (configs.rmsnorm_gelu_dag(EPS), [((R, C), "bf16"), ((R, C), "bf16"), ((C,), "bf16")], (R, C), "bf16")
        kw = dict(extras=[(configs.RMSNORM_H, (R, C), "bf16")])
        xs = [((R, C), torch.bfloat16)]
    runs = []
    for layout in ("rc=0,lc=0", "rc=1,lc=0", "rc=0,lc=2", "rc=3,lc=1", "rc=1,lc=64", ""):
        monkeypatch.setenv("PSK_LAYOUT", "tiled=1" + ("," + layout if layout else ""))
        g = P.Group(*args, **kw)
        assert g.info.kind == 3
        out = torch.full((R, C), float("nan"), dtype=ins[0].dtype, device=DEV)
        ex = [torch.full(sh, float("nan"), dtype=dt, device=DEV) for sh, dt in xs]
        g.run(ins, out, extra_outs=ex or None)
        torch.cuda.synchronize()
        runs.append([to_np(out)] + [to_np(e) for e in ex])
    for other in runs[1:]:
        for a, b in zip(runs[0], other):
            np.testing.assert_array_equal(a.view(np.uint8), b.view(np.uint8), f"register cache, {case}")


def test_wide_softmax_full_size_sampled_rows():
    """[8192, 131072] f32 in the layout that is timed (each row split over 4
    workgroups of 512 lanes)."""
    R, C = 8192, 131072
    x = configs.softmax_scores(R, C, device=DEV)
    g = P.Group(configs.softmax_dag(0.125), [((R, C), "f32")], (R, C), "f32")
    assert g.info.kind == 4 and g.info.split == 4 and g.info.block == 512
    out = torch.empty_like(x)
    g.run([x], out)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, R - 1], np.random.default_rng(93).integers(0, R, 40)]))
    ri = torch.from_numpy(rows).to(DEV)
    ref = oracle.eval_group(configs.softmax_dag(0.125), [to_np(x[ri])], (len(rows), C), F32)
    assert_f32_close(to_np(out[ri]), ref, "wide softmax full size")
    g.check()


# ------------------------------------------------------------- split rows
def _split_softmax(R, C, **kw):
    return P.Group(configs.softmax_dag(0.125), [((R, C), "f32")], (R, C), "f32", **kw)


def test_split_rows_same_bits_across_runs_and_graph_replays():
    """A split-rows group gives the same bits on every run: eager runs, and
    replays of a captured HIP graph with eager work in between (the tags of
    the exchange come from a device-side generation counter, not from the
    launch arguments a graph freezes)."""
    R, C = 300, 131072
    x = configs.softmax_scores(R, C, device=DEV, seed=41)
    g = _split_softmax(R, C)
    assert g.info.kind == 4
    ref = torch.full_like(x, float("nan"))
    g.run([x], ref)                                   # first run: loads the kernel, allocates the state
    torch.cuda.synchronize()
    want = to_np(ref)
    oref = oracle.eval_group(configs.softmax_dag(0.125), [to_np(x[:7])], (7, C), F32)
    assert_f32_close(want[:7], oref, "split softmax")
    for k in range(3):
        out = torch.full_like(x, float("nan"))
        g.run([x], out)
        torch.cuda.synchronize()
        assert_bits(to_np(out), want, f"eager run {k}")
    out = torch.full_like(x, float("nan"))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        g.run([x], out)
    torch.cuda.synchronize()
    for k in range(4):
        out.fill_(float("nan"))
        other = torch.full_like(x, 0.0)
        g.run([x], other)                             # eager work between the replays
        graph.replay()
        torch.cuda.synchronize()
        assert_bits(to_np(out), want, f"graph replay {k}")
        assert_bits(to_np(other), want, f"eager run between replays {k}")
    g.check()


def test_split_rows_fewer_rows_than_teams():
    for R in (1, 3, 9):
        C = 70000
        x = configs.softmax_scores(R, C, device=DEV, seed=R)
        g = _split_softmax(R, C)
        assert g.info.kind == 4
        out = torch.full_like(x, float("nan"))
        g.run([x], out)
        torch.cuda.synchronize()
        ref = oracle.eval_group(configs.softmax_dag(0.125), [to_np(x)], (R, C), F32)
        assert_f32_close(to_np(out), ref, f"split softmax, {R} rows")
        g.check()


def test_split_rows_bounded_wait_is_reported(monkeypatch):
    """A wait that runs out is reported, not hung on: with the bound set to
    no tries at all (from the host, at the group's creation), a wait that
    does not find its partial at once gives up, the launch still finishes,
    and psk_group_check reports PSK_E_HIP once; the same group shape with
    the default bound then gives the oracle's result."""
    R, C = 2048, 131072
    x = configs.softmax_scores(R, C, device=DEV, seed=43)
    monkeypatch.setenv("PSK_SPLIT_WAIT", "0")
    g = _split_softmax(R, C)
    monkeypatch.delenv("PSK_SPLIT_WAIT")
    out = torch.full_like(x, float("nan"))
    g.run([x], out)
    with pytest.raises(P.PskError) as ei:
        g.check()
    assert ei.value.status == P.PSK_E_HIP
    g.check()                                          # reported once
    ok = _split_softmax(R, C)
    out.fill_(float("nan"))
    ok.run([x], out)
    torch.cuda.synchronize()
    ok.check()
    rows = torch.tensor([0, 1, R // 2, R - 1], device=DEV)
    ref = oracle.eval_group(configs.softmax_dag(0.125), [to_np(x[rows])], (4, C), F32)
    assert_f32_close(to_np(out[rows]), ref, "after a reported timeout")
