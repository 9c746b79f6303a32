"""GPU parity of the online normalizer (PSK_GROUP_ONLINE: a softmax's sum
taken in its maximum's pass, rescaled as the running maximum grows) against
the oracle's exact two-pass softmax.  The sum's rounding differs from the
exact one (declared differs), so the bar is the f32 tolerance (one bf16
ulp for bf16 results), and refused positions must still be +0 bits."""
import random

import numpy as np
import pytest
import torch

import oracle
from synth import configs
from tests.gpu_util import assert_bf16_close, assert_bits, assert_f32_close, to_np
from tests.random_groups import random_online_group

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


def _widen(a):
    return (a.astype(np.uint32) << 16).view(np.float32) if a.dtype == np.uint16 else a


class _Normalized:
    """The group's softmax evaluated with an exact normalizer: the oracle's
    own exponentials e (f32, as the oracle computes them, the group's stored
    values included, since a value stored as bf16 is read rounded), their
    float64 row sum s64, and the members after the sum (e / s, a product
    with an input, a WHERE) applied in float64.  The oracle's sequential f32
    sum of n terms is itself within about n ulps only, so a kernel that adds
    in another order is compared with the exact sum instead, within its own
    order's bound: at most `per_lane` terms in sequence on a lane, each with
    at most one rescaling product, then at most 64 more steps across lanes,
    waves and workgroups, one rounding of 2^-24 each; the terms themselves
    are within 2e-6 of the oracle's, and each later member rounds once."""

    def __init__(self, nodes, ins, shape, extras, info):
        self.s_node = next(i for i, n in enumerate(nodes) if n.op == "row_sum")
        e = nodes[self.s_node].args[0]
        refx = [(m, np.zeros(xsh, np.float32 if xdt == "f32" else np.uint16)) for m, xsh, xdt in extras if m != e]
        ex = np.zeros(shape, np.float32)
        oracle.eval_group(nodes, ins, shape, F32, root=len(nodes) - 1, extras=refx + [(e, ex)])
        self.s64 = ex.astype(np.float64).sum(axis=-1, keepdims=True)
        v = {}
        for i in range(self.s_node + 1, len(nodes)):
            nd = nodes[i]
            if nd.op == "div":
                v[i] = ex.astype(np.float64) / self.s64
            elif nd.op == "mul":
                v[i] = v[nd.args[0]] * _widen(ins[nodes[nd.args[1]].iparam]).astype(np.float64)
            elif nd.op == "where":
                v[i] = np.where(ins[nodes[nd.args[0]].iparam] != 0, v[nd.args[1]], nd.imm)
            else:
                raise AssertionError(f"no float64 form for {nd.op}")
        self.root64 = v[len(nodes) - 1]
        per_lane = -(-shape[-1] // (max(1, info.lanes_per_row) * max(1, info.split)))
        self.sum_rel = 2e-6 + (2 * per_lane + 64) * 2.0 ** -24
        self.root_rel = self.sum_rel + 4e-6 + 3 * 2.0 ** -24

    @staticmethod
    def _close(got, ref, rel, what):
        g = _widen(got).astype(np.float64)
        ref = np.broadcast_to(ref, g.shape)
        fin = np.isfinite(ref)
        ok = np.isnan(g) == np.isnan(ref)
        ok[fin] &= np.abs(g[fin] - ref[fin]) <= 1e-7 + rel * np.abs(ref[fin])
        if not ok.all():
            i = tuple(np.argwhere(~ok)[0])
            raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outside 1e-7 + {rel:.2e}|exact|; "
                                 f"first at {i}: gpu {g[i]!r} exact {ref[i]!r}")

    def check_oracle(self, ref, cols, what):
        """The oracle's own root (sequential f32 sum) lies within its
        summation bound of the exact reference: a check of the float64 tail."""
        if ref.dtype == np.float32:
            self._close(ref, self.root64, 4e-6 + (2 * cols + 8) * 2.0 ** -24, what)

    def check_sum(self, got, what):
        self._close(got, self.s64, self.sum_rel, what)

    def check_root(self, got, what):
        if got.dtype == np.uint16:       # bf16: within one ulp of the exact value rounded once
            ref = torch.from_numpy(self.root64.astype(np.float32)).to(torch.bfloat16)
            assert_bf16_close(got, to_np(ref), what)
        else:
            self._close(got, self.root64, self.root_rel, what)


def _make(shape, dt, gen):
    if dt == "u8":
        return (torch.randint(0, 3, shape, generator=gen).to(torch.uint8) * 3).to(DEV)     # 0, 3, 6
    x = torch.rand(shape, generator=gen) * 4.0 - 2.0
    return x.to(torch.bfloat16 if dt == "bf16" else torch.float32).to(DEV)


@pytest.mark.parametrize("layout,chunk", [("", 0), ("", 1), ("lanes=16", 2), ("lanes=32", 3), ("sept=16", 4),
                                          ("tiled=1", 5)])
def test_random_online_groups(layout, chunk, monkeypatch):
    """Seeded random groups holding the normalizer's pattern
    (tests/random_groups.py: element chains before the maximum, causal and
    byte masks, broadcast inputs, f32 and bf16 storage, rows of 3 to
    300 000 columns, stored maxima, differences, exponentials and sums),
    under the default launch layouts and forced ones, against the oracle:
    the chain's members (exact operations) bit for bit, the stored maxima,
    differences and exponentials within the f32 tolerance (one bf16 ulp for
    bf16 values), the stored sums and the root against the oracle's
    exponentials normalized exactly (_Normalized).  Rows a byte mask
    empties (short rows) hold a NaN sum, as the exact sum is."""
    if layout:
        monkeypatch.setenv("PSK_LAYOUT", layout)
    _online_groups(random.Random(4000 + chunk), torch.Generator().manual_seed(4100 + chunk), layout, chunk, False)


@pytest.mark.parametrize("chunk", range(2))
def test_random_online_groups_over_strided_views(chunk):
    """The same random groups with their float inputs given as strided
    views (padded rows at an offset, every second element, transposed
    storage), against the oracle on the contiguous inputs."""
    _online_groups(random.Random(4500 + chunk), torch.Generator().manual_seed(4600 + chunk), "", chunk, True)


def _strided(x, gen, rng):
    """x's values in a view over a larger buffer (padded rows at an offset,
    every second element, or the last two axes stored transposed)."""
    S = tuple(x.shape)
    how = rng.choice(["pad", "step"] + (["transpose"] if len(S) >= 2 else []))
    if how == "pad":
        off = int(torch.randint(0, 3, (1,), generator=gen))
        v = torch.full(S[:-1] + (S[-1] + 5 + off,), 7.0, device=DEV).to(x.dtype)[..., off:off + S[-1]]
    elif how == "step":
        v = torch.full(S[:-1] + (2 * S[-1],), 7.0, device=DEV).to(x.dtype)[..., ::2]
    else:
        v = torch.full(S[:-2] + (S[-1], S[-2]), 7.0, device=DEV).to(x.dtype).transpose(-1, -2)
    v.copy_(x)
    return v


def _online_groups(rng, gen, layout, chunk, strided):
    for trial in range(8):
        nodes, inputs, shape, dt, extras = random_online_group(rng)
        tensors = [_make(s, t, gen) for s, t in inputs]
        specs, views = list(inputs), list(tensors)
        if strided:
            for k, ((s, t), x) in enumerate(zip(inputs, tensors)):
                if t != "u8" and len(s) > 0 and rng.random() < 0.7:
                    views[k] = _strided(x, gen, rng)
                    specs[k] = (s, t, tuple(views[k].stride()))
        g = P.Group(nodes, specs, shape, dt, root=len(nodes) - 1, extras=extras, online=True)
        out = torch.full(shape, float("nan"), dtype=torch.bfloat16 if dt == "bf16" else torch.float32, device=DEV)
        xs = [torch.full(xsh, float("nan"), dtype=torch.bfloat16 if xdt == "bf16" else torch.float32, device=DEV)
              for _, xsh, xdt in extras]
        g.run(views, out, extra_outs=xs or None)
        torch.cuda.synchronize()
        ins = [t.cpu().numpy().view(np.uint8) if t.dtype == torch.uint8 else to_np(t) for t in tensors]
        refx = [(m, np.zeros(xsh, np.float32 if xdt == "f32" else np.uint16)) for m, xsh, xdt in extras]
        ref = oracle.eval_group(nodes, ins, shape, F32 if dt == "f32" else BF16, root=len(nodes) - 1, extras=refx)
        what = (f"{layout or 'default'} chunk {chunk} trial {trial}: kind {g.info.kind} shape {shape} {dt} "
                f"inputs {specs} extras {extras} ops {[n.op for n in nodes]}")
        first_max = next(i for i, n in enumerate(nodes) if n.op == "row_max")
        exact = _Normalized(nodes, ins, shape, extras, g.info)
        exact.check_oracle(ref, shape[-1], f"{what}: the oracle's root")
        exact.check_root(to_np(out), f"{what}: root")
        for (m, r), x in zip(refx, xs):
            name, got = f"{what}: extra {m}", to_np(x)
            if m < first_max and nodes[m].op not in ("causal_mask", "where"):
                assert_bits(got, r, name)          # finite exact operations
            elif m == exact.s_node:
                exact.check_sum(got, name)
            elif got.dtype == np.uint16:
                assert_bf16_close(got, r, name)
            else:
                assert_f32_close(got, r, name)
