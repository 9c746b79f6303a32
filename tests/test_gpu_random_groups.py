"""GPU parity of seeded random pointwise groups of IEEE-exact operations
(tests/random_groups.py: every output rank, broadcast inputs of every kind,
bf16/f32 storage, byte masks, extra stored values, some inputs misaligned
so the element path runs) against the oracle, bit for bit: both sides round
once per operation and store the same roundings.  NaN compares as NaN (any
payload)."""
import random

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import assert_bf16_close, to_np
from tests.random_groups import random_group

P = pytest.importorskip("elementwise_reduction_groups_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TD = {"f32": torch.float32, "bf16": torch.bfloat16}
OD = {"f32": P.PSK_F32, "bf16": P.PSK_BF16}


def same_bits(got, ref):
    if got.dtype == np.float32:
        g, r = got.view(np.uint32), ref.view(np.uint32)
        gn, rn = np.isnan(got), np.isnan(ref)
    else:
        g, r = got, ref
        gn = ((g & 0x7F80) == 0x7F80) & ((g & 0x7F) != 0)
        rn = ((r & 0x7F80) == 0x7F80) & ((r & 0x7F) != 0)
    ok = (gn & rn) | (~gn & ~rn & (g == r))
    return ok


def make_input(shape, dt, gen, misaligned):
    if dt == "u8":
        v = torch.randint(0, 3, shape, generator=gen, device="cpu").to(torch.uint8) * 3   # 0, 3, 6
        return v.to(DEV)
    x = (torch.rand(shape, generator=gen) * 4.0 - 2.0)
    x[torch.rand(shape, generator=gen) < 0.05] = 0.0                                  # exact zeros
    x = x.to(TD[dt])
    if misaligned and x.numel() > 0:
        buf = torch.empty(x.numel() + 1, dtype=x.dtype, device=DEV)
        v = buf[1:].view(shape)
        v.copy_(x.to(DEV))
        return v
    return x.to(DEV)


@pytest.mark.parametrize("chunk", range(5))
def test_random_exact_groups_bit_for_bit(chunk):
    rng = random.Random(1000 + chunk)
    gen = torch.Generator().manual_seed(77 + chunk)
    for trial in range(12):
        nodes, inputs, shape, dt, extras = random_group(rng)
        mis = rng.random() < 0.25
        tensors = [make_input(s, t, gen, mis and k == 0) for k, (s, t) in enumerate(inputs)]
        g = P.Group(nodes, inputs, shape, dt, root=len(nodes) - 1, extras=[(m, shape, xdt) for m, xdt in extras])
        out = torch.full(shape, float("nan"), dtype=TD[dt], device=DEV)
        xs = [torch.full(shape, float("nan"), dtype=TD[xdt], device=DEV) for _, xdt in extras]
        g.run(tensors, out, extra_outs=xs or None)
        torch.cuda.synchronize()
        ins_np = [t.cpu().numpy().view(np.uint8) if t.dtype == torch.uint8 else to_np(t) for t in tensors]
        refx = [(m, np.zeros(shape, np.float32 if xdt == "f32" else np.uint16)) for m, xdt in extras]
        ref = oracle.eval_group(nodes, ins_np, shape, OD[dt], root=len(nodes) - 1, extras=refx)
        what = f"chunk {chunk} trial {trial}: shape {shape} {dt} inputs {inputs} extras {extras} misaligned {mis}"
        ok = same_bits(to_np(out), ref)
        assert ok.all(), f"{what}: root differs at {int((~ok).sum())} of {ok.size}"
        for (m, r), x in zip(refx, xs):
            ok = same_bits(to_np(x), r)
            assert ok.all(), f"{what}: extra {m} differs at {int((~ok).sum())} of {ok.size}"


@pytest.mark.parametrize("chunk", range(3))
def test_random_exact_tree_groups_bit_for_bit(chunk):
    """The same operations mapped over random trees (ragged leaves, one
    launch): every leaf's outputs equal the oracle's evaluation of that
    leaf, bit for bit."""
    from tests.random_groups import random_tree_group
    rng = random.Random(2000 + chunk)
    gen = torch.Generator().manual_seed(99 + chunk)
    for trial in range(10):
        nodes, inputs, dt, extras = random_tree_group(rng)
        n_el = sum(1 for s, _ in inputs if s == (1,))
        sizes = [rng.choice([1, 3, 7, 8, 100, 4095, 4096, 4097, 20000]) for _ in range(rng.randint(1, 6))]
        leaves = []
        for n in sizes:
            slots = [make_input((n,), t, gen, False) for s, t in inputs if s == (1,)]
            slots.append(torch.full((n,), float("nan"), dtype=TD[dt], device=DEV))
            slots += [torch.full((n,), float("nan"), dtype=TD[xdt], device=DEV) for _, xdt in extras]
            leaves.append(slots)
        scalars = [None if s == (1,) else make_input((), t, gen, False) for s, t in inputs]
        g = P.Group(nodes, inputs, (1,), dt, root=len(nodes) - 1, tree=True,
                    extras=[(m, (1,), xdt) for m, xdt in extras])
        tree = P.Tree(leaves)
        in_slots = [k if s == (1,) else -1 for k, (s, _) in enumerate(inputs)]
        outs = [n_el + j for j in range(1 + len(extras))]
        g.run_tree(tree, in_slots, outs[0] if not extras else outs, scalars)
        torch.cuda.synchronize()
        sc_np = [None if t is None else to_np(t) for t in scalars]
        for li, (n, slots) in enumerate(zip(sizes, leaves)):
            ins = [sc_np[k] if s == () else to_np(slots[k]) for k, (s, _) in enumerate(inputs)]
            refx = [(m, np.zeros((n,), np.float32 if xdt == "f32" else np.uint16)) for m, xdt in extras]
            ref = oracle.eval_group(nodes, ins, (n,), OD[dt], root=len(nodes) - 1, extras=refx)
            what = f"chunk {chunk} trial {trial} leaf {li} (n={n}): inputs {inputs} extras {extras}"
            ok = same_bits(to_np(slots[n_el]), ref)
            assert ok.all(), f"{what}: root differs at {int((~ok).sum())} of {ok.size}"
            for j, (m, r) in enumerate(refx):
                ok = same_bits(to_np(slots[n_el + 1 + j]), r)
                assert ok.all(), f"{what}: extra {m} differs at {int((~ok).sum())} of {ok.size}"


@pytest.mark.parametrize("chunk", range(4))
def test_random_exact_row_groups_bit_for_bit(chunk):
    """Random row groups of the exact operations and row maxima (register,
    tiled and persistent row kernels, one or more reduction phases, row
    values stored at [rows, 1]): a maximum does not depend on the order the
    lanes combine in, so the GPU and the oracle agree bit for bit (bf16
    results within one ulp: a quotient by a row statistic that only bf16
    results read is the row's reciprocal times the element).  Rows where a
    maximum's operand holds a NaN (0/0 of equal values, say) are compared
    too: a row maximum over a NaN is NaN on both sides, whatever order the
    lanes combine in."""
    _row_groups(random.Random(3000 + chunk), torch.Generator().manual_seed(55 + chunk), chunk, masks=False)


@pytest.mark.parametrize("chunk", range(4))
def test_random_masked_row_groups_bit_for_bit(chunk):
    """The same with one causal or byte mask over the first input: the row
    kernels skip refused vectors (neither loaded nor computed; members
    uniform there take their one refused value), and a member stored as
    bf16 is read rounded by the members after it in either branch."""
    _row_groups(random.Random(3500 + chunk), torch.Generator().manual_seed(65 + chunk), chunk, masks=True)


def _row_groups(rng, gen, chunk, masks):
    from tests.random_groups import random_row_group
    for trial in range(10):
        nodes, inputs, shape, dt, extras = random_row_group(rng, masks=masks)
        tensors = []
        for s, t in inputs:
            x = make_input(s, t, gen, False)
            tensors.append(x if t == "u8" else torch.where(x == 0, torch.ones_like(x), x))   # no exact zeros
        g = P.Group(nodes, inputs, shape, dt, root=len(nodes) - 1, extras=extras)
        out = torch.full(shape, float("nan"), dtype=TD[dt], device=DEV)
        xs = [torch.full(xsh, float("nan"), dtype=TD[xdt], device=DEV) for _, xsh, xdt in extras]
        g.run(tensors, out, extra_outs=xs or None)
        torch.cuda.synchronize()
        refx = [(m, np.zeros(xsh, np.float32 if xdt == "f32" else np.uint16)) for m, xsh, xdt in extras]
        ins = [t.cpu().numpy().view(np.uint8) if t.dtype == torch.uint8 else to_np(t) for t in tensors]
        ref = oracle.eval_group(nodes, ins, shape, OD[dt], root=len(nodes) - 1, extras=refx)
        what = (f"chunk {chunk} trial {trial}: kind {g.info.kind} shape {shape} {dt} inputs {inputs} "
                f"extras {extras} ops {[n.op for n in nodes]}")
        for name, got, r in [("root", to_np(out), ref)] + [
                (f"extra {m}", to_np(x), r) for (m, r), x in zip(refx, xs)]:
            if got.dtype == np.uint16:
                assert_bf16_close(got, r, f"{what}: {name}")
            else:
                ok = same_bits(got, r)
                assert ok.all(), f"{what}: {name} differs at {int((~ok).sum())} of {ok.size}"


@pytest.mark.parametrize("layout,chunk", [
    ("tiled=1,lanes=128,tn=1,rc=1,lc=1", 10),          # registers, LDS and memory tiles; unrolled memory loop
    ("tiled=1,lanes=256,tn=2,rc=2,lc=2,mu=3", 11),     # an unroll that leaves a remainder
    ("tiled=1,lanes=128,tn=1,rc=0,lc=0,alt=0", 12),    # every tile from memory, every phase forwards
    ("persist=2", 13),                                 # persistent rows (next row loaded during this one)
    ("persist=3,pf=3", 15),                            # persistent rows loading three rows ahead
    ("lanes=32", 14),                                  # half-wave rows (the 32-lane join)
])
def test_random_exact_row_groups_through_other_layouts(layout, chunk, monkeypatch):
    """The same random exact row groups under other launch layouts: forced
    through the tiled wide-row kernel with small tiles (rows of a few
    hundred columns already span several tiles, the three loops over
    register, LDS and memory tiles, the walks in both directions), through
    persistent rows, and with 32-lane rows: bit for bit against the oracle,
    as above."""
    monkeypatch.setenv("PSK_LAYOUT", layout)
    test_random_exact_row_groups_bit_for_bit(chunk)
