"""GPU parity of the softmax variants against the oracle, through the C ABI:
a mask read from a byte buffer (causal pattern, key padding with emptied
rows, random), and bf16 storage of scores and probabilities."""
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


def tdt(t):
    return {torch.float32: "f32", torch.bfloat16: "bf16", torch.bool: "u8", torch.uint8: "u8"}[t.dtype]


def masked(x, m, scale=0.125):
    g = P.Group(configs.softmax_masked_dag(scale), [(tuple(x.shape), tdt(x)), (tuple(m.shape), "u8")],
                tuple(x.shape), tdt(x))
    out = torch.full_like(x, float("nan"))
    g.run([x, m], out)
    torch.cuda.synchronize()
    return g, out


def mask_np(m):
    return m.cpu().numpy().view(np.uint8)


@pytest.mark.parametrize("B,H,T", [(2, 4, 256), (1, 3, 200), (2, 2, 1024), (1, 1, 77)])
def test_causal_mask_buffer_equals_causal_op(B, H, T):
    x = configs.softmax_scores(B * H * T, T, device=DEV, seed=T + B).reshape(B, H, T, T)
    m = configs.causal_mask_bytes(T, device=DEV)
    _, out = masked(x, m)
    g2 = P.Group(configs.softmax_causal_dag(0.125, T), [((B * H * T, T), "f32")], (B * H * T, T), "f32")
    out2 = torch.empty(B * H * T, T, device=DEV)
    g2.run([x.reshape(B * H * T, T)], out2)
    torch.cuda.synchronize()
    # one reduction order in both kernels: the same bits
    assert torch.equal(out.reshape(-1, T).view(torch.int32), out2.view(torch.int32))
    ref = oracle.eval_group(configs.softmax_masked_dag(0.125), [to_np(x), mask_np(m)], (B, H, T, T), F32)
    assert_f32_close(to_np(out), ref, f"causal buffer {B}x{H}x{T}")


@pytest.mark.parametrize("T", [200, 203, 1024])
def test_padding_mask_with_emptied_rows(T):
    B, H = 4, 2
    lengths = [T, T // 3, 0, 1]
    x = configs.softmax_scores(B * H * T, T, device=DEV, seed=T).reshape(B, H, T, T)
    m = configs.padding_mask(lengths, T, device=DEV)
    _, out = masked(x, m)
    got = to_np(out)
    ref = oracle.eval_group(configs.softmax_masked_dag(0.125), [to_np(x), mask_np(m)], (B, H, T, T), F32)
    assert_f32_close(got, ref, f"padding T={T}")
    assert np.all(got[2].view(np.uint32) == 0)               # the emptied batch: +0 everywhere
    assert np.all(got[1][..., T // 3:].view(np.uint32) == 0)


def test_random_mask_bf16_with_emptied_rows():
    R, C = 64, 1000
    x = configs.softmax_scores(R, C, device=DEV, seed=21).to(torch.bfloat16)
    m = configs.random_mask(R, C, 0.3, empty_rows=[0, 17, 63], device=DEV, seed=22)
    _, out = masked(x, m)
    got = to_np(out)
    ref = oracle.eval_group(configs.softmax_masked_dag(0.125), [to_np(x), mask_np(m)], (R, C), BF16)
    assert_bf16_close(got, ref, "random mask bf16")
    assert np.all(got[[0, 17, 63]] == 0)


def test_masked_full_size_sampled_rows():
    B, H, T = 8, 16, 1024
    x = configs.softmax_scores(B * H * T, T, device=DEV).reshape(B, H, T, T)
    m = configs.random_mask(T, T, 0.7, empty_rows=[5], device=DEV, seed=23)
    g, out = masked(x, m)
    rows = np.unique(np.concatenate([[0, 5, 1023, 1024 + 5, B * H * T - 1],
                                     np.random.default_rng(3).integers(0, B * H * T, 400)]))
    idx = torch.from_numpy(rows).to(DEV)
    xs = to_np(x.reshape(-1, T)[idx])
    ms = mask_np(m)[rows % T]
    ref = oracle.eval_group(configs.softmax_masked_dag(0.125), [xs, ms], (len(rows), T), F32)
    assert_f32_close(to_np(out.reshape(-1, T)[idx]), ref, "masked full size")


@pytest.mark.parametrize("R,C", [(300, 1024), (64, 4096), (33, 1000), (9, 12)])
def test_causal_softmax_bf16_storage(R, C):
    x = configs.softmax_scores(R, C, device=DEV, seed=R + C).to(torch.bfloat16)
    g = P.Group(configs.softmax_causal_dag(0.125, C), [((R, C), "bf16")], (R, C), "bf16")
    out = torch.full((R, C), float("nan"), dtype=torch.bfloat16, device=DEV)
    g.run([x], out)
    torch.cuda.synchronize()
    ref = oracle.eval_group(configs.softmax_causal_dag(0.125, C), [to_np(x)], (R, C), BF16)
    assert_bf16_close(to_np(out), ref, f"bf16 softmax {R}x{C}")
    q = np.arange(R)[:, None] % C
    assert np.all(to_np(out)[np.arange(C)[None, :] > q] == 0)


def test_causal_softmax_bf16_full_size_sampled_rows():
    R, C = 131072, 1024
    x = configs.softmax_scores(R, C, device=DEV).to(torch.bfloat16)
    g = P.Group(configs.softmax_causal_dag(0.125, 1024), [((R, C), "bf16")], (R, C), "bf16")
    out = torch.empty_like(x)
    g.run([x], out)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 1023, R - 1], np.random.default_rng(4).integers(0, R, 400)]))
    xs = to_np(x[torch.from_numpy(rows).to(DEV)])
    # row r keeps columns c <= r mod 1024: each sampled row is evaluated at
    # that position of a 1024-row block, alone (rows=(q, q + 1))
    refs = []
    block = np.zeros((1024, C), np.uint16)
    for k, r in enumerate(rows):
        q = int(r % 1024)
        block[q] = xs[k]
        refs.append(oracle.eval_group(configs.softmax_causal_dag(0.125, 1024), [block], (1024, C), BF16,
                                      rows=(q, q + 1))[q])
    assert_bf16_close(to_np(out[torch.from_numpy(rows).to(DEV)]), np.stack(refs), "bf16 softmax full size")


def test_groups_differing_only_in_where_fill():
    """Two groups that differ only in a WHERE's fill value, created and run
    in one process: each gets its own kernel and its own fill, bit for bit
    against the oracle."""
    from synth.dag import parse_dag
    x = configs.softmax_scores(64, 96, device=DEV, seed=17)
    m = configs.random_mask(64, 96, p_keep=0.5, device=DEV)
    ins = [to_np(x), mask_np(m)]
    for fill in ("-inf", "0.0", "-2.5", "inf"):
        nodes = parse_dag(f"%0 = input 0\n%1 = input 1\n%2 = where %1 %0 {fill}\n%3 = neg %2\n")
        g = P.Group(nodes, [((64, 96), "f32"), ((64, 96), "u8")], (64, 96), "f32")
        out = torch.full_like(x, float("nan"))
        g.run([x, m], out)
        torch.cuda.synchronize()
        ref = oracle.eval_group(nodes, ins, (64, 96))
        assert_bits(to_np(out), ref, f"where fill {fill}")


@pytest.mark.parametrize("mask", ["causal", "bytes"])
@pytest.mark.parametrize("online", [False, True])
def test_scaled_scores_stored_bf16_are_read_rounded(mask, online):
    """The scaled scores stored as a bf16 extra output: every member after
    them (the mask, the maximum, the exponentials) reads the rounded value,
    also where the kernel skips refused vectors and computes the allowed
    ones in a branch of their own.  f32 probabilities against the oracle,
    which evaluates the group with the same stored value."""
    R, C = 300, 1000
    x = configs.softmax_scores(R, C, device=DEV, seed=31)
    if mask == "causal":
        dag = configs.softmax_causal_dag(0.125, 256)
        ins, specs = [x], [((R, C), "f32")]
    else:
        dag = configs.softmax_masked_dag(0.125)
        m = configs.random_mask(R, C, 0.4, device=DEV, seed=32)
        ins, specs = [x, m], [((R, C), "f32"), ((R, C), "u8")]
    scaled = [i for i, n in enumerate(dag) if n.op == "mul"][0]
    g = P.Group(dag, specs, (R, C), "f32", extras=[(scaled, (R, C), "bf16")], online=online)
    out = torch.full_like(x, float("nan"))
    xs = torch.full((R, C), float("nan"), dtype=torch.bfloat16, device=DEV)
    g.run(ins, out, extra_outs=[xs])
    torch.cuda.synchronize()
    ins_np = [to_np(x)] + ([mask_np(m)] if mask == "bytes" else [])
    refx = [(scaled, np.zeros((R, C), np.uint16))]
    ref = oracle.eval_group(dag, ins_np, (R, C), F32, extras=refx)
    assert_bits(to_np(xs), refx[0][1], f"{mask} online={online}: stored scaled scores")
    assert_f32_close(to_np(out), ref, f"{mask} online={online}: probabilities")
