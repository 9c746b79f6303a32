"""Runs on the caller's streams and inside HIP graphs.  Groups launched on
two side streams at once give the bits they give alone; a group run and an
AdamW step (plain and clipped with a schedule) captured in a graph after a
first run (which loads the code object) replay correctly several times, with
eager work and synchronisations between replays, each replay checked against
the same call made eagerly."""
import pytest
import torch

from synth import configs
from tests.gpu_util import assert_bits, to_np

P = pytest.importorskip("elementwise_reduction_groups_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
EPS = configs.f32(1e-5)


def test_two_side_streams():
    R, C = 4096, 1024
    x = configs.softmax_scores(R, C, device=DEV, seed=81)
    a, r, gm = configs.rmsnorm_inputs(2048, 4096, device=DEV, seed=82)
    sm = P.Group(configs.softmax_causal_dag(0.125, 1024), [((R, C), "f32")], (R, C), "f32")
    rms = P.Group(configs.rmsnorm_gelu_dag(EPS), [((2048, 4096), "bf16"), ((2048, 4096), "bf16"), ((4096,), "bf16")],
                  (2048, 4096), "bf16")
    y0, z0 = torch.empty_like(x), torch.empty_like(a)
    sm.run([x], y0)
    rms.run([a, r, gm], z0)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    y1, z1 = torch.full_like(x, float("nan")), torch.full_like(a, float("nan"))
    torch.cuda.synchronize()
    for _ in range(3):
        sm.run([x], y1, stream=s1)
        rms.run([a, r, gm], z1, stream=s2)
    torch.cuda.synchronize()
    assert_bits(to_np(y1), to_np(y0), "softmax on a side stream")
    assert_bits(to_np(z1), to_np(z0), "rmsnorm on a side stream")


def test_group_run_in_a_graph():
    R, C = 2048, 1024
    x = configs.softmax_scores(R, C, device=DEV, seed=83)
    y = torch.empty_like(x)
    g = P.Group(configs.softmax_causal_dag(0.125, 1024), [((R, C), "f32")], (R, C), "f32")
    g.run([x], y)                       # loads the code object
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g.run([x], y)
    for k in range(3):
        x.copy_(configs.softmax_scores(R, C, device=DEV, seed=84 + k))   # eager work between replays
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = torch.empty_like(x)
        g.run([x], ref)
        torch.cuda.synchronize()
        assert_bits(to_np(y), to_np(ref), f"graph replay {k}")


@pytest.mark.parametrize("clip", [False, True])
def test_adamw_step_in_a_graph(clip):
    shapes = [(1000,), (64, 65), (4097,)]
    HP = configs.ADAMW_HP
    hp = (HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"], HP["t"])
    kw = dict(total=1000, warmup=10, schedule="cosine", grad_clip=0.5) if clip else {}
    st = configs.adamw_state(shapes, theta_dtype=torch.bfloat16, grad_dtype=torch.bfloat16, mv_dtype=torch.float32,
                             device=DEV, seed=85)
    ref = [{k: v.clone() for k, v in s.items()} for s in st]
    tree = P.Tree([[s["theta"], s["grad"], s["m"], s["v"]] for s in st])
    rtree = P.Tree([[s["theta"], s["grad"], s["m"], s["v"]] for s in ref])
    tree.adamw_step(*hp, **kw)          # first run, eager, on both
    rtree.adamw_step(*hp, **kw)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        tree.adamw_step(*hp, **kw)
    for k in range(3):
        for s, q in zip(st, ref):       # new gradients, eagerly, on both
            g = (torch.randn(s["grad"].shape, device=DEV, generator=torch.Generator(DEV).manual_seed(86 + k)) * 0.01)
            s["grad"].copy_(g.to(torch.bfloat16))
            q["grad"].copy_(s["grad"])
        torch.cuda.synchronize()
        graph.replay()
        rtree.adamw_step(*hp, **kw)
        torch.cuda.synchronize()
        for i, (s, q) in enumerate(zip(st, ref)):
            for name in ("theta", "m", "v"):
                assert_bits(to_np(s[name]), to_np(q[name]), f"replay {k} leaf {i} {name} (clip={clip})")
