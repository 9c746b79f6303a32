"""psk_adamw_step_config_noalloc (the clipped AdamW step whose clipping pass
keeps its scratch in the library's static device array) against
psk_adamw_step_config, through the C ABI, bit for bit: two calls in a row,
the second on a smaller tree, so the second reuses the array the first left
behind."""
import numpy as np
import pytest
import torch

from synth import configs
from tests.gpu_util import assert_bits, to_np

P = pytest.importorskip("elementwise_reduction_groups_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
HP = configs.ADAMW_HP
CFG = dict(total=200, warmup=20, schedule="cosine", grad_clip=0.05)


def _pair(shapes, seed):
    a = configs.adamw_state(shapes, theta_dtype=torch.bfloat16, grad_dtype=torch.bfloat16, mv_dtype=torch.float32,
                            device=DEV, seed=seed)
    b = [{k: t.clone() for k, t in s.items()} for s in a]
    return a, b


def test_noalloc_step_equals_config_step_twice():
    big = [(1000, 777), (4096,), (33, 65), (2048, 2048), (5,)]          # 3.2M elements, ragged leaves
    small = [(300, 7), (129,)]
    for call, (shapes, seed) in enumerate([(big, 61), (small, 62)]):
        ref_state, got_state = _pair(shapes, seed)
        ref_tree = P.Tree([[s["theta"], s["grad"], s["m"], s["v"]] for s in ref_state])
        got_tree = P.Tree([[s["theta"], s["grad"], s["m"], s["v"]] for s in got_state])
        args = (HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"], 37)
        ref_tree.adamw_step(*args, **CFG)
        got_tree.adamw_step_noalloc(*args, **CFG)
        torch.cuda.synchronize()
        _, factor = ref_tree.clip_result()
        assert 0.0 < factor < 1.0, f"call {call}: the clipping is active (factor {factor})"
        for leaf, (r, g) in enumerate(zip(ref_state, got_state)):
            for k in ("theta", "m", "v"):
                assert_bits(to_np(g[k]), to_np(r[k]), f"call {call} leaf {leaf} {k}")
            assert_bits(to_np(g["grad"]), to_np(r["grad"]), f"call {call} leaf {leaf} grad unchanged")


def test_noalloc_without_clipping_equals_config_step():
    ref_state, got_state = _pair([(513, 9), (64,)], 63)
    ref_tree = P.Tree([[s["theta"], s["grad"], s["m"], s["v"]] for s in ref_state])
    got_tree = P.Tree([[s["theta"], s["grad"], s["m"], s["v"]] for s in got_state])
    args = (HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"], 5)
    ref_tree.adamw_step(*args, schedule="linear", total=50, warmup=10)
    got_tree.adamw_step_noalloc(*args, schedule="linear", total=50, warmup=10)
    torch.cuda.synchronize()
    for leaf, (r, g) in enumerate(zip(ref_state, got_state)):
        for k in ("theta", "m", "v"):
            assert_bits(to_np(g[k]), to_np(r[k]), f"leaf {leaf} {k}")
