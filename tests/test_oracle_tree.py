"""Pins for the oracle's tree-mapped group evaluation: a group mapped over
the leaves of a parameter tree is the group applied to each leaf alone, with
rank-0 inputs shared.  Checked against numpy's IEEE f32 arithmetic and
PyTorch's bf16 rounding (the SGD step), a float64 evaluation of the formula
(a transcendental group), and the property that mapping over leaves equals
mapping over their concatenation."""
import math

import numpy as np
import torch

from synth import configs

F32, BF16 = 0, 1


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _widen(u: np.ndarray) -> np.ndarray:
    return (u.astype(np.uint32) << 16).view(np.float32)


def _leaves(sizes, seed, std=1.0):
    r = np.random.default_rng(seed)
    return [(r.standard_normal(n) * std).astype(np.float32) for n in sizes]


SIZES = [1, 3, 7, 513, 4097, 0, 12288]


def test_sgd_f32_matches_numpy_ieee(orc):
    th, g = _leaves(SIZES, 1), _leaves(SIZES, 2, 0.1)
    lr = np.float32(0.0123)
    out = orc.tree_map_group(configs.tree_sgd_dag(), [[a, b, None] for a, b in zip(th, g)],
                             [None, None, lr], F32)
    for a, b, o in zip(th, g, out):
        np.testing.assert_array_equal(o.view(np.uint32), (a - lr * b).view(np.uint32))


def test_sgd_bf16_rounds_once_like_torch(orc):
    th = [_bf16_bits(a) for a in _leaves(SIZES, 3)]
    g = [_bf16_bits(a) for a in _leaves(SIZES, 4, 0.1)]
    lr = np.float32(3e-4)
    out = orc.tree_map_group(configs.tree_sgd_dag(), [[a, b, None] for a, b in zip(th, g)],
                             [None, None, lr], BF16)
    for a, b, o in zip(th, g, out):
        # f32 arithmetic on the widened values, one rounding to bf16 at the root
        np.testing.assert_array_equal(o, _bf16_bits(_widen(a) - lr * _widen(b)))
    # a bf16 scalar is widened exactly: 0x3F00 is 0.5
    one = [np.ones(4, np.float32), np.full(4, 2.0, np.float32), None]
    np.testing.assert_array_equal(orc.tree_map_group(configs.tree_sgd_dag(), [one], [None, None, np.uint16(0x3F00)],
                                                     F32)[0], np.zeros(4, np.float32))


def test_mixed_group_against_float64_formula(orc):
    x = _leaves(SIZES, 5, 2.0)
    y = [_bf16_bits(a) for a in _leaves(SIZES, 6, 2.0)]
    s = np.float32(-0.75)
    out = orc.tree_map_group(configs.tree_mixed_dag(), [[a, b, None] for a, b in zip(x, y)], [None, None, s], F32)
    for a, b, o in zip(x, y, out):
        for xi, yi, oi in zip(a.astype(float), _widen(b).astype(float), o.astype(float)):
            t7 = math.tanh(xi) * math.exp(-abs(yi))
            t9 = 0.5 * xi * math.erfc(-xi / math.sqrt(2.0)) * float(s)
            # each f32 operation within a few ulps of its operands' scale
            assert abs(oi - (t7 + t9)) <= 1e-6 * (abs(t7) + abs(t9)) + 1e-30, (xi, yi, oi, t7 + t9)


def test_mapping_over_leaves_equals_mapping_over_their_concatenation(orc):
    th, g = _leaves(SIZES, 7), _leaves(SIZES, 8)
    lr = np.float32(0.5)
    per_leaf = orc.tree_map_group(configs.tree_sgd_dag(), [[a, b, None] for a, b in zip(th, g)],
                                  [None, None, lr], F32)
    whole = orc.tree_map_group(configs.tree_sgd_dag(), [[np.concatenate(th), np.concatenate(g), None]],
                               [None, None, lr], F32)[0]
    np.testing.assert_array_equal(np.concatenate(per_leaf), whole)
    assert [o.size for o in per_leaf] == SIZES
