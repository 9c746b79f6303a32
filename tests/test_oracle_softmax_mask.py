"""Pins for the masked softmax (a mask read from a byte buffer): with the
causal pattern it is the causal softmax bit for bit; on rows the mask does
not empty it is PyTorch's softmax of the masked scores; a row the mask
empties gives zeros (presk language reference, "Typing", builtins:
softmax(..., where = m); presk manual, "Native execution")."""
import numpy as np
import torch

from synth import configs

F32, BF16 = 0, 1


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def test_causal_buffer_equals_causal_op(orc):
    B, H, T = 2, 3, 64
    x = configs.softmax_scores(B * H * T, T, seed=11)
    m = configs.causal_mask_bytes(T).numpy().view(np.uint8)
    a = orc.eval_group(configs.softmax_masked_dag(0.125), [x.numpy().reshape(B, H, T, T), m], (B, H, T, T), F32)
    b = orc.eval_group(configs.softmax_causal_dag(0.125, T), [x.numpy()], (B * H * T, T), F32)
    np.testing.assert_array_equal(a.reshape(B * H * T, T).view(np.uint32), b.view(np.uint32))


def test_padding_mask_against_torch_and_empty_rows(orc):
    B, H, T = 3, 2, 40
    lengths = [40, 17, 0]
    x = configs.softmax_scores(B * H * T, T, seed=12).reshape(B, H, T, T)
    m = configs.padding_mask(lengths, T)
    out = orc.eval_group(configs.softmax_masked_dag(0.125), [x.numpy(), m.numpy().view(np.uint8)], (B, H, T, T), F32)
    ref = torch.softmax((x.double() * 0.125).masked_fill(~m, float("-inf")), dim=-1)
    for b, n in enumerate(lengths):
        if n == 0:
            assert np.all(out[b].view(np.uint32) == 0)        # emptied rows: +0 everywhere
            continue
        got = torch.from_numpy(out[b]).double()
        assert torch.all((got - ref[b]).abs() <= 1e-7 + 2e-6 * ref[b].abs())
        assert np.all(out[b][..., n:].view(np.uint32) == 0)   # refused: +0
        np.testing.assert_allclose(out[b].sum(-1), 1.0, rtol=2e-6 * T)


def test_random_mask_bf16_storage(orc):
    R, C = 50, 96
    x = configs.softmax_scores(R, C, seed=13).to(torch.bfloat16)
    m = configs.random_mask(R, C, 0.3, empty_rows=[4, 31], seed=14)
    out = orc.eval_group(configs.softmax_masked_dag(0.125), [_bits(x), m.numpy().view(np.uint8)], (R, C), BF16)
    ref = torch.softmax((x.double() * 0.125).masked_fill(~m, float("-inf")), dim=-1).float().to(torch.bfloat16)
    keep = m.any(dim=1)
    d = np.abs(out.astype(np.int32) - _bits(ref).astype(np.int32))
    assert d[keep.numpy()].max() <= 1                         # one bf16 rounding of an f32 value
    assert np.all(out[~keep.numpy()] == 0)
    assert np.all(out[~m.numpy()] == 0)
