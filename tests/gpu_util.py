"""Helpers shared by the GPU parity tests: device tensors to oracle arrays and
the comparison rules.

Comparison rules (what a parity test asserts):
  * integer / index results and exact special cases: bit for bit;
  * f32 results: |gpu - ref| <= 1e-7 + 2e-6 |ref|, non-finite values of the
    same class;
  * bf16 results: at most 1 bf16 ulp apart (ordered 16-bit distance, +0 == -0).
"""
import numpy as np
import torch

TOL_REL, TOL_ABS = 2e-6, 1e-7


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def f32_close_mask(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    g = got.astype(np.float64)
    r = ref.astype(np.float64)
    fin = np.isfinite(r)
    ok = np.zeros(r.shape, bool)
    ok[fin] = np.abs(g[fin] - r[fin]) <= TOL_ABS + TOL_REL * np.abs(r[fin])
    nan = np.isnan(r)
    ok[nan] = np.isnan(g[nan])
    inf = np.isinf(r)
    ok[inf] = g[inf] == r[inf]
    return ok


def assert_f32_close(got, ref, what=""):
    ok = f32_close_mask(got, ref)
    if not ok.all():
        i = np.argwhere(~ok)[0]
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outside 1e-7 + 2e-6|ref|; first at "
                             f"{tuple(i)}: gpu {got[tuple(i)]!r} ref {ref[tuple(i)]!r}")


def bf16_ulps(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    def ordered(u):
        s = u.astype(np.int32)
        mag = s & 0x7FFF
        return np.where(s & 0x8000, -mag, mag)
    return np.abs(ordered(a) - ordered(b))


def assert_bf16_close(got, ref, what=""):
    gnan = (got & 0x7F80) == 0x7F80
    gnan &= (got & 0x7F) != 0
    rnan = ((ref & 0x7F80) == 0x7F80) & ((ref & 0x7F) != 0)
    assert np.array_equal(gnan, rnan), f"{what}: NaN positions differ"
    d = bf16_ulps(got[~rnan], ref[~rnan])
    if d.size and d.max() > 1:
        raise AssertionError(f"{what}: {int((d > 1).sum())} of {d.size} more than 1 bf16 ulp apart (max {d.max()})")


def assert_bits(got, ref, what=""):
    gb = got.view(np.uint32) if got.dtype == np.float32 else got
    rb = ref.view(np.uint32) if ref.dtype == np.float32 else ref
    if not np.array_equal(gb, rb):
        bad = int((gb != rb).sum())
        i = np.argwhere(gb != rb)[0]
        raise AssertionError(f"{what}: {bad} of {gb.size} elements differ in bits; first at {tuple(i)}: "
                             f"gpu {got[tuple(i)]!r} ref {ref[tuple(i)]!r}")


def compare_all(got: np.ndarray, ref: np.ndarray, rule: str, what: str = "", chunk: int = 1 << 24) -> int:
    """Compare every element of two large arrays chunk by chunk under one of
    the rules above ("f32", "bf16" or "bits"); raises on the first chunk
    with a mismatch and returns the number of elements compared."""
    g, r = got.reshape(-1), ref.reshape(-1)
    assert g.size == r.size and g.dtype == r.dtype, f"{what}: {g.shape} {g.dtype} vs {r.shape} {r.dtype}"
    check = {"f32": assert_f32_close, "bf16": assert_bf16_close, "bits": assert_bits}[rule]
    n = 0
    for a in range(0, g.size, chunk):
        b = min(g.size, a + chunk)
        check(g[a:b], r[a:b], f"{what} (elements {a}..{b})")
        n += b - a
    return n
