"""Host-threaded driver of the oracle -- TEST INFRASTRUCTURE ONLY.

Splits one oracle computation into blocks of rows (row groups), of elements
(AdamW, whose elements are independent) or of leaves, and runs the blocks
on host threads.  Each block runs the same sequential C code over its own
range, and no row, element or leaf reads another's result, so the output is
bit for bit the single-threaded one (the tests check that).  ctypes releases
the GIL for the duration of each C call, so the threads run in parallel.

Only the tests, the smoke check and the benchmark's CPU-baseline leg use
this; the product path never does.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Callable, List, Optional, Sequence, Tuple

import numpy as np

from . import adamw as _adamw
from . import eval_group as _eval_group
from . import rmsnorm_gelu as _rmsnorm_gelu
from . import softmax_causal as _softmax_causal


def host_threads(limit: int = 16) -> int:
    """Threads to use: the host's CPUs, at most `limit` (a GPU machine's share)."""
    return max(1, min(limit, os.cpu_count() or 1))


def ranges(n: int, parts: int) -> List[Tuple[int, int]]:
    """[0, n) cut into at most `parts` contiguous, nearly equal ranges."""
    parts = max(1, min(parts, n)) if n > 0 else 1
    bounds = [n * k // parts for k in range(parts + 1)]
    return [(bounds[k], bounds[k + 1]) for k in range(parts) if bounds[k] < bounds[k + 1]]


def run_blocks(fn: Callable[[int, int], None], n: int, threads: int, blocks_per_thread: int = 4):
    """fn(a, b) over blocks of [0, n); with one thread, one call over all of it."""
    if threads <= 1 or n <= 1:
        if n > 0:
            fn(0, n)
        return
    rs = ranges(n, threads * blocks_per_thread)
    with ThreadPoolExecutor(max_workers=threads) as ex:
        for f in [ex.submit(fn, a, b) for a, b in rs]:
            f.result()


def softmax_causal(x: np.ndarray, period: int, scale: float, threads: int,
                   out: Optional[np.ndarray] = None) -> np.ndarray:
    C = x.shape[-1]
    if out is None:
        out = np.zeros_like(x)
    run_blocks(lambda a, b: _softmax_causal(x, period, scale, rows=(a, b), out=out), x.size // C, threads)
    return out


def rmsnorm_gelu(x, res, gamma, eps: float, threads: int, out: Optional[np.ndarray] = None) -> np.ndarray:
    C = x.shape[-1]
    if out is None:
        out = np.zeros_like(x)
    run_blocks(lambda a, b: _rmsnorm_gelu(x, res, gamma, eps, rows=(a, b), out=out), x.size // C, threads)
    return out


def eval_group(nodes, inputs: Sequence[np.ndarray], out_shape: Sequence[int], out_dtype: int, threads: int,
               out: Optional[np.ndarray] = None, root: Optional[int] = None) -> np.ndarray:
    out_shape = tuple(int(s) for s in out_shape)
    if out is None:
        out = np.zeros(out_shape, np.float32 if out_dtype == 0 else np.uint16)
    R = int(np.prod(out_shape[:-1])) if len(out_shape) > 1 else 1
    run_blocks(lambda a, b: _eval_group(nodes, inputs, out_shape, out_dtype, rows=(a, b), out=out, root=root),
               R, threads)
    return out


def adamw_leaves(leaves: Sequence[Sequence[np.ndarray]], hp: Sequence[float], threads: int,
                 block: int = 1 << 22) -> List[Tuple[np.ndarray, np.ndarray, np.ndarray]]:
    """One AdamW step over every leaf (theta, g, m, v arrays, 1-D), out of
    place; elements are cut into blocks of at most `block` so that one large
    leaf spreads over the threads too."""
    outs = [(np.empty_like(t), np.empty_like(m), np.empty_like(v)) for t, _, m, v in leaves]
    work = []
    for k, (t, g, m, v) in enumerate(leaves):
        for a in range(0, t.size, block):
            work.append((k, a, min(t.size, a + block)))

    def one(item):
        k, a, b = item
        t, g, m, v = leaves[k]
        to, mo, vo = outs[k]
        _adamw(t[a:b], g[a:b], m[a:b], v[a:b], *hp, out=(to[a:b], mo[a:b], vo[a:b]))

    if threads <= 1:
        for item in work:
            one(item)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            for f in [ex.submit(one, item) for item in work]:
                f.result()
    return outs
