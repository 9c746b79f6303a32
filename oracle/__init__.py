"""CPU oracle for fusion groups -- TEST INFRASTRUCTURE ONLY.

Loaded by the tests, the smoke check and the benchmark's CPU-baseline leg;
never by the product path.  ``oracle.c`` is the f32 reference (one IEEE
operation at a time, program order, no contraction); this module wraps it
with ctypes and adds two float64 companions used to pin it:

* ``eval_group_f64``: the same let-list evaluated op by op in numpy float64;
* ``interval_bounds``: interval arithmetic over a let-list, used to decide
  whether a randomly drawn chain is well posed.

Nothing here is shared with, or imported from, the GPU library.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared"]

F32, BF16, U8 = 0, 1, 2

# this oracle's own op numbering (mirrors the enum in oracle.c)
_OPCODE = {name: i for i, name in enumerate([
    "input", "const",
    "add", "sub", "mul", "div", "max", "min",
    "neg", "abs", "exp", "log", "sqrt", "tanh", "erf", "gelu", "sqrtabs",
    "pow2", "pown", "select", "causal_mask",
    "row_max", "row_sum", "row_mean",
    "where",
])}


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (no contraction, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _orc_node(ctypes.Structure):
    _fields_ = [("op", ctypes.c_int32), ("a", ctypes.c_int32), ("b", ctypes.c_int32),
                ("c", ctypes.c_int32), ("imm", ctypes.c_float), ("iparam", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        L = ctypes.CDLL(build())
        i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        L.orc_bf16_widen_array.argtypes = [i64, vp, vp]
        L.orc_bf16_round_array.argtypes = [i64, vp, vp]
        L.orc_eval_group.argtypes = [ctypes.c_int, ctypes.POINTER(_orc_node), ctypes.c_int, ctypes.c_int,
                                     ctypes.POINTER(vp), vp, vp, vp, ctypes.c_int, vp, ctypes.c_int, vp,
                                     i64, i64]
        L.orc_eval_group.restype = ctypes.c_int
        L.orc_eval_group_multi.argtypes = [ctypes.c_int, ctypes.POINTER(_orc_node), ctypes.c_int, ctypes.c_int,
                                           ctypes.POINTER(vp), vp, vp, vp, ctypes.c_int, vp, ctypes.c_int, vp,
                                           ctypes.c_int, vp, vp, vp, ctypes.POINTER(vp), i64, i64]
        L.orc_eval_group_multi.restype = ctypes.c_int
        L.orc_adamw_scalars.argtypes = [ctypes.c_double] * 5 + [i64, vp]
        L.orc_adamw.argtypes = [i64, ctypes.c_int, vp, ctypes.c_int, vp, ctypes.c_int, vp, vp,
                                ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                ctypes.c_double, i64, vp, vp, vp]
        L.orc_lr_schedule.argtypes = [ctypes.c_int, ctypes.c_double, i64, i64, i64]
        L.orc_lr_schedule.restype = ctypes.c_double
        L.orc_sumsq.argtypes = [i64, ctypes.c_int, vp, ctypes.POINTER(ctypes.c_double),
                                ctypes.POINTER(ctypes.c_double)]
        L.orc_sumsq.restype = None
        L.orc_clip_factor.argtypes = [ctypes.c_double, ctypes.c_double]
        L.orc_clip_factor.restype = ctypes.c_float
        L.orc_adamw_scaled.argtypes = [i64, ctypes.c_int, vp, ctypes.c_int, vp, ctypes.c_int, vp, vp,
                                       ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                       ctypes.c_double, i64, ctypes.c_float, vp, vp, vp]
        L.orc_softmax_causal.argtypes = [i64, i64, i64, ctypes.c_float, vp, vp, i64, i64]
        L.orc_rmsnorm_gelu.argtypes = [i64, i64, vp, vp, vp, ctypes.c_float, vp, i64, i64]
        L.orc_partition.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, vp, vp]
        L.orc_partition.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


# --------------------------------------------------------------------- bf16
def bf16_widen(u16: np.ndarray) -> np.ndarray:
    u16 = np.ascontiguousarray(u16, dtype=np.uint16)
    out = np.empty(u16.shape, np.float32)
    lib().orc_bf16_widen_array(u16.size, _ptr(u16), _ptr(out))
    return out


def bf16_round(f: np.ndarray) -> np.ndarray:
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, np.uint16)
    lib().orc_bf16_round_array(f.size, _ptr(f), _ptr(out))
    return out


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype in (np.uint8, np.bool_):
        return U8
    raise TypeError(f"oracle arrays are float32, uint16 (bf16 bits) or uint8/bool (a mask), got {a.dtype}")


# ------------------------------------------------------------ group evaluator
def eval_group(nodes, inputs: Sequence[np.ndarray], out_shape: Sequence[int], out_dtype: int = F32,
               rows: Optional[Tuple[int, int]] = None, out: Optional[np.ndarray] = None,
               root: Optional[int] = None, extras: Sequence[Tuple[int, np.ndarray]] = ()) -> np.ndarray:
    """Evaluate a let-list (``synth.Node`` sequence) over broadcast inputs.

    Inputs are float32 arrays or uint16 arrays holding bf16 bits.  Returns the
    output as float32 (f32) or uint16 (bf16 bits); with ``rows=(r0, r1)``
    only those rows of the [R, C] view are computed (others are left as
    they are in ``out``, zero if ``out`` is not given).

    ``extras``: (node, array) pairs, further stored values of a multi-output
    group; the array (float32 or uint16 bf16 bits) has the output's shape,
    or the output's shape with a last axis of 1 for a value that is one per
    row.  A bf16 stored value is read rounded by later nodes."""
    n = len(nodes)
    arr = (_orc_node * n)()
    for i, nd in enumerate(nodes):
        a = list(nd.args) + [-1] * (3 - len(nd.args))
        arr[i].op = _OPCODE[nd.op]
        arr[i].a, arr[i].b, arr[i].c = a[0], a[1], a[2]
        arr[i].imm = float(nd.imm) if nd.imm is not None else 0.0
        arr[i].iparam = int(nd.iparam) if nd.iparam is not None else 0
    inputs = [np.ascontiguousarray(x) for x in inputs]
    k = len(inputs)
    ptrs = (ctypes.c_void_p * max(k, 1))(*[_ptr(x) for x in inputs])
    dts = np.array([_dtype_code(x) for x in inputs] or [0], np.int32)
    ranks = np.array([x.ndim for x in inputs] or [0], np.int32)
    shapes = np.zeros((max(k, 1), 8), np.int64)
    for j, x in enumerate(inputs):
        shapes[j, :x.ndim] = x.shape
    out_shape = tuple(int(s) for s in out_shape)
    oshape = np.zeros(8, np.int64)
    oshape[:len(out_shape)] = out_shape
    C = out_shape[-1]
    R = int(np.prod(out_shape[:-1])) if len(out_shape) > 1 else 1
    if out is None:
        out = np.zeros(out_shape, np.float32 if out_dtype == F32 else np.uint16)
    r0, r1 = rows if rows is not None else (0, R)
    ne = len(extras)
    for _, a in extras:
        assert a.flags["C_CONTIGUOUS"] and a.size in (R * C, R)
    xroot = np.array([int(nd) for nd, _ in extras] or [0], np.int32)
    xdt = np.array([_dtype_code(a) for _, a in extras] or [0], np.int32)
    xrow = np.array([int(a.shape[-1] == 1 and C != 1) for _, a in extras] or [0], np.int32)
    xout = (ctypes.c_void_p * max(ne, 1))(*[_ptr(a) for _, a in extras])
    rc = lib().orc_eval_group_multi(n, arr, n - 1 if root is None else root, k, ptrs, _ptr(dts), _ptr(ranks),
                                    _ptr(shapes), len(out_shape), _ptr(oshape), out_dtype, _ptr(out),
                                    ne, _ptr(xroot), _ptr(xdt), _ptr(xrow), xout, r0, r1)
    if rc != 0:
        raise ValueError("oracle refused the node list")
    return out


# ---------------------------------------------------- tree-mapped groups
def tree_map_group(nodes, leaves: Sequence[Sequence[Optional[np.ndarray]]],
                   scalars: Sequence[Optional[np.ndarray]], out_dtype: int = F32,
                   root: Optional[int] = None) -> List[np.ndarray]:
    """A group mapped over the leaves of a parameter tree (PSK-Realize, "What
    a group is", parameter trees): each leaf's result is the group evaluated
    on that leaf alone, its rank-1 inputs taken from the leaf and its rank-0
    inputs shared by every leaf.  ``leaves[l][k]`` is input k of leaf l (1-D;
    ignored where ``scalars[k]`` is given), ``scalars[k]`` a 0-d array."""
    outs = []
    for leaf in leaves:
        ins = [np.asarray(scalars[k]) if scalars[k] is not None else leaf[k] for k in range(len(scalars))]
        n = next(x.size for k, x in enumerate(leaf) if scalars[k] is None)
        outs.append(eval_group(nodes, ins, (n,), out_dtype, root=root) if n else
                    np.zeros(0, np.float32 if out_dtype == F32 else np.uint16))
    return outs


# ----------------------------------------------------------------- AdamW
def adamw_scalars(lr, beta1, beta2, eps, weight_decay, t) -> np.ndarray:
    s = np.zeros(9, np.float32)
    lib().orc_adamw_scalars(lr, beta1, beta2, eps, weight_decay, int(t), _ptr(s))
    return s


def adamw(theta: np.ndarray, grad: np.ndarray, m: np.ndarray, v: np.ndarray,
          lr, beta1, beta2, eps, weight_decay, t, out=None):
    """One AdamW step (out of place).  Arrays are float32 or uint16 (bf16
    bits); m and v share a dtype.  Returns (theta', m', v'), written into
    ``out`` (three contiguous arrays like theta, m, v) when given."""
    theta, grad, m, v = (np.ascontiguousarray(a) for a in (theta, grad, m, v))
    assert m.dtype == v.dtype and theta.size == grad.size == m.size == v.size
    if out is None:
        to, mo, vo = np.empty_like(theta), np.empty_like(m), np.empty_like(v)
    else:
        to, mo, vo = out
        assert to.dtype == theta.dtype and mo.dtype == vo.dtype == m.dtype and to.size == mo.size == vo.size == m.size
    lib().orc_adamw(theta.size, _dtype_code(theta), _ptr(theta), _dtype_code(grad), _ptr(grad),
                    _dtype_code(m), _ptr(m), _ptr(v), lr, beta1, beta2, eps, weight_decay, int(t),
                    _ptr(to), _ptr(mo), _ptr(vo))
    return to, mo, vo


SCHEDULES = {"constant": 0, "linear": 1, "cosine": 2}


def lr_schedule(kind: str, lr: float, t: int, total: int = 0, warmup: int = 0) -> float:
    return lib().orc_lr_schedule(SCHEDULES[kind], lr, int(t), int(total), int(warmup))


def tree_sumsq(grads: Sequence[np.ndarray]) -> float:
    """Squared global norm of a gradient tree: squares exact in f64, summed
    with compensation (exact to about one f64 rounding)."""
    s, c = ctypes.c_double(0.0), ctypes.c_double(0.0)
    for g in grads:
        g = np.ascontiguousarray(g)
        lib().orc_sumsq(g.size, _dtype_code(g), _ptr(g), ctypes.byref(s), ctypes.byref(c))
    return s.value + c.value


def clip_factor(sumsq: float, c: float) -> np.float32:
    return np.float32(lib().orc_clip_factor(sumsq, c))


def adamw_scaled(theta, grad, m, v, lr, beta1, beta2, eps, weight_decay, t, gscale):
    """AdamW with the gradient scaled by the f32 factor gscale first; lr is
    the schedule's value at t."""
    theta, grad, m, v = (np.ascontiguousarray(a) for a in (theta, grad, m, v))
    to, mo, vo = np.empty_like(theta), np.empty_like(m), np.empty_like(v)
    lib().orc_adamw_scaled(theta.size, _dtype_code(theta), _ptr(theta), _dtype_code(grad), _ptr(grad),
                           _dtype_code(m), _ptr(m), _ptr(v), lr, beta1, beta2, eps, weight_decay, int(t),
                           float(gscale), _ptr(to), _ptr(mo), _ptr(vo))
    return to, mo, vo


# ------------------------------------------------------------- row groups
def softmax_causal(x: np.ndarray, period: int, scale: float, rows=None, out=None) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    C = x.shape[-1]
    if out is None:
        out = np.zeros_like(x)
    if C == 0:
        return out
    R = x.size // C
    r0, r1 = rows if rows is not None else (0, R)
    lib().orc_softmax_causal(R, C, period, scale, _ptr(x), _ptr(out), r0, r1)
    return out


def rmsnorm_gelu(x: np.ndarray, res: np.ndarray, gamma: np.ndarray, eps: float, rows=None, out=None) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.uint16)
    res = np.ascontiguousarray(res, dtype=np.uint16)
    gamma = np.ascontiguousarray(gamma, dtype=np.uint16)
    C = x.shape[-1]
    R = x.size // C
    assert gamma.size == C and res.shape == x.shape
    if out is None:
        out = np.zeros_like(x)
    r0, r1 = rows if rows is not None else (0, R)
    lib().orc_rmsnorm_gelu(R, C, _ptr(x), _ptr(res), _ptr(gamma), eps, _ptr(out), r0, r1)
    return out


# -------------------------------------------------------------- partition
_CLASS = {"leaf": 0, "ew": 1, "row": 2, "nonew": 2}


def partition(nodes, types, is_output: Sequence[bool], cap: int = 64, rows: bool = False):
    """Greedy fusion-group partition; returns (group_of, is_root) as int32
    arrays.  ``types[i]`` is node i's (shape, storage type) or an integer
    type id (then rows must be False).  ``pown`` with an exponent above 2 is
    a boundary; with ``rows`` last-axis row reductions fuse."""
    from synth.dag import OPS
    n = len(nodes)
    cls = np.zeros(n, np.int32)
    args = np.full((n, 3), -1, np.int32)
    for i, nd in enumerate(nodes):
        c = _CLASS[OPS[nd.op][1]]
        if nd.op == "pown" and (nd.iparam or 0) > 2:
            c = 2
        if rows and OPS[nd.op][1] == "row":
            c = 3
        cls[i] = c
        a = list(nd.args)[:3]
        args[i, :len(a)] = a
    ids, shape_ids = {}, {}
    tid = np.zeros(n, np.int32)
    sid = np.zeros(n, np.int32)
    rsid = np.full(n, -1, np.int32)
    for i, t in enumerate(types):
        if isinstance(t, (int, np.integer)):
            assert not rows, "row fusion needs shapes"
            tid[i] = int(t)
            continue
        shape, dt = tuple(int(x) for x in t[0]), str(t[1])
        tid[i] = ids.setdefault((shape, dt), len(ids))
        sid[i] = shape_ids.setdefault(shape, len(shape_ids))
        if shape and shape[-1] > 1:
            rsid[i] = shape_ids.setdefault(shape[:-1] + (1,), len(shape_ids))
    outp = np.ascontiguousarray([1 if o else 0 for o in is_output], np.uint8)
    g = np.zeros(n, np.int32)
    r = np.zeros(n, np.int32)
    rc = lib().orc_partition(n, _ptr(cls), _ptr(args), _ptr(tid), _ptr(sid), _ptr(rsid), _ptr(outp), cap,
                             1 if rows else 0, _ptr(g), _ptr(r))
    if rc < 0:
        raise ValueError("oracle refused the node list")
    return g, r


# ------------------------------------------------- float64 companion (numpy)
def _erf64(x):
    from scipy.special import erf
    return erf(x)


def _gelu64(x):
    # x * Phi(x) with Phi written through erfc, accurate in the negative tail
    from scipy.special import erfc
    return 0.5 * x * erfc(-x / math.sqrt(2.0))


def eval_group_f64(nodes, inputs: Sequence[np.ndarray], out_shape: Sequence[int], root: Optional[int] = None,
                   row_offset: int = 0) -> np.ndarray:
    """The same let-list evaluated op by op in float64 with numpy, whole
    tensors at a time (reductions over the last axis, keepdim).  bf16 inputs
    (uint16) are widened exactly.  ``row_offset`` is the global index of the
    first row (it only matters for a causal mask)."""
    out_shape = tuple(int(s) for s in out_shape)
    C = out_shape[-1]
    R = int(np.prod(out_shape[:-1])) if len(out_shape) > 1 else 1
    vals = []
    rows = (np.arange(R, dtype=np.int64) + row_offset)[:, None]
    cols = np.arange(C, dtype=np.int64)[None, :]
    for nd in nodes:
        a = [vals[i] for i in nd.args]
        op = nd.op
        if op == "input":
            x = inputs[nd.iparam]
            x = bf16_widen(x) if x.dtype == np.uint16 else x
            v = np.broadcast_to(x.astype(np.float64), out_shape).reshape(R, C)
        elif op == "const":
            v = np.full((R, C), float(nd.imm))
        elif op == "add": v = a[0] + a[1]
        elif op == "sub": v = a[0] - a[1]
        elif op == "mul": v = a[0] * a[1]
        elif op == "div": v = a[0] / a[1]
        elif op == "max": v = np.where(a[0] > a[1], a[0], a[1])
        elif op == "min": v = np.where(a[0] < a[1], a[0], a[1])
        elif op == "neg": v = -a[0]
        elif op == "abs": v = np.abs(a[0])
        elif op == "exp": v = np.exp(a[0])
        elif op == "log": v = np.log(a[0])
        elif op == "sqrt": v = np.sqrt(a[0])
        elif op == "tanh": v = np.tanh(a[0])
        elif op == "erf": v = _erf64(a[0])
        elif op == "gelu": v = _gelu64(a[0])
        elif op == "sqrtabs": v = np.sqrt(np.abs(a[0]))
        elif op == "pow2": v = a[0] * a[0]
        elif op == "pown": v = a[0] ** int(nd.iparam)
        elif op == "select": v = np.where(a[0] != 0, a[1], a[2])
        elif op == "causal_mask":
            v = np.where(cols <= rows % int(nd.iparam), a[0], -np.inf)
        elif op == "row_max": v = np.broadcast_to(a[0].max(axis=1, keepdims=True), (R, C))
        elif op == "row_sum": v = np.broadcast_to(a[0].sum(axis=1, keepdims=True), (R, C))
        elif op == "row_mean": v = np.broadcast_to(a[0].sum(axis=1, keepdims=True) / C, (R, C))
        else:
            raise ValueError(op)
        vals.append(v)
    return np.asarray(vals[len(nodes) - 1 if root is None else root]).reshape(out_shape)


# ---------------------------------------------------------- interval bounds
def _mono(f, lo, hi):
    return f(lo), f(hi)


def interval_bounds(nodes, input_bounds: Sequence[Tuple[float, float]]) -> List[Tuple[float, float]]:
    """Interval enclosure of every node's value for inputs within the given
    bounds (pointwise ops only), in float64.  Used to reject a random chain
    whose values could overflow."""
    out: List[Tuple[float, float]] = []

    def gelu64(x):
        return 0.5 * x * (1.0 + math.erf(x / math.sqrt(2.0)))
    for nd in nodes:
        a = [out[i] for i in nd.args]
        op = nd.op
        if op == "input":
            iv = tuple(input_bounds[nd.iparam])
        elif op == "const":
            iv = (float(nd.imm), float(nd.imm))
        elif op == "add":
            iv = (a[0][0] + a[1][0], a[0][1] + a[1][1])
        elif op == "sub":
            iv = (a[0][0] - a[1][1], a[0][1] - a[1][0])
        elif op == "mul":
            p = [x * y for x in a[0] for y in a[1]]
            iv = (min(p), max(p))
        elif op in ("exp", "tanh", "erf"):
            f = {"exp": lambda x: math.exp(min(x, 700.0)), "tanh": math.tanh, "erf": math.erf}[op]
            iv = _mono(f, *a[0])
        elif op == "neg":
            iv = (-a[0][1], -a[0][0])
        elif op in ("abs", "sqrtabs", "pow2"):
            lo, hi = a[0]
            m_lo = 0.0 if lo <= 0.0 <= hi else min(abs(lo), abs(hi))
            m_hi = max(abs(lo), abs(hi))
            if op == "abs":
                iv = (m_lo, m_hi)
            elif op == "sqrtabs":
                iv = (math.sqrt(m_lo), math.sqrt(m_hi))
            else:
                iv = (m_lo * m_lo, m_hi * m_hi)
        elif op == "gelu":
            # gelu has its minimum at x0 ~ -0.7518 and is monotone on each side
            lo, hi = a[0]
            x0 = -0.7517915246935835
            cands = [gelu64(lo), gelu64(hi)]
            if lo <= x0 <= hi:
                cands.append(gelu64(x0))
            iv = (min(cands), max(cands))
        else:
            raise ValueError(f"no interval rule for {op}")
        out.append((float(iv[0]), float(iv[1])))
    return out
