"""Python binding of psk_fused (libpsk_fused.so): argument marshalling only.

Every function keeps its C name (include/psk_fused.h) and raises PskError
instead of returning a status.  Device memory and streams come from PyTorch
(``tensor.data_ptr()``, ``torch.cuda.current_stream().cuda_stream``); all
computation happens in the library's HIP kernels.  There is no fallback: if
the library is not built, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpsk_fused.so")

# ----------------------------------------------------------------- constants
PSK_OK = 0
STATUS_NAMES = ["PSK_OK", "PSK_E_NULL", "PSK_E_CAP", "PSK_E_ORDER", "PSK_E_ROOT", "PSK_E_DEAD", "PSK_E_OP",
                "PSK_E_TYPE", "PSK_E_BROADCAST", "PSK_E_ROW", "PSK_E_ALIGN", "PSK_E_ALIAS", "PSK_E_SHAPE",
                "PSK_E_UNSUPPORTED", "PSK_E_JIT", "PSK_E_HIP"]
for _i, _n in enumerate(STATUS_NAMES):
    globals()[_n] = _i

PSK_F32, PSK_BF16, PSK_U8 = 0, 1, 2
PSK_GROUP_TREE = 1
PSK_GROUP_ONLINE = 2
PSK_PARTITION_ROWS = 1
PSK_MAX_RANK = 4
PSK_VERSION = 200            # the C ABI this binding marshals (psk_tensor_desc with strides)
PSK_MAX_SLOTS = 8
PSK_TREE_CHUNK = 4096

OPCODES = {
    "input": 1, "const": 2,
    "add": 10, "sub": 11, "mul": 12, "div": 13, "max": 14, "min": 15,
    "neg": 20, "abs": 21, "exp": 22, "log": 23, "sqrt": 24, "tanh": 25, "erf": 26, "gelu": 27,
    "sqrtabs": 28, "pow2": 29, "pown": 30,
    "select": 40, "causal_mask": 41, "where": 42,
    "row_max": 50, "row_sum": 51, "row_mean": 52,
    "reduce": 60, "contract": 61, "matmul": 61, "cast": 62, "opaque": 63,
}


class PskError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status
        self.name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)


# ------------------------------------------------------------------- structs
class psk_node(ctypes.Structure):
    _fields_ = [("op", ctypes.c_int32), ("a", ctypes.c_int32), ("b", ctypes.c_int32), ("c", ctypes.c_int32),
                ("imm", ctypes.c_float), ("iparam", ctypes.c_int32)]


class psk_tensor_desc(ctypes.Structure):
    _fields_ = [("rank", ctypes.c_int32), ("dtype", ctypes.c_int32), ("shape", ctypes.c_int64 * PSK_MAX_RANK),
                ("stride", ctypes.c_int64 * PSK_MAX_RANK)]


class psk_group_desc(ctypes.Structure):
    _fields_ = [("n_nodes", ctypes.c_int32), ("nodes", ctypes.POINTER(psk_node)), ("root", ctypes.c_int32),
                ("n_inputs", ctypes.c_int32), ("inputs", ctypes.POINTER(psk_tensor_desc)),
                ("out", psk_tensor_desc), ("arith", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("n_extra", ctypes.c_int32), ("extra_root", ctypes.POINTER(ctypes.c_int32)),
                ("extra_out", ctypes.POINTER(psk_tensor_desc))]


class psk_dispatch_report(ctypes.Structure):
    _fields_ = [("lets", ctypes.c_int32), ("launches_unfused", ctypes.c_int32), ("launches_fused", ctypes.c_int32),
                ("fused_groups", ctypes.c_int32), ("bytes_unfused", ctypes.c_int64), ("bytes_fused", ctypes.c_int64)]


class psk_group_info(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("members", ctypes.c_int32), ("n_reductions", ctypes.c_int32),
                ("phases", ctypes.c_int32), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("lanes_per_row", ctypes.c_int32), ("vec", ctypes.c_int32), ("block", ctypes.c_int32),
                ("rows_per_block", ctypes.c_int32), ("algorithmic_bytes", ctypes.c_int64),
                ("kernel", ctypes.c_char * 48), ("tiles", ctypes.c_int32), ("split", ctypes.c_int32)]


class psk_leaf(ctypes.Structure):
    _fields_ = [("numel", ctypes.c_int64), ("slot", ctypes.c_void_p * PSK_MAX_SLOTS)]


class psk_tree_info(ctypes.Structure):
    _fields_ = [("n_leaves", ctypes.c_int32), ("n_slots", ctypes.c_int32), ("n_chunks", ctypes.c_int64),
                ("total_numel", ctypes.c_int64), ("chunk_elems", ctypes.c_int64),
                ("vector_leaves", ctypes.c_int32)]


class psk_adamw_hp(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double), ("t", ctypes.c_int64)]


class psk_adamw_config(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double), ("t", ctypes.c_int64),
                ("total", ctypes.c_int64), ("warmup", ctypes.c_int64), ("schedule", ctypes.c_int32),
                ("grad_clip", ctypes.c_double)]


PSK_SCHED = {"constant": 0, "linear": 1, "cosine": 2}


class psk_stats(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int64), ("jit_compiles", ctypes.c_int64), ("jit_hits", ctypes.c_int64)]


# ---------------------------------------------------------------- loading
_lib = None

EXPORTED = ["psk_group_create", "psk_group_run", "psk_group_destroy", "psk_group_get_info", "psk_group_source",
            "psk_group_code_object", "psk_tree_create", "psk_tree_destroy", "psk_tree_get_info",
            "psk_tree_get_tables", "psk_tree_plan", "psk_adamw_step", "psk_adamw_step_config",
            "psk_adamw_step_config_noalloc", "psk_adamw_lr",
            "psk_tree_clip_result", "psk_group_run_tree", "psk_group_run_multi", "psk_group_run_tree_multi",
            "psk_partition", "psk_partition_ex", "psk_dispatch_count", "psk_last_error",
            "psk_status_str", "psk_version", "psk_get_stats", "psk_group_check"]


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(LIB_PATH)
    if L.psk_version() != PSK_VERSION:
        raise RuntimeError(f"{LIB_PATH} is version {L.psk_version()}, this binding {PSK_VERSION}: rebuild it")
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.psk_group_create.argtypes = [ctypes.POINTER(psk_group_desc), ctypes.POINTER(vp)]
    L.psk_group_run.argtypes = [vp, ctypes.POINTER(vp), vp, vp]
    L.psk_group_destroy.argtypes = [vp]
    L.psk_group_destroy.restype = None
    L.psk_group_check.argtypes = [vp]
    L.psk_group_get_info.argtypes = [vp, ctypes.POINTER(psk_group_info)]
    L.psk_group_source.argtypes = [ctypes.POINTER(psk_group_desc), ctypes.c_char_p, sz, ctypes.POINTER(sz)]
    L.psk_group_code_object.argtypes = [ctypes.POINTER(psk_group_desc), vp, sz, ctypes.POINTER(sz)]
    L.psk_tree_create.argtypes = [ctypes.POINTER(psk_leaf), i32, i32, ctypes.POINTER(i32), ctypes.POINTER(vp)]
    L.psk_tree_destroy.argtypes = [vp]
    L.psk_tree_destroy.restype = None
    L.psk_tree_get_info.argtypes = [vp, ctypes.POINTER(psk_tree_info)]
    L.psk_tree_get_tables.argtypes = [vp, vp, vp, vp, vp]
    L.psk_tree_plan.argtypes = [vp, i32, ctypes.POINTER(i64), vp, vp, vp, vp]
    L.psk_adamw_step.argtypes = [vp, ctypes.POINTER(psk_adamw_hp), vp]
    L.psk_adamw_step_config.argtypes = [vp, ctypes.POINTER(psk_adamw_config), vp]
    L.psk_adamw_step_config_noalloc.argtypes = [vp, ctypes.POINTER(psk_adamw_config), vp]
    L.psk_adamw_lr.argtypes = [ctypes.POINTER(psk_adamw_config), ctypes.POINTER(ctypes.c_double)]
    L.psk_tree_clip_result.argtypes = [vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_float)]
    L.psk_group_run_tree.argtypes = [vp, vp, ctypes.POINTER(i32), i32, ctypes.POINTER(vp), vp]
    L.psk_group_run_multi.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), vp]
    L.psk_group_run_tree_multi.argtypes = [vp, vp, ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(vp), vp]
    L.psk_partition.argtypes = [i32, ctypes.POINTER(psk_node), ctypes.POINTER(psk_tensor_desc),
                                ctypes.POINTER(ctypes.c_uint8), ctypes.POINTER(i32), ctypes.POINTER(i32),
                                ctypes.POINTER(i32)]
    L.psk_partition_ex.argtypes = [i32, ctypes.POINTER(psk_node), ctypes.POINTER(psk_tensor_desc),
                                   ctypes.POINTER(ctypes.c_uint8), ctypes.c_uint32, ctypes.POINTER(i32),
                                   ctypes.POINTER(i32), ctypes.POINTER(i32)]
    L.psk_dispatch_count.argtypes = [i32, ctypes.POINTER(psk_node), ctypes.POINTER(psk_tensor_desc),
                                     ctypes.POINTER(ctypes.c_uint8), ctypes.c_uint32, ctypes.POINTER(psk_dispatch_report)]
    L.psk_last_error.restype = ctypes.c_char_p
    L.psk_status_str.restype = ctypes.c_char_p
    L.psk_status_str.argtypes = [ctypes.c_int]
    L.psk_version.restype = i32
    L.psk_get_stats.argtypes = [ctypes.POINTER(psk_stats)]
    for name in EXPORTED:
        f = getattr(L, name)
        if name not in ("psk_group_destroy", "psk_tree_destroy", "psk_last_error", "psk_status_str", "psk_version"):
            f.restype = ctypes.c_int
    _lib = L
    return L


def _check(status: int):
    if status != PSK_OK:
        msg = lib().psk_last_error().decode(errors="replace")
        raise PskError(status, msg or STATUS_NAMES[status])


# ------------------------------------------------------- descriptor helpers
def _dtype_code(dt) -> int:
    if isinstance(dt, int):
        return dt
    s = str(dt)
    if s in ("f32", "float32", "torch.float32"):
        return PSK_F32
    if s in ("bf16", "bfloat16", "torch.bfloat16"):
        return PSK_BF16
    if s in ("u8", "uint8", "bool", "torch.uint8", "torch.bool"):
        return PSK_U8
    raise ValueError(f"unsupported storage type {dt!r}")


def tensor_desc(shape: Sequence[int], dtype, strides: Optional[Sequence[int]] = None) -> psk_tensor_desc:
    """strides: each axis's step in elements (None: dense row-major); a
    stride of 0 broadcasts that axis."""
    d = psk_tensor_desc()
    shape = tuple(int(s) for s in shape)
    if len(shape) > PSK_MAX_RANK:
        raise ValueError("rank above 4")
    if strides is not None:
        strides = tuple(int(x) for x in strides)
        if len(strides) != len(shape):
            raise ValueError("one stride per axis")
        if any(x < 0 for x in strides):
            raise ValueError("negative strides are not supported")
        # all-zero strides mean dense to the library: a view expanded from one
        # element along every axis is one value, described by sizes of 1
        if not any(strides) and any(n > 1 for n in shape):
            raise ValueError("a tensor expanded from one element: give it with shape of 1s")
        for i, x in enumerate(strides):
            d.stride[i] = x
    d.rank = len(shape)
    d.dtype = _dtype_code(dtype)
    for i, s in enumerate(shape):
        d.shape[i] = s
    return d


def node_array(nodes) -> ctypes.Array:
    """Nodes are objects with .op (name or code), .args, .imm, .iparam."""
    arr = (psk_node * len(nodes))()
    for i, nd in enumerate(nodes):
        op = nd.op if isinstance(nd.op, int) else OPCODES[nd.op]
        args = list(nd.args) + [-1] * (3 - len(nd.args))
        arr[i].op = op
        arr[i].a, arr[i].b, arr[i].c = args[0], args[1], args[2]
        arr[i].imm = float(nd.imm) if nd.imm is not None else 0.0
        arr[i].iparam = int(nd.iparam) if nd.iparam is not None else 0
    return arr


class GroupDesc:
    """Keeps a psk_group_desc and the arrays it points to alive."""

    def __init__(self, nodes, inputs: Sequence[Tuple[Sequence[int], object]], out_shape: Sequence[int], out_dtype,
                 root: Optional[int] = None, arith=PSK_F32, flags: int = 0,
                 extras: Sequence[Tuple[int, Sequence[int], object]] = ()):
        """inputs: (shape, storage type) of each dense input, or (shape,
        storage type, strides) of a strided one; extras: (node index, shape,
        storage type) of each further stored value."""
        self._nodes = node_array(nodes)
        self._inputs = (psk_tensor_desc * max(1, len(inputs)))(*[tensor_desc(*spec) for spec in inputs])
        self.desc = psk_group_desc()
        self.desc.n_nodes = len(nodes)
        self.desc.nodes = self._nodes
        self.desc.root = len(nodes) - 1 if root is None else root
        self.desc.n_inputs = len(inputs)
        self.desc.inputs = self._inputs
        self.desc.out = tensor_desc(out_shape, out_dtype)
        self.desc.arith = _dtype_code(arith)
        self.desc.flags = flags
        self._extra_root = (ctypes.c_int32 * max(1, len(extras)))(*[int(n) for n, _, _ in extras])
        self._extra_out = (psk_tensor_desc * max(1, len(extras)))(*[tensor_desc(sh, d) for _, sh, d in extras])
        self.desc.n_extra = len(extras)
        self.desc.extra_root = self._extra_root
        self.desc.extra_out = self._extra_out


# ------------------------------------------------------------ C functions
def psk_group_create(desc: GroupDesc) -> int:
    h = ctypes.c_void_p()
    _check(lib().psk_group_create(ctypes.byref(desc.desc), ctypes.byref(h)))
    return h.value


def psk_group_run(group: int, inputs: Sequence[int], out: int, stream: Optional[int] = None):
    """inputs/out are device addresses (ints)."""
    arr = (ctypes.c_void_p * max(1, len(inputs)))(*[ctypes.c_void_p(p) for p in inputs])
    _check(lib().psk_group_run(ctypes.c_void_p(group), arr, ctypes.c_void_p(out), ctypes.c_void_p(stream or 0)))


def psk_group_run_multi(group: int, inputs: Sequence[int], outs: Sequence[int], stream: Optional[int] = None):
    """outs[0]: the root's output, outs[1 + k]: extra output k (device addresses)."""
    arr = (ctypes.c_void_p * max(1, len(inputs)))(*[ctypes.c_void_p(p) for p in inputs])
    oa = (ctypes.c_void_p * len(outs))(*[ctypes.c_void_p(p) for p in outs])
    _check(lib().psk_group_run_multi(ctypes.c_void_p(group), arr, oa, ctypes.c_void_p(stream or 0)))


def psk_group_check(group: int):
    """Raises PskError (PSK_E_HIP) when a bounded wait of the group's split
    rows ran out since the last check (waits for the device first)."""
    _check(lib().psk_group_check(ctypes.c_void_p(group)))


def psk_group_destroy(group: int):
    lib().psk_group_destroy(ctypes.c_void_p(group))


def psk_group_get_info(group: int) -> psk_group_info:
    info = psk_group_info()
    _check(lib().psk_group_get_info(ctypes.c_void_p(group), ctypes.byref(info)))
    return info


def psk_group_source(desc: GroupDesc) -> str:
    n = ctypes.c_size_t()
    _check(lib().psk_group_source(ctypes.byref(desc.desc), None, 0, ctypes.byref(n)))
    buf = ctypes.create_string_buffer(n.value + 1)
    _check(lib().psk_group_source(ctypes.byref(desc.desc), buf, n.value + 1, ctypes.byref(n)))
    return buf.value.decode()


def psk_group_code_object(desc: GroupDesc) -> bytes:
    n = ctypes.c_size_t()
    _check(lib().psk_group_code_object(ctypes.byref(desc.desc), None, 0, ctypes.byref(n)))
    buf = ctypes.create_string_buffer(n.value)
    _check(lib().psk_group_code_object(ctypes.byref(desc.desc), buf, n.value, ctypes.byref(n)))
    return buf.raw[:n.value]


def psk_group_run_tree(group: int, tree: int, in_slots: Sequence[int], out_slot: int,
                       scalars: Sequence[int] = (), stream: Optional[int] = None):
    """in_slots[k]: the tree slot of rank-1 input k; scalars[k]: the device
    address of rank-0 input k (0 for rank-1 inputs)."""
    n = max(len(in_slots), len(scalars), 1)
    sl = (ctypes.c_int32 * n)(*[int(x) for x in list(in_slots) + [0] * (n - len(in_slots))])
    sc = (ctypes.c_void_p * n)(*[ctypes.c_void_p(int(p)) for p in list(scalars) + [0] * (n - len(scalars))])
    _check(lib().psk_group_run_tree(ctypes.c_void_p(group), ctypes.c_void_p(tree), sl, int(out_slot), sc,
                                    ctypes.c_void_p(stream or 0)))


def psk_group_run_tree_multi(group: int, tree: int, in_slots: Sequence[int], out_slots: Sequence[int],
                             scalars: Sequence[int] = (), stream: Optional[int] = None):
    """out_slots[0]: the root's slot, out_slots[1 + k]: extra output k's."""
    n = max(len(in_slots), len(scalars), 1)
    sl = (ctypes.c_int32 * n)(*[int(x) for x in list(in_slots) + [0] * (n - len(in_slots))])
    sc = (ctypes.c_void_p * n)(*[ctypes.c_void_p(int(p)) for p in list(scalars) + [0] * (n - len(scalars))])
    os_ = (ctypes.c_int32 * max(1, len(out_slots)))(*[int(x) for x in out_slots])
    _check(lib().psk_group_run_tree_multi(ctypes.c_void_p(group), ctypes.c_void_p(tree), sl, os_, sc,
                                          ctypes.c_void_p(stream or 0)))


def psk_tree_create(leaves: Sequence[Tuple[int, Sequence[int]]], slot_dtypes: Sequence) -> int:
    """leaves: (numel, [slot device addresses]) per leaf."""
    n_slots = len(slot_dtypes)
    arr = (psk_leaf * max(1, len(leaves)))()
    for i, (numel, slots) in enumerate(leaves):
        arr[i].numel = int(numel)
        for s, p in enumerate(slots):
            arr[i].slot[s] = p
    dts = (ctypes.c_int32 * n_slots)(*[_dtype_code(d) for d in slot_dtypes])
    h = ctypes.c_void_p()
    _check(lib().psk_tree_create(arr, len(leaves), n_slots, dts, ctypes.byref(h)))
    return h.value


def psk_tree_destroy(tree: int):
    lib().psk_tree_destroy(ctypes.c_void_p(tree))


def psk_tree_get_info(tree: int) -> psk_tree_info:
    info = psk_tree_info()
    _check(lib().psk_tree_get_info(ctypes.c_void_p(tree), ctypes.byref(info)))
    return info


def psk_tree_get_tables(tree: int):
    import numpy as np
    info = psk_tree_get_info(tree)
    off = np.zeros(info.n_leaves + 1, np.int64)
    cl = np.zeros(info.n_chunks, np.int32)
    cs = np.zeros(info.n_chunks, np.int64)
    cc = np.zeros(info.n_chunks, np.int32)
    _check(lib().psk_tree_get_tables(ctypes.c_void_p(tree), off.ctypes.data, cl.ctypes.data, cs.ctypes.data,
                                     cc.ctypes.data))
    return off, cl, cs, cc


def psk_tree_plan(numel: Sequence[int]):
    import numpy as np
    n = np.ascontiguousarray(numel, np.int64)
    nc = ctypes.c_int64()
    _check(lib().psk_tree_plan(n.ctypes.data, len(n), ctypes.byref(nc), None, None, None, None))
    off = np.zeros(len(n) + 1, np.int64)
    cl = np.zeros(nc.value, np.int32)
    cs = np.zeros(nc.value, np.int64)
    cc = np.zeros(nc.value, np.int32)
    _check(lib().psk_tree_plan(n.ctypes.data, len(n), ctypes.byref(nc), off.ctypes.data, cl.ctypes.data,
                               cs.ctypes.data, cc.ctypes.data))
    return off, cl, cs, cc


def psk_adamw_step(tree: int, lr: float, beta1: float, beta2: float, eps: float, weight_decay: float, t: int,
                   stream: Optional[int] = None):
    hp = psk_adamw_hp(lr, beta1, beta2, eps, weight_decay, int(t))
    _check(lib().psk_adamw_step(ctypes.c_void_p(tree), ctypes.byref(hp), ctypes.c_void_p(stream or 0)))


def adamw_config(lr, beta1, beta2, eps, weight_decay, t, total=0, warmup=0, schedule="constant",
                 grad_clip=0.0) -> psk_adamw_config:
    return psk_adamw_config(lr, beta1, beta2, eps, weight_decay, int(t), int(total), int(warmup),
                            PSK_SCHED[schedule] if isinstance(schedule, str) else int(schedule), grad_clip)


def psk_adamw_step_config(tree: int, cfg: psk_adamw_config, stream: Optional[int] = None):
    _check(lib().psk_adamw_step_config(ctypes.c_void_p(tree), ctypes.byref(cfg), ctypes.c_void_p(stream or 0)))


def psk_adamw_step_config_noalloc(tree: int, cfg: psk_adamw_config, stream: Optional[int] = None):
    _check(lib().psk_adamw_step_config_noalloc(ctypes.c_void_p(tree), ctypes.byref(cfg),
                                               ctypes.c_void_p(stream or 0)))


def psk_adamw_lr(cfg: psk_adamw_config) -> float:
    x = ctypes.c_double()
    _check(lib().psk_adamw_lr(ctypes.byref(cfg), ctypes.byref(x)))
    return x.value


def psk_tree_clip_result(tree: int):
    ss, f = ctypes.c_double(), ctypes.c_float()
    _check(lib().psk_tree_clip_result(ctypes.c_void_p(tree), ctypes.byref(ss), ctypes.byref(f)))
    return ss.value, f.value


def _body_arrays(nodes, types, is_output):
    n = len(nodes)
    arr = node_array(nodes) if n else (psk_node * 1)()
    tys = (psk_tensor_desc * max(1, n))(*[tensor_desc(s, d) for s, d in types])
    outs = (ctypes.c_uint8 * max(1, n))(*[1 if o else 0 for o in is_output])
    return n, arr, tys, outs


def psk_partition(nodes, types: Sequence[Tuple[Sequence[int], object]], is_output: Sequence[bool], rows=False):
    """(group_of, is_root, n_groups); rows=True fuses last-axis row
    reductions (psk_partition_ex with PSK_PARTITION_ROWS)."""
    import numpy as np
    n, arr, tys, outs = _body_arrays(nodes, types, is_output)
    g = (ctypes.c_int32 * max(1, n))()
    r = (ctypes.c_int32 * max(1, n))()
    ng = ctypes.c_int32()
    if rows:
        _check(lib().psk_partition_ex(n, arr, tys, outs, PSK_PARTITION_ROWS, g, r, ctypes.byref(ng)))
    else:
        _check(lib().psk_partition(n, arr, tys, outs, g, r, ctypes.byref(ng)))
    return np.array(g[:n], np.int32), np.array(r[:n], np.int32), ng.value


def psk_dispatch_count(nodes, types, is_output, rows=False) -> dict:
    n, arr, tys, outs = _body_arrays(nodes, types, is_output)
    rep = psk_dispatch_report()
    _check(lib().psk_dispatch_count(n, arr, tys, outs, PSK_PARTITION_ROWS if rows else 0, ctypes.byref(rep)))
    return {k: getattr(rep, k) for k, _ in psk_dispatch_report._fields_}


def psk_last_error() -> str:
    return lib().psk_last_error().decode(errors="replace")


def psk_status_str(status: int) -> str:
    return lib().psk_status_str(status).decode()


def psk_version() -> int:
    return lib().psk_version()


def psk_get_stats() -> psk_stats:
    s = psk_stats()
    _check(lib().psk_get_stats(ctypes.byref(s)))
    return s


# ----------------------------------------------------- torch conveniences
def _stream_handle(stream) -> int:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _numel(shape) -> int:
    n = 1
    for d in shape:
        n *= int(d)
    return n


def _check_buffer(t, numel: int, code: int, what: str, dev: int):
    """A tensor for one of a group's buffers: its element count and storage
    type, on the current device."""
    if t.numel() != numel:
        raise ValueError(f"{what}: {t.numel()} elements where the group's buffer has {numel}")
    try:
        tcode = _dtype_code(str(t.dtype))
    except ValueError:
        tcode = None
    if tcode != code:
        raise ValueError(f"{what}: {t.dtype} does not hold the group's storage type {('f32', 'bf16', 'u8')[code]}")
    if t.device.index != dev:
        raise ValueError(f"{what}: on {t.device}, the current device is cuda:{dev}")


class Group:
    """A compiled fusion group, run on torch tensors."""

    def __init__(self, nodes, inputs, out_shape, out_dtype, root=None, tree=False, extras=(), online=False):
        """online: take a row sum of exp(y - row_max(y)) in the maximum's pass
        (PSK_GROUP_ONLINE)."""
        flags = (PSK_GROUP_TREE if tree else 0) | (PSK_GROUP_ONLINE if online else 0)
        self.desc = GroupDesc(nodes, inputs, out_shape, out_dtype, root=root, flags=flags, extras=extras)
        self.n_extra = len(extras)
        self.handle = psk_group_create(self.desc)
        self.out_shape = tuple(out_shape)
        self.out_dtype = out_dtype
        # what each buffer must hold: the kernel reads and writes exactly
        # these extents, so a smaller or differently typed tensor is refused
        # here, before the launch
        self.tree = tree
        self._in_specs = [(_numel(spec[0]), _dtype_code(spec[1])) for spec in inputs]
        # strided inputs: the shape and strides a tensor must have
        self._in_layout = [(tuple(int(x) for x in spec[0]), tuple(int(x) for x in spec[2]))
                           if len(spec) > 2 and spec[2] is not None else None for spec in inputs]
        self._out_specs = [(_numel(out_shape), _dtype_code(out_dtype))] + [
            (_numel(sh), _dtype_code(d)) for _, sh, d in extras]

    @property
    def info(self) -> psk_group_info:
        return psk_group_get_info(self.handle)

    def check(self):
        """psk_group_check: raises if a split-row wait of this group ran out."""
        psk_group_check(self.handle)

    def run(self, inputs, out, stream=None, extra_outs=None):
        """extra_outs: one tensor per extra output (a group with extra outputs
        runs through psk_group_run_multi)."""
        outs = [out] + list(extra_outs or [])
        for t in outs:
            if not t.is_cuda or not t.is_contiguous():
                raise ValueError("group outputs must be contiguous device tensors")
        for k, t in enumerate(inputs):
            layout = self._in_layout[k] if k < len(self._in_layout) else None
            if not t.is_cuda:
                raise ValueError(f"input {k} must be a device tensor")
            if layout is None:
                if not t.is_contiguous():
                    raise ValueError(f"input {k}: the group was created for a dense input; create it with this "
                                     f"tensor's strides {tuple(t.stride())} to read the view in place")
            else:
                shape, strides = layout
                got = tuple(x if n > 1 else 0 for n, x in zip(t.shape, t.stride()))
                want = tuple(x if n > 1 else 0 for n, x in zip(shape, strides))
                if tuple(t.shape) != shape or got != want:
                    raise ValueError(f"input {k}: shape {tuple(t.shape)} strides {tuple(t.stride())}, where the "
                                     f"group reads shape {shape} strides {strides}")
        # Each tensor against the group's buffer: without extra_outs only the
        # root's (the library refuses the call if the group has extra
        # outputs); none for a tree-mapped group, which the library refuses
        # here since its buffers are a tree's leaves.
        if not self.tree:
            out_specs = self._out_specs if extra_outs is not None else self._out_specs[:1]
            if len(inputs) != len(self._in_specs) or len(outs) != len(out_specs):
                raise ValueError(f"the group takes {len(self._in_specs)} inputs and {len(self._out_specs)} outputs")
            import torch
            dev = torch.cuda.current_device()
            for what, ts, specs in (("input", inputs, self._in_specs), ("output", outs, out_specs)):
                for k, (t, (n, code)) in enumerate(zip(ts, specs)):
                    _check_buffer(t, n, code, f"{what} {k}", dev)
        if extra_outs is None:
            psk_group_run(self.handle, [t.data_ptr() for t in inputs], out.data_ptr(), _stream_handle(stream))
        else:
            psk_group_run_multi(self.handle, [t.data_ptr() for t in inputs], [t.data_ptr() for t in outs],
                                _stream_handle(stream))
        return out

    def run_tree(self, tree: "Tree", in_slots, out_slot, scalars=(), stream=None):
        """Map the group over every leaf of `tree` (one launch); scalars are
        0-d device tensors (or None for per-element inputs)."""
        if len(scalars) > len(self._in_specs):
            raise ValueError(f"the group takes {len(self._in_specs)} inputs")
        for k, t in enumerate(scalars):
            if t is not None:
                if not t.is_cuda:
                    raise ValueError(f"scalar input {k} must be a device tensor")
                _check_buffer(t, 1, self._in_specs[k][1], f"scalar input {k}", t.device.index)
        ptrs = [0 if t is None else t.data_ptr() for t in scalars]
        if isinstance(out_slot, int):
            psk_group_run_tree(self.handle, tree.handle, in_slots, out_slot, ptrs, _stream_handle(stream))
        else:
            psk_group_run_tree_multi(self.handle, tree.handle, in_slots, out_slot, ptrs, _stream_handle(stream))

    def __del__(self):
        h = getattr(self, "handle", None)
        if h and _lib is not None:
            psk_group_destroy(h)
            self.handle = None


class Tree:
    """A parameter tree over torch tensors: slots theta, g, m, v (in place) or
    theta, g, m, v, theta', m', v'."""

    def __init__(self, slots: Sequence[Sequence], n_slots: Optional[int] = None):
        self._keep = [list(s) for s in slots]       # keep the tensors alive
        if n_slots is None:
            n_slots = len(self._keep[0]) if self._keep else 4
        dts = [self._dt(t) for t in self._keep[0]] if self._keep else [PSK_F32] * n_slots
        leaves = []
        dev = None
        for i, s in enumerate(self._keep):
            if len(s) != n_slots:
                raise ValueError(f"leaf {i} has {len(s)} slots, the tree {n_slots}")
            n = s[0].numel()
            for k, t in enumerate(s):
                if t.numel() != n or (n and (not t.is_cuda or not t.is_contiguous())):
                    raise ValueError("leaf slots must be contiguous device tensors of equal numel")
                # a slot has one storage type over every leaf: the kernels
                # read and write each leaf's buffer at that type's size
                if self._dt(t) != dts[k]:
                    raise ValueError(f"leaf {i} slot {k}: {t.dtype}, where slot {k} of leaf 0 has another type")
                if n:
                    if dev is None:
                        import torch
                        dev = torch.cuda.current_device()
                    if t.device.index != dev:
                        raise ValueError(f"leaf {i} slot {k}: on {t.device}, the current device is cuda:{dev}")
            leaves.append((n, [t.data_ptr() for t in s]))
        self.handle = psk_tree_create(leaves, dts)

    @staticmethod
    def _dt(t) -> int:
        import torch
        if t.dtype == torch.float32:
            return PSK_F32
        if t.dtype == torch.bfloat16:
            return PSK_BF16
        raise ValueError(f"unsupported dtype {t.dtype}")

    @property
    def info(self) -> psk_tree_info:
        return psk_tree_get_info(self.handle)

    def adamw_step(self, lr, beta1, beta2, eps, weight_decay, t, stream=None, **config):
        """One AdamW step; keyword arguments total, warmup, schedule and
        grad_clip select psk_adamw_step_config."""
        if config:
            cfg = adamw_config(lr, beta1, beta2, eps, weight_decay, t, **config)
            psk_adamw_step_config(self.handle, cfg, _stream_handle(stream))
        else:
            psk_adamw_step(self.handle, lr, beta1, beta2, eps, weight_decay, t, _stream_handle(stream))

    def adamw_step_noalloc(self, lr, beta1, beta2, eps, weight_decay, t, stream=None, **config):
        """The configured step through psk_adamw_step_config_noalloc (the
        clipping pass's scratch in the library's static device array)."""
        cfg = adamw_config(lr, beta1, beta2, eps, weight_decay, t, **config)
        psk_adamw_step_config_noalloc(self.handle, cfg, _stream_handle(stream))

    def clip_result(self):
        return psk_tree_clip_result(self.handle)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h and _lib is not None:
            psk_tree_destroy(h)
            self.handle = None
