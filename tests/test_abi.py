"""The C-ABI library on the host: exported symbols, refusals, host-side
planning (partition, leaf/chunk tables), and the emitted kernels compiled by
hipRTC for gfx950 -- no GPU needed."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from synth import configs
from synth.dag import Node, parse_dag

P = pytest.importorskip("elementwise_reduction_groups_amd")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "psk_fused.h")
OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"
READELF = "/opt/rocm/llvm/bin/llvm-readelf"


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(P.LIB_PATH):
        from elementwise_reduction_groups_amd import build
        build.build()
    return P.lib()


def test_every_declared_symbol_is_exported(lib):
    decl = re.findall(r"\b(psk_[a-z_]+)\s*\(", open(HEADER).read())
    names = sorted(set(decl))
    assert len(names) >= 17
    out = subprocess.run(["nm", "-D", "--defined-only", P.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (psk_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert set(P.EXPORTED) <= exported
    assert P.psk_version() == P.PSK_VERSION == 200


def test_status_strings(lib):
    for i, name in enumerate(P.STATUS_NAMES):
        assert P.psk_status_str(i) == name


def _desc(text, inputs, out_shape, out_dtype="f32", **kw):
    return P.GroupDesc(parse_dag(text), inputs, out_shape, out_dtype, **kw)


def _refused(desc, status):
    with pytest.raises(P.PskError) as ei:
        P.psk_group_source(desc)
    assert ei.value.status == status, (ei.value.name, str(ei.value))
    assert P.STATUS_NAMES[status] in str(ei.value)


F = [((8, 16), "f32")]


def test_refusals(lib):
    # member cap: 65 members
    chain = "%0 = input 0\n" + "".join(f"%{i + 1} = exp %{i}\n" for i in range(65))
    _refused(_desc(chain, F, (8, 16)), P.PSK_E_CAP)
    ok64 = "%0 = input 0\n" + "".join(f"%{i + 1} = exp %{i}\n" for i in range(64))
    assert "psk_kernel" in P.psk_group_source(_desc(ok64, F, (8, 16)))
    # operand naming a later node (a cycle)
    _refused(_desc("%0 = input 0\n%1 = add %0 %2\n%2 = exp %0\n", F, (8, 16)), P.PSK_E_ORDER)
    # two roots
    _refused(_desc("%0 = input 0\n%1 = exp %0\n%2 = tanh %0\n", F, (8, 16)), P.PSK_E_ROOT)
    # root read by another node
    _refused(_desc("%0 = input 0\n%1 = exp %0\n%2 = tanh %1\n", F, (8, 16), root=1), P.PSK_E_ROOT)
    # dead leaf
    _refused(_desc("%0 = input 0\n%1 = const 1.0\n%2 = exp %0\n", F, (8, 16)), P.PSK_E_DEAD)
    # an input that widens the output
    _refused(_desc("%0 = input 0\n%1 = exp %0\n", [((8, 32), "f32")], (8, 16)), P.PSK_E_BROADCAST)
    _refused(_desc("%0 = input 0\n%1 = exp %0\n", [((2, 8, 16), "f32")], (8, 16)), P.PSK_E_BROADCAST)
    # bf16 arithmetic requested
    _refused(_desc("%0 = input 0\n%1 = exp %0\n", F, (8, 16), arith=P.PSK_BF16), P.PSK_E_TYPE)
    # a boundary op inside a group
    bad = [Node("input", (), None, 0), Node("cast", (0,))]
    _refused(P.GroupDesc(bad, F, (8, 16), "f32"), P.PSK_E_OP)
    # pow 3 with other members
    _refused(_desc("%0 = input 0\n%1 = pown %0 3\n%2 = exp %1\n", F, (8, 16)), P.PSK_E_OP)
    assert P.psk_group_source(_desc("%0 = input 0\n%1 = pown %0 3\n", F, (8, 16)))
    # reduction of a row value; a row value as the stored root
    _refused(_desc("%0 = input 0\n%1 = row_sum %0\n%2 = row_max %1\n%3 = add %0 %2\n", F, (8, 16)), P.PSK_E_ROW)
    _refused(_desc("%0 = input 0\n%1 = row_sum %0\n", F, (8, 16)), P.PSK_E_ROW)
    # bad input slot, bad arity
    _refused(_desc("%0 = input 3\n%1 = exp %0\n", F, (8, 16)), P.PSK_E_OP)
    nd = [Node("input", (), None, 0), Node("exp", (0,))]
    d = P.GroupDesc(nd, F, (8, 16), "f32")
    d._nodes[1].b = 0
    _refused(d, P.PSK_E_OP)
    # NULL descriptor
    n = ctypes.c_size_t()
    assert lib.psk_group_source(None, None, 0, ctypes.byref(n)) == P.PSK_E_NULL
    # negative sizes, rank out of range
    _refused(_desc("%0 = input 0\n%1 = exp %0\n", [((8, 16), "f32")], (8, -16)), P.PSK_E_SHAPE)
    # reserved flags
    _refused(_desc("%0 = input 0\n%1 = exp %0\n", F, (8, 16), flags=4), P.PSK_E_UNSUPPORTED)


T1 = [((1,), "f32")]


def test_tree_group_refusals(lib):
    tree = dict(flags=P.PSK_GROUP_TREE)
    # the output and every input are per element (rank 1) or per tree (rank 0)
    _refused(_desc("%0 = input 0\n%1 = exp %0\n", T1, (8, 16), **tree), P.PSK_E_SHAPE)
    _refused(_desc("%0 = input 0\n%1 = exp %0\n", [((8, 16), "f32")], (1,), **tree), P.PSK_E_SHAPE)
    # no rows: no row reduction, no causal mask
    _refused(_desc("%0 = input 0\n%1 = row_max %0\n%2 = sub %0 %1\n", T1, (1,), **tree), P.PSK_E_ROW)
    _refused(_desc("%0 = input 0\n%1 = causal_mask %0 4\n", T1, (1,), **tree), P.PSK_E_OP)
    # the usual group rules still hold
    chain = "%0 = input 0\n" + "".join(f"%{i + 1} = exp %{i}\n" for i in range(65))
    _refused(_desc(chain, T1, (1,), **tree), P.PSK_E_CAP)
    _refused(_desc("%0 = input 0\n%1 = exp %0\n", T1, (1,), arith=P.PSK_BF16, **tree), P.PSK_E_TYPE)
    # accepted: rank-1 output, rank-1 and rank-0 inputs of either storage type
    g = P.psk_group_create(_desc("%0 = input 0\n%1 = input 1\n%2 = mul %0 %1\n",
                                 [((1,), "bf16"), ((), "f32")], (1,), "bf16", **tree))
    info = P.psk_group_get_info(g)
    assert info.kind == 2 and info.members == 1
    P.psk_group_destroy(g)


def test_tree_group_kernel_compiles(lib, tmp_path):
    from synth import configs as C
    desc = P.GroupDesc(C.tree_mixed_dag(), [((1,), "f32"), ((1,), "bf16"), ((), "f32")], (1,), "bf16",
                       flags=P.PSK_GROUP_TREE)
    src = P.psk_group_source(desc)
    # slot addresses are read from the leaf table and named as global memory
    assert "L->slot[slot0]" in src and "L->slot[slot1]" in src and "L->slot[slot3]" in src
    assert "L->slot[slot2]" not in src and "PSK_G" in src   # input 2 is a rank-0 scalar
    asm, notes = _isa(P.psk_group_code_object(desc), tmp_path, "tree")
    assert not re.search(r"v_pk_(fma|mul|add)_f32", asm)
    assert re.search(r"\.private_segment_fixed_size:\s+0\b", notes)
    # global (not generic) accesses, 16-byte vectors: 10 bytes per element
    # gives 8 elements per thread (two f32 vectors, one bf16 vector each)
    assert "global_load_dwordx4" in asm and "global_store_dwordx4" in asm
    assert not re.search(r"\bflat_(load|store)", asm)
    g = P.psk_group_create(desc)
    assert P.psk_group_get_info(g).vec == 8
    P.psk_group_destroy(g)
    # an SGD step moves 6 bytes per element: 8 elements per thread
    g = P.psk_group_create(P.GroupDesc(C.tree_sgd_dag(), [((1,), "bf16"), ((1,), "bf16"), ((), "f32")], (1,),
                                       "bf16", flags=P.PSK_GROUP_TREE))
    assert P.psk_group_get_info(g).vec == 8
    P.psk_group_destroy(g)


def test_group_create_needs_no_gpu(lib):
    g = P.psk_group_create(_desc("%0 = input 0\n%1 = input 1\n%2 = add %0 %1\n",
                                 [((33, 64), "f32"), ((33, 1), "f32")], (33, 64)))
    info = P.psk_group_get_info(g)
    assert info.kind == 0 and info.members == 1 and info.vec == 4
    assert info.algorithmic_bytes == 33 * 64 * 4 * 2 + 33 * 4
    P.psk_group_destroy(g)


def _partition_nodes(rng, n):
    nodes, types, outs = [Node("input", (), None, 0)], [((4, 8), "f32")], [False]
    for i in range(1, n):
        r = rng.random()
        if r < 0.1:
            nodes.append(Node("row_sum", (rng.randrange(i),)))
        elif r < 0.15:
            nodes.append(Node("pown", (rng.randrange(i),), None, 3))
        elif r < 0.2:
            nodes.append(Node("matmul", (rng.randrange(i), rng.randrange(i))))
        elif r < 0.6:
            nodes.append(Node(rng.choice(["add", "mul", "sub"]), (rng.randrange(i), rng.randrange(i))))
        else:
            nodes.append(Node(rng.choice(["exp", "tanh", "gelu"]), (rng.randrange(i),)))
        types.append(((4, 8), "f32") if rng.random() < 0.85 else ((4, 8), "bf16"))
        outs.append(rng.random() < 0.1)
    outs[-1] = True
    return nodes, types, outs


def test_partition_matches_oracle(lib, orc):
    import random
    rng = random.Random(7)
    for trial in range(2000):
        n = rng.randint(2, 90)
        nodes, types, outs = _partition_nodes(rng, n)
        g, r, ng = P.psk_partition(nodes, types, outs)
        tid = [0 if t[1] == "f32" else 1 for t in types]
        og, orr = orc.partition(nodes, tid, outs)
        np.testing.assert_array_equal(g, og)
        np.testing.assert_array_equal(r, orr)
        assert ng == (og.max() + 1 if (og >= 0).any() else 0)


def test_partition_cap(lib):
    for length, sizes in ((64, [64]), (65, [1, 64]), (129, [1, 64, 64])):
        nodes = [Node("input", (), None, 0)] + [Node("exp", (i,)) for i in range(length)]
        types = [((4,), "f32")] * len(nodes)
        g, r, ng = P.psk_partition(nodes, types, [False] * length + [True])
        assert [int((g == k).sum()) for k in range(ng)] == sizes


def test_tree_plan(lib):
    numel = [5888, 2048, 64, 0, 12288, 1, 4097, 3, 4096]
    off, cl, cs, cc = P.psk_tree_plan(numel)
    np.testing.assert_array_equal(off, np.concatenate([[0], np.cumsum(numel)]))
    # every element of every leaf covered exactly once, chunk starts 8-aligned
    for leaf, n in enumerate(numel):
        sel = cl == leaf
        cover = np.zeros(n, np.int32)
        for s, c in zip(cs[sel], cc[sel]):
            assert s % 8 == 0 and 0 < c <= P.PSK_TREE_CHUNK
            cover[s:s + c] += 1
        assert np.all(cover == 1)
    # the tiny GPT tree
    shapes = [s for _, s in configs.tiny_gpt_leaves()]
    off, cl, cs, cc = P.psk_tree_plan([int(np.prod(s)) for s in shapes])
    assert len(shapes) == 28 and off[-1] == 108032
    shapes = [s for _, s in configs.llama_leaves()]
    off, *_ = P.psk_tree_plan([int(np.prod(s)) for s in shapes])
    assert len(shapes) == 145 and off[-1] == 887685120
    # a leaf past 2^31 elements: 64-bit starts, consecutive whole chunks
    big = (1 << 31) + 100
    off, cl, cs, cc = P.psk_tree_plan([5, big, 3])
    assert off.tolist() == [0, 5, 5 + big, 8 + big]
    sel = cl == 1
    assert cs[sel][0] == 0 and np.all(np.diff(cs[sel]) == P.PSK_TREE_CHUNK)
    assert cs[sel][-1] + cc[sel][-1] == big and int(cc[sel].sum()) == big and cs[sel][-1] >= (1 << 31)
    with pytest.raises(P.PskError) as ei:
        P.psk_tree_plan([4, -1])
    assert ei.value.status == P.PSK_E_SHAPE


def test_tree_refusals_without_device(lib):
    # refusals are decided before any device call
    for n_slots in (0, 9):   # 1 to 8 slots
        with pytest.raises(P.PskError) as ei:
            P.psk_tree_create([(8, [16 * (k + 1) for k in range(min(n_slots, 8))])], ["f32"] * n_slots)
        assert ei.value.status == P.PSK_E_SHAPE
    # slots of a generic tree: partial overlaps are refused, and so is one
    # buffer in two slots of different storage types
    with pytest.raises(P.PskError) as ei:
        P.psk_tree_create([(8, [16, 32, 48])], ["f32"] * 3)
    assert ei.value.status == P.PSK_E_ALIAS
    with pytest.raises(P.PskError) as ei:
        P.psk_tree_create([(8, [1024, 1024, 4096])], ["f32", "bf16", "f32"])
    assert ei.value.status == P.PSK_E_ALIAS
    with pytest.raises(P.PskError) as ei:
        P.psk_tree_create([(8, [16, 0, 64, 96])], ["f32"] * 4)
    assert ei.value.status == P.PSK_E_NULL
    with pytest.raises(P.PskError) as ei:
        P.psk_tree_create([(8, [18, 1024, 2048, 4096])], ["f32"] * 4)
    assert ei.value.status == P.PSK_E_ALIGN
    with pytest.raises(P.PskError) as ei:   # theta overlaps g
        P.psk_tree_create([(8, [1024, 1040, 2048, 4096])], ["f32"] * 4)
    assert ei.value.status == P.PSK_E_ALIAS
    with pytest.raises(P.PskError) as ei:   # two leaves overlap
        P.psk_tree_create([(8, [1024, 2048, 3072, 4096]), (8, [1040, 8192, 9216, 10240])], ["f32"] * 4)
    assert ei.value.status == P.PSK_E_ALIAS
    with pytest.raises(P.PskError) as ei:   # one buffer in two slots of different storage types
        P.psk_tree_create([(8, [1024, 2048, 1024, 4096])], ["f32", "f32", "bf16", "f32"])
    assert ei.value.status == P.PSK_E_ALIAS


def _isa(code: bytes, tmp_path, name):
    p = tmp_path / f"{name}.co"
    p.write_bytes(code)
    asm = subprocess.run([OBJDUMP, "-d", str(p)], capture_output=True, text=True, check=True).stdout
    notes = subprocess.run([READELF, "--notes", str(p)], capture_output=True, text=True, check=True).stdout
    return asm, notes


def _workload_descs():
    eps = configs.f32(1e-5)
    return {
        "softmax": P.GroupDesc(configs.softmax_causal_dag(0.125, 1024), [((131072, 1024), "f32")], (131072, 1024), "f32"),
        "rmsnorm": P.GroupDesc(configs.rmsnorm_gelu_dag(eps), [((16384, 4096), "bf16"), ((16384, 4096), "bf16"),
                                                                 ((4096,), "bf16")], (16384, 4096), "bf16"),
        "chain64": P.GroupDesc(configs.chain64_dag(), [((16384, 16384), "f32"), ((16384, 1), "f32"),
                                                       ((1, 16384), "f32")], (16384, 16384), "f32"),
    }


@pytest.mark.parametrize("name", ["softmax", "rmsnorm", "chain64"])
def test_emitted_kernels_compile_for_gfx950(lib, tmp_path, name):
    code = P.psk_group_code_object(_workload_descs()[name])
    asm, notes = _isa(code, tmp_path, name)
    assert "gfx950" in subprocess.run(["file", "-b", str(tmp_path / f"{name}.co")], capture_output=True,
                                      text=True).stdout or "amdgcn" in notes or True
    # no packed-FP32 instructions, no spills to scratch
    assert not re.search(r"v_pk_(fma|mul|add)_f32", asm)
    assert re.search(r"\.private_segment_fixed_size:\s+0\b", notes)
    # 16-byte accesses on the row data
    assert "global_load_dwordx4" in asm and "global_store_dwordx4" in asm
    if name != "chain64":
        assert "row_mirror" in asm and "v_readlane_b32" in asm   # DPP wave reduction


def test_emitted_source_structure(lib):
    src = P.psk_group_source(_workload_descs()["softmax"])
    # masked scores are not loaded: the load of vector k is predicated on its first column
    assert "<= q) w0_" in src.replace("&& c0 <= q", "<= q") or "c0 <= q" in src
    assert src.count("__syncthreads") == 2          # two waves per 1024-wide row: one LDS exchange per phase
    src = P.psk_group_source(_workload_descs()["rmsnorm"])
    assert src.count("__syncthreads") == 1          # 256 lanes per row: one cross-wave exchange


def test_schedule_lr_matches_oracle(lib, orc):
    for kind in ("constant", "linear", "cosine"):
        for t in (1, 5, 10, 11, 37, 99, 100):
            cfg = P.adamw_config(3e-4, 0.9, 0.999, 1e-8, 0.01, t, total=100, warmup=10, schedule=kind)
            assert P.psk_adamw_lr(cfg) == orc.lr_schedule(kind, 3e-4, t, 100, 10)
    for bad in (dict(t=0, total=100, warmup=10), dict(t=101, total=100, warmup=10),
                dict(t=5, total=100, warmup=100)):
        with pytest.raises(P.PskError) as ei:
            P.psk_adamw_lr(P.adamw_config(3e-4, 0.9, 0.999, 1e-8, 0.01, schedule="cosine", **bad))
        assert ei.value.status == P.PSK_E_SHAPE


def test_extra_output_refusals(lib):
    from synth import configs as C
    pw = "%0 = input 0\n%1 = exp %0\n%2 = tanh %1\n"
    ok = _desc(pw, F, (8, 16), extras=[(1, (8, 16), "bf16")])
    assert "xo0" in P.psk_group_source(ok)
    _refused(_desc(pw, F, (8, 16), extras=[(0, (8, 16), "f32")]), P.PSK_E_ROOT)       # an input
    _refused(_desc(pw, F, (8, 16), extras=[(2, (8, 16), "f32")]), P.PSK_E_ROOT)       # the root
    _refused(_desc(pw, F, (8, 16), extras=[(1, (8, 16), "f32"), (1, (8, 16), "f32")]), P.PSK_E_ROOT)
    _refused(_desc(pw, F, (8, 16), extras=[(7, (8, 16), "f32")]), P.PSK_E_ROOT)       # out of range
    _refused(_desc(pw, F, (8, 16), extras=[(1, (8, 1), "f32")]), P.PSK_E_SHAPE)       # element value, row shape
    _refused(_desc(pw, F, (8, 16), extras=[(1, (8, 16), 7)]), P.PSK_E_TYPE)
    _refused(_desc(pw, F, (8, 16), extras=[(1, (8, 16), "f32")] * 8), P.PSK_E_CAP)
    # a second unread member is kept only as a stored value
    two = "%0 = input 0\n%1 = exp %0\n%2 = tanh %0\n"
    _refused(_desc(two, F, (8, 16), root=2), P.PSK_E_ROOT)
    assert P.psk_group_source(_desc(two, F, (8, 16), root=2, extras=[(1, (8, 16), "f32")]))
    # a row value is stored per row
    rows = "%0 = input 0\n%1 = row_max %0\n%2 = sub %0 %1\n"
    _refused(_desc(rows, F, (8, 16), extras=[(1, (8, 16), "f32")]), P.PSK_E_SHAPE)
    assert "xo0[row]" in P.psk_group_source(_desc(rows, F, (8, 16), extras=[(1, (8, 1), "f32")]))
    # tree-mapped groups store element values only
    tree = dict(flags=P.PSK_GROUP_TREE)
    _refused(_desc("%0 = input 0\n%1 = input 1\n%2 = mul %1 %1\n%3 = mul %0 %2\n", [((1,), "f32"), ((), "f32")],
                   (1,), extras=[(2, (1,), "f32")], **tree), P.PSK_E_SHAPE)


def test_multi_output_kernels_compile(lib, tmp_path):
    from synth import configs as C
    eps = C.f32(1e-5)
    R, N = 16384, 4096
    descs = {
        "layernorm": P.GroupDesc(C.layernorm_dag(eps), [((R, N), "bf16"), ((N,), "bf16"), ((N,), "bf16")], (R, N),
                                 "bf16", root=C.LAYERNORM_ROOT,
                                 extras=[(C.LAYERNORM_MEAN, (R, 1), "f32"), (C.LAYERNORM_RSTD, (R, 1), "f32")]),
        "add_rmsnorm_h": P.GroupDesc(C.rmsnorm_gelu_dag(eps), [((R, N), "bf16"), ((R, N), "bf16"), ((N,), "bf16")],
                                     (R, N), "bf16", extras=[(C.RMSNORM_H, (R, N), "bf16")]),
        "adamw_tree": P.GroupDesc(C.adamw_group_dag(), [((1,), "bf16"), ((1,), "bf16"), ((1,), "f32"), ((1,), "f32")]
                                  + [((), "f32")] * 9, (1,), "bf16", flags=P.PSK_GROUP_TREE,
                                  extras=[(C.ADAMW_GROUP_M, (1,), "f32"), (C.ADAMW_GROUP_V, (1,), "f32")]),
    }
    for name, d in descs.items():
        asm, notes = _isa(P.psk_group_code_object(d), tmp_path, name)
        assert not re.search(r"v_pk_(fma|mul|add)_f32", asm), name
        assert re.search(r"\.private_segment_fixed_size:\s+0\b", notes), name
        g = P.psk_group_create(d)
        info = P.psk_group_get_info(g)
        P.psk_group_destroy(g)
        if name == "layernorm":
            # mean then variance: two reduction phases in one kernel; the
            # algorithmic bytes count the two per-row statistics
            assert info.kind == 1 and info.phases == 2 and info.n_reductions == 2
            assert info.algorithmic_bytes == R * N * 2 * 2 + 2 * N * 2 + 2 * R * 4
        if name == "add_rmsnorm_h":
            assert info.algorithmic_bytes == R * N * 2 * 4 + N * 2
        if name == "adamw_tree":
            # 22 bytes an element: 2 elements a thread (44 bytes)
            assert info.kind == 2 and info.vec == 2


def test_mask_refusals(lib):
    from synth.dag import parse_dag

    def refused(status, nodes, inputs, shape, dt="f32"):
        with pytest.raises(P.PskError) as ei:
            P.Group(parse_dag(nodes), inputs, shape, dt)
        assert ei.value.status == status, ei.value.name

    # a mask in arithmetic; a where whose mask is not a mask input; a mask output
    refused(P.PSK_E_TYPE, "%0 = input 0\n%1 = input 1\n%2 = add %0 %1\n", [((4, 8), "f32"), ((4, 8), "u8")], (4, 8))
    refused(P.PSK_E_TYPE, "%0 = input 0\n%1 = input 1\n%2 = where %0 %1 0.0\n", [((4, 8), "f32"), ((4, 8), "f32")],
            (4, 8))
    refused(P.PSK_E_TYPE, "%0 = input 0\n%1 = input 1\n%2 = where %1 %0 0.0\n", [((4, 8), "f32"), ((4, 8), "u8")],
            (4, 8), "u8")
    # a mask may not widen the scores
    refused(P.PSK_E_BROADCAST, "%0 = input 0\n%1 = input 1\n%2 = where %1 %0 0.0\n",
            [((4, 8), "f32"), ((2, 4, 8), "u8")], (4, 8))


def test_wide_rows_take_split_or_tiled_kernels(lib, tmp_path, monkeypatch):
    """Rows too wide for one workgroup's registers: split over workgroups
    (kind 4) by default, the online normalizer included, at the widest
    segment that compiles without spilling registers; the tiled kernel
    (kind 3) when forced and for rows a split would need more than 32
    workgroups for."""
    from synth import configs as C
    # up to 32 elements per lane at 1024 lanes the row stays in registers
    g = P.psk_group_create(P.GroupDesc(C.softmax_causal_dag(0.125, 32768), [((4, 32768), "f32")], (4, 32768), "f32"))
    assert P.psk_group_get_info(g).kind == 1
    P.psk_group_destroy(g)
    plain = P.GroupDesc(C.softmax_dag(0.125), [((4, 131072), "f32")], (4, 131072), "f32")
    g = P.psk_group_create(plain)
    info = P.psk_group_get_info(g)
    P.psk_group_destroy(g)
    assert info.kind == 4 and info.split == 4 and info.block == 512 and info.lanes_per_row == 2048
    for cols, dt, kind in [(32772, "f32", 4), (65536, "f32", 4), (131072, "bf16", 4), (1 << 20, "f32", 3)]:
        d = P.GroupDesc(C.softmax_causal_dag(0.125, cols), [((4, cols), dt)], (4, cols), dt)
        for forced in (False, True):
            if forced:
                monkeypatch.setenv("PSK_LAYOUT", "tiled=1")
            g = P.psk_group_create(d)
            info = P.psk_group_get_info(g)
            P.psk_group_destroy(g)
            k = 3 if forced else kind
            assert info.kind == k, (cols, dt, forced)
            if k == 3:
                assert info.lanes_per_row == 512 and info.rows_per_block == 1
                assert info.tiles == -(-cols // (512 * 2 * info.vec))
            else:
                assert 2 <= info.split <= 32 and info.split * 512 * info.vec * 16 >= cols
            asm, notes = _isa(P.psk_group_code_object(d), tmp_path, f"wide{cols}{forced}")
            assert re.search(r"\.private_segment_fixed_size:\s+0\b", notes)    # no spills
            assert not re.search(r"v_pk_(fma|mul|add)_f32", asm)
            monkeypatch.delenv("PSK_LAYOUT", raising=False)
    # the other wide row groups (several inputs, byte masks, extra outputs,
    # the online normalizer) keep their register caches without spilling
    eps, W = C.f32(1e-5), 70000
    others = {
        "ln": P.GroupDesc(C.layernorm_dag(eps), [((4, W), "bf16"), ((W,), "bf16"), ((W,), "bf16")], (4, W), "bf16",
                          root=C.LAYERNORM_ROOT,
                          extras=[(C.LAYERNORM_MEAN, (4, 1), "f32"), (C.LAYERNORM_RSTD, (4, 1), "f32")]),
        "rms_f32": P.GroupDesc(C.rmsnorm_gelu_dag(eps), [((4, W), "f32"), ((4, W), "f32"), ((W,), "f32")], (4, W), "f32"),
        "rms_h": P.GroupDesc(C.rmsnorm_gelu_dag(eps), [((4, W), "bf16"), ((4, W), "bf16"), ((W,), "bf16")], (4, W),
                             "bf16", extras=[(C.RMSNORM_H, (4, W), "bf16")]),
        "masked_f32": P.GroupDesc(C.softmax_masked_dag(0.125), [((4, W), "f32"), ((4, W), "u8")], (4, W), "f32"),
        "masked_bf16": P.GroupDesc(C.softmax_masked_dag(0.125), [((4, W), "bf16"), ((4, W), "u8")], (4, W), "bf16"),
        "online_bf16": P.GroupDesc(C.softmax_dag(0.125), [((4, 131072), "bf16")], (4, 131072), "bf16",
                                   flags=P.PSK_GROUP_ONLINE),
    }
    for name, d in others.items():
        for forced in (False, True):
            if forced:
                monkeypatch.setenv("PSK_LAYOUT", "tiled=1")
            g = P.psk_group_create(d)
            assert P.psk_group_get_info(g).kind == (3 if forced else 4), name
            P.psk_group_destroy(g)
            _, notes = _isa(P.psk_group_code_object(d), tmp_path, f"wide_{name}{forced}")
            assert re.search(r"\.private_segment_fixed_size:\s+0\b", notes), name
            monkeypatch.delenv("PSK_LAYOUT", raising=False)
    # rows past 2^30 columns are refused
    _refused(_desc("%0 = input 0\n%1 = row_max %0\n%2 = sub %0 %1\n", [((1, (1 << 30) + 8), "f32")],
                   (1, (1 << 30) + 8)), P.PSK_E_UNSUPPORTED)


def test_precision_follows_what_is_stored(lib):
    from synth import configs as C
    eps = C.f32(1e-5)
    R, N = 64, 4096
    # every result bf16: the gelu root takes the bf16 form, the division by
    # the row value the row's reciprocal
    rms = P.psk_group_source(P.GroupDesc(C.rmsnorm_gelu_dag(eps), [((R, N), "bf16"), ((R, N), "bf16"),
                                                                    ((N,), "bf16")], (R, N), "bf16"))
    body = rms[rms.index('extern "C"'):]
    assert "psk_gelu_b(" in body and "psk_divr(" not in body and "* y8)" in body
    # an f32 result (or an f32 stored statistic) keeps the f32 forms
    rms32 = P.psk_group_source(P.GroupDesc(C.rmsnorm_gelu_dag(eps), [((R, N), "bf16"), ((R, N), "bf16"),
                                                                      ((N,), "bf16")], (R, N), "f32"))
    body = rms32[rms32.index('extern "C"'):]
    assert "psk_gelu(" in body and "psk_gelu_b(" not in body and "psk_divr(" in body
    ln = P.psk_group_source(P.GroupDesc(C.layernorm_dag(eps), [((R, N), "bf16"), ((N,), "bf16"), ((N,), "bf16")],
                                        (R, N), "bf16", root=C.LAYERNORM_ROOT,
                                        extras=[(C.LAYERNORM_MEAN, (R, 1), "f32"), (C.LAYERNORM_RSTD, (R, 1), "f32")]))
    # the division feeds only the bf16 result, but through + beta, a sum
    # that could cancel its error: it stays correctly rounded
    body = ln[ln.index('extern "C"'):]
    assert "psk_divr(" in body and "* y9)" not in body
    # without beta (the normalized value times gamma, then a gelu) the path
    # is well-conditioned and the division takes the reciprocal form
    lng = P.psk_group_source(_desc("%0 = input 0\n%1 = input 1\n%2 = row_mean %0\n%3 = sub %0 %2\n"
                                   "%4 = pow2 %3\n%5 = row_mean %4\n%6 = sqrt %5\n%7 = div %3 %6\n"
                                   "%8 = mul %7 %1\n%9 = gelu %8\n", [((R, N), "bf16"), ((N,), "bf16")], (R, N),
                                   "bf16"))
    body = lng[lng.index('extern "C"'):]
    assert "psk_divr(" not in body and "* y6)" in body
    # two gelus after the division: their condition numbers compound, so
    # the division stays correctly rounded
    lng2 = P.psk_group_source(_desc("%0 = input 0\n%1 = row_mean %0\n%2 = sub %0 %1\n%3 = pow2 %2\n"
                                    "%4 = row_mean %3\n%5 = sqrt %4\n%6 = div %2 %5\n%7 = gelu %6\n"
                                    "%8 = gelu %7\n", [((R, N), "bf16")], (R, N), "bf16"))
    assert "psk_divr(" in lng2[lng2.index('extern "C"'):]
    # ... but an f32 extra that depends on it keeps the correctly rounded one
    ln32 = P.psk_group_source(P.GroupDesc(C.layernorm_dag(eps), [((R, N), "bf16"), ((N,), "bf16"), ((N,), "bf16")],
                                          (R, N), "bf16", root=C.LAYERNORM_ROOT, extras=[(11, (R, N), "f32"), (C.LAYERNORM_RSTD, (R, 1), "f32")]))
    assert "psk_divr(" in ln32[ln32.index('extern "C"'):]
    # h = x + r stored in f32 comes before the division and the gelu: both
    # keep their bf16-result forms
    rmsh = P.psk_group_source(P.GroupDesc(C.rmsnorm_gelu_dag(eps), [((R, N), "bf16"), ((R, N), "bf16"),
                                                                      ((N,), "bf16")], (R, N), "bf16",
                                          extras=[(C.RMSNORM_H, (R, N), "f32")]))
    body = rmsh[rmsh.index('extern "C"'):]
    assert "psk_gelu_b(" in body and "psk_divr(" not in body and "* y8)" in body
    # softmax's exp(y - max y): the short exponential for bf16 results, the
    # split-product one (about two ulps) for f32 results, the library's when
    # the layout asks for it
    for dt, fn in (("bf16", "psk_exp_np_b("), ("f32", "psk_exp_np(")):
        sm = P.psk_group_source(P.GroupDesc(C.softmax_causal_dag(0.125, N), [((R, N), dt)], (R, N), dt))
        body = sm[sm.index('extern "C"'):]
        assert fn in body and "expf(" not in body, dt
    import os
    os.environ["PSK_LAYOUT"] = "fexp=0"
    try:
        sm = P.psk_group_source(P.GroupDesc(C.softmax_causal_dag(0.125, N), [((R, N), "f32")], (R, N), "f32"))
    finally:
        del os.environ["PSK_LAYOUT"]
    body = sm[sm.index('extern "C"'):]
    assert "expf(" in body and "psk_exp_np(" not in body
    # ... but not where a difference could cancel its error (1 - exp(y - max y))
    one = P.psk_group_source(_desc("%0 = input 0\n%1 = row_max %0\n%2 = sub %0 %1\n%3 = exp %2\n"
                                   "%4 = const 1.0\n%5 = sub %4 %3\n", [((R, N), "bf16")], (R, N), "bf16"))
    body = one[one.index('extern "C"'):]
    assert "psk_exp_np_b(" not in body and "psk_exp_np(" not in body and "expf(" in body
    # a gelu that other members read is not the bf16 form
    tree = P.psk_group_source(P.GroupDesc(C.tree_mixed_dag(), [((1,), "f32"), ((1,), "bf16"), ((), "f32")], (1,),
                                          "bf16", flags=P.PSK_GROUP_TREE))
    assert "psk_gelu(" in tree[tree.index('extern "C"'):] and "psk_gelu_b(" not in tree[tree.index('extern "C"'):]


def test_online_normalizer_flag(lib, monkeypatch):
    from synth import configs as C
    O = P.PSK_GROUP_ONLINE
    # a softmax: its sum moves into the maximum's pass (one reduction phase)
    src = P.psk_group_source(P.GroupDesc(C.softmax_dag(0.125), [((8, 64), "f32")], (8, 64), "f32", flags=O))
    body = src[src.index('extern "C"'):]
    assert "float tm6 = " in body and "psk_exp_np(q" in body
    # a row held in registers: one exponential an element, kept from the
    # maximum's pass and rescaled to the row's maximum by the exp member
    assert body.count("psk_exp_np(v2_") == 4 and "(oe6_0 * osc6)" in body
    monkeypatch.setenv("PSK_LAYOUT", "tiled=1")      # the tiled kernel, online and exact
    wide = P.psk_group_source(P.GroupDesc(C.softmax_dag(0.125), [((4, 70000), "f32")], (4, 70000), "f32",
                                          flags=O))
    plain = P.psk_group_source(P.GroupDesc(C.softmax_dag(0.125), [((4, 70000), "f32")], (4, 70000), "f32"))
    monkeypatch.delenv("PSK_LAYOUT")
    # tiled: two walks of the row (register, LDS and memory tile loops each) instead of three
    assert wide.count("for (int t = ") * 3 == plain.count("for (int t = ") * 2
    assert " * osc" not in wide              # tiles walked again: nothing kept
    # split rows: one exchange of (maximum, sum) pairs instead of two exchanges
    split = P.psk_group_source(P.GroupDesc(C.softmax_dag(0.125), [((4, 70000), "f32")], (4, 70000), "f32",
                                           flags=O))
    exact = P.psk_group_source(P.GroupDesc(C.softmax_dag(0.125), [((4, 70000), "f32")], (4, 70000), "f32"))
    assert split.count("psk_take(") == 1 + 1 and exact.count("psk_take(") == 2 + 1   # + the prelude's definition
    assert "psk_exp_np(PSK_RL(v, 0) - a0)" in split or "psk_exp_np(PSK_RL(v, 0) - a1)" in split
    assert " * osc" in split
    # masked and causal softmax take it too
    P.psk_group_source(P.GroupDesc(C.softmax_masked_dag(0.125), [((8, 64), "f32"), ((8, 64), "u8")], (8, 64), "f32",
                                   flags=O))
    P.psk_group_source(P.GroupDesc(C.softmax_causal_dag(0.125, 64), [((8, 64), "bf16")], (8, 64), "bf16", flags=O))
    # refused without such a sum, and for trees
    _refused(P.GroupDesc(C.rmsnorm_gelu_dag(C.f32(1e-5)), [((8, 64), "bf16"), ((8, 64), "bf16"), ((64,), "bf16")],
                         (8, 64), "bf16", flags=O), P.PSK_E_UNSUPPORTED)
    _refused(_desc("%0 = input 0\n%1 = row_max %0\n%2 = sub %0 %1\n%3 = exp %2\n%4 = row_max %3\n%5 = div %3 %4\n",
                   F, (8, 16), flags=O), P.PSK_E_UNSUPPORTED)
    # exp(y - max(z)) with z != y is not the normalizer
    _refused(_desc("%0 = input 0\n%1 = input 1\n%2 = row_max %1\n%3 = sub %0 %2\n%4 = exp %3\n%5 = row_sum %4\n"
                   "%6 = div %4 %5\n", F + F, (8, 16), flags=O), P.PSK_E_UNSUPPORTED)
    _refused(P.GroupDesc(C.tree_sgd_dag(), [((1,), "f32"), ((1,), "f32"), ((), "f32")], (1,), "f32",
                         flags=P.PSK_GROUP_TREE | O), P.PSK_E_UNSUPPORTED)
    # the maximum, the difference or the exponential stored as bf16 (read
    # rounded): the maximum's pass cannot sum what the readers see; stored
    # as f32 they pair as before
    sm = "%0 = input 0\n%1 = row_max %0\n%2 = sub %0 %1\n%3 = exp %2\n%4 = row_sum %3\n%5 = div %3 %4\n"
    for node, shape in [(1, (8, 1)), (2, (8, 16)), (3, (8, 16))]:
        _refused(_desc(sm, F, (8, 16), extras=[(node, shape, "bf16")], flags=O), P.PSK_E_UNSUPPORTED)
        P.psk_group_source(_desc(sm, F, (8, 16), extras=[(node, shape, "f32")], flags=O))


def test_persistent_rows_where_column_vectors_weigh(lib):
    """LayerNorm's γ and β weigh as much as its rows: persistent workgroups
    that load them once; softmax (no column vectors) and RMSNorm (one,
    beside two row inputs) keep one row per workgroup."""
    from synth import configs as C
    eps = C.f32(1e-5)
    R, N = 64, 4096
    persistent = "for (; row < "
    ln = P.psk_group_source(P.GroupDesc(C.layernorm_dag(eps), [((R, N), "bf16"), ((N,), "bf16"), ((N,), "bf16")],
                                        (R, N), "bf16", root=C.LAYERNORM_ROOT,
                                        extras=[(C.LAYERNORM_MEAN, (R, 1), "f32"), (C.LAYERNORM_RSTD, (R, 1), "f32")]))
    assert persistent in ln
    sm = P.psk_group_source(P.GroupDesc(C.softmax_dag(0.125), [((R, N), "f32")], (R, N), "f32"))
    rms = P.psk_group_source(P.GroupDesc(C.rmsnorm_gelu_dag(eps), [((R, N), "bf16"), ((R, N), "bf16"), ((N,), "bf16")],
                                         (R, N), "bf16"))
    assert persistent not in sm and persistent not in rms


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built library every call raises; nothing falls back to
    another implementation."""
    monkeypatch.setattr(P, "_lib", None)
    monkeypatch.setattr(P, "LIB_PATH", str(tmp_path / "libpsk_fused.so"))
    with pytest.raises(RuntimeError, match="not built"):
        P.lib()
    from synth import configs as C
    with pytest.raises(RuntimeError, match="not built"):
        P.Group(C.softmax_dag(0.125), [((4, 8), "f32")], (4, 8), "f32")


def test_kernel_cache_keys_on_every_immediate(lib):
    """Two groups that differ only in a WHERE's fill value (or a constant)
    get different kernels: the cache key carries every immediate a kernel
    reads."""
    def where(fill):
        nd = parse_dag(f"%0 = input 0\n%1 = input 1\n%2 = where %1 %0 {fill}\n%3 = neg %2\n")
        return P.GroupDesc(nd, [((8, 16), "f32"), ((8, 16), "u8")], (8, 16), "f32")
    a, b = where("-inf"), where("0.0")
    assert P.psk_group_source(a) != P.psk_group_source(b)
    ca, cb = P.psk_group_code_object(a), P.psk_group_code_object(b)
    assert ca != cb
    assert P.psk_group_code_object(where("-inf")) == ca
    # constants: the same
    c1 = _desc("%0 = input 0\n%1 = const 2.0\n%2 = mul %0 %1\n", F, (8, 16))
    c2 = _desc("%0 = input 0\n%1 = const 3.0\n%2 = mul %0 %1\n", F, (8, 16))
    assert P.psk_group_code_object(c1) != P.psk_group_code_object(c2)


def test_strided_inputs_host(lib):
    """Strided input descriptors: a transposed or sliced view is described in
    place; vector accesses only where every per-element input has a unit
    last-axis step and vector-aligned rows; dense strides given explicitly
    are the dense layout; the strides are part of the kernel's key."""
    from synth import configs as C
    R, N = 64, 512
    soft = C.softmax_dag(0.125)
    dense = P.Group(soft, [((R, N), "f32")], (R, N), "f32")
    given = P.Group(soft, [((R, N), "f32", (N, 1))], (R, N), "f32")
    assert dense.info.kernel == given.info.kernel and dense.info.vec == 4
    sliced = P.Group(soft, [((R, N), "f32", (2 * N, 1))], (R, N), "f32")
    assert sliced.info.vec == 4 and sliced.info.kernel != dense.info.kernel
    odd = P.Group(soft, [((R, N), "f32", (N + 2, 1))], (R, N), "f32")        # rows not at whole vectors
    transposed = P.Group(soft, [((R, N), "f32", (1, R))], (R, N), "f32")
    assert odd.info.vec == 1 and transposed.info.vec == 1
    # an expanded [R, 1] input (stride 0 along the row) is one value a row
    d = _desc("%0 = input 0\n%1 = input 1\n%2 = add %0 %1\n", [((R, N), "f32"), ((R, N), "f32", (1, 0))], (R, N))
    src = P.psk_group_source(d)
    assert "xr1" in src
    # refusals: negative strides, strided outputs and extra outputs, tree leaves read with a step
    neg = _desc("%0 = input 0\n%1 = neg %0\n", [((R, N), "f32", (N, 1))], (R, N))
    neg.desc.inputs[0].stride[1] = -1
    _refused(neg, P.PSK_E_SHAPE)
    with pytest.raises(ValueError):
        P.tensor_desc((R, N), "f32", (N, -1))
    nd = parse_dag("%0 = input 0\n%1 = neg %0\n")
    bad_out = P.GroupDesc(nd, F, (8, 16), "f32")
    bad_out.desc.out.stride[0], bad_out.desc.out.stride[1] = 32, 1
    _refused(bad_out, P.PSK_E_UNSUPPORTED)
    extra = P.GroupDesc(parse_dag("%0 = input 0\n%1 = neg %0\n%2 = neg %1\n"), F, (8, 16), "f32",
                        extras=[(1, (8, 16), "f32")])
    extra.desc.extra_out[0].stride[0], extra.desc.extra_out[0].stride[1] = 16, 2
    _refused(extra, P.PSK_E_UNSUPPORTED)
    tree = P.GroupDesc(C.tree_sgd_dag(), [((1,), "f32", (2,)), ((1,), "f32"), ((), "f32")], (1,), "f32",
                       flags=P.PSK_GROUP_TREE)
    _refused(tree, P.PSK_E_UNSUPPORTED)
    # the binding refuses all-zero strides of a tensor larger than one element
    with pytest.raises(ValueError):
        P.tensor_desc((4, 8), "f32", (0, 0))


def test_strided_inputs_compile(lib, tmp_path):
    """Element-path and vector-path strided kernels, and a 64-bit offset when
    a view's span passes 2^31 elements, compile for gfx950."""
    from synth import configs as C
    for name, spec, out in [("transposed", ((512, 384), "bf16", (1, 512)), (512, 384)),
                            ("sliced", ((512, 384), "bf16", (1024, 1)), (512, 384)),
                            ("huge_span", ((2, 8), "f32", (1 << 31, 1)), (2, 8))]:
        d = P.GroupDesc(C.softmax_dag(0.125), [spec], out, spec[1])
        src = P.psk_group_source(d)
        if name == "huge_span":
            assert "long long" in src[src.index('extern "C"'):]
        asm, _ = _isa(P.psk_group_code_object(d), tmp_path, name)
        assert "scratch_" not in asm


def test_stored_bf16_member_rounded_before_its_readers_in_skipping_branches(lib):
    """Where a kernel skips refused vectors, the allowed ones are computed in
    a branch of their own; a member stored as bf16 is rounded right after
    it is computed there, before the members that read it."""
    from synth import configs as C
    dag = C.softmax_causal_dag(0.125, 256)        # %2 scaled scores, %3 the causal mask reading them
    src = P.psk_group_source(P.GroupDesc(dag, [((64, 1000), "f32")], (64, 1000), "f32",
                                         extras=[(2, (64, 1000), "bf16")]))
    body = src[src.index('extern "C"'):]
    branch = body[body.index("    if ("):]
    assert branch.index("v2_0 = psk_rt(v2_0);") < branch.index("v3_0 = ")
