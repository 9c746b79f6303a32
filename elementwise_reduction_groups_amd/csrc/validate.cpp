// Descriptor validation and analysis of a fusion group.  Host-only integer
// code: no HIP call, so it runs (and is tested) without a GPU.
//
// The checks follow the membership conditions of a group (presk manual,
// "PSK-Realize", section "What a group is"): elementwise members, one result
// type for the element members (inputs may be smaller and broadcast), every
// member but the root read only by members, at most 64 members, and pow n
// with n > 2 never joining a group.  Row reductions are last-axis keepdim
// reductions whose value feeds an elementwise epilogue (poot, "Fusion and
// Planning", section "Reduction-rooted regions").
#include <algorithm>
#include <cmath>
#include <cstring>
#include <sstream>

#include "psk_internal.h"

namespace psk {

bool op_is_leaf(int op) { return op == PSK_OP_INPUT || op == PSK_OP_CONST; }

bool op_is_row(int op) { return op == PSK_OP_ROW_MAX || op == PSK_OP_ROW_SUM || op == PSK_OP_ROW_MEAN; }

bool op_is_boundary(int op)
{
    return op == PSK_OP_REDUCE || op == PSK_OP_CONTRACT || op == PSK_OP_CAST || op == PSK_OP_OPAQUE;
}

bool op_is_elementwise(int op)
{
    switch (op) {
    case PSK_OP_ADD: case PSK_OP_SUB: case PSK_OP_MUL: case PSK_OP_DIV: case PSK_OP_MAX: case PSK_OP_MIN:
    case PSK_OP_NEG: case PSK_OP_ABS: case PSK_OP_EXP: case PSK_OP_LOG: case PSK_OP_SQRT: case PSK_OP_TANH:
    case PSK_OP_ERF: case PSK_OP_GELU: case PSK_OP_SQRTABS: case PSK_OP_POW2: case PSK_OP_POWN:
    case PSK_OP_SELECT: case PSK_OP_CAUSAL_MASK: case PSK_OP_WHERE:
        return true;
    default:
        return false;
    }
}

int op_arity(int op)
{
    switch (op) {
    case PSK_OP_INPUT: case PSK_OP_CONST: return 0;
    case PSK_OP_ADD: case PSK_OP_SUB: case PSK_OP_MUL: case PSK_OP_DIV: case PSK_OP_MAX: case PSK_OP_MIN:
    case PSK_OP_CONTRACT: case PSK_OP_WHERE:
        return 2;
    case PSK_OP_SELECT: return 3;
    case PSK_OP_OPAQUE: return -1;  // any number of operands
    default: return 1;
    }
}

const char* op_name(int op)
{
    switch (op) {
    case PSK_OP_INPUT: return "input"; case PSK_OP_CONST: return "const";
    case PSK_OP_ADD: return "add"; case PSK_OP_SUB: return "sub"; case PSK_OP_MUL: return "mul";
    case PSK_OP_DIV: return "div"; case PSK_OP_MAX: return "max"; case PSK_OP_MIN: return "min";
    case PSK_OP_NEG: return "neg"; case PSK_OP_ABS: return "abs"; case PSK_OP_EXP: return "exp";
    case PSK_OP_LOG: return "log"; case PSK_OP_SQRT: return "sqrt"; case PSK_OP_TANH: return "tanh";
    case PSK_OP_ERF: return "erf"; case PSK_OP_GELU: return "gelu"; case PSK_OP_SQRTABS: return "sqrtabs";
    case PSK_OP_POW2: return "pow2"; case PSK_OP_POWN: return "pown"; case PSK_OP_SELECT: return "select";
    case PSK_OP_CAUSAL_MASK: return "causal_mask"; case PSK_OP_WHERE: return "where";
    case PSK_OP_ROW_MAX: return "row_max";
    case PSK_OP_ROW_SUM: return "row_sum"; case PSK_OP_ROW_MEAN: return "row_mean";
    case PSK_OP_REDUCE: return "reduce"; case PSK_OP_CONTRACT: return "contract"; case PSK_OP_CAST: return "cast";
    case PSK_OP_OPAQUE: return "opaque";
    default: return "?";
    }
}

static bool dtype_ok(int32_t d) { return d == PSK_F32 || d == PSK_BF16; }
static bool input_dtype_ok(int32_t d) { return dtype_ok(d) || d == PSK_U8; }

static std::string at(int i) { return "node " + std::to_string(i) + ": "; }

// The descriptor's rank where it can index its arrays (callers check the
// rank itself where it matters).
static int rank_of(const psk_tensor_desc& t) { return std::max(0, std::min<int>(t.rank, PSK_MAX_RANK)); }

// Row-major strides of a shape (elements).
static void dense_strides(const psk_tensor_desc& t, int64_t* st)
{
    int64_t s = 1;
    for (int d = rank_of(t) - 1; d >= 0; --d) {
        st[d] = s;
        s *= t.shape[d] > 0 ? t.shape[d] : 1;
    }
}

// Strides were given (some entry within the rank is nonzero) and differ
// from the dense ones on an axis longer than 1.
static bool strides_given(const psk_tensor_desc& t)
{
    for (int d = 0; d < rank_of(t); ++d)
        if (t.stride[d] != 0) return true;
    return false;
}

static bool strides_dense(const psk_tensor_desc& t)
{
    if (!strides_given(t)) return true;
    int64_t st[PSK_MAX_RANK];
    dense_strides(t, st);
    for (int d = 0; d < rank_of(t); ++d)
        if (t.shape[d] > 1 && t.stride[d] != st[d]) return false;
    return true;
}

// Outputs (and tree-mapped inputs) are dense: zero or the dense strides.
static psk_status dense_only(const psk_tensor_desc& t, const std::string& what)
{
    for (int d = 0; d < rank_of(t); ++d)
        if (t.stride[d] < 0) return fail(PSK_E_SHAPE, what + ": negative stride");
    if (!strides_dense(t)) return fail(PSK_E_UNSUPPORTED, what + " must be dense (row-major strides)");
    return PSK_OK;
}

bool inputs_vector_ok(const Analysis& an, int V)
{
    for (const InputInfo& in : an.inputs) {
        if (!in.used || in.kind == InKind::Scalar || in.kind == InKind::RowConst) continue;
        if (in.stride4[3] != 1) return false;
        for (int d = 0; d < 3; ++d)
            if (in.stride4[d] % V != 0) return false;
    }
    return true;
}

psk_status analyse(const psk_group_desc* desc, Analysis& an)
{
    if (!desc)
        return fail(PSK_E_NULL, "group descriptor is NULL");
    if (desc->n_nodes < 1 || desc->n_nodes > PSK_MAX_NODES)
        return fail(PSK_E_CAP, "n_nodes must be in 1.." + std::to_string(PSK_MAX_NODES));
    if (!desc->nodes)
        return fail(PSK_E_NULL, "nodes is NULL");
    if (desc->n_inputs < 0 || desc->n_inputs > PSK_MAX_INPUTS)
        return fail(PSK_E_CAP, "n_inputs must be in 0.." + std::to_string(PSK_MAX_INPUTS));
    if (desc->n_inputs > 0 && !desc->inputs)
        return fail(PSK_E_NULL, "inputs is NULL");
    if (desc->arith != PSK_F32)
        return fail(PSK_E_TYPE, "the arithmetic type must be f32 (bf16 is storage only)");
    if (desc->flags & ~(PSK_GROUP_TREE | PSK_GROUP_ONLINE))
        return fail(PSK_E_UNSUPPORTED, "unknown flags");

    // ---- output
    const psk_tensor_desc& o = desc->out;
    if (o.rank < 1 || o.rank > PSK_MAX_RANK)
        return fail(PSK_E_SHAPE, "output rank must be in 1..4");
    {
        psk_status st = dense_only(o, "the output");
        if (st != PSK_OK) return st;
    }
    if (!dtype_ok(o.dtype))
        return fail(PSK_E_TYPE, "output storage type must be f32 or bf16");
    an = Analysis();
    an.out_dtype = (psk_dtype)o.dtype;
    an.out_rank = o.rank;
    for (int d = 0; d < o.rank; ++d) {
        if (o.shape[d] < 0)
            return fail(PSK_E_SHAPE, "output shape has a negative size");
        an.out_shape4[PSK_MAX_RANK - o.rank + d] = o.shape[d];
    }
    an.cols = an.out_shape4[3];
    an.rows = an.out_shape4[0] * an.out_shape4[1] * an.out_shape4[2];
    an.numel = an.rows * an.cols;
    if (an.numel > (int64_t(1) << 40))
        return fail(PSK_E_SHAPE, "output larger than 2^40 elements");

    // ---- inputs
    an.inputs.resize(desc->n_inputs);
    for (int k = 0; k < desc->n_inputs; ++k) {
        const psk_tensor_desc& t = desc->inputs[k];
        InputInfo& in = an.inputs[k];
        if (t.rank < 0 || t.rank > PSK_MAX_RANK)
            return fail(PSK_E_SHAPE, "input " + std::to_string(k) + ": rank must be in 0..4");
        if ((desc->flags & PSK_GROUP_TREE) && (t.rank > 1 || o.rank != 1))
            return fail(PSK_E_SHAPE, "a tree-mapped group has a rank-1 output and inputs of rank 1 (per "
                                     "element) or 0 (per tree)");
        if (t.rank > o.rank)
            return fail(PSK_E_BROADCAST, "input " + std::to_string(k) + ": rank above the output's");
        if (!input_dtype_ok(t.dtype))
            return fail(PSK_E_TYPE, "input " + std::to_string(k) + ": storage type must be f32, bf16 or u8 (a mask)");
        if (t.dtype == PSK_U8 && (desc->flags & PSK_GROUP_TREE))
            return fail(PSK_E_TYPE, "input " + std::to_string(k) + ": a tree-mapped group has no mask inputs");
        in.dtype = (psk_dtype)t.dtype;
        in.rank = t.rank;
        for (int d = 0; d < t.rank; ++d) {
            if (t.shape[d] < 0)
                return fail(PSK_E_SHAPE, "input " + std::to_string(k) + ": negative size");
            if (t.stride[d] < 0)
                return fail(PSK_E_SHAPE, "input " + std::to_string(k) + ": negative stride");
            in.shape[d] = t.shape[d];
            in.aligned[PSK_MAX_RANK - t.rank + d] = t.shape[d];
        }
        // each output axis's step in this input: the given strides (all zero
        // means dense), 0 where the input broadcasts
        int64_t dense[PSK_MAX_RANK] = {0, 0, 0, 0};
        dense_strides(t, dense);
        const bool given = strides_given(t);
        in.strided = !strides_dense(t);
        for (int d = 0; d < t.rank; ++d)
            in.stride4[PSK_MAX_RANK - t.rank + d] = t.shape[d] == 1 ? 0 : (given ? t.stride[d] : dense[d]);
        in.numel = 1;
        in.span = 1;
        for (int d = 0; d < PSK_MAX_RANK; ++d) {
            if (in.aligned[d] == 0) in.numel = in.span = 0;
            if (in.stride4[d] != 0) {
                in.numel *= in.aligned[d];
                in.span += (in.aligned[d] - 1) * in.stride4[d];
            }
        }
        if (in.numel == 0) in.span = 0;
        an.max_span = std::max(an.max_span, in.span);
        if (desc->flags & PSK_GROUP_TREE) {
            // leaf-mapped: rank 1 is one element per leaf element, rank 0 one
            // value for the whole tree; lengths are the leaves'
            if (t.rank > 1)
                return fail(PSK_E_SHAPE, "a tree-mapped group's inputs have rank 1 (per element) or 0 (per tree)");
            if (given && t.rank == 1 && t.stride[0] != 1)
                return fail(PSK_E_UNSUPPORTED, "input " + std::to_string(k) + ": a tree-mapped group reads its "
                                               "leaves densely");
            in.kind = t.rank == 0 ? InKind::Scalar : InKind::Full;
            continue;
        }
        bool same = true;
        for (int d = 0; d < PSK_MAX_RANK; ++d) {
            int64_t a = in.aligned[d], od = an.out_shape4[d];
            if (a != od && a != 1)
                return fail(PSK_E_BROADCAST, "input " + std::to_string(k) + ": axis " + std::to_string(d) +
                                                 " of length " + std::to_string(a) + " does not broadcast to " +
                                                 std::to_string(od) + " (an input may not widen the output)");
            if (a != od) same = false;
        }
        const bool lead0 = in.stride4[0] == 0 && in.stride4[1] == 0 && in.stride4[2] == 0;
        if (lead0 && in.stride4[3] == 0)
            in.kind = InKind::Scalar;
        else if (in.stride4[3] == 0)
            in.kind = InKind::RowConst;
        else if (same && !in.strided)
            in.kind = InKind::Full;
        else if (lead0)
            in.kind = InKind::ColVec;
        else
            in.kind = InKind::General;
    }

    // ---- nodes: ops, operands, order
    const int n = desc->n_nodes;
    an.nodes.assign(desc->nodes, desc->nodes + n);
    an.n_readers.assign(n, 0);
    for (int i = 0; i < n; ++i) {
        const psk_node& nd = an.nodes[i];
        if (op_is_boundary(nd.op))
            return fail(PSK_E_OP, at(i) + std::string(op_name(nd.op)) +
                                      " is a group boundary (reduction, contraction or cast), not a member");
        if (!op_is_leaf(nd.op) && !op_is_elementwise(nd.op) && !op_is_row(nd.op))
            return fail(PSK_E_OP, at(i) + "unknown op " + std::to_string(nd.op));
        int ar = op_arity(nd.op);
        const int32_t opnd[3] = {nd.a, nd.b, nd.c};
        for (int k = 0; k < 3; ++k) {
            if (k < ar) {
                if (opnd[k] < 0 || opnd[k] >= i)
                    return fail(PSK_E_ORDER, at(i) + "operand " + std::to_string(k) +
                                                 " must name an earlier node, got " + std::to_string(opnd[k]));
                an.n_readers[opnd[k]]++;
            } else if (opnd[k] != -1) {
                return fail(PSK_E_OP, at(i) + std::string(op_name(nd.op)) + " takes " + std::to_string(ar) +
                                          " operand(s); unused operands must be -1");
            }
        }
        if (nd.op == PSK_OP_INPUT && (nd.iparam < 0 || nd.iparam >= desc->n_inputs))
            return fail(PSK_E_OP, at(i) + "input slot " + std::to_string(nd.iparam) + " out of range");
        if (nd.op == PSK_OP_POWN && (nd.iparam < 0 || nd.iparam > 64))
            return fail(PSK_E_OP, at(i) + "pown exponent must be in 0..64");
        if (nd.op == PSK_OP_CAUSAL_MASK && nd.iparam < 1)
            return fail(PSK_E_OP, at(i) + "causal_mask period must be >= 1");
        if (!op_is_leaf(nd.op))
            an.members++;
    }
    // a mask (u8 input) is read only as the mask of a WHERE, and a WHERE's
    // mask is a mask input
    for (int i = 0; i < n; ++i) {
        const psk_node& nd = an.nodes[i];
        auto is_mask = [&](int j) {
            return an.nodes[j].op == PSK_OP_INPUT && desc->inputs[an.nodes[j].iparam].dtype == PSK_U8;
        };
        const int ar = op_arity(nd.op);
        const int32_t opnd[3] = {nd.a, nd.b, nd.c};
        for (int k = 0; k < ar; ++k) {
            const bool mask_slot = nd.op == PSK_OP_WHERE && k == 0;
            if (is_mask(opnd[k]) != mask_slot)
                return fail(PSK_E_TYPE, at(i) + (mask_slot ? "the first operand of where must be a mask (u8) input"
                                                           : "a mask (u8 input) enters no arithmetic; only where reads it"));
        }
    }
    if (an.members > PSK_MAX_MEMBERS)
        return fail(PSK_E_CAP, "group has " + std::to_string(an.members) +
                                   " members; past 64 a group stops growing");
    if (desc->root < 0 || desc->root >= n)
        return fail(PSK_E_ROOT, "root index out of range");
    an.root = desc->root;
    if (op_is_leaf(an.nodes[an.root].op))
        return fail(PSK_E_ROOT, "the root must be a member, not an input or a constant");
    if (an.n_readers[an.root] != 0)
        return fail(PSK_E_ROOT, "the root is read by another node");
    // ---- extra outputs: members stored besides the root
    if (desc->n_extra < 0 || desc->n_extra > PSK_MAX_EXTRA)
        return fail(PSK_E_CAP, "n_extra must be in 0.." + std::to_string(PSK_MAX_EXTRA));
    if (desc->n_extra > 0 && (!desc->extra_root || !desc->extra_out))
        return fail(PSK_E_NULL, "extra_root or extra_out is NULL");
    an.stored.assign(n, 0);
    for (int k = 0; k < desc->n_extra; ++k) {
        const int i = desc->extra_root[k];
        if (i < 0 || i >= n) return fail(PSK_E_ROOT, "extra output " + std::to_string(k) + ": node out of range");
        if (op_is_leaf(an.nodes[i].op))
            return fail(PSK_E_ROOT, "extra output " + std::to_string(k) + ": an input or a constant is not stored");
        if (i == an.root || an.stored[i])
            return fail(PSK_E_ROOT, "extra output " + std::to_string(k) + ": node " + std::to_string(i) +
                                        " is already an output");
        if (!dtype_ok(desc->extra_out[k].dtype))
            return fail(PSK_E_TYPE, "extra output " + std::to_string(k) + ": storage type must be f32 or bf16");
        {
            psk_status st = dense_only(desc->extra_out[k], "extra output " + std::to_string(k));
            if (st != PSK_OK) return st;
        }
        an.stored[i] = k + 1;
        an.extras.push_back({i, (psk_dtype)desc->extra_out[k].dtype, false});
    }
    for (int i = 0; i < n; ++i)
        if (i != an.root && !an.stored[i] && an.n_readers[i] == 0 && !op_is_leaf(an.nodes[i].op))
            return fail(PSK_E_ROOT, at(i) + "a second unread member: a group has one root (store it as an "
                                            "extra output to keep it)");
    // reachability from the root and the extra outputs
    an.needed.assign(n, 0);
    an.needed[an.root] = 1;
    for (auto& x : an.extras) an.needed[x.node] = 1;
    for (int i = n - 1; i >= 0; --i) {
        if (!an.needed[i]) continue;
        const psk_node& nd = an.nodes[i];
        int ar = op_arity(nd.op);
        const int32_t opnd[3] = {nd.a, nd.b, nd.c};
        for (int k = 0; k < ar; ++k) an.needed[opnd[k]] = 1;
    }
    for (int i = 0; i < n; ++i)
        if (!an.needed[i])
            return fail(PSK_E_DEAD, at(i) + "not read on any path to the root or a stored value (dead code)");
    for (int i = 0; i < n; ++i)
        if (an.nodes[i].op == PSK_OP_POWN && an.nodes[i].iparam > 2 && an.members > 1)
            return fail(PSK_E_OP, at(i) + "pow n with n > 2 never joins a group");

    // ---- online normalizer: ROW_SUM(EXP(SUB(y, ROW_MAX(y)))), y an element
    // value read through exactly these nodes' operands.  Not where the
    // maximum, the difference or the exponential is read rounded (stored as
    // bf16): the maximum's pass would sum exponentials that the group's
    // readers never see.
    an.online_max.assign(n, -1);
    an.online_sum.assign(n, -1);
    if (desc->flags & PSK_GROUP_ONLINE) {
        if (desc->flags & PSK_GROUP_TREE)
            return fail(PSK_E_UNSUPPORTED, "the online normalizer needs row reductions; a tree-mapped group has none");
        for (int i = 0; i < n; ++i) {
            const psk_node& s = an.nodes[i];
            if (s.op != PSK_OP_ROW_SUM) continue;
            const psk_node& e = an.nodes[s.a];
            if (e.op != PSK_OP_EXP) continue;
            const psk_node& d = an.nodes[e.a];
            if (d.op != PSK_OP_SUB) continue;
            const psk_node& m = an.nodes[d.b];
            if (m.op != PSK_OP_ROW_MAX || m.a != d.a || an.online_sum[d.b] >= 0) continue;
            if (an.rounded(d.b) || an.rounded(e.a) || an.rounded(s.a)) continue;
            an.online_max[i] = d.b;
            an.online_sum[d.b] = i;
        }
        bool any = false;
        for (int i = 0; i < n; ++i) any = any || an.online_max[i] >= 0;
        if (!any)
            return fail(PSK_E_UNSUPPORTED, "PSK_GROUP_ONLINE: no row sum of exp(y - row_max(y)) in the group");
    }

    // ---- row-level values and reduction depth
    an.is_row.assign(n, 0);
    an.depth.assign(n, 0);
    for (int i = 0; i < n; ++i) {
        const psk_node& nd = an.nodes[i];
        int ar = op_arity(nd.op);
        const int32_t opnd[3] = {nd.a, nd.b, nd.c};
        int dep = 0;
        for (int k = 0; k < ar; ++k) dep = std::max(dep, an.depth[opnd[k]]);
        if (nd.op == PSK_OP_INPUT) {
            InputInfo& in = an.inputs[nd.iparam];
            in.used = true;
            an.is_row[i] = (in.kind == InKind::Scalar || in.kind == InKind::RowConst);
        } else if (nd.op == PSK_OP_CONST) {
            an.is_row[i] = 1;
        } else if (op_is_row(nd.op)) {
            if (an.is_row[nd.a])
                return fail(PSK_E_ROW, at(i) + "a row reduction must reduce an element value, not a row value");
            an.is_row[i] = 1;
            // an online sum finishes with its maximum, in the pass over y
            dep = an.online_max[i] >= 0 ? an.depth[an.online_max[i]] : an.depth[nd.a] + 1;
            an.n_reductions++;
        } else if (nd.op == PSK_OP_CAUSAL_MASK) {
            an.is_row[i] = 0;
        } else {
            bool all_row = true;
            for (int k = 0; k < ar; ++k) all_row = all_row && an.is_row[opnd[k]];
            an.is_row[i] = all_row;
        }
        an.depth[i] = dep;
    }
    // extra outputs' shapes: the output's (element value) or the output's
    // with a last axis of 1 (one value per row)
    for (int k = 0; k < (int)an.extras.size(); ++k) {
        Analysis::Extra& x = an.extras[k];
        const psk_tensor_desc& t = desc->extra_out[k];
        x.per_row = an.is_row[x.node] != 0;
        bool ok = t.rank == desc->out.rank;
        for (int d = 0; ok && d < t.rank; ++d) {
            int64_t want = (x.per_row && d == t.rank - 1) ? 1 : desc->out.shape[d];
            ok = t.shape[d] == want;
        }
        if (!ok)
            return fail(PSK_E_SHAPE, "extra output " + std::to_string(k) + ": shape must be the output's" +
                                         std::string(x.per_row ? " with a last axis of 1 (the node is one value "
                                                                 "per row)" : " (the node is an element value)"));
        if (x.per_row && (desc->flags & PSK_GROUP_TREE))
            return fail(PSK_E_SHAPE, "extra output " + std::to_string(k) + ": a tree-mapped group stores element "
                                         "values only");
    }
    an.row_kind = an.n_reductions > 0;
    an.flags = desc->flags;
    an.tree = (desc->flags & PSK_GROUP_TREE) != 0;
    if (an.tree) {
        if (an.out_rank != 1) return fail(PSK_E_SHAPE, "a tree-mapped group has a rank-1 output");
        for (int k = 0; k < desc->n_inputs; ++k)
            if (desc->inputs[k].rank > 1)
                return fail(PSK_E_SHAPE, "a tree-mapped group's inputs have rank 1 (per element) or 0 (per tree)");
        if (an.row_kind) return fail(PSK_E_ROW, "a tree-mapped group has no row reduction");
        for (int i = 0; i < n; ++i)
            if (an.nodes[i].op == PSK_OP_CAUSAL_MASK)
                return fail(PSK_E_OP, at(i) + "a tree-mapped group has no rows for a causal mask");
    }
    an.phases = an.depth[an.root];
    for (auto& x : an.extras) an.phases = std::max(an.phases, an.depth[x.node]);
    if (an.is_row[an.root] && an.cols > 1)
        return fail(PSK_E_ROW, "the root is one value per row but the output has " + std::to_string(an.cols) +
                                   " columns: a reduction cannot be the stored value here");
    if (an.row_kind && an.cols > (int64_t(1) << 30))
        return fail(PSK_E_UNSUPPORTED, "row groups over rows longer than 2^30 are not implemented");

    // ---- inputs read only where a causal mask allows them
    // A value is irrelevant at refused positions when every reader is a
    // causal mask or an element member whose own value is irrelevant there;
    // the root is stored everywhere.  Only when every mask shares one period.
    int period = -1;
    bool one_period = true;
    for (int i = 0; i < n; ++i)
        if (an.nodes[i].op == PSK_OP_CAUSAL_MASK) {
            if (period < 0) period = an.nodes[i].iparam;
            else if (period != an.nodes[i].iparam) one_period = false;
        }
    if (period > 0 && one_period) {
        std::vector<std::vector<int>> readers(n);
        for (int i = 0; i < n; ++i) {
            const psk_node& nd = an.nodes[i];
            int ar = op_arity(nd.op);
            const int32_t opnd[3] = {nd.a, nd.b, nd.c};
            for (int k = 0; k < ar; ++k) readers[opnd[k]].push_back(i);
        }
        an.mask_period = period;
        std::vector<char>& irrelevant = an.irrelevant;
        irrelevant.assign(n, 0);
        for (int i = n - 1; i >= 0; --i) {
            // stored values are written everywhere, refused positions included
            if (i == an.root || an.stored[i] || readers[i].empty() || an.is_row[i]) continue;
            bool irr = true;
            for (int r : readers[i]) {
                const psk_node& rd = an.nodes[r];
                if (rd.op == PSK_OP_CAUSAL_MASK) continue;
                if (op_is_row(rd.op) || an.is_row[r] || !irrelevant[r]) { irr = false; break; }
            }
            irrelevant[i] = irr;
        }
        // An element value is uniform at refused positions when it is a
        // causal mask (-inf there) or an elementwise member whose operands
        // are all uniform there or one value per row.
        an.uniform.assign(n, 0);
        for (int i = 0; i < n; ++i) {
            const psk_node& nd = an.nodes[i];
            if (an.is_row[i] || op_is_leaf(nd.op) || op_is_row(nd.op)) continue;
            if (nd.op == PSK_OP_CAUSAL_MASK) { an.uniform[i] = 1; continue; }
            int ar = op_arity(nd.op);
            const int32_t opnd[3] = {nd.a, nd.b, nd.c};
            bool u = true;
            for (int k = 0; k < ar; ++k) u = u && (an.is_row[opnd[k]] || an.uniform[opnd[k]]);
            an.uniform[i] = u;
        }
        for (auto& in : an.inputs) in.mask_guarded = in.used;
        for (int i = 0; i < n; ++i)
            if (an.nodes[i].op == PSK_OP_INPUT) {
                InputInfo& in = an.inputs[an.nodes[i].iparam];
                if (!irrelevant[i] || in.kind == InKind::Scalar || in.kind == InKind::RowConst)
                    in.mask_guarded = false;
            }
    }

    // ---- inputs read only where a byte mask allows them
    // The same analysis for WHERE, when there is no causal mask and every
    // WHERE reads one mask input: a value read only as a WHERE's value (or
    // by members themselves irrelevant there) is not needed where the mask
    // refuses, and its vector is loaded only when a mask byte under it
    // allows.
    if (period < 0) {
        int mask_slot = -1;
        bool one_mask = true;
        for (int i = 0; i < n; ++i)
            if (an.nodes[i].op == PSK_OP_WHERE) {
                const int slot = an.nodes[an.nodes[i].a].iparam;
                if (mask_slot < 0) mask_slot = slot;
                else if (mask_slot != slot) one_mask = false;
            }
        if (mask_slot >= 0 && one_mask) {
            std::vector<std::vector<int>> readers(n);
            for (int i = 0; i < n; ++i) {
                const psk_node& nd = an.nodes[i];
                int ar = op_arity(nd.op);
                const int32_t opnd[3] = {nd.a, nd.b, nd.c};
                for (int k = 0; k < ar; ++k) readers[opnd[k]].push_back(i);
            }
            std::vector<char> irrelevant(n, 0);
            for (int i = n - 1; i >= 0; --i) {
                if (i == an.root || an.stored[i] || readers[i].empty() || an.is_row[i]) continue;
                if (an.nodes[i].op == PSK_OP_INPUT && an.nodes[i].iparam == mask_slot) continue;
                bool irr = true;
                for (int r : readers[i]) {
                    const psk_node& rd = an.nodes[r];
                    if (rd.op == PSK_OP_WHERE && rd.b == i) continue;
                    if (op_is_row(rd.op) || an.is_row[r] || !irrelevant[r]) { irr = false; break; }
                }
                irrelevant[i] = irr;
            }
            an.irrelevant = irrelevant;
            // uniform where the mask refuses: a WHERE (its fill value), and
            // members whose operands are uniform there or one value per row
            an.uniform.assign(n, 0);
            for (int i = 0; i < n; ++i) {
                const psk_node& nd = an.nodes[i];
                if (an.is_row[i] || op_is_leaf(nd.op) || op_is_row(nd.op)) continue;
                if (nd.op == PSK_OP_WHERE) { an.uniform[i] = 1; continue; }
                int ar = op_arity(nd.op);
                const int32_t opnd[3] = {nd.a, nd.b, nd.c};
                bool u = true;
                for (int k = 0; k < ar; ++k) u = u && (an.is_row[opnd[k]] || an.uniform[opnd[k]]);
                an.uniform[i] = u;
            }
            bool any = false;
            for (auto& in : an.inputs) in.mask_guarded = in.used;
            for (int i = 0; i < n; ++i)
                if (an.nodes[i].op == PSK_OP_INPUT) {
                    InputInfo& in = an.inputs[an.nodes[i].iparam];
                    if (!irrelevant[i] || in.kind == InKind::Scalar || in.kind == InKind::RowConst)
                        in.mask_guarded = false;
                }
            for (auto& in : an.inputs) any = any || in.mask_guarded;
            an.where_mask = mask_slot;
            (void)any;
        }
    }
    return PSK_OK;
}

}  // namespace psk
