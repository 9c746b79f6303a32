// Fusion-group partition of a function body.  Host-only integer code.
//
// The pages state what a group is, not how to find one (presk manual,
// "PSK-Realize", section "What a group is"): elementwise members only (a
// reduction ends a group), one result type, every member but the root read
// only by members, at most 64 members, pow n with n > 2 never joining.  The
// partition here is a single scan from the last let to the first: a let
// joins the group all of its readers belong to when the conditions allow,
// otherwise it roots a new group.  A let that is read from outside the group
// must reach memory, so it can only be a root; joining whenever allowed keeps
// every let interior that can be, which gives the fewest groups.
#include <cstring>

#include "psk_internal.h"

namespace psk {

static bool same_type(const psk_tensor_desc& x, const psk_tensor_desc& y)
{
    if (x.rank != y.rank || x.dtype != y.dtype) return false;
    for (int d = 0; d < x.rank; ++d)
        if (x.shape[d] != y.shape[d]) return false;
    return true;
}

static bool same_shape(const psk_tensor_desc& x, const psk_tensor_desc& y)
{
    if (x.rank != y.rank) return false;
    for (int d = 0; d < x.rank; ++d)
        if (x.shape[d] != y.shape[d]) return false;
    return true;
}

// `row` has the shape of `elem` with a last axis of 1 (a value that is one
// per row of elem's rows; its storage type does not matter inside a group)
static bool row_shape_of(const psk_tensor_desc& row, const psk_tensor_desc& elem)
{
    if (row.rank != elem.rank || row.rank < 1 || elem.shape[elem.rank - 1] <= 1) return false;
    for (int d = 0; d + 1 < row.rank; ++d)
        if (row.shape[d] != elem.shape[d]) return false;
    return row.shape[row.rank - 1] == 1;
}

// 0 leaf, 1 elementwise member candidate, 2 boundary (a group of its own),
// 3 last-axis row reduction (a member candidate when rows fuse)
static int node_class(const psk_node& nd, bool rows)
{
    if (op_is_leaf(nd.op)) return 0;
    if (nd.op == PSK_OP_POWN && nd.iparam > 2) return 2;
    if (op_is_elementwise(nd.op)) return 1;
    if (rows && op_is_row(nd.op)) return 3;
    return 2;
}

psk_status partition(int32_t n, const psk_node* body, const psk_tensor_desc* types, const uint8_t* is_output,
                     uint32_t flags, int32_t* group_of, int32_t* is_root, int32_t* n_groups)
{
    if (flags & ~PSK_PARTITION_ROWS) return fail(PSK_E_UNSUPPORTED, "unknown partition flags");
    const bool rows = (flags & PSK_PARTITION_ROWS) != 0;
    if (n < 0) return fail(PSK_E_SHAPE, "negative node count");
    if (n > 0 && (!body || !types || !is_output || !group_of || !is_root))
        return fail(PSK_E_NULL, "psk_partition: a required array is NULL");
    if (!n_groups) return fail(PSK_E_NULL, "psk_partition: n_groups is NULL");
    // readers of every let
    std::vector<std::vector<int32_t>> readers(n);
    for (int32_t i = 0; i < n; ++i) {
        const psk_node& nd = body[i];
        if (!op_is_leaf(nd.op) && !op_is_elementwise(nd.op) && !op_is_row(nd.op) && !op_is_boundary(nd.op))
            return fail(PSK_E_OP, "node " + std::to_string(i) + ": unknown op");
        const int32_t opnd[3] = {nd.a, nd.b, nd.c};
        int ar = op_arity(nd.op);
        for (int k = 0; k < 3; ++k) {
            int32_t a = opnd[k];
            if (ar >= 0 && k >= ar) {
                if (a != -1) return fail(PSK_E_OP, "node " + std::to_string(i) + ": unused operand must be -1");
                continue;
            }
            if (a == -1 && ar < 0) continue;  // opaque: any operand count
            if (a < 0 || a >= i)
                return fail(PSK_E_ORDER, "node " + std::to_string(i) + ": operand must name an earlier node");
            readers[a].push_back(i);
        }
    }
    std::vector<int32_t> gsize, groot;
    std::vector<int32_t> gid(n, -1);
    for (int32_t i = n - 1; i >= 0; --i) {
        is_root[i] = 0;
        int cls = node_class(body[i], rows);
        if (cls == 0) continue;
        int32_t join = -1;
        if ((cls == 1 || cls == 3) && !is_output[i] && !readers[i].empty()) {
            int32_t g = gid[readers[i][0]];
            bool ok = g >= 0;
            for (int32_t r : readers[i]) {
                int rc = node_class(body[r], rows);
                if ((rc != 1 && rc != 3) || gid[r] != g) { ok = false; break; }
            }
            // an element member has the group's type; with rows fused, a
            // value one per row of the group's rows joins as well: a member
            // of row values, or a reduction of a value of the group's shape.
            // A group rooted at a reduction takes no member: the reduction
            // reduces an element value, and its own value is one per row
            // (with a last axis of length 1 the types would agree, but the
            // group the row kernels run would not)
            const psk_tensor_desc& rt = types[groot[g]];
            if (ok && node_class(body[groot[g]], rows) == 3) ok = false;
            bool typed = ok && ((cls == 1 && same_type(types[i], rt)) ||
                                (rows && row_shape_of(types[i], rt) &&
                                 (cls == 1 || same_shape(types[body[i].a], rt))));
            if (typed && gsize[g] < PSK_MAX_MEMBERS) join = g;
        }
        if (join >= 0) {
            gid[i] = join;
            gsize[join]++;
        } else {
            gid[i] = (int32_t)gsize.size();
            gsize.push_back(1);
            groot.push_back(i);
            is_root[i] = 1;
        }
    }
    // number groups by their root's position (roots were found last to first)
    const int32_t G = (int32_t)gsize.size();
    for (int32_t i = 0; i < n; ++i) group_of[i] = gid[i] >= 0 ? G - 1 - gid[i] : -1;
    *n_groups = G;
    return PSK_OK;
}

// ------------------------------------------------------------------ trees
psk_status plan_tree(const int64_t* numel, int32_t n_leaves, int64_t chunk_elems, TreePlan& plan)
{
    if (n_leaves < 0) return fail(PSK_E_SHAPE, "negative leaf count");
    if (n_leaves > 0 && !numel) return fail(PSK_E_NULL, "numel is NULL");
    if (chunk_elems <= 0 || chunk_elems % 8 != 0) return fail(PSK_E_SHAPE, "chunk size must be a positive multiple of 8");
    plan = TreePlan();
    plan.leaf_offset.resize((size_t)n_leaves + 1);
    int64_t off = 0;
    for (int32_t l = 0; l < n_leaves; ++l) {
        if (numel[l] < 0) return fail(PSK_E_SHAPE, "leaf " + std::to_string(l) + ": negative numel");
        plan.leaf_offset[l] = off;
        off += numel[l];
        for (int64_t s = 0; s < numel[l]; s += chunk_elems) {
            plan.chunk_leaf.push_back(l);
            plan.chunk_start.push_back(s);
            plan.chunk_count.push_back((int32_t)std::min<int64_t>(chunk_elems, numel[l] - s));
        }
    }
    plan.leaf_offset[n_leaves] = off;
    if ((int64_t)plan.chunk_leaf.size() > (int64_t(1) << 31) - 1)
        return fail(PSK_E_SHAPE, "too many chunks");
    return PSK_OK;
}

}  // namespace psk

// ------------------------------------------------------------ dispatch count
namespace psk {

static int64_t type_bytes(const psk_tensor_desc& t)
{
    int64_t n = 1;
    for (int d = 0; d < t.rank; ++d) n *= t.shape[d];
    return n * (t.dtype == PSK_BF16 ? 2 : t.dtype == PSK_U8 ? 1 : 4);
}

psk_status dispatch_count(int32_t n, const psk_node* body, const psk_tensor_desc* types, const uint8_t* is_output,
                          uint32_t flags, psk_dispatch_report* rep)
{
    if (!rep) return fail(PSK_E_NULL, "report is NULL");
    std::vector<int32_t> group_of(n > 0 ? n : 1), is_root(n > 0 ? n : 1);
    int32_t G = 0;
    psk_status st = partition(n, body, types, is_output, flags, group_of.data(), is_root.data(), &G);
    if (st != PSK_OK) return st;
    std::memset(rep, 0, sizeof *rep);
    std::vector<int32_t> gsize(G, 0);
    for (int32_t i = 0; i < n; ++i) {
        const psk_node& nd = body[i];
        if (op_is_leaf(nd.op)) continue;
        rep->lets++;
        gsize[group_of[i]]++;
        // unfused: every let a launch that reads its operands and writes its value
        rep->bytes_unfused += type_bytes(types[i]);
        const int32_t opnd[3] = {nd.a, nd.b, nd.c};
        for (int k = 0; k < 3; ++k)
            if (opnd[k] >= 0) rep->bytes_unfused += type_bytes(types[opnd[k]]);
    }
    rep->launches_unfused = rep->lets;
    rep->launches_fused = G;
    for (int32_t g = 0; g < G; ++g)
        if (gsize[g] > 1) rep->fused_groups++;
    // fused: a group reads each value from outside it once and writes its root
    for (int32_t g = 0; g < G; ++g) {
        std::vector<int32_t> seen;
        for (int32_t i = 0; i < n; ++i) {
            if (group_of[i] != g) continue;
            if (is_root[i]) rep->bytes_fused += type_bytes(types[i]);
            const psk_node& nd = body[i];
            const int32_t opnd[3] = {nd.a, nd.b, nd.c};
            for (int k = 0; k < 3; ++k) {
                int32_t a = opnd[k];
                if (a < 0 || group_of[a] == g) continue;
                bool dup = false;
                for (int32_t x : seen) dup = dup || x == a;
                if (!dup) {
                    seen.push_back(a);
                    rep->bytes_fused += type_bytes(types[a]);
                }
            }
        }
    }
    return PSK_OK;
}

}  // namespace psk
