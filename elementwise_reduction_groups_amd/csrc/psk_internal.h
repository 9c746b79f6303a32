// Internal declarations of the psk_fused library (not part of the C ABI).
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "psk_fused.h"

namespace psk {

// ------------------------------------------------------------------ errors
// Records a message for the calling thread and returns the status.
psk_status fail(psk_status st, const std::string& msg);
void clear_error();

// --------------------------------------------------------------- analysis
enum class InKind : int {
    Scalar = 0,     // every axis broadcast: one value for the whole output
    RowConst = 1,   // last axis broadcast: one value per row
    ColVec = 2,     // only the last axis varies: the same row vector for every row
    General = 3,    // leading axes and the last axis by their strides
    Full = 4        // dense, the output's shape: flat index
};

struct InputInfo {
    psk_dtype dtype = PSK_F32;
    int rank = 0;
    int64_t shape[PSK_MAX_RANK] = {0, 0, 0, 0};
    int64_t aligned[PSK_MAX_RANK] = {1, 1, 1, 1};  // shape right-aligned to the output's 4 axes
    // step of each of the output's 4 axes in elements: 0 where the input
    // broadcasts (a size-1 axis, a stride-0 axis, an axis it does not have)
    int64_t stride4[PSK_MAX_RANK] = {0, 0, 0, 0};
    bool strided = false;        // the descriptor gave strides other than the dense ones
    int64_t numel = 0;           // distinct elements read (the extents of the non-broadcast axes)
    int64_t span = 0;            // 1 + the largest element offset read (0 when empty)
    InKind kind = InKind::Scalar;
    bool used = false;
    bool mask_guarded = false;   // read only where the group's mask (causal or WHERE) allows
};

// Everything the emitter needs to know about a validated group.
struct Analysis {
    std::vector<psk_node> nodes;
    int root = -1;
    int members = 0;
    int n_reductions = 0;
    int phases = 0;                     // max reduction depth of the root
    std::vector<char> is_row;           // node value is one per row
    std::vector<int> depth;             // reduction phases that precede the node
    // online normalizer (PSK_GROUP_ONLINE): node -> the ROW_MAX whose pass
    // also takes this ROW_SUM of exp(y - max) (-1: none); and for a ROW_MAX,
    // the ROW_SUM it carries (-1: none)
    std::vector<int> online_max, online_sum;
    std::vector<int> n_readers;
    std::vector<char> needed;           // reachable from the root
    // causal masks (one period): values at refused positions
    int mask_period = 0;                // 0: no causal mask, or masks of different periods
    int where_mask = -1;                // the input every WHERE reads as its mask (or -1): inputs
                                        // marked mask_guarded are then read only where it allows
    std::vector<char> irrelevant;       // element value never used at a refused position
    std::vector<char> uniform;          // element value at refused positions is one value per row
    std::vector<InputInfo> inputs;
    psk_dtype out_dtype = PSK_F32;
    int out_rank = 1;
    int64_t out_shape4[PSK_MAX_RANK] = {1, 1, 1, 1};  // output right-aligned to 4 axes
    int64_t rows = 0, cols = 0, numel = 0;
    int64_t max_span = 0;               // the largest input span (64-bit indexing beyond 2^31)
    bool row_kind = false;              // has at least one row reduction
    bool tree = false;                  // PSK_GROUP_TREE: mapped over tree leaves
    uint32_t flags = 0;
    // extra outputs: node, storage type, one per row (stored [rows, 1])
    struct Extra {
        int node;
        psk_dtype dtype;
        bool per_row;
    };
    std::vector<Extra> extras;
    std::vector<int> stored;            // node -> 1 + extra index, or 0
    // members that read node i read it rounded to bf16 (a bf16 extra output)
    bool rounded(int i) const { return stored[i] > 0 && extras[stored[i] - 1].dtype == PSK_BF16; }
};

// Validates the descriptor; on success fills `an`.
psk_status analyse(const psk_group_desc* desc, Analysis& an);
// Every input the kernel loads per element takes V-element vector accesses:
// last-axis stride 1 and the other strides multiples of V.
bool inputs_vector_ok(const Analysis& an, int V);

bool op_is_leaf(int op);
bool op_is_elementwise(int op);
bool op_is_row(int op);
bool op_is_boundary(int op);
int op_arity(int op);
const char* op_name(int op);

// ------------------------------------------------------------------- emit
struct KernelPlan {
    int kind = 0;            // 0 pointwise, 1 row, 2 tree-mapped, 3 row tiled (wide rows), 4 split rows
    int vec = 1;             // elements per vector access
    int block = 256;         // threads per workgroup
    int lanes = 64;          // row kernel: lanes per row
    int rows_per_block = 1;  // row kernel
    int nv = 1;              // row kernel: vectors per lane (tiled: per lane per tile)
    int tiles = 0;           // tiled row kernel (kind 3): tiles per row, each phase re-reads the row
    bool tcache = true;      // tiled row kernel: cached (plain) loads before the last phase
    int rcache = 0;          // tiled row kernel: leading tiles whose per-row inputs stay in registers
    int lcache = 0;          // tiled row kernel: the tiles after those whose per-row inputs stay in LDS
    bool alt = true;         // tiled row kernel: odd phases walk the tiles last to first
    int munroll = 1;         // tiled row kernel: unroll of the loop over tiles read from memory
    int lunroll = 1;         // tiled row kernel: unroll of the loop over tiles kept in LDS
    int wpe = 0;             // tiled row kernel: at most this many waves per SIMD (0: no limit)
    int wmin = 0;            // tiled row kernel: registers for at least this many waves per SIMD (0: any)
    int persist = 0;         // row kernel: persistent workgroups per CU (0: one workgroup per row)
    int pf = 1;              // persistent rows: rows whose inputs are loaded ahead of the current one
    int split = 0;           // split rows (kind 4): workgroups that share one row, each a segment of
                             // lanes * nv * vec columns kept in registers
    int exch = 0;            // split rows: row values exchanged per row (one per reduction)
    bool nt = true;          // nontemporal loads and stores
    bool sc1 = false;        // stores of device scope (the sc1 cache policy)
    bool bnt = false;        // nontemporal loads also for inputs read again by other rows (broadcast)
    bool fexp = true;        // exp(y - max y) with f32 results by the split-product exponential
    int ftanh = 1;           // tanh: 1 the emitted one, 2 its branch-free form, 0 the device library's
    bool xcd = true;         // each XCD takes a contiguous eighth of the blocks
    int64_t blocks = 0;      // workgroups that carry work
    int64_t per_xcd = 0;     // blocks per XCD (xcd layout)
    int64_t grid = 0;        // workgroups launched (blocks, padded to 8 * per_xcd)
    std::string key() const;
};

// split_ept: elements a lane holds in a split-rows kernel (-1: the default
// rule, 0: no split rows, > 0: that many)
KernelPlan plan_kernel(const Analysis& an, bool allow_vector, int split_ept = -1);
// a key of PSK_LAYOUT ("key=value,..."), else dflt: launch shapes for measurement
int layout_value(const char* key, int dflt);
// Bytes of scratch (register spills) a compiled code object's kernel uses,
// from its metadata; -1 when the metadata does not say.
int64_t code_scratch_bytes(const std::vector<char>& code);
// HIP source for the group under `plan`, entry point named `kernel_name`.
std::string emit_source(const Analysis& an, const KernelPlan& plan, const std::string& kernel_name);
// Canonical text of the group (what the kernel cache is keyed by).
std::string canonical_text(const Analysis& an);
uint64_t fnv1a(const std::string& s);

// -------------------------------------------------------------------- JIT
// Compile HIP source for gfx950 with hipRTC; returns the code object.
psk_status jit_compile(const std::string& source, const std::string& name, std::vector<char>& code);
extern const char* const kJitOptions[];
extern const int kJitOptionCount;

// -------------------------------------------------------------- partition
psk_status partition(int32_t n, const psk_node* body, const psk_tensor_desc* types, const uint8_t* is_output,
                     uint32_t flags, int32_t* group_of, int32_t* is_root, int32_t* n_groups);
psk_status dispatch_count(int32_t n, const psk_node* body, const psk_tensor_desc* types, const uint8_t* is_output,
                          uint32_t flags, psk_dispatch_report* rep);

// ------------------------------------------------------------------ trees
struct TreePlan {
    std::vector<int64_t> leaf_offset;    // n_leaves + 1
    std::vector<int32_t> chunk_leaf;
    std::vector<int64_t> chunk_start;
    std::vector<int32_t> chunk_count;
};
psk_status plan_tree(const int64_t* numel, int32_t n_leaves, int64_t chunk_elems, TreePlan& plan);

// ------------------------------------------------------------------ AdamW
// f32 scalars of one step, each formed in f64 and rounded once.  rc1 and
// rc2 are the correctly rounded reciprocals of bc1 and bc2 when both lie in
// [2^-40, 2^40] (the kernel then divides by them with one multiply and a
// correction), else 0 (the kernel divides).
struct AdamwScalars {
    float b1, b2, c1, c2, bc1, bc2, lr, eps, wd, rc1, rc2;
};
AdamwScalars adamw_scalars(const psk_adamw_hp& hp);

// Device-side leaf descriptor: input slots theta, g, m, v; output slots
// theta', m', v' (the input's address when updated in place).
struct LeafDev {
    const void* in[4];
    void* out[3];
    int64_t flags;      // bit 0: every slot 16-byte aligned (vector path)
};
// Device-side chunk: `count` elements of leaf `leaf` from element `start`.
struct ChunkDev {
    int32_t leaf;
    int32_t count;
    int64_t start;
};
// Device-side leaf descriptor of any tree: every slot's address.
struct GenLeafDev {
    void* slot[PSK_MAX_SLOTS];
    int64_t flags;      // bit 0: every slot 16-byte aligned
};
static_assert(sizeof(LeafDev) == 64, "LeafDev layout");
static_assert(sizeof(GenLeafDev) == 72, "GenLeafDev layout");
// Launch shape of the AdamW tree kernel: 128 threads, 4 elements each,
// PSK_TREE_CHUNK / 512 workgroups per chunk.  Emitted tree-mapped groups
// choose their own (KernelPlan: block threads, vec elements per thread).
constexpr int kTreeBlock = 128;
constexpr int kTreePer = 4;
constexpr int kTreeSub = PSK_TREE_CHUNK / (kTreeBlock * kTreePer);
static_assert(sizeof(ChunkDev) == 16, "ChunkDev layout");

// Result of a tree-wide clipping pass, in device memory owned by the tree.
struct ClipOut {
    double sumsq;
    float factor;
    float pad;
};

// One launch over every chunk (defined in adamw.hip).  gscale: NULL, or a
// device f32 that multiplies every gradient element first.
psk_status launch_adamw(const LeafDev* d_leaves, const ChunkDev* d_chunks, int64_t n_chunks, int theta_dt,
                        int grad_dt, int mv_dt, const AdamwScalars& s, const float* gscale, void* stream);

// Tree-wide sum of squares of the gradient slot and the clipping factor
// min(1, c / (sqrt(sumsq) + 1e-6)): one launch writes a partial sum per
// chunk into `partials` (n_chunks doubles), a second, one-workgroup launch
// combines them in a fixed order and writes `out`.
psk_status launch_clip(const LeafDev* d_leaves, const ChunkDev* d_chunks, int64_t n_chunks, int grad_dt,
                       double* partials, ClipOut* out, double c, void* stream);

// Library-static device scratch of the clipping pass (defined in adamw.hip):
// room for kStaticChunks partials and one ClipOut on every device; the
// addresses on the current device (looked up once per device).
constexpr int64_t kStaticChunks = int64_t(1) << 20;
constexpr int kMaxScratchDevices = 64;
psk_status static_scratch(double** partials, ClipOut** out);

// --------------------------------------------------------------- counters
void count_launch();
void count_jit(bool hit);

}  // namespace psk
