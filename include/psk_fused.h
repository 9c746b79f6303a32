/*
 * psk_fused -- fusion groups as single HIP kernels on MI355X (gfx950).
 *
 * A fusion group is a connected set of elementwise lets of one function that
 * share one loop nest: every member is an elementwise primitive, every member
 * has the same result type (inputs may be smaller and broadcast), and every
 * member but the root is read only by members.  Intermediates stay in
 * registers in the arithmetic type (f32, also for bf16 storage); only the
 * root reaches memory, rounded to its storage type.  Past 64 members a group
 * stops growing.  (presk manual, "PSK-Realize: fusion groups", section "What
 * a group is"; "Native execution", section "The realization".)
 *
 * Three kinds of group run here, each as one kernel launch:
 *   - a pointwise chain (poot, "Fusion and Planning", section "Fusable region
 *     shapes": one thread per element);
 *   - a chain with row-reduction roots: last-axis keepdim reductions whose
 *     results feed an elementwise epilogue in the same kernel, the shape of
 *     softmax and RMSNorm (same page, "Reduction-rooted regions");
 *   - a chain mapped over every leaf of a parameter tree: the AdamW step
 *     (presk manual, "PSK-Realize", section "What a group is", paragraph on
 *     parameter trees; presk language reference, section "Configuration blocks", the optimizer), in one
 *     launch for all leaves, driven by a device-side leaf/chunk table (the
 *     role of poot's launch metadata buffer, "Kernel specialization").
 *
 * Conventions shared by every entry point:
 *   - Every function returns a psk_status; on failure nothing is launched,
 *     no object is created, and psk_last_error() returns a message for the
 *     calling thread.  A request is refused, never silently adjusted
 *     (presk manual, "PSK-Realize", section "The realization plan": an
 *     ill-formed plan is refused).
 *   - Device buffers and streams belong to the caller.  Group and tree
 *     objects, their device tables and compiled kernels belong to the library.
 *   - *_run / *_step calls are asynchronous on the given HIP stream (NULL =
 *     the null stream); buffers must stay alive until the stream has reached
 *     the launch.  Device faults surface at the caller's next synchronisation.
 *   - A launch goes to the calling thread's current HIP device: the stream
 *     and every buffer must belong to it (a tree also checks that it is the
 *     device it was created on).  Buffer extents are the caller's to
 *     guarantee: the library sees addresses, not sizes.
 *   - Kernels never write their inputs unless an output is the same buffer
 *     (in-place).  Outputs are not zeroed beforehand.
 *   - The library allocates no device memory for data in *_run / *_step
 *     (tree tables and the clipping pass's partials are allocated by
 *     psk_tree_create).  The first run of a group on a device loads its
 *     code object there (hipModuleLoadData), and a group with split rows
 *     (see psk_group_check) allocates its exchange buffer there; later runs
 *     only launch, so a group run or an AdamW step may be captured in a HIP
 *     graph once it has run once on that device.
 *   - All functions are thread-safe.
 */
#ifndef PSK_FUSED_H
#define PSK_FUSED_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PSK_VERSION 200
#define PSK_MAX_MEMBERS 64      /* member (non-leaf) nodes per group */
#define PSK_MAX_NODES 256       /* total nodes, leaves included */
#define PSK_MAX_INPUTS 16
#define PSK_MAX_RANK 4
#define PSK_MAX_SLOTS 8
#define PSK_MAX_EXTRA 7         /* stored values besides the root */

typedef enum psk_status {
    PSK_OK = 0,
    PSK_E_NULL = 1,          /* a required pointer is NULL */
    PSK_E_CAP = 2,           /* more than PSK_MAX_MEMBERS members, or too many nodes/inputs */
    PSK_E_ORDER = 3,         /* an operand does not name an earlier node */
    PSK_E_ROOT = 4,          /* the root is not the single unread member */
    PSK_E_DEAD = 5,          /* a node no other node reads (dead code) */
    PSK_E_OP = 6,            /* unknown op, wrong operand count, bad parameter, or a boundary op */
    PSK_E_TYPE = 7,          /* arithmetic type other than f32, unknown storage type, dtype mismatch */
    PSK_E_BROADCAST = 8,     /* an input that would widen the output, or a rank above the output's */
    PSK_E_ROW = 9,           /* misuse of a row reduction */
    PSK_E_ALIGN = 10,        /* a pointer not aligned to its element size */
    PSK_E_ALIAS = 11,        /* an output overlapping an input it may not overlap */
    PSK_E_SHAPE = 12,        /* a negative size, a rank out of range, sizes that disagree */
    PSK_E_UNSUPPORTED = 13,  /* valid, but outside what this library implements */
    PSK_E_JIT = 14,          /* hipRTC could not compile the emitted kernel */
    PSK_E_HIP = 15           /* a HIP runtime call failed */
} psk_status;

/* Storage types.  bf16 is storage only: a load widens exactly (a 16-bit
 * shift), a store rounds to nearest even (presk manual, "Native execution",
 * section "The realization"). */
/* Storage types.  PSK_U8 is an input-only mask: one byte per element, 0
 * refuses and any other value allows (presk language reference, "Typing",
 * builtins: a bool mask is an index buffer of 0 and 1 that enters no
 * arithmetic).  torch.bool and torch.uint8 buffers are such masks. */
typedef enum psk_dtype { PSK_F32 = 0, PSK_BF16 = 1, PSK_U8 = 2 } psk_dtype;

/* Node ops.  Elementwise set after poot "Fusion and Planning" (binary ops;
 * Neg, Exp, Log, Sqrt, Tanh, Erf; Select) and the presk builtins (gelu,
 * abs, max/min, pow n).  Semantics, all in f32:
 *   ADD SUB MUL DIV          IEEE-754 binary32, correctly rounded
 *   MAX MIN                  second operand at a tie (presk language
 *                            reference, section "Typing", builtins)
 *   NEG ABS                  sign operations
 *   EXP LOG TANH ERF         device libm (last bits are the library's)
 *   SQRT                     correctly rounded
 *   SQRTABS                  sqrt(|a|)
 *   GELU                     a * Phi(a), Phi(a) = erfc(-a/sqrt 2) / 2 (the
 *                            exact x * Phi(x) through the error function,
 *                            presk manual, "Native execution", "The
 *                            realization"); relative error ~1e-7
 *   POW2                     a * a
 *   POWN (iparam n >= 0)     n-1 products of a, left to right; n = 0 gives 1.
 *                            With n > 2 it never joins a group (PSK-Realize,
 *                            "What a group is"): only as a group's sole member
 *   SELECT                   a != 0 ? b : c, moving bits: the branch not
 *                            picked never reaches the result (poot, "Fusable
 *                            region shapes")
 *   CAUSAL_MASK (iparam T)   a where column <= row mod T, else -inf; row is the
 *                            flattened index over all axes but the last
 *                            (causal_mask: allowed where seq2 <= seq, presk
 *                            language reference, section "Typing", builtins)
 *   WHERE (imm = fill)       b where the mask a allows (a != 0), else imm: a
 *                            is a PSK_U8 input, the only op that may read one.
 *                            With fill -inf before a row max and 0 after the
 *                            division it gives the masked softmax of the
 *                            presk manual ("Native execution", "The
 *                            realization"): maximum and sum over the allowed
 *                            positions, 0 where refused, a row the mask
 *                            empties giving zeros
 *   ROW_MAX ROW_SUM ROW_MEAN reduction over the last axis, keepdim; the
 *                            result broadcasts back along the row.  ROW_MEAN
 *                            is ROW_SUM divided by the row length.  ROW_MAX
 *                            is IEEE 754-2019 maximum over the row: NaN if
 *                            any element is NaN, +0 above -0 (the same bits
 *                            whatever the combining order).
 * Leaves: INPUT (iparam = input slot), CONST (imm = an f32 value).
 * Boundary ops (REDUCE, CONTRACT, CAST, OPAQUE) are accepted by
 * psk_partition only: a reduction ends a group, contractions and casts are
 * boundaries (PSK-Realize, "What a group is"; poot, "Fusable region shapes").
 */
typedef enum psk_op {
    PSK_OP_INPUT = 1, PSK_OP_CONST = 2,
    PSK_OP_ADD = 10, PSK_OP_SUB = 11, PSK_OP_MUL = 12, PSK_OP_DIV = 13, PSK_OP_MAX = 14, PSK_OP_MIN = 15,
    PSK_OP_NEG = 20, PSK_OP_ABS = 21, PSK_OP_EXP = 22, PSK_OP_LOG = 23, PSK_OP_SQRT = 24, PSK_OP_TANH = 25,
    PSK_OP_ERF = 26, PSK_OP_GELU = 27, PSK_OP_SQRTABS = 28, PSK_OP_POW2 = 29, PSK_OP_POWN = 30,
    PSK_OP_SELECT = 40, PSK_OP_CAUSAL_MASK = 41, PSK_OP_WHERE = 42,
    PSK_OP_ROW_MAX = 50, PSK_OP_ROW_SUM = 51, PSK_OP_ROW_MEAN = 52,
    PSK_OP_REDUCE = 60, PSK_OP_CONTRACT = 61, PSK_OP_CAST = 62, PSK_OP_OPAQUE = 63
} psk_op;

/* One let of the group, in static single assignment: operands name earlier
 * nodes (a let-list in the manner of PSK-Core's ANF, presk language
 * reference, "PSK-Core").  Unused operands are -1. */
typedef struct psk_node {
    int32_t op;        /* psk_op */
    int32_t a, b, c;   /* operand node indices, each < this node's index, or -1 */
    float imm;         /* PSK_OP_CONST: the value */
    int32_t iparam;    /* PSK_OP_INPUT: slot; PSK_OP_POWN: n; PSK_OP_CAUSAL_MASK: T */
} psk_node;

/* A tensor: shape, storage type and the step of each axis in elements.
 * Inputs align with the output from the last axis; an input axis of length
 * 1 broadcasts (numpy's rule, which the configs' [N,1] and [1,N] inputs
 * use); an input may never widen the output (PSK-Realize, "What a group
 * is": inputs may be smaller and broadcast).  One compiled kernel serves
 * the layout the descriptor states (poot, "Fusion and Planning", "Launch
 * metadata": the metadata a kernel is specialised on).
 *
 * Strides: all zero (over the rank) means dense row-major, so a descriptor
 * filled with zeros but for rank, dtype and shape is dense.  Otherwise
 * stride[d] is axis d's step in elements, >= 0, and 0 broadcasts the axis
 * (a view expanded along it): a transposed or sliced view is read in place,
 * with no copy.  An input whose last-axis stride is 1 and whose other
 * strides are multiples of the vector width (4 elements for an f32 output,
 * 8 for bf16) takes 16-byte accesses; any other layout the element path.
 * A tensor expanded from one element along every axis is given as rank 0
 * (or with sizes 1), since all-zero strides mean dense.  Outputs, extra
 * outputs and the inputs of tree-mapped groups are dense (their strides
 * must be zero or the dense ones: PSK_E_UNSUPPORTED otherwise); negative
 * strides are refused (PSK_E_SHAPE). */
typedef struct psk_tensor_desc {
    int32_t rank;                    /* 0..PSK_MAX_RANK (output: 1..PSK_MAX_RANK) */
    int32_t dtype;                   /* psk_dtype */
    int64_t shape[PSK_MAX_RANK];     /* entries at and beyond rank are ignored */
    int64_t stride[PSK_MAX_RANK];    /* elements; all zero: dense row-major */
} psk_tensor_desc;

typedef struct psk_group_desc {
    int32_t n_nodes;                 /* 1..PSK_MAX_NODES */
    const psk_node* nodes;
    int32_t root;                    /* the one member no node reads; usually n_nodes-1 */
    int32_t n_inputs;                /* 0..PSK_MAX_INPUTS; slot k is INPUT iparam k */
    const psk_tensor_desc* inputs;
    psk_tensor_desc out;             /* the root's storage type and shape */
    int32_t arith;                   /* arithmetic type: must be PSK_F32 */
    uint32_t flags;                  /* 0, PSK_GROUP_TREE or PSK_GROUP_ONLINE */
    /* Further stored values (multi-output groups; 0 for a single root).
     * PSK-Realize, "Not in this version", names multi-output kernels as what
     * keeps a value read both inside and outside a group from splitting it,
     * and "What it buys, measured" the layer normalization that splits for
     * want of it.  extra_root[k] is a member other than the root, each
     * named once; extra_out[k] its storage: an element value has the
     * output's shape, a value that is one per row (a reduction, or a member
     * of row values) the output's shape with a last axis of 1.  Members that
     * read a stored value read it as stored (rounded to its storage type),
     * so the group computes what the partitioned program would: the stored
     * value ends one group and the next reads it from memory. */
    int32_t n_extra;                 /* 0..PSK_MAX_EXTRA */
    const int32_t* extra_root;
    const psk_tensor_desc* extra_out;
} psk_group_desc;

/* A group mapped over the leaves of a parameter tree (psk_group_run_tree):
 * output rank 1, every input rank 1 (one element per leaf element) or rank 0
 * (one value for the whole tree); shape lengths are not used, each leaf has
 * its own; no row reductions and no causal mask.  Extra outputs are element
 * values stored to further slots. */
#define PSK_GROUP_TREE 1u

/* The online normalizer (poot, "Flash attention rewrite": the planner's
 * online-softmax generator).  A row sum of exp(y - m) where m is the row
 * maximum of the same y is taken in the maximum's pass: each lane keeps a
 * running maximum and a sum of exponentials relative to it, rescaled by
 * exp(old - new) when the maximum grows, and lanes, waves and the
 * workgroups sharing a split row combine their pairs the same way.  One pass
 * over the row fewer (a row walked from memory by the tiled kernel is read
 * once less; split rows exchange once instead of twice); the sum's rounding
 * differs from the exact two-pass sum (a few f32 ulps: declared differs,
 * tested within the f32 tolerance).  Refused (PSK_E_UNSUPPORTED) unless the
 * group holds such a sum whose maximum, difference and exponential are not
 * stored as bf16 (their readers would see rounded values the maximum's pass
 * never sums), and for trees. */
#define PSK_GROUP_ONLINE 2u

typedef struct psk_group psk_group;
typedef struct psk_tree psk_tree;

/* Validate a group, emit its HIP kernel and compile it with hipRTC for
 * gfx950 (kernels are cached by the group's canonical text, in memory and,
 * when PSK_CACHE_DIR is set, on disk).  Validation covers: node order,
 * operand counts, a single root, no dead node, the member cap, one result
 * type for the element members, broadcast legality, row-reduction use (a
 * reduction's operand is an element value; the root is an element value),
 * storage types.  Does not need a GPU: the kernel is loaded on first run.
 * The launch layout (lanes a row, workgroup size, tiling, caches) follows
 * from the shapes; the environment variable PSK_LAYOUT ("key=value,...")
 * overrides it at create time, for measurement: it never changes which
 * elements are computed, only, for some keys, a reduction's bracketing. */
psk_status psk_group_create(const psk_group_desc* desc, psk_group** out);

/* Run the group as one kernel launch.  inputs[k] is the device address of
 * input slot k's first element, laid out as desc.inputs[k] (shape and
 * strides); out is the device address of the (dense) output.  The output may be the same buffer as an input of the same shape
 * and storage type (in place); any other overlap with an input is refused
 * (PSK_E_ALIAS).  Pointers must be aligned to their element size
 * (PSK_E_ALIGN); 16-byte alignment takes the vector path.  Empty outputs
 * launch nothing. */
psk_status psk_group_run(const psk_group* group, const void* const* inputs, void* out, void* hip_stream);

/* The same for a group with extra outputs: outs[0] is the root's output,
 * outs[1 + k] extra output k's (laid out as desc.extra_out[k]).  An element
 * output may be the same buffer as an input of its shape and storage type
 * (in place); outputs never overlap one another, and a per-row output
 * overlaps nothing (PSK_E_ALIAS).  psk_group_run refuses a group with extra
 * outputs (PSK_E_UNSUPPORTED). */
psk_status psk_group_run_multi(const psk_group* group, const void* const* inputs, void* const* outs,
                               void* hip_stream);

void psk_group_destroy(psk_group* group);

/* Rows too wide for one workgroup's registers are shared by several
 * workgroups (kind 4), which exchange partial row values (a maximum, a sum)
 * through the group's device memory: launches of the group are persistent,
 * with no more workgroups than the device holds at once, so all of them run
 * together, and every wait is bounded.  The group's first run on a device
 * allocates that memory (like loading the code object); runs of one group
 * on one device must follow one another (one stream, or ordered streams):
 * two at once would share it.  A wait that ran out (the device was shared
 * with other work long enough, for instance) leaves that run's results
 * invalid; psk_group_check waits for the device and returns PSK_E_HIP if any
 * wait of the group on the current device ran out since the last check
 * (PSK_OK at once for groups without split rows). */
psk_status psk_group_check(const psk_group* group);

/* Kernel shape chosen for a group (for tests and measurement). */
typedef struct psk_group_info {
    int32_t kind;            /* 0 pointwise, 1 row, 2 tree-mapped, 3 row tiled, 4 split rows */
    int32_t members;         /* member count */
    int32_t n_reductions;    /* row reductions */
    int32_t phases;          /* reduction phases (longest chain of dependent reductions) */
    int64_t rows, cols;      /* output viewed as [rows, cols] */
    int32_t lanes_per_row;   /* row kernel: threads per row */
    int32_t vec;             /* elements per vector access */
    int32_t block;           /* threads per workgroup */
    int32_t rows_per_block;  /* row kernel */
    int64_t algorithmic_bytes; /* inputs read once at their own size + outputs written once */
    char kernel[48];         /* the emitted kernel's name (as profilers show it), NUL-terminated */
    int32_t tiles;           /* tiled row kernel (kind 3: rows too wide for registers that split
                                rows cannot take, i.e. more than 32 workgroups a row or more
                                than 64 partials a phase): tiles per row; each reduction phase
                                re-reads the row.  0 otherwise */
    int32_t split;           /* split rows (kind 4): workgroups that share one row, each holding
                                a segment in registers and exchanging partial row values with
                                the others.  0 otherwise */
} psk_group_info;
psk_status psk_group_get_info(const psk_group* group, psk_group_info* info);

/* Validate a descriptor and write the emitted HIP source (NUL-terminated)
 * into buf; *len receives the full length.  Touches no device and does not
 * compile. */
psk_status psk_group_source(const psk_group_desc* desc, char* buf, size_t cap, size_t* len);

/* Validate, emit and compile with hipRTC, returning the gfx950 code object
 * (no device needed).  *len receives its size; buf may be NULL to query. */
psk_status psk_group_code_object(const psk_group_desc* desc, void* buf, size_t cap, size_t* len);

/* ------------------------------------------------------ parameter trees */
/* One leaf of a parameter tree: numel elements in each slot.  For AdamW the
 * slots are theta, g, m, v (4 slots: updated in place), or theta, g, m, v,
 * theta', m', v' (7 slots: outputs apart; an output may also be the same
 * buffer as its input). */
typedef struct psk_leaf {
    int64_t numel;                   /* >= 0; a leaf of 0 elements is skipped */
    void* slot[PSK_MAX_SLOTS];       /* device addresses, dense, each aligned to its element size */
} psk_leaf;

/* Build the leaf table (prefix offsets) and the chunk map: each leaf is cut
 * into chunks of PSK_TREE_CHUNK elements (the last one shorter); chunk
 * starts are multiples of 8 elements within a leaf, so 16-byte vector
 * accesses stay inside one leaf.  The tables are uploaded to the current
 * device once.  Slot dtypes apply to every leaf; 1 to 8 slots.  A leaf may
 * repeat a buffer across its slots when they share a storage type; buffers
 * never overlap partly, and leaves never share memory.  Refuses: NULL
 * pointers of non-empty leaves, negative numel, misaligned pointers,
 * overlaps as above (PSK_E_ALIAS).  AdamW's slot roles (theta, g, m, v
 * [, theta', m', v']: 4 or 7 slots, m and v of one storage type, each output
 * of its input's type, every slot its own buffer except an output over its
 * own input) are not required here: psk_adamw_step refuses a tree without
 * them, with the reason. */
#define PSK_TREE_CHUNK 4096
psk_status psk_tree_create(const psk_leaf* leaves, int32_t n_leaves, int32_t n_slots,
                           const int32_t* slot_dtypes, psk_tree** out);
void psk_tree_destroy(psk_tree* tree);

typedef struct psk_tree_info {
    int32_t n_leaves, n_slots;
    int64_t n_chunks;
    int64_t total_numel;
    int64_t chunk_elems;             /* PSK_TREE_CHUNK */
    int32_t vector_leaves;           /* leaves whose slots are all 16-byte aligned */
} psk_tree_info;
psk_status psk_tree_get_info(const psk_tree* tree, psk_tree_info* info);

/* Copy the host copy of the tables: leaf_offset[n_leaves+1] (exclusive
 * prefix sums of numel), and per chunk its leaf, start element within the
 * leaf and element count.  Any pointer may be NULL to skip it. */
psk_status psk_tree_get_tables(const psk_tree* tree, int64_t* leaf_offset, int32_t* chunk_leaf,
                               int64_t* chunk_start, int32_t* chunk_count);

/* Host-only planning of the same tables without device pointers or a
 * device (for tests): numel[n_leaves] in, tables out as above. */
psk_status psk_tree_plan(const int64_t* numel, int32_t n_leaves, int64_t* n_chunks, int64_t* leaf_offset,
                         int32_t* chunk_leaf, int64_t* chunk_start, int32_t* chunk_count);

/* AdamW hyperparameters (presk language reference, section "Configuration blocks", the optimizer):
 *   m' = b1 m + (1-b1) g;  v' = b2 v + (1-b2) g^2;
 *   mh = m'/(1-b1^t);  vh = v'/(1-b2^t);
 *   theta' = theta - lr (mh/(sqrt(vh)+eps) + wd theta)
 * t counts steps from 1.  Hyperparameter arithmetic (1-b, b^t) is done in
 * f64 on the host and each scalar is rounded once to f32. */
typedef struct psk_adamw_hp {
    double lr, beta1, beta2, eps, weight_decay;
    int64_t t;
} psk_adamw_hp;

/* One AdamW step over every leaf of the tree in a single kernel launch.
 * Slot dtypes: theta and g each f32 or bf16; m and v the same type, f32 or
 * bf16; outputs the type of their input.  Arithmetic is f32; theta' is
 * rounded once to theta's storage; m' and v' are stored, and theta' reads
 * the stored values.  Refuses t < 1, non-finite hyperparameters, and a
 * tree without AdamW's slot roles (see psk_tree_create): PSK_E_SHAPE for a
 * slot count other than 4 or 7, PSK_E_TYPE for storage types, PSK_E_ALIAS
 * for a buffer in two slots other than an output over its own input. */
psk_status psk_adamw_step(const psk_tree* tree, const psk_adamw_hp* hp, void* hip_stream);

/* Learning-rate schedules (presk language reference, section "Configuration
 * blocks", the optimizer): constant: lr; linear(warmup w): lr*t/w for t <= w,
 * then lr*(total - t)/(total - w); cosine(warmup w): lr*t/w for t <= w, then
 * lr/2 * (1 + cos(pi (t - w)/(total - w))); both reach 0 at total. */
typedef enum psk_schedule { PSK_SCHED_CONSTANT = 0, PSK_SCHED_LINEAR = 1, PSK_SCHED_COSINE = 2 } psk_schedule;

/* A full AdamW configuration.  With grad_clip = c > 0 the gradient is first
 * scaled by min(1, c / (||g||_2 + 1e-6)), ||g||_2 the global norm over every
 * leaf of the tree (as clip_grad_norm_ does); the squared norm is
 * accumulated in f64 and the factor, formed in f64, is rounded once to f32
 * and multiplies each gradient element in f32 before the step.  The
 * schedule's lr(t, total) is computed in f64 on the host and rounded once. */
typedef struct psk_adamw_config {
    double lr, beta1, beta2, eps, weight_decay;
    int64_t t;            /* step, counted from 1 */
    int64_t total;        /* total steps (linear, cosine) */
    int64_t warmup;       /* warmup steps, 0 <= warmup < total (linear, cosine) */
    int32_t schedule;     /* psk_schedule */
    double grad_clip;     /* c > 0: clip by the global norm; <= 0: no clipping */
} psk_adamw_config;

/* The step of psk_adamw_step under a full configuration: with clipping,
 * three launches on the stream -- the tree-wide sum of squares (a partial
 * sum per chunk), a one-workgroup pass that combines the partials in a fixed
 * order and forms the factor in device memory owned by the tree, and the
 * step, which reads the factor; no host synchronisation.  Refuses t < 1, t > total or
 * warmup >= total for the decaying schedules, non-finite values. */
psk_status psk_adamw_step_config(const psk_tree* tree, const psk_adamw_config* cfg, void* hip_stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the step
 * of psk_adamw_step_config, bit for bit, whose clipping pass keeps its
 * per-chunk partial sums and its result in a library-static device array
 * (one per GPU, 8 MiB, held until the process ends) instead of the tree's
 * memory.  The call allocates nothing (no hipMalloc, no allocating library
 * routine); the tree and its tables were created beforehand.  Every such
 * call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (on different streams, or from several threads without ordering) race.
 * With clipping, a tree of more than 2^20 chunks (2^32 elements) is refused
 * (PSK_E_UNSUPPORTED) before any launch.  psk_tree_clip_result does not see
 * the result of a step taken here.  Other refusals as psk_adamw_step_config. */
psk_status psk_adamw_step_config_noalloc(const psk_tree* tree, const psk_adamw_config* cfg, void* hip_stream);

/* Host-only: the schedule's learning rate at cfg->t (before rounding). */
psk_status psk_adamw_lr(const psk_adamw_config* cfg, double* lr);

/* The squared global norm and the f32 factor of the last clipped step on
 * this tree: waits for the whole device (every stream), then copies them
 * back.  The current device must be the tree's (else PSK_E_HIP).  Zeros
 * before any clipped step.  For checks and reporting. */
psk_status psk_tree_clip_result(const psk_tree* tree, double* sumsq, float* factor);

/* Run a PSK_GROUP_TREE group over every leaf of a tree in one launch
 * (PSK-Realize, "What a group is", parameter trees: the chain is mapped over
 * the leaves).  Input k of rank 1 reads slot in_slot[k] of each leaf; input
 * k of rank 0 reads the device address scalars[k] (one f32 or bf16 value
 * shared by every leaf; in_slot[k] is ignored).  The root is written, rounded
 * to the output storage type, to slot out_slot of each leaf.  Slot storage
 * types must equal the group's (PSK_E_TYPE); slots out of range give
 * PSK_E_SHAPE, a NULL or misaligned scalar PSK_E_NULL / PSK_E_ALIGN, and a
 * scalar that lies inside an output-slot buffer PSK_E_ALIAS.  out_slot may
 * equal an input's slot (in place: each element is read before it is
 * written, by the same thread); other overlaps were refused when the tree
 * was created.  The tree must have been created on the current device.
 * Leaves whose slots are all 16-byte aligned take 8/16-byte accesses; a
 * tree with no elements launches nothing.  Buffers stay the caller's. */
psk_status psk_group_run_tree(const psk_group* group, const psk_tree* tree, const int32_t* in_slot, int32_t out_slot,
                              const void* const* scalars, void* hip_stream);

/* The same for a tree-mapped group with extra outputs: out_slot[0] receives
 * the root, out_slot[1 + k] extra output k; output slots are distinct
 * (PSK_E_ALIAS otherwise), and a scalar may lie in none of them.
 * psk_group_run_tree refuses a group with extra outputs. */
psk_status psk_group_run_tree_multi(const psk_group* group, const psk_tree* tree, const int32_t* in_slot,
                                    const int32_t* out_slot, const void* const* scalars, void* hip_stream);

/* --------------------------------------------------------------- partition */
/* Partition a function body (a let-list of n nodes, leaves included) into
 * fusion groups (PSK-Realize, "What a group is").  types[i] is node i's
 * result type (shape and storage type; two types are equal when rank, dtype
 * and shape agree), is_output[i] marks values read outside the body.
 * Scanning from the last let to the first, an elementwise let joins the
 * group of its readers when it is not an output, every reader is an
 * elementwise member of that one group, its type is the group's, and the
 * group has fewer than 64 members; otherwise it roots a new group.  Leaves
 * get group -1; a boundary let (row reduction, REDUCE, CONTRACT, CAST,
 * OPAQUE, POWN with n > 2) is a group of its own.  Groups are numbered by
 * their root's position.  group_of[n], is_root[n] out; *n_groups out. */
psk_status psk_partition(int32_t n, const psk_node* body, const psk_tensor_desc* types,
                         const uint8_t* is_output, int32_t* group_of, int32_t* is_root, int32_t* n_groups);

/* The same with options.  PSK_PARTITION_ROWS fuses reductions as the row
 * kernels run them (poot, "Fusion and Planning", "Reduction-rooted
 * regions"; PSK-Realize, "Not in this version", reduction fusion): a
 * last-axis row reduction is a member candidate, and a let whose shape is
 * the group root's with a last axis of 1 (a value one per row, whatever its
 * storage type) joins under the same reader rule.  flags 0 is psk_partition.
 * Unknown flags: PSK_E_UNSUPPORTED. */
#define PSK_PARTITION_ROWS 1u
psk_status psk_partition_ex(int32_t n, const psk_node* body, const psk_tensor_desc* types,
                            const uint8_t* is_output, uint32_t flags, int32_t* group_of, int32_t* is_root,
                            int32_t* n_groups);

/* Static launch count and traffic of a body before and after the partition
 * (what poot's dispatch_count reports, "What fusion reports"; PSK-Realize,
 * "What it removes").  Unfused, every non-leaf let is a launch that reads
 * each operand and writes its value; fused, every group is one launch that
 * reads each value from outside it once and writes its root.  Bytes are
 * tensor sizes at their storage types (f32 4, bf16 2, u8 1). */
typedef struct psk_dispatch_report {
    int32_t lets;               /* non-leaf lets */
    int32_t launches_unfused;   /* = lets */
    int32_t launches_fused;     /* groups */
    int32_t fused_groups;       /* groups with more than one member */
    int64_t bytes_unfused;
    int64_t bytes_fused;
} psk_dispatch_report;
psk_status psk_dispatch_count(int32_t n, const psk_node* body, const psk_tensor_desc* types,
                              const uint8_t* is_output, uint32_t flags, psk_dispatch_report* report);

/* ------------------------------------------------------------------ misc */
const char* psk_last_error(void);
const char* psk_status_str(psk_status status);
int32_t psk_version(void);

typedef struct psk_stats {
    int64_t launches;      /* kernel launches issued by this library */
    int64_t jit_compiles;  /* hipRTC compilations */
    int64_t jit_hits;      /* kernels found in the memory or disk cache */
} psk_stats;
psk_status psk_get_stats(psk_stats* stats);

#ifdef __cplusplus
}
#endif

#endif /* PSK_FUSED_H */
