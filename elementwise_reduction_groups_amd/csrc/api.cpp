// The C ABI of psk_fused: group and tree objects, kernel loading and launch,
// error reporting.  Entry points validate everything on the host before any
// device work and return a psk_status; nothing is launched on a refusal.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "psk_internal.h"

// ------------------------------------------------------------ error state
namespace psk {

static thread_local std::string t_last_error;
static std::atomic<int64_t> g_launches{0}, g_jit_compiles{0}, g_jit_hits{0};

psk_status fail(psk_status st, const std::string& msg)
{
    t_last_error = std::string(psk_status_str(st)) + ": " + msg;
    return st;
}

void clear_error() { t_last_error.clear(); }
void count_launch() { g_launches++; }
void count_jit(bool hit) { (hit ? g_jit_hits : g_jit_compiles)++; }

AdamwScalars adamw_scalars(const psk_adamw_hp& hp)
{
    // hyperparameter arithmetic in f64, each scalar rounded once to f32
    AdamwScalars s;
    s.b1 = (float)hp.beta1;
    s.b2 = (float)hp.beta2;
    s.c1 = (float)(1.0 - hp.beta1);
    s.c2 = (float)(1.0 - hp.beta2);
    s.bc1 = (float)(1.0 - std::pow(hp.beta1, (double)hp.t));
    s.bc2 = (float)(1.0 - std::pow(hp.beta2, (double)hp.t));
    s.lr = (float)hp.lr;
    s.eps = (float)hp.eps;
    s.wd = (float)hp.weight_decay;
    // 1/bc in f64 rounded to f32 is the correctly rounded f32 reciprocal:
    // rounding twice is harmless for a quotient when the first rounding keeps
    // at least 2*24+2 bits (Figueroa's condition; f64 keeps 53)
    auto in_range = [](float b) { return b >= 0x1p-40f && b <= 0x1p40f; };
    const bool rec = in_range(s.bc1) && in_range(s.bc2);
    s.rc1 = rec ? (float)(1.0 / (double)s.bc1) : 0.0f;
    s.rc2 = rec ? (float)(1.0 / (double)s.bc2) : 0.0f;
    return s;
}

// ---------------------------------------------------------- kernel cache
constexpr int kMaxDevices = 64;

struct Kernel {
    KernelPlan plan;
    std::string name;
    std::vector<char> code;
    std::mutex mu;
    hipModule_t mod[kMaxDevices] = {};
    hipFunction_t fn[kMaxDevices] = {};
    int capacity[kMaxDevices] = {};   // split rows: workgroups the device holds at once (0: not yet asked)
};

static std::mutex g_cache_mu;
static std::map<std::string, std::shared_ptr<Kernel>>& cache()
{
    static auto* m = new std::map<std::string, std::shared_ptr<Kernel>>();  // lives until exit
    return *m;
}

static psk_status get_kernel_plan(const Analysis& an, const KernelPlan& plan, std::shared_ptr<Kernel>& out);

// A split-rows kernel holds its segment in registers: the planned width is
// compiled first and, if the compiled kernel spills registers, narrower
// segments (more workgroups a row) are tried; if every width spills, the
// tiled kernel takes the group.  Other plans compile as planned.
static psk_status get_kernel(const Analysis& an, bool vector, std::shared_ptr<Kernel>& out)
{
    KernelPlan plan = plan_kernel(an, vector);
    if (plan.kind != 4) return get_kernel_plan(an, plan, out);
    const int first = plan.nv * plan.vec;
    const int widths[] = {first, 48, 32, 16};
    for (int i = 0; i < 4; ++i) {
        const int ept = widths[i];
        if (i > 0 && ept >= first) continue;
        KernelPlan p = plan_kernel(an, vector, ept);
        if (p.kind != 4) break;
        psk_status st = get_kernel_plan(an, p, out);
        if (st != PSK_OK) return st;
        if (code_scratch_bytes(out->code) == 0) return PSK_OK;
        if (std::getenv("PSK_LAYOUT") && std::strstr(std::getenv("PSK_LAYOUT"), "sept=")) return PSK_OK;
    }
    return get_kernel_plan(an, plan_kernel(an, vector, 0), out);
}

static psk_status get_kernel_plan(const Analysis& an, const KernelPlan& plan, std::shared_ptr<Kernel>& out)
{
    std::string canon = canonical_text(an);
    std::string key = canon + plan.key();
    {
        std::lock_guard<std::mutex> lk(g_cache_mu);
        auto it = cache().find(key);
        if (it != cache().end()) {
            out = it->second;
            count_jit(true);
            return PSK_OK;
        }
    }
    auto k = std::make_shared<Kernel>();
    k->plan = plan;
    char nm[64];
    static const char* const kind_name[5] = {"pw", "row", "tree", "rowt", "rows"};
    std::snprintf(nm, sizeof nm, "psk_%s_%016llx", kind_name[plan.kind], (unsigned long long)fnv1a(key));
    k->name = nm;
    std::string src = emit_source(an, plan, k->name);
    psk_status st = jit_compile(src, k->name, k->code);
    if (st != PSK_OK) return st;
    std::lock_guard<std::mutex> lk(g_cache_mu);
    auto it = cache().find(key);
    if (it != cache().end()) { out = it->second; return PSK_OK; }
    cache()[key] = k;
    out = k;
    return PSK_OK;
}

static psk_status kernel_function(Kernel& k, hipFunction_t& fn)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(PSK_E_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(PSK_E_HIP, "device index out of range");
    std::lock_guard<std::mutex> lk(k.mu);
    if (!k.fn[dev]) {
        e = hipModuleLoadData(&k.mod[dev], k.code.data());
        if (e != hipSuccess) return fail(PSK_E_HIP, std::string("hipModuleLoadData: ") + hipGetErrorString(e));
        e = hipModuleGetFunction(&k.fn[dev], k.mod[dev], k.name.c_str());
        if (e != hipSuccess) return fail(PSK_E_HIP, std::string("hipModuleGetFunction: ") + hipGetErrorString(e));
    }
    fn = k.fn[dev];
    return PSK_OK;
}

static int esize(int dt) { return dt == PSK_BF16 ? 2 : dt == PSK_U8 ? 1 : 4; }

}  // namespace psk

using namespace psk;

// ------------------------------------------------------------------ groups
// Device state of a split-rows kernel on one device: the generation counter,
// the count of finished workgroups, the status word of the bounded waits,
// then the teams' partial slots (teams x exchanged values x K, 8 bytes each).
struct SplitState {
    void* mem = nullptr;
    int64_t teams = 0;
};

struct psk_group {
    Analysis an;
    std::shared_ptr<Kernel> vec;      // 16-byte accesses
    std::shared_ptr<Kernel> scalar;   // element accesses (compiled on first need)
    std::mutex mu;
    SplitState split[kMaxDevices][2];   // [device][vector, element kernel]
    int wait_limit = 1 << 20;           // tries a bounded wait makes (PSK_SPLIT_WAIT overrides)
    ~psk_group()
    {
        for (auto& d : split)
            for (auto& st : d)
                if (st.mem) (void)hipFree(st.mem);
    }
};

// The launch shape of a split-rows kernel on the current device: teams of K
// workgroups, the whole grid no larger than what the device holds at once
// (so every member of a team runs while the others wait for it); teams of
// one XCD when the grid is a multiple of 8 K.  Allocates the device state on
// the first run on a device (zeroed: generation 0, no tags).
static psk_status split_launch(psk_group* g, Kernel& k, int which, hipFunction_t fn, int64_t rows, int64_t& teams,
                               int& xmap, void*& mem)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(PSK_E_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    const int K = k.plan.split;
    std::lock_guard<std::mutex> lk(g->mu);
    {
        std::lock_guard<std::mutex> lk2(k.mu);
        if (!k.capacity[dev]) {
            int per_cu = 0, cus = 0, regs = 0;
            e = hipModuleOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, k.plan.block, 0);
            if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
            if (e == hipSuccess) e = hipFuncGetAttribute(&regs, HIP_FUNC_ATTRIBUTE_NUM_REGS, fn);
            if (e != hipSuccess) return fail(PSK_E_HIP, std::string("occupancy query: ") + hipGetErrorString(e));
            // never more than the register file holds by gfx950's rules: 512
            // registers a lane, allocated in granules of 8, at most 8 waves
            // a SIMD, a workgroup's waves spread over the CU's 4 SIMDs
            // (a grid larger than what is resident at once would leave a
            // team waiting for members that start only as others finish)
            if (regs > 0) {
                const int waves_simd = std::min(8, 512 / (((regs + 7) / 8) * 8));
                const int waves_wg = (k.plan.block + 63) / 64;
                per_cu = std::min(per_cu, 4 * waves_simd / waves_wg);
            }
            k.capacity[dev] = per_cu * cus;
        }
    }
    const int64_t cap = k.capacity[dev];
    if (cap < K)
        return fail(PSK_E_UNSUPPORTED, "the device holds " + std::to_string(cap) + " of these workgroups at once; a "
                                       "row needs " + std::to_string(K));
    teams = cap / K;
    xmap = 0;
    if (cap >= 8 * K && layout_value("xmap", 1)) {
        teams = (cap / (8 * K)) * 8;
        xmap = 1;
    }
    SplitState& st = g->split[dev][which];
    if (!st.mem) {
        const size_t bytes = 16 + (size_t)teams * k.plan.exch * K * 8;
        e = hipMalloc(&st.mem, bytes);
        if (e == hipSuccess) e = hipMemset(st.mem, 0, bytes);
        if (e != hipSuccess) {
            if (st.mem) (void)hipFree(st.mem);
            st.mem = nullptr;
            return fail(PSK_E_HIP, std::string("split-row state: ") + hipGetErrorString(e));
        }
        st.teams = teams;
    }
    teams = std::min(teams, st.teams);
    if (teams > rows) {
        teams = rows;
        xmap = 0;
    }
    mem = st.mem;
    return PSK_OK;
}

extern "C" psk_status psk_group_create(const psk_group_desc* desc, psk_group** out)
{
    clear_error();
    if (!out) return fail(PSK_E_NULL, "out is NULL");
    *out = nullptr;
    auto g = std::make_unique<psk_group>();
    psk_status st = analyse(desc, g->an);
    if (st != PSK_OK) return st;
    KernelPlan p = plan_kernel(g->an, true);
    if (!g->an.tree && p.grid > 0x7fffffffLL) return fail(PSK_E_UNSUPPORTED, "output too large for one launch");
    st = get_kernel(g->an, true, g->vec);
    if (st != PSK_OK) return st;
    if (g->vec->plan.vec == 1) g->scalar = g->vec;
    if (const char* w = std::getenv("PSK_SPLIT_WAIT")) g->wait_limit = std::max(0, std::atoi(w));
    *out = g.release();
    return PSK_OK;
}

extern "C" void psk_group_destroy(psk_group* group) { delete group; }

extern "C" psk_status psk_group_get_info(const psk_group* group, psk_group_info* info)
{
    clear_error();
    if (!group || !info) return fail(PSK_E_NULL, "group or info is NULL");
    const Analysis& an = group->an;
    const KernelPlan& p = group->vec->plan;
    info->kind = p.kind;
    info->members = an.members;
    info->n_reductions = an.n_reductions;
    info->phases = an.phases;
    info->rows = an.rows;
    info->cols = an.cols;
    info->lanes_per_row = (p.kind == 1 || p.kind == 3) ? p.lanes : p.kind == 4 ? p.lanes * p.split : 1;
    info->vec = p.vec;
    info->block = p.block;
    info->rows_per_block = (p.kind == 1 || p.kind == 3 || p.kind == 4) ? p.rows_per_block : 0;
    info->tiles = p.tiles;
    info->split = p.split;
    int64_t bytes = an.numel * esize(an.out_dtype);
    for (const InputInfo& in : an.inputs)
        if (in.used) bytes += in.numel * esize(in.dtype);
    for (const auto& x : an.extras) bytes += (x.per_row ? an.rows : an.numel) * esize(x.dtype);
    info->algorithmic_bytes = bytes;
    std::snprintf(info->kernel, sizeof info->kernel, "%s", group->vec->name.c_str());
    return PSK_OK;
}

// One launch of a group: outs[0] is the root's output, outs[1 + k] extra output k's.
static psk_status run_group(const psk_group* group, const void* const* inputs, void* const* outs, void* hip_stream)
{
    const Analysis& an = group->an;
    if (an.tree) return fail(PSK_E_UNSUPPORTED, "a tree-mapped group runs with psk_group_run_tree");
    if (an.numel == 0) return PSK_OK;
    if (!an.inputs.empty() && !inputs) return fail(PSK_E_NULL, "inputs is NULL");
    // every output: [b, e), element size, per row or per element
    struct Out {
        uintptr_t b, e;
        int size;
        bool per_row;
        psk_dtype dt;
    };
    const int n_out = 1 + (int)an.extras.size();
    std::vector<Out> ov(n_out);
    bool aligned16 = true;
    for (int k = 0; k < n_out; ++k) {
        const std::string name = k == 0 ? "out" : "extra output " + std::to_string(k - 1);
        if (!outs[k]) return fail(PSK_E_NULL, name + " is NULL");
        const psk_dtype dt = k == 0 ? an.out_dtype : an.extras[k - 1].dtype;
        const bool per_row = k > 0 && an.extras[k - 1].per_row;
        const uintptr_t b = reinterpret_cast<uintptr_t>(outs[k]);
        if (b % esize(dt)) return fail(PSK_E_ALIGN, name + " is not aligned to its element size");
        if (!per_row && b % 16) aligned16 = false;
        ov[k] = {b, b + (uintptr_t)(per_row ? an.rows : an.numel) * esize(dt), esize(dt), per_row, dt};
        for (int j = 0; j < k; ++j)
            if (ov[j].b < ov[k].e && ov[k].b < ov[j].e)
                return fail(PSK_E_ALIAS, name + " overlaps another output");
    }
    for (size_t k = 0; k < an.inputs.size(); ++k) {
        const InputInfo& in = an.inputs[k];
        if (!in.used) continue;
        if (in.numel == 0) return PSK_OK;  // cannot happen for a non-empty output; kept for safety
        const uintptr_t b = reinterpret_cast<uintptr_t>(inputs[k]);
        if (!b) return fail(PSK_E_NULL, "input " + std::to_string(k) + " is NULL");
        if (b % esize(in.dtype)) return fail(PSK_E_ALIGN, "input " + std::to_string(k) + " is not aligned to its element size");
        if (b % 16) aligned16 = false;
        // the bytes the input's layout reaches: first element to last offset
        const uintptr_t e = b + (uintptr_t)in.span * esize(in.dtype);
        for (const Out& o : ov) {
            if (!(b < o.e && o.b < e)) continue;
            // in place: an element output over a same-shape, same-type input
            bool same = b == o.b && !o.per_row && in.kind == InKind::Full && in.dtype == o.dt;
            if (!same)
                return fail(PSK_E_ALIAS, "an output overlaps input " + std::to_string(k) +
                                             " (only an in-place update of a same-shape, same-type input is allowed)");
        }
    }
    std::shared_ptr<Kernel> k;
    if (aligned16 || group->vec->plan.vec == 1) {
        k = group->vec;
    } else {
        psk_group* g = const_cast<psk_group*>(group);
        std::lock_guard<std::mutex> lk(g->mu);
        if (!g->scalar) {
            psk_status st = get_kernel(an, false, g->scalar);
            if (st != PSK_OK) return st;
        }
        k = g->scalar;
    }
    hipFunction_t fn = nullptr;
    psk_status st = kernel_function(*k, fn);
    if (st != PSK_OK) return st;
    std::vector<void*> args;
    std::vector<const void*> ptrs(an.inputs.size());
    for (size_t i = 0; i < an.inputs.size(); ++i) ptrs[i] = inputs ? inputs[i] : nullptr;
    const KernelPlan& p = k->plan;
    long long n_total = (p.kind == 1 || p.kind == 3 || p.kind == 4) ? (long long)an.rows : (long long)an.numel;
    for (size_t i = 0; i < ptrs.size(); ++i) args.push_back(&ptrs[i]);
    std::vector<void*> optr(outs, outs + n_out);
    for (int i = 0; i < n_out; ++i) args.push_back(&optr[i]);
    args.push_back(&n_total);
    int64_t grid = p.grid;
    void* xslots = nullptr;
    unsigned* xstate = nullptr;
    unsigned teams = 0;
    int xmap = 0, limit = group->wait_limit;
    if (p.kind == 4) {
        int64_t t = 0;
        void* mem = nullptr;
        st = split_launch(const_cast<psk_group*>(group), *k, k == group->vec ? 0 : 1, fn, an.rows, t, xmap, mem);
        if (st != PSK_OK) return st;
        xstate = static_cast<unsigned*>(mem);
        xslots = static_cast<char*>(mem) + 16;
        teams = (unsigned)t;
        grid = t * p.split;
        args.push_back(&xslots);
        args.push_back(&xstate);
        args.push_back(&teams);
        args.push_back(&xmap);
        args.push_back(&limit);
    }
    hipError_t e = hipModuleLaunchKernel(fn, (unsigned)grid, 1, 1, (unsigned)p.block, 1, 1, 0,
                                         static_cast<hipStream_t>(hip_stream), args.data(), nullptr);
    if (e != hipSuccess) return fail(PSK_E_HIP, std::string("hipModuleLaunchKernel: ") + hipGetErrorString(e));
    count_launch();
    return PSK_OK;
}

extern "C" psk_status psk_group_run(const psk_group* group, const void* const* inputs, void* out, void* hip_stream)
{
    clear_error();
    if (!group) return fail(PSK_E_NULL, "group is NULL");
    if (!group->an.extras.empty())
        return fail(PSK_E_UNSUPPORTED, "the group has extra outputs: run it with psk_group_run_multi");
    void* outs[1] = {out};
    return run_group(group, inputs, outs, hip_stream);
}

extern "C" psk_status psk_group_check(const psk_group* group)
{
    clear_error();
    if (!group) return fail(PSK_E_NULL, "group is NULL");
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) return fail(PSK_E_HIP, "hipGetDevice failed");
    psk_group* g = const_cast<psk_group*>(group);
    std::lock_guard<std::mutex> lk(g->mu);
    bool any = false;
    for (auto& st : g->split[dev]) any = any || st.mem;
    if (!any) return PSK_OK;
    e = hipDeviceSynchronize();
    if (e != hipSuccess) return fail(PSK_E_HIP, std::string("hipDeviceSynchronize: ") + hipGetErrorString(e));
    unsigned timed_out = 0;
    for (auto& st : g->split[dev]) {
        if (!st.mem) continue;
        unsigned w = 0;
        e = hipMemcpy(&w, static_cast<unsigned*>(st.mem) + 2, sizeof w, hipMemcpyDeviceToHost);
        if (e == hipSuccess && w) e = hipMemset(static_cast<unsigned*>(st.mem) + 2, 0, sizeof w);
        if (e != hipSuccess) return fail(PSK_E_HIP, std::string("reading the wait status: ") + hipGetErrorString(e));
        timed_out |= w;
    }
    if (timed_out)
        return fail(PSK_E_HIP, "a run's workgroups sharing a row waited past their bound for one another (the "
                               "device was shared, or its workgroups did not all run at once): that run's "
                               "results are not valid");
    return PSK_OK;
}

extern "C" psk_status psk_group_run_multi(const psk_group* group, const void* const* inputs, void* const* outs,
                                          void* hip_stream)
{
    clear_error();
    if (!group) return fail(PSK_E_NULL, "group is NULL");
    if (!outs) return fail(PSK_E_NULL, "outs is NULL");
    return run_group(group, inputs, outs, hip_stream);
}

extern "C" psk_status psk_group_source(const psk_group_desc* desc, char* buf, size_t cap, size_t* len)
{
    clear_error();
    Analysis an;
    psk_status st = analyse(desc, an);
    if (st != PSK_OK) return st;
    KernelPlan p = plan_kernel(an, true);
    std::string src = emit_source(an, p, "psk_kernel");
    if (len) *len = src.size();
    if (buf && cap) {
        size_t n = std::min(cap - 1, src.size());
        std::memcpy(buf, src.data(), n);
        buf[n] = '\0';
    }
    return PSK_OK;
}

extern "C" psk_status psk_group_code_object(const psk_group_desc* desc, void* buf, size_t cap, size_t* len)
{
    clear_error();
    Analysis an;
    psk_status st = analyse(desc, an);
    if (st != PSK_OK) return st;
    std::shared_ptr<Kernel> k;
    st = get_kernel(an, true, k);
    if (st != PSK_OK) return st;
    if (len) *len = k->code.size();
    if (buf && cap >= k->code.size()) std::memcpy(buf, k->code.data(), k->code.size());
    return PSK_OK;
}

// ------------------------------------------------------------------- trees
namespace {
// one slot buffer of one leaf: [b, e)
struct Range {
    uintptr_t b, e;
    int32_t leaf, slot;
};
}  // namespace

struct psk_tree {
    int32_t n_leaves = 0, n_slots = 0;
    int32_t dt[PSK_MAX_SLOTS] = {};
    TreePlan plan;
    std::vector<LeafDev> leaves;
    std::vector<ChunkDev> chunks;
    LeafDev* d_leaves = nullptr;
    GenLeafDev* d_gleaves = nullptr;  // every slot's address, for tree-mapped groups
    ChunkDev* d_chunks = nullptr;
    double* d_partials = nullptr;   // clipping: one partial sum of squares per chunk
    ClipOut* d_clip = nullptr;      // clipping: squared norm and factor
    std::vector<Range> ranges;      // every slot buffer, sorted by start; equal ranges are adjacent
    uint8_t shared[PSK_MAX_SLOTS][PSK_MAX_SLOTS] = {};   // some leaf has one buffer in both slots
    int device = 0;
    int32_t vector_leaves = 0;
    // AdamW's slot roles (theta, g, m, v [, theta', m', v']): PSK_OK when
    // the tree can take an AdamW step, else why not (checked at the step)
    psk_status adamw_status = PSK_OK;
    std::string adamw_refusal;
    ~psk_tree()
    {
        if (d_leaves) (void)hipFree(d_leaves);
        if (d_gleaves) (void)hipFree(d_gleaves);
        if (d_chunks) (void)hipFree(d_chunks);
        if (d_partials) (void)hipFree(d_partials);
        if (d_clip) (void)hipFree(d_clip);
    }
};

extern "C" psk_status psk_tree_create(const psk_leaf* leaves, int32_t n_leaves, int32_t n_slots,
                                      const int32_t* slot_dtypes, psk_tree** out)
{
    clear_error();
    if (!out) return fail(PSK_E_NULL, "out is NULL");
    *out = nullptr;
    if (n_leaves < 0) return fail(PSK_E_SHAPE, "negative leaf count");
    if (n_leaves > 0 && !leaves) return fail(PSK_E_NULL, "leaves is NULL");
    if (n_slots < 1 || n_slots > PSK_MAX_SLOTS) return fail(PSK_E_SHAPE, "a tree has 1 to 8 slots");
    const bool adamw_roles = n_slots == 4 || n_slots == 7;
    if (!slot_dtypes) return fail(PSK_E_NULL, "slot_dtypes is NULL");
    auto t = std::make_unique<psk_tree>();
    t->n_leaves = n_leaves;
    t->n_slots = n_slots;
    for (int s = 0; s < n_slots; ++s) {
        if (slot_dtypes[s] != PSK_F32 && slot_dtypes[s] != PSK_BF16)
            return fail(PSK_E_TYPE, "slot " + std::to_string(s) + ": storage type must be f32 or bf16");
        t->dt[s] = slot_dtypes[s];
    }
    // what an AdamW step needs beyond a valid tree (refused at the step)
    auto no_adamw = [&](psk_status st, const std::string& why) {
        if (t->adamw_status == PSK_OK) {
            t->adamw_status = st;
            t->adamw_refusal = why;
        }
    };
    if (!adamw_roles)
        no_adamw(PSK_E_SHAPE, "an AdamW tree has 4 slots (theta, g, m, v) or 7 (plus theta', m', v')");
    if (adamw_roles && t->dt[2] != t->dt[3]) no_adamw(PSK_E_TYPE, "m and v must share a storage type");
    if (n_slots == 7 && (t->dt[4] != t->dt[0] || t->dt[5] != t->dt[2] || t->dt[6] != t->dt[3]))
        no_adamw(PSK_E_TYPE, "an output slot must have its input's storage type");
    std::vector<int64_t> numel(n_leaves);
    for (int32_t l = 0; l < n_leaves; ++l) numel[l] = leaves[l].numel;
    psk_status st = plan_tree(numel.data(), n_leaves, PSK_TREE_CHUNK, t->plan);
    if (st != PSK_OK) return st;
    // slot roles: inputs 0..3; outputs of theta, m, v
    const int out_slot[3] = {n_slots == 7 ? 4 : 0, n_slots == 7 ? 5 : 2, n_slots == 7 ? 6 : 3};
    std::vector<Range> ranges;
    t->leaves.resize(n_leaves);
    std::vector<GenLeafDev> gleaves(n_leaves);
    for (int32_t l = 0; l < n_leaves; ++l) {
        const psk_leaf& lf = leaves[l];
        LeafDev& d = t->leaves[l];
        std::memset(&d, 0, sizeof d);
        std::memset(&gleaves[l], 0, sizeof gleaves[l]);
        if (lf.numel == 0) continue;
        bool v16 = true;
        for (int s = 0; s < n_slots; ++s) {
            uintptr_t p = reinterpret_cast<uintptr_t>(lf.slot[s]);
            if (!p) return fail(PSK_E_NULL, "leaf " + std::to_string(l) + " slot " + std::to_string(s) + " is NULL");
            if (p % esize(t->dt[s]))
                return fail(PSK_E_ALIGN, "leaf " + std::to_string(l) + " slot " + std::to_string(s) +
                                             " is not aligned to its element size");
            if (p % 16) v16 = false;
            ranges.push_back({p, p + (uintptr_t)lf.numel * esize(t->dt[s]), l, s});
        }
        if (adamw_roles) {
            for (int s = 0; s < 4; ++s) d.in[s] = lf.slot[s];
            for (int s = 0; s < 3; ++s) d.out[s] = lf.slot[out_slot[s]];
        }
        d.flags = v16 ? 1 : 0;
        for (int s = 0; s < n_slots; ++s) gleaves[l].slot[s] = lf.slot[s];
        gleaves[l].flags = v16 ? 1 : 0;
        t->vector_leaves += v16;
    }
    // aliasing: one buffer may fill two slots of a leaf that share a storage
    // type; any other overlap is refused.  AdamW's roles allow less: only an
    // input and its own output (7 slots) share a buffer.
    std::sort(ranges.begin(), ranges.end(), [](const Range& x, const Range& y) {
        return x.b != y.b ? x.b < y.b : x.e < y.e;
    });
    auto pair_ok = [&](const Range& x, const Range& y) {
        return x.leaf == y.leaf && t->dt[x.slot] == t->dt[y.slot];
    };
    auto adamw_pair_ok = [&](const Range& x, const Range& y) {
        int a = std::min(x.slot, y.slot), b = std::max(x.slot, y.slot);
        if (n_slots == 4) return false;   // in place: every slot is its own buffer
        return (a == 0 && b == 4) || (a == 2 && b == 5) || (a == 3 && b == 6);
    };
    uintptr_t max_end = 0;
    size_t prev = 0;
    for (size_t i = 0; i < ranges.size(); ++i) {
        const Range& r = ranges[i];
        if (i > 0 && r.b < max_end) {
            const Range& q = ranges[prev];
            const std::string what = "leaf " + std::to_string(r.leaf) + " slot " + std::to_string(r.slot) +
                                     " overlaps leaf " + std::to_string(q.leaf) + " slot " + std::to_string(q.slot);
            if (!(q.b == r.b && q.e == r.e && pair_ok(q, r))) return fail(PSK_E_ALIAS, what);
            if (adamw_roles && !adamw_pair_ok(q, r)) no_adamw(PSK_E_ALIAS, what + " (AdamW's slots are distinct)");
        }
        if (r.e > max_end) { max_end = r.e; prev = i; }
    }
    t->ranges = ranges;
    for (size_t i = 0; i < ranges.size();) {
        size_t j = i + 1;
        while (j < ranges.size() && ranges[j].b == ranges[i].b && ranges[j].e == ranges[i].e) ++j;
        for (size_t a = i; a < j; ++a)
            for (size_t b = i; b < j; ++b) t->shared[ranges[a].slot][ranges[b].slot] = 1;
        i = j;
    }
    const size_t nc = t->plan.chunk_leaf.size();
    t->chunks.resize(nc);
    for (size_t c = 0; c < nc; ++c)
        t->chunks[c] = {t->plan.chunk_leaf[c], t->plan.chunk_count[c], t->plan.chunk_start[c]};
    hipError_t e = hipGetDevice(&t->device);
    if (e != hipSuccess) return fail(PSK_E_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    if (n_leaves > 0) {
        e = hipMalloc(&t->d_leaves, sizeof(LeafDev) * (size_t)n_leaves);
        if (e == hipSuccess)
            e = hipMemcpy(t->d_leaves, t->leaves.data(), sizeof(LeafDev) * (size_t)n_leaves, hipMemcpyHostToDevice);
    }
    if (e == hipSuccess && n_leaves > 0) {
        e = hipMalloc(&t->d_gleaves, sizeof(GenLeafDev) * (size_t)n_leaves);
        if (e == hipSuccess)
            e = hipMemcpy(t->d_gleaves, gleaves.data(), sizeof(GenLeafDev) * (size_t)n_leaves, hipMemcpyHostToDevice);
    }
    if (e == hipSuccess && nc > 0) {
        e = hipMalloc(&t->d_chunks, sizeof(ChunkDev) * nc);
        if (e == hipSuccess)
            e = hipMemcpy(t->d_chunks, t->chunks.data(), sizeof(ChunkDev) * nc, hipMemcpyHostToDevice);
    }
    if (e == hipSuccess && nc > 0) {
        // device state of the clipping pass, owned by the tree
        e = hipMalloc(&t->d_partials, sizeof(double) * nc);
        if (e == hipSuccess) e = hipMalloc(&t->d_clip, sizeof(ClipOut));
        if (e == hipSuccess) e = hipMemset(t->d_clip, 0, sizeof(ClipOut));
    }
    if (e != hipSuccess) return fail(PSK_E_HIP, std::string("tree upload: ") + hipGetErrorString(e));
    *out = t.release();
    return PSK_OK;
}

extern "C" void psk_tree_destroy(psk_tree* tree) { delete tree; }

extern "C" psk_status psk_tree_get_info(const psk_tree* tree, psk_tree_info* info)
{
    clear_error();
    if (!tree || !info) return fail(PSK_E_NULL, "tree or info is NULL");
    info->n_leaves = tree->n_leaves;
    info->n_slots = tree->n_slots;
    info->n_chunks = (int64_t)tree->chunks.size();
    info->total_numel = tree->plan.leaf_offset.empty() ? 0 : tree->plan.leaf_offset.back();
    info->chunk_elems = PSK_TREE_CHUNK;
    info->vector_leaves = tree->vector_leaves;
    return PSK_OK;
}

extern "C" psk_status psk_tree_get_tables(const psk_tree* tree, int64_t* leaf_offset, int32_t* chunk_leaf,
                                          int64_t* chunk_start, int32_t* chunk_count)
{
    clear_error();
    if (!tree) return fail(PSK_E_NULL, "tree is NULL");
    const TreePlan& p = tree->plan;
    if (leaf_offset) std::copy(p.leaf_offset.begin(), p.leaf_offset.end(), leaf_offset);
    if (chunk_leaf) std::copy(p.chunk_leaf.begin(), p.chunk_leaf.end(), chunk_leaf);
    if (chunk_start) std::copy(p.chunk_start.begin(), p.chunk_start.end(), chunk_start);
    if (chunk_count) std::copy(p.chunk_count.begin(), p.chunk_count.end(), chunk_count);
    return PSK_OK;
}

extern "C" psk_status psk_tree_plan(const int64_t* numel, int32_t n_leaves, int64_t* n_chunks, int64_t* leaf_offset,
                                    int32_t* chunk_leaf, int64_t* chunk_start, int32_t* chunk_count)
{
    clear_error();
    TreePlan p;
    psk_status st = plan_tree(numel, n_leaves, PSK_TREE_CHUNK, p);
    if (st != PSK_OK) return st;
    if (n_chunks) *n_chunks = (int64_t)p.chunk_leaf.size();
    if (leaf_offset) std::copy(p.leaf_offset.begin(), p.leaf_offset.end(), leaf_offset);
    if (chunk_leaf) std::copy(p.chunk_leaf.begin(), p.chunk_leaf.end(), chunk_leaf);
    if (chunk_start) std::copy(p.chunk_start.begin(), p.chunk_start.end(), chunk_start);
    if (chunk_count) std::copy(p.chunk_count.begin(), p.chunk_count.end(), chunk_count);
    return PSK_OK;
}

extern "C" psk_status psk_adamw_step(const psk_tree* tree, const psk_adamw_hp* hp, void* hip_stream)
{
    clear_error();
    if (!tree || !hp) return fail(PSK_E_NULL, "tree or hp is NULL");
    if (hp->t < 1) return fail(PSK_E_SHAPE, "t counts steps from 1");
    const double v[5] = {hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay};
    for (double x : v)
        if (!std::isfinite(x)) return fail(PSK_E_SHAPE, "hyperparameters must be finite");
    if (tree->adamw_status != PSK_OK) return fail(tree->adamw_status, tree->adamw_refusal);
    if (tree->chunks.empty()) return PSK_OK;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != tree->device)
        return fail(PSK_E_HIP, "the current device is not the device the tree was created on");
    AdamwScalars s = adamw_scalars(*hp);
    return launch_adamw(tree->d_leaves, tree->d_chunks, (int64_t)tree->chunks.size(), tree->dt[0], tree->dt[1],
                        tree->dt[2], s, nullptr, hip_stream);
}

static psk_status schedule_lr(const psk_adamw_config* c, double* lr)
{
    if (c->t < 1) return fail(PSK_E_SHAPE, "t counts steps from 1");
    if (c->schedule == PSK_SCHED_CONSTANT) {
        *lr = c->lr;
        return PSK_OK;
    }
    if (c->schedule != PSK_SCHED_LINEAR && c->schedule != PSK_SCHED_COSINE)
        return fail(PSK_E_OP, "unknown schedule");
    if (c->warmup < 0 || c->warmup >= c->total) return fail(PSK_E_SHAPE, "warmup must satisfy 0 <= warmup < total");
    if (c->t > c->total) return fail(PSK_E_SHAPE, "t is past total");
    const double t = (double)c->t, w = (double)c->warmup, T = (double)c->total;
    if (c->t <= c->warmup) *lr = c->lr * t / w;
    else if (c->schedule == PSK_SCHED_LINEAR) *lr = c->lr * (T - t) / (T - w);
    else *lr = c->lr * 0.5 * (1.0 + std::cos(3.14159265358979323846 * (t - w) / (T - w)));
    return PSK_OK;
}

extern "C" psk_status psk_adamw_lr(const psk_adamw_config* cfg, double* lr)
{
    clear_error();
    if (!cfg || !lr) return fail(PSK_E_NULL, "cfg or lr is NULL");
    return schedule_lr(cfg, lr);
}

// The configured step; the clipping pass keeps its partials and result in
// the tree's device memory, or (no_alloc) in the library's static scratch.
static psk_status adamw_config_step(const psk_tree* tree, const psk_adamw_config* cfg, void* hip_stream,
                                    bool no_alloc)
{
    if (!tree || !cfg) return fail(PSK_E_NULL, "tree or cfg is NULL");
    const double v[6] = {cfg->lr, cfg->beta1, cfg->beta2, cfg->eps, cfg->weight_decay, cfg->grad_clip};
    for (double x : v)
        if (!std::isfinite(x)) return fail(PSK_E_SHAPE, "hyperparameters must be finite");
    double lr = 0.0;
    psk_status st = schedule_lr(cfg, &lr);
    if (st != PSK_OK) return st;
    if (tree->adamw_status != PSK_OK) return fail(tree->adamw_status, tree->adamw_refusal);
    if (tree->chunks.empty()) return PSK_OK;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != tree->device)
        return fail(PSK_E_HIP, "the current device is not the device the tree was created on");
    psk_adamw_hp hp = {lr, cfg->beta1, cfg->beta2, cfg->eps, cfg->weight_decay, cfg->t};
    AdamwScalars s = adamw_scalars(hp);
    const int64_t nc = (int64_t)tree->chunks.size();
    const float* gscale = nullptr;
    if (cfg->grad_clip > 0.0) {
        double* partials = tree->d_partials;
        ClipOut* clip = tree->d_clip;
        if (no_alloc) {
            if (nc > kStaticChunks)
                return fail(PSK_E_UNSUPPORTED, "the tree has " + std::to_string(nc) + " chunks; the static scratch of "
                                               "the clipping pass holds " + std::to_string(kStaticChunks) +
                                               " (trees of up to 2^32 elements)");
            st = static_scratch(&partials, &clip);
            if (st != PSK_OK) return st;
        }
        st = launch_clip(tree->d_leaves, tree->d_chunks, nc, tree->dt[1], partials, clip, cfg->grad_clip, hip_stream);
        if (st != PSK_OK) return st;
        gscale = &clip->factor;
    }
    return launch_adamw(tree->d_leaves, tree->d_chunks, nc, tree->dt[0], tree->dt[1], tree->dt[2], s, gscale,
                        hip_stream);
}

extern "C" psk_status psk_adamw_step_config(const psk_tree* tree, const psk_adamw_config* cfg, void* hip_stream)
{
    clear_error();
    return adamw_config_step(tree, cfg, hip_stream, false);
}

extern "C" psk_status psk_adamw_step_config_noalloc(const psk_tree* tree, const psk_adamw_config* cfg,
                                                    void* hip_stream)
{
    clear_error();
    return adamw_config_step(tree, cfg, hip_stream, true);
}

extern "C" psk_status psk_tree_clip_result(const psk_tree* tree, double* sumsq, float* factor)
{
    clear_error();
    if (!tree) return fail(PSK_E_NULL, "tree is NULL");
    ClipOut h = {0.0, 0.0f, 0.0f};
    if (tree->d_clip) {
        int dev = -1;
        if (hipGetDevice(&dev) != hipSuccess || dev != tree->device)
            return fail(PSK_E_HIP, "the current device is not the device the tree was created on");
        // the step may have run on a non-blocking stream: wait for the whole device
        hipError_t e = hipDeviceSynchronize();
        if (e != hipSuccess) return fail(PSK_E_HIP, std::string("hipDeviceSynchronize: ") + hipGetErrorString(e));
        e = hipMemcpy(&h, tree->d_clip, sizeof h, hipMemcpyDeviceToHost);
        if (e != hipSuccess) return fail(PSK_E_HIP, std::string("hipMemcpy: ") + hipGetErrorString(e));
    }
    if (sumsq) *sumsq = h.sumsq;
    if (factor) *factor = h.factor;
    return PSK_OK;
}

// ------------------------------------------------------- tree-mapped groups
static psk_status run_tree(const psk_group* group, const psk_tree* tree, const int32_t* in_slot,
                           const int32_t* out_slot, const void* const* scalars, void* hip_stream)
{
    const Analysis& an = group->an;
    if (!an.tree) return fail(PSK_E_UNSUPPORTED, "the group was not created with PSK_GROUP_TREE");
    const int n_in = (int)an.inputs.size();
    const int n_out = 1 + (int)an.extras.size();
    if (n_in > 0 && !in_slot) return fail(PSK_E_NULL, "in_slot is NULL");
    std::vector<int> slot_args(n_in + n_out, 0);
    for (int k = 0; k < n_out; ++k) {
        const int s = out_slot[k];
        if (s < 0 || s >= tree->n_slots) return fail(PSK_E_SHAPE, "output slot out of range");
        if (tree->dt[s] != (k == 0 ? an.out_dtype : an.extras[k - 1].dtype))
            return fail(PSK_E_TYPE, "output " + std::to_string(k) + ": the slot's storage type is not the group's");
        for (int j = 0; j < k; ++j)
            if (tree->shared[out_slot[j]][s] || out_slot[j] == s)
                return fail(PSK_E_ALIAS, "outputs " + std::to_string(j) + " and " + std::to_string(k) +
                                             " would write the same buffer");
        slot_args[n_in + k] = s;
    }
    std::vector<const void*> sc(n_in, nullptr);
    for (int k = 0; k < n_in; ++k) {
        const InputInfo& in = an.inputs[k];
        if (!in.used) continue;
        if (in.kind == InKind::Scalar) {
            if (!scalars || !scalars[k]) return fail(PSK_E_NULL, "scalar input " + std::to_string(k) + " is NULL");
            const uintptr_t a = reinterpret_cast<uintptr_t>(scalars[k]);
            if (a % esize(in.dtype)) return fail(PSK_E_ALIGN, "scalar input " + std::to_string(k) + " is misaligned");
            // every thread reads the scalar: it may not lie in a buffer the launch writes.  Ranges
            // that hold a are identical (partial overlaps were refused), so they sit side by side
            // just before the first range that starts after a.
            auto it = std::upper_bound(tree->ranges.begin(), tree->ranges.end(), a,
                                       [](uintptr_t x, const Range& r) { return x < r.b; });
            while (it != tree->ranges.begin()) {
                --it;
                if (a >= it->e) break;
                for (int j = 0; j < n_out; ++j)
                    if (it->slot == out_slot[j])
                        return fail(PSK_E_ALIAS, "scalar input " + std::to_string(k) + " lies in leaf " +
                                                     std::to_string(it->leaf) + "'s output slot " +
                                                     std::to_string(it->slot));
            }
            sc[k] = scalars[k];
        } else {
            const int s = in_slot[k];
            if (s < 0 || s >= tree->n_slots) return fail(PSK_E_SHAPE, "in_slot out of range");
            if (tree->dt[s] != in.dtype)
                return fail(PSK_E_TYPE, "input " + std::to_string(k) + ": the slot's storage type is not the group's");
            slot_args[k] = s;
        }
    }
    if (tree->chunks.empty()) return PSK_OK;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != tree->device)
        return fail(PSK_E_HIP, "the current device is not the device the tree was created on");
    const KernelPlan& kp = group->vec->plan;   // kp.blocks workgroups of kp.block threads per chunk
    const int64_t n_virtual = (int64_t)tree->chunks.size() * kp.blocks;
    const int64_t per = (n_virtual + 7) / 8;
    if (per * 8 > 0x7fffffffLL) return fail(PSK_E_UNSUPPORTED, "tree too large for one launch");
    hipFunction_t fn = nullptr;
    psk_status st = kernel_function(*group->vec, fn);
    if (st != PSK_OK) return st;
    const void* lp = tree->d_gleaves;
    const void* cp = tree->d_chunks;
    unsigned nv = (unsigned)n_virtual, pv = (unsigned)per;
    std::vector<void*> args = {&lp, &cp, &nv, &pv};
    for (int k = 0; k < n_in + n_out; ++k) args.push_back(&slot_args[k]);
    for (int k = 0; k < n_in; ++k) args.push_back(&sc[k]);
    hipError_t e = hipModuleLaunchKernel(fn, (unsigned)(per * 8), 1, 1, (unsigned)kp.block, 1, 1, 0,
                                         static_cast<hipStream_t>(hip_stream), args.data(), nullptr);
    if (e != hipSuccess) return fail(PSK_E_HIP, std::string("hipModuleLaunchKernel: ") + hipGetErrorString(e));
    count_launch();
    return PSK_OK;
}

extern "C" psk_status psk_group_run_tree(const psk_group* group, const psk_tree* tree, const int32_t* in_slot,
                                         int32_t out_slot, const void* const* scalars, void* hip_stream)
{
    clear_error();
    if (!group || !tree) return fail(PSK_E_NULL, "group or tree is NULL");
    if (!group->an.extras.empty())
        return fail(PSK_E_UNSUPPORTED, "the group has extra outputs: run it with psk_group_run_tree_multi");
    const int32_t outs[1] = {out_slot};
    return run_tree(group, tree, in_slot, outs, scalars, hip_stream);
}

extern "C" psk_status psk_group_run_tree_multi(const psk_group* group, const psk_tree* tree, const int32_t* in_slot,
                                               const int32_t* out_slot, const void* const* scalars, void* hip_stream)
{
    clear_error();
    if (!group || !tree) return fail(PSK_E_NULL, "group or tree is NULL");
    if (!out_slot) return fail(PSK_E_NULL, "out_slot is NULL");
    return run_tree(group, tree, in_slot, out_slot, scalars, hip_stream);
}

// --------------------------------------------------------------- partition
extern "C" psk_status psk_partition(int32_t n, const psk_node* body, const psk_tensor_desc* types,
                                    const uint8_t* is_output, int32_t* group_of, int32_t* is_root, int32_t* n_groups)
{
    clear_error();
    return partition(n, body, types, is_output, 0u, group_of, is_root, n_groups);
}

extern "C" psk_status psk_partition_ex(int32_t n, const psk_node* body, const psk_tensor_desc* types,
                                       const uint8_t* is_output, uint32_t flags, int32_t* group_of, int32_t* is_root,
                                       int32_t* n_groups)
{
    clear_error();
    return partition(n, body, types, is_output, flags, group_of, is_root, n_groups);
}

extern "C" psk_status psk_dispatch_count(int32_t n, const psk_node* body, const psk_tensor_desc* types,
                                         const uint8_t* is_output, uint32_t flags, psk_dispatch_report* report)
{
    clear_error();
    return dispatch_count(n, body, types, is_output, flags, report);
}

// -------------------------------------------------------------------- misc
extern "C" const char* psk_last_error(void) { return t_last_error.c_str(); }

extern "C" const char* psk_status_str(psk_status s)
{
    switch (s) {
    case PSK_OK: return "PSK_OK";
    case PSK_E_NULL: return "PSK_E_NULL";
    case PSK_E_CAP: return "PSK_E_CAP";
    case PSK_E_ORDER: return "PSK_E_ORDER";
    case PSK_E_ROOT: return "PSK_E_ROOT";
    case PSK_E_DEAD: return "PSK_E_DEAD";
    case PSK_E_OP: return "PSK_E_OP";
    case PSK_E_TYPE: return "PSK_E_TYPE";
    case PSK_E_BROADCAST: return "PSK_E_BROADCAST";
    case PSK_E_ROW: return "PSK_E_ROW";
    case PSK_E_ALIGN: return "PSK_E_ALIGN";
    case PSK_E_ALIAS: return "PSK_E_ALIAS";
    case PSK_E_SHAPE: return "PSK_E_SHAPE";
    case PSK_E_UNSUPPORTED: return "PSK_E_UNSUPPORTED";
    case PSK_E_JIT: return "PSK_E_JIT";
    case PSK_E_HIP: return "PSK_E_HIP";
    }
    return "PSK_E_UNKNOWN";
}

extern "C" int32_t psk_version(void) { return PSK_VERSION; }

extern "C" psk_status psk_get_stats(psk_stats* stats)
{
    clear_error();
    if (!stats) return fail(PSK_E_NULL, "stats is NULL");
    stats->launches = g_launches.load();
    stats->jit_compiles = g_jit_compiles.load();
    stats->jit_hits = g_jit_hits.load();
    return PSK_OK;
}
