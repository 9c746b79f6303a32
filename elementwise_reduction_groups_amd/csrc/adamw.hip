// Multi-tensor AdamW: one launch for every leaf of a parameter tree.
//
// The optimizer step is one elementwise chain over every parameter (presk
// manual, "PSK-Realize", section "What a group is", parameter trees; the
// formula is the presk language reference's, section "Configuration blocks", the optimizer).  Here the
// chain is mapped over all leaves in a single launch: a device-side chunk
// table (leaf index, first element, count; 4096 elements per chunk) is split
// into 8 workgroups per chunk; a workgroup reads its chunk entry and the
// leaf's slot addresses from a device-side leaf table and streams 512
// elements, 4 consecutive ones per thread.  The three results theta', m', v'
// are stored once each; theta' reads m' and v' as stored (they are outputs),
// which matters only for bf16 moments.
//
// Arithmetic is f32, one rounding per operation in the formula's order: this
// file is compiled with -ffp-contract=off, correctly rounded division and
// square root, and no denormal flush, so it reproduces the plain sequential
// evaluation bit for bit.
#include <hip/hip_runtime.h>

#include <mutex>

#include "psk_internal.h"

namespace psk {

// ------------------------------------------- static scratch (no allocation)
// The clipping pass's per-chunk partial sums and its result (ClipOut) for
// psk_adamw_step_config_noalloc, the entry point for callers that cannot
// allocate: a file-scope device array, one copy on every GPU the library
// runs on, alive until the process ends.  kStaticChunks partials followed
// by one ClipOut (two doubles' room); trees of up to 2^20 chunks (2^32
// elements).  Nothing here must start at zero: the sum-of-squares kernel
// writes every partial it covers and the combine writes the result.
static __device__ __align__(256) double scratch[kStaticChunks + 2];

static std::mutex g_scratch_mu;
static double* g_scratch[kMaxScratchDevices] = {};

// The device address of `scratch` on the current device, looked up once per
// device with that device current.  Host code never passes the array's own
// name to a kernel: on the host it is a stand-in, not a device address.
psk_status static_scratch(double** partials, ClipOut** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(PSK_E_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxScratchDevices) return fail(PSK_E_HIP, "device index out of range");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(PSK_E_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
        g_scratch[dev] = static_cast<double*>(p);
    }
    *partials = g_scratch[dev];
    *out = reinterpret_cast<ClipOut*>(g_scratch[dev] + kStaticChunks);
    return PSK_OK;
}

namespace {

// Launch shape, chosen by measurement on MI355X over the 145-leaf tree
// (bf16 theta and g, f32 m and v; medians of 12 runs): workgroups of 128
// threads, 2 elements per thread (4-byte bf16 and 8-byte f32 accesses, one
// per stream), nontemporal loads and stores (every byte is touched once):
// 6.14 TB/s with each XCD given one contiguous eighth of the chunks,
// against 5.99 with 4 elements per thread, 6.03 with 2 elements and
// 64-thread workgroups, 6.09 with 512-thread workgroups.  Storing theta'
// first, loading the moments first or reading the leaf pointers from the
// chunk table change nothing measurable.  Workgroups taken in the
// dispatcher's round-robin order instead (consecutive blocks on
// consecutive XCDs, every XCD in the same stretch of the tree) run at 6.62
// TB/s against 6.10 for the contiguous eighths in the same process (2.951
// against 3.204 ms), so that is the default.
constexpr int kBlock = 128;
constexpr int kPer = 2;                                   // elements per thread
constexpr int kSub = PSK_TREE_CHUNK / (kBlock * kPer);   // workgroups per chunk
static_assert(kSub * kBlock * kPer == PSK_TREE_CHUNK, "a chunk must split into whole workgroups");
constexpr int kXcds = 8;

typedef float f2v __attribute__((ext_vector_type(2)));
typedef __bf16 b2v __attribute__((ext_vector_type(2)));
typedef unsigned u2v __attribute__((ext_vector_type(2)));
typedef unsigned u4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ unsigned pack_bf16(float a, float b)
{
    f2v f = {a, b};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f, b2v));
}

// Slot addresses come out of a device-side table, so the compiler cannot
// tell that they point to global memory and would use generic (flat)
// accesses.  Every data access goes through these casts to the global
// address space instead, which gives global loads and stores.
#define PSK_GLOBAL __attribute__((address_space(1)))
template <typename T> __device__ __forceinline__ const PSK_GLOBAL T* gbl(const void* p, int64_t e)
{
    return (const PSK_GLOBAL T*)p + e;   // address-space casts take the C form
}
template <typename T> __device__ __forceinline__ PSK_GLOBAL T* gbl(void* p, int64_t e)
{
    return (PSK_GLOBAL T*)p + e;
}

template <typename T> struct Io;

// The step's stores: relaxed stores of device (agent) scope, which gfx950
// issues with the sc1 cache policy.  Measured on the 145-leaf tree (one
// process, the launches interleaved): 3.065 -> 2.968 ms for a step right
// after a step, 2.998 -> 2.951 ms after a 1 GiB read, against nontemporal
// stores (nt); with sc1 and nt together 3.009 / 2.942, with no policy bits
// 3.25 / 3.20.  The loads stay nontemporal: relaxed loads of device or
// system scope, or plain ones, take 3.14 / 3.12 ms.
template <typename W> __device__ __forceinline__ void store_dev(PSK_GLOBAL W* p, W w)
{
    __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <> struct Io<float> {
    static __device__ __forceinline__ void load4(const void* p, int64_t e, float* x)
    {
        u4v w = __builtin_nontemporal_load((const PSK_GLOBAL u4v*)gbl<float>(p, e));
        x[0] = __uint_as_float(w[0]); x[1] = __uint_as_float(w[1]);
        x[2] = __uint_as_float(w[2]); x[3] = __uint_as_float(w[3]);
    }
    static __device__ __forceinline__ void load2(const void* p, int64_t e, float* x)
    {
        u2v w = __builtin_nontemporal_load((const PSK_GLOBAL u2v*)gbl<float>(p, e));
        x[0] = __uint_as_float(w[0]); x[1] = __uint_as_float(w[1]);
    }
    static __device__ __forceinline__ float load1(const void* p, int64_t e) { return *gbl<float>(p, e); }
    static __device__ __forceinline__ void store2(void* p, int64_t e, const float* x)
    {
        const u2v w = {__float_as_uint(x[0]), __float_as_uint(x[1])};
        store_dev((PSK_GLOBAL unsigned long long*)gbl<float>(p, e), __builtin_bit_cast(unsigned long long, w));
    }
    static __device__ __forceinline__ void store1(void* p, int64_t e, float x) { *gbl<float>(p, e) = x; }
    static __device__ __forceinline__ float through(float x) { return x; }
};

template <> struct Io<__bf16> {
    // 8 elements, one 16-byte access
    static __device__ __forceinline__ void load8(const void* p, int64_t e, float* x)
    {
        u4v w = __builtin_nontemporal_load((const PSK_GLOBAL u4v*)gbl<unsigned short>(p, e));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            x[2 * q] = __uint_as_float(w[q] << 16);
            x[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void load2(const void* p, int64_t e, float* x)
    {
        unsigned w = __builtin_nontemporal_load((const PSK_GLOBAL unsigned*)gbl<unsigned short>(p, e));
        x[0] = __uint_as_float(w << 16); x[1] = __uint_as_float(w & 0xffff0000u);
    }
    static __device__ __forceinline__ float load1(const void* p, int64_t e)
    {
        return __uint_as_float(((unsigned)*gbl<unsigned short>(p, e)) << 16);
    }
    static __device__ __forceinline__ void store2(void* p, int64_t e, const float* x)
    {
        store_dev((PSK_GLOBAL unsigned*)gbl<unsigned short>(p, e), pack_bf16(x[0], x[1]));
    }
    static __device__ __forceinline__ void store1(void* p, int64_t e, float x)
    {
        *gbl<unsigned short>(p, e) = (unsigned short)(pack_bf16(x, 0.0f) & 0xffffu);
    }
    // the value a store leaves behind, read back
    static __device__ __forceinline__ float through(float x)
    {
        return __uint_as_float(pack_bf16(x, 0.0f) << 16);
    }
};

// Workgroups are dispatched to the XCDs round robin (block b runs on XCD
// b mod 8).  The grid is padded to 8 * per blocks; with per_xcd given,
// block b takes virtual block (b mod 8) * per + b / 8, so XCD x works
// through the contiguous range [x * per, (x + 1) * per); with per_xcd 0
// block b is virtual block b.  Virtual blocks past the end exit.
__device__ __forceinline__ unsigned xcd_block(unsigned b, unsigned per) { return (b % kXcds) * per + b / kXcds; }

// a / b for a divisor b in [2^-40, 2^40] shared by every element, given y,
// the correctly rounded 1/b: q = a*y is within an ulp of a/b, the fma gives
// the exact remainder a - b*q, and a second fma rounds q + remainder*y to
// the correctly rounded quotient (Markstein).  That needs a zero or in
// [2^-86, 2^87] (no underflow of the remainder, no overflow of q); `bad`
// records a lane where it is not.  A zero a returns q itself, which keeps
// the sign of -0.
__device__ __forceinline__ float div_shared(float a, float b, float y, bool& bad)
{
    const float q = a * y;
    const float rem = fmaf(-q, b, a);
    const bool zero = a == 0.0f;
    bad |= !((fabsf(a) >= 0x1p-86f || zero) && fabsf(a) <= 0x1p87f);
    return zero ? q : fmaf(rem, y, q);
}

template <typename TP, typename TG, typename TM, bool SCALE>
__global__ void __launch_bounds__(kBlock)
adamw_tree_kernel(const LeafDev* __restrict__ leaves, const ChunkDev* __restrict__ chunks, unsigned n_virtual,
                  unsigned per_xcd, AdamwScalars s, const float* __restrict__ gscale)
{
    const unsigned vb = per_xcd ? xcd_block(blockIdx.x, per_xcd) : blockIdx.x;
    if (vb >= n_virtual) return;
    const ChunkDev ch = chunks[vb / kSub];
    const LeafDev L = leaves[ch.leaf];     // the seven slots and the flags, read together
    const int i0 = ((int)(vb % kSub) * kBlock + (int)threadIdx.x) * kPer;   // offset within the chunk
    const int cnt = ch.count - i0;
    if (cnt <= 0) return;
    const int64_t e0 = ch.start + i0;
    const bool full = (L.flags & 1) != 0 && cnt >= kPer;

    float th[kPer], g[kPer], m[kPer], v[kPer];
    if (full) {
        Io<TP>::load2(L.in[0], e0, th);
        Io<TG>::load2(L.in[1], e0, g);
        Io<TM>::load2(L.in[2], e0, m);
        Io<TM>::load2(L.in[3], e0, v);
    } else {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            th[j] = g[j] = m[j] = v[j] = 0.0f;
            if (j < cnt) {
                th[j] = Io<TP>::load1(L.in[0], e0 + j);
                g[j] = Io<TG>::load1(L.in[1], e0 + j);
                m[j] = Io<TM>::load1(L.in[2], e0 + j);
                v[j] = Io<TM>::load1(L.in[3], e0 + j);
            }
        }
    }
    // the moments first: their stores leave while theta' is computed
    float to[kPer], mo[kPer], vo[kPer];
    const float gs = SCALE ? *gscale : 1.0f;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const float gj = SCALE ? g[j] * gs : g[j];
        mo[j] = Io<TM>::through(s.b1 * m[j] + s.c1 * gj);
        vo[j] = Io<TM>::through(s.b2 * v[j] + s.c2 * (gj * gj));
    }
    if (full) {
        Io<TM>::store2(L.out[1], e0, mo);
        Io<TM>::store2(L.out[2], e0, vo);
    } else {
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            if (j < cnt) {
                Io<TM>::store1(L.out[1], e0 + j, mo[j]);
                Io<TM>::store1(L.out[2], e0 + j, vo[j]);
            }
    }
    // the bias corrections: by the reciprocals where the host gave them and
    // every dividend lies in range, else by division, which gives the same
    // bits
    float mh[kPer], vh[kPer];
    bool bad = s.rc1 == 0.0f;
    if (!bad) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            mh[j] = div_shared(mo[j], s.bc1, s.rc1, bad);
            vh[j] = div_shared(vo[j], s.bc2, s.rc2, bad);
        }
    }
    if (bad) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            mh[j] = mo[j] / s.bc1;
            vh[j] = vo[j] / s.bc2;
        }
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const float upd = mh[j] / (sqrtf(vh[j]) + s.eps) + s.wd * th[j];
        to[j] = th[j] - s.lr * upd;
    }
    if (full) {
        Io<TP>::store2(L.out[0], e0, to);
    } else {
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            if (j < cnt) Io<TP>::store1(L.out[0], e0 + j, to[j]);
    }
}

template <typename TP, typename TG, typename TM>
hipError_t launch(const LeafDev* l, const ChunkDev* c, int64_t n_chunks, const AdamwScalars& s, const float* gscale,
                  hipStream_t st)
{
    const int64_t n_virtual = n_chunks * kSub;
    const int64_t per = (n_virtual + kXcds - 1) / kXcds;
    if (per * kXcds > 0x7fffffffLL) return hipErrorInvalidValue;
    const unsigned pv = layout_value("axcd", 0) ? (unsigned)per : 0u;
    if (gscale)
        hipLaunchKernelGGL((adamw_tree_kernel<TP, TG, TM, true>), dim3((unsigned)(per * kXcds)), dim3(kBlock), 0, st,
                           l, c, (unsigned)n_virtual, pv, s, gscale);
    else
        hipLaunchKernelGGL((adamw_tree_kernel<TP, TG, TM, false>), dim3((unsigned)(per * kXcds)), dim3(kBlock), 0,
                           st, l, c, (unsigned)n_virtual, pv, s, gscale);
    return hipGetLastError();
}

// ------------------------------------------------------ global-norm clipping
constexpr int kClipBlock = 256;
constexpr int kClipPer = PSK_TREE_CHUNK / kClipBlock;      // 16 elements per thread
static_assert(kClipPer % 4 == 0, "clip pass reads 4 elements at a time");

__device__ __forceinline__ double wave_sum(double x)
{
    // butterfly over the 64 lanes; every lane ends with the same sum
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
    return x;
}

template <typename TG>
__global__ void __launch_bounds__(kClipBlock)
sumsq_kernel(const LeafDev* __restrict__ leaves, const ChunkDev* __restrict__ chunks,
             double* __restrict__ partials)
{
    __shared__ double red[kClipBlock / 64];
    const ChunkDev ch = chunks[blockIdx.x];
    const LeafDev L = leaves[ch.leaf];
    const bool vec = (L.flags & 1) != 0;
    double acc = 0.0;
    // squares of f32 values are exact in f64; the sum runs in f64
    // 16-byte accesses: 4 f32 or 8 bf16 elements
    constexpr int kW = sizeof(TG) == 2 ? 8 : 4;
#pragma unroll
    for (int k = 0; k < kClipPer / kW; ++k) {
        const int i0 = (k * kClipBlock + (int)threadIdx.x) * kW;
        const int cnt = ch.count - i0;
        float x[kW];
#pragma unroll
        for (int j = 0; j < kW; ++j) x[j] = 0.0f;
        if (vec && cnt >= kW) {
            if constexpr (kW == 8) Io<TG>::load8(L.in[1], ch.start + i0, x);
            else Io<TG>::load4(L.in[1], ch.start + i0, x);
        } else {
#pragma unroll
            for (int j = 0; j < kW; ++j)
                if (j < cnt) x[j] = Io<TG>::load1(L.in[1], ch.start + i0 + j);
        }
#pragma unroll
        for (int j = 0; j < kW; ++j) acc += (double)x[j] * (double)x[j];
    }
    acc = wave_sum(acc);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        double p = red[0];
        for (int w = 1; w < kClipBlock / 64; ++w) p += red[w];
        partials[blockIdx.x] = p;
    }
}

// One workgroup: the chunk partials combined in a fixed order (each thread
// a fixed strided subset in increasing order, then a fixed tree), so the
// result is reproducible; then the factor, formed in f64.
constexpr int kFinalBlock = 1024;
__global__ void __launch_bounds__(kFinalBlock)
clip_finalize_kernel(const double* __restrict__ partials, unsigned n, ClipOut* out, double c)
{
    __shared__ double red[kFinalBlock / 64];
    double s = 0.0;
    // loads issued ahead, additions in increasing i as before
#pragma unroll 8
    for (unsigned i = threadIdx.x; i < n; i += kFinalBlock) s += partials[i];
    s = wave_sum(s);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = red[0];
        for (int w = 1; w < kFinalBlock / 64; ++w) t += red[w];
        double f = c / (sqrt(t) + 1e-6);
        if (!(f < 1.0)) f = 1.0;
        out->sumsq = t;
        out->factor = (float)f;
    }
}

}  // namespace

psk_status launch_clip(const LeafDev* d_leaves, const ChunkDev* d_chunks, int64_t n_chunks, int grad_dt,
                       double* partials, ClipOut* out, double c, void* stream)
{
    if (n_chunks <= 0) return PSK_OK;
    if (n_chunks > 0x7fffffffLL) return fail(PSK_E_UNSUPPORTED, "too many chunks");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (grad_dt == PSK_BF16)
        hipLaunchKernelGGL((sumsq_kernel<__bf16>), dim3((unsigned)n_chunks), dim3(kClipBlock), 0, st, d_leaves,
                           d_chunks, partials);
    else
        hipLaunchKernelGGL((sumsq_kernel<float>), dim3((unsigned)n_chunks), dim3(kClipBlock), 0, st, d_leaves,
                           d_chunks, partials);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) {
        hipLaunchKernelGGL(clip_finalize_kernel, dim3(1), dim3(kFinalBlock), 0, st, (const double*)partials,
                           (unsigned)n_chunks, out, c);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return fail(PSK_E_HIP, std::string("clip launch: ") + hipGetErrorString(e));
    count_launch();
    count_launch();
    return PSK_OK;
}

psk_status launch_adamw(const LeafDev* d_leaves, const ChunkDev* d_chunks, int64_t n_chunks, int theta_dt,
                        int grad_dt, int mv_dt, const AdamwScalars& s, const float* gscale, void* stream)
{
    if (n_chunks <= 0) return PSK_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int key = (theta_dt == PSK_BF16) * 4 + (grad_dt == PSK_BF16) * 2 + (mv_dt == PSK_BF16);
    hipError_t e;
    switch (key) {
    case 0: e = launch<float, float, float>(d_leaves, d_chunks, n_chunks, s, gscale, st); break;
    case 1: e = launch<float, float, __bf16>(d_leaves, d_chunks, n_chunks, s, gscale, st); break;
    case 2: e = launch<float, __bf16, float>(d_leaves, d_chunks, n_chunks, s, gscale, st); break;
    case 3: e = launch<float, __bf16, __bf16>(d_leaves, d_chunks, n_chunks, s, gscale, st); break;
    case 4: e = launch<__bf16, float, float>(d_leaves, d_chunks, n_chunks, s, gscale, st); break;
    case 5: e = launch<__bf16, float, __bf16>(d_leaves, d_chunks, n_chunks, s, gscale, st); break;
    case 6: e = launch<__bf16, __bf16, float>(d_leaves, d_chunks, n_chunks, s, gscale, st); break;
    default: e = launch<__bf16, __bf16, __bf16>(d_leaves, d_chunks, n_chunks, s, gscale, st); break;
    }
    if (e != hipSuccess) return fail(PSK_E_HIP, std::string("AdamW launch: ") + hipGetErrorString(e));
    count_launch();
    return PSK_OK;
}

}  // namespace psk
