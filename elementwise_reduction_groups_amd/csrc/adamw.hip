// Multi-tensor AdamW: one launch for every leaf of a parameter tree.
//
// The optimizer step is one elementwise chain over every parameter (presk
// manual, "PSK-Realize", section "What a group is", parameter trees; the
// formula is the presk language reference's, "The optimizer").  Here the
// chain is mapped over all leaves in a single launch: workgroup b takes chunk
// b of a device-side chunk table (leaf index, first element, count), reads
// the leaf's slot addresses from a device-side leaf table, and streams its
// 4096 elements.  Each thread handles 8 consecutive elements per step with
// 16-byte accesses (one for 8 bf16, two for 8 f32), two steps per thread,
// with every load of both steps issued before the arithmetic.  The three
// results theta', m', v' are stored once each; theta' reads m' and v' as
// stored (they are outputs), which matters only for bf16 moments.
//
// Arithmetic is f32, one rounding per operation in the formula's order: this
// file is compiled with -ffp-contract=off, correctly rounded division and
// square root, and no denormal flush, so it reproduces the plain sequential
// evaluation bit for bit.
#include <hip/hip_runtime.h>

#include "psk_internal.h"

namespace psk {
namespace {

constexpr int kBlock = 256;
constexpr int kPer = 8;                          // elements per thread per step
constexpr int kSteps = PSK_TREE_CHUNK / (kBlock * kPer);
static_assert(kSteps * kBlock * kPer == PSK_TREE_CHUNK, "chunk must be a whole number of steps");

typedef float f2v __attribute__((ext_vector_type(2)));
typedef __bf16 b2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ unsigned pack_bf16(float a, float b)
{
    f2v f = {a, b};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f, b2v));
}

template <typename T> struct Io;

template <> struct Io<float> {
    static __device__ __forceinline__ void load8(const void* p, int64_t e, float* x)
    {
        const float4* q = reinterpret_cast<const float4*>(static_cast<const float*>(p) + e);
        float4 a = q[0], b = q[1];
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
    static __device__ __forceinline__ float load1(const void* p, int64_t e) { return static_cast<const float*>(p)[e]; }
    static __device__ __forceinline__ void store8(void* p, int64_t e, const float* x)
    {
        float4* q = reinterpret_cast<float4*>(static_cast<float*>(p) + e);
        q[0] = make_float4(x[0], x[1], x[2], x[3]);
        q[1] = make_float4(x[4], x[5], x[6], x[7]);
    }
    static __device__ __forceinline__ void store1(void* p, int64_t e, float x) { static_cast<float*>(p)[e] = x; }
    static __device__ __forceinline__ float through(float x) { return x; }
};

template <> struct Io<__bf16> {
    static __device__ __forceinline__ void load8(const void* p, int64_t e, float* x)
    {
        uint4 w = *reinterpret_cast<const uint4*>(static_cast<const unsigned short*>(p) + e);
        const unsigned ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x[2 * k] = __uint_as_float(ws[k] << 16);
            x[2 * k + 1] = __uint_as_float(ws[k] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ float load1(const void* p, int64_t e)
    {
        return __uint_as_float(((unsigned)static_cast<const unsigned short*>(p)[e]) << 16);
    }
    static __device__ __forceinline__ void store8(void* p, int64_t e, const float* x)
    {
        *reinterpret_cast<uint4*>(static_cast<unsigned short*>(p) + e) =
            make_uint4(pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]), pack_bf16(x[6], x[7]));
    }
    static __device__ __forceinline__ void store1(void* p, int64_t e, float x)
    {
        static_cast<unsigned short*>(p)[e] = (unsigned short)(pack_bf16(x, 0.0f) & 0xffffu);
    }
    // the value a store leaves behind, read back
    static __device__ __forceinline__ float through(float x)
    {
        return __uint_as_float(pack_bf16(x, 0.0f) << 16);
    }
};

template <typename TP, typename TG, typename TM>
__global__ void __launch_bounds__(kBlock)
adamw_tree_kernel(const LeafDev* __restrict__ leaves, const ChunkDev* __restrict__ chunks, AdamwScalars s)
{
    const ChunkDev ch = chunks[blockIdx.x];
    const LeafDev L = leaves[ch.leaf];
    const bool vec = (L.flags & 1) != 0;

    float th[kSteps][kPer], g[kSteps][kPer], m[kSteps][kPer], v[kSteps][kPer];
    int64_t e0[kSteps];
    bool full[kSteps];
    int cnt[kSteps];
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
        const int i0 = (u * kBlock + (int)threadIdx.x) * kPer;   // offset within the chunk
        e0[u] = ch.start + i0;
        cnt[u] = ch.count - i0;
        full[u] = vec && cnt[u] >= kPer;
        if (full[u]) {
            Io<TP>::load8(L.in[0], e0[u], th[u]);
            Io<TG>::load8(L.in[1], e0[u], g[u]);
            Io<TM>::load8(L.in[2], e0[u], m[u]);
            Io<TM>::load8(L.in[3], e0[u], v[u]);
        } else {
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                th[u][j] = g[u][j] = m[u][j] = v[u][j] = 0.0f;
                if (j < cnt[u]) {
                    th[u][j] = Io<TP>::load1(L.in[0], e0[u] + j);
                    g[u][j] = Io<TG>::load1(L.in[1], e0[u] + j);
                    m[u][j] = Io<TM>::load1(L.in[2], e0[u] + j);
                    v[u][j] = Io<TM>::load1(L.in[3], e0[u] + j);
                }
            }
        }
    }
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
        if (cnt[u] <= 0) continue;
        float to[kPer], mo[kPer], vo[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const float gj = g[u][j];
            float m2 = s.b1 * m[u][j] + s.c1 * gj;
            float v2 = s.b2 * v[u][j] + s.c2 * (gj * gj);
            m2 = Io<TM>::through(m2);
            v2 = Io<TM>::through(v2);
            const float mh = m2 / s.bc1;
            const float vh = v2 / s.bc2;
            const float upd = mh / (sqrtf(vh) + s.eps) + s.wd * th[u][j];
            to[j] = th[u][j] - s.lr * upd;
            mo[j] = m2;
            vo[j] = v2;
        }
        if (full[u]) {
            Io<TP>::store8(L.out[0], e0[u], to);
            Io<TM>::store8(L.out[1], e0[u], mo);
            Io<TM>::store8(L.out[2], e0[u], vo);
        } else {
#pragma unroll
            for (int j = 0; j < kPer; ++j)
                if (j < cnt[u]) {
                    Io<TP>::store1(L.out[0], e0[u] + j, to[j]);
                    Io<TM>::store1(L.out[1], e0[u] + j, mo[j]);
                    Io<TM>::store1(L.out[2], e0[u] + j, vo[j]);
                }
        }
    }
}

template <typename TP, typename TG, typename TM>
hipError_t launch(const LeafDev* l, const ChunkDev* c, int64_t n, const AdamwScalars& s, hipStream_t st)
{
    hipLaunchKernelGGL((adamw_tree_kernel<TP, TG, TM>), dim3((unsigned)n), dim3(kBlock), 0, st, l, c, s);
    return hipGetLastError();
}

}  // namespace

psk_status launch_adamw(const LeafDev* d_leaves, const ChunkDev* d_chunks, int64_t n_chunks, int theta_dt,
                        int grad_dt, int mv_dt, const AdamwScalars& s, void* stream)
{
    if (n_chunks <= 0) return PSK_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int key = (theta_dt == PSK_BF16) * 4 + (grad_dt == PSK_BF16) * 2 + (mv_dt == PSK_BF16);
    hipError_t e;
    switch (key) {
    case 0: e = launch<float, float, float>(d_leaves, d_chunks, n_chunks, s, st); break;
    case 1: e = launch<float, float, __bf16>(d_leaves, d_chunks, n_chunks, s, st); break;
    case 2: e = launch<float, __bf16, float>(d_leaves, d_chunks, n_chunks, s, st); break;
    case 3: e = launch<float, __bf16, __bf16>(d_leaves, d_chunks, n_chunks, s, st); break;
    case 4: e = launch<__bf16, float, float>(d_leaves, d_chunks, n_chunks, s, st); break;
    case 5: e = launch<__bf16, float, __bf16>(d_leaves, d_chunks, n_chunks, s, st); break;
    case 6: e = launch<__bf16, __bf16, float>(d_leaves, d_chunks, n_chunks, s, st); break;
    default: e = launch<__bf16, __bf16, __bf16>(d_leaves, d_chunks, n_chunks, s, st); break;
    }
    if (e != hipSuccess) return fail(PSK_E_HIP, std::string("AdamW launch: ") + hipGetErrorString(e));
    count_launch();
    return PSK_OK;
}

}  // namespace psk
