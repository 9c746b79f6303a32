// HIP source emitter: a validated group and its launch plan become one
// gfx950 kernel.
//
// Kernel shapes (poot, "Fusion and Planning", section "Kernel
// specialization": elementwise = one thread per element; reduction = block
// reduce with the epilogue in the same kernel):
//
//  * pointwise: each thread owns `vec` consecutive output elements, loads
//    every input at its broadcast position with 16-byte accesses where the
//    layout allows, evaluates the members in let order in f32 registers and
//    stores the root (and any extra stored values) once, rounded to its
//    storage type;
//
//  * row: `lanes` threads own one row of the [rows, cols] output view; each
//    lane holds nv vectors of vec elements (columns (k*lanes + lane)*vec + j,
//    so every wave access is contiguous).  The members are evaluated phase by
//    phase: phase p computes the values that depend on p reductions, then
//    the reductions of phase p run lane-sequentially, across the lanes with
//    DPP (and a lane swizzle for 32-lane rows) and across waves through LDS.
//    The row stays in registers, so each input is read from HBM once; a
//    persistent variant walks several rows per workgroup;
//
//  * tiled row: rows too wide for registers are walked in tiles by every
//    phase, the leading tiles' inputs kept in registers and the next ones in
//    LDS, the rest re-read; odd phases walk from the last tile to the first,
//    so they begin where the phase before ended (in L2);
//
//  * tree-mapped: the group over every leaf of a parameter tree, one launch,
//    chunks of leaves from a device table.
//
// Every value is a named SSA register: a value read twice is read twice from
// its register, never recomputed from memory nor written back.  Nothing is
// contracted (the JIT compiles with -ffp-contract=off, correctly rounded
// division and square root).  The deliberate departures, each declared:
// the reduction tree's bracketing; division by a row value through a
// correctly rounded reciprocal and Markstein's correction (IEEE results); and,
// for members that only bf16 results depend on, the reciprocal product, the
// short erfc exponent in gelu and the short exponential in softmax; the
// opt-in online normalizer.
//
// Host-only: nothing here calls HIP.
#include <cinttypes>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <sstream>

#include "psk_internal.h"

namespace psk {

uint64_t fnv1a(const std::string& s)
{
    uint64_t h = 1469598103934665603ull;
    for (unsigned char ch : s) {
        h ^= ch;
        h *= 1099511628211ull;
    }
    return h;
}

// A literal f32 operand.  +0.0 is emitted as psk_pz(), a zero the compiler
// cannot see through: the backend folds 0 - x, when another instruction
// reads it, into a negation of x, which gives -0 where 0 - (+0) is +0.
static std::string flit(float x)
{
    if (x == 0.0f && !std::signbit(x)) return "psk_pz()";
    if (std::isnan(x)) return "__builtin_nanf(\"\")";
    if (std::isinf(x)) return x > 0 ? "__builtin_inff()" : "(-__builtin_inff())";
    char buf[64];
    std::snprintf(buf, sizeof buf, "%af", (double)x);
    return std::string("(") + buf + ")";
}

// ops whose value depends on the node's imm field: a constant's value and
// WHERE's fill; the kernel cache key must carry its bits for both
static bool op_reads_imm(int op) { return op == PSK_OP_CONST || op == PSK_OP_WHERE; }

std::string canonical_text(const Analysis& an)
{
    std::ostringstream s;
    s << "out " << an.out_dtype << " [" << an.out_shape4[0] << "," << an.out_shape4[1] << "," << an.out_shape4[2]
      << "," << an.out_shape4[3] << "] root " << an.root << "\n";
    for (size_t k = 0; k < an.inputs.size(); ++k) {
        const InputInfo& in = an.inputs[k];
        s << "in" << k << " " << in.dtype << " [" << in.aligned[0] << "," << in.aligned[1] << "," << in.aligned[2]
          << "," << in.aligned[3] << "] step [" << in.stride4[0] << "," << in.stride4[1] << "," << in.stride4[2]
          << "," << in.stride4[3] << "]\n";
    }
    for (size_t i = 0; i < an.nodes.size(); ++i) {
        const psk_node& nd = an.nodes[i];
        uint32_t bits;
        std::memcpy(&bits, &nd.imm, 4);
        s << i << " " << nd.op << " " << nd.a << " " << nd.b << " " << nd.c << " " << nd.iparam << " "
          << (op_reads_imm(nd.op) ? bits : 0u) << "\n";
    }
    for (const auto& x : an.extras) s << "extra " << x.node << " " << x.dtype << " " << (x.per_row ? 1 : 0) << "\n";
    s << "flags " << an.flags << "\n";
    return s.str();
}

namespace {

const char* kPrelude = R"PSK(
typedef unsigned int psk_u32;
typedef unsigned short psk_u16;
typedef unsigned char psk_u8;
typedef float psk_f2 __attribute__((ext_vector_type(2)));
typedef __bf16 psk_b2 __attribute__((ext_vector_type(2)));
typedef unsigned psk_u4v __attribute__((ext_vector_type(4)));
typedef unsigned psk_u2v __attribute__((ext_vector_type(2)));
// every input byte is read once and every output byte written once:
// nontemporal accesses when PSK_NT is set
template <typename T> __device__ __forceinline__ T psk_ld(const T* p) {
#if PSK_NT
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}
// a relaxed store of device scope (the sc1 cache policy), 16 bytes as two
// of 8
template <typename T> __device__ __forceinline__ void psk_st_dev(T* p, T v) {
  if constexpr (sizeof(T) == 16) {
    unsigned long long* q = (unsigned long long*)p;
    const psk_u4v w = __builtin_bit_cast(psk_u4v, v);
    __hip_atomic_store(q, ((unsigned long long)w[1] << 32) | w[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + 1, ((unsigned long long)w[3] << 32) | w[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else if constexpr (sizeof(T) == 8) {
    __hip_atomic_store((unsigned long long*)p, __builtin_bit_cast(unsigned long long, v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  } else if constexpr (sizeof(T) == 4) {
    __hip_atomic_store((unsigned*)p, __builtin_bit_cast(unsigned, v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    __hip_atomic_store((unsigned short*)p, __builtin_bit_cast(unsigned short, v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}
template <typename T> __device__ __forceinline__ void psk_st(T* p, T v) {
#if PSK_SC1
  psk_st_dev(p, v);
#elif PSK_NT
  __builtin_nontemporal_store(v, p);
#else
  *p = v;
#endif
}
// a load whose data is read again (an early phase of the tiled row kernel)
template <typename T> __device__ __forceinline__ T psk_ldc(const T* p) { return *p; }
// the same for pointers named as global memory (addresses read from a
// device table would otherwise be accessed through generic instructions)
#define PSK_G __attribute__((address_space(1)))
template <typename T> __device__ __forceinline__ T psk_ld(const PSK_G T* p) {
#if PSK_NT
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}
template <typename T> __device__ __forceinline__ void psk_st(PSK_G T* p, T v) {
#if PSK_SC1
  psk_st_dev((T*)p, v);
#elif PSK_NT
  __builtin_nontemporal_store(v, p);
#else
  *p = v;
#endif
}
// bf16 is the top half of a binary32: widening is a shift
__device__ __forceinline__ float psk_lo(psk_u32 w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float psk_hi(psk_u32 w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float psk_h(psk_u16 h) { return __uint_as_float(((psk_u32)h) << 16); }
// round two f32 to nearest-even bf16 and pack them (v_cvt_pk_bf16_f32)
__device__ __forceinline__ psk_u32 psk_pack2(float a, float b) {
  psk_f2 f = {a, b};
  return __builtin_bit_cast(psk_u32, __builtin_convertvector(f, psk_b2));
}
__device__ __forceinline__ psk_u16 psk_r1(float a) { return (psk_u16)(psk_pack2(a, 0.0f) & 0xffffu); }
// a value as stored to bf16 and read back (members read stored values so)
__device__ __forceinline__ float psk_rt(float a) { return psk_h(psk_r1(a)); }
// gelu(x) = x * Phi(x) with Phi(x) = erfc(-x/sqrt 2) / 2.  erfc(w), w >= 0,
// is the Chebyshev-fitted form of Press, Teukolsky, Vetterling and Flannery,
// Numerical Recipes (2nd ed.), section 6.2: erfc(w) = t exp(-w^2 + P(t)),
// t = 1/(1 + w/2), fractional error below 1.2e-7 for all w >= 0.  The
// exponent z = P(t) - w^2 is formed with one rounding (an fma), taken to
// base 2 and passed to the hardware 2^x.  The roundings of z and of its
// base-2 form grow with w^2: against erfc of the same rounded w the result
// is within 1.2e-6 relative where |x| <= 4.3 (emulated in f32 with a
// correctly rounded 2^x and reciprocal), negligible beside gelu's size
// beyond.  Results of 2^x below 2^-126 (|x|
// above about 13.2) may be flushed to zero: gelu is then below 1e-37 in
// magnitude, inside the f32 tolerance's absolute part.  For x > 0,
// Phi = 1 - erfc(w)/2.  w is clamped at 10, where erfc(w) < 2^-149: Phi is
// then 0 or 1, also for infinite x (a NaN x stays NaN).
__device__ __forceinline__ float psk_gelu(float x) {
  const float w = fminf(fabsf(x) * 0.70710678118654752440f, 10.0f);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.5f, w, 1.0f));
  float p = 0.17087277f;
  p = fmaf(p, t, -0.82215223f); p = fmaf(p, t, 1.48851587f); p = fmaf(p, t, -1.13520398f);
  p = fmaf(p, t, 0.27886807f);  p = fmaf(p, t, -0.18628806f); p = fmaf(p, t, 0.09678418f);
  p = fmaf(p, t, 0.37409196f);  p = fmaf(p, t, 1.00002368f);  p = fmaf(p, t, -1.26551223f);
  const float ec = t * __builtin_amdgcn_exp2f(fmaf(-w, w, p) * 1.44269504088896341f);
  const float phi = (x > 0.0f) ? fmaf(-0.5f, ec, 1.0f) : 0.5f * ec;
  return x * phi;
}
// gelu whose value is only rounded to bf16 (a stored result of a group
// whose results are all bf16, read by no member): the same form with a
// degree-5 exponent polynomial, fitted here (weighted least squares towards
// minimax on t in [1/6, 1], w in [0, 10]); its relative error in erfc is
// below 8e-6.  erfc(w)/2 = t 2^(z - 1) is taken as 2^(z + 63) 2^-64: the
// shifted argument keeps the hardware 2^x in its normal range and the exact
// scaling by 2^-64 makes the tiny results subnormal, at the price of one
// more rounding of the exponent (relative error below 3e-6).  All far inside
// a bf16 half-ulp (2^-9): the rounded result is the exact one's or its
// neighbour.
__device__ __forceinline__ float psk_gelu_b(float x) {
  const float w = fminf(fabsf(x) * 0.70710678118654752440f, 10.0f);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.5f, w, 1.0f));
  float p = 0.228792509f;
  p = fmaf(p, t, -0.709197821f); p = fmaf(p, t, 0.474501494f); p = fmaf(p, t, 0.254438582f);
  p = fmaf(p, t, 1.01801471f);   p = fmaf(p, t, -1.26654186f);
  const float z = fmaf(fmaf(-w, w, p), 1.44269504088896341f, 63.0f);
  const float half_ec = t * (__builtin_amdgcn_exp2f(z) * 0x1p-64f);
  const float phi = (x > 0.0f) ? 1.0f - half_ec : half_ec;
  return x * phi;
}
// tanh of a = |x| >= 0 on either side of 0.625.  Below: a + a^3 P(a^2), P
// of degree 4 fitted here (Lawson-weighted least squares towards minimax
// relative error on [0, 0.625]; 0.07 ulp as a real polynomial, below 0.75
// ulp evaluated in f32).  Above: 1 - 2/(1 + e^{2a}), e^{2a} formed as
// 2^t (1 + r ln 2) with t = fl(2a log2 e) and r its remainder from two fmas
// (2 log2 e to about 2^-48), so the argument's rounding does not grow with
// a; with the hardware 2^x and reciprocal each within an ulp the result is
// within 2.5 ulps (emulated in f32 with both off by an ulp either way).  a
// is clamped at 16, where tanh rounds to 1, so e stays finite.
__device__ __forceinline__ float psk_tanh_lo(float a) {
  const float u = a * a;
  float p = -0x1.75e62ap-8f;
  p = fmaf(p, u, 0x1.52279p-6f); p = fmaf(p, u, -0x1.b83c7ep-5f); p = fmaf(p, u, 0x1.110728p-3f);
  p = fmaf(p, u, -0x1.555532p-2f);
  return fmaf(a * u, p, a);
}
__device__ __forceinline__ float psk_tanh_hi(float a) {
  const float ac = fminf(a, 16.0f);
  const float t = ac * 0x1.715476p+1f;
  const float r = fmaf(ac, 0x1.4ae0cp-25f, fmaf(ac, 0x1.715476p+1f, -t));
  const float e2 = __builtin_amdgcn_exp2f(t);
  const float e = fmaf(e2, r * 0x1.62e43p-1f, e2);
  return fmaf(-2.0f, __builtin_amdgcn_rcpf(e + 1.0f), 1.0f);
}
// tanh(x): the side for |x| taken with the sign of x last (-0 stays -0,
// infinite x gives +-1, a NaN x takes the lower side: NaN).  A wave whose
// active lanes all fall on one side evaluates that side alone (the test is
// wave-uniform, so the branch is a scalar one); a mixed wave evaluates both
// and selects.
__device__ __forceinline__ float psk_tanh(float x) {
  const float a = fabsf(x);
  const bool hi = a >= 0.625f;
  const unsigned long long m = __builtin_amdgcn_ballot_w64(hi);
  float r;
  if (m == 0) r = psk_tanh_lo(a);
  else if (m == __builtin_amdgcn_read_exec()) r = psk_tanh_hi(a);
  else r = hi ? psk_tanh_hi(a) : psk_tanh_lo(a);
  return __builtin_copysignf(r, x);
}
// the same values without the wave-uniform test
__device__ __forceinline__ float psk_tanh_s(float x) {
  const float a = fabsf(x);
  return __builtin_copysignf(a >= 0.625f ? psk_tanh_hi(a) : psk_tanh_lo(a), x);
}
// exp(x) for an argument known to be <= 0 (an element minus its row's
// maximum) whose value only reaches bf16 results: 2^(x log2 e + 64) 2^-64,
// the hardware 2^x kept in its normal range by the shift and the exact
// power-of-two scaling making tiny results subnormal (or 0).  The rounding
// of log2 e and of the fused multiply-add cost a relative error below
// about 6e-6 for x >= -88 (far inside a bf16 half-ulp, 2^-9); -inf gives 0
// and NaN stays NaN.
__device__ __forceinline__ float psk_exp_np_b(float x) {
  return __builtin_amdgcn_exp2f(fmaf(x, 1.44269504088896341f, 64.0f)) * 0x1p-64f;
}
// exp(x) for an argument known to be <= 0 whose results reach f32 values
// through well-conditioned operations: x log2 e split into t = fl(x L) and
// its remainder r = x L - t, formed with two fmas (L + L_lo is log2 e to
// about 2^-48), then exp(x) = 2^t (1 + r ln 2): the hardware 2^t (within an
// ulp), one multiply-add, r^2 terms below 2^-34.  Within about two f32 ulps,
// in eight instructions (the library's expf takes fourteen).  Results below
// 2^-126 may be flushed to 0 (far below the f32 tolerance's absolute
// part); -inf gives 0 and NaN stays NaN.
__device__ __forceinline__ float psk_exp_np(float x) {
  const float t = x * 1.44269504088896341f;
  const float r = fmaf(x, 1.925963033500e-8f, fmaf(x, 1.44269504088896341f, -t));
  const float p = __builtin_amdgcn_exp2f(t);
  return (t > -128.0f) ? fmaf(p, r * 0.693147180559945309f, p) : p;
}
// a / b for a value b shared by the whole row, given b's magnitude, the
// correctly rounded y = 1/|b| and b's sign bit sg: the quotient is
// (a with sg applied) / |b|, the same value (rounding to nearest is
// symmetric).  q = a*y is within an ulp of a/|b|; the fma gives the exact
// remainder a - |b|*q, and one more fma rounds q + remainder*y to the
// correctly rounded quotient (Markstein's correction).  That holds while
// |b| lies in [2^-40, 2^40] and a is zero or in [2^-86, 2^87] (no underflow
// of the remainder, no overflow of q).  For a zero a the remainder, formed
// as -(q*|b| - a), is -0, and -0 * y added to q leaves q, a zero of a's
// sign (with a negative y it would not: +0 / -2 would come out +0, hence
// the positive divisor).  The range of a group of dividends is gathered two
// elements an instruction: `lo` keeps the least of (bits(a) << 1) - 2 (the
// magnitude's bits less one, doubled; a zero wraps to the top, so zeros
// never count as small), `hi` the largest |a| (an infinity counts; a NaN
// dividend gives NaN either way).  psk_divr_bad then says whether the group
// must be redone with IEEE division.
__device__ __forceinline__ float psk_divr(float a, float b, float y, unsigned sg, unsigned& lo, float& hi) {
  a = __uint_as_float(__float_as_uint(a) ^ sg);
  const float q = a * y;
  const float rem = -fmaf(q, b, -a);
  const unsigned t = (__float_as_uint(a) << 1) - 2u;
  lo = t < lo ? t : lo;
  hi = fmaxf(hi, fabsf(a));
  return fmaf(rem, y, q);
}
__device__ __forceinline__ bool psk_divr_bad(unsigned lo, float hi) {
  return lo < (0x14800000u << 1) - 2u || !(hi <= 0x1p87f);   // 0x14800000: 2^-86
}
// +0.0 as an opaque register value (see the emitter's literals)
__device__ __forceinline__ float psk_pz() { float z = 0.0f; __asm__("" : "+v"(z)); return z; }
__device__ __forceinline__ float psk_max(float a, float b) { return (a > b) ? a : b; }
__device__ __forceinline__ float psk_min(float a, float b) { return (a < b) ? a : b; }
// one step of a row maximum: IEEE 754-2019 maximum (NaN on either side
// gives NaN; +0 above -0), so the row's maximum does not depend on the order
// lanes and waves combine in; v_maximum3_f32 takes two elements a step
__device__ __forceinline__ float psk_rmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
// the same step by compares and selects, for kernels at their register cap
// (the tiled row kernel): there the compiler's scheduling around the
// maximum instructions spilled registers.  A NaN on either side gives NaN;
// of two equal values the bitwise AND is that value, and +0 for zeros of
// both signs
__device__ __forceinline__ float psk_rmax_s(float a, float b) {
  const float r = (a > b || a != a) ? a : b;
  return (a == b) ? __uint_as_float(__float_as_uint(a) & __float_as_uint(b)) : r;
}
#define PSK_DPP(x, ctl) __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, (x)), (ctl), 0xF, 0xF, false))
#define PSK_RL(x, l) __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, (x)), (l)))
// all-reduce within each 16-lane row: xor 1, xor 2 (quad_perm), then the
// half-row and row mirrors; every lane of the row ends with the same value
__device__ __forceinline__ float psk_sum16(float x) {
  x = x + PSK_DPP(x, 0xB1); x = x + PSK_DPP(x, 0x4E);
  x = x + PSK_DPP(x, 0x141); x = x + PSK_DPP(x, 0x140); return x;
}
__device__ __forceinline__ float psk_max16(float x) {
  x = psk_rmax(x, PSK_DPP(x, 0xB1)); x = psk_rmax(x, PSK_DPP(x, 0x4E));
  x = psk_rmax(x, PSK_DPP(x, 0x141)); x = psk_rmax(x, PSK_DPP(x, 0x140)); return x;
}
// 32 lanes: the 16-lane results of the two halves combined, the lower
// half's first (ds_swizzle in bit mode, xor 16, exchanges them within each
// 32-lane group); `upper`: the lane is in the upper half
#define PSK_SWZ16(x) __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, (x)), 0x401F))
__device__ __forceinline__ float psk_sum32(float x, bool upper) {
  x = psk_sum16(x);
  const float y = PSK_SWZ16(x);
  return upper ? y + x : x + y;
}
__device__ __forceinline__ float psk_max32(float x, bool upper) {
  x = psk_max16(x);
  const float y = PSK_SWZ16(x);
  return upper ? psk_rmax(y, x) : psk_rmax(x, y);
}
// whole wave: the four row results combined in lane order 0, 16, 32, 48
__device__ __forceinline__ float psk_sum64(float x) {
  x = psk_sum16(x);
  return ((PSK_RL(x, 0) + PSK_RL(x, 16)) + PSK_RL(x, 32)) + PSK_RL(x, 48);
}
__device__ __forceinline__ float psk_max64(float x) {
  x = psk_max16(x);
  return psk_rmax(psk_rmax(psk_rmax(PSK_RL(x, 0), PSK_RL(x, 16)), PSK_RL(x, 32)), PSK_RL(x, 48));
}
)PSK";

// Split rows: the workgroups that share a row exchange their partial row
// values through device memory.  A partial travels with its tag in one
// 64-bit word, stored and loaded as a relaxed atomic at device scope: a
// reader that sees the tag sees that value, so no fence is needed.  Waits
// are bounded: a wait that runs out of tries (or finds that another wait
// of the launch already has) records it in *status and goes on with what
// it holds (the host reports it; the row's results are then not to be
// used).  Nothing is stored through the scalar cache.
const char* kSplitPrelude = R"PSK(
__device__ __forceinline__ void psk_put(unsigned long long* p, unsigned tag, float v) {
  __hip_atomic_store(p, ((unsigned long long)tag << 32) | (unsigned long long)__float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float psk_take(unsigned long long* p, unsigned tag, int limit, unsigned* status) {
  unsigned long long w = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int n = 0; (unsigned)(w >> 32) != tag; ++n) {
    if (n >= limit || __hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
      __hip_atomic_store(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
    w = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return __uint_as_float((unsigned)w);
}
)PSK";

struct Emitter {
    const Analysis& an;
    const KernelPlan& pl;
    std::ostringstream o;
    int NE;                 // elements per thread
    bool big;               // 64-bit indexing
    int period = 0;         // causal mask period (0: none)
    bool ragged = false;    // some lane columns fall past the row end

    // node -> some f32 stored value depends on it (through any members)
    std::vector<char> f32_reach;
    // node -> every path from it to a stored value keeps a small relative
    // error small: products, quotients, selections, sign and magnitude
    // operations, square roots, squares, maxima and minima, and the row sum
    // of a never-negative exponential (no sum or difference that can cancel,
    // no logarithm)
    std::vector<char> conditioned;
    // node -> the most gelus on any path from it to a stored value whose
    // other steps are all well-conditioned as above (kUncond: some path
    // passes an operation that may cancel).  gelu's relative condition
    // number 1 + x phi(x)/Phi(x) stays below about 170 wherever its result
    // is a normal f32 (x > -13), so one gelu turns a relative error of 1.5
    // f32 ulps (2e-7) into at most 3e-5, far inside a bf16 half-ulp (2^-9)
    std::vector<int> gelu_path;
    static constexpr int kUncond = 1 << 20;

    Emitter(const Analysis& a, const KernelPlan& p) : an(a), pl(p)
    {
        const int n = (int)an.nodes.size();
        f32_reach.assign(n, 0);
        for (int i = n - 1; i >= 0; --i) {
            const bool f32_store = (i == an.root && an.out_dtype != PSK_BF16) ||
                                   (an.stored[i] > 0 && an.extras[an.stored[i] - 1].dtype != PSK_BF16);
            if (f32_store) f32_reach[i] = 1;
            if (!f32_reach[i]) continue;
            const psk_node& nd = an.nodes[i];
            const int32_t opnd[3] = {nd.a, nd.b, nd.c};
            for (int k = 0; k < op_arity(nd.op); ++k) f32_reach[opnd[k]] = 1;
        }
        conditioned.assign(n, 1);
        for (int j = n - 1; j >= 0; --j) {
            const psk_node& nd = an.nodes[j];
            const int32_t opnd[3] = {nd.a, nd.b, nd.c};
            for (int k = 0; k < op_arity(nd.op); ++k) {
                bool ok = conditioned[j];
                switch (nd.op) {
                case PSK_OP_MUL: case PSK_OP_DIV: case PSK_OP_NEG: case PSK_OP_ABS: case PSK_OP_SQRT:
                case PSK_OP_POW2: case PSK_OP_MAX: case PSK_OP_MIN: case PSK_OP_CAUSAL_MASK: case PSK_OP_ROW_MAX:
                    break;
                case PSK_OP_WHERE: ok = ok && k == 1; break;            // the value, not the mask
                case PSK_OP_SELECT: ok = ok && k != 0; break;           // a chosen value, not the condition
                case PSK_OP_ROW_SUM: ok = ok && an.nodes[opnd[k]].op == PSK_OP_EXP; break;
                default: ok = false;
                }
                if (!ok) conditioned[opnd[k]] = 0;
            }
        }
        gelu_path.assign(n, 0);
        for (int j = n - 1; j >= 0; --j) {
            const psk_node& nd = an.nodes[j];
            const int32_t opnd[3] = {nd.a, nd.b, nd.c};
            for (int k = 0; k < op_arity(nd.op); ++k) {
                int via = gelu_path[j];
                switch (nd.op) {
                case PSK_OP_MUL: case PSK_OP_DIV: case PSK_OP_NEG: case PSK_OP_ABS: case PSK_OP_SQRT:
                case PSK_OP_POW2: case PSK_OP_MAX: case PSK_OP_MIN: case PSK_OP_CAUSAL_MASK: case PSK_OP_ROW_MAX:
                    break;
                case PSK_OP_GELU: via = std::min(kUncond, via + 1); break;
                case PSK_OP_WHERE: if (k != 1) via = kUncond; break;
                case PSK_OP_SELECT: if (k == 0) via = kUncond; break;
                case PSK_OP_ROW_SUM: if (an.nodes[opnd[k]].op != PSK_OP_EXP) via = kUncond; break;
                default: via = kUncond;
                }
                gelu_path[opnd[k]] = std::max(gelu_path[opnd[k]], via);
            }
        }
        NE = (pl.kind == 1 || pl.kind == 3 || pl.kind == 4 ? pl.nv : 1) * pl.vec;   // tree: elements per thread
        big = an.numel >= (int64_t(1) << 31) - 4096 || an.max_span >= (int64_t(1) << 31) - 4096;
        for (auto& nd : an.nodes)
            if (nd.op == PSK_OP_CAUSAL_MASK) period = nd.iparam;
        // online sums whose exponentials the maximum's pass keeps: on rows
        // held in registers that pass sees every element of the lane at once
        kept_sum.assign(n, -1);
        if ((pl.kind == 1 || pl.kind == 4) && !pl.persist)
            for (int i = 0; i < n; ++i)
                if (an.online_max[i] >= 0) kept_sum[an.nodes[i].a] = i;
        if (pl.kind == 1)
            ragged = (int64_t)pl.nv * pl.lanes * pl.vec != an.cols;
        if (pl.kind == 3)
            ragged = an.cols % ((int64_t)pl.nv * pl.lanes * pl.vec) != 0;
        if (pl.kind == 4)
            ragged = (int64_t)pl.split * pl.nv * pl.lanes * pl.vec != an.cols;
    }

    const char* I() const { return big ? "long long" : "int"; }

    // column expression of element e of this thread
    std::string col(int e) const
    {
        int k = e / pl.vec, j = e % pl.vec;
        if (pl.kind == 1 || pl.kind == 3 || pl.kind == 4)
            return "(c" + std::to_string(k) + " + " + std::to_string(j) + ")";
        return "(c0 + " + std::to_string(j) + ")";
    }

    // value of node i at element e (element value or a row value)
    std::string val(int i, int e) const
    {
        if (use_refused) return refused(i);
        if (an.is_row[i]) return "r" + std::to_string(i);
        return "v" + std::to_string(i) + "_" + std::to_string(e);
    }

    // node i's value at a refused position: a row value
    std::string refused(int i) const
    {
        if (an.is_row[i]) return "r" + std::to_string(i);
        return "u" + std::to_string(i);
    }

    std::string refused_expr(int i) const
    {
        const psk_node& nd = an.nodes[i];
        if (nd.op == PSK_OP_CAUSAL_MASK) return "(-__builtin_inff())";
        if (nd.op == PSK_OP_WHERE) return flit(nd.imm);      // the group's one mask refuses here
        // the member's own expression with every operand at its refused value
        Emitter& self = const_cast<Emitter&>(*this);
        self.use_refused = true;
        std::string s = expr(i, 0);
        self.use_refused = false;
        return s;
    }

    bool use_refused = false;
    std::vector<int> kept_sum;    // exp node -> the online sum whose pass keeps its values, or -1
    bool divr_ok = true;          // row-value divisors use psk_divr
    bool cached_loads = false;    // loads whose data a later phase reads again
    std::string ld_fn() const { return cached_loads ? "psk_ldc" : "psk_ld"; }

    // node i's defining expression as its readers see it: a value stored as
    // bf16 (an extra output) is read back rounded
    std::string rt(int i, const std::string& e) const { return an.rounded(i) ? "psk_rt(" + e + ")" : e; }
    void round_elems(int i, const std::vector<int>& elems, const char* indent)
    {
        if (!an.rounded(i)) return;
        for (int e : elems) o << indent << "v" << i << "_" << e << " = psk_rt(v" << i << "_" << e << ");\n";
    }

    // a row value that divides element values: its reciprocal, once per row
    void row_reciprocal(int i)
    {
        if (!divr_ok) return;
        bool used = false;
        for (size_t j = 0; j < an.nodes.size(); ++j)
            if (an.nodes[j].op == PSK_OP_DIV && an.nodes[j].b == i && !an.is_row[j]) used = true;
        if (!used) return;
        // the correctly rounded reciprocal; for psk_divr the divisor's
        // magnitude, its reciprocal's (the same rounding, mirrored) and its
        // sign bit
        o << "    const float y" << i << " = 1.0f / r" << i << ";\n";
        o << "    const float ra" << i << " = fabsf(r" << i << ");\n";
        o << "    const float ya" << i << " = fabsf(y" << i << ");\n";
        o << "    const unsigned sg" << i << " = __float_as_uint(r" << i << ") & 0x80000000u;\n";
        o << "    const bool yok" << i << " = ra" << i << " >= 0x1p-40f && ra" << i << " <= 0x1p40f;\n";
    }

    // element divided by a row value (a reduction's result, or a scalar)
    bool row_div(int i) const
    {
        const psk_node& nd = an.nodes[i];
        return !use_refused && divr_ok && nd.op == PSK_OP_DIV && !an.is_row[i] && an.is_row[nd.b];
    }

    // the other element divisions by a row value: Markstein's correction
    bool divr_node(int i) const { return row_div(i) && !recip_node(i); }

    // node i's value is stored only as bf16 and read by no member: it
    // reaches memory only through a rounding to 8 significant bits
    bool bf16_terminal(int i) const
    {
        if (f32_reach[i] || an.n_readers[i] != 0) return false;
        return i == an.root || an.stored[i] > 0;
    }

    // exp(y - row_max(y)): an argument that is <= 0 (or NaN)
    bool exp_nonpos(int i) const
    {
        const psk_node& nd = an.nodes[i];
        if (nd.op != PSK_OP_EXP) return false;
        const psk_node& d = an.nodes[nd.a];
        return d.op == PSK_OP_SUB && an.nodes[d.b].op == PSK_OP_ROW_MAX && an.nodes[d.b].a == d.a;
    }

    // ... whose value only bf16 results depend on, through well-conditioned
    // operations: the short exponential
    bool cheap_exp(int i) const { return exp_nonpos(i) && !f32_reach[i] && conditioned[i]; }

    // ... whose value f32 results depend on, through well-conditioned
    // operations: the split-product exponential (about two ulps)
    bool split_exp(int i) const { return pl.fexp && exp_nonpos(i) && f32_reach[i] && conditioned[i]; }

    // element / row statistic (a value computed from a reduction) that only
    // bf16 results depend on, through well-conditioned operations and at
    // most one gelu: the row's reciprocal (correctly rounded) times the
    // element, within 1.5 f32 ulps of the quotient.  A division by a scalar
    // input, or one whose error a later sum or difference could magnify
    // (LayerNorm's + beta), stays correctly rounded.
    bool recip_node(int i) const
    {
        return row_div(i) && !f32_reach[i] && an.depth[an.nodes[i].b] > 0 && gelu_path[i] <= 1;
    }

    // elements of member i (given as element indices) written through
    // psk_divr: declare the group's range accumulators before, and after,
    // redo the group with IEEE division where the divisor or a dividend
    // lies outside the range the correction covers
    void divr_open(int i)
    {
        if (divr_node(i)) o << "    unsigned lo" << i << " = 0xffffffffu; float hi" << i << " = 0.0f;\n";
    }
    void divr_close(int i, const std::vector<int>& elems, const char* indent)
    {
        if (!divr_node(i)) return;
        const psk_node& nd = an.nodes[i];
        o << indent << "if (!yok" << nd.b << " || psk_divr_bad(lo" << i << ", hi" << i << ")) {\n";
        for (int e : elems)
            o << indent << "  v" << i << "_" << e << " = " << val(nd.a, e) << " / " << val(nd.b, e) << ";\n";
        o << indent << "}\n";
    }

    std::string expr(int i, int e) const
    {
        const psk_node& nd = an.nodes[i];
        if (!use_refused && kept_sum[i] >= 0) {
            // exp(y - row maximum) as the maximum's pass left it: exp(y - m)
            // for the lane's maximum m, times exp(m - row maximum)
            const std::string s = std::to_string(kept_sum[i]);
            return "(oe" + s + "_" + std::to_string(e) + " * osc" + s + ")";
        }
        auto A = [&] { return val(nd.a, e); };
        auto B = [&] { return val(nd.b, e); };
        auto C = [&] { return val(nd.c, e); };
        switch (nd.op) {
        case PSK_OP_ADD: return "(" + A() + " + " + B() + ")";
        case PSK_OP_SUB: return "(" + A() + " - " + B() + ")";
        case PSK_OP_MUL: return "(" + A() + " * " + B() + ")";
        case PSK_OP_DIV:
            if (recip_node(i)) return "(" + A() + " * y" + std::to_string(nd.b) + ")";
            if (divr_node(i))
                return "psk_divr(" + A() + ", ra" + std::to_string(nd.b) + ", ya" + std::to_string(nd.b) + ", sg" +
                       std::to_string(nd.b) + ", lo" + std::to_string(i) +
                       ", hi" + std::to_string(i) + ")";
            return "(" + A() + " / " + B() + ")";
        case PSK_OP_MAX: return "psk_max(" + A() + ", " + B() + ")";
        case PSK_OP_MIN: return "psk_min(" + A() + ", " + B() + ")";
        case PSK_OP_NEG: return "(-" + A() + ")";
        case PSK_OP_ABS: return "fabsf(" + A() + ")";
        case PSK_OP_EXP: return std::string(cheap_exp(i) ? "psk_exp_np_b(" : split_exp(i) ? "psk_exp_np(" : "expf(") +
                                A() + ")";
        case PSK_OP_LOG: return "logf(" + A() + ")";
        case PSK_OP_SQRT: return "sqrtf(" + A() + ")";
        case PSK_OP_TANH: return std::string(pl.ftanh == 0 ? "tanhf(" : pl.ftanh == 2 ? "psk_tanh_s(" : "psk_tanh(") +
                                 A() + ")";
        case PSK_OP_ERF: return "erff(" + A() + ")";
        case PSK_OP_GELU: return (bf16_terminal(i) ? "psk_gelu_b(" : "psk_gelu(") + A() + ")";
        case PSK_OP_SQRTABS: return "sqrtf(fabsf(" + A() + "))";
        case PSK_OP_POW2: return "(" + A() + " * " + A() + ")";
        case PSK_OP_POWN: {
            if (nd.iparam == 0) return "1.0f";
            std::string s = A();
            for (int k = 1; k < nd.iparam; ++k) s = "(" + s + " * " + A() + ")";
            return s;
        }
        case PSK_OP_SELECT: return "((" + A() + " != 0.0f) ? " + B() + " : " + C() + ")";
        case PSK_OP_WHERE: return "((" + A() + " != 0.0f) ? " + B() + " : " + flit(nd.imm) + ")";
        case PSK_OP_CAUSAL_MASK: return "((" + col(e) + " <= q) ? " + A() + " : (-__builtin_inff()))";
        default: return "0.0f";
        }
    }

    static int esize(psk_dtype d) { return d == PSK_BF16 ? 2 : d == PSK_U8 ? 1 : 4; }

    std::string ptype(psk_dtype d) const { return d == PSK_BF16 ? "psk_u16" : d == PSK_U8 ? "psk_u8" : "float"; }

    // a loaded element as f32: bf16 widened, a mask byte as 0.0 or its value
    static std::string widen(psk_dtype d, const std::string& x)
    {
        if (d == PSK_BF16) return "psk_h(" + x + ")";
        if (d == PSK_U8) return "(float)(" + x + ")";
        return x;
    }

    // offset expression of input k's row part for the current row variable
    // `rv`: each leading output axis's index times the input's step along it
    std::string row_offset(const InputInfo& in, const std::string& rv) const
    {
        // output leading axes O0,O1,O2 (right-aligned), row = (i0*O1 + i1)*O2 + i2
        const int64_t* O = an.out_shape4;
        const int64_t* st = in.stride4;
        std::string s = "0";
        for (int d = 0; d < 3; ++d) {
            if (st[d] == 0) continue;
            int64_t inner = 1;
            for (int dd = d + 1; dd < 3; ++dd) inner *= O[dd];
            std::string idx = "(" + rv;
            if (inner != 1) idx += " / (" + std::string(I()) + ")" + std::to_string(inner);
            idx += ")";
            if (d > 0) idx = "(" + idx + " % (" + std::string(I()) + ")" + std::to_string(O[d]) + ")";
            s += " + " + idx + " * (" + std::string(I()) + ")" + std::to_string(st[d]);
        }
        return s;
    }

    // The variables a vector load of input k at element e0 fills before
    // widening: type, name, zero value, and the loaded expression's type and
    // element offset (one 4-, 8- or 16-byte load each; V == 1 loads a float).
    struct RawVar { std::string type, name, zero; int eoff; };
    std::vector<RawVar> raw_vars(int k, int e0) const
    {
        const InputInfo& in = an.inputs[k];
        const int V = pl.vec;
        const std::string ks = std::to_string(k), es = std::to_string(e0);
        if (V == 1) return {{"float", "x" + ks + "_" + es, "0.0f", 0}};
        if (in.dtype == PSK_U8) {
            const int nw = std::max(1, V / 4);
            return {{nw == 1 ? "psk_u32" : nw == 2 ? "psk_u2v" : "psk_u4v", "w" + ks + "_" + es, "{}", 0}};
        }
        std::vector<RawVar> r;
        const int nwords = V * esize(in.dtype) / 4, epw = 4 / esize(in.dtype);
        int piece = 0;
        for (int w = 0; w < nwords; w += 4, ++piece) {
            const bool four = nwords - w >= 4;
            r.push_back({four ? "psk_u4v" : "psk_u2v", "w" + ks + "_" + es + "_" + std::to_string(piece),
                         four ? "{0u, 0u, 0u, 0u}" : "{0u, 0u}", w * epw});
        }
        return r;
    }

    // How load_vec fills its raw variables: 0 loads, 1 loads and keeps a copy
    // in the register cache slot `cache_slot`, 2 takes them from that slot;
    // 3 loads and keeps a copy in this lane's LDS cache slot, 4 takes them
    // from there (each lane reads back only what it wrote itself)
    int cache_mode = 0;
    std::string cache_slot = "t";

    // emit loading of a vector of input k at element offset `off` into x{k}_{e0..}
    void load_vec(int k, const std::string& off, int e0, const std::string& cond)
    {
        const InputInfo& in = an.inputs[k];
        const int V = pl.vec;
        std::string ks = std::to_string(k);
        std::string p = "(in" + ks + " + " + off + ")";
        auto dst = [&](int j) { return "x" + ks + "_" + std::to_string(e0 + j); };
        std::vector<RawVar> raw = raw_vars(k, e0);
        for (const RawVar& r : raw) {
            const std::string lds = "l" + r.name + "[" + cache_slot + "][lane]";
            if (cache_mode == 4) {
                o << "    " << r.type << " " << r.name << " = " << lds << ";\n";
                continue;
            }
            if (cache_mode == 2) {
                // the empty asm makes the words a new value, so the compiler
                // widens them again instead of keeping an earlier phase's
                // widened copies alive (twice the registers for bf16 and masks)
                o << "    " << r.type << " " << r.name << " = k" << r.name << "[" << cache_slot << "];\n";
                o << "    __asm__ volatile(\"\" : \"+v\"(" << r.name << "));\n";
                continue;
            }
            o << "    " << r.type << " " << r.name << " = " << r.zero << ";\n";
            std::string ld;
            // an input other rows read again (it broadcasts over some axis of
            // the output) is loaded through the caches
            const std::string fn = (in.numel < an.numel && !pl.bnt) ? "psk_ldc" : ld_fn();
            if (V == 1) ld = widen(in.dtype, fn + "(" + p + ")");
            else ld = fn + "((const " + r.type + "*)(" + p + (r.eoff ? " + " + std::to_string(r.eoff) : "") + "))";
            o << "    if (" << cond << ") " << r.name << " = " << ld << ";\n";
            if (cache_mode == 1) o << "    k" << r.name << "[" << cache_slot << "] = " << r.name << ";\n";
            if (cache_mode == 3) o << "    " << lds << " = " << r.name << ";\n";
        }
        if (V == 1) return;
        if (in.dtype == PSK_U8) {
            const int nw = std::max(1, V / 4);
            for (int j = 0; j < V; ++j) {
                std::string w = nw == 1 ? raw[0].name : raw[0].name + "[" + std::to_string(j / 4) + "]";
                o << "    const float " << dst(j) << " = (float)((" << w << " >> " << 8 * (j % 4) << ") & 255u);\n";
            }
            return;
        }
        std::vector<std::string> words;
        for (const RawVar& r : raw)
            for (int q = 0; q < (r.type == "psk_u4v" ? 4 : 2); ++q) words.push_back(r.name + "[" + std::to_string(q) + "]");
        for (int j = 0; j < V; ++j) {
            std::string v;
            if (in.dtype == PSK_F32) v = "__uint_as_float(" + words[j] + ")";
            else v = (j % 2 == 0 ? "psk_lo(" : "psk_hi(") + words[j / 2] + ")";
            o << "    const float " << dst(j) << " = " << v << ";\n";
        }
    }

    // Extra load condition for a vector of `in` at element e0 (columns from
    // c): under a causal mask, the vector's first column is allowed; under a
    // byte mask read by every WHERE, some mask byte under the vector allows
    // (the mask's own vector at e0 is loaded first).
    std::string guard(const InputInfo& in, int e0, const std::string& c) const
    {
        if (!in.mask_guarded) return "";
        if (an.mask_period > 0) return " && " + c + " <= q";
        if (an.where_mask < 0) return "";
        const InputInfo& m = an.inputs[an.where_mask];
        const std::string mk = std::to_string(an.where_mask);
        if (m.kind == InKind::Scalar || m.kind == InKind::RowConst) return " && xr" + mk + " != 0.0f";
        const int V = pl.vec;
        if (V == 1) return " && x" + mk + "_" + std::to_string(e0) + " != 0.0f";
        const std::string w = "w" + mk + "_" + std::to_string(e0);
        const int nw = std::max(1, V / 4);
        if (nw == 1) return " && " + w + " != 0u";
        std::string any = w + "[0]";
        for (int q = 1; q < nw; ++q) any += " | " + w + "[" + std::to_string(q) + "]";
        return " && (" + any + ") != 0u";
    }

    // lane vector k has an allowed position: its first column under a causal
    // mask, a nonzero byte of the group's mask under a WHERE mask
    std::string allowed_vec(int k) const
    {
        if (an.mask_period > 0) return "c" + std::to_string(k) + " <= q";
        InputInfo probe;
        probe.mask_guarded = true;
        std::string g = guard(probe, k * pl.vec, "c" + std::to_string(k));   // " && <cond>"
        return g.empty() ? "true" : g.substr(4);
    }

    // input indices in load order: the unguarded first (the mask among them)
    std::vector<int> load_order() const
    {
        std::vector<int> ks;
        for (int pass = 0; pass < 2; ++pass)
            for (size_t k = 0; k < an.inputs.size(); ++k)
                if (an.inputs[k].mask_guarded == (pass == 1)) ks.push_back((int)k);
        return ks;
    }

    // The pieces input k's vector at element e0 arrives in: (type, name
    // suffix, element offset); V == 1 arrives as one widened float.
    struct Piece {
        std::string type, name;
        int eoff;
    };
    std::vector<Piece> pieces(int k, int e0) const
    {
        const InputInfo& in = an.inputs[k];
        const int V = pl.vec;
        const std::string base = std::to_string(k) + "_" + std::to_string(e0);
        if (V == 1) return {{"float", base, 0}};
        if (in.dtype == PSK_U8) {
            const int nw = std::max(1, V / 4);
            return {{nw == 1 ? "psk_u32" : nw == 2 ? "psk_u2v" : "psk_u4v", base, 0}};
        }
        std::vector<Piece> ps;
        const int nwords = V * esize(in.dtype) / 4, epw = 4 / esize(in.dtype);
        for (int w = 0, piece = 0; w < nwords; w += 4, ++piece)
            ps.push_back({nwords - w >= 4 ? "psk_u4v" : "psk_u2v", base + "_" + std::to_string(piece), w * epw});
        return ps;
    }

    // declare input k's pieces as `pfx`<name> and load them (zero when cond
    // fails); with declare false, load into the pieces declared before
    // (left as they were when cond fails)
    void load_pieces(int k, const std::string& off, int e0, const std::string& cond, const std::string& pfx,
                     bool declare = true)
    {
        const InputInfo& in = an.inputs[k];
        const std::string p = "(in" + std::to_string(k) + " + " + off + ")";
        const std::string fn = (in.numel < an.numel && !pl.bnt) ? "psk_ldc" : ld_fn();   // read again by other rows
        for (const Piece& pc : pieces(k, e0)) {
            if (declare) o << "    " << pc.type << " " << pfx << pc.name << " = {};\n";
            if (pc.type == "float")
                o << "    if (" << cond << ") " << pfx << pc.name << " = " << widen(in.dtype, fn + "(" + p + ")")
                  << ";\n";
            else
                o << "    if (" << cond << ") " << pfx << pc.name << " = " << fn << "((const " << pc.type << "*)("
                  << p << " + " << pc.eoff << "));\n";
        }
    }

    // the f32 values x<k>_<e> of input k's vector at e0 from pieces `pfx`<name>
    void decode_pieces(int k, int e0, const std::string& pfx)
    {
        const InputInfo& in = an.inputs[k];
        const int V = pl.vec;
        const std::vector<Piece> ps = pieces(k, e0);
        auto dst = [&](int j) { return "x" + std::to_string(k) + "_" + std::to_string(e0 + j); };
        if (V == 1) {
            o << "    const float " << dst(0) << " = " << pfx << ps[0].name << ";\n";
            return;
        }
        if (in.dtype == PSK_U8) {
            const int nw = std::max(1, V / 4);
            for (int j = 0; j < V; ++j) {
                std::string w = pfx + ps[0].name + (nw == 1 ? "" : "[" + std::to_string(j / 4) + "]");
                o << "    const float " << dst(j) << " = (float)((" << w << " >> " << 8 * (j % 4) << ") & 255u);\n";
            }
            return;
        }
        std::vector<std::string> words;
        for (const Piece& pc : ps)
            for (int q = 0; q < (pc.type == "psk_u4v" ? 4 : 2); ++q)
                words.push_back(pfx + pc.name + "[" + std::to_string(q) + "]");
        for (int j = 0; j < V; ++j) {
            std::string v = in.dtype == PSK_F32 ? "__uint_as_float(" + words[j] + ")"
                                                : (j % 2 == 0 ? "psk_lo(" : "psk_hi(") + words[j / 2] + ")";
            o << "    const float " << dst(j) << " = " << v << ";\n";
        }
    }

    void store_vec(const std::string& off, int e0, const std::string& cond)
    {
        store_node(an.root, "out", an.out_dtype, off, e0, cond);
    }

    // store element values of node i (elements e0 .. e0+vec-1) to `ptr`
    void store_node(int i, const std::string& ptr, psk_dtype dt, const std::string& off, int e0,
                    const std::string& cond)
    {
        const int V = pl.vec;
        std::string p = "(" + ptr + " + " + off + ")";
        auto src = [&](int j) { return val(i, e0 + j); };
        if (V == 1) {
            o << "    if (" << cond << ") psk_st(" << p << ", "
              << (dt == PSK_BF16 ? "psk_r1(" + src(0) + ")" : src(0)) << ");\n";
            return;
        }
        // 32-bit words of the V elements, written as 16-byte pieces (one
        // 8-byte piece when only two words are left: four bf16 values)
        std::vector<std::string> words;
        if (dt == PSK_F32)
            for (int j = 0; j < V; ++j) words.push_back("__float_as_uint(" + src(j) + ")");
        else
            for (int j = 0; j < V; j += 2) words.push_back("psk_pack2(" + src(j) + ", " + src(j + 1) + ")");
        const int epw = dt == PSK_F32 ? 1 : 2;   // elements per word
        for (size_t w = 0; w < words.size(); w += 4) {
            const size_t cnt = std::min<size_t>(4, words.size() - w);
            const char* vt = cnt == 4 ? "psk_u4v" : "psk_u2v";
            o << "    if (" << cond << ") psk_st((" << vt << "*)(" << p << " + " << w * epw << "), (" << vt << "){";
            for (size_t q = 0; q < cnt; ++q) o << (q ? ", " : "") << words[w + q];
            o << "});\n";
        }
    }

    // Workgroups go to the 8 XCDs round robin; with the XCD layout block b
    // takes virtual block (b mod 8) * per + b / 8, so each XCD streams one
    // contiguous eighth of the output.  The grid is padded to a multiple of
    // 8; padding blocks exit (whole workgroups, before any barrier).
    void block_index()
    {
        if (pl.xcd) {
            o << "    const unsigned vb = (blockIdx.x % 8u) * " << pl.per_xcd << "u + blockIdx.x / 8u;\n";
            o << "    if (vb >= " << pl.blocks << "u) return;\n";
        } else {
            o << "    const unsigned vb = blockIdx.x;\n";
        }
    }

    void signature(const std::string& name)
    {
        o << "extern \"C\" __global__ void __launch_bounds__(" << pl.block << ") ";
        if (pl.wmin > 0)
            o << "__attribute__((amdgpu_waves_per_eu(" << pl.wmin << ", " << std::max(pl.wmin, pl.wpe > 0 ? pl.wpe : 8)
              << "))) ";
        else if (pl.wpe > 0)
            o << "__attribute__((amdgpu_waves_per_eu(1, " << pl.wpe << "))) ";
        o << name << "(";
        // no __restrict__: the output may be the same buffer as an input
        // (in place); every load of an element precedes its store
        for (size_t k = 0; k < an.inputs.size(); ++k)
            o << "const void* in" << k << "_, ";
        o << "void* out_, ";
        for (size_t k = 0; k < an.extras.size(); ++k) o << "void* xo" << k << "_, ";
        o << "long long n_total";
        if (pl.kind == 4)
            o << ", unsigned long long* psk_xslots, unsigned* psk_xstate, unsigned psk_teams, int psk_xmap, "
                 "int psk_limit";
        o << ")\n{\n";
        for (size_t k = 0; k < an.inputs.size(); ++k)
            o << "  const " << ptype(an.inputs[k].dtype) << "* in" << k << " = (const "
              << ptype(an.inputs[k].dtype) << "*)in" << k << "_;\n";
        o << "  " << ptype(an.out_dtype) << "* out = (" << ptype(an.out_dtype) << "*)out_;\n";
        for (size_t k = 0; k < an.extras.size(); ++k)
            o << "  " << ptype(an.extras[k].dtype) << "* xo" << k << " = (" << ptype(an.extras[k].dtype) << "*)xo" << k
              << "_;\n";
    }

    // Row kernel with a causal mask: a lane's vector k whose first column
    // lies past the row's last allowed column is refused entirely.  There,
    // members uniform at refused positions take their per-row refused value,
    // members irrelevant at refused positions are not computed, and the rest
    // are computed as usual.
    bool skip_refused() const
    {
        if (pl.kind != 1 || pl.persist || (an.mask_period <= 0 && an.where_mask < 0)) return false;
        for (size_t i = 0; i < an.nodes.size(); ++i)
            if (an.uniform[i] && an.nodes[i].op != PSK_OP_CAUSAL_MASK) return true;
        return false;
    }

    void members_at_skipping(int p)
    {
        const int n = (int)an.nodes.size();
        std::vector<int> elems;
        for (int i = 0; i < n; ++i) {
            const psk_node& nd = an.nodes[i];
            if (op_is_leaf(nd.op) || op_is_row(nd.op) || an.depth[i] != p) continue;
            if (an.is_row[i]) {
                o << "    const float r" << i << " = " << rt(i, expr(i, 0)) << ";\n";
                row_reciprocal(i);
            } else {
                elems.push_back(i);
            }
        }
        for (int i : elems)
            if (an.uniform[i]) o << "    const float u" << i << " = " << rt(i, refused_expr(i)) << ";\n";
        for (int k = 0; k < pl.nv; ++k) {
            for (int i : elems)
                for (int j = 0; j < pl.vec; ++j) o << "    float v" << i << "_" << k * pl.vec + j << ";\n";
            // a member stored as bf16 is rounded as soon as it is computed:
            // the members after it in the branch read the rounded value
            std::vector<int> es;
            for (int j = 0; j < pl.vec; ++j) es.push_back(k * pl.vec + j);
            o << "    if (" << allowed_vec(k) << ") {\n";
            for (int i : elems) {
                divr_open(i);
                for (int e : es) o << "      v" << i << "_" << e << " = " << expr(i, e) << ";\n";
                divr_close(i, es, "      ");
                round_elems(i, es, "      ");
            }
            o << "    } else {\n";
            for (int i : elems) {
                for (int e : es) {
                    o << "      v" << i << "_" << e << " = ";
                    if (an.uniform[i]) o << "u" << i;
                    else if (an.irrelevant[i]) o << "0.0f";
                    else if (divr_node(i)) o << val(an.nodes[i].a, e) << " / " << val(an.nodes[i].b, e);
                    else o << expr(i, e);
                    o << ";\n";
                }
                if (!an.uniform[i] && !an.irrelevant[i]) round_elems(i, es, "      ");   // u is rounded already
            }
            o << "    }\n";
        }
    }

    // element members of the given depth, and row members of that depth
    // mode 0: element and row members, 1: element members only, 2: row
    // members only; `only`, when given, selects the members emitted
    void members_at(int p, int mode = 0, const std::vector<char>* only = nullptr)
    {
        if (mode == 0 && skip_refused()) { members_at_skipping(p); return; }
        for (size_t i = 0; i < an.nodes.size(); ++i) {
            const psk_node& nd = an.nodes[i];
            if (op_is_leaf(nd.op) || op_is_row(nd.op) || an.depth[i] != p) continue;
            if ((mode == 1 && an.is_row[i]) || (mode == 2 && !an.is_row[i])) continue;
            if (only && !(*only)[i]) continue;
            if (an.is_row[i]) {
                o << "    const float r" << i << " = " << rt((int)i, expr((int)i, 0)) << ";\n";
                row_reciprocal((int)i);
            } else if (divr_node((int)i)) {
                // one vector at a time, each with its own fallback: a vector's
                // numerators are dead once its quotients are checked (all of a
                // lane's numerators live at once would double the registers)
                for (int e = 0; e < NE; ++e) o << "    float v" << i << "_" << e << ";\n";
                for (int e0 = 0; e0 < NE; e0 += pl.vec) {
                    o << "    {\n";
                    divr_open((int)i);
                    std::vector<int> es;
                    for (int e = e0; e < std::min(NE, e0 + pl.vec); ++e) {
                        o << "    v" << i << "_" << e << " = " << expr((int)i, e) << ";\n";
                        es.push_back(e);
                    }
                    divr_close((int)i, es, "    ");
                    round_elems((int)i, es, "    ");
                    o << "    }\n";
                }
            } else {
                for (int e = 0; e < NE; ++e)
                    o << "    const float v" << i << "_" << e << " = " << rt((int)i, expr((int)i, e)) << ";\n";
            }
        }
    }

    // mode 0: every leaf, 1: constants and row-valued inputs, 2: element
    // inputs (those in `only`, when given)
    void leaves(int mode = 0, const std::vector<char>* only = nullptr)
    {
        for (size_t i = 0; i < an.nodes.size(); ++i) {
            const psk_node& nd = an.nodes[i];
            const bool elem = nd.op == PSK_OP_INPUT && !an.is_row[i];
            if ((mode == 1 && elem) || (mode == 2 && !elem)) continue;
            if (only && !(*only)[i]) continue;
            if (nd.op == PSK_OP_CONST) {
                o << "    const float r" << i << " = " << flit(nd.imm) << ";\n";
                row_reciprocal((int)i);
            } else if (nd.op == PSK_OP_INPUT) {
                const InputInfo& in = an.inputs[nd.iparam];
                if (an.is_row[i]) {
                    o << "    const float r" << i << " = xr" << nd.iparam << ";\n";
                    row_reciprocal((int)i);
                } else {
                    (void)in;
                    for (int e = 0; e < NE; ++e)
                        o << "    const float v" << i << "_" << e << " = x" << nd.iparam << "_" << e << ";\n";
                }
            }
        }
    }

    // row-value inputs: one load per row (or one per thread for scalars)
    void row_inputs(const std::string& rv, const std::string& cond)
    {
        for (size_t k = 0; k < an.inputs.size(); ++k) {
            const InputInfo& in = an.inputs[k];
            if (!in.used || !(in.kind == InKind::Scalar || in.kind == InKind::RowConst)) continue;
            std::string off = in.kind == InKind::Scalar ? "0" : row_offset(in, rv);
            std::string p = "(in" + std::to_string(k) + " + " + off + ")";
            o << "    const float xr" << k << " = (" << cond << ") ? " << widen(in.dtype, "*" + p) << " : 0.0f;\n";
        }
    }

    // the column part: the column index times the input's last-axis step
    std::string col_offset(const InputInfo& in, const std::string& cexpr) const
    {
        if (in.stride4[3] == 1) return cexpr;
        return "(" + std::string(I()) + ")(" + cexpr + ") * (" + std::string(I()) + ")" + std::to_string(in.stride4[3]);
    }

    std::string elem_offset(const InputInfo& in, const std::string& rv, const std::string& cexpr)
    {
        switch (in.kind) {
        case InKind::Full: return "(" + rv + ") * (" + std::string(I()) + ")" + std::to_string(an.cols) + " + " + cexpr;
        case InKind::ColVec: return col_offset(in, cexpr);
        default: return "(" + row_offset(in, rv) + ") + " + col_offset(in, cexpr);
        }
    }

    // ------------------------------------------------------------ pointwise
    std::string pointwise(const std::string& name)
    {
        o << "#define PSK_NT " << (pl.nt ? 1 : 0) << "\n#define PSK_SC1 " << (pl.sc1 ? 1 : 0) << "\n" << kPrelude;
        signature(name);
        const int V = pl.vec;
        o << "  {\n";
        block_index();
        o << "    const " << I() << " t = (" << I() << ")vb * " << pl.block << " + (" << I() << ")threadIdx.x;\n";
        o << "    const " << I() << " e0 = t * " << V << ";\n";
        o << "    if (e0 >= (" << I() << ")n_total) return;\n";
        o << "    const " << I() << " row = e0 / (" << I() << ")" << an.cols << ";\n";
        o << "    const " << I() << " c0 = e0 - row * (" << I() << ")" << an.cols << ";\n";
        if (period > 0) o << "    const " << I() << " q = row % (" << I() << ")" << period << ";\n";
        row_inputs("row", "true");
        for (int k : load_order()) {
            const InputInfo& in = an.inputs[k];
            if (!in.used || in.kind == InKind::Scalar || in.kind == InKind::RowConst) continue;
            load_vec(k, elem_offset(in, "row", "c0"), 0, "true" + guard(in, 0, "c0"));
        }
        leaves();
        members_at(0);
        for (size_t k = 0; k < an.extras.size(); ++k) {
            const Analysis::Extra& x = an.extras[k];
            std::string xo = "xo" + std::to_string(k);
            if (x.per_row)
                o << "    if (c0 == 0) " << xo << "[row] = " << scalar_store(x.node, x.dtype) << ";\n";
            else
                store_node(x.node, xo, x.dtype, "e0", 0, "true");
        }
        store_vec("e0", 0, "true");
        o << "  }\n}\n";
        return o.str();
    }

    // a row value of node i as stored to `dt`
    std::string scalar_store(int i, psk_dtype dt) const
    {
        return dt == PSK_BF16 ? "psk_r1(r" + std::to_string(i) + ")" : "r" + std::to_string(i);
    }

    // ----------------------------------------------------------------- tree
    // A workgroup takes block * NE consecutive elements of a chunk of the
    // tree's chunk table; per-element inputs come from the leaf's slots,
    // per-tree inputs from device scalars; the root goes to the output slot.
    // A thread whose NE elements are all present in a leaf whose slots are
    // 16-byte aligned moves them as vectors of up to 16 bytes (NE of 2: 4
    // bytes of bf16, 8 of f32); the last thread of a ragged leaf goes
    // element by element.
    std::string tree(const std::string& name)
    {
        const int TB = pl.block, TS = (int)pl.blocks;
        o << "#define PSK_NT " << (pl.nt ? 1 : 0) << "\n#define PSK_SC1 " << (pl.sc1 ? 1 : 0) << "\n" << kPrelude;
        o << "struct psk_leaf_dev { void* slot[" << PSK_MAX_SLOTS << "]; long long flags; };\n";
        o << "struct psk_chunk_dev { int leaf; int count; long long start; };\n";
        o << "extern \"C\" __global__ void __launch_bounds__(" << TB << ") " << name
          << "(const psk_leaf_dev* __restrict__ leaves, const psk_chunk_dev* __restrict__ chunks, "
             "unsigned n_virtual, unsigned per_xcd";
        // inputs' slots, then the outputs' (root first, then the extra outputs)
        for (size_t k = 0; k <= an.inputs.size() + an.extras.size(); ++k) o << ", int slot" << k;
        for (size_t k = 0; k < an.inputs.size(); ++k) o << ", const void* s" << k;
        o << ")\n{\n";
        if (pl.xcd) o << "  const unsigned vb = (blockIdx.x % 8u) * per_xcd + blockIdx.x / 8u;\n";
        else o << "  const unsigned vb = blockIdx.x;\n";
        o << "  if (vb >= n_virtual) return;\n";
        o << "  const psk_chunk_dev ch = chunks[vb / " << TS << "u];\n";
        o << "  const psk_leaf_dev* L = leaves + ch.leaf;\n";
        o << "  const int i0 = ((int)(vb % " << TS << "u) * " << TB << " + (int)threadIdx.x) * " << NE << ";\n";
        o << "  const int cnt = ch.count - i0;\n";
        o << "  if (cnt <= 0) return;\n";
        o << "  const long long e0 = ch.start + i0;\n";
        o << "  const bool full = (L->flags & 1) != 0 && cnt >= " << NE << ";\n";
        o << "  {\n";
        // per-tree scalars and per-element inputs: every input's vector
        // loads in one branch, issued before any of them is waited for, the
        // element-by-element loads of a ragged thread in the other
        std::vector<size_t> vin;
        for (size_t k = 0; k < an.inputs.size(); ++k) {
            const InputInfo& in = an.inputs[k];
            if (!in.used) continue;
            std::string T = ptype(in.dtype);
            if (in.kind == InKind::Scalar) {
                std::string p = "(const " + T + "*)s" + std::to_string(k);
                o << "    const float xr" << k << " = "
                  << (in.dtype == PSK_BF16 ? "psk_h(*" + p + ")" : "*" + p) << ";\n";
                continue;
            }
            vin.push_back(k);
            o << "    const PSK_G " << T << "* in" << k << " = (const PSK_G " << T << "*)L->slot[slot" << k << "] + e0;\n";
            o << "    float";
            for (int j = 0; j < NE; ++j) o << (j ? ", x" : " x") << k << "_" << j;
            o << ";\n";
        }
        o << "    if (full) {\n";
        for (size_t k : vin) {
            const InputInfo& in = an.inputs[k];
            const int nw = NE * esize(in.dtype) / 4;   // 32-bit words of the thread's elements
            std::string w = "w" + std::to_string(k);
            o << "      unsigned " << w << "[" << nw << "];\n";
            if (nw == 1) {
                o << "      " << w << "[0] = psk_ld((const PSK_G unsigned*)in" << k << ");\n";
            } else if (nw == 2) {
                o << "      const psk_u2v t" << k << " = psk_ld((const PSK_G psk_u2v*)in" << k << ");\n";
                o << "      " << w << "[0] = t" << k << "[0]; " << w << "[1] = t" << k << "[1];\n";
            } else {
                for (int q = 0; q < nw / 4; ++q) {
                    std::string t = "t" + std::to_string(k) + "_" + std::to_string(q);
                    o << "      const psk_u4v " << t << " = psk_ld((const PSK_G psk_u4v*)in" << k << " + " << q << ");\n";
                    for (int j = 0; j < 4; ++j) o << "      " << w << "[" << 4 * q + j << "] = " << t << "[" << j << "];\n";
                }
            }
        }
        for (size_t k : vin) {
            const InputInfo& in = an.inputs[k];
            std::string w = "w" + std::to_string(k);
            for (int j = 0; j < NE; ++j) {
                o << "      x" << k << "_" << j << " = ";
                if (in.dtype == PSK_F32) o << "__uint_as_float(" << w << "[" << j << "]);\n";
                else o << (j % 2 == 0 ? "psk_lo(" : "psk_hi(") << w << "[" << j / 2 << "]);\n";
            }
        }
        o << "    } else {\n";
        for (size_t k : vin) {
            const InputInfo& in = an.inputs[k];
            for (int j = 0; j < NE; ++j)
                o << "      x" << k << "_" << j << " = " << j << " < cnt ? " << (in.dtype == PSK_BF16 ? "psk_h(in" : "(in")
                  << k << "[" << j << "]) : 0.0f;\n";
        }
        o << "    }\n";
        leaves();
        members_at(0);
        for (size_t k = 0; k < an.extras.size(); ++k)
            tree_store(an.extras[k].node, an.extras[k].dtype, (int)(an.inputs.size() + 1 + k), "xo" + std::to_string(k));
        tree_store(an.root, an.out_dtype, (int)an.inputs.size(), "out");
        o << "  }\n}\n";
        return o.str();
    }

    // tree kernel: node i's elements to slot `slot_arg` of the leaf
    void tree_store(int root, psk_dtype dt, int slot_arg, const std::string& name)
    {
        std::string T = ptype(dt);
        o << "    {\n";
        o << "    PSK_G " << T << "* " << name << " = (PSK_G " << T << "*)L->slot[slot" << slot_arg << "] + e0;\n";
        const std::string out = name;
        o << "    if (full) {\n";
        if (dt == PSK_F32 && NE == 2) {
            o << "      psk_st((PSK_G psk_u2v*)" << out << ", (psk_u2v){__float_as_uint(" << val(root, 0)
              << "), __float_as_uint(" << val(root, 1) << ")});\n";
        } else if (dt == PSK_F32) {
            for (int q = 0; q < NE / 4; ++q) {
                o << "      psk_st((PSK_G psk_u4v*)" << out << " + " << q << ", (psk_u4v){";
                for (int j = 0; j < 4; ++j) o << (j ? ", " : "") << "__float_as_uint(" << val(root, 4 * q + j) << ")";
                o << "});\n";
            }
        } else if (NE == 2) {
            o << "      psk_st((PSK_G unsigned*)" << out << ", psk_pack2(" << val(root, 0) << ", " << val(root, 1) << "));\n";
        } else if (NE == 4) {
            o << "      psk_st((PSK_G psk_u2v*)" << out << ", (psk_u2v){psk_pack2(" << val(root, 0) << ", " << val(root, 1)
              << "), psk_pack2(" << val(root, 2) << ", " << val(root, 3) << ")});\n";
        } else {
            for (int q = 0; q < NE / 8; ++q) {
                o << "      psk_st((PSK_G psk_u4v*)" << out << " + " << q << ", (psk_u4v){";
                for (int j = 0; j < 4; ++j)
                    o << (j ? ", " : "") << "psk_pack2(" << val(root, 8 * q + 2 * j) << ", "
                      << val(root, 8 * q + 2 * j + 1) << ")";
                o << "});\n";
            }
        }
        o << "    } else {\n";
        for (int j = 0; j < NE; ++j)
            o << "      if (" << j << " < cnt) " << out << "[" << j << "] = "
              << (dt == PSK_BF16 ? "psk_r1(" + val(root, j) + ")" : val(root, j)) << ";\n";
        o << "    }\n";
        o << "    }\n";
    }

    // ------------------------------------------------------------------ row
    // reductions whose operand has depth p
    std::vector<int> reductions_of(int p) const
    {
        std::vector<int> reds;
        for (size_t i = 0; i < an.nodes.size(); ++i)
            if (op_is_row(an.nodes[i].op) && an.depth[i] == p + 1) reds.push_back((int)i);
        return reds;
    }

    void reduce_declare(const std::vector<int>& reds)
    {
        for (int i : reds)
            o << "    float p" << i << " = " << (an.nodes[i].op == PSK_OP_ROW_MAX ? "(-__builtin_inff())" : "0.0f")
              << ";\n";
    }

    // this lane's elements folded into its partials, in element order
    void reduce_accumulate(const std::vector<int>& reds, const char* indent = "    ")
    {
        for (int i : reds) {
            const psk_node& nd = an.nodes[i];
            bool mx = nd.op == PSK_OP_ROW_MAX;
            if (an.online_max[i] >= 0) continue;      // taken with its maximum
            if (an.online_sum[i] >= 0) {
                online_accumulate(i, an.online_sum[i], indent);
                continue;
            }
            for (int e = 0; e < NE; ++e) {
                std::string v = val(nd.a, e);
                std::string acc = mx ? std::string(pl.kind == 3 ? "psk_rmax_s(p" : "psk_rmax(p") + std::to_string(i) +
                                           ", " + v + ")"
                                     : "(p" + std::to_string(i) + " + " + v + ")";
                if (ragged)
                    o << indent << "if (" << col(e) << " < " << an.cols << ") p" << i << " = " << acc << ";\n";
                else
                    o << indent << "p" << i << " = " << acc << ";\n";
            }
        }
    }

    // the exponential an online sum uses: its exp node's form (every
    // argument here is <= 0 as well)
    std::string online_exp(int sm) const
    {
        const int e = an.nodes[sm].a;
        return cheap_exp(e) ? "psk_exp_np_b" : split_exp(e) ? "psk_exp_np" : "expf";
    }

    // Online normalizer: this lane's elements of y (the maximum's operand)
    // update the running maximum p<mx> once for the group of elements and
    // the sum p<sm> of exp(y - running maximum), rescaled by
    // exp(old - new) when the maximum grows.  While the maximum is still
    // -inf every y so far is -inf, and the exponentials are taken against 0
    // (giving exp(-inf) = 0 rather than exp(NaN)).  Where the pass is the
    // lane's only one (kept_sum), the exponentials stay in registers as
    // oe<sm>_<e> for the exp member, which rescales them once the row's
    // maximum is known instead of taking each again.
    void online_accumulate(int mx, int sm, const char* indent)
    {
        const int y = an.nodes[mx].a;
        const std::string P = "p" + std::to_string(mx), S = "p" + std::to_string(sm);
        const std::string ex = online_exp(sm);
        const bool keep = kept_sum[an.nodes[sm].a] == sm;
        const std::string in = keep ? std::string(indent) : std::string(indent) + "  ";
        const std::string tm = "tm" + std::to_string(sm), mref = "mref" + std::to_string(sm);
        if (!keep) o << indent << "{\n";
        o << in << "float " << tm << " = (-__builtin_inff());\n";
        for (int e = 0; e < NE; ++e) {
            std::string acc = tm + " = " + (pl.kind == 3 ? "psk_rmax_s" : "psk_rmax") + "(" + tm + ", " + val(y, e) +
                              ");";
            if (ragged) o << in << "if (" << col(e) << " < " << an.cols << ") " << acc << "\n";
            else o << in << acc << "\n";
        }
        // the running maximum becomes the maximum with this group's; the sum
        // is rescaled when it changes (a NaN maximum makes the sum NaN)
        o << in << "{ const float pn = psk_rmax(" << P << ", " << tm << "); if (!(pn == " << P << ")) " << S << " = "
          << S << " * " << ex << "(" << P << " - pn); " << P << " = pn; }\n";
        o << in << "const float " << mref << " = " << P << " == (-__builtin_inff()) ? 0.0f : " << P << ";\n";
        for (int e = 0; e < NE; ++e) {
            std::string term = ex + "(" + val(y, e) + " - " + mref + ")";
            if (keep) {
                const std::string oe = "oe" + std::to_string(sm) + "_" + std::to_string(e);
                o << in << "const float " << oe << " = " << term << ";\n";
                term = oe;
            }
            std::string acc = S + " = (" + S + " + " + term + ");";
            if (ragged) o << in << "if (" << col(e) << " < " << an.cols << ") " << acc << "\n";
            else o << in << acc << "\n";
        }
        if (!keep) o << indent << "}\n";
    }

    // lanes of a wave (DPP), then waves (LDS), then the row values
    void reduce_finish(const std::vector<int>& reds, int p)
    {
        const int W = pl.lanes / 64;
        auto lane_reduce = [&](int i) {
            bool mx = an.nodes[i].op == PSK_OP_ROW_MAX;
            if (pl.lanes == 16)
                o << "    p" << i << " = " << (mx ? "psk_max16" : "psk_sum16") << "(p" << i << ");\n";
            else if (pl.lanes == 32)
                o << "    p" << i << " = " << (mx ? "psk_max32" : "psk_sum32") << "(p" << i << ", (lane & 16) != 0);\n";
            else
                o << "    p" << i << " = " << (mx ? "psk_max64" : "psk_sum64") << "(p" << i << ");\n";
        };
        for (int i : reds) {
            if (an.online_max[i] >= 0) continue;
            if (an.online_sum[i] >= 0) o << "    const float q" << i << " = p" << i << ";\n";
            lane_reduce(i);
        }
        // an online sum: each lane's part rescaled to the maximum of its
        // wave (or row part) before the lanes add up
        for (int i : reds) {
            const int m = an.online_max[i];
            if (m < 0) continue;
            o << "    p" << i << " = (q" << m << " == p" << m << ") ? p" << i << " : p" << i << " * " << online_exp(i)
              << "(q" << m << " - p" << m << ");\n";
            lane_reduce(i);
        }
        if (W > 1) {
            const int NR = (int)reds.size();
            const int size = pl.rows_per_block * W * NR;
            // a persistent workgroup alternates two halves, so a wave that is
            // one row ahead never overwrites values another wave still reads
            const std::string base = pl.persist ? "par * " + std::to_string(size) + " + " : "";
            std::string arr = "psk_red" + std::to_string(p);
            o << "    __shared__ float " << arr << "[" << (pl.persist ? 2 : 1) * size << "];\n";
            o << "    if ((lane & 63) == 0) {\n";
            for (int r = 0; r < NR; ++r)
                o << "      " << arr << "[" << base << "(slot * " << W << " + (lane >> 6)) * " << NR << " + " << r
                  << "] = p" << reds[r] << ";\n";
            o << "    }\n    __syncthreads();\n";
            auto slot_of = [&](int w, int r) {
                return arr + "[" + base + "(slot * " + std::to_string(W) + " + " + std::to_string(w) + ") * " +
                       std::to_string(NR) + " + " + std::to_string(r) + "]";
            };
            for (int r = 0; r < NR; ++r) {
                int i = reds[r];
                bool mx = an.nodes[i].op == PSK_OP_ROW_MAX;
                const int m = an.online_max[i];
                if (m >= 0) {
                    // the waves' sums, each rescaled from its wave's maximum to
                    // the row's (already combined: the maximum precedes)
                    const int rm = (int)(std::find(reds.begin(), reds.end(), m) - reds.begin());
                    for (int w = 0; w < W; ++w) {
                        std::string mw = slot_of(w, rm), sw = slot_of(w, r);
                        std::string t = "((" + mw + " == p" + std::to_string(m) + ") ? " + sw + " : " + sw + " * " +
                                        online_exp(i) + "(" + mw + " - p" + std::to_string(m) + "))";
                        if (w == 0) o << "    p" << i << " = " << t << ";\n";
                        else o << "    p" << i << " = p" << i << " + " << t << ";\n";
                    }
                    continue;
                }
                o << "    p" << i << " = " << slot_of(0, r) << ";\n";
                for (int w = 1; w < W; ++w) {
                    std::string el = slot_of(w, r);
                    if (mx) o << "    p" << i << " = psk_rmax(p" << i << ", " << el << ");\n";
                    else o << "    p" << i << " = p" << i << " + " << el << ";\n";
                }
            }
        }
        if (pl.kind == 4) exchange(reds, p);
        for (int i : reds) {
            if (an.nodes[i].op == PSK_OP_ROW_MEAN)
                o << "    const float r" << i << " = " << rt(i, "p" + std::to_string(i) + " / " + flit((float)an.cols))
                  << ";\n";
            else if (an.online_max[i] >= 0)
                // an online sum over a row of -inf is NaN, as the exact sum
                // of exp(-inf - (-inf)) is; its lanes summed zeros
                o << "    const float r" << i << " = (r" << an.online_max[i]
                  << " == (-__builtin_inff())) ? __builtin_nanf(\"\") : p" << i << ";\n";
            else
                o << "    const float r" << i << " = " << rt(i, "p" + std::to_string(i)) << ";\n";
            row_reciprocal(i);
        }
        // kept exponentials: the factor exp(q - M) from the lane's maximum q
        // to the row's M (neither is rounded: such pairs are not formed).
        // exp(y - q) * 1 is exp(y - M) itself where q = M; a lane of -inf
        // holds zeros, which stay zero (NaN when M is -inf or NaN, as
        // exp(y - M) is then)
        for (int i : reds) {
            const int m = an.online_max[i];
            if (m < 0 || kept_sum[an.nodes[i].a] != i) continue;
            const std::string q = "q" + std::to_string(m), M = "r" + std::to_string(m);
            const std::string ninf = "(-__builtin_inff())", nan = "__builtin_nanf(\"\")";
            o << "    const float osc" << i << " = (" << q << " == " << M << ") ? ((" << q << " == " << ninf << ") ? "
              << nan << " : 1.0f) : (" << q << " == " << ninf << ") ? ((" << M << " == " << M << ") ? 0.0f : " << nan
              << ") : " << online_exp(i) << "(" << q << " - " << M << ");\n";
        }
    }

    // Split rows: this workgroup's partials of phase p go to its member slot
    // of the team's slot block, tagged; lanes r*K + m of the first wave take
    // member m's partial of reduction r (waiting, bounded, for its tag) and
    // every one of them combines the K partials of each reduction in member
    // order, so every member of the team holds the same row values.
    void exchange(const std::vector<int>& reds, int p)
    {
        const int K = pl.split, NR = (int)reds.size();
        int off = 0;
        for (int q = 0; q < p; ++q) off += (int)reductions_of(q).size();
        const std::string arr = "psk_xv" + std::to_string(p);
        o << "    {\n";
        o << "      const unsigned psk_tag = psk_gen * psk_stride + psk_it * " << std::max(1, an.phases) << "u + "
          << p + 1 << "u;\n";
        o << "      unsigned long long* psk_s = psk_xslots + ((unsigned long long)psk_t * " << pl.exch << "u + " << off
          << "u) * " << K << "u;\n";
        o << "      if (lane == 0) {\n";
        for (int r = 0; r < NR; ++r)
            o << "        psk_put(psk_s + " << r * K << "u + psk_j, psk_tag, p" << reds[r] << ");\n";
        o << "      }\n";
        o << "      __shared__ float " << arr << "[" << NR << "];\n";
        o << "      if (lane < " << NR * K << ") {\n";
        o << "        const float v = psk_take(psk_s + lane, psk_tag, psk_limit, psk_xstate + 2);\n";
        // maxima and plain sums first; then an online sum, whose members'
        // parts are each rescaled from their member's maximum to the row's
        // (combined just before) and added in member order
        for (int pass = 0; pass < 2; ++pass)
            for (int r = 0; r < NR; ++r) {
                const int i = reds[r], om = an.online_max[i];
                if ((om >= 0) != (pass == 1)) continue;
                const bool mx = an.nodes[i].op == PSK_OP_ROW_MAX;
                auto lane_of = [&](int rr, int m) { return "PSK_RL(v, " + std::to_string(rr * K + m) + ")"; };
                if (om >= 0) {
                    const int rm = (int)(std::find(reds.begin(), reds.end(), om) - reds.begin());
                    const std::string M = "a" + std::to_string(rm);
                    for (int m = 0; m < K; ++m) {
                        const std::string mm = lane_of(rm, m), sm = lane_of(r, m);
                        const std::string t = "((" + mm + " == " + M + ") ? " + sm + " : " + sm + " * " +
                                              online_exp(i) + "(" + mm + " - " + M + "))";
                        if (m == 0) o << "        float a" << r << " = " << t << ";\n";
                        else o << "        a" << r << " = a" << r << " + " << t << ";\n";
                    }
                } else {
                    o << "        float a" << r << " = " << lane_of(r, 0) << ";\n";
                    for (int m = 1; m < K; ++m) {
                        if (mx) o << "        a" << r << " = psk_rmax(a" << r << ", " << lane_of(r, m) << ");\n";
                        else o << "        a" << r << " = a" << r << " + " << lane_of(r, m) << ";\n";
                    }
                }
                o << "        if (lane == 0) " << arr << "[" << r << "] = a" << r << ";\n";
            }
        o << "      }\n";
        o << "      __syncthreads();\n";
        for (int r = 0; r < NR; ++r) o << "      p" << reds[r] << " = " << arr << "[" << r << "];\n";
        o << "    }\n";
    }

    void reductions_at(int p)
    {
        std::vector<int> reds = reductions_of(p);
        if (reds.empty()) return;
        reduce_declare(reds);
        reduce_accumulate(reds);
        reduce_finish(reds, p);
    }

    // element nodes the targets read, through element values only (row
    // values are known by the phase that reads them)
    std::vector<char> needed_for(const std::vector<int>& targets) const
    {
        std::vector<char> need(an.nodes.size(), 0);
        std::vector<int> st;
        for (int t : targets)
            if (!an.is_row[t]) st.push_back(t);
        while (!st.empty()) {
            int i = st.back();
            st.pop_back();
            if (need[i]) continue;
            need[i] = 1;
            const psk_node& nd = an.nodes[i];
            const int32_t opnd[3] = {nd.a, nd.b, nd.c};
            for (int k = 0; k < op_arity(nd.op); ++k)
                if (!an.is_row[opnd[k]]) st.push_back(opnd[k]);
        }
        return need;
    }

    void store_row_extras(int depth)
    {
        for (size_t k = 0; k < an.extras.size(); ++k) {
            const Analysis::Extra& x = an.extras[k];
            if (x.per_row && an.depth[x.node] == depth)
                o << "    if (rok && lane == 0) xo" << k << "[row] = " << scalar_store(x.node, x.dtype) << ";\n";
        }
    }

    // Wide rows: one workgroup per row; every phase walks the row in tiles
    // of lanes x nv vectors, re-reading the inputs it needs and recomputing
    // the element members it needs; partial reductions stay in registers
    // until the phase ends.  The last phase stores the root and the element
    // extra outputs.
    std::string row_tiled(const std::string& name)
    {
        o << "#define PSK_NT " << (pl.nt ? 1 : 0) << "\n#define PSK_SC1 " << (pl.sc1 ? 1 : 0) << "\n" << kPrelude;
        signature(name);
        const int L = pl.lanes, V = pl.vec, TN = pl.nv;
        const int64_t tile = (int64_t)L * TN * V;
        o << "  {\n";
        o << "    const int slot = 0;\n";
        o << "    const int lane = (int)threadIdx.x;\n";
        block_index();
        o << "    const " << I() << " row = (" << I() << ")vb;\n";
        o << "    const bool rok = row < (" << I() << ")n_total;\n";
        if (period > 0) o << "    const int q = (int)(row % (" << I() << ")" << period << ");\n";
        row_inputs("row", "rok");
        leaves(1);
        members_at(0, 2);
        store_row_extras(0);
        // what each phase computes and which inputs it loads
        std::vector<std::vector<char>> need(an.phases + 1);
        std::vector<std::vector<char>> loads(an.phases + 1, std::vector<char>(an.inputs.size(), 0));
        for (int p = 0; p <= an.phases; ++p) {
            std::vector<int> targets;
            if (p < an.phases) {
                for (int r : reductions_of(p))
                    if (an.online_max[r] < 0) targets.push_back(an.nodes[r].a);
            } else {
                targets.push_back(an.root);
                for (const auto& x : an.extras)
                    if (!x.per_row) targets.push_back(x.node);
            }
            need[p] = needed_for(targets);
            for (size_t i = 0; i < an.nodes.size(); ++i)
                if (need[p][i] && an.nodes[i].op == PSK_OP_INPUT) loads[p][an.nodes[i].iparam] = 1;
        }
        // Register cache: a per-row input that two or more phases load keeps
        // the raw words of the leading pl.rcache tiles from the phase that
        // first loads them; later phases take them from there instead of
        // memory.  The arithmetic and its order do not change.
        const int RC = pl.rcache, LC = pl.lcache;
        std::vector<int> first(an.inputs.size(), -1);
        for (size_t k = 0; k < an.inputs.size(); ++k) {
            const InputInfo& in = an.inputs[k];
            if (RC + LC <= 0 || !in.used || !(in.kind == InKind::General || in.kind == InKind::Full)) continue;
            int n = 0;
            for (int p = 0; p <= an.phases; ++p)
                if (loads[p][k]) {
                    if (first[k] < 0) first[k] = p;
                    ++n;
                }
            if (n < 2) first[k] = -1;
            if (first[k] < 0) continue;
            for (int v = 0; v < TN; ++v)
                for (const RawVar& r : raw_vars((int)k, v * V)) {
                    if (RC > 0) o << "    " << r.type << " k" << r.name << "[" << RC << "];\n";
                    if (LC > 0) o << "    __shared__ " << r.type << " l" << r.name << "[" << LC << "][" << L << "];\n";
                }
        }
        // cached: 0 memory, 1 registers, 2 LDS
        auto tile_body = [&](int p, int cached) {
            o << "    const int cb = t * " << tile << ";\n";
            for (int k = 0; k < TN; ++k)
                o << "    const int c" << k << " = cb + (" << k * L << " + lane) * " << V << ";\n";
            for (int k : load_order()) {
                const InputInfo& in = an.inputs[k];
                if (!in.used || in.kind == InKind::Scalar || in.kind == InKind::RowConst) continue;
                if (!loads[p][k]) continue;
                cache_mode = 0;
                if (cached && first[k] >= 0) cache_mode = (first[k] == p ? 1 : 2) + (cached == 2 ? 2 : 0);
                cache_slot = cached == 2 ? "t - " + std::to_string(RC) : "t";
                // what a cache keeps is not read from memory again
                const bool keep = cached_loads;
                if (cache_mode == 1 || cache_mode == 3) cached_loads = false;
                for (int v = 0; v < TN; ++v) {
                    std::string c = "c" + std::to_string(v);
                    std::string cond = "rok";
                    if (ragged) cond += " && " + c + " < " + std::to_string(an.cols);
                    load_vec(k, elem_offset(in, "row", c), v * V, cond + guard(in, v * V, c));
                }
                cache_mode = 0;
                cached_loads = keep;
            }
            leaves(2, &need[p]);
            for (int d = 0; d <= p; ++d) members_at(d, 1, &need[p]);
            if (p < an.phases) {
                reduce_accumulate(reductions_of(p));
            } else {
                for (int v = 0; v < TN; ++v) {
                    std::string c = "c" + std::to_string(v);
                    std::string cond = "rok";
                    if (ragged) cond += " && " + c + " < " + std::to_string(an.cols);
                    std::string off = "row * (" + std::string(I()) + ")" + std::to_string(an.cols) + " + " + c;
                    for (size_t k = 0; k < an.extras.size(); ++k)
                        if (!an.extras[k].per_row)
                            store_node(an.extras[k].node, "xo" + std::to_string(k), an.extras[k].dtype, off, v * V, cond);
                    store_vec(off, v * V, cond);
                }
            }
        };
        for (int p = 0; p <= an.phases; ++p) {
            std::vector<int> reds = p < an.phases ? reductions_of(p) : std::vector<int>();
            // data read again by a later phase stays in the caches: plain
            // loads before the last phase, nontemporal ones in it
            cached_loads = p < an.phases && pl.tcache;
            reduce_declare(reds);
            // Odd phases walk the tiles from last to first, so they begin on
            // the tiles the phase before read last.  The order depends on
            // the phase alone (the caches hold leading tiles), not on what
            // is cached.
            const bool back = pl.alt && p % 2 == 1;
            auto walk = [&](int lo, int hi, int cached, const char* unroll) {
                if (lo >= hi) return;
                o << "    #pragma " << unroll << "\n";
                if (back)
                    o << "    for (int t = " << hi - 1 << "; t >= " << lo << "; --t) {\n";
                else
                    o << "    for (int t = " << lo << "; t < " << hi << "; ++t) {\n";
                tile_body(p, cached);
                o << "    }\n";
            };
            const std::string mu = "unroll " + std::to_string(pl.munroll);
            const std::string lu = "unroll " + std::to_string(pl.lunroll);
            if (back) {
                walk(RC + LC, pl.tiles, 0, mu.c_str());
                walk(RC, RC + LC, 2, lu.c_str());
                walk(0, RC, 1, "unroll");
            } else {
                walk(0, RC, 1, "unroll");
                walk(RC, RC + LC, 2, lu.c_str());
                walk(RC + LC, pl.tiles, 0, mu.c_str());
            }
            if (p < an.phases) {
                reduce_finish(reds, p);
                members_at(p + 1, 2);
                store_row_extras(p + 1);
            }
        }
        o << "  }\n}\n";
        return o.str();
    }

    // the phases of one row and its stores (rows of the register kernel)
    void row_body()
    {
        const int L = pl.lanes, V = pl.vec;
        leaves();
        for (int p = 0; p <= an.phases; ++p) {
            members_at(p);
            for (size_t k = 0; k < an.extras.size(); ++k) {
                const Analysis::Extra& x = an.extras[k];
                if (an.depth[x.node] != p) continue;
                std::string xo = "xo" + std::to_string(k);
                if (x.per_row) {
                    o << "    if (rok && lane == 0) " << xo << "[row] = " << scalar_store(x.node, x.dtype) << ";\n";
                    continue;
                }
                for (int v = 0; v < pl.nv; ++v) {
                    std::string c = "c" + std::to_string(v);
                    std::string cond = "rok";
                    if ((int64_t)(v + 1) * L * V > an.cols) cond += " && " + c + " < " + std::to_string(an.cols);
                    store_node(x.node, xo, x.dtype, "row * (" + std::string(I()) + ")" + std::to_string(an.cols) + " + " + c,
                               v * V, cond);
                }
            }
            if (p < an.phases) reductions_at(p);
        }
        for (int v = 0; v < pl.nv; ++v) {
            std::string c = "c" + std::to_string(v);
            std::string cond = "rok";
            if ((int64_t)(v + 1) * L * V > an.cols) cond += " && " + c + " < " + std::to_string(an.cols);
            store_vec("row * (" + std::string(I()) + ")" + std::to_string(an.cols) + " + " + c, v * V, cond);
        }
    }

    // Persistent rows: gridDim.x workgroups walk the rows (row, row + G,
    // ...); the element inputs of the next rows are loaded before the
    // current row is computed, so their loads are in flight during the
    // arithmetic.  Column vectors (gamma) are loaded and widened once per
    // workgroup.
    std::string row_persistent(const std::string& name)
    {
        o << "#define PSK_NT " << (pl.nt ? 1 : 0) << "\n#define PSK_SC1 " << (pl.sc1 ? 1 : 0) << "\n" << kPrelude;
        signature(name);
        const int L = pl.lanes, V = pl.vec;
        auto streamed = [&](const InputInfo& in) {
            return in.used && in.kind != InKind::Scalar && in.kind != InKind::RowConst && in.kind != InKind::ColVec;
        };
        auto vcond = [&](int v, const std::string& ok, const std::string& qv, const InputInfo& in) {
            std::string c = "c" + std::to_string(v);
            std::string cond = ok;
            if ((int64_t)(v + 1) * L * V > an.cols) cond += " && " + c + " < " + std::to_string(an.cols);
            if (in.mask_guarded && an.mask_period > 0) cond += " && " + c + " <= " + qv;   // byte masks: no skip here
            return cond;
        };
        o << "  {\n";
        o << "    const int slot = 0;\n";
        o << "    const int lane = (int)threadIdx.x;\n";
        for (int k = 0; k < pl.nv; ++k)
            o << "    const int c" << k << " = (" << k * L << " + lane) * " << V << ";\n";
        // column vectors: once
        for (size_t k = 0; k < an.inputs.size(); ++k) {
            const InputInfo& in = an.inputs[k];
            if (!in.used || in.kind != InKind::ColVec) continue;
            for (int v = 0; v < pl.nv; ++v) {
                std::string c = "c" + std::to_string(v);
                std::string cond = "true";
                if ((int64_t)(v + 1) * L * V > an.cols) cond = c + " < " + std::to_string(an.cols);
                load_vec((int)k, elem_offset(in, "0", c), v * V, cond);
            }
        }
        o << "    " << I() << " row = (" << I() << ")blockIdx.x;\n";
        o << "    const " << I() << " G = (" << I() << ")gridDim.x;\n";
        o << "    const " << I() << " rend = (" << I() << ")n_total;\n";
        o << "    int par = 0;\n";
        // Prefetch depth D: buffers b0 .. b(D-1) hold the element inputs of
        // rows row, row + G, ..., row + (D - 1) G when an iteration starts.
        // The loop is unrolled D times, one row a buffer: a row widens its
        // buffer's words, loads row + D G into the same buffer and then
        // computes, so D rows are in flight during the arithmetic and no
        // buffer is ever copied (a copy of registers still being loaded
        // would wait for the load).
        const int D = std::max(1, std::min(4, pl.pf));
        auto bufname = [&](int d) { return "b" + std::to_string(d) + "_"; };
        for (int d = 0; d < D; ++d) {
            const std::string pr = "pr" + std::to_string(d);
            o << "    const " << I() << " " << pr << " = row + (" << I() << ")" << d << " * G;\n";
            if (period > 0)
                o << "    const int q" << pr << " = (int)(" << pr << " % (" << I() << ")" << period << ");\n";
            for (size_t k = 0; k < an.inputs.size(); ++k) {
                const InputInfo& in = an.inputs[k];
                if (!streamed(in)) continue;
                for (int v = 0; v < pl.nv; ++v)
                    load_pieces((int)k, elem_offset(in, pr, "c" + std::to_string(v)), v * V,
                                vcond(v, pr + " < rend", "q" + pr, in), bufname(d));
            }
        }
        o << "    for (; row < rend; row += (" << I() << ")" << D << " * G) {\n";
        for (int d = 0; d < D; ++d) {
            o << "    if (row + (" << I() << ")" << d << " * G < rend) {\n";
            o << "    const " << I() << " nrow = row + (" << I() << ")" << d + D << " * G;\n";
            o << "    const bool nok = nrow < rend;\n";
            if (period > 0) o << "    const int qn = (int)(nrow % (" << I() << ")" << period << ");\n";
            o << "    {\n";
            o << "    const " << I() << " row2 = row + (" << I() << ")" << d << " * G;\n";
            o << "    {\n";
            o << "    const " << I() << " row = row2;\n";
            o << "    const bool rok = true;\n";
            if (period > 0) o << "    const int q = (int)(row % (" << I() << ")" << period << ");\n";
            row_inputs("row", "rok");
            for (size_t k = 0; k < an.inputs.size(); ++k) {
                const InputInfo& in = an.inputs[k];
                if (!streamed(in)) continue;
                for (int v = 0; v < pl.nv; ++v) decode_pieces((int)k, v * V, bufname(d));
            }
            for (size_t k = 0; k < an.inputs.size(); ++k) {
                const InputInfo& in = an.inputs[k];
                if (!streamed(in)) continue;
                for (int v = 0; v < pl.nv; ++v)
                    load_pieces((int)k, elem_offset(in, "nrow", "c" + std::to_string(v)), v * V,
                                vcond(v, "nok", "qn", in), bufname(d), false);
            }
            row_body();
            o << "    }\n";
            o << "    }\n";
            o << "    par ^= 1;\n";
            o << "    }\n";
        }
        o << "    }\n";
        o << "  }\n}\n";
        return o.str();
    }

    // Split rows: the grid is the device's resident capacity (every
    // workgroup runs at once); K consecutive members form a team (on one
    // XCD when the grid is a multiple of 8 K: workgroups reach the XCDs
    // round robin), and team t takes rows t, t + teams, ...  Member j holds
    // columns [j S, (j + 1) S) of the row in registers (S = lanes * nv *
    // vec), reduces them as the register row kernel does, and exchanges
    // each phase's partials with the other members (exchange above).  The
    // tags of a launch come from a generation counter in device memory that
    // the last workgroup to finish advances, so they never repeat from one
    // launch (or graph replay) to the next.
    std::string row_split(const std::string& name)
    {
        o << "#define PSK_NT " << (pl.nt ? 1 : 0) << "\n#define PSK_SC1 " << (pl.sc1 ? 1 : 0) << "\n" << kPrelude << kSplitPrelude;
        signature(name);
        const int L = pl.lanes, V = pl.vec, K = pl.split;
        const int64_t S = (int64_t)L * pl.nv * V;
        o << "  {\n";
        o << "    const int slot = 0;\n";
        o << "    const int lane = (int)threadIdx.x;\n";
        o << "    const unsigned psk_b = blockIdx.x;\n";
        o << "    unsigned psk_t, psk_j;\n";
        o << "    if (psk_xmap) { const unsigned idx = psk_b / 8u; psk_t = (idx / " << K << "u) * 8u + psk_b % 8u; psk_j = "
             "idx % " << K << "u; }\n";
        o << "    else { psk_t = psk_b / " << K << "u; psk_j = psk_b % " << K << "u; }\n";
        o << "    const unsigned psk_gen = __hip_atomic_load(psk_xstate, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);\n";
        o << "    const unsigned psk_stride = (unsigned)(" << std::max(1, an.phases)
          << "LL * ((n_total + psk_teams - 1) / psk_teams) + 1);\n";
        o << "    unsigned psk_it = 0;\n";
        o << "    for (" << I() << " row = (" << I() << ")psk_t; row < (" << I() << ")n_total; row += ("
          << I() << ")psk_teams, ++psk_it) {\n";
        o << "    const bool rok = true;\n";
        if (period > 0) o << "    const int q = (int)(row % (" << I() << ")" << period << ");\n";
        for (int k = 0; k < pl.nv; ++k)
            o << "    const int c" << k << " = (int)psk_j * " << S << " + (" << k * L << " + lane) * " << V << ";\n";
        row_inputs("row", "rok");
        auto cond_of = [&](int v) {
            std::string c = "c" + std::to_string(v);
            return ragged ? "rok && " + c + " < " + std::to_string(an.cols) : std::string("rok");
        };
        for (int k : load_order()) {
            const InputInfo& in = an.inputs[k];
            if (!in.used || in.kind == InKind::Scalar || in.kind == InKind::RowConst) continue;
            for (int v = 0; v < pl.nv; ++v)
                load_vec(k, elem_offset(in, "row", "c" + std::to_string(v)), v * V,
                         cond_of(v) + guard(in, v * V, "c" + std::to_string(v)));
        }
        leaves();
        const std::string roff = "row * (" + std::string(I()) + ")" + std::to_string(an.cols) + " + ";
        for (int p = 0; p <= an.phases; ++p) {
            members_at(p);
            for (size_t k = 0; k < an.extras.size(); ++k) {
                const Analysis::Extra& x = an.extras[k];
                if (an.depth[x.node] != p) continue;
                std::string xo = "xo" + std::to_string(k);
                if (x.per_row) {
                    o << "    if (lane == 0 && psk_j == 0u) " << xo << "[row] = " << scalar_store(x.node, x.dtype)
                      << ";\n";
                    continue;
                }
                for (int v = 0; v < pl.nv; ++v)
                    store_node(x.node, xo, x.dtype, roff + "c" + std::to_string(v), v * V, cond_of(v));
            }
            if (p < an.phases) reductions_at(p);
        }
        for (int v = 0; v < pl.nv; ++v) store_vec(roff + "c" + std::to_string(v), v * V, cond_of(v));
        o << "    __syncthreads();\n";
        o << "    }\n";
        // the last workgroup to finish advances the generation
        o << "    if (threadIdx.x == 0) {\n";
        o << "      const unsigned d = __hip_atomic_fetch_add(psk_xstate + 1, 1u, __ATOMIC_RELAXED, "
             "__HIP_MEMORY_SCOPE_AGENT);\n";
        o << "      if (d == gridDim.x - 1u) {\n";
        o << "        __hip_atomic_store(psk_xstate + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);\n";
        o << "        __hip_atomic_fetch_add(psk_xstate, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);\n";
        o << "      }\n";
        o << "    }\n";
        o << "  }\n}\n";
        return o.str();
    }

    std::string row(const std::string& name)
    {
        if (pl.persist) return row_persistent(name);
        o << "#define PSK_NT " << (pl.nt ? 1 : 0) << "\n#define PSK_SC1 " << (pl.sc1 ? 1 : 0) << "\n" << kPrelude;
        signature(name);
        const int L = pl.lanes, V = pl.vec;
        o << "  {\n";
        o << "    const int slot = (int)threadIdx.x / " << L << ";\n";
        o << "    const int lane = (int)threadIdx.x % " << L << ";\n";
        block_index();
        o << "    const " << I() << " row = (" << I() << ")vb * " << pl.rows_per_block << " + slot;\n";
        o << "    const bool rok = row < (" << I() << ")n_total;\n";
        if (period > 0) o << "    const int q = (int)(row % (" << I() << ")" << period << ");\n";
        for (int k = 0; k < pl.nv; ++k)
            o << "    const int c" << k << " = (" << k * L << " + lane) * " << V << ";\n";
        row_inputs("row", "rok");
        for (int k : load_order()) {
            const InputInfo& in = an.inputs[k];
            if (!in.used || in.kind == InKind::Scalar || in.kind == InKind::RowConst) continue;
            for (int v = 0; v < pl.nv; ++v) {
                std::string c = "c" + std::to_string(v);
                std::string cond = "rok";
                if ((int64_t)(v + 1) * L * V > an.cols) cond += " && " + c + " < " + std::to_string(an.cols);
                load_vec(k, elem_offset(in, "row", c), v * V, cond + guard(in, v * V, c));
            }
        }
        leaves();
        for (int p = 0; p <= an.phases; ++p) {
            members_at(p);
            // extra outputs computed by now: stored at once
            for (size_t k = 0; k < an.extras.size(); ++k) {
                const Analysis::Extra& x = an.extras[k];
                if (an.depth[x.node] != p) continue;
                std::string xo = "xo" + std::to_string(k);
                if (x.per_row) {
                    o << "    if (rok && lane == 0) " << xo << "[row] = " << scalar_store(x.node, x.dtype) << ";\n";
                    continue;
                }
                for (int v = 0; v < pl.nv; ++v) {
                    std::string c = "c" + std::to_string(v);
                    std::string cond = "rok";
                    if ((int64_t)(v + 1) * L * V > an.cols) cond += " && " + c + " < " + std::to_string(an.cols);
                    store_node(x.node, xo, x.dtype, "row * (" + std::string(I()) + ")" + std::to_string(an.cols) + " + " + c,
                               v * V, cond);
                }
            }
            if (p < an.phases) reductions_at(p);
        }
        for (int v = 0; v < pl.nv; ++v) {
            std::string c = "c" + std::to_string(v);
            std::string cond = "rok";
            if ((int64_t)(v + 1) * L * V > an.cols) cond += " && " + c + " < " + std::to_string(an.cols);
            store_vec("row * (" + std::string(I()) + ")" + std::to_string(an.cols) + " + " + c, v * V, cond);
        }
        o << "  }\n}\n";
        return o.str();
    }
};

}  // namespace

std::string emit_source(const Analysis& an, const KernelPlan& plan, const std::string& kernel_name)
{
    Emitter em(an, plan);
    std::ostringstream hdr;
    hdr << "// psk_fused emitted kernel\n// group:\n";
    std::istringstream ct(canonical_text(an));
    std::string line;
    while (std::getline(ct, line)) hdr << "//   " << line << "\n";
    hdr << "// plan: " << plan.key() << "\n";
    if (plan.kind == 2) return hdr.str() + em.tree(kernel_name);
    if (plan.kind == 3) return hdr.str() + em.row_tiled(kernel_name);
    if (plan.kind == 4) return hdr.str() + em.row_split(kernel_name);
    return hdr.str() + (plan.kind == 1 ? em.row(kernel_name) : em.pointwise(kernel_name));
}

}  // namespace psk
