/*
 * CPU oracle for fusion groups -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, sequential evaluation of what a fusion group computes.  Only
 * the tests, the smoke check and the benchmark's CPU-baseline leg may load
 * this library; the product path never does.  It shares no source with the
 * GPU library.
 *
 * Numerics (presk manual, "Native execution", section "The realization";
 * "PSK-Realize", section "What a group is"):
 *   - every member of a group is computed in f32, the arithmetic type of both
 *     f32 and bf16 storage; only the root is rounded to its storage type;
 *   - bf16 is storage only: a load is a 16-bit shift (exact), a store is one
 *     round to nearest even;
 *   - each operation is one IEEE-754 binary32 operation in program order:
 *     this file must be compiled with -ffp-contract=off and without any
 *     fast-math flag, so nothing is fused or reassociated (fusion keeps the
 *     order of operations: PSK-Realize, section "What it buys, measured");
 *   - exp, log, tanh, erf are the C library's f32 functions; their last bits
 *     are the library's, not a specification (presk manual, "Native
 *     execution", section "Conformance").
 *
 * Parity pins (tests/test_oracle_*.py) tie every function here to something
 * other than itself: closed forms, invariants, PyTorch CPU library routines,
 * float64 brute force.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ bf16 */
/* bf16 holds the top 16 bits of an IEEE binary32; widening is exact. */
float orc_bf16_widen(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round to nearest, ties to even; a NaN stays a NaN of the same sign. */
uint16_t orc_bf16_round(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

void orc_bf16_widen_array(int64_t n, const uint16_t *in, float *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_bf16_widen(in[i]);
}

void orc_bf16_round_array(int64_t n, const float *in, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_bf16_round(in[i]);
}

/* storage types; ORC_U8 is a mask (one byte per element, read as its value) */
enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_U8 = 2 };

static float load_elem(const void *base, int dtype, int64_t i)
{
    if (dtype == ORC_BF16)
        return orc_bf16_widen(((const uint16_t *)base)[i]);
    if (dtype == ORC_U8)
        return (float)((const uint8_t *)base)[i];
    return ((const float *)base)[i];
}

static void store_elem(void *base, int dtype, int64_t i, float x)
{
    if (dtype == ORC_BF16)
        ((uint16_t *)base)[i] = orc_bf16_round(x);
    else
        ((float *)base)[i] = x;
}

/* The value a store to `dtype` leaves behind, read back in f32. */
static float through_storage(int dtype, float x)
{
    return dtype == ORC_BF16 ? orc_bf16_widen(orc_bf16_round(x)) : x;
}

/* ------------------------------------------------------------ primitives */
/* gelu is the exact x * Phi(x) through the error function (presk manual,
 * "Native execution", section "The realization").  The pages fix the real
 * function, not its f32 composition.  Chosen: Phi(x) = erfc(-x/sqrt 2) / 2,
 * i.e. (0.5*x) * erfc(-(x * f32(1/sqrt 2))).  The complementary form avoids
 * the cancellation of 1 + erf(x/sqrt 2) for x << 0, where a one-ulp
 * difference between two erf implementations would move the result by many
 * bf16 ulps. */
static float orc_gelu(float x)
{
    const float inv_sqrt2 = 0.70710678118654752440f;
    return (0.5f * x) * erfcf(-(x * inv_sqrt2));
}

/* max and min give their second operand at a tie (presk language reference,
 * section "Typing", builtins). */
static float orc_max(float x, float y) { return (x > y) ? x : y; }
static float orc_min(float x, float y) { return (x < y) ? x : y; }

/* One step of a row maximum folded left to right: the running maximum m
 * against the next element y.  The pages give elementwise max's tie rule
 * (the second operand) but nothing a reduction could keep independent of
 * the order its elements are combined in; the row maximum is IEEE 754-2019
 * maximum folded over the row: NaN if any element is NaN, otherwise the
 * largest element, +0 counting above -0. */
static float orc_row_max_step(float m, float y)
{
    if (m != m)
        return m;
    if (y != y)
        return y;
    if (m == y)                 /* equal: the same bits, or zeros of both signs (+0 wins) */
        return signbit(m) ? y : m;
    return (m > y) ? m : y;
}

/* -------------------------------------------------- generic group evaluator */
/* Op codes of this oracle (its own numbering). */
enum {
    O_INPUT = 0, O_CONST,
    O_ADD, O_SUB, O_MUL, O_DIV, O_MAX, O_MIN,
    O_NEG, O_ABS, O_EXP, O_LOG, O_SQRT, O_TANH, O_ERF, O_GELU, O_SQRTABS,
    O_POW2, O_POWN, O_SELECT, O_CAUSAL_MASK,
    O_ROW_MAX, O_ROW_SUM, O_ROW_MEAN,
    O_WHERE,
    O_NUM_OPS
};

typedef struct {
    int32_t op, a, b, c;
    float imm;
    int32_t iparam;
} orc_node;

/* Offset of output element (row r, column col) in an input of rank in_rank
 * aligned to the output from the last axis; a size-1 axis of the input is
 * broadcast (stride 0). */
static int64_t bcast_offset(int out_rank, const int64_t *out_shape, int64_t r, int64_t col,
                            int in_rank, const int64_t *in_shape)
{
    int64_t idx[8];
    idx[out_rank - 1] = col;
    int64_t rem = r;
    for (int d = out_rank - 2; d >= 0; --d) {
        idx[d] = rem % out_shape[d];
        rem /= out_shape[d];
    }
    int64_t off = 0, stride = 1;
    for (int j = in_rank - 1; j >= 0; --j) {
        int od = j + (out_rank - in_rank);
        if (in_shape[j] != 1)
            off += idx[od] * stride;
        stride *= in_shape[j];
    }
    return off;
}

/*
 * Evaluate rows [row_begin, row_end) of a group whose output is viewed as
 * [R, C] (C = last axis, R = product of the others).  Each node is evaluated
 * over the whole row, op by op, into its own f32 array; a row reduction fills
 * its array with the reduced value (keepdim, broadcast along the row).  The
 * root is rounded to out_dtype and stored at its global position in `out`.
 *
 * Reductions run sequentially over the row in increasing column order:
 *   row_max:  m = v[0]; m = max(m, v[c])   (from the first position)
 *   row_sum:  s = v[0]; s = s + v[c]
 *   row_mean: row_sum, then s / C
 * A causal mask replaces a refused position by -inf: column c of row r is
 * allowed where c <= r mod T (presk language reference, section "Typing", builtins:
 * causal_mask is true where seq2 <= seq), which gives the bits of the
 * softmax over the allowed positions (presk manual, "Native execution").
 *
 * Extra stored values (orc_eval_group_multi): node extra_root[k] is stored
 * to extra_out[k] as well, rounded to extra_dtype[k]: at [r, c] for an
 * element value, at [r] when extra_per_row[k] (a value that is one per row).
 * A stored value is what its readers read: a bf16 one is rounded before any
 * later node uses it, as in the partitioned program where the stored value
 * ends one group and the next group loads it (PSK-Realize, "What a group
 * is": the root is the only value that reaches memory, rounded once).
 *
 * Returns 0, or -1 on a malformed node list.
 */
int orc_eval_group_multi(int n_nodes, const orc_node *nodes, int root,
                         int n_inputs, const void *const *inputs, const int32_t *in_dtype,
                         const int32_t *in_rank, const int64_t *in_shape /* n_inputs x 8 */,
                         int out_rank, const int64_t *out_shape, int out_dtype, void *out,
                         int n_extra, const int32_t *extra_root, const int32_t *extra_dtype,
                         const int32_t *extra_per_row, void *const *extra_out,
                         int64_t row_begin, int64_t row_end)
{
    if (out_rank < 1 || out_rank > 8 || root < 0 || root >= n_nodes || n_extra < 0)
        return -1;
    for (int k = 0; k < n_extra; ++k)
        if (extra_root[k] < 0 || extra_root[k] >= n_nodes)
            return -1;
    int64_t C = out_shape[out_rank - 1];
    if (C <= 0)
        return 0;
    float *val = (float *)malloc(sizeof(float) * (size_t)n_nodes * (size_t)C);
    if (!val)
        return -1;
    int rc = 0;
    for (int64_t r = row_begin; r < row_end && rc == 0; ++r) {
        for (int i = 0; i < n_nodes && rc == 0; ++i) {
            const orc_node *nd = &nodes[i];
            float *v = val + (size_t)i * C;
            const float *A = nd->a >= 0 ? val + (size_t)nd->a * C : NULL;
            const float *B = nd->b >= 0 ? val + (size_t)nd->b * C : NULL;
            const float *Cc = nd->c >= 0 ? val + (size_t)nd->c * C : NULL;
            if ((nd->a >= i) || (nd->b >= i) || (nd->c >= i)) {
                rc = -1;
                break;
            }
            switch (nd->op) {
            case O_INPUT: {
                int k = nd->iparam;
                if (k < 0 || k >= n_inputs) { rc = -1; break; }
                for (int64_t c = 0; c < C; ++c) {
                    int64_t off = bcast_offset(out_rank, out_shape, r, c, in_rank[k], in_shape + 8 * k);
                    v[c] = load_elem(inputs[k], in_dtype[k], off);
                }
                break;
            }
            case O_CONST: for (int64_t c = 0; c < C; ++c) v[c] = nd->imm; break;
            case O_ADD: for (int64_t c = 0; c < C; ++c) v[c] = A[c] + B[c]; break;
            case O_SUB: for (int64_t c = 0; c < C; ++c) v[c] = A[c] - B[c]; break;
            case O_MUL: for (int64_t c = 0; c < C; ++c) v[c] = A[c] * B[c]; break;
            case O_DIV: for (int64_t c = 0; c < C; ++c) v[c] = A[c] / B[c]; break;
            case O_MAX: for (int64_t c = 0; c < C; ++c) v[c] = orc_max(A[c], B[c]); break;
            case O_MIN: for (int64_t c = 0; c < C; ++c) v[c] = orc_min(A[c], B[c]); break;
            case O_NEG: for (int64_t c = 0; c < C; ++c) v[c] = -A[c]; break;
            case O_ABS: for (int64_t c = 0; c < C; ++c) v[c] = fabsf(A[c]); break;
            case O_EXP: for (int64_t c = 0; c < C; ++c) v[c] = expf(A[c]); break;
            case O_LOG: for (int64_t c = 0; c < C; ++c) v[c] = logf(A[c]); break;
            case O_SQRT: for (int64_t c = 0; c < C; ++c) v[c] = sqrtf(A[c]); break;
            case O_TANH: for (int64_t c = 0; c < C; ++c) v[c] = tanhf(A[c]); break;
            case O_ERF: for (int64_t c = 0; c < C; ++c) v[c] = erff(A[c]); break;
            case O_GELU: for (int64_t c = 0; c < C; ++c) v[c] = orc_gelu(A[c]); break;
            case O_SQRTABS: for (int64_t c = 0; c < C; ++c) v[c] = sqrtf(fabsf(A[c])); break;
            case O_POW2: for (int64_t c = 0; c < C; ++c) v[c] = A[c] * A[c]; break;
            case O_POWN:
                /* x^n as n-1 products of x, left to right; x^0 = 1 */
                for (int64_t c = 0; c < C; ++c) {
                    float p = 1.0f;
                    if (nd->iparam >= 1) {
                        p = A[c];
                        for (int k = 1; k < nd->iparam; ++k)
                            p = p * A[c];
                    }
                    v[c] = p;
                }
                break;
            case O_SELECT:
                /* bit-moving select: the branch not picked is never read */
                for (int64_t c = 0; c < C; ++c) v[c] = (A[c] != 0.0f) ? B[c] : Cc[c];
                break;
            case O_WHERE:
                /* a mask selects: b where it allows, the fill value where it refuses
                 * (presk language reference, "Typing": softmax(..., where = m)) */
                for (int64_t c = 0; c < C; ++c) v[c] = (A[c] != 0.0f) ? B[c] : nd->imm;
                break;
            case O_CAUSAL_MASK: {
                int64_t T = nd->iparam;
                if (T <= 0) { rc = -1; break; }
                int64_t q = r % T;
                for (int64_t c = 0; c < C; ++c) v[c] = (c <= q) ? A[c] : -INFINITY;
                break;
            }
            case O_ROW_MAX: {
                float m = A[0];
                for (int64_t c = 1; c < C; ++c) m = orc_row_max_step(m, A[c]);
                for (int64_t c = 0; c < C; ++c) v[c] = m;
                break;
            }
            case O_ROW_SUM:
            case O_ROW_MEAN: {
                float s = A[0];
                for (int64_t c = 1; c < C; ++c) s = s + A[c];
                if (nd->op == O_ROW_MEAN)
                    s = s / (float)C;
                for (int64_t c = 0; c < C; ++c) v[c] = s;
                break;
            }
            default:
                rc = -1;
            }
            /* a value stored as bf16 is read back rounded */
            for (int k = 0; k < n_extra && rc == 0; ++k)
                if (extra_root[k] == i && extra_dtype[k] == ORC_BF16)
                    for (int64_t c = 0; c < C; ++c)
                        v[c] = orc_bf16_widen(orc_bf16_round(v[c]));
        }
        if (rc == 0) {
            const float *res = val + (size_t)root * C;
            for (int64_t c = 0; c < C; ++c)
                store_elem(out, out_dtype, r * C + c, res[c]);
            for (int k = 0; k < n_extra; ++k) {
                const float *x = val + (size_t)extra_root[k] * C;
                if (extra_per_row[k])
                    store_elem(extra_out[k], extra_dtype[k], r, x[0]);
                else
                    for (int64_t c = 0; c < C; ++c)
                        store_elem(extra_out[k], extra_dtype[k], r * C + c, x[c]);
            }
        }
    }
    free(val);
    return rc;
}

int orc_eval_group(int n_nodes, const orc_node *nodes, int root,
                   int n_inputs, const void *const *inputs, const int32_t *in_dtype,
                   const int32_t *in_rank, const int64_t *in_shape /* n_inputs x 8 */,
                   int out_rank, const int64_t *out_shape, int out_dtype, void *out,
                   int64_t row_begin, int64_t row_end)
{
    return orc_eval_group_multi(n_nodes, nodes, root, n_inputs, inputs, in_dtype, in_rank, in_shape, out_rank,
                                out_shape, out_dtype, out, 0, NULL, NULL, NULL, NULL, row_begin, row_end);
}

/* ---------------------------------------------------------------- AdamW */
/*
 * One AdamW step over one leaf (presk language reference, section "Configuration blocks", the optimizer):
 *   m' = b1*m + (1-b1)*g
 *   v' = b2*v + (1-b2)*g^2
 *   mh = m' / (1 - b1^t),  vh = v' / (1 - b2^t)
 *   theta' = theta - lr * (mh / (sqrt(vh) + eps) + wd*theta)
 * Hyperparameter arithmetic (1-b, b^t) is done in f64 and each scalar is
 * rounded once to f32 where it enters the f32 chain.  theta, g load from
 * their storage; m', v' are stored (rounded to their storage) and theta'
 * reads the stored values; theta' is rounded to theta's storage.
 * Outputs may alias the inputs (in-place update).
 */
void orc_adamw_scalars(double lr, double beta1, double beta2, double eps, double wd, int64_t t,
                       float *s /* 9: b1 b2 c1 c2 bc1 bc2 lr eps wd */)
{
    s[0] = (float)beta1;
    s[1] = (float)beta2;
    s[2] = (float)(1.0 - beta1);
    s[3] = (float)(1.0 - beta2);
    s[4] = (float)(1.0 - pow(beta1, (double)t));
    s[5] = (float)(1.0 - pow(beta2, (double)t));
    s[6] = (float)lr;
    s[7] = (float)eps;
    s[8] = (float)wd;
}

void orc_adamw(int64_t n, int theta_dt, const void *theta, int grad_dt, const void *grad,
               int mv_dt, const void *m, const void *v,
               double lr, double beta1, double beta2, double eps, double wd, int64_t t,
               void *theta_out, void *m_out, void *v_out)
{
    float s[9];
    orc_adamw_scalars(lr, beta1, beta2, eps, wd, t, s);
    const float b1 = s[0], b2 = s[1], c1 = s[2], c2 = s[3], bc1 = s[4], bc2 = s[5];
    const float lr_f = s[6], eps_f = s[7], wd_f = s[8];
    for (int64_t i = 0; i < n; ++i) {
        float th = load_elem(theta, theta_dt, i);
        float g = load_elem(grad, grad_dt, i);
        float mm = load_elem(m, mv_dt, i);
        float vv = load_elem(v, mv_dt, i);
        float m2 = b1 * mm + c1 * g;
        float v2 = b2 * vv + c2 * (g * g);
        m2 = through_storage(mv_dt, m2);
        v2 = through_storage(mv_dt, v2);
        float mh = m2 / bc1;
        float vh = v2 / bc2;
        float u = mh / (sqrtf(vh) + eps_f) + wd_f * th;
        float th2 = th - lr_f * u;
        store_elem(theta_out, theta_dt, i, th2);
        store_elem(m_out, mv_dt, i, m2);
        store_elem(v_out, mv_dt, i, v2);
    }
}

/*
 * Learning-rate schedule lr(t, total) (presk language reference, section
 * "Configuration blocks", the optimizer): constant: lr; linear(warmup w):
 * lr*t/w for t <= w, then lr*(total - t)/(total - w); cosine(warmup w):
 * lr*t/w for t <= w, then lr * 1/2 * (1 + cos(pi (t - w)/(total - w))).
 * Scalar arithmetic, in f64.  kind: 0 constant, 1 linear, 2 cosine.
 */
double orc_lr_schedule(int kind, double lr, int64_t t, int64_t total, int64_t warmup)
{
    if (kind == 0)
        return lr;
    if (t <= warmup)
        return lr * (double)t / (double)warmup;
    if (kind == 1)
        return lr * (double)(total - t) / (double)(total - warmup);
    const double pi = 3.14159265358979323846;
    return lr * 0.5 * (1.0 + cos(pi * (double)(t - warmup) / (double)(total - warmup)));
}

/* Sum of squares of a gradient leaf, added to a running (sum, compensation)
 * pair (the squared norm of a tree is the sum over its leaves).  Squares of
 * f32 values are exact in f64; the sum is compensated (Neumaier's variant of
 * Kahan summation), so the result is the exact sum to about one f64
 * rounding, whatever the length: the norm is a scalar definition, not a
 * bracketing of the tree's elements. */
void orc_sumsq(int64_t n, int dtype, const void *g, double *sum, double *comp)
{
    double s = *sum, c = *comp;
    for (int64_t i = 0; i < n; ++i) {
        double x = (double)load_elem(g, dtype, i);
        double y = x * x;
        double t = s + y;
        if (fabs(s) >= fabs(y))
            c += (s - t) + y;
        else
            c += (y - t) + s;
        s = t;
    }
    *sum = s;
    *comp = c;
}

/* Global-norm clipping factor min(1, c / (sqrt(sumsq) + 1e-6)) in f64,
 * rounded once to f32 (as clip_grad_norm_ scales the gradient). */
float orc_clip_factor(double sumsq, double c)
{
    double f = c / (sqrt(sumsq) + 1e-6);
    return (float)(f < 1.0 ? f : 1.0);
}

/* One AdamW step with the gradient first scaled by an f32 factor:
 * g_c = g * gscale (one f32 multiply), then the step of orc_adamw with lr
 * taken as given (the schedule's value). */
void orc_adamw_scaled(int64_t n, int theta_dt, const void *theta, int grad_dt, const void *grad,
                      int mv_dt, const void *m, const void *v,
                      double lr, double beta1, double beta2, double eps, double wd, int64_t t, float gscale,
                      void *theta_out, void *m_out, void *v_out)
{
    float s[9];
    orc_adamw_scalars(lr, beta1, beta2, eps, wd, t, s);
    const float b1 = s[0], b2 = s[1], c1 = s[2], c2 = s[3], bc1 = s[4], bc2 = s[5];
    const float lr_f = s[6], eps_f = s[7], wd_f = s[8];
    for (int64_t i = 0; i < n; ++i) {
        float th = load_elem(theta, theta_dt, i);
        float g = load_elem(grad, grad_dt, i) * gscale;
        float mm = load_elem(m, mv_dt, i);
        float vv = load_elem(v, mv_dt, i);
        float m2 = b1 * mm + c1 * g;
        float v2 = b2 * vv + c2 * (g * g);
        m2 = through_storage(mv_dt, m2);
        v2 = through_storage(mv_dt, v2);
        float mh = m2 / bc1;
        float vh = v2 / bc2;
        float u = mh / (sqrtf(vh) + eps_f) + wd_f * th;
        float th2 = th - lr_f * u;
        store_elem(theta_out, theta_dt, i, th2);
        store_elem(m_out, mv_dt, i, m2);
        store_elem(v_out, mv_dt, i, v2);
    }
}

/* ------------------------------------------------------ causal softmax */
/*
 * Masked softmax over each row of x [R, C], mask causal with period T:
 * position c of row r is allowed where c <= r mod T.  Following the masked
 * softmax of the presk manual ("Native execution", section "The
 * realization"): the maximum starts from the first allowed position, the sum
 * runs over the allowed positions in increasing order, a refused position
 * gives +0, a row with no allowed position gives zeros.  Scores are first
 * multiplied by `scale`.
 */
void orc_softmax_causal(int64_t R, int64_t C, int64_t T, float scale, const float *x, float *out,
                        int64_t row_begin, int64_t row_end)
{
    (void)R; /* rows are addressed by [row_begin, row_end) */
    for (int64_t r = row_begin; r < row_end; ++r) {
        const float *xr = x + r * C;
        float *o = out + r * C;
        int64_t last = r % T;                 /* last allowed column */
        if (last > C - 1)
            last = C - 1;
        int64_t first = -1;
        float m = 0.0f;
        for (int64_t c = 0; c <= last; ++c) {
            float y = xr[c] * scale;
            if (first < 0) { m = y; first = c; }
            else m = orc_row_max_step(m, y);
        }
        if (first < 0) {
            for (int64_t c = 0; c < C; ++c) o[c] = 0.0f;
            continue;
        }
        float s = 0.0f;
        int started = 0;
        for (int64_t c = 0; c <= last; ++c) {
            float e = expf(xr[c] * scale - m);
            if (!started) { s = e; started = 1; }
            else s = s + e;
        }
        for (int64_t c = 0; c < C; ++c)
            o[c] = (c <= last) ? expf(xr[c] * scale - m) / s : 0.0f;
    }
}

/* -------------------------------------------- add + RMSNorm + gamma + GELU */
/*
 * Per row of bf16 x, res [R, C] with bf16 gamma [C]:
 *   h = x + res;  ms = (sum h^2) / C;  y = h / sqrt(ms + eps) * gamma;
 *   out = bf16(gelu(y))
 * RMSNorm as sum of squares -> sqrt -> divide (poot, "Fusion and Planning",
 * section "Reduction-rooted regions"); gamma is widened inside the group
 * (same page, table of stages: widening-cast folding).  The sum of squares
 * runs sequentially in increasing column order.
 */
void orc_rmsnorm_gelu(int64_t R, int64_t C, const uint16_t *x, const uint16_t *res,
                      const uint16_t *gamma, float eps, uint16_t *out,
                      int64_t row_begin, int64_t row_end)
{
    (void)R; /* rows are addressed by [row_begin, row_end) */
    float *h = (float *)malloc(sizeof(float) * (size_t)C);
    if (!h)
        return;
    for (int64_t r = row_begin; r < row_end; ++r) {
        for (int64_t c = 0; c < C; ++c)
            h[c] = orc_bf16_widen(x[r * C + c]) + orc_bf16_widen(res[r * C + c]);
        float ss = h[0] * h[0];
        for (int64_t c = 1; c < C; ++c)
            ss = ss + h[c] * h[c];
        float ms = ss / (float)C;
        float den = sqrtf(ms + eps);
        for (int64_t c = 0; c < C; ++c) {
            float y = (h[c] / den) * orc_bf16_widen(gamma[c]);
            out[r * C + c] = orc_bf16_round(orc_gelu(y));
        }
    }
    free(h);
}

/* ------------------------------------------------------------ partition */
/*
 * Fusion-group partition of a let-list (PSK-Realize, section "What a group
 * is").  A group is a set of lets where every member is elementwise, every
 * member has one result type, and every member but the root is read only by
 * members; past 64 members a group stops growing; pow n with n > 2 never
 * joins a group.
 *
 * The pages state conditions, not a procedure.  This oracle takes them as a
 * greedy scan from the last let to the first: an elementwise let joins the
 * group of its readers when it is not a body output, it has readers, all of
 * them are elementwise members of one group G, its type equals G's, and G has
 * fewer than `cap` members; otherwise it roots a new group.  Leaves (inputs,
 * constants) belong to no group (-1).  A boundary let (reduction,
 * contraction, cast, pow n>2) is a group of its own that nothing joins.
 * Groups are numbered in increasing order of their root's position.
 *
 * With `rows` set, reductions fuse as the row kernels run them (poot,
 * "Fusion and Planning", reduction-rooted regions): a last-axis row
 * reduction (op_class 3) is a member candidate like an elementwise let, and
 * a candidate whose shape is the group root's with a last axis of 1 (a
 * value that is one per row: shape_id[i] equals rowshape_id of the root)
 * joins as well as one of the root's type; a reduction joins only so,
 * and only when it reduces a value of the root's shape.
 *
 * op_class: 0 leaf, 1 elementwise, 2 boundary, 3 row reduction.
 * args: n x 3 operand indices (-1 unused).
 * type_id: shape and storage type; shape_id: shape alone; rowshape_id: the
 * shape with its last axis set to 1 (-1 when the last axis is already 1).
 */
int orc_partition(int n, const int32_t *op_class, const int32_t *args, const int32_t *type_id,
                  const int32_t *shape_id, const int32_t *rowshape_id, const uint8_t *is_output, int cap, int rows,
                  int32_t *group_of, int32_t *is_root)
{
    int32_t *nread = (int32_t *)calloc((size_t)n + 1, sizeof(int32_t));
    int32_t *gsize = (int32_t *)calloc((size_t)n + 1, sizeof(int32_t));
    int32_t *gtype = (int32_t *)calloc((size_t)n + 1, sizeof(int32_t));
    int32_t *groot = (int32_t *)calloc((size_t)n + 1, sizeof(int32_t));
    int32_t *renum = (int32_t *)calloc((size_t)n + 1, sizeof(int32_t));
    if (!nread || !gsize || !gtype || !groot || !renum) {
        free(nread); free(gsize); free(gtype); free(groot); free(renum);
        return -1;
    }
    for (int i = 0; i < n; ++i)
        for (int k = 0; k < 3; ++k) {
            int a = args[3 * i + k];
            if (a >= i) { free(nread); free(gsize); free(gtype); free(groot); free(renum); return -1; }
            if (a >= 0)
                nread[a]++;
        }
    int ngroups = 0;
    for (int i = n - 1; i >= 0; --i) {
        group_of[i] = -1;
        is_root[i] = 0;
        if (op_class[i] == 0)
            continue;
        int join = -1;
        int cand = op_class[i] == 1 || (rows && op_class[i] == 3);
        if (cand && !is_output[i] && nread[i] > 0) {
            int G = -2, ok = 1;
            for (int j = i + 1; j < n && ok; ++j)
                for (int k = 0; k < 3; ++k)
                    if (args[3 * j + k] == i) {
                        int member = op_class[j] == 1 || (rows && op_class[j] == 3);
                        if (!member) { ok = 0; break; }
                        if (G == -2) G = group_of[j];
                        else if (group_of[j] != G) { ok = 0; break; }
                    }
            /* a row value joins when its shape is the root's with a last
             * axis of 1; a reduction only when it reduces a value of the
             * root's shape; a group whose root is a reduction takes no
             * member (the reduction reads an element value and is itself
             * one value per row) */
            if (ok && G >= 0 && op_class[groot[G]] == 3)
                ok = 0;
            int typed = ok && G >= 0 &&
                        ((op_class[i] == 1 && gtype[G] == type_id[i]) ||
                         (rows && rowshape_id[groot[G]] >= 0 && shape_id[i] == rowshape_id[groot[G]] &&
                          (op_class[i] == 1 || shape_id[args[3 * i]] == shape_id[groot[G]])));
            if (typed && gsize[G] < cap)
                join = G;
        }
        if (join >= 0) {
            group_of[i] = join;
            gsize[join]++;
        } else {
            group_of[i] = ngroups;
            gsize[ngroups] = 1;
            gtype[ngroups] = type_id[i];
            groot[ngroups] = i;
            is_root[i] = 1;
            ngroups++;
        }
    }
    /* renumber: group with the earliest root first; roots were created in
     * decreasing position order, so the order is reversed */
    for (int g = 0; g < ngroups; ++g)
        renum[g] = ngroups - 1 - g;
    for (int i = 0; i < n; ++i)
        if (group_of[i] >= 0)
            group_of[i] = renum[group_of[i]];
    free(nread); free(gsize); free(gtype); free(groot); free(renum);
    return ngroups;
}
