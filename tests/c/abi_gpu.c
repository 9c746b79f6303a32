/* The C ABI on the GPU from plain C99 (no C++, no Python, no torch): device
 * buffers come from the HIP runtime's C API, the group and the tree from
 * psk_fused, and the expected values from the C oracle (test
 * infrastructure, linked into this test only).
 *
 *   - softmax (scale, row max, subtract, exp, row sum, divide) on a
 *     stream: causal over [300, 1000] f32 (register row kernel) and plain
 *     over [6, 40000] f32 (rows split over workgroups, then the bounded
 *     waits checked) and [3, 40000] (the tiled kernel, forced through the
 *     PSK_LAYOUT variable), within 1e-7 + 2e-6 |ref| of the oracle;
 *   - one AdamW step over a 3-leaf f32 tree (1, 1000 and 4097 elements, in
 *     place): bit for bit against the oracle.
 *
 * Inputs come from a xorshift generator of this file.  Prints "ok" and
 * exits 0 on success; prints the failing check and exits 1 otherwise. */
#define _POSIX_C_SOURCE 200112L   /* setenv */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "psk_fused.h"

/* the C oracle (oracle/oracle.c) */
void orc_softmax_causal(int64_t R, int64_t C, int64_t T, float scale, const float *x, float *out,
                        int64_t row_begin, int64_t row_end);
typedef struct {
    int32_t op, a, b, c;
    float imm;
    int32_t iparam;
} orc_node;
enum { O_INPUT = 0, O_CONST, O_ADD, O_SUB, O_MUL, O_DIV, O_EXP = 10, O_ROW_MAX = 21, O_ROW_SUM = 22 };
int orc_eval_group(int n_nodes, const orc_node *nodes, int root,
                   int n_inputs, const void *const *inputs, const int32_t *in_dtype,
                   const int32_t *in_rank, const int64_t *in_shape,
                   int out_rank, const int64_t *out_shape, int out_dtype, void *out,
                   int64_t row_begin, int64_t row_end);
void orc_adamw(int64_t n, int theta_dt, const void *theta, int grad_dt, const void *grad,
               int mv_dt, const void *m, const void *v,
               double lr, double beta1, double beta2, double eps, double wd, int64_t t,
               void *theta_out, void *m_out, void *v_out);

#define CHECK(c) do { if (!(c)) { printf("check failed: %s (line %d): %s\n", #c, __LINE__, psk_last_error()); \
                                  return 1; } } while (0)
#define HIP(c) do { hipError_t e_ = (c); if (e_ != hipSuccess) { \
                        printf("%s (line %d): %s\n", #c, __LINE__, hipGetErrorString(e_)); return 1; } } while (0)

static uint64_t g_state = 0x9e3779b97f4a7c15ull;

/* uniform in [-a, a) */
static float uniform(float a)
{
    g_state ^= g_state << 13;
    g_state ^= g_state >> 7;
    g_state ^= g_state << 17;
    return a * (2.0f * (float)((g_state >> 40) * (1.0 / 16777216.0)) - 1.0f);
}

static psk_node node(int op, int a, int b, float imm, int iparam)
{
    psk_node n;
    memset(&n, 0, sizeof n);
    n.op = op; n.a = a; n.b = b; n.c = -1; n.imm = imm; n.iparam = iparam;
    return n;
}

static psk_tensor_desc tensor2(int64_t d0, int64_t d1)
{
    psk_tensor_desc t;
    memset(&t, 0, sizeof t);
    t.rank = 2; t.shape[0] = d0; t.shape[1] = d1; t.dtype = PSK_F32;
    return t;
}

/* T > 0: the causal softmax of period T (against the oracle's dedicated
 * softmax); T == 0: the plain softmax (against its generic evaluator) */
static int softmax_case(int64_t R, int64_t C, int64_t T, int want_kind, hipStream_t stream)
{
    const float scale = 0.125f;
    psk_node nodes[9];
    int k = 0;
    nodes[k++] = node(PSK_OP_INPUT, -1, -1, 0.0f, 0);
    nodes[k++] = node(PSK_OP_CONST, -1, -1, scale, 0);
    nodes[k++] = node(PSK_OP_MUL, 0, 1, 0.0f, 0);
    if (T > 0) nodes[k++] = node(PSK_OP_CAUSAL_MASK, 2, -1, 0.0f, (int)T);
    const int yi = k - 1;
    nodes[k++] = node(PSK_OP_ROW_MAX, yi, -1, 0.0f, 0);
    nodes[k++] = node(PSK_OP_SUB, yi, yi + 1, 0.0f, 0);
    nodes[k++] = node(PSK_OP_EXP, yi + 2, -1, 0.0f, 0);
    nodes[k++] = node(PSK_OP_ROW_SUM, yi + 3, -1, 0.0f, 0);
    nodes[k++] = node(PSK_OP_DIV, yi + 3, yi + 4, 0.0f, 0);
    psk_tensor_desc in = tensor2(R, C);
    psk_group_desc d;
    memset(&d, 0, sizeof d);
    d.n_nodes = k; d.nodes = nodes; d.root = k - 1; d.n_inputs = 1; d.inputs = &in;
    d.out = tensor2(R, C); d.arith = PSK_F32;
    psk_group *g = NULL;
    CHECK(psk_group_create(&d, &g) == PSK_OK);
    psk_group_info info;
    CHECK(psk_group_get_info(g, &info) == PSK_OK && info.kind == want_kind);

    const size_t n = (size_t)(R * C), bytes = n * sizeof(float);
    float *x = (float *)malloc(bytes), *y = (float *)malloc(bytes), *ref = (float *)malloc(bytes);
    CHECK(x && y && ref);
    for (size_t i = 0; i < n; ++i) x[i] = uniform(24.0f);
    void *dx = NULL, *dy = NULL;
    HIP(hipMalloc(&dx, bytes));
    HIP(hipMalloc(&dy, bytes));
    HIP(hipMemcpy(dx, x, bytes, hipMemcpyHostToDevice));
    const void *ins[1] = {dx};
    CHECK(psk_group_run(g, ins, dy, (void *)stream) == PSK_OK);
    HIP(hipStreamSynchronize(stream));
    CHECK(psk_group_check(g) == PSK_OK);
    HIP(hipMemcpy(y, dy, bytes, hipMemcpyDeviceToHost));
    if (T > 0) {
        orc_softmax_causal(R, C, T, scale, x, ref, 0, R);
    } else {
        const orc_node on[8] = {{O_INPUT, -1, -1, -1, 0.0f, 0}, {O_CONST, -1, -1, -1, scale, 0},
                                {O_MUL, 0, 1, -1, 0.0f, 0},       {O_ROW_MAX, 2, -1, -1, 0.0f, 0},
                                {O_SUB, 2, 3, -1, 0.0f, 0},       {O_EXP, 4, -1, -1, 0.0f, 0},
                                {O_ROW_SUM, 5, -1, -1, 0.0f, 0},  {O_DIV, 5, 6, -1, 0.0f, 0}};
        const void *xin[1] = {x};
        const int32_t dt[1] = {0}, rank[1] = {2};
        int64_t shape[8] = {R, C, 0, 0, 0, 0, 0, 0};
        CHECK(orc_eval_group(8, on, 7, 1, xin, dt, rank, shape, 2, shape, 0, ref, 0, R) == 0);
    }
    size_t bad = 0;
    for (size_t i = 0; i < n; ++i)
        if (!(fabsf(y[i] - ref[i]) <= 1e-7f + 2e-6f * fabsf(ref[i]))) {
            if (bad == 0) printf("softmax [%lld,%lld] element %zu: gpu %.9g ref %.9g\n", (long long)R, (long long)C, i,
                                 (double)y[i], (double)ref[i]);
            ++bad;
        }
    CHECK(bad == 0);
    HIP(hipFree(dx));
    HIP(hipFree(dy));
    free(x); free(y); free(ref);
    psk_group_destroy(g);
    return 0;
}

static int adamw_case(hipStream_t stream)
{
    enum { L = 3 };
    const int64_t sizes[L] = {1, 1000, 4097};
    const double lr = 3e-4, b1 = 0.9, b2 = 0.999, eps = 1e-8, wd = 0.01;
    const int64_t t = 10;
    psk_leaf leaves[L];
    float *host[L][4], *want[L][3];
    void *dev[L][4];
    memset(leaves, 0, sizeof leaves);
    for (int l = 0; l < L; ++l) {
        const size_t bytes = (size_t)sizes[l] * sizeof(float);
        leaves[l].numel = sizes[l];
        for (int s = 0; s < 4; ++s) {
            host[l][s] = (float *)malloc(bytes);
            CHECK(host[l][s]);
            for (int64_t i = 0; i < sizes[l]; ++i) {
                float u = uniform(1.0f);
                host[l][s][i] = s == 0 ? 0.02f * u : s == 1 ? 0.01f * u : s == 2 ? 1e-3f * u : 1e-4f * fabsf(u);
            }
            HIP(hipMalloc(&dev[l][s], bytes));
            HIP(hipMemcpy(dev[l][s], host[l][s], bytes, hipMemcpyHostToDevice));
            leaves[l].slot[s] = dev[l][s];
        }
        for (int s = 0; s < 3; ++s) {
            want[l][s] = (float *)malloc(bytes);
            CHECK(want[l][s]);
        }
        orc_adamw(sizes[l], 0, host[l][0], 0, host[l][1], 0, host[l][2], host[l][3], lr, b1, b2, eps, wd, t,
                  want[l][0], want[l][1], want[l][2]);
    }
    const int32_t dts[4] = {PSK_F32, PSK_F32, PSK_F32, PSK_F32};
    psk_tree *tree = NULL;
    CHECK(psk_tree_create(leaves, L, 4, dts, &tree) == PSK_OK);
    psk_adamw_hp hp;
    memset(&hp, 0, sizeof hp);
    hp.lr = lr; hp.beta1 = b1; hp.beta2 = b2; hp.eps = eps; hp.weight_decay = wd; hp.t = t;
    CHECK(psk_adamw_step(tree, &hp, (void *)stream) == PSK_OK);
    HIP(hipStreamSynchronize(stream));
    /* in place: slots theta, m, v now hold theta', m', v' */
    const int out_slot[3] = {0, 2, 3};
    for (int l = 0; l < L; ++l) {
        const size_t bytes = (size_t)sizes[l] * sizeof(float);
        for (int k = 0; k < 3; ++k) {
            HIP(hipMemcpy(host[l][out_slot[k]], dev[l][out_slot[k]], bytes, hipMemcpyDeviceToHost));
            if (memcmp(host[l][out_slot[k]], want[l][k], bytes) != 0) {
                printf("adamw leaf %d output %d differs from the oracle\n", l, k);
                return 1;
            }
        }
    }
    psk_tree_destroy(tree);
    for (int l = 0; l < L; ++l) {
        for (int s = 0; s < 4; ++s) {
            HIP(hipFree(dev[l][s]));
            free(host[l][s]);
        }
        for (int s = 0; s < 3; ++s) free(want[l][s]);
    }
    return 0;
}

int main(void)
{
    int ndev = 0;
    HIP(hipGetDeviceCount(&ndev));
    CHECK(ndev > 0);
    HIP(hipSetDevice(0));
    hipStream_t stream;
    HIP(hipStreamCreate(&stream));
    if (softmax_case(300, 1000, 1000, 1, stream)) return 1;    /* register row kernel */
    if (softmax_case(6, 40000, 0, 4, stream)) return 1;        /* rows split over workgroups */
    setenv("PSK_LAYOUT", "tiled=1", 1);                          /* the tiled wide-row kernel */
    if (softmax_case(3, 40000, 0, 3, stream)) return 1;
    unsetenv("PSK_LAYOUT");
    if (adamw_case(stream)) return 1;
    HIP(hipStreamDestroy(stream));
    printf("ok\n");
    return 0;
}
