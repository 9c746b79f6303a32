/* The C ABI used from plain C99 (no C++ and no Python): the header compiles
 * as C, the library links, and the host-side calls behave as documented.
 * No GPU is touched: groups are created and emitted (hipRTC compiles without
 * a device), bodies partitioned, tree plans built.  Prints "ok" and exits 0
 * on success; prints the failing check and exits 1 otherwise. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "psk_fused.h"

#define CHECK(c) do { if (!(c)) { printf("check failed: %s (line %d): %s\n", #c, __LINE__, psk_last_error()); \
                                  return 1; } } while (0)

static psk_node node(int op, int a, int b, float imm, int iparam)
{
    psk_node n;
    memset(&n, 0, sizeof n);
    n.op = op; n.a = a; n.b = b; n.c = -1; n.imm = imm; n.iparam = iparam;
    return n;
}

static psk_tensor_desc tensor(int rank, int64_t d0, int64_t d1, int dtype)
{
    psk_tensor_desc t;
    memset(&t, 0, sizeof t);
    t.rank = rank; t.shape[0] = d0; t.shape[1] = d1; t.dtype = dtype;
    return t;
}

int main(void)
{
    CHECK(psk_version() == PSK_VERSION);
    CHECK(strcmp(psk_status_str(PSK_OK), "PSK_OK") == 0);

    /* softmax over [8, 64] f32: x*s, row max, subtract, exp, row sum, divide */
    psk_node nodes[8];
    nodes[0] = node(PSK_OP_INPUT, -1, -1, 0.0f, 0);
    nodes[1] = node(PSK_OP_CONST, -1, -1, 0.125f, 0);
    nodes[2] = node(PSK_OP_MUL, 0, 1, 0.0f, 0);
    nodes[3] = node(PSK_OP_ROW_MAX, 2, -1, 0.0f, 0);
    nodes[4] = node(PSK_OP_SUB, 2, 3, 0.0f, 0);
    nodes[5] = node(PSK_OP_EXP, 4, -1, 0.0f, 0);
    nodes[6] = node(PSK_OP_ROW_SUM, 5, -1, 0.0f, 0);
    nodes[7] = node(PSK_OP_DIV, 5, 6, 0.0f, 0);
    psk_tensor_desc in = tensor(2, 8, 64, PSK_F32);
    psk_group_desc d;
    memset(&d, 0, sizeof d);
    d.n_nodes = 8; d.nodes = nodes; d.root = 7; d.n_inputs = 1; d.inputs = &in;
    d.out = tensor(2, 8, 64, PSK_F32); d.arith = PSK_F32;

    size_t len = 0;
    CHECK(psk_group_source(&d, NULL, 0, &len) == PSK_OK && len > 0);
    char* src = (char*)malloc(len + 1);
    CHECK(src && psk_group_source(&d, src, len + 1, &len) == PSK_OK);
    CHECK(strstr(src, "extern \"C\" __global__") != NULL);
    free(src);

    psk_group* g = NULL;
    CHECK(psk_group_create(&d, &g) == PSK_OK && g != NULL);
    psk_group_info info;
    CHECK(psk_group_get_info(g, &info) == PSK_OK && info.kind == 1);
    psk_group_destroy(g);

    /* the online normalizer takes the same group; refusals leave no object */
    d.flags = PSK_GROUP_ONLINE;
    g = NULL;
    CHECK(psk_group_create(&d, &g) == PSK_OK);
    psk_group_destroy(g);
    d.flags = 0;
    d.root = 3;                       /* node 7 would be dead */
    g = (psk_group*)&d;
    CHECK(psk_group_create(&d, &g) != PSK_OK && g == NULL && strlen(psk_last_error()) > 0);
    CHECK(psk_group_create(NULL, &g) == PSK_E_NULL);

    /* partition: the chain x -> exp -> tanh is one group, with rows fused the
     * whole softmax is one group too */
    psk_tensor_desc types[8];
    for (int i = 0; i < 8; ++i) types[i] = tensor(2, 8, 64, PSK_F32);
    types[1] = tensor(0, 0, 0, PSK_F32);
    types[3] = tensor(2, 8, 1, PSK_F32);
    types[6] = tensor(2, 8, 1, PSK_F32);
    uint8_t out[8] = {0, 0, 0, 0, 0, 0, 0, 1};
    int32_t group_of[8], is_root[8], n_groups = 0;
    CHECK(psk_partition(8, nodes, types, out, group_of, is_root, &n_groups) == PSK_OK && n_groups == 5);
    CHECK(psk_partition_ex(8, nodes, types, out, PSK_PARTITION_ROWS, group_of, is_root, &n_groups) == PSK_OK);
    CHECK(n_groups == 1 && is_root[7] == 1 && group_of[0] == -1 && group_of[2] == group_of[7]);

    /* random damage to a valid descriptor: every request is either accepted
     * or refused with a status and a message; nothing else happens */
    {
        uint32_t seed = 12345u;
        psk_node pool[32];
        psk_tensor_desc ins[4], xout[2];
        int32_t xroot[2];
        int accepted = 0, refused = 0;
        for (int trial = 0; trial < 3000; ++trial) {
            memcpy(pool, nodes, sizeof nodes);
            for (int i = 8; i < 32; ++i) pool[i] = node(PSK_OP_ADD, i - 1, 0, 0.0f, 0);
            ins[0] = in; ins[1] = tensor(1, 64, 0, PSK_BF16); ins[2] = tensor(0, 0, 0, PSK_F32);
            ins[3] = tensor(2, 8, 64, PSK_U8);
            psk_group_desc q = d;
            q.nodes = pool; q.inputs = ins; q.n_inputs = 1; q.root = 7; q.n_nodes = 8; q.flags = 0;
            int n_damage = 1 + (int)((seed >> 8) % 3);
            for (int k = 0; k < n_damage; ++k) {
                seed = seed * 1664525u + 1013904223u;
                int i = (int)((seed >> 4) % 32);
                int what = (int)((seed >> 16) % 10);
                int v = (int)((seed >> 20) % 70) - 5;
                switch (what) {
                case 0: pool[i].op = v; break;
                case 1: pool[i].a = v; break;
                case 2: pool[i].b = v; break;
                case 3: q.root = v % 40; break;
                case 4: q.n_nodes = 1 + (int)((seed >> 9) % 32); q.root = q.n_nodes - 1; break;
                case 5: q.n_inputs = (int)((seed >> 9) % 5); break;
                case 6: ins[(seed >> 9) % 4].rank = v % 7; break;
                case 7: ins[(seed >> 9) % 4].shape[(seed >> 12) % 2] = v * 13; break;
                case 8: q.flags = (uint32_t)((seed >> 9) % 4); break;
                default:
                    xroot[0] = v % 10; xroot[1] = (v + 3) % 10;
                    xout[0] = tensor(2, 8, 64, (int)((seed >> 9) % 3)); xout[1] = tensor(2, 8, 1, PSK_F32);
                    q.n_extra = 1 + (int)((seed >> 11) % 2); q.extra_root = xroot; q.extra_out = xout;
                }
            }
            char buf[64];
            size_t n = 0;
            psk_status st = psk_group_source(&q, buf, sizeof buf, &n);
            if (st == PSK_OK) { CHECK(n > sizeof buf && strlen(buf) == sizeof buf - 1); ++accepted; }
            else {
                CHECK(st > PSK_OK && strlen(psk_last_error()) > 0);
                ++refused;
            }
        }
        CHECK(accepted > 100 && refused > 1000);
    }

    /* tree plan: prefix offsets and whole chunks */
    int64_t numel[3] = {5, 4096 * 3 + 1, 0}, n_chunks = 0, off[4];
    CHECK(psk_tree_plan(numel, 3, &n_chunks, off, NULL, NULL, NULL) == PSK_OK);
    CHECK(n_chunks == 5 && off[0] == 0 && off[1] == 5 && off[2] == 5 + 4096 * 3 + 1 && off[3] == off[2]);

    printf("ok\n");
    return 0;
}
