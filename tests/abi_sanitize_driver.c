/* Host-only exercise of the library's validation, planning and sizing code,
 * built with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_sanitize_cpu.py.  No call here touches a GPU: every pointer is a
 * fake address, used only for range and aliasing arithmetic.  Exits nonzero
 * (and the sanitizers abort) on any unexpected status or memory error. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "muon_step.h"

static int failures = 0;

#define EXPECT(cond)                                                           \
    do {                                                                       \
        if (!(cond)) {                                                         \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                        \
        }                                                                      \
    } while (0)

/* Disjoint fake device ranges: matrix i's tensors start 2^36 bytes apart. */
static void *fake(int64_t i, int k) { return (void *)(uintptr_t)((1ull << 40) + (uint64_t)i * (1ull << 36) + (uint64_t)k * (1ull << 34)); }

static muon_matrix mat(int64_t i, int64_t rows, int64_t cols, int pd, int gd) {
    muon_matrix m;
    memset(&m, 0, sizeof m);
    m.param = fake(i, 0);
    m.grad = fake(i, 1);
    m.momentum = (float *)fake(i, 2);
    m.ns_out = (i % 3 == 0) ? (float *)fake(i, 3) : NULL;
    m.rows = rows;
    m.cols = cols;
    m.param_dtype = pd;
    m.grad_dtype = gd;
    return m;
}

static void plan(const muon_matrix *ms, int64_t n, const muon_hparams *hp, const char *what) {
    size_t bytes = 0;
    char msg[256];
    muon_status st = muon_check_step_args(ms, n, hp, msg, sizeof msg);
    EXPECT(st == MUON_OK);
    st = muon_workspace_bytes(ms, n, hp, &bytes);
    EXPECT(st == MUON_OK);
    EXPECT(bytes > 0);
    printf("%s: %lld matrices, workspace %zu bytes\n", what, (long long)n, bytes);
}

int main(void) {
    muon_ns_coeff sched[16];
    int64_t n = muon_schedule("deepseekv4", sched, 16);
    EXPECT(n == 10);
    EXPECT(muon_schedule("quintic", sched, 2) == 5);
    EXPECT(muon_schedule("quintic", NULL, 0) == 5);
    EXPECT(muon_schedule("no-such", sched, 16) == -1);
    EXPECT(muon_schedule(NULL, sched, 16) == -1);
    EXPECT(muon_abi_version() == MUON_STEP_ABI_VERSION);
    for (int s = -1; s < 7; ++s) EXPECT(muon_status_string((muon_status)s) != NULL);
    EXPECT(strlen(muon_last_error(NULL)) > 0);

    muon_hparams hp;
    memset(&hp, 0, sizeof hp);
    hp.lr = 0.02;
    hp.momentum = 0.95;
    hp.weight_decay = 0.1;
    hp.gamma = 0.2;
    hp.schedule = sched;
    hp.num_ns_steps = 10;
    hp.nesterov = 1;
    muon_schedule("deepseekv4", sched, 16);

    /* every workload's shapes, both precisions */
    for (int prec = 0; prec < 2; ++prec) {
        hp.ns_precision = prec;
        muon_matrix one = mat(0, 64, 128, MUON_F32, MUON_F32);
        plan(&one, 1, &hp, "single 64x128");
        muon_matrix dense[7];
        for (int i = 0; i < 4; ++i) dense[i] = mat(i, 4096, 4096, MUON_BF16, MUON_BF16);
        dense[4] = mat(4, 4096, 14336, MUON_BF16, MUON_BF16);
        dense[5] = mat(5, 4096, 14336, MUON_BF16, MUON_BF16);
        dense[6] = mat(6, 14336, 4096, MUON_BF16, MUON_BF16);
        plan(dense, 7, &hp, "dense block");
        muon_matrix aspect[4] = {mat(0, 1024, 16384, 1, 1), mat(1, 16384, 1024, 1, 1), mat(2, 7168, 7168, 1, 1),
                                 mat(3, 512, 32768, 1, 1)};
        plan(aspect, 4, &hp, "aspect-ratio set");
        muon_matrix *moe = (muon_matrix *)calloc(256, sizeof(muon_matrix));
        for (int i = 0; i < 256; ++i) moe[i] = mat(i, 2048, 7168, MUON_BF16, MUON_BF16);
        plan(moe, 256, &hp, "MoE expert batch");
        free(moe);
        muon_matrix *c5 = (muon_matrix *)calloc(27 * 196, sizeof(muon_matrix));
        int64_t k = 0;
        for (int layer = 0; layer < 27; ++layer) {
            for (int a = 0; a < 4; ++a, ++k) c5[k] = mat(k, 2048, 2048, 1, 1);
            for (int e = 0; e < 64; ++e) {
                c5[k] = mat(k, 2048, 1408, 1, 1); ++k;
                c5[k] = mat(k, 2048, 1408, 1, 1); ++k;
                c5[k] = mat(k, 1408, 2048, 1, 1); ++k;
            }
        }
        plan(c5, k, &hp, "16B-MoE step");
        free(c5);
        /* odd shapes, one of each */
        int64_t shapes[][2] = {{1, 1}, {1, 7}, {7, 1}, {33, 65}, {65, 33}, {257, 513}, {1408, 2048}, {300, 3000}};
        muon_matrix odd[8];
        for (int i = 0; i < 8; ++i) odd[i] = mat(i, shapes[i][0], shapes[i][1], i & 1, (i >> 1) & 1);
        plan(odd, 8, &hp, "odd shapes");
    }

    /* documented rejections */
    char msg[256];
    muon_matrix m2[2] = {mat(0, 64, 128, 1, 1), mat(1, 64, 128, 1, 1)};
    EXPECT(muon_check_step_args(NULL, 1, &hp, msg, sizeof msg) == MUON_ERR_INVALID_ARGUMENT);
    EXPECT(muon_check_step_args(m2, -1, &hp, msg, sizeof msg) == MUON_ERR_INVALID_ARGUMENT);
    EXPECT(muon_check_step_args(m2, 0, &hp, msg, sizeof msg) == MUON_OK);
    EXPECT(muon_check_step_args(m2, 2, NULL, msg, sizeof msg) == MUON_ERR_INVALID_ARGUMENT);
    m2[1].grad = m2[0].param; /* grad aliases another matrix's param */
    EXPECT(muon_check_step_args(m2, 2, &hp, msg, sizeof msg) == MUON_ERR_INVALID_ARGUMENT);
    m2[1] = mat(1, 0, 128, 1, 1);
    EXPECT(muon_check_step_args(m2, 2, &hp, msg, sizeof msg) == MUON_ERR_INVALID_ARGUMENT);
    m2[1] = mat(1, (int64_t)1 << 32, 128, 1, 1);
    EXPECT(muon_check_step_args(m2, 2, &hp, msg, sizeof msg) == MUON_ERR_INVALID_ARGUMENT);
    m2[1] = mat(1, 64, 128, 7, 1);
    EXPECT(muon_check_step_args(m2, 2, &hp, msg, sizeof msg) == MUON_ERR_INVALID_ARGUMENT);
    m2[1] = mat(1, 64, 128, 1, 1);
    m2[1].momentum = NULL;
    EXPECT(muon_check_step_args(m2, 2, &hp, msg, sizeof msg) == MUON_ERR_INVALID_ARGUMENT);
    m2[1] = mat(1, 64, 128, 1, 1);
    hp.num_ns_steps = 65;
    EXPECT(muon_check_step_args(m2, 2, &hp, msg, sizeof msg) == MUON_ERR_INVALID_ARGUMENT);
    hp.num_ns_steps = 3;
    hp.schedule = NULL;
    EXPECT(muon_check_step_args(m2, 2, &hp, msg, sizeof msg) == MUON_ERR_INVALID_ARGUMENT);
    hp.schedule = sched;
    hp.num_ns_steps = 0;
    EXPECT(muon_check_step_args(m2, 2, &hp, msg, sizeof msg) == MUON_OK);
    hp.num_ns_steps = 10;
    hp.lr = 1.0 / 0.0;
    EXPECT(muon_check_step_args(m2, 2, &hp, msg, sizeof msg) == MUON_ERR_INVALID_ARGUMENT);
    hp.lr = 0.02;
    hp.scale_mode = 9;
    EXPECT(muon_check_step_args(m2, 2, &hp, msg, sizeof msg) == MUON_ERR_INVALID_ARGUMENT);
    hp.scale_mode = MUON_SCALE_UNIT_RMS;
    EXPECT(muon_check_step_args(m2, 2, &hp, msg, sizeof msg) == MUON_OK);
    /* a truncated message buffer, and none at all */
    m2[1].grad = m2[0].param;
    EXPECT(muon_check_step_args(m2, 2, &hp, msg, 4) == MUON_ERR_INVALID_ARGUMENT);
    EXPECT(strlen(msg) == 3);
    EXPECT(muon_check_step_args(m2, 2, &hp, NULL, 0) == MUON_ERR_INVALID_ARGUMENT);

    muon_adamw_tensor t[2];
    memset(t, 0, sizeof t);
    for (int i = 0; i < 2; ++i) {
        t[i].param = fake(i, 0);
        t[i].grad = fake(i, 1);
        t[i].exp_avg = (float *)fake(i, 2);
        t[i].exp_avg_sq = (float *)fake(i, 3);
        t[i].numel = 102400 * 2048;
    }
    muon_adamw_hparams ah = {0.02, 0.9, 0.95, 1e-8, 0.1, 1};
    EXPECT(muon_check_adamw_args(t, 2, &ah, msg, sizeof msg) == MUON_OK);
    t[1].param_dtype = MUON_BF16;
    EXPECT(muon_check_adamw_args(t, 2, &ah, msg, sizeof msg) == MUON_ERR_UNSUPPORTED);
    t[1].param_dtype = MUON_F32;
    t[1].exp_avg = (float *)t[0].exp_avg_sq;
    EXPECT(muon_check_adamw_args(t, 2, &ah, msg, sizeof msg) == MUON_ERR_INVALID_ARGUMENT);
    ah.step = 0;
    EXPECT(muon_check_adamw_args(t, 1, &ah, msg, sizeof msg) == MUON_ERR_INVALID_ARGUMENT);

    size_t bytes = 0;
    EXPECT(muon_workspace_bytes(m2, 2, &hp, NULL) == MUON_ERR_INVALID_ARGUMENT);
    EXPECT(muon_workspace_bytes(NULL, 1, &hp, &bytes) == MUON_ERR_INVALID_ARGUMENT);
    if (failures) {
        fprintf(stderr, "%d expectations failed\n", failures);
        return 1;
    }
    printf("sanitized host checks: ok\n");
    return 0;
}
