/*
 * abi_check.c -- a C caller of the library, built with gcc against
 * include/ecmd.h and linked to libecmd.so (tests/test_abi_c.py builds and
 * runs it).
 *
 *   abi_check          host only: builds the mixed-precision configuration
 *                      (fp16 x, y, z; t = x*y, u = t + z, v = t - z;
 *                      out0 = fp16(u*v), out1 = u + s) through the cmd_* calls,
 *                      plans a launch, walks every error status and checks
 *                      cmd_last_error, round-trips the Command through YAML.
 *   abi_check --gpu N  also launches it on the GPU over N elements holding the
 *                      hand-worked cases (tests/golden/hand_worked.txt) side by
 *                      side, checks every element, and times cmd_launch from C:
 *                      prints "launch_us <host us per call> <us per launch
 *                      back to back>".
 *
 * Prints "ABI OK" (and "GPU OK") and exits 0 on success; any failed check
 * prints its line and exits 1.
 */
#define _POSIX_C_SOURCE 199309L   /* clock_gettime */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

#include "ecmd.h"

#ifdef ECMD_ABI_GPU
#include <hip/hip_runtime_api.h>
#endif

static int failures = 0;
#define CHECK(cond)                                                          \
    do {                                                                     \
        if (!(cond)) {                                                       \
            fprintf(stderr, "abi_check.c:%d: check failed: %s\n", __LINE__, #cond); \
            ++failures;                                                      \
        }                                                                    \
    } while (0)
#define EXPECT_STATUS(call, want, h)                                         \
    do {                                                                     \
        int rc_ = (call);                                                    \
        if (rc_ != (want)) {                                                 \
            fprintf(stderr, "abi_check.c:%d: %s returned %d, expected %d (%s)\n", __LINE__, #call, rc_, \
                    (want), cmd_last_error(h));                              \
            ++failures;                                                      \
        } else if ((want) != CMD_OK && cmd_last_error(h)[0] == 0) {          \
            fprintf(stderr, "abi_check.c:%d: %s: empty error message\n", __LINE__, #call); \
            ++failures;                                                      \
        }                                                                    \
    } while (0)

/* The mixed-precision Command; arguments 0..2 fp16 loads, 3 the fp32 scalar,
 * 4 and 5 the stores. */
static cmd_t build_mixed(void)
{
    cmd_t h = NULL;
    cmd_tag x, y, z, s, xf, yf, zf, t, u, v, uv, o0, o1;
    int32_t ai;
    if (cmd_create(&h) != CMD_OK) return NULL;
    EXPECT_STATUS(cmd_load(h, CMD_F16, 1, &x, &ai), CMD_OK, h);
    CHECK(ai == 0);
    EXPECT_STATUS(cmd_load(h, CMD_F16, 1, &y, &ai), CMD_OK, h);
    EXPECT_STATUS(cmd_load(h, CMD_F16, 1, &z, &ai), CMD_OK, h);
    EXPECT_STATUS(cmd_scalar(h, CMD_F32, &s, &ai), CMD_OK, h);
    CHECK(ai == 3);
    EXPECT_STATUS(cmd_op(h, E_CVT, CMD_F32, x, -1, &xf), CMD_OK, h);
    EXPECT_STATUS(cmd_op(h, E_CVT, CMD_F32, y, -1, &yf), CMD_OK, h);
    EXPECT_STATUS(cmd_op(h, E_CVT, CMD_F32, z, -1, &zf), CMD_OK, h);
    EXPECT_STATUS(cmd_op(h, E_MUL, CMD_F32, xf, yf, &t), CMD_OK, h);
    EXPECT_STATUS(cmd_op(h, E_ADD, CMD_F32, t, zf, &u), CMD_OK, h);
    EXPECT_STATUS(cmd_op(h, E_SUB, CMD_F32, t, zf, &v), CMD_OK, h);
    EXPECT_STATUS(cmd_op(h, E_MUL, CMD_F32, u, v, &uv), CMD_OK, h);
    EXPECT_STATUS(cmd_op(h, E_CVT, CMD_F16, uv, -1, &o0), CMD_OK, h);
    EXPECT_STATUS(cmd_op(h, E_ADD, CMD_F32, u, s, &o1), CMD_OK, h);
    EXPECT_STATUS(cmd_store(h, o0, 1, &ai), CMD_OK, h);
    CHECK(ai == 4);
    EXPECT_STATUS(cmd_store(h, o1, 1, &ai), CMD_OK, h);
    CHECK(ai == 5);
    return h;
}

static void tensor(cmd_arg *a, int dtype, void *ptr, int64_t n)
{
    memset(a, 0, sizeof *a);
    a->kind = CMD_ARG_TENSOR;
    a->dtype = dtype;
    a->ptr = ptr;
    a->size[0] = n;
    a->stride[0] = 1;
}

static void scalar_f32(cmd_arg *a, float v)
{
    memset(a, 0, sizeof *a);
    a->kind = CMD_ARG_SCALAR;
    a->dtype = CMD_F32;
    memcpy(&a->bits, &v, 4);
}

static void mixed_args(cmd_arg *args, char *base, int64_t n)
{
    tensor(&args[0], CMD_F16, base, n);
    tensor(&args[1], CMD_F16, base + (4 << 20), n);
    tensor(&args[2], CMD_F16, base + (8 << 20), n);
    scalar_f32(&args[3], 0.5f);
    tensor(&args[4], CMD_F16, base + (12 << 20), n);
    tensor(&args[5], CMD_F32, base + (16 << 20), n);
}

static void host_checks(void)
{
    cmd_t h = build_mixed();
    CHECK(h != NULL);
    cmd_arg args[6];
    /* plan with addresses that are never dereferenced (cmd_plan is host only) */
    char *base = (char *)(uintptr_t)0x7f0000000000ull;
    mixed_args(args, base, 1 << 20);
    cmd_plan_info info;
    EXPECT_STATUS(cmd_plan(h, args, 6, &info), CMD_OK, h);
    CHECK(info.path == CMD_PATH_LINEAR);
    CHECK(info.specialised == 1);
    CHECK(strcmp(info.kernel, "linear_mixed_two_out") == 0);
    CHECK(info.block > 0 && info.grid > 0);
    CHECK(info.dims == 1 && info.size[3] == (1 << 20));
    /* the shared t is one multiply in the lowered program */
    char listing[4096];
    CHECK(cmd_dump(h, listing, sizeof listing) > 0);
    int muls = 0;
    for (const char *p = listing; (p = strstr(p, "mul.f32")) != NULL; ++p) ++muls;
    CHECK(muls == 2 * 2);   /* t and u*v, in the register and the LDS-entry listing */
    uint64_t hash1 = 0, hash2 = 0;
    EXPECT_STATUS(cmd_program_hash(h, &hash1), CMD_OK, h);

    /* --- launch-time checks, all before any HIP call --- */
    EXPECT_STATUS(cmd_plan(h, args, 5, &info), CMD_E_ARG, h);            /* argument count */
    EXPECT_STATUS(cmd_plan(h, NULL, 6, &info), CMD_E_ARG, h);
    EXPECT_STATUS(cmd_plan(h, args, 6, NULL), CMD_E_ARG, h);
    cmd_arg bad[6];
    memcpy(bad, args, sizeof bad);
    bad[3].kind = CMD_ARG_TENSOR;                                          /* kind */
    EXPECT_STATUS(cmd_plan(h, bad, 6, &info), CMD_E_ARG, h);
    memcpy(bad, args, sizeof bad);
    bad[1].dtype = CMD_F32;                                                /* dtype */
    EXPECT_STATUS(cmd_plan(h, bad, 6, &info), CMD_E_DTYPE, h);
    memcpy(bad, args, sizeof bad);
    bad[2].size[0] = 1000;                                                 /* shape */
    EXPECT_STATUS(cmd_plan(h, bad, 6, &info), CMD_E_SHAPE, h);
    memcpy(bad, args, sizeof bad);
    bad[0].stride[0] = -1;                                                 /* negative stride */
    EXPECT_STATUS(cmd_plan(h, bad, 6, &info), CMD_E_STRIDE, h);
    memcpy(bad, args, sizeof bad);
    bad[4].stride[0] = 0;                                                  /* store not one-to-one */
    EXPECT_STATUS(cmd_plan(h, bad, 6, &info), CMD_E_STRIDE, h);
    memcpy(bad, args, sizeof bad);
    bad[5].ptr = base + (12 << 20) + 4096;                                 /* outputs overlap */
    EXPECT_STATUS(cmd_plan(h, bad, 6, &info), CMD_E_ALIAS, h);
    memcpy(bad, args, sizeof bad);
    bad[4].ptr = (char *)args[1].ptr + 2;                                  /* output shifted over an input */
    EXPECT_STATUS(cmd_plan(h, bad, 6, &info), CMD_E_ALIAS, h);
    memcpy(bad, args, sizeof bad);
    bad[4].ptr = NULL;                                                     /* NULL with elements */
    EXPECT_STATUS(cmd_plan(h, bad, 6, &info), CMD_E_ARG, h);
    /* same checks on cmd_launch: refused before the runtime is touched */
    memcpy(bad, args, sizeof bad);
    bad[2].size[0] = 7;
    EXPECT_STATUS(cmd_launch(h, bad, 6, NULL), CMD_E_SHAPE, h);
    /* frozen after the plan */
    cmd_tag extra;
    EXPECT_STATUS(cmd_op(h, E_NEG, CMD_F32, 4, -1, &extra), CMD_E_STATE, h);
    EXPECT_STATUS(cmd_store(h, 4, 1, NULL), CMD_E_STATE, h);
    /* an empty shape succeeds with nothing launched */
    mixed_args(bad, NULL, 0);
    EXPECT_STATUS(cmd_launch(h, bad, 6, NULL), CMD_OK, h);

    /* YAML round trip: same program */
    int64_t len = cmd_to_yaml(h, NULL, 0);
    CHECK(len > 0);
    char *yaml = (char *)malloc((size_t)len + 1);
    CHECK(cmd_to_yaml(h, yaml, len + 1) == len);
    cmd_t h2 = NULL;
    EXPECT_STATUS(cmd_from_yaml(yaml, &h2), CMD_OK, NULL);
    EXPECT_STATUS(cmd_program_hash(h2, &hash2), CMD_OK, h2);
    CHECK(hash1 == hash2);
    CHECK(cmd_num_args(h2) == 6);
    free(yaml);
    cmd_destroy(h2);
    cmd_destroy(h);

    /* --- build-time checks --- */
    EXPECT_STATUS(cmd_create(NULL), CMD_E_ARG, NULL);
    CHECK(cmd_last_error(NULL)[0] != 0);
    cmd_t b = NULL;
    EXPECT_STATUS(cmd_create(&b), CMD_OK, b);
    cmd_tag a, f, q;
    EXPECT_STATUS(cmd_load(b, CMD_F32, 1, &a, NULL), CMD_OK, b);
    EXPECT_STATUS(cmd_load(b, CMD_I32, 1, &f, NULL), CMD_OK, b);
    EXPECT_STATUS(cmd_load(b, 9, 1, &q, NULL), CMD_E_DTYPE, b);            /* unknown dtype */
    EXPECT_STATUS(cmd_load(b, CMD_F32, 5, &q, NULL), CMD_E_LIMIT, b);      /* rank 5 */
    EXPECT_STATUS(cmd_op(b, E_ADD, CMD_F32, a, 7, &q), CMD_E_TAG, b);      /* forward tag */
    EXPECT_STATUS(cmd_op(b, E_ADD, CMD_F32, a, f, &q), CMD_E_DTYPE, b);    /* f32 + i32 */
    EXPECT_STATUS(cmd_op(b, E_CMP_LTU, 0, a, a, &q), CMD_E_DTYPE, b);      /* unsigned compare of f32 */
    EXPECT_STATUS(cmd_op(b, E_SELECT, 0, f, a, &q), CMD_E_ARG, b);         /* select needs cmd_select */
    EXPECT_STATUS(cmd_select(b, a, a, a, &q), CMD_E_DTYPE, b);             /* f32 condition */
    EXPECT_STATUS(cmd_op(b, 77, CMD_F32, a, a, &q), CMD_E_ARG, b);         /* unknown opcode */
    cmd_arg one[2];
    tensor(&one[0], CMD_F32, base, 16);
    tensor(&one[1], CMD_I32, base + 4096, 16);
    EXPECT_STATUS(cmd_plan(b, one, 2, &info), CMD_E_NOSTORE, b);           /* nothing stored */
    cmd_destroy(b);
    /* capacities */
    cmd_t c = NULL;
    EXPECT_STATUS(cmd_create(&c), CMD_OK, c);
    int rc = CMD_OK;
    for (int k = 0; k < CMD_MAX_ARGS + 1 && rc == CMD_OK; ++k) rc = cmd_scalar(c, CMD_F32, &q, NULL);
    CHECK(rc == CMD_E_LIMIT && cmd_last_error(c)[0] != 0);
    cmd_destroy(c);
    CHECK(cmd_destroy(NULL) == CMD_OK);
    CHECK(cmd_version() >= 100);
}

#ifdef ECMD_ABI_GPU
static double now_us(void)
{
    struct timespec ts;
    clock_gettime(CLOCK_MONOTONIC, &ts);
    return ts.tv_sec * 1e6 + ts.tv_nsec / 1e3;
}

#define HIP_OK(call)                                                                   \
    do {                                                                               \
        hipError_t e_ = (call);                                                        \
        if (e_ != hipSuccess) {                                                        \
            fprintf(stderr, "abi_check.c:%d: %s: %s\n", __LINE__, #call, hipGetErrorString(e_)); \
            exit(1);                                                                   \
        }                                                                              \
    } while (0)

/* The hand-worked mixed-precision cases: x, y, z (fp16 bits), out0 (fp16),
 * out1 (fp32), with s = 0.5. */
static const uint32_t kCases[][5] = {
    {0x3C00, 0x4000, 0x3800, 0x4380, 0x40400000},  /* 1, 2, 0.5: u*v = 3.75, u + s = 3 */
    {0x3C01, 0x3C00, 0x0000, 0x3C02, 0x3FC02000},  /* 1+2^-10, 1, 0 */
    {0x2400, 0x2400, 0x0000, 0x0001, 0x3F001000},  /* 2^-6 twice: u*v = 2^-24, the smallest subnormal */
    {0x0001, 0x3C00, 0x0000, 0x0000, 0x3F000001},  /* a subnormal input: 2^-48 underflows */
};

static void gpu_checks(int64_t n)
{
    cmd_t h = build_mixed();
    const int ncase = (int)(sizeof kCases / sizeof kCases[0]);
    uint16_t *hx = (uint16_t *)malloc(n * 2), *hy = (uint16_t *)malloc(n * 2), *hz = (uint16_t *)malloc(n * 2);
    uint16_t *h0 = (uint16_t *)malloc(n * 2);
    uint32_t *h1 = (uint32_t *)malloc(n * 4);
    for (int64_t i = 0; i < n; ++i) {
        hx[i] = (uint16_t)kCases[i % ncase][0];
        hy[i] = (uint16_t)kCases[i % ncase][1];
        hz[i] = (uint16_t)kCases[i % ncase][2];
    }
    void *dx, *dy, *dz, *d0, *d1;
    HIP_OK(hipMalloc(&dx, n * 2));
    HIP_OK(hipMalloc(&dy, n * 2));
    HIP_OK(hipMalloc(&dz, n * 2));
    HIP_OK(hipMalloc(&d0, n * 2));
    HIP_OK(hipMalloc(&d1, n * 4));
    HIP_OK(hipMemcpy(dx, hx, n * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dy, hy, n * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dz, hz, n * 2, hipMemcpyHostToDevice));
    cmd_arg args[6];
    tensor(&args[0], CMD_F16, dx, n);
    tensor(&args[1], CMD_F16, dy, n);
    tensor(&args[2], CMD_F16, dz, n);
    scalar_f32(&args[3], 0.5f);
    tensor(&args[4], CMD_F16, d0, n);
    tensor(&args[5], CMD_F32, d1, n);
    EXPECT_STATUS(cmd_launch(h, args, 6, NULL), CMD_OK, h);
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(h0, d0, n * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(h1, d1, n * 4, hipMemcpyDeviceToHost));
    int64_t bad = 0;
    for (int64_t i = 0; i < n; ++i)
        bad += h0[i] != kCases[i % ncase][3] || h1[i] != kCases[i % ncase][4];
    if (bad) fprintf(stderr, "abi_check.c: %lld of %lld elements differ from the hand-worked results\n",
                     (long long)bad, (long long)n);
    CHECK(bad == 0);
    /* host cost of one cmd_launch from C (same argument values: the cached
     * launch), and the rate of launches back to back */
    const int reps = 2000;
    for (int k = 0; k < 100; ++k) cmd_launch(h, args, 6, NULL);
    HIP_OK(hipDeviceSynchronize());
    double t0 = now_us();
    for (int k = 0; k < 20; ++k) CHECK(cmd_launch(h, args, 6, NULL) == CMD_OK);
    const double host_us = (now_us() - t0) / 20;
    HIP_OK(hipDeviceSynchronize());
    t0 = now_us();
    for (int k = 0; k < reps; ++k) cmd_launch(h, args, 6, NULL);
    HIP_OK(hipDeviceSynchronize());
    const double b2b_us = (now_us() - t0) / reps;
    printf("launch_us %.3f %.3f\n", host_us, b2b_us);
    /* a timed launch: the dispatch records the two events around the kernel */
    hipEvent_t e0, e1;
    HIP_OK(hipEventCreate(&e0));
    HIP_OK(hipEventCreate(&e1));
    EXPECT_STATUS(cmd_launch_timed(h, args, 6, NULL, e0, e1), CMD_OK, h);
    HIP_OK(hipEventSynchronize(e1));
    float kernel_ms = 0.f;
    HIP_OK(hipEventElapsedTime(&kernel_ms, e0, e1));
    CHECK(kernel_ms > 0.f && kernel_ms < 1000.f);
    printf("kernel_us %.3f\n", kernel_ms * 1e3);
    HIP_OK(hipEventDestroy(e0));
    HIP_OK(hipEventDestroy(e1));
    HIP_OK(hipFree(dx));
    HIP_OK(hipFree(dy));
    HIP_OK(hipFree(dz));
    HIP_OK(hipFree(d0));
    HIP_OK(hipFree(d1));
    free(hx), free(hy), free(hz), free(h0), free(h1);
    cmd_destroy(h);
}
#endif

int main(int argc, char **argv)
{
    host_checks();
    if (failures) return 1;
    printf("ABI OK\n");
#ifdef ECMD_ABI_GPU
    if (argc > 2 && strcmp(argv[1], "--gpu") == 0) {
        gpu_checks(atoll(argv[2]));
        if (failures) return 1;
        printf("GPU OK\n");
    }
#else
    (void)argc, (void)argv;
#endif
    fflush(stdout);
    return 0;
}
