/*
 * A C11 client of libfused_ar.so that uses nothing but include/fused_ar.h (and the HIP runtime for
 * device memory): evidence that the boundary is a plain C ABI.
 *
 *   fused_ar_c_check cpu   entry points that need no GPU: path rule, launch plans, argument checks
 *   fused_ar_c_check gpu   a ragged problem through path 1, path 2 and the unfused sequence,
 *                          compared with the CPU oracle (liboracle.so, test infrastructure)
 * Exit status 0 on success; the first failure is printed.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fused_ar.h"

/* The oracle library's entry points (oracle/fused_ar_oracle.c); it has no header of its own. */
int oracle_reduce(const uint16_t *const *inputs, int n, long long count, uint16_t *reduced);
int oracle_fused_ar_rmsnorm(const uint16_t *const *inputs, int n, const uint16_t *residual,
                            const uint16_t *weight, float eps, int m, int hidden,
                            uint16_t *residual_out, uint16_t *out);

#define CHECK(cond)                                                                  \
    do {                                                                             \
        if (!(cond)) {                                                               \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
            return 1;                                                                \
        }                                                                            \
    } while (0)

static const fa_bf16 *fake(uintptr_t i) { return (const fa_bf16 *)(0x7F0000000000u + i * (1u << 30)); }

static int cpu_checks(void)
{
    CHECK(fused_ar_auto_path(8, 16, 7168) == FUSED_AR_PATH_ONESTAGE);
    CHECK(fused_ar_auto_path(8, 4096, 7168) == FUSED_AR_PATH_ONESTAGE);
    CHECK(fused_ar_auto_path(8, 48, 32768) == FUSED_AR_PATH_TWOSTAGE);
    CHECK(fused_ar_auto_path(8, 49, 32768) == FUSED_AR_PATH_ONESTAGE);
    CHECK(fused_ar_auto_path(6, 16, 24576) == FUSED_AR_PATH_TWOSTAGE);
    CHECK(fused_ar_auto_path(6, 17, 24576) == FUSED_AR_PATH_ONESTAGE);
    CHECK(fused_ar_auto_path(0, 1, 7168) == FUSED_AR_ERR_INVALID);
    CHECK(fused_ar_auto_path(8, 1, 0) == FUSED_AR_ERR_INVALID);
    CHECK(fused_ar_auto_path_tp(8, 16, 7168) == FUSED_AR_PATH_ONESTAGE);
    CHECK(fused_ar_auto_path_tp(8, 17, 7168) == FUSED_AR_PATH_TWOSTAGE);
    CHECK(fused_ar_auto_path_tp(4, 32, 7168) == FUSED_AR_PATH_ONESTAGE);
    CHECK(fused_ar_auto_path_tp(0, 1, 7168) == FUSED_AR_ERR_INVALID);

    fused_ar_launch_plan plan;
    CHECK(fused_ar_describe_launch(8, 4096, 7168, FUSED_AR_PATH_ONESTAGE, &plan) == FUSED_AR_OK);
    CHECK(plan.kernels == 1 && strcmp(plan.launch[0].name, "onestage") == 0);
    CHECK(plan.launch[0].grid == 4096 && plan.launch[0].block == 448 && plan.launch[0].per_thread == 2 &&
          plan.launch[0].lds_bytes == 64u * 1024u); /* a long streaming call: two packs per thread */
    CHECK(fused_ar_describe_launch(8, 4096, 7168, FUSED_AR_PATH_UNFUSED, &plan) == FUSED_AR_OK);
    CHECK(plan.kernels == 3 && strcmp(plan.launch[2].name, "rmsnorm") == 0);
    fused_ar_options opt = {FUSED_AR_WAVE_BPERMUTE, FUSED_AR_STAGE1_LDS, 0, 0, FUSED_AR_LOAD_AUTO, 0,
                            FUSED_AR_CHUNKS_AUTO, 0};
    CHECK(fused_ar_describe_launch_ex(4, 64, 7168, FUSED_AR_PATH_TWOSTAGE, &opt, &plan) == FUSED_AR_OK);
    CHECK(strcmp(plan.launch[0].name, "stage1_reduce_lds") == 0 && plan.launch[0].block == 256);

    const fa_bf16 *ins[3] = {fake(0), fake(1), fake(2)};
    CHECK(fused_ar_rmsnorm_check(ins, 3, fake(3), fake(4), 1e-6f, 8, 4096, (fa_bf16 *)fake(5),
                                 (fa_bf16 *)fake(6), FUSED_AR_PATH_AUTO) == FUSED_AR_OK);
    CHECK(fused_ar_rmsnorm_check(ins, 3, fake(3), fake(4), 1e-6f, 8, 4100, (fa_bf16 *)fake(5),
                                 (fa_bf16 *)fake(6), FUSED_AR_PATH_AUTO) == FUSED_AR_ERR_SHAPE);
    CHECK(fused_ar_rmsnorm_check(ins, 3, fake(3), fake(4), 1e-6f, 8, 4096, (fa_bf16 *)fake(1),
                                 (fa_bf16 *)fake(6), FUSED_AR_PATH_AUTO) == FUSED_AR_ERR_ALIAS);
    CHECK(fused_ar_rmsnorm(ins, 3, fake(3), fake(4), -1.0f, 8, 4096, (fa_bf16 *)fake(5),
                           (fa_bf16 *)fake(6), FUSED_AR_PATH_AUTO, NULL) == FUSED_AR_ERR_INVALID);
    CHECK(fused_ar_strerror(FUSED_AR_ERR_ALIGN) != NULL);
    CHECK(fused_ar_strerror(12345) != NULL && fused_ar_strerror(-12345) != NULL);

    /* extremes of the scalar arguments: no overflow in the plan arithmetic */
    CHECK(fused_ar_describe_launch(8, 2147483647, 32768, FUSED_AR_PATH_ONESTAGE, &plan) == FUSED_AR_OK);
    CHECK(plan.launch[0].launches == 2048u && plan.launch[0].grid == (1u << 20));
    CHECK(fused_ar_describe_launch(8, 2147483647, 32768, FUSED_AR_PATH_UNFUSED, &plan) == FUSED_AR_OK);
    CHECK(plan.kernels == 3);
    CHECK(fused_ar_describe_launch(8, 2147483647, 32768, FUSED_AR_PATH_TWOSTAGE, &plan) == FUSED_AR_OK);
    /* (2^31 - 1) * 4096 packs: 8192 flat launches of 2^30 packs (the last one short), 512-thread
       workgroups at this size */
    CHECK(plan.launch[0].launches == 8192u && plan.launch[0].grid == (1u << 21) &&
          plan.launch[0].block == 512u && plan.launch[0].per_thread == 1u);
    fused_ar_options lds = {FUSED_AR_WAVE_DPP, FUSED_AR_STAGE1_LDS, 0, 0, FUSED_AR_LOAD_STREAM, 0,
                            FUSED_AR_CHUNKS_AUTO, 0};
    CHECK(fused_ar_describe_launch_ex(8, 2147483647, 32768, FUSED_AR_PATH_TWOSTAGE, &lds, &plan) ==
          FUSED_AR_OK);
    CHECK(plan.launch[0].launches == 8192u && plan.launch[0].grid == (1u << 21));
    /* 2^30 + 4096 packs: a second launch for the last row */
    CHECK(fused_ar_describe_launch(2, 262145, 32768, FUSED_AR_PATH_TWOSTAGE, &plan) == FUSED_AR_OK);
    CHECK(plan.launch[0].launches == 2u && plan.launch[0].grid == (1u << 21));
    /* the flat workgroup: 256 threads below 2^20 packs, 512 from there on */
    CHECK(fused_ar_describe_launch(8, 1023, 8192, FUSED_AR_PATH_TWOSTAGE, &plan) == FUSED_AR_OK);
    CHECK(plan.launch[0].block == 256u && plan.launch[0].grid == 1023u * 4u);
    CHECK(fused_ar_describe_launch(8, 1024, 8192, FUSED_AR_PATH_TWOSTAGE, &plan) == FUSED_AR_OK);
    CHECK(plan.launch[0].block == 512u && plan.launch[0].grid == 1024u * 2u);
    CHECK(fused_ar_describe_launch(8, -2147483647 - 1, 8, 1, &plan) == FUSED_AR_ERR_INVALID);
    CHECK(fused_ar_describe_launch(8, 1, 2147483647, 1, &plan) == FUSED_AR_ERR_SHAPE);
    CHECK(fused_ar_describe_launch(8, 1, 2147483640, 1, &plan) == FUSED_AR_ERR_SHAPE);
    CHECK(fused_ar_describe_launch(8, 1, 8, 1, NULL) == FUSED_AR_ERR_INVALID);
    for (int n = -1; n <= 9; ++n)
        for (int path = -1; path <= 4; ++path)
            for (int m = 0; m <= 40; m += 17) {
                const int rc = fused_ar_describe_launch(n, m, 7168, path, &plan);
                CHECK(rc == ((n >= 1 && n <= 8 && path >= 0 && path <= 3) ? FUSED_AR_OK
                                                                          : FUSED_AR_ERR_INVALID));
            }
    /* a huge m: the byte extents are checked without wrapping */
    CHECK(fused_ar_rmsnorm_check(ins, 3, fake(3), fake(4), 1e-6f, 2147483647, 32768,
                                 (fa_bf16 *)fake(5), (fa_bf16 *)fake(6), 1) == FUSED_AR_ERR_ALIAS);
    const fa_bf16 *top[1] = {(const fa_bf16 *)(uintptr_t)0xFFFFFFFFFFFF0000u};
    CHECK(fused_ar_rmsnorm_check(top, 1, fake(3), fake(4), 1e-6f, 8, 4096, (fa_bf16 *)fake(5),
                                 (fa_bf16 *)fake(6), 1) == FUSED_AR_ERR_INVALID);
    /* 2^31 rows of 2^31 - 8 elements: 2^63 bytes per plane, no size_t overflow; the extents
       overlap the inputs, and an output near the top of the address space wraps */
    CHECK(fused_ar_reduce(ins, 3, 2147483647, 2147483640, (fa_bf16 *)fake(9), NULL) ==
          FUSED_AR_ERR_ALIAS);
    CHECK(fused_ar_reduce(ins, 3, 2147483647, 2147483640,
                          (fa_bf16 *)(uintptr_t)0xFFFF000000000000u, NULL) == FUSED_AR_ERR_INVALID);
    fused_ar_options bad = {0, 0, 96, 0, 0, 0, 0, 0};
    fused_ar_options bad_policy = {0, 0, 0, 0, 3, 0, 0, 0};
    fused_ar_options bad_rows = {0, 0, 0, 0, 0, (1 << 20) + 1, 0, 0};
    fused_ar_options bad_schedule = {0, 0, 0, 0, 0, 0, 3, 0};
    fused_ar_options bad_stage1 = {0, 0, 0, 0, 0, 0, 0, 3};
    fused_ar_options stage1_chunks = {0, 0, 0, 0, 0, 512, 0, FUSED_AR_RESIDUAL_STAGE1};
    CHECK(fused_ar_describe_launch_ex(8, 64, 7168, 2, &bad_stage1, &plan) == FUSED_AR_ERR_INVALID);
    CHECK(fused_ar_describe_launch_ex(8, 64, 7168, 2, &stage1_chunks, &plan) == FUSED_AR_ERR_INVALID);
    fused_ar_options stage1_res = {0, 0, 0, 0, 0, 0, 0, FUSED_AR_RESIDUAL_STAGE1};
    CHECK(fused_ar_describe_launch_ex(8, 4096, 7168, 2, &stage1_res, &plan) == FUSED_AR_OK);
    CHECK(plan.kernels == 2 && strcmp(plan.launch[0].name, "stage1_reduce_residual") == 0 &&
          strcmp(plan.launch[1].name, "stage2_rmsnorm") == 0 && plan.launch[1].per_thread == 2u);
    CHECK(fused_ar_describe_launch_ex(8, 64, 7168, 2, &bad_rows, &plan) == FUSED_AR_ERR_INVALID);
    CHECK(fused_ar_describe_launch_ex(8, 64, 7168, 2, &bad_schedule, &plan) == FUSED_AR_ERR_INVALID);
    /* the two-stage path in chunks of one row at the largest m: no overflow in the chunk count */
    fused_ar_options one_row = {0, 0, 0, 0, 0, 1, FUSED_AR_CHUNKS_SEQUENTIAL, 0};
    CHECK(fused_ar_describe_launch_ex(8, 2147483647, 32768, 2, &one_row, &plan) == FUSED_AR_OK);
    CHECK(plan.kernels == 2 && plan.launch[0].launches == 2147483647u &&
          plan.launch[1].launches == 2147483647u && plan.launch[1].grid == 1u);
    one_row.schedule = FUSED_AR_CHUNKS_PIPELINED;
    CHECK(fused_ar_describe_launch_ex(8, 2147483647, 32768, 2, &one_row, &plan) == FUSED_AR_OK);
    CHECK(plan.kernels == 3 && strcmp(plan.launch[1].name, "stage_pipe") == 0 &&
          plan.launch[1].launches == 2147483646u && plan.launch[1].grid == 2u);
    fused_ar_options big_rows = {0, 0, 0, 0, 0, 1 << 20, FUSED_AR_CHUNKS_SEQUENTIAL, 0};
    CHECK(fused_ar_describe_launch_ex(8, 2147483647, 32768, 2, &big_rows, &plan) == FUSED_AR_OK);
    /* 2048 chunks of 2^20 rows (the last one row short) of 2^32 packs: four flat launches each */
    CHECK(plan.launch[0].launches == 2048u * 4u && plan.launch[1].launches == 2048u);
    CHECK(fused_ar_rmsnorm_ex(ins, 3, fake(3), fake(4), 1e-6f, 8, 4096, (fa_bf16 *)fake(5),
                              (fa_bf16 *)fake(6), 1, &bad, NULL) == FUSED_AR_ERR_INVALID);
    CHECK(fused_ar_rmsnorm_ex(ins, 3, fake(3), fake(4), 1e-6f, 8, 4096, (fa_bf16 *)fake(5),
                              (fa_bf16 *)fake(6), 1, &bad_policy, NULL) == FUSED_AR_ERR_INVALID);
    /* automatic load policy: ordinary loads up to 128 MiB read per call, streaming above */
    CHECK(fused_ar_describe_launch(8, 1040, 7168, 1, &plan) == FUSED_AR_OK && plan.launch[0].streaming == 0);
    CHECK(fused_ar_describe_launch(8, 1041, 7168, 1, &plan) == FUSED_AR_OK && plan.launch[0].streaming == 1);
    /* split rows: workspace size, scalar and buffer checks (all rejected before any launch) */
    CHECK(fused_ar_split_workspace_bytes(3, 7168, 0) == 3u * 4u * sizeof(float));
    CHECK(fused_ar_split_workspace_bytes(2147483647, 32768, 64) == (size_t)2147483647 * 64u * 4u);
    CHECK(fused_ar_split_workspace_bytes(-1, 7168, 0) == 0 && fused_ar_split_workspace_bytes(1, 7168, 65) == 0);
    CHECK(fused_ar_split_workspace_bytes(1, 16384, 1) == 0 && fused_ar_split_workspace_bytes(1, 4100, 0) == 0);
    {
        void *ws = (void *)fake(7);
        const size_t need = fused_ar_split_workspace_bytes(8, 4096, 0);
        CHECK(fused_ar_rmsnorm_split(ins, 3, fake(3), fake(4), 1e-6f, 8, 4096, (fa_bf16 *)fake(5),
                                     (fa_bf16 *)fake(6), 0, NULL, need, NULL) == FUSED_AR_ERR_INVALID);
        CHECK(fused_ar_rmsnorm_split(ins, 3, fake(3), fake(4), 1e-6f, 8, 4096, (fa_bf16 *)fake(5),
                                     (fa_bf16 *)fake(6), 0, ws, need - 1, NULL) == FUSED_AR_ERR_INVALID);
        CHECK(fused_ar_rmsnorm_split(ins, 3, fake(3), fake(4), 1e-6f, 8, 4096, (fa_bf16 *)fake(5),
                                     (fa_bf16 *)fake(6), 0, (char *)ws + 8, need, NULL) == FUSED_AR_ERR_ALIGN);
        CHECK(fused_ar_rmsnorm_split(ins, 3, fake(3), fake(4), 1e-6f, 8, 4096, (fa_bf16 *)fake(5),
                                     (fa_bf16 *)fake(6), 0, (void *)fake(6), need, NULL) == FUSED_AR_ERR_ALIAS);
        CHECK(fused_ar_rmsnorm_split(ins, 3, fake(3), fake(4), 1e-6f, 8, 4096, (fa_bf16 *)fake(5),
                                     (fa_bf16 *)fake(6), 99, ws, need, NULL) == FUSED_AR_ERR_INVALID);
        CHECK(fused_ar_rmsnorm_split(ins, 3, fake(3), fake(4), 1e-6f, 8, 16384, (fa_bf16 *)fake(5),
                                     (fa_bf16 *)fake(6), 1, ws, need, NULL) == FUSED_AR_ERR_SHAPE);
        CHECK(fused_ar_rmsnorm_split(NULL, 3, NULL, NULL, 1e-6f, 0, 4096, NULL, NULL, 0, NULL, 0, NULL) ==
              FUSED_AR_OK); /* m == 0 */
    }
    printf("cpu checks passed\n");
    return 0;
}

/* Random bf16 bits with a moderate exponent range, from a 64-bit LCG (test input only). */
static uint64_t lcg_state = 0x853c49e6748fea9bu;
static fa_bf16 random_bf16(int lo_exp, int hi_exp)
{
    lcg_state = lcg_state * 6364136223846793005u + 1442695040888963407u;
    uint32_t r = (uint32_t)(lcg_state >> 33);
    uint32_t sign = r & 1u, mant = (r >> 1) & 0x7Fu;
    uint32_t expo = (uint32_t)(lo_exp + 127) + (r >> 8) % (uint32_t)(hi_exp - lo_exp + 1);
    return (fa_bf16)((sign << 15) | (expo << 7) | mant);
}

static int ordinal(fa_bf16 b) { return (b & 0x8000) ? -(int)(b & 0x7FFF) : (int)b; }

#define HIP_OK(call) CHECK((call) == hipSuccess)

static int gpu_checks(void)
{
    enum { N = 5, M = 7, H = 520 };  /* 65 packs per row: a ragged second wave */
    const size_t plane = (size_t)M * H;
    fa_bf16 *h_in[N], *h_res = malloc(plane * 2), *h_w = malloc(H * 2);
    fa_bf16 *want_ro = malloc(plane * 2), *want_out = malloc(plane * 2);
    fa_bf16 *got_ro = malloc(plane * 2), *got_out = malloc(plane * 2);
    CHECK(h_res && h_w && want_ro && want_out && got_ro && got_out);
    for (int i = 0; i < N; ++i) {
        h_in[i] = malloc(plane * 2);
        CHECK(h_in[i]);
        for (size_t j = 0; j < plane; ++j)
            h_in[i][j] = random_bf16(-8, 2);
    }
    for (size_t j = 0; j < plane; ++j)
        h_res[j] = random_bf16(-4, 1);
    for (int j = 0; j < H; ++j)
        h_w[j] = random_bf16(-1, 0);
    const float eps = 1e-6f;
    CHECK(oracle_fused_ar_rmsnorm((const uint16_t *const *)h_in, N, h_res, h_w, eps, M, H, want_ro,
                                  want_out) == 0);

    void *d_in[N], *d_res, *d_w, *d_ro, *d_out;
    for (int i = 0; i < N; ++i) {
        HIP_OK(hipMalloc(&d_in[i], plane * 2));
        HIP_OK(hipMemcpy(d_in[i], h_in[i], plane * 2, hipMemcpyHostToDevice));
    }
    HIP_OK(hipMalloc(&d_res, plane * 2));
    HIP_OK(hipMalloc(&d_w, H * 2));
    HIP_OK(hipMalloc(&d_ro, plane * 2));
    HIP_OK(hipMalloc(&d_out, plane * 2));
    HIP_OK(hipMemcpy(d_res, h_res, plane * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_w, h_w, H * 2, hipMemcpyHostToDevice));

    const fa_bf16 *ins[N];
    for (int i = 0; i < N; ++i)
        ins[i] = (const fa_bf16 *)d_in[i];
    /* variants 0-2: path 1, path 2 and the unfused sequence on the null stream; 3-4: paths 1 and 2
       captured from a stream of the caller's into a HIP graph, the graph replayed three times */
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    for (int variant = 0; variant < 5; ++variant) {
        hipGraph_t graph = NULL;
        hipGraphExec_t exec = NULL;
        if (variant >= 3) {
            HIP_OK(hipStreamBeginCapture(stream, hipStreamCaptureModeGlobal));
            const int rc = fused_ar_rmsnorm(ins, N, d_res, d_w, eps, M, H, d_ro, d_out, variant - 2,
                                            stream);
            HIP_OK(hipStreamEndCapture(stream, &graph));
            CHECK(rc == FUSED_AR_OK);
            HIP_OK(hipGraphInstantiate(&exec, graph, NULL, NULL, 0));
        }
        for (int replay = 0; replay < (variant >= 3 ? 3 : 1); ++replay) {
            HIP_OK(hipMemset(d_ro, 0xFF, plane * 2));
            HIP_OK(hipMemset(d_out, 0xFF, plane * 2));
            HIP_OK(hipDeviceSynchronize());
            int rc = FUSED_AR_OK;
            if (variant < 2)
                rc = fused_ar_rmsnorm(ins, N, d_res, d_w, eps, M, H, d_ro, d_out, variant + 1, NULL);
            else if (variant == 2)
                rc = fused_ar_unfused_rmsnorm(ins, N, d_res, d_w, eps, M, H, d_ro, d_out, NULL);
            else
                HIP_OK(hipGraphLaunch(exec, stream));
            CHECK(rc == FUSED_AR_OK);
            HIP_OK(hipDeviceSynchronize());
            HIP_OK(hipMemcpy(got_ro, d_ro, plane * 2, hipMemcpyDeviceToHost));
            HIP_OK(hipMemcpy(got_out, d_out, plane * 2, hipMemcpyDeviceToHost));
            for (size_t j = 0; j < plane; ++j) {
                if (got_ro[j] != want_ro[j]) {
                    fprintf(stderr, "variant %d replay %d: residual_out[%zu] = %#06x, oracle %#06x\n",
                            variant, replay, j, got_ro[j], want_ro[j]);
                    return 1;
                }
                const int d = ordinal(got_out[j]) - ordinal(want_out[j]);
                if (d > 1 || d < -1) {
                    fprintf(stderr, "variant %d replay %d: out[%zu] = %#06x, oracle %#06x\n",
                            variant, replay, j, got_out[j], want_out[j]);
                    return 1;
                }
            }
        }
        if (exec != NULL) {
            HIP_OK(hipGraphExecDestroy(exec));
            HIP_OK(hipGraphDestroy(graph));
        }
    }
    HIP_OK(hipStreamDestroy(stream));

    /* split rows: 3 slices of 22, 22 and 21 packs per row, the square-sums in a workspace */
    {
        const size_t ws_bytes = fused_ar_split_workspace_bytes(M, H, 3);
        CHECK(ws_bytes == (size_t)M * 3 * sizeof(float));
        void *d_ws;
        HIP_OK(hipMalloc(&d_ws, ws_bytes));
        HIP_OK(hipMemset(d_ro, 0xFF, plane * 2));
        HIP_OK(hipMemset(d_out, 0xFF, plane * 2));
        CHECK(fused_ar_rmsnorm_split(ins, N, d_res, d_w, eps, M, H, d_ro, d_out, 3, d_ws, ws_bytes - 4,
                                     NULL) == FUSED_AR_ERR_INVALID);
        CHECK(fused_ar_rmsnorm_split(ins, N, d_res, d_w, eps, M, H, d_ro, d_out, 3, d_ws, ws_bytes,
                                     NULL) == FUSED_AR_OK);
        HIP_OK(hipDeviceSynchronize());
        HIP_OK(hipMemcpy(got_ro, d_ro, plane * 2, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(got_out, d_out, plane * 2, hipMemcpyDeviceToHost));
        for (size_t j = 0; j < plane; ++j) {
            const int d = ordinal(got_out[j]) - ordinal(want_out[j]);
            if (got_ro[j] != want_ro[j] || d > 1 || d < -1) {
                fprintf(stderr, "split rows: element %zu: residual_out %#06x (oracle %#06x), out %#06x "
                        "(oracle %#06x)\n", j, got_ro[j], want_ro[j], got_out[j], want_out[j]);
                return 1;
            }
        }
        HIP_OK(hipFree(d_ws));
    }

    /* the reduce alone, bit-exact against the oracle's */
    CHECK(oracle_reduce((const uint16_t *const *)h_in, N, (long long)plane, want_ro) == 0);
    HIP_OK(hipMemset(d_ro, 0xFF, plane * 2));
    CHECK(fused_ar_reduce(ins, N, M, H, d_ro, NULL) == FUSED_AR_OK);
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(got_ro, d_ro, plane * 2, hipMemcpyDeviceToHost));
    for (size_t j = 0; j < plane; ++j) {
        if (got_ro[j] != want_ro[j]) {
            fprintf(stderr, "reduce[%zu] = %#06x, oracle %#06x\n", j, got_ro[j], want_ro[j]);
            return 1;
        }
    }
    for (int i = 0; i < N; ++i) {
        HIP_OK(hipFree(d_in[i]));
        free(h_in[i]);
    }
    HIP_OK(hipFree(d_res));
    HIP_OK(hipFree(d_w));
    HIP_OK(hipFree(d_ro));
    HIP_OK(hipFree(d_out));
    free(h_res); free(h_w); free(want_ro); free(want_out); free(got_ro); free(got_out);
    printf("gpu checks passed: path 1, path 2 and unfused (eager and graph-captured), split rows and the reduce match the oracle\n");
    return 0;
}

int main(int argc, char **argv)
{
    if (argc == 2 && strcmp(argv[1], "cpu") == 0)
        return cpu_checks();
    if (argc == 2 && strcmp(argv[1], "gpu") == 0)
        return gpu_checks();
    fprintf(stderr, "usage: %s cpu|gpu\n", argv[0]);
    return 2;
}
