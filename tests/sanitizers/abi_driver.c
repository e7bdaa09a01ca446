/*
 * Host sanitizer run of the C ABI (test infrastructure).  Built with
 * AddressSanitizer and UndefinedBehaviorSanitizer around kda_api.cpp's host
 * code, it drives every entry point of include/kda.h through the host-side
 * work that precedes a launch: argument checks, workspace quotes and plans
 * over a grid of shapes (up to 2^40 tokens, where the size arithmetic is
 * widest), and the window planning of kda_chunk_fwd_windowed(_ex), whose
 * loops read the caller's host copy of cu_seqlens (a heap block of exactly
 * N + 1 values here).  It runs only where no GPU is visible: the device
 * pointers are placeholders that nothing dereferences, and every launch
 * fails with KDA_ERR_HIP before any kernel runs.
 * Exit status 0: every check held; 77: a GPU is visible, nothing was run.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kda.h"

int hipGetDeviceCount(int* count);   /* hipError_t, 0 = hipSuccess */

#define DEV ((void*)(uintptr_t)0x10000)   /* 256-byte aligned placeholder, never dereferenced */
#define ODD ((void*)(uintptr_t)0x10004)

static int failures = 0;
#define CHECK(cond, ...)                                         \
    do {                                                         \
        if (!(cond)) {                                           \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);                        \
            fputc('\n', stderr);                                 \
            ++failures;                                          \
        }                                                        \
    } while (0)

static kda_chunk_params_t params(int32_t batch, int64_t seqlen, int32_t n, int32_t H, int32_t dk, int32_t dv,
                                 int32_t C, int32_t dtype) {
    kda_chunk_params_t p;
    memset(&p, 0, sizeof p);
    p.batch = batch;
    p.seqlen = seqlen;
    p.num_seqs = n;
    p.num_heads = H;
    p.head_dim_k = dk;
    p.head_dim_v = dv;
    p.chunk_size = C;
    p.scale = 1.f;
    p.qkv_dtype = dtype;
    p.o_dtype = dtype;
    return p;
}

/* Quotes and plans over a grid of shapes: each returns a status, and a
 * shape the library accepts gets a nonzero quote. */
static void quotes(void) {
    static const int64_t lens[] = {0, 1, 63, 64, 65, 1000, 65536, (int64_t)1 << 34, (int64_t)1 << 40};
    static const int32_t dims[] = {16, 32, 64, 96, 128};
    static const int32_t heads[] = {1, 3, 32, 1 << 20};
    static const int32_t chunks[] = {16, 32, 64, 48};
    kda_chunk_options_t gated;
    memset(&gated, 0, sizeof gated);
    gated.gate = DEV;
    for (size_t a = 0; a < sizeof lens / sizeof lens[0]; ++a)
        for (size_t b = 0; b < sizeof dims / sizeof dims[0]; ++b)
            for (size_t c = 0; c < sizeof heads / sizeof heads[0]; ++c)
                for (size_t d = 0; d < sizeof chunks / sizeof chunks[0]; ++d)
                    for (int32_t dtype = 0; dtype < 3; ++dtype)
                        for (int32_t batch = 1; batch <= 4; batch += 3) {
                            kda_chunk_params_t p =
                                params(batch, lens[a], batch, heads[c], dims[b], dims[(b + 1) % 5], chunks[d], dtype);
                            size_t plain = 0, gate = 0;
                            kda_chunk_plan_t plan;
                            const kda_status_t s1 = kda_chunk_fwd_workspace_size(&p, &plain);
                            const kda_status_t s2 = kda_chunk_fwd_ex_workspace_size(&p, &gated, &gate);
                            const kda_status_t s3 = kda_chunk_fwd_plan(&p, 0, &plan);
                            CHECK(s1 == s2, "quote statuses %d %d", (int)s1, (int)s2);
                            CHECK(s1 != KDA_OK || (plain > 0 && gate >= plain && s3 == KDA_OK),
                                  "quote %zu gated %zu plan %d", plain, gate, (int)s3);
                            CHECK(kda_status_string(s1) != NULL, "status string");
                        }
    size_t out = 0;
    CHECK(kda_chunk_fwd_workspace_size(NULL, &out) == KDA_ERR_INVALID_ARG, "NULL params");
    kda_chunk_params_t p = params(1, 64, 1, 1, 64, 64, 64, KDA_DTYPE_BF16);
    CHECK(kda_chunk_fwd_workspace_size(&p, NULL) == KDA_ERR_INVALID_ARG, "NULL out");
    CHECK(kda_status_string((kda_status_t)99) != NULL, "unknown status string");
}

/* Argument errors of the one-piece calls: each returns before a launch. */
static void argument_errors(void) {
    kda_chunk_params_t p = params(1, 256, 1, 2, 128, 128, 64, KDA_DTYPE_BF16);
    CHECK(kda_chunk_fwd(&p, ODD, DEV, DEV, DEV, DEV, NULL, NULL, DEV, DEV, DEV, (size_t)1 << 40, NULL) ==
              KDA_ERR_INVALID_ARG, "misaligned q");
    CHECK(kda_chunk_fwd(&p, DEV, DEV, DEV, DEV, DEV, NULL, NULL, DEV, DEV, DEV, 16, NULL) == KDA_ERR_WORKSPACE,
          "small workspace");
    CHECK(kda_chunk_fwd(&p, DEV, DEV, DEV, DEV, DEV, NULL, NULL, DEV, DEV, ODD, (size_t)1 << 40, NULL) ==
              KDA_ERR_WORKSPACE, "misaligned workspace");
    kda_chunk_options_t op;
    memset(&op, 0, sizeof op);
    op.ckpt_every = 100;
    op.max_ckpts = 1;
    op.checkpoints = (float*)DEV;
    CHECK(kda_chunk_fwd_ex(&p, &op, DEV, DEV, DEV, DEV, DEV, NULL, NULL, DEV, DEV, DEV, (size_t)1 << 40, NULL) ==
              KDA_ERR_INVALID_ARG, "ckpt_every not a multiple of 64");
    kda_chunk_params_t huge = params(1, (int64_t)1 << 34, 1, 1, 128, 128, 64, KDA_DTYPE_BF16);
    CHECK(kda_chunk_fwd(&huge, DEV, DEV, DEV, DEV, DEV, NULL, NULL, DEV, DEV, DEV, (size_t)1 << 62, NULL) ==
              KDA_ERR_UNSUPPORTED, "beyond one dispatch");
    CHECK(kda_chunk_fwd_status(ODD, NULL) == KDA_ERR_INVALID_ARG, "status of a misaligned workspace");
    CHECK(kda_decode_step(0, 2, 128, 128, 1.f, 1, 1, DEV, DEV, DEV, DEV, DEV, DEV, DEV, NULL) == KDA_ERR_INVALID_ARG,
          "decode without sequences");
    kda_decode_options_t dop;
    memset(&dop, 0, sizeof dop);
    dop.pool_entries = -1;
    CHECK(kda_decode_step_ex(4, 2, 128, 128, 1.f, 1, 1, &dop, DEV, DEV, DEV, DEV, DEV, DEV, DEV, NULL) ==
              KDA_ERR_INVALID_ARG, "negative pool");
}

/* Window planning: a packed call of N sequences with the given lengths, in a
 * workspace of `bytes`; the plan runs to its first launch. */
static kda_status_t windowed(const int32_t* lens, int32_t n, int32_t H, size_t bytes, const kda_chunk_options_t* op,
                             int scramble) {
    int32_t* cu = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n + 1));
    if (!cu) return KDA_ERR_HIP;
    cu[0] = 0;
    for (int32_t i = 0; i < n; ++i) cu[i + 1] = cu[i] + lens[i];
    if (scramble && n > 1) cu[1] = cu[n] + 1;   /* breaks the layout: rejected on the host */
    kda_chunk_params_t p = params(1, cu[n], n, H, 128, 128, 64, KDA_DTYPE_BF16);
    const kda_status_t s = kda_chunk_fwd_windowed_ex(&p, op, DEV, DEV, DEV, DEV, DEV, DEV, DEV, cu, DEV,
                                                     (float*)DEV + (1 << 24), DEV, bytes, NULL);
    free(cu);
    return s;
}

static void window_planning(void) {
    static const int32_t lens[] = {0, 300, 4000, 17, 0, 900, 2500, 64, 1};
    const int32_t n = (int32_t)(sizeof lens / sizeof lens[0]);
    size_t one_chunk = 0, row = 0;
    kda_chunk_params_t p1 = params(1, 64, 1, 2, 128, 128, 64, KDA_DTYPE_BF16);
    kda_chunk_params_t p2 = params(1, 1024, 1, 2, 128, 128, 64, KDA_DTYPE_BF16);
    CHECK(kda_chunk_fwd_workspace_size(&p1, &one_chunk) == KDA_OK, "quote");
    CHECK(kda_chunk_fwd_workspace_size(&p2, &row) == KDA_OK, "quote");
    kda_chunk_options_t gated, ckpt;
    memset(&gated, 0, sizeof gated);
    gated.gate = DEV;
    gated.fuse_inputs = 1;
    gated.alpha_mode = 1;
    memset(&ckpt, 0, sizeof ckpt);
    ckpt.checkpoints = (float*)DEV + (1 << 26);
    ckpt.ckpt_every = 256;
    ckpt.max_ckpts = 5;
    const size_t budgets[] = {one_chunk, one_chunk * 3, row, row * 7, (size_t)1 << 40};
    for (size_t b = 0; b < sizeof budgets / sizeof budgets[0]; ++b) {
        /* plans that fit reach the first launch, which fails without a GPU */
        const kda_status_t s0 = windowed(lens, n, 2, budgets[b], NULL, 0);
        const kda_status_t s1 = windowed(lens, n, 2, budgets[b], &gated, 0);
        const kda_status_t s2 = windowed(lens, n, 2, budgets[b], &ckpt, 0);
        CHECK(s0 == KDA_ERR_HIP, "plain plan in %zu bytes: %d", budgets[b], (int)s0);
        CHECK(s1 == KDA_ERR_HIP || (s1 == KDA_ERR_WORKSPACE && b == 0), "gated plan in %zu bytes: %d", budgets[b],
              (int)s1);
        CHECK(s2 == KDA_ERR_HIP || (s2 == KDA_ERR_WORKSPACE && budgets[b] < row), "ckpt plan in %zu bytes: %d",
              budgets[b], (int)s2);
        CHECK(windowed(lens, n, 2, budgets[b], NULL, 1) == KDA_ERR_INVALID_ARG, "broken host cu_seqlens");
    }
    CHECK(windowed(lens, n, 2, 4096, NULL, 0) == KDA_ERR_WORKSPACE, "below one chunk");
    /* fixed-length rows, in windows of one chunk */
    kda_chunk_params_t p = params(3, 700, 3, 2, 128, 128, 64, KDA_DTYPE_BF16);
    CHECK(kda_chunk_fwd_windowed(&p, DEV, DEV, DEV, DEV, DEV, NULL, NULL, NULL, DEV, DEV, DEV, one_chunk, NULL) ==
              KDA_ERR_HIP, "rows in one-chunk windows");
}

int main(void) {
    int count = 0;
    if (hipGetDeviceCount(&count) == 0 && count > 0) {
        puts("a GPU is visible: the placeholder pointers must not reach it; not run");
        return 77;
    }
    quotes();
    argument_errors();
    window_planning();
    CHECK(kda_chunk_fwd_noalloc(NULL, DEV, DEV, DEV, DEV, DEV, NULL, NULL, DEV, DEV, NULL) == KDA_ERR_INVALID_ARG,
          "noalloc without params");
    if (failures) return 1;
    puts("ABI sanitizer run: ok");
    return 0;
}
