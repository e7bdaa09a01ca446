/*
 * Host sanitizer run of the fp64 oracle (test infrastructure).  Built with
 * AddressSanitizer and UndefinedBehaviorSanitizer together with
 * oracle/kda_oracle.c, it calls the oracle on small inputs whose arrays are
 * heap blocks of exactly the sizes the oracle's header comment documents, so
 * a read or write past any of them is reported.  It also checks the argument
 * errors and one closed form: with alpha = 1 and beta = 0 the state never
 * changes, so the final state is S0 and o_t = scale * q_t S0.
 * Exit status 0: every call returned what it should.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int kda_oracle_forward_ex(int64_t num_seqs, const int64_t* cu_seqlens, int32_t H, int32_t dk, int32_t dv,
                          int32_t h_begin, int32_t h_end, double scale, const void* q, const void* k,
                          const void* v, int32_t qkv_dtype, const void* alpha, int32_t alpha_dtype,
                          const void* beta, int32_t beta_dtype, const void* s0, int32_t s0_dtype,
                          int64_t ckpt_every, int64_t max_ckpts, double* ckpt, double decay_floor,
                          int32_t alpha_scalar, int32_t fuse_inputs, const void* gate, int32_t gate_dtype,
                          const void* norm_weight, double norm_eps, double* o, double* s_final);

enum { F32 = 0, BF16 = 1 };

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double urand(void) {   /* xorshift64*, uniform in [0, 1) */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (double)((rng_state * 0x2545F4914F6CDD1Dull) >> 11) * 0x1.0p-53;
}

static void* xmalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

/* An array of n values drawn as lo + (hi - lo) u, stored as fp32 or bf16. */
static void* draw(size_t n, int dtype, double lo, double hi) {
    if (dtype == F32) {
        float* p = (float*)xmalloc(n * sizeof(float));
        for (size_t i = 0; i < n; ++i) p[i] = (float)(lo + (hi - lo) * urand());
        return p;
    }
    uint16_t* p = (uint16_t*)xmalloc(n * sizeof(uint16_t));
    for (size_t i = 0; i < n; ++i) {
        const float f = (float)(lo + (hi - lo) * urand());
        uint32_t u;
        memcpy(&u, &f, sizeof u);
        p[i] = (uint16_t)(u >> 16);   /* truncation: any bf16 value is a valid input */
    }
    return p;
}

static double value(const void* p, int dtype, size_t i) {
    if (dtype == F32) return ((const float*)p)[i];
    const uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static int failures = 0;
#define CHECK(cond, ...)                                    \
    do {                                                    \
        if (!(cond)) {                                      \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);                   \
            fputc('\n', stderr);                            \
            ++failures;                                     \
        }                                                   \
    } while (0)

typedef struct {
    int n;
    const int64_t* lens;
    int H, dk, dv, h0, h1, dtype;
    int64_t every, max_ckpts;
    int alpha_scalar, fuse, gated, identity;
    double floor;
} Case;

static void run(const Case* c) {
    int64_t* cu = (int64_t*)xmalloc(sizeof(int64_t) * (size_t)(c->n + 1));
    cu[0] = 0;
    for (int i = 0; i < c->n; ++i) cu[i + 1] = cu[i] + c->lens[i];
    const size_t T = (size_t)cu[c->n], H = (size_t)c->H, dk = (size_t)c->dk, dv = (size_t)c->dv;
    const size_t nh = (size_t)(c->h1 - c->h0), N = (size_t)c->n;
    const size_t na = c->alpha_scalar ? T * H : T * H * dk;
    void* q = draw(T * H * dk, c->dtype, -1.0, 1.0);
    void* k = draw(T * H * dk, c->dtype, -0.3, 0.3);
    void* v = draw(T * H * dv, c->dtype, -1.0, 1.0);
    float* alpha = (float*)draw(na, F32, c->fuse ? -2.0 : 0.5, c->fuse ? 4.0 : 1.0);
    float* beta = (float*)draw(T * H, F32, c->fuse ? -3.0 : 0.0, c->fuse ? 3.0 : 1.0);
    float* s0 = (float*)draw(N * H * dk * dv, F32, -0.05, 0.05);
    void* gate = c->gated ? draw(T * H * dv, c->dtype, -2.0, 2.0) : NULL;
    float* nw = c->gated ? (float*)draw(dv, F32, 0.5, 1.5) : NULL;
    if (c->identity) {
        for (size_t i = 0; i < na; ++i) alpha[i] = 1.f;
        for (size_t i = 0; i < T * H; ++i) beta[i] = 0.f;
    }
    double* o = (double*)xmalloc(sizeof(double) * T * nh * dv);
    double* sf = (double*)xmalloc(sizeof(double) * N * nh * dk * dv);
    const size_t nck = c->every ? N * (size_t)c->max_ckpts * nh * dk * dv : 0;
    double* ck = c->every ? (double*)xmalloc(sizeof(double) * nck) : NULL;
    for (size_t i = 0; i < nck; ++i) ck[i] = NAN;
    const double scale = 0.75;
    const int st = kda_oracle_forward_ex((int64_t)N, cu, c->H, c->dk, c->dv, c->h0, c->h1, scale, q, k, v,
                                         c->dtype, alpha, F32, beta, F32, s0, F32, c->every, c->max_ckpts, ck,
                                         c->floor, c->alpha_scalar, c->fuse, gate, c->dtype, nw, 1e-5, o, sf);
    CHECK(st == 0, "forward returned %d", st);
    size_t bad = 0;
    for (size_t i = 0; i < T * nh * dv; ++i) bad += !isfinite(o[i]);
    for (size_t i = 0; i < N * nh * dk * dv; ++i) bad += !isfinite(sf[i]);
    CHECK(bad == 0, "%zu values are not finite", bad);
    if (c->every) {   /* exactly the reached slots are written */
        const size_t slot = nh * dk * dv;
        for (size_t n = 0; n < N; ++n)
            for (int64_t j = 0; j < c->max_ckpts; ++j) {
                const int reached = (j + 1) * c->every <= c->lens[n];
                const int written = !isnan(ck[(n * (size_t)c->max_ckpts + (size_t)j) * slot]);
                CHECK(reached == written, "checkpoint %zu/%lld written=%d reached=%d", n, (long long)j, written,
                      reached);
            }
    }
    if (c->identity) {   /* S stays S0; o_t = scale q_t S0 */
        double worst = 0.0;
        for (size_t n = 0; n < N; ++n)
            for (size_t hl = 0; hl < nh; ++hl) {
                const size_t h = (size_t)c->h0 + hl;
                const float* S = s0 + (n * H + h) * dk * dv;
                for (size_t i = 0; i < dk * dv; ++i)
                    worst = fmax(worst, fabs(sf[(n * nh + hl) * dk * dv + i] - (double)S[i]));
                for (int64_t t = cu[n]; t < cu[n + 1]; ++t)
                    for (size_t j = 0; j < dv; ++j) {
                        double want = 0.0;
                        for (size_t cc = 0; cc < dk; ++cc)
                            want += value(q, c->dtype, ((size_t)t * H + h) * dk + cc) * (double)S[cc * dv + j];
                        worst = fmax(worst, fabs(o[((size_t)t * nh + hl) * dv + j] - scale * want));
                    }
            }
        CHECK(worst < 1e-12, "identity case off by %g", worst);
    }
    free(cu);
    free(q);
    free(k);
    free(v);
    free(alpha);
    free(beta);
    free(s0);
    free(gate);
    free(nw);
    free(o);
    free(sf);
    free(ck);
}

int main(void) {
    static const int64_t packed[] = {0, 5, 17, 0, 40, 1};
    static const int64_t rows[] = {33, 33, 33};
    static const int64_t one[] = {70};
    const Case cases[] = {
        {6, packed, 3, 16, 8, 0, 3, BF16, 0, 0, 0, 0, 0, 0, 0.0},
        {6, packed, 3, 16, 8, 1, 3, F32, 8, 4, 0, 0, 0, 0, 0.0},        /* head subset, checkpoints */
        {3, rows, 2, 8, 16, 0, 2, BF16, 16, 1, 1, 1, 1, 0, 0.6},        /* scalar decay, fused, gated */
        {3, rows, 2, 8, 16, 0, 2, F32, 0, 0, 0, 1, 1, 0, 0.0},          /* fused, gated, no weight floor */
        {1, one, 1, 4, 4, 0, 1, F32, 32, 2, 0, 0, 0, 0, 0.0},           /* slots run out before the end */
        {6, packed, 2, 8, 8, 0, 2, F32, 0, 0, 0, 0, 0, 1, 0.0},         /* identity closed form */
        {3, rows, 2, 8, 16, 1, 2, BF16, 0, 0, 1, 0, 0, 1, 0.0},         /* identity, scalar decay */
    };
    for (size_t i = 0; i < sizeof cases / sizeof cases[0]; ++i) run(&cases[i]);

    /* argument errors: -1, nothing written */
    const int64_t cu_ok[3] = {0, 2, 4}, cu_down[3] = {0, 3, 2};
    float buf[64] = {0};
    double out[64];
    CHECK(kda_oracle_forward_ex(-1, cu_ok, 1, 4, 4, 0, 1, 1.0, buf, buf, buf, F32, buf, F32, buf, F32, NULL, F32, 0,
                                0, NULL, 0.0, 0, 0, NULL, F32, NULL, 0.0, out, out) == -1, "num_seqs < 0");
    CHECK(kda_oracle_forward_ex(2, cu_down, 1, 4, 4, 0, 1, 1.0, buf, buf, buf, F32, buf, F32, buf, F32, NULL, F32, 0,
                                0, NULL, 0.0, 0, 0, NULL, F32, NULL, 0.0, out, out) == -1, "decreasing cu");
    CHECK(kda_oracle_forward_ex(2, cu_ok, 1, 4, 4, 1, 1, 1.0, buf, buf, buf, F32, buf, F32, buf, F32, NULL, F32, 0,
                                0, NULL, 0.0, 0, 0, NULL, F32, NULL, 0.0, out, out) == -1, "empty head range");
    CHECK(kda_oracle_forward_ex(2, cu_ok, 1, 4, 4, 0, 1, 1.0, buf, buf, buf, 7, buf, F32, buf, F32, NULL, F32, 0,
                                0, NULL, 0.0, 0, 0, NULL, F32, NULL, 0.0, out, out) == -1, "bad dtype");
    CHECK(kda_oracle_forward_ex(2, cu_ok, 1, 4, 4, 0, 1, 1.0, buf, buf, buf, F32, buf, F32, buf, F32, NULL, F32, 4,
                                2, NULL, 0.0, 0, 0, NULL, F32, NULL, 0.0, out, out) == -1, "checkpoints without array");
    if (failures) return 1;
    puts("oracle sanitizer run: ok");
    return 0;
}
