/*
 * kda_oracle.c -- plain fp64 CPU reference of the Kimi Delta Attention (KDA)
 * recurrence.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * benchmark's CPU-baseline leg load it; the library path never does.  It
 * shares no source, header or table with the HIP implementation.
 *
 * What it computes, for every (sequence, head) independently, token by token,
 * with a state S of dk rows (key channels) by dv columns (value channels):
 *
 *   1. decay   S[c][j] *= alpha_t[c]                 for every key channel c
 *   2. recall  r[j]     = sum_c k_t[c] * S[c][j]      on the decayed state
 *   3. correct S[c][j] += beta_t * k_t[c] * (v_t[j] - r[j])
 *   4. read    o_t[j]   = scale * sum_c q_t[c] * S[c][j]   on the updated state
 *
 * Sources (the fact each step follows):
 *  - "Kimi K3 architecture: KDA, MLA and MoE", section "KDA is a writable
 *    state, not a smaller KV cache": the delta rule measures what the state
 *    already holds for a key and writes the correction towards the new value;
 *    the decay gate is per channel, so channels fade at different rates.
 *  - "Kimi K3 Architecture Teardown", section "Hybrid Attention for 1M Tokens"
 *    and Visual 5 ("One KDA step"): per token the state is decayed in every
 *    channel, then a beta-scaled share of what is stored under the key is
 *    erased, then the new key-value pair is written scaled by beta; the state
 *    has a fixed size.
 *  - "Kimi K3 Architecture: KDA, MoE, and Attention", section "Memory as a
 *    First-Class Problem: Kimi Delta Attention": alpha is a channel-wise decay,
 *    beta is one scalar used both to erase and to write, and the output is the
 *    query read from the updated state.
 * Readings where the pages are silent or disagree: erase and write are one
 * correction computed from the decayed state (steps 2-3); the read happens
 * after the correction; alpha scales rows (key channels); scale defaults to 1;
 * no decay floor unless one is asked for; inputs are taken exactly as stored
 * (bf16 or fp32 upcast to fp64).  kda_oracle_forward_ex adds the options
 * documented above it; kda_oracle_forward is the plain recurrence.
 *
 * Layouts (row-major, token-major): q,k [Ttot][H][dk], v [Ttot][H][dv],
 * alpha [Ttot][H][dk], beta [Ttot][H], S0 [N][H][dk][dv].  Sequence n covers
 * tokens [cu[n], cu[n+1]) of the packed token axis.  Only heads
 * [h_begin, h_end) are computed; outputs hold those heads only:
 * o [Ttot][nh][dv] and s_final [N][nh][dk][dv] (fp64), nh = h_end - h_begin.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { KDA_ORACLE_F32 = 0, KDA_ORACLE_BF16 = 1, KDA_ORACLE_F64 = 2 };

/* Read element i of an array stored as fp32, bf16 (raw 16-bit pattern) or fp64. */
static double load_elem(const void* p, int dtype, int64_t i)
{
    if (dtype == KDA_ORACLE_F32) return (double)((const float*)p)[i];
    if (dtype == KDA_ORACLE_BF16) {
        uint32_t bits = (uint32_t)((const uint16_t*)p)[i] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return ((const double*)p)[i];
}

static int valid_dtype(int d) { return d == KDA_ORACLE_F32 || d == KDA_ORACLE_BF16 || d == KDA_ORACLE_F64; }

/* Options beyond the plain recurrence (all off when zero / NULL).
 *
 *  ckpt_every, max_ckpts, ckpt: state checkpoints at prefix boundaries
 *    ("Kimi K3 architecture: KDA, MLA and MoE", section "Serving K3 means
 *    managing two cache lifecycles": the fixed-size state is checkpointed at
 *    selected prefix boundaries; "Kimi K3 Architecture Teardown", section
 *    "Scale: Total vs Active Parameters and Serving Economics": prefill
 *    resumes from the checkpoint).  Checkpoint j of sequence n is the state
 *    after the first (j+1)*ckpt_every tokens of the sequence, for j < max_ckpts
 *    while the sequence is that long: ckpt [N][max_ckpts][nh][dk][dv] fp64;
 *    slots that are not reached keep their contents.
 *  decay_floor: alpha below it is raised to it (a floor on the decay, "Kimi
 *    K3 Architecture Teardown", section "Hybrid Attention for 1M Tokens").
 *  alpha_scalar: alpha holds one value per (token, head), [Ttot][H], used for
 *    every key channel (the scalar gate of Gated DeltaNet that KDA refines,
 *    "Kimi K3 architecture: KDA, MLA and MoE", section "KDA is a writable
 *    state, not a smaller KV cache").
 *  fuse_inputs: the layer's neighbours of the token mixer ("Kimi K3
 *    Architecture Teardown", Visual 1, the KDA inset): q and k are
 *    L2-normalised per (token, head) as x / max(|x|, 1e-12); alpha and beta are
 *    logits and pass through a sigmoid 1 / (1 + e^-x) first; the floor, if
 *    any, applies after the sigmoid.
 *  gate (+ gate_dtype), norm_weight, norm_eps: the output side of the same
 *    inset: o_t is normalised over its dv values as o / sqrt(mean(o^2) + eps),
 *    scaled by norm_weight[j] (NULL: 1) and multiplied by sigmoid(gate_t[j]);
 *    gate is [Ttot][H][dv].
 */
static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* Returns 0 on success, -1 on a bad argument, -2 if memory ran out. */
int kda_oracle_forward_ex(int64_t num_seqs, const int64_t* cu_seqlens,
                          int32_t H, int32_t dk, int32_t dv,
                          int32_t h_begin, int32_t h_end, double scale,
                          const void* q, const void* k, const void* v, int32_t qkv_dtype,
                          const void* alpha, int32_t alpha_dtype,
                          const void* beta, int32_t beta_dtype,
                          const void* s0, int32_t s0_dtype,
                          int64_t ckpt_every, int64_t max_ckpts, double* ckpt,
                          double decay_floor, int32_t alpha_scalar, int32_t fuse_inputs,
                          const void* gate, int32_t gate_dtype, const void* norm_weight, double norm_eps,
                          double* o, double* s_final)
{
    if (num_seqs < 0 || !cu_seqlens || H <= 0 || dk <= 0 || dv <= 0) return -1;
    if (h_begin < 0 || h_end > H || h_begin >= h_end) return -1;
    if (!q || !k || !v || !alpha || !beta || !o) return -1;
    if (!valid_dtype(qkv_dtype) || !valid_dtype(alpha_dtype) || !valid_dtype(beta_dtype)) return -1;
    if (s0 && !valid_dtype(s0_dtype)) return -1;
    if (gate && !valid_dtype(gate_dtype)) return -1;
    if (ckpt_every < 0 || (ckpt_every > 0 && (max_ckpts < 1 || !ckpt))) return -1;
    for (int64_t n = 0; n < num_seqs; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;

    const int64_t nh = h_end - h_begin;
    const int64_t units = num_seqs * nh;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < units; ++u) {
        const int64_t n = u / nh;
        const int64_t hl = u % nh;          /* head index within the output */
        const int64_t h = h_begin + hl;     /* head index within the inputs */
        double* S = (double*)malloc(sizeof(double) * (size_t)dk * (size_t)dv);
        double* r = (double*)malloc(sizeof(double) * (size_t)dv);
        double* qt = (double*)malloc(sizeof(double) * (size_t)dk);
        double* kt = (double*)malloc(sizeof(double) * (size_t)dk);
        double* at = (double*)malloc(sizeof(double) * (size_t)dk);
        if (!S || !r || !qt || !kt || !at) {
            free(S);
            free(r);
            free(qt);
            free(kt);
            free(at);
#pragma omp atomic write
            failed = 1;
            continue;
        }
        /* initial state: S0 of this (sequence, head), or zeros */
        for (int64_t c = 0; c < dk; ++c)
            for (int64_t j = 0; j < dv; ++j)
                S[c * dv + j] = s0 ? load_elem(s0, s0_dtype, ((n * H + h) * dk + c) * dv + j) : 0.0;

        for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
            const int64_t qk_base = (t * H + h) * dk;
            const int64_t v_base = (t * H + h) * dv;
            double b = load_elem(beta, beta_dtype, t * H + h);

            /* the token's q, k and per-channel alpha, as the recurrence uses them */
            double nq = 0.0, nk = 0.0;
            for (int64_t c = 0; c < dk; ++c) {
                qt[c] = load_elem(q, qkv_dtype, qk_base + c);
                kt[c] = load_elem(k, qkv_dtype, qk_base + c);
                at[c] = alpha_scalar ? load_elem(alpha, alpha_dtype, t * H + h)
                                     : load_elem(alpha, alpha_dtype, qk_base + c);
                nq += qt[c] * qt[c];
                nk += kt[c] * kt[c];
            }
            if (fuse_inputs) {
                const double iq = 1.0 / fmax(sqrt(nq), 1e-12), ik = 1.0 / fmax(sqrt(nk), 1e-12);
                for (int64_t c = 0; c < dk; ++c) {
                    qt[c] *= iq;
                    kt[c] *= ik;
                    at[c] = sigmoid(at[c]);
                }
                b = sigmoid(b);
            }
            if (decay_floor > 0.0)
                for (int64_t c = 0; c < dk; ++c) at[c] = fmax(at[c], decay_floor);

            /* 1. decay every key channel (row) by its own alpha */
            for (int64_t c = 0; c < dk; ++c)
                for (int64_t j = 0; j < dv; ++j) S[c * dv + j] *= at[c];
            /* 2. recall: what the decayed state associates with k_t */
            for (int64_t j = 0; j < dv; ++j) r[j] = 0.0;
            for (int64_t c = 0; c < dk; ++c)
                for (int64_t j = 0; j < dv; ++j) r[j] += kt[c] * S[c * dv + j];
            /* 3. erase and write as one correction scaled by the same beta */
            for (int64_t c = 0; c < dk; ++c)
                for (int64_t j = 0; j < dv; ++j)
                    S[c * dv + j] += b * kt[c] * (load_elem(v, qkv_dtype, v_base + j) - r[j]);
            /* 4. read the updated state with the query */
            double* ot = o + (t * nh + hl) * dv;
            for (int64_t j = 0; j < dv; ++j) ot[j] = 0.0;
            for (int64_t c = 0; c < dk; ++c)
                for (int64_t j = 0; j < dv; ++j) ot[j] += qt[c] * S[c * dv + j];
            for (int64_t j = 0; j < dv; ++j) ot[j] *= scale;
            /* output side: norm over dv, weight, sigmoid gate */
            if (gate) {
                double ms = 0.0;
                for (int64_t j = 0; j < dv; ++j) ms += ot[j] * ot[j];
                const double inv = 1.0 / sqrt(ms / (double)dv + norm_eps);
                for (int64_t j = 0; j < dv; ++j) {
                    const double w = norm_weight ? (double)((const float*)norm_weight)[j] : 1.0;
                    ot[j] = ot[j] * inv * w * sigmoid(load_elem(gate, gate_dtype, v_base + j));
                }
            }
            /* checkpoint after (j + 1) * ckpt_every tokens of the sequence */
            const int64_t done = t - cu_seqlens[n] + 1;
            if (ckpt_every > 0 && done % ckpt_every == 0 && done / ckpt_every <= max_ckpts)
                memcpy(ckpt + (((size_t)n * (size_t)max_ckpts + (size_t)(done / ckpt_every - 1)) * (size_t)nh +
                               (size_t)hl) * (size_t)dk * (size_t)dv,
                       S, sizeof(double) * (size_t)dk * (size_t)dv);
        }
        if (s_final)
            memcpy(s_final + (size_t)u * (size_t)dk * (size_t)dv, S,
                   sizeof(double) * (size_t)dk * (size_t)dv);
        free(S);
        free(r);
        free(qt);
        free(kt);
        free(at);
    }
    return failed ? -2 : 0;
}

/* The plain recurrence: every option off. */
int kda_oracle_forward(int64_t num_seqs, const int64_t* cu_seqlens,
                       int32_t H, int32_t dk, int32_t dv,
                       int32_t h_begin, int32_t h_end, double scale,
                       const void* q, const void* k, const void* v, int32_t qkv_dtype,
                       const void* alpha, int32_t alpha_dtype,
                       const void* beta, int32_t beta_dtype,
                       const void* s0, int32_t s0_dtype,
                       double* o, double* s_final)
{
    return kda_oracle_forward_ex(num_seqs, cu_seqlens, H, dk, dv, h_begin, h_end, scale, q, k, v, qkv_dtype,
                                 alpha, alpha_dtype, beta, beta_dtype, s0, s0_dtype, 0, 0, NULL, 0.0, 0, 0,
                                 NULL, 0, NULL, 0.0, o, s_final);
}

/* Number of threads the parallel loop above runs with. */
int kda_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
