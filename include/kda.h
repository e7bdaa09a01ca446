/*
 * kda.h -- C ABI of libkda.so, the MI355X (gfx950) implementation of the
 * Kimi Delta Attention (KDA) token mixer.
 *
 * The operation.  Each (sequence, head) carries a fixed-size fp32 state S of
 * dk rows (key channels) by dv columns (value channels).  For every token t:
 *   S'  = diag(alpha_t) S            decay each key channel by its own gate
 *   r   = S'^T k_t                   what the decayed state holds for k_t
 *   S   = S' + beta_t k_t (v_t - r)^T   erase and write with the same beta
 *   o_t = scale * S^T q_t            read the updated state with the query
 * Sources: "Kimi K3 architecture: KDA, MLA and MoE", section "KDA is a
 * writable state, not a smaller KV cache" (delta-rule correction, per-channel
 * decay, queries read the current matrix); "Kimi K3 Architecture Teardown",
 * section "Hybrid Attention for 1M Tokens" and Visual 5 (decay, erase, write;
 * fixed-size state); "Kimi K3 Architecture: KDA, MoE, and Attention", section
 * "Memory as a First-Class Problem: Kimi Delta Attention" (channel-wise
 * alpha, one scalar beta for erase and write, output read from the updated
 * state).  Prefix-cache resume (initial/final state) follows "Kimi K3
 * architecture: KDA, MLA and MoE", section "Serving K3 means managing two
 * cache lifecycles", and "Kimi K3 Architecture Teardown", section "Scale".
 *
 * Conventions shared by every entry point:
 *  - Every tensor argument is a DEVICE pointer owned by the caller (the one
 *    host array is kda_chunk_fwd_windowed(_ex)'s copy of cu_seqlens).  The
 *    library allocates no device memory, keeps no pointer after returning and
 *    takes scratch only through the caller's workspace; the one exception is
 *    kda_chunk_fwd_noalloc, whose scratch is a fixed device array the
 *    library holds (see there).
 *  - Tensors are dense, row-major, last index fastest, with the shapes given
 *    below.  q, k, v, o, alpha and states must be 16-byte aligned; beta and
 *    cu_seqlens 4-byte aligned; workspace 256-byte aligned.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream) and never synchronise the host.
 *  - Arguments are validated before anything is launched: a call that
 *    returns an error has touched no output.  KDA_ERR_HIP reports a launch
 *    failure (the HIP error is consumed).  No C++ exception crosses the ABI.
 *  - Inputs must be finite.  The only mutable global state is a per-device
 *    cache of the compute-unit count and of kda_chunk_fwd_noalloc's scratch
 *    address, each filled once; calls on different streams may run
 *    concurrently if their outputs and workspaces do not overlap (never two
 *    kda_chunk_fwd_noalloc calls on one device).
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage type of q, k, v and o.  alpha, beta and the states are always fp32. */
typedef enum { KDA_DTYPE_F32 = 0, KDA_DTYPE_BF16 = 1 } kda_dtype_t;

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size or shape    */
    KDA_ERR_UNSUPPORTED = 2, /* head dim, chunk size or dtype not built, or a */
                             /* call beyond one dispatch (2^32 work-items)     */
    KDA_ERR_WORKSPACE = 3,   /* workspace missing, too small or misaligned    */
    KDA_ERR_HIP = 4,         /* a HIP launch or runtime call failed           */
    KDA_ERR_RANGE = 5        /* the result is not finite (kda_chunk_fwd_status) */
} kda_status_t;

/* Shape of one chunked-prefill call.  All fields are plain int32/int64/float
 * so the struct layout is fixed: {int32 batch; [pad]; int64 seqlen; int32
 * num_seqs, num_heads, head_dim_k, head_dim_v, chunk_size; float scale;
 * int32 qkv_dtype, o_dtype}. */
typedef struct {
    int32_t batch;      /* B rows; must be 1 when cu_seqlens is given          */
    int64_t seqlen;     /* T tokens per row, or total packed tokens (>= 0)      */
    int32_t num_seqs;   /* N: == batch without cu_seqlens, else len(cu)-1 >= 1  */
    int32_t num_heads;  /* H >= 1                                               */
    int32_t head_dim_k; /* dk in {16, 32, 64, 128}                              */
    int32_t head_dim_v; /* dv in {16, 32, 64, 128}                              */
    int32_t chunk_size; /* C in {16, 32, 64}; the result does not depend on it  */
                        /* beyond rounding.  fp32 inputs with dk = 128 run with */
                        /* chunks of at most 32 (on-chip memory).               */
    float scale;        /* query scale; 1.0 reproduces the pages' read          */
    int32_t qkv_dtype;  /* kda_dtype_t of q, k, v                               */
    int32_t o_dtype;    /* kda_dtype_t of o (fp32, or bf16 rounded to nearest   */
                        /* even from the fp32 result)                           */
} kda_chunk_params_t;

/* Human-readable name of a status code (static string, never NULL). */
const char* kda_status_string(kda_status_t status);

/* Bytes of workspace kda_chunk_fwd needs for `params` (written to *bytes).
 * The size depends only on the shape, not on the cu_seqlens values: it covers
 * the worst case ceil(T / C) + N chunks per head for packed input.
 * Errors: KDA_ERR_INVALID_ARG / KDA_ERR_UNSUPPORTED as for kda_chunk_fwd. */
kda_status_t kda_chunk_fwd_workspace_size(const kda_chunk_params_t* params, size_t* bytes);

/* How kda_chunk_fwd runs a call of `params` on the current device, for tuning
 * and diagnostics (the results do not depend on it beyond rounding).
 * `packed` != 0 describes a call with cu_seqlens (then batch must be 1).
 * Without a usable device the plan assumes 256 compute units.  Fields:
 *   chunk_size    the chunk length used (fp32 inputs with dk = 128: <= 32)
 *   whole_rows    1 when each inter-chunk workgroup carries whole state rows
 *                 of one (sequence, head), 0 when it carries 16 columns
 *   range_chunks  L > 0 when the inter-chunk pass cuts every sequence into
 *                 ranges of L chunks that run side by side: the affine map
 *                 S -> A S + B of each range is formed first, a scan of those
 *                 maps gives every range its start state, then the ranges
 *                 run.  0 when one workgroup walks each whole sequence.
 *   max_ranges    ranges per head held in the workspace (0 without ranges)
 * Errors: KDA_ERR_INVALID_ARG (NULL plan, packed with batch != 1) and the
 * shape errors of kda_chunk_fwd. */
typedef struct {
    int32_t chunk_size;
    int32_t whole_rows;
    int32_t range_chunks;
    int32_t max_ranges;
} kda_chunk_plan_t;

kda_status_t kda_chunk_fwd_plan(const kda_chunk_params_t* params, int32_t packed, kda_chunk_plan_t* plan);

/* Chunked prefill: run the recurrence over every token of every sequence.
 *
 * Layout (D = params->qkv_dtype, B = batch, T = seqlen, H = num_heads):
 *   q, k        [B, T, H, dk]  D
 *   v           [B, T, H, dv]  D
 *   alpha       [B, T, H, dk]  fp32, per-key-channel decay in [0, 1]
 *   beta        [B, T, H]      fp32, one update strength per token and head
 *   initial_state [N, H, dk, dv] fp32, or NULL for zeros
 *   cu_seqlens  [N + 1] int32 on the device, or NULL.  NULL: each of the B rows
 *               is one sequence (N == B).  Non-NULL: B == 1 and sequence n is
 *               tokens [cu[n], cu[n+1]) of the row; requires cu[0] == 0,
 *               non-decreasing, cu[N] == T.  The host does not read it (that
 *               would need a device-to-host copy); the first kernel of the call
 *               checks it on the device, and a call that breaks it reads and
 *               writes no token (its o and final_state must not be used) and
 *               kda_chunk_fwd_status then reports KDA_ERR_INVALID_ARG.
 *               Empty sequences are allowed: their final state is the initial one.
 *   o           [B, T, H, dv]  params->o_dtype (written for every token of every
 *               sequence)
 *   final_state [N, H, dk, dv] fp32, or NULL (not written).  May alias
 *               initial_state exactly (in-place resume).
 *   workspace   device scratch of at least kda_chunk_fwd_workspace_size bytes.
 * The chunk form evaluates the same recurrence with intra-chunk products on
 * the matrix cores; results agree with the token-by-token recurrence up to
 * rounding.  fp32 inputs: fp32 arithmetic throughout.  bf16 inputs: matrix-
 * core operands and chunk intermediates in fp16 (11-bit mantissa, largest
 * value 65504) with fp32 accumulation and an fp32 state.  Range contract: a
 * call whose intermediates leave that range (in practice |v| or the state of
 * order 1e4 and above, or keys far from unit norm) does not return a silent
 * result: every value the call writes to o, final_state and checkpoints is
 * checked on the device, and kda_chunk_fwd_status then reports
 * KDA_ERR_RANGE; the outputs of such a call hold inf or NaN and must not be
 * used.  Results that kda_chunk_fwd_status accepts are finite. */
kda_status_t kda_chunk_fwd(const kda_chunk_params_t* params,
                           const void* q, const void* k, const void* v,
                           const float* alpha, const float* beta,
                           const float* initial_state, const int32_t* cu_seqlens,
                           void* o, float* final_state,
                           void* workspace, size_t workspace_bytes,
                           void* stream);

/* kda_chunk_fwd without a workspace argument, for callers that cannot
 * allocate device memory: code running under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It allocates nothing and calls no
 * allocating routine; its scratch is a device array of
 * KDA_NOALLOC_SCRATCH_BYTES (64 MiB) that the library holds on every device it
 * runs on until the process ends.
 *  - Limit: a call whose workspace (kda_chunk_fwd_workspace_size) exceeds
 *    KDA_NOALLOC_SCRATCH_BYTES returns KDA_ERR_WORKSPACE before anything is
 *    launched; at dk = dv = 128, chunk 64, bf16 that is about 900 (chunk,
 *    head) pairs, e.g. 57,000 token-heads of one sequence.
 *  - Every call on a device shares that device's array: calls that may
 *    overlap on one device (on different streams, or from host threads that
 *    do not order them) race and must not be issued.  Calls ordered on one
 *    stream are safe; no part of the array needs to start at zero.
 *  - The first call on a device looks up the array's device address
 *    (hipGetSymbolAddress) with that device current; KDA_ERR_HIP if it fails.
 * Otherwise arguments, validation and results are those of kda_chunk_fwd:
 * the same kernels run on the same layout, so the outputs are identical. */
#define KDA_NOALLOC_SCRATCH_BYTES (64ull << 20)
kda_status_t kda_chunk_fwd_noalloc(const kda_chunk_params_t* params,
                                   const void* q, const void* k, const void* v,
                                   const float* alpha, const float* beta,
                                   const float* initial_state, const int32_t* cu_seqlens,
                                   void* o, float* final_state, void* stream);

/* kda_chunk_fwd in bounded memory, for callers that cannot hold the whole
 * call's workspace: the per-(chunk, head) blocks take about 73 KiB each at
 * dk = dv = 128, chunk 64, bf16, so a pack of 1M tokens over 16 heads would
 * need 18 GB at once.  The operation and its results are those of
 * kda_chunk_fwd (same sources); the work is split into calls that each fit
 * `workspace_bytes`, run in order on `stream`:
 *  - whole sequences (batch rows) are grouped while the group's
 *    kda_chunk_fwd_workspace_size fits;
 *  - a sequence that does not fit alone runs in windows of whole chunks; each
 *    window starts from the state the previous one left in final_state (the
 *    prefix-cache resume of "Kimi K3 architecture: KDA, MLA and MoE", section
 *    "Serving K3 means managing two cache lifecycles").
 * Results agree with kda_chunk_fwd up to rounding (the windows end on chunk
 * boundaries; the inter-chunk pass may be organised differently).
 * Arguments: those of kda_chunk_fwd, plus `cu_seqlens_host`, a HOST copy of
 * cu_seqlens (the one host pointer of this ABI; NULL exactly when
 * cu_seqlens is NULL), which the call reads to plan the windows and checks
 * (cu[0] == 0, non-decreasing, cu[N] == T).  final_state is required (it
 * carries the state between windows) and may alias initial_state exactly.
 * kda_chunk_fwd_status(workspace) afterwards reports a range error of any of
 * the calls.  The host reads nothing from the device.
 * Errors (before anything is launched): KDA_ERR_INVALID_ARG (a NULL
 * final_state, cu_seqlens without its host copy or the reverse, a bad host
 * cu_seqlens, the argument errors of kda_chunk_fwd), KDA_ERR_WORKSPACE (NULL
 * or misaligned workspace, or `workspace_bytes` below what one chunk of one
 * sequence needs: kda_chunk_fwd_workspace_size of one sequence of `chunk`
 * tokens), the shape errors of kda_chunk_fwd; KDA_ERR_HIP from a launch. */
kda_status_t kda_chunk_fwd_windowed(const kda_chunk_params_t* params,
                                    const void* q, const void* k, const void* v,
                                    const float* alpha, const float* beta,
                                    const float* initial_state, const int32_t* cu_seqlens,
                                    const int32_t* cu_seqlens_host,
                                    void* o, float* final_state,
                                    void* workspace, size_t workspace_bytes,
                                    void* stream);

/* Device-side status of the last kda_chunk_fwd / kda_chunk_fwd_ex /
 * kda_chunk_fwd_windowed(_ex) call (or _intra + _inter pair) made with
 * `workspace`: KDA_ERR_INVALID_ARG when its cu_seqlens broke the layout that
 * kda_chunk_fwd requires; else KDA_OK when every value it wrote to o,
 * final_state and checkpoints is finite, KDA_ERR_RANGE when one is not (see
 * the range contract above).  The intra-chunk half writes the status words
 * (the first 256 bytes of the workspace) and the inter-chunk half may set the
 * range word, so it is read after both on the same stream.  This call copies
 * 12 bytes to the host and SYNCHRONISES `stream`.  Errors:
 * KDA_ERR_INVALID_ARG (NULL or misaligned workspace), KDA_ERR_HIP. */
kda_status_t kda_chunk_fwd_status(const void* workspace, void* stream);

/* The two halves of kda_chunk_fwd, for callers that schedule them separately
 * (for example to time them, or to overlap the intra-chunk half of one call
 * with other work).  Same arguments and validation as kda_chunk_fwd.
 * kda_chunk_fwd_intra reads q, k, v, alpha, beta (and cu_seqlens) and fills
 * the workspace with each chunk's intra-chunk factors; kda_chunk_fwd_inter
 * then reads only the workspace, initial_state and cu_seqlens and writes o and
 * final_state.  Calling _intra then _inter on one stream with the same
 * arguments and an untouched workspace is exactly kda_chunk_fwd. */
kda_status_t kda_chunk_fwd_intra(const kda_chunk_params_t* params,
                                 const void* q, const void* k, const void* v,
                                 const float* alpha, const float* beta,
                                 const float* initial_state, const int32_t* cu_seqlens,
                                 void* o, float* final_state,
                                 void* workspace, size_t workspace_bytes,
                                 void* stream);
kda_status_t kda_chunk_fwd_inter(const kda_chunk_params_t* params,
                                 const void* q, const void* k, const void* v,
                                 const float* alpha, const float* beta,
                                 const float* initial_state, const int32_t* cu_seqlens,
                                 void* o, float* final_state,
                                 void* workspace, size_t workspace_bytes,
                                 void* stream);

/* Options of kda_chunk_fwd_ex.  A zero-filled struct is exactly kda_chunk_fwd.
 * Option values are validated before anything is launched. */
typedef struct {
    /* State checkpoints at prefix boundaries.  The serving side keeps the
     * fixed-size recurrent state at selected prefix boundaries so that a
     * repeated prompt resumes prefill there ("Kimi K3 architecture: KDA, MLA
     * and MoE", section "Serving K3 means managing two cache lifecycles";
     * "Kimi K3 Architecture Teardown", section "Scale: Total vs Active
     * Parameters and Serving Economics").  When ckpt_every > 0, checkpoint j
     * of sequence n is the state after the first (j + 1) * ckpt_every tokens
     * of that sequence, written to checkpoints [N, max_ckpts, H, dk, dv] fp32
     * (16-byte aligned, not overlapping the states) for every j < max_ckpts
     * with (j + 1) * ckpt_every <= the length of sequence n; other slots are
     * left untouched.  ckpt_every must be a multiple of 64 and max_ckpts >= 1.
     * Fed back as initial_state, checkpoint j resumes the sequence at token
     * (j + 1) * ckpt_every. */
    float* checkpoints;
    int64_t ckpt_every;
    int32_t max_ckpts;
    /* Floored decay: alpha values below decay_floor (>= 0) are raised to it
     * (0: no floor); K3 floors its decay ("Kimi K3 Architecture Teardown",
     * section "Hybrid Attention for 1M Tokens").  Applied after the sigmoid
     * of fuse_inputs. */
    float decay_floor;
    /* 0: alpha is per key channel [B, T, H, dk]; 1: one decay per token and
     * head, alpha [B, T, H], for every channel (the scalar gate of Gated
     * DeltaNet that KDA refines per channel, "Kimi K3 architecture: KDA, MLA
     * and MoE", section "KDA is a writable state, not a smaller KV cache");
     * alpha is then 4-byte aligned. */
    int32_t alpha_mode;
    /* 1: the neighbours of the token mixer run inside the kernels ("Kimi K3
     * Architecture Teardown", Visual 1, the KDA inset): q and k are
     * L2-normalised per (token, head) as x / max(|x|, 1e-12), and alpha, beta
     * are logits passed through 1 / (1 + e^-x). */
    int32_t fuse_inputs;
    /* Output norm and gate of the same inset: NULL, or gate logits
     * [B, T, H, dv] (qkv dtype); then o = o / sqrt(mean_j(o_j^2) + norm_eps)
     * * norm_weight * sigmoid(gate), the mean over the dv values of the
     * (token, head), norm_weight [dv] fp32 or NULL for ones. */
    const void* gate;
    const float* norm_weight;
    float norm_eps;
} kda_chunk_options_t;

/* Workspace bytes kda_chunk_fwd_ex needs for `params` with `options` (NULL:
 * as kda_chunk_fwd_workspace_size).  A gate adds scratch for un-normalised
 * fp32 outputs and per-slice sums of squares (about (dv + dv/16) * 4 bytes
 * per token and head) when the shape takes one-slice inter-chunk workgroups
 * (kda_chunk_fwd_plan: whole_rows == 0, i.e. fewer (sequence, head) pairs
 * than compute units and no chunk ranges): the norm is then finished by a
 * small epilogue kernel.  Otherwise the inter-chunk pass finishes it and no
 * scratch is quoted. */
kda_status_t kda_chunk_fwd_ex_workspace_size(const kda_chunk_params_t* params, const kda_chunk_options_t* options,
                                             size_t* bytes);

/* kda_chunk_fwd with the options above (NULL options = kda_chunk_fwd).  The
 * workspace must hold kda_chunk_fwd_ex_workspace_size bytes for the same
 * options.  Errors as kda_chunk_fwd, plus KDA_ERR_INVALID_ARG for bad option
 * values (negative or NaN floor or eps, a norm weight without a gate,
 * misaligned option pointers, bad checkpoint layout). */
kda_status_t kda_chunk_fwd_ex(const kda_chunk_params_t* params, const kda_chunk_options_t* options,
                              const void* q, const void* k, const void* v,
                              const float* alpha, const float* beta,
                              const float* initial_state, const int32_t* cu_seqlens,
                              void* o, float* final_state,
                              void* workspace, size_t workspace_bytes,
                              void* stream);

/* kda_chunk_fwd_windowed with the options of kda_chunk_fwd_ex (NULL options =
 * kda_chunk_fwd_windowed): the gated, fused-input layer of "Kimi K3
 * Architecture Teardown" (Visual 1, the KDA inset) in bounded memory.  Each
 * call of the split takes the rows of gate and alpha of its tokens; a
 * call fits when the workspace of its own shape and layout (at most
 * kda_chunk_fwd_ex_workspace_size of that shape, the gate's epilogue scratch
 * included where the shape takes it) is within workspace_bytes.  With checkpoints, a
 * sequence that does not fit alone runs in windows of whole checkpoint
 * intervals (multiples of ckpt_every tokens), so every window writes its
 * checkpoints into its sequence's slots, as the one-piece call does; the
 * workspace must then hold a call of one sequence of ckpt_every tokens (else
 * KDA_ERR_WORKSPACE).  Option values are checked on the whole call before
 * anything is launched; errors as kda_chunk_fwd_windowed plus those of
 * kda_chunk_fwd_ex's options. */
kda_status_t kda_chunk_fwd_windowed_ex(const kda_chunk_params_t* params, const kda_chunk_options_t* options,
                                       const void* q, const void* k, const void* v,
                                       const float* alpha, const float* beta,
                                       const float* initial_state, const int32_t* cu_seqlens,
                                       const int32_t* cu_seqlens_host,
                                       void* o, float* final_state,
                                       void* workspace, size_t workspace_bytes,
                                       void* stream);

/* One decode step: every (sequence, head) consumes a single token and its
 * state is updated in place.
 *   q, k   [N, H, dk]  D        v  [N, H, dv]  D      o  [N, H, dv]  o_dtype
 *   alpha  [N, H, dk]  fp32     beta  [N, H]      fp32
 *   state  [N, H, dk, dv] fp32, read and overwritten in place.
 * dk, dv in {16, 32, 64, 128}; num_seqs >= 1; num_heads >= 1.  The step is
 * computed in fp32.  The state is streamed through the GPU once: each element
 * is read once and written once. */
kda_status_t kda_decode_step(int32_t num_seqs, int32_t num_heads,
                             int32_t head_dim_k, int32_t head_dim_v,
                             float scale, int32_t qkv_dtype, int32_t o_dtype,
                             const void* q, const void* k, const void* v,
                             const float* alpha, const float* beta,
                             float* state, void* o, void* stream);

/* Options of kda_decode_step_ex.  A zero-filled struct is exactly
 * kda_decode_step. */
typedef struct {
    /* Paged state pool: NULL, or [N] int32 on the device.  Then `state` is a
     * pool [P, H, dk, dv] fp32 and sequence n reads and updates pool entry
     * state_slots[n] in place (the unified paged pool that holds the KDA
     * states, "Kimi K3 architecture: KDA, MLA and MoE", section "Serving K3
     * means managing two cache lifecycles").  Slots must be distinct within a
     * call (device data, not checked); see pool_entries for their range. */
    const int32_t* state_slots;
    /* Floored decay: alpha values below decay_floor are raised to it (0: no
     * floor), applied after the sigmoid of fuse_inputs. */
    float decay_floor;
    /* 0: alpha [N, H, dk] per key channel; 1: alpha [N, H], one decay per
     * (sequence, head) for every channel (the scalar gate of Gated DeltaNet,
     * "Kimi K3 architecture: KDA, MLA and MoE", section "KDA is a writable
     * state, not a smaller KV cache"). */
    int32_t alpha_mode;
    /* 1: the neighbours of the token mixer run inside the step ("Kimi K3
     * Architecture Teardown", Visual 1, the KDA inset): q and k are
     * L2-normalised as x / max(|x|, 1e-12), alpha and beta are logits passed
     * through 1 / (1 + e^-x). */
    int32_t fuse_inputs;
    /* Output norm and gate of the same inset: NULL, or gate logits [N, H, dv]
     * (qkv dtype); then o = o / sqrt(mean_j(o_j^2) + norm_eps) * norm_weight
     * * sigmoid(gate), the mean over the dv values of the head, norm_weight
     * [dv] fp32 or NULL for ones. */
    const void* gate;
    const float* norm_weight;
    float norm_eps;
    /* P, the entries of the state pool (state_slots given), or 0.  When > 0 a
     * slot outside [0, P) is checked on the device and not used: that
     * sequence's state is not touched and its o is written as NaN (in every
     * head).  0 leaves the slots unchecked (they must then lie in [0, P)). */
    int32_t pool_entries;
} kda_decode_options_t;

/* kda_decode_step with the options above (NULL options = kda_decode_step).
 * Errors as kda_decode_step, plus KDA_ERR_INVALID_ARG for bad option values
 * (a negative or NaN floor or eps, a negative pool_entries, misaligned
 * pointers). */
kda_status_t kda_decode_step_ex(int32_t num_seqs, int32_t num_heads,
                                int32_t head_dim_k, int32_t head_dim_v,
                                float scale, int32_t qkv_dtype, int32_t o_dtype,
                                const kda_decode_options_t* options,
                                const void* q, const void* k, const void* v,
                                const float* alpha, const float* beta,
                                float* state, void* o, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
