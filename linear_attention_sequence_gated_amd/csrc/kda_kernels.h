// kda_kernels.h -- launch interface between the C ABI (kda_api.cpp) and the
// HIP kernels.  Internal to libkda.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const float* beta;
    const float* s0;             // [N, H, dk, dv] or null
    float* s_final;              // [N, H, dk, dv] or null
    const int32_t* cu_seqlens;   // [N + 1] or null (fixed length rows)
    const int32_t* chunk_off;    // [N + 1] chunk index of each sequence (packed input)
    void* o;
    char* ws_chunks;             // per-(chunk, head) blocks
    int32_t* status;             // range status of the call: cleared by the intra-chunk kernel, set to 1 by
                                 // the inter-chunk kernel when a value it writes is not finite
    int64_t T;                   // tokens per row, or total packed tokens
    int32_t N, H, DV;
    int32_t chunks_per_seq;      // fixed length: ceil(T / C)
    float scale;
    int32_t o_f32;               // 1: o is fp32, 0: o is bf16
    float* ckpt;                 // [N, max_ckpts, H, dk, dv] state checkpoints, or null
    int64_t ckpt_every;          // tokens between checkpoints (a multiple of the chunk)
    int32_t max_ckpts;
    float alpha_floor;           // alpha = max(alpha, floor); 0 leaves it as is
    int32_t alpha_scalar;        // alpha [B, T, H]: one decay per token and head
    int32_t fuse_inputs;         // L2 norm of q, k; sigmoid of alpha, beta logits
    const void* gate;            // [B, T, H, dv] output gate logits (q dtype), or null
    const float* norm_w;         // [dv] or null
    float norm_eps;
    int32_t gsl;                 // value slices per slice group (slice_group())
    int32_t gate_split;          // gated output through o_scratch + part_scratch and an epilogue
    int32_t whole_rows;          // plain output from whole-row inter-chunk workgroups
    // Chunk-range scan (few (sequence, head) pairs, long sequences): each
    // sequence's chunks are cut into ranges of range_len chunks (at least one
    // range per sequence, empty or not); a range's map S_end = A S_start + B
    // is formed first, the ranges' start states are then scanned, and the
    // whole-row pass runs every range from its own start state.
    int32_t range_len;           // chunks per range, 0: no ranges
    int32_t ranges_per_seq;      // fixed-length input: max(1, ceil(chunks_per_seq / range_len))
    int32_t max_ranges;          // ranges of the call at most (the range kernels' grid)
    const int32_t* range_off;    // packed input: [N + 1] first range of each sequence
    float* range_ab;             // [ranges, H, dk, dk + dv] fp32: A (dk columns), then B (dv columns)
    float* range_start;          // [ranges, H, dk, dv] fp32: state at the start of each range (first unused)
    // packed input, whole-row pass without ranges: [N] the sequences by
    // decreasing chunk count (workgroup b walks sequence seq_order[b / H]), or null
    const int32_t* seq_order;
    float* o_scratch;            // [B*T*H, dv] un-normalised outputs (split gate)
    float* part_scratch;         // [B*T*H, dv/16] per-slice sums of squares (split gate)
};

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const float* beta;
    float* state;
    void* o;
    int32_t units;               // N * H
    int32_t H;
    float scale;
    int32_t o_f32;               // 1: o is fp32, 0: o is bf16
    const int32_t* slots;        // [N] pool entries of the states, or null (state n * H + h)
    int32_t pool_entries;        // > 0: slots outside [0, pool_entries) are skipped (o = NaN)
    float alpha_floor;           // alpha = max(alpha, floor); 0 leaves it as is
    int32_t alpha_scalar;        // alpha [N, H]
    int32_t fuse_inputs;         // L2 norm of q, k; sigmoid of alpha, beta logits
    const void* gate;            // [N, H, dv] gate logits (q dtype), or null
    const float* norm_w;         // [dv] or null
    float norm_eps;
};

// Status words at the head of the workspace: [0] range status of the call,
// [1] the running range status of a windowed call, [kLayoutWord] 1 when the
// call's cu_seqlens broke its layout.
constexpr int kLayoutWord = 2;
// Chunk offsets of the packed sequences (chunk_off [n + 1]).  With T >= 0 the
// layout of cu first is checked (cu[0] == 0, non-decreasing, cu[n] == T): a
// broken one empties the tables and sets status[kLayoutWord]; T < 0 skips the
// check (offsets the caller has checked).
hipError_t launch_chunk_offsets(const int32_t* cu, int32_t n, int32_t C, int32_t* chunk_off, int64_t T,
                                int32_t* status, hipStream_t s);
// Also the first range of each packed sequence (range_off [n + 1]) for ranges of L chunks.
hipError_t launch_chunk_range_offsets(const int32_t* cu, int32_t n, int32_t C, int32_t L, int32_t* chunk_off,
                                      int32_t* range_off, int64_t T, int32_t* status, hipStream_t s);
// Packed sequences by decreasing chunk count, ties by index (order [n]); more
// than kSeqOrderMax sequences keep their input order.
constexpr int kSeqOrderMax = 4096;
hipError_t launch_seq_order(const int32_t* cu, int32_t n, int32_t C, int32_t* order, hipStream_t s);
// Chunks per range of the chunk-range scan for this call shape, or 0 when the
// scan does not run (it needs dk == dv in {64, 128}, bf16 inputs, 64-token
// chunks, fewer (sequence, head) pairs than CUs and at least three ranges per
// sequence on average).
int range_length(int DK, int DV, int C, bool bf16, int64_t units, int64_t chunks_per_unit);
// Clears the range status word (calls without tokens launch no intra-chunk kernel).
hipError_t launch_clear_status(int32_t* status, hipStream_t s);
// Folds the range status words of the calls that make up a windowed call.
enum { kFoldClear = 0, kFoldOr = 1, kFoldBack = 2 };
hipError_t launch_fold_status(int32_t* status, int mode, hipStream_t s);
// C is the requested chunk size; the chunk the kernels use is
// effective_chunk(DK, C, bf16) (fp32 operands with dk = 128 use at most 32).
int effective_chunk(int DK, int C, bool bf16);
hipError_t launch_intra(const PrefillArgs& a, int DK, int C, bool bf16, int max_chunks, hipStream_t s);
hipError_t launch_inter(const PrefillArgs& a, int DK, int C, bool bf16, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, int DK, int DV, bool bf16, hipStream_t s);
// Value columns one decode workgroup owns (the output gate needs the whole row).
int decode_columns(int DV);
// Value slices per inter-chunk workgroup (and per Utilde group of the
// workspace): all dv / 16 for whole-row workgroups, else the plain grouping.
int slice_group(int DV, bool whole);
// Whether there are enough (sequence, head) units for whole-row workgroups:
// at least as many as the device has CUs (queried once per device).  With
// fewer, calls that take chunk ranges still run whole rows (one per range);
// the others spread one-slice workgroups over every CU, and gated ones then
// finish the norm in an epilogue kernel.
bool whole_rows(int64_t units);
hipError_t launch_gate_epilogue(const PrefillArgs& a, int64_t rows, bool bf16, hipStream_t s);
int64_t chunk_block_bytes(int DK, int C, int DV, bool bf16, int gsl);

}  // namespace kda
