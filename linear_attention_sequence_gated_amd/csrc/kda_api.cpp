// kda_api.cpp -- the C ABI of libkda.so: argument validation, workspace
// sizing and kernel launches.  Declarations and the contract of every entry
// point are in include/kda.h.
#include "../../include/kda.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <vector>

#include "kda_kernels.h"

// Scratch of kda_chunk_fwd_noalloc: device memory the library owns, so that
// that entry point needs no allocation by anyone.  Each device that loads the
// library holds its own copy until the process ends.  In host code the name
// `scratch` is only a host-side stand-in; its device address is taken once
// per device with hipGetSymbolAddress (noalloc_scratch() below) and that
// address is what the kernels receive.
static __device__ __align__(256) char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kWsAlign = 256;

bool head_dim_ok(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace: [range status words (kWsAlign bytes): the call's, then the one
// kda_chunk_fwd_windowed folds its calls' words into] [chunk-offset table and
// sequence order (packed input only)] [per (chunk, head) blocks] [chunk-range
// scan: range-offset table (packed), range maps, range start states] [gate
// scratch (split gated calls)].
constexpr size_t kStatusBytes = kWsAlign;

struct PrefillPlan {
    int64_t max_chunks;     // per head, worst case
    int64_t block_bytes;    // per (chunk, head)
    size_t off_bytes;       // chunk-offset table and sequence order (packed input only)
    bool whole;             // whole-row inter-chunk workgroups
    bool seq_order;         // the whole-row pass takes the packed sequences longest first
    int range_len;          // chunks per range of the chunk-range scan (0: none)
    int64_t max_ranges;     // ranges of the call at most
    int ranges_per_seq;     // fixed-length input
    size_t range_off;       // byte offsets of the range tables in the workspace
    size_t range_ab;
    size_t range_start;
    size_t total;
};

bool dtype_ok(int32_t d) { return d == KDA_DTYPE_F32 || d == KDA_DTYPE_BF16; }

kda_status_t check_params(const kda_chunk_params_t* p) {
    if (!p) return KDA_ERR_INVALID_ARG;
    if (p->batch < 1 || p->seqlen < 0 || p->num_seqs < 1 || p->num_heads < 1) return KDA_ERR_INVALID_ARG;
    if (!dtype_ok(p->qkv_dtype) || !dtype_ok(p->o_dtype)) return KDA_ERR_UNSUPPORTED;
    if (!head_dim_ok(p->head_dim_k) || !head_dim_ok(p->head_dim_v)) return KDA_ERR_UNSUPPORTED;
    if (p->chunk_size != 16 && p->chunk_size != 32 && p->chunk_size != 64) return KDA_ERR_UNSUPPORTED;
    if (!(p->scale == p->scale)) return KDA_ERR_INVALID_ARG;  // NaN
    // every flattened index must fit comfortably in int64 and the chunk
    // counts in int32
    const int64_t tokens = (int64_t)p->batch * p->seqlen;
    if (p->seqlen > 0 && tokens / p->seqlen != p->batch) return KDA_ERR_INVALID_ARG;
    if (tokens > (int64_t)1 << 40) return KDA_ERR_INVALID_ARG;
    if ((int64_t)p->num_seqs * p->num_heads > ((int64_t)1 << 31) - 1) return KDA_ERR_INVALID_ARG;
    return KDA_OK;
}

int chunk_of(const kda_chunk_params_t* p) {
    return kda::effective_chunk(p->head_dim_k, p->chunk_size, p->qkv_dtype == KDA_DTYPE_BF16);
}

// The layout of one call: packed or fixed-length input, with or without the
// output gate (gated calls take whole rows or chunk ranges where plain calls
// do, and otherwise one-slice workgroups with the norm finished by the
// epilogue kernel).
PrefillPlan plan_prefill(const kda_chunk_params_t* p, bool packed, bool gate) {
    PrefillPlan pl{};
    const int64_t C = chunk_of(p);
    const bool bf16 = p->qkv_dtype == KDA_DTYPE_BF16;
    const int64_t units = (int64_t)p->num_seqs * p->num_heads;
    const int64_t cps = (p->seqlen + C - 1) / C;   // fixed-length chunks per sequence
    if (packed)
        pl.max_chunks = p->seqlen / C + p->num_seqs + 1;
    else
        pl.max_chunks = (int64_t)p->batch * cps;
    // average chunks per sequence, for the choice of ranges
    const int64_t per_unit = packed ? (p->seqlen / C + p->num_seqs) / p->num_seqs : cps;
    pl.range_len = kda::range_length(p->head_dim_k, p->head_dim_v, (int)C, bf16, units, per_unit);
    pl.whole = kda::whole_rows(units) || pl.range_len > 0;
    pl.block_bytes = kda::chunk_block_bytes(p->head_dim_k, (int)C, p->head_dim_v, bf16,
                                            kda::slice_group(p->head_dim_v, pl.whole));
    pl.off_bytes = packed ? round_up(sizeof(int32_t) * ((size_t)p->num_seqs + 1), kWsAlign) +
                                round_up(sizeof(int32_t) * (size_t)p->num_seqs, kWsAlign)
                          : 0;
    pl.seq_order = packed && pl.whole && pl.range_len == 0;
    size_t at = kStatusBytes + pl.off_bytes + (size_t)pl.max_chunks * (size_t)p->num_heads * (size_t)pl.block_bytes;
    if (pl.range_len > 0) {
        const int64_t L = pl.range_len;
        // every sequence has max(1, ceil(chunks / L)) ranges
        pl.ranges_per_seq = (int)(cps > L ? (cps + L - 1) / L : 1);
        pl.max_ranges = packed ? pl.max_chunks / L + p->num_seqs + 1 : (int64_t)p->num_seqs * pl.ranges_per_seq;
        at = round_up(at, kWsAlign);
        pl.range_off = at;
        at += packed ? round_up(sizeof(int32_t) * ((size_t)p->num_seqs + 1), kWsAlign) : 0;
        const size_t dk = p->head_dim_k, dv = p->head_dim_v, rh = (size_t)pl.max_ranges * p->num_heads;
        pl.range_ab = at;
        at += round_up(rh * dk * (dk + dv) * sizeof(float), kWsAlign);
        pl.range_start = at;
        at += round_up(rh * dk * dv * sizeof(float), kWsAlign);
    }
    pl.total = at;
    return pl;
}

// Every grid of a call stays below the 2^32 work-items one dispatch can
// cover (the intra-chunk kernel has 256 threads per (chunk, head); the
// inter-chunk and range kernels at most 1,024 per workgroup; the epilogue one
// per four outputs).  Only calls far larger than one GPU's memory reach it.
bool fits_dispatch(const kda_chunk_params_t* p, const PrefillPlan& pl, bool split) {
    constexpr uint64_t kLimit = 1ull << 32;
    const uint64_t H = (uint64_t)p->num_heads, units = (uint64_t)p->num_seqs * H, slices = p->head_dim_v / 16;
    const uint64_t intra = (uint64_t)pl.max_chunks * H * 256;
    const uint64_t inter = (pl.range_len > 0 ? (uint64_t)pl.max_ranges * H : (units + 7) / 8 * 8 * slices) * 1024;
    const uint64_t scan = (units + 7) / 8 * 8 * slices * 1024;
    const uint64_t epilogue = split ? (uint64_t)p->batch * (uint64_t)p->seqlen * H * (p->head_dim_v / 4) : 0;
    return intra < kLimit && inter < kLimit && scan < kLimit && epilogue < kLimit;
}

// Scratch of gated calls whose norm is finished by the epilogue kernel:
// un-normalised fp32 outputs and per-slice sums of squares.
size_t gate_scratch_bytes(const kda_chunk_params_t* p) {
    const size_t rows = (size_t)p->batch * (size_t)p->seqlen * (size_t)p->num_heads;
    return round_up(rows * (size_t)p->head_dim_v * 4, kWsAlign) +
           round_up(rows * (size_t)(p->head_dim_v / 16) * 4, kWsAlign);
}

// The quote covers packed and fixed-length calls of the shape.
size_t base_workspace(const kda_chunk_params_t* p, bool gate) {
    size_t most = 0;
    for (int packed = 0; packed < 2; ++packed) {
        const PrefillPlan pl = plan_prefill(p, packed, gate);
        most = pl.total > most ? pl.total : most;
    }
    return most;
}

}  // namespace

extern "C" {

const char* kda_status_string(kda_status_t s) {
    // a C caller may pass any int: its bits are read as one, since a value
    // outside the enumerators' range is not a valid kda_status_t in C++
    int code = 0;
    std::memcpy(&code, &s, sizeof code);
    switch (code) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG: invalid argument (pointer, size or shape)";
        case KDA_ERR_UNSUPPORTED:
            return "KDA_ERR_UNSUPPORTED: head dim, chunk size or dtype not supported, or a call larger than one "
                   "dispatch (2^32 work-items)";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace missing, too small or misaligned";
        case KDA_ERR_HIP: return "KDA_ERR_HIP: a HIP launch or runtime call failed";
        case KDA_ERR_RANGE:
            return "KDA_ERR_RANGE: the result is not finite (an fp16 matrix-core operand of the bf16 path, or an "
                   "fp32 value, left its range)";
    }
    return "KDA: unknown status";
}

kda_status_t kda_chunk_fwd_workspace_size(const kda_chunk_params_t* p, size_t* bytes) {
    if (!bytes) return KDA_ERR_INVALID_ARG;
    const kda_status_t st = check_params(p);
    if (st != KDA_OK) return st;
    // the size is quoted for the worst case of either layout so that one
    // buffer serves packed and fixed-length calls of the same shape
    *bytes = base_workspace(p, false);
    return KDA_OK;
}

kda_status_t kda_chunk_fwd_plan(const kda_chunk_params_t* p, int32_t packed, kda_chunk_plan_t* plan) {
    if (!plan) return KDA_ERR_INVALID_ARG;
    const kda_status_t st = check_params(p);
    if (st != KDA_OK) return st;
    if (packed && p->batch != 1) return KDA_ERR_INVALID_ARG;
    const PrefillPlan pl = plan_prefill(p, packed != 0, false);
    plan->chunk_size = chunk_of(p);
    plan->whole_rows = pl.whole ? 1 : 0;
    plan->range_chunks = pl.range_len;
    plan->max_ranges = pl.range_len > 0 ? (int32_t)pl.max_ranges : 0;
    return KDA_OK;
}

kda_status_t kda_chunk_fwd_ex_workspace_size(const kda_chunk_params_t* p, const kda_chunk_options_t* options,
                                             size_t* bytes) {
    if (!bytes) return KDA_ERR_INVALID_ARG;
    const kda_status_t st = check_params(p);
    if (st != KDA_OK) return st;
    const bool gate = options && options->gate;
    // gated calls add the epilogue's scratch only where they take one-slice
    // workgroups (few (sequence, head) pairs and no chunk ranges)
    size_t most = 0;
    for (int packed = 0; packed < 2; ++packed) {
        const PrefillPlan pl = plan_prefill(p, packed, gate);
        const size_t need = round_up(pl.total, kWsAlign) + (gate && !pl.whole ? gate_scratch_bytes(p) : 0);
        most = need > most ? need : most;
    }
    *bytes = most;
    return KDA_OK;
}

namespace {

enum Phase { kBoth = 3, kIntra = 1, kInter = 2 };

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const char* x = reinterpret_cast<const char*>(a);
    const char* y = reinterpret_cast<const char*>(b);
    return a && b && x < y + nb && y < x + na;
}

// Options: everything zero is the plain operation; only the fields that are
// built are accepted.
kda_status_t check_options(const kda_chunk_params_t* p, const kda_chunk_options_t* op,
                           const float* initial_state, const float* final_state) {
    if (!op) return KDA_OK;
    if (op->norm_weight && !op->gate) return KDA_ERR_INVALID_ARG;   // a norm weight needs a gate
    if (op->gate && !aligned(op->gate, p->qkv_dtype == KDA_DTYPE_BF16 ? 2 : 4)) return KDA_ERR_INVALID_ARG;
    if (op->norm_weight && !aligned(op->norm_weight, 4)) return KDA_ERR_INVALID_ARG;
    if (!(op->norm_eps >= 0.f)) return KDA_ERR_INVALID_ARG;       // also NaN
    if (!(op->decay_floor >= 0.f)) return KDA_ERR_INVALID_ARG;   // also NaN
    if (op->alpha_mode != 0 && op->alpha_mode != 1) return KDA_ERR_INVALID_ARG;
    if (op->fuse_inputs != 0 && op->fuse_inputs != 1) return KDA_ERR_INVALID_ARG;
    if (op->ckpt_every < 0) return KDA_ERR_INVALID_ARG;
    if (op->ckpt_every > 0) {
        if (op->ckpt_every % 64 != 0 || op->max_ckpts < 1 || !op->checkpoints || !aligned(op->checkpoints, 16))
            return KDA_ERR_INVALID_ARG;
        const size_t state = (size_t)p->num_heads * p->head_dim_k * p->head_dim_v * sizeof(float);
        const size_t cb = (size_t)p->num_seqs * (size_t)op->max_ckpts * state;
        if (cb / state / (size_t)p->num_seqs != (size_t)op->max_ckpts) return KDA_ERR_INVALID_ARG;
        const size_t sb = (size_t)p->num_seqs * state;
        if (overlaps(op->checkpoints, cb, initial_state, sb) || overlaps(op->checkpoints, cb, final_state, sb))
            return KDA_ERR_INVALID_ARG;
    }
    return KDA_OK;
}

// `layout_checked`: cu_seqlens holds token offsets the caller has already
// checked (kda_chunk_fwd_windowed's groups, whose offsets start at
// `tok_base`, the value of cu_seqlens[0]); otherwise the chunk-offset kernel
// checks its layout on the device and tok_base is 0.
kda_status_t chunk_fwd_impl(const kda_chunk_params_t* p, const kda_chunk_options_t* op, const void* q,
                            const void* k, const void* v, const float* alpha, const float* beta,
                            const float* initial_state, const int32_t* cu_seqlens, void* o, float* final_state,
                            void* workspace, size_t workspace_bytes, void* stream, int phases,
                            bool layout_checked = false, int64_t tok_base = 0) {
    kda_status_t st = check_params(p);
    if (st != KDA_OK) return st;
    st = check_options(p, op, initial_state, final_state);
    if (st != KDA_OK) return st;
    const bool ckpt = op && op->ckpt_every > 0;
    const bool scalar_alpha = op && op->alpha_mode == 1;
    const bool packed = cu_seqlens != nullptr;
    if (packed && p->batch != 1) return KDA_ERR_INVALID_ARG;
    if (!packed && p->num_seqs != p->batch) return KDA_ERR_INVALID_ARG;
    const bool has_tokens = p->seqlen > 0;
    if (has_tokens) {
        if (!q || !k || !v || !alpha || !beta || !o) return KDA_ERR_INVALID_ARG;
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
            !aligned(alpha, scalar_alpha ? 4 : 16) || !aligned(beta, 4))
            return KDA_ERR_INVALID_ARG;
    }
    if (initial_state && !aligned(initial_state, 16)) return KDA_ERR_INVALID_ARG;
    if (final_state && !aligned(final_state, 16)) return KDA_ERR_INVALID_ARG;
    if (packed && !aligned(cu_seqlens, 4)) return KDA_ERR_INVALID_ARG;
    if (initial_state && final_state && initial_state != final_state) {
        // partial overlap would race between slices; exact aliasing is fine
        const size_t sb = (size_t)p->num_seqs * p->num_heads * p->head_dim_k * p->head_dim_v * sizeof(float);
        if (overlaps(initial_state, sb, final_state, sb)) return KDA_ERR_INVALID_ARG;
    }
    const bool gate = op && op->gate;
    const PrefillPlan pl = plan_prefill(p, packed, gate);
    const bool whole = pl.whole;
    const bool split = gate && !whole;
    if (!fits_dispatch(p, pl, split)) return KDA_ERR_UNSUPPORTED;
    const size_t need = round_up(pl.total, kWsAlign) + (split ? gate_scratch_bytes(p) : 0);
    if (need > 0) {
        if (!workspace || !aligned(workspace, kWsAlign)) return KDA_ERR_WORKSPACE;
        if (workspace_bytes < need) return KDA_ERR_WORKSPACE;
    }
    if (!final_state && !has_tokens) {   // nothing to compute or write (no checkpoint is reached)
        if (!(phases & kIntra)) return KDA_OK;
        // the range status still reads clear afterwards
        return kda::launch_clear_status(reinterpret_cast<int32_t*>(workspace), reinterpret_cast<hipStream_t>(stream)) ==
                       hipSuccess
                   ? KDA_OK
                   : KDA_ERR_HIP;
    }

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char* ws = reinterpret_cast<char*>(workspace);
    kda::PrefillArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.alpha = alpha;
    a.beta = beta;
    a.s0 = initial_state;
    a.s_final = final_state;
    a.cu_seqlens = cu_seqlens;
    a.status = reinterpret_cast<int32_t*>(ws);
    a.chunk_off = packed ? reinterpret_cast<const int32_t*>(ws + kStatusBytes) : nullptr;
    int32_t* const seq_order =
        packed ? reinterpret_cast<int32_t*>(ws + kStatusBytes +
                                            round_up(sizeof(int32_t) * ((size_t)p->num_seqs + 1), kWsAlign))
               : nullptr;
    a.seq_order = pl.seq_order ? seq_order : nullptr;
    a.o = o;
    a.ws_chunks = ws + kStatusBytes + pl.off_bytes;
    a.T = p->seqlen;
    a.N = p->num_seqs;
    a.H = p->num_heads;
    a.DV = p->head_dim_v;
    const int C = chunk_of(p);
    a.chunks_per_seq = (int32_t)((p->seqlen + C - 1) / C);
    a.scale = p->scale;
    a.o_f32 = p->o_dtype == KDA_DTYPE_F32;
    a.ckpt = ckpt ? op->checkpoints : nullptr;
    a.ckpt_every = ckpt ? op->ckpt_every : 0;
    a.max_ckpts = ckpt ? op->max_ckpts : 0;
    if (op) {
        a.alpha_floor = op->decay_floor;
        a.alpha_scalar = op->alpha_mode;
        a.fuse_inputs = op->fuse_inputs;
        a.gate = op->gate;
        a.norm_w = op->norm_weight;
        a.norm_eps = op->norm_eps;
    }
    a.gsl = kda::slice_group(p->head_dim_v, whole);
    a.whole_rows = whole;
    if (pl.range_len > 0) {
        a.range_len = pl.range_len;
        a.ranges_per_seq = pl.ranges_per_seq;
        a.max_ranges = (int32_t)pl.max_ranges;
        a.range_off = packed ? reinterpret_cast<const int32_t*>(ws + pl.range_off) : nullptr;
        a.range_ab = reinterpret_cast<float*>(ws + pl.range_ab);
        a.range_start = reinterpret_cast<float*>(ws + pl.range_start);
    }
    const int64_t rows = (int64_t)p->batch * p->seqlen * p->num_heads;
    const bool bf16 = p->qkv_dtype == KDA_DTYPE_BF16;
    // The split gate's scratch holds the call's rows (token * H + head) from
    // row 0, while the inter-chunk kernel indexes rows by the token offsets of
    // cu_seqlens: with offsets starting at tok_base the kernel gets scratch
    // pointers moved back by tok_base tokens (every row it touches lands in the
    // scratch), and the epilogue, which counts rows from 0, gets o and the gate
    // moved forward by tok_base tokens.
    kda::PrefillArgs ep{};
    if (split) {
        float* const o_scr = reinterpret_cast<float*>(ws + round_up(pl.total, kWsAlign));
        float* const part = reinterpret_cast<float*>(reinterpret_cast<char*>(o_scr) +
                                                     round_up((size_t)rows * p->head_dim_v * 4, kWsAlign));
        const uint64_t back = (uint64_t)tok_base * (uint64_t)p->num_heads;   // rows before the call's first
        a.gate_split = 1;
        a.o_scratch = reinterpret_cast<float*>(reinterpret_cast<uintptr_t>(o_scr) - back * p->head_dim_v * 4);
        a.part_scratch = reinterpret_cast<float*>(reinterpret_cast<uintptr_t>(part) - back * (p->head_dim_v / 16) * 4);
        ep = a;
        ep.o_scratch = o_scr;
        ep.part_scratch = part;
        ep.o = static_cast<char*>(o) + back * p->head_dim_v * (p->o_dtype == KDA_DTYPE_BF16 ? 2 : 4);
        ep.gate = static_cast<const char*>(op->gate) + back * p->head_dim_v * (bf16 ? 2 : 4);
    }

    hipError_t e = hipSuccess;
    if (phases & kIntra) {
        if (packed) {
            int32_t* chunk_off = reinterpret_cast<int32_t*>(ws + kStatusBytes);
            const int64_t check_T = layout_checked ? -1 : p->seqlen;
            e = pl.range_len > 0 ? kda::launch_chunk_range_offsets(cu_seqlens, p->num_seqs, C, pl.range_len, chunk_off,
                                                                   reinterpret_cast<int32_t*>(ws + pl.range_off),
                                                                   check_T, a.status, s)
                                 : kda::launch_chunk_offsets(cu_seqlens, p->num_seqs, C, chunk_off, check_T, a.status,
                                                             s);
            if (e != hipSuccess) return KDA_ERR_HIP;
            if (pl.seq_order) {
                e = kda::launch_seq_order(cu_seqlens, p->num_seqs, C, seq_order, s);
                if (e != hipSuccess) return KDA_ERR_HIP;
            }
        }
        // the intra-chunk kernel clears the range status; without chunks to
        // process it is not launched and a one-thread kernel clears it
        e = pl.max_chunks > 0 ? kda::launch_intra(a, p->head_dim_k, C, bf16, (int)pl.max_chunks, s)
                              : kda::launch_clear_status(a.status, s);
        if (e != hipSuccess) return KDA_ERR_HIP;
    }
    if (phases & kInter) {
        e = kda::launch_inter(a, p->head_dim_k, C, bf16, s);
        if (e != hipSuccess) return KDA_ERR_HIP;
        if (split) {
            e = kda::launch_gate_epilogue(ep, rows, bf16, s);
            if (e != hipSuccess) return KDA_ERR_HIP;
        }
    }
    return KDA_OK;
}

}  // namespace

}  // extern "C"

namespace {

// Device address of `scratch` on each device, taken on the first
// kda_chunk_fwd_noalloc call with that device current (null: not yet).  Two
// threads racing on the first call store the same address.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];

kda_status_t noalloc_scratch(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return KDA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return KDA_ERR_UNSUPPORTED;
    void* ptr = g_scratch[dev].load(std::memory_order_acquire);
    if (!ptr) {
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();   // consume the error: the call reports it
            return KDA_ERR_HIP;
        }
        g_scratch[dev].store(ptr, std::memory_order_release);
    }
    *out = ptr;
    return KDA_OK;
}

}  // namespace

extern "C" {

kda_status_t kda_chunk_fwd_noalloc(const kda_chunk_params_t* p, const void* q, const void* k, const void* v,
                                   const float* alpha, const float* beta, const float* initial_state,
                                   const int32_t* cu_seqlens, void* o, float* final_state, void* stream) {
    kda_status_t st = check_params(p);
    if (st != KDA_OK) return st;
    if (base_workspace(p, false) > (size_t)KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_WORKSPACE;
    void* ws = nullptr;
    st = noalloc_scratch(&ws);
    if (st != KDA_OK) return st;
    // every byte of the scratch a kernel reads is written earlier in the same
    // call (chunk offsets, then the per-chunk blocks), so nothing is cleared
    return chunk_fwd_impl(p, nullptr, q, k, v, alpha, beta, initial_state, cu_seqlens, o, final_state, ws,
                          (size_t)KDA_NOALLOC_SCRATCH_BYTES, stream, kBoth);
}

}  // extern "C"

namespace {

// One call of a windowed prefill: a shape, where its token pointers start,
// its cu_seqlens (device, absolute token offsets) or none, its first sequence,
// the token of that sequence it starts at and whether it resumes from
// final_state.
struct SubCall {
    kda_chunk_params_t p;
    int64_t tok;
    const int32_t* cu;
    int64_t seq0;
    int64_t t0;
    bool resume;
};

// Workspace of one call in one layout (the gate's epilogue scratch included
// where the shape takes it).
size_t call_quote(const kda_chunk_params_t& sp, bool packed, bool gate) {
    const PrefillPlan pl = plan_prefill(&sp, packed, gate);
    return round_up(pl.total, kWsAlign) + (gate && !pl.whole ? gate_scratch_bytes(&sp) : 0);
}

// Cuts a run of `len` tokens of one sequence (starting at token `tok` of the
// flattened token axis) into windows of whole multiples of `step` chunks that
// fit `bytes`; each window after the first resumes from the state the one
// before left.  An empty sequence is one call without tokens (its final state
// is the initial one).
kda_status_t plan_windows(const kda_chunk_params_t* p, bool gate, int64_t step, int64_t tok, int64_t len,
                          int64_t seq, size_t bytes, std::vector<SubCall>& calls) {
    kda_chunk_params_t w = *p;
    w.batch = 1;
    w.num_seqs = 1;
    if (len == 0) {
        w.seqlen = 0;
        if (call_quote(w, false, gate) > bytes) return KDA_ERR_WORKSPACE;
        calls.push_back({w, tok, nullptr, seq, 0, false});
        return KDA_OK;
    }
    const int64_t C = chunk_of(p), padded = (len + C - 1) / C * C;
    auto fits = [&](int64_t m) {   // m windows' worth of `step` chunks
        w.seqlen = std::min(m * step * C, padded);
        return call_quote(w, false, gate) <= bytes;
    };
    if (!fits(1)) return KDA_ERR_WORKSPACE;
    int64_t lo = 1, hi = (padded / C + step - 1) / step;   // the largest multiple that fits
    while (lo < hi) {
        const int64_t mid = lo + (hi - lo + 1) / 2;
        if (fits(mid)) lo = mid; else hi = mid - 1;
    }
    const int64_t span = lo * step * C;
    for (int64_t t0 = 0; t0 < len; t0 += span) {
        w.seqlen = std::min(span, len - t0);
        calls.push_back({w, tok + t0, nullptr, seq, t0, t0 > 0});
    }
    return KDA_OK;
}

kda_status_t chunk_fwd_windowed_impl(const kda_chunk_params_t* p, const kda_chunk_options_t* op, const void* q,
                                     const void* k, const void* v, const float* alpha, const float* beta,
                                     const float* initial_state, const int32_t* cu_seqlens,
                                     const int32_t* cu_seqlens_host, void* o, float* final_state, void* workspace,
                                     size_t workspace_bytes, void* stream) {
    kda_status_t st = check_params(p);
    if (st != KDA_OK) return st;
    const bool packed = cu_seqlens != nullptr;
    if (packed != (cu_seqlens_host != nullptr)) return KDA_ERR_INVALID_ARG;
    if (packed && p->batch != 1) return KDA_ERR_INVALID_ARG;
    if (!packed && p->num_seqs != p->batch) return KDA_ERR_INVALID_ARG;
    if (!final_state || !aligned(final_state, 16)) return KDA_ERR_INVALID_ARG;
    if (initial_state && !aligned(initial_state, 16)) return KDA_ERR_INVALID_ARG;
    if (initial_state && initial_state != final_state) {
        const size_t sb = (size_t)p->num_seqs * p->num_heads * p->head_dim_k * p->head_dim_v * sizeof(float);
        if (overlaps(initial_state, sb, final_state, sb)) return KDA_ERR_INVALID_ARG;
    }
    // the options are checked on the whole call: each call below takes a
    // slice of the gate, alpha and checkpoint arrays, which keeps their
    // alignment and stays clear of the states
    st = check_options(p, op, initial_state, final_state);
    if (st != KDA_OK) return st;
    const bool scalar_alpha = op && op->alpha_mode == 1;
    const bool gate = op && op->gate;
    const bool ckpt = op && op->ckpt_every > 0;
    // every window's pointers keep the alignment of the call's (a token's row
    // is a multiple of 32 bytes), so checking them here covers every window
    if (p->seqlen > 0) {
        if (!q || !k || !v || !alpha || !beta || !o) return KDA_ERR_INVALID_ARG;
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
            !aligned(alpha, scalar_alpha ? 4 : 16) || !aligned(beta, 4))
            return KDA_ERR_INVALID_ARG;
    }
    if (packed && !aligned(cu_seqlens, 4)) return KDA_ERR_INVALID_ARG;
    if (!workspace || !aligned(workspace, kWsAlign)) return KDA_ERR_WORKSPACE;
    const int64_t N = p->num_seqs, T = p->seqlen;
    if (packed) {   // the host copy makes the layout checkable
        if (cu_seqlens_host[0] != 0 || cu_seqlens_host[N] != T) return KDA_ERR_INVALID_ARG;
        for (int64_t n = 0; n < N; ++n)
            if (cu_seqlens_host[n + 1] < cu_seqlens_host[n]) return KDA_ERR_INVALID_ARG;
    }
    // Plan every call before launching any: whole sequences (rows) are grouped
    // while their quote fits, a sequence that does not fit alone runs in
    // windows of whole chunks.  With checkpoints a window holds whole
    // checkpoint intervals, so that its checkpoints are slots of its
    // sequence's row.
    const int64_t step = ckpt ? op->ckpt_every / chunk_of(p) : 1;
    std::vector<SubCall> calls;
    int64_t n0 = 0;
    while (n0 < N) {
        auto group = [&](int64_t n1) {
            kda_chunk_params_t g = *p;
            g.num_seqs = (int32_t)(n1 - n0);
            if (packed) {
                g.batch = 1;
                g.seqlen = (int64_t)cu_seqlens_host[n1] - cu_seqlens_host[n0];
            } else {
                g.batch = g.num_seqs;
            }
            return g;
        };
        int64_t n1 = n0;   // the longest group [n0, n1) that fits
        {
            int64_t lo = n0, hi = N;
            while (lo < hi) {
                const int64_t mid = lo + (hi - lo + 1) / 2;
                if (call_quote(group(mid), packed, gate) <= workspace_bytes) lo = mid; else hi = mid - 1;
            }
            n1 = lo;
        }
        if (n1 > n0) {
            calls.push_back({group(n1), packed ? 0 : n0 * T, packed ? cu_seqlens + n0 : nullptr, n0, 0, false});
            n0 = n1;
        } else {
            const int64_t tok = packed ? cu_seqlens_host[n0] : n0 * T;
            const int64_t len = packed ? (int64_t)cu_seqlens_host[n0 + 1] - cu_seqlens_host[n0] : T;
            st = plan_windows(p, gate, step, tok, len, n0, workspace_bytes, calls);
            if (st != KDA_OK) return st;
            ++n0;
        }
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    int32_t* status = reinterpret_cast<int32_t*>(workspace);
    if (kda::launch_fold_status(status, kda::kFoldClear, s) != hipSuccess) return KDA_ERR_HIP;
    const size_t in_bytes = p->qkv_dtype == KDA_DTYPE_BF16 ? 2 : 4;
    const size_t eq = (size_t)p->num_heads * p->head_dim_k * in_bytes;
    const size_t ev = (size_t)p->num_heads * p->head_dim_v * in_bytes;   // also the gate's row
    const size_t eo = (size_t)p->num_heads * p->head_dim_v * (p->o_dtype == KDA_DTYPE_BF16 ? 2 : 4);
    const size_t ea = (size_t)p->num_heads * (scalar_alpha ? 1 : p->head_dim_k), eb = (size_t)p->num_heads;
    const size_t es = (size_t)p->num_heads * p->head_dim_k * p->head_dim_v;   // floats per state
    for (const SubCall& c : calls) {
        const size_t t = (size_t)c.tok;
        kda_chunk_options_t so{};
        if (op) {
            so = *op;
            if (gate) so.gate = static_cast<const char*>(op->gate) + t * ev;
            if (ckpt) {   // checkpoint j of this call is slot c.t0 / every + j of its sequence
                const int64_t k0 = c.t0 / op->ckpt_every;
                if (k0 < op->max_ckpts) {
                    so.checkpoints = op->checkpoints + ((size_t)c.seq0 * op->max_ckpts + (size_t)k0) * es;
                    so.max_ckpts = op->max_ckpts - (int32_t)k0;
                } else {   // past the last slot: nothing to write
                    so.checkpoints = nullptr;
                    so.ckpt_every = 0;
                    so.max_ckpts = 0;
                }
            }
        }
        const float* s0 = c.resume ? final_state + c.seq0 * es : initial_state ? initial_state + c.seq0 * es : nullptr;
        // a packed group keeps the call's token pointers and its absolute offsets
        const int64_t tok_base = c.cu ? cu_seqlens_host[c.seq0] : 0;
        st = chunk_fwd_impl(&c.p, op ? &so : nullptr, static_cast<const char*>(q) + t * eq,
                            static_cast<const char*>(k) + t * eq, static_cast<const char*>(v) + t * ev,
                            alpha + t * ea, beta + t * eb, s0, c.cu, static_cast<char*>(o) + t * eo,
                            final_state + c.seq0 * es, workspace, workspace_bytes, stream, kBoth, true, tok_base);
        if (st != KDA_OK) return st;
        if (kda::launch_fold_status(status, kda::kFoldOr, s) != hipSuccess) return KDA_ERR_HIP;
    }
    return kda::launch_fold_status(status, kda::kFoldBack, s) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

extern "C" {

kda_status_t kda_chunk_fwd_windowed(const kda_chunk_params_t* p, const void* q, const void* k, const void* v,
                                    const float* alpha, const float* beta, const float* initial_state,
                                    const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, void* o,
                                    float* final_state, void* workspace, size_t workspace_bytes, void* stream) {
    return chunk_fwd_windowed_impl(p, nullptr, q, k, v, alpha, beta, initial_state, cu_seqlens, cu_seqlens_host,
                                   o, final_state, workspace, workspace_bytes, stream);
}

kda_status_t kda_chunk_fwd_windowed_ex(const kda_chunk_params_t* p, const kda_chunk_options_t* options,
                                       const void* q, const void* k, const void* v, const float* alpha,
                                       const float* beta, const float* initial_state, const int32_t* cu_seqlens,
                                       const int32_t* cu_seqlens_host, void* o, float* final_state,
                                       void* workspace, size_t workspace_bytes, void* stream) {
    return chunk_fwd_windowed_impl(p, options, q, k, v, alpha, beta, initial_state, cu_seqlens, cu_seqlens_host,
                                   o, final_state, workspace, workspace_bytes, stream);
}

kda_status_t kda_chunk_fwd_status(const void* workspace, void* stream) {
    if (!workspace || !aligned(workspace, kWsAlign)) return KDA_ERR_INVALID_ARG;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    int32_t words[kda::kLayoutWord + 1] = {};
    if (hipMemcpyAsync(words, workspace, sizeof words, hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess) {
        (void)hipGetLastError();
        return KDA_ERR_HIP;
    }
    if (words[kda::kLayoutWord]) return KDA_ERR_INVALID_ARG;   // cu_seqlens broke its layout
    return words[0] ? KDA_ERR_RANGE : KDA_OK;
}

kda_status_t kda_chunk_fwd(const kda_chunk_params_t* p, const void* q, const void* k, const void* v,
                           const float* alpha, const float* beta, const float* initial_state,
                           const int32_t* cu_seqlens, void* o, float* final_state, void* workspace,
                           size_t workspace_bytes, void* stream) {
    return chunk_fwd_impl(p, nullptr, q, k, v, alpha, beta, initial_state, cu_seqlens, o, final_state, workspace,
                          workspace_bytes, stream, kBoth);
}

kda_status_t kda_chunk_fwd_ex(const kda_chunk_params_t* p, const kda_chunk_options_t* options, const void* q,
                              const void* k, const void* v, const float* alpha, const float* beta,
                              const float* initial_state, const int32_t* cu_seqlens, void* o, float* final_state,
                              void* workspace, size_t workspace_bytes, void* stream) {
    return chunk_fwd_impl(p, options, q, k, v, alpha, beta, initial_state, cu_seqlens, o, final_state, workspace,
                          workspace_bytes, stream, kBoth);
}

kda_status_t kda_chunk_fwd_intra(const kda_chunk_params_t* p, const void* q, const void* k, const void* v,
                                 const float* alpha, const float* beta, const float* initial_state,
                                 const int32_t* cu_seqlens, void* o, float* final_state, void* workspace,
                                 size_t workspace_bytes, void* stream) {
    return chunk_fwd_impl(p, nullptr, q, k, v, alpha, beta, initial_state, cu_seqlens, o, final_state, workspace,
                          workspace_bytes, stream, kIntra);
}

kda_status_t kda_chunk_fwd_inter(const kda_chunk_params_t* p, const void* q, const void* k, const void* v,
                                 const float* alpha, const float* beta, const float* initial_state,
                                 const int32_t* cu_seqlens, void* o, float* final_state, void* workspace,
                                 size_t workspace_bytes, void* stream) {
    return chunk_fwd_impl(p, nullptr, q, k, v, alpha, beta, initial_state, cu_seqlens, o, final_state, workspace,
                          workspace_bytes, stream, kInter);
}

namespace {

kda_status_t decode_impl(int32_t num_seqs, int32_t num_heads, int32_t dk, int32_t dv, float scale,
                         int32_t qkv_dtype, int32_t o_dtype, const kda_decode_options_t* op, const void* q,
                         const void* k, const void* v, const float* alpha, const float* beta, float* state,
                         void* o, void* stream) {
    if (num_seqs < 1 || num_heads < 1) return KDA_ERR_INVALID_ARG;
    if ((int64_t)num_seqs * num_heads > ((int64_t)1 << 31) - 1) return KDA_ERR_INVALID_ARG;
    if (!dtype_ok(qkv_dtype) || !dtype_ok(o_dtype)) return KDA_ERR_UNSUPPORTED;
    if (!head_dim_ok(dk) || !head_dim_ok(dv)) return KDA_ERR_UNSUPPORTED;
    // one dispatch: (sequence, head, column block) workgroups of at most 256 threads
    if ((uint64_t)num_seqs * num_heads * (uint64_t)(dv / kda::decode_columns(dv)) * 256 >= (1ull << 32))
        return KDA_ERR_UNSUPPORTED;
    if (!(scale == scale)) return KDA_ERR_INVALID_ARG;
    if (!q || !k || !v || !alpha || !beta || !state || !o) return KDA_ERR_INVALID_ARG;
    const bool scalar_alpha = op && op->alpha_mode == 1;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        !aligned(alpha, scalar_alpha ? 4 : 16) || !aligned(state, 16) || !aligned(beta, 4))
        return KDA_ERR_INVALID_ARG;
    if (op) {
        if (!(op->decay_floor >= 0.f) || !(op->norm_eps >= 0.f)) return KDA_ERR_INVALID_ARG;  // also NaN
        if (op->alpha_mode != 0 && op->alpha_mode != 1) return KDA_ERR_INVALID_ARG;
        if (op->fuse_inputs != 0 && op->fuse_inputs != 1) return KDA_ERR_INVALID_ARG;
        if (op->state_slots && !aligned(op->state_slots, 4)) return KDA_ERR_INVALID_ARG;
        if (op->pool_entries < 0) return KDA_ERR_INVALID_ARG;
        if (op->gate && !aligned(op->gate, qkv_dtype == KDA_DTYPE_BF16 ? 2 : 4)) return KDA_ERR_INVALID_ARG;
        if (op->norm_weight && !aligned(op->norm_weight, 4)) return KDA_ERR_INVALID_ARG;
        if (op->norm_weight && !op->gate) return KDA_ERR_INVALID_ARG;
        if (op->gate && kda::decode_columns(dv) < dv) return KDA_ERR_UNSUPPORTED;  // row split over workgroups
    }
    kda::DecodeArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.alpha = alpha;
    a.beta = beta;
    a.state = state;
    a.o = o;
    a.units = num_seqs * num_heads;
    a.H = num_heads;
    a.scale = scale;
    a.o_f32 = o_dtype == KDA_DTYPE_F32;
    if (op) {
        a.slots = op->state_slots;
        a.pool_entries = op->pool_entries;
        a.alpha_floor = op->decay_floor;
        a.alpha_scalar = op->alpha_mode;
        a.fuse_inputs = op->fuse_inputs;
        a.gate = op->gate;
        a.norm_w = op->norm_weight;
        a.norm_eps = op->norm_eps;
    }
    const hipError_t e = kda::launch_decode(a, dk, dv, qkv_dtype == KDA_DTYPE_BF16, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

kda_status_t kda_decode_step(int32_t num_seqs, int32_t num_heads, int32_t dk, int32_t dv, float scale,
                             int32_t qkv_dtype, int32_t o_dtype, const void* q, const void* k, const void* v,
                             const float* alpha, const float* beta, float* state, void* o, void* stream) {
    return decode_impl(num_seqs, num_heads, dk, dv, scale, qkv_dtype, o_dtype, nullptr, q, k, v, alpha, beta, state,
                       o, stream);
}

kda_status_t kda_decode_step_ex(int32_t num_seqs, int32_t num_heads, int32_t dk, int32_t dv, float scale,
                                int32_t qkv_dtype, int32_t o_dtype, const kda_decode_options_t* options,
                                const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                                float* state, void* o, void* stream) {
    return decode_impl(num_seqs, num_heads, dk, dv, scale, qkv_dtype, o_dtype, options, q, k, v, alpha, beta, state,
                       o, stream);
}

}  // extern "C"
