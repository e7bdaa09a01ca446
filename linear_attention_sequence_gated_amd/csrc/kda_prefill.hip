// kda_prefill.hip -- chunked KDA prefill on gfx950.
//
// The recurrence (per sequence and head, state S of dk x dv):
//   S' = diag(alpha_t) S ;  S = S' + beta_t k_t (v_t - S'^T k_t)^T ;  o_t = scale S^T q_t
// follows "Kimi K3 Architecture Teardown", Visual 5 (decay, erase, write) and
// "Kimi K3 Architecture: KDA, MoE, and Attention", section "Memory as a
// First-Class Problem: Kimi Delta Attention" (channel-wise alpha, one beta,
// read after the update).  The pages give no parallel form; the chunk form
// used here is derived from the recurrence.  For a chunk of C tokens entering
// state S, with g_r = sum_{s<=r} log2 alpha_s (per key channel, inclusive):
//   Ktilde_r = k_r 2^{g_r},  Qtilde_r = q_r 2^{g_r},  Kbar_i = k_i 2^{g_C - g_i}
//   M_ri  = beta_r sum_c k_r[c] k_i[c] 2^{g_r[c] - g_i[c]}   (i < r)
//   P_ri  =        sum_c q_r[c] k_i[c] 2^{g_r[c] - g_i[c]}   (i <= r)
//   Tm = (I + M)^{-1} diag(beta),  W = Tm Ktilde,  Utilde = Tm V
//   U = Utilde - W S ;  O = scale (Qtilde S + P U) ;  S <- diag(2^{g_C}) S + Kbar^T U
// (U holds the per-token corrections beta_r (v_r - S'_r^T k_r) of the chunk.)
//
// Kernels:
//   kda_chunk_offsets  : chunk index of each packed sequence (one workgroup)
//   kda_intra_kernel   : one workgroup per (chunk, head); everything above
//                        that does not depend on S, written to the workspace
//                        in the register layout the next kernel consumes
//   kda_inter_kernel   : one workgroup per (sequence, head, 16 value
//                        columns); walks the chunks in order with its slice
//                        of S held in MFMA accumulator registers (fp32)
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "kda_kernels.h"
#include "kda_quads.h"

namespace kda {

// DPP lane moves inside rows of 16 lanes (CTRL: row_shl:n = 0x100 + n, row_shr:n
// = 0x110 + n); a lane whose source falls outside its row reads 0.
template <int CTRL> __device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float lane_value(float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}
// Inclusive prefix sum over a row of 16 lanes: row_shr moves, each unmasked
// (a lane whose source lies before its row reads 0).  The moves must stay
// unconditional: a select around one let the compiler run it under a lane
// mask, and a DPP read from a masked-off lane returns 0.
__device__ __forceinline__ float row_scan16(float x) {
    x += dpp<0x111>(x);
    x += dpp<0x112>(x);
    x += dpp<0x114>(x);
    x += dpp<0x118>(x);
    return x;
}

template <bool B> struct BoolTag { static constexpr bool value = B; };

// Two fp16 quads that are adjacent in memory (the halves of one 16-byte
// fragment slot) stored with one 16-byte write.
__device__ __forceinline__ void store_pair(_Float16* p, const f32x4& lo, const f32x4& hi) {
    const f16x4 a = make_quad<_Float16>(lo), b = make_quad<_Float16>(hi);
    *reinterpret_cast<f16x8*>(p) = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}



// log2(alpha) is floored here: alpha below 2^-40 is treated as 2^-40, a
// relative change of the decayed terms far below fp32 resolution.
constexpr float kLog2Floor = -40.f;
// Largest decay (log2 units) a 16-token block may show in any channel for the
// factored Gram path; see the intra-chunk kernel.
constexpr float kFastRange = 12.f;

__device__ __forceinline__ float sigmoid(float x) { return 1.f / (1.f + __expf(-x)); }

// Whether all four values are finite.  The inter-chunk kernel checks what it
// writes: with finite inputs, an operand that left its format's range (fp16
// matrix-core operands on the bf16 path) shows up as inf or NaN in o or in
// the state, and the call's status word records it.
__device__ __forceinline__ bool finite4(const f32x4& v) {
    return __builtin_isfinite(v[0]) & __builtin_isfinite(v[1]) & __builtin_isfinite(v[2]) & __builtin_isfinite(v[3]);
}

// Workgroup barrier for LDS producer/consumer hand-offs only.  __syncthreads
// also waits for every outstanding global load and store of the wave (vmcnt),
// which would expose the workspace stores and the early v loads of the
// intra-chunk kernel at each phase boundary; no thread there reads global
// memory another thread of the kernel writes.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// alpha of (token row tok, head h, key channel c) as the recurrence uses it:
// per channel or one per (token, head), through a sigmoid for fused inputs,
// then floored.
__device__ __forceinline__ float alpha_at(const PrefillArgs& a, int64_t tok, int h, int DK, int c) {
    float al = a.alpha_scalar ? a.alpha[tok * a.H + h] : a.alpha[(tok * a.H + h) * DK + c];
    if (a.fuse_inputs) al = sigmoid(al);
    return fmaxf(al, a.alpha_floor);
}

// ---------------------------------------------------------------------------
// K0: exclusive prefix of ceil(len_n / C) over the packed sequences, and, for
// the chunk-range scan (range_off non-null), of max(1, ceil(chunks_n / L)).
// First, when T >= 0, the layout of cu_seqlens is checked: cu[0] == 0,
// non-decreasing, cu[N] == T.  A call that breaks it gets empty tables (no
// chunk and no range is ever located, so no token is read or written) and
// layout status 1 (status word kLayoutWord), else 0.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kda_chunk_offsets(const int32_t* __restrict__ cu, int32_t n_seqs,
                                                         int32_t C, int32_t L, int32_t* __restrict__ chunk_off,
                                                         int32_t* __restrict__ range_off, int64_t T,
                                                         int32_t* __restrict__ status) {
    __shared__ int32_t part[2][256];
    __shared__ int32_t carry[2];
    const int tid = threadIdx.x;
    int bad = 0;
    if (T >= 0) {
        for (int n = tid; n < n_seqs; n += 256) bad |= cu[n + 1] < cu[n];
        if (tid == 0) bad |= cu[0] != 0 || (int64_t)cu[n_seqs] != T;
    }
    bad = __syncthreads_or(bad);
    if (tid == 0) status[kLayoutWord] = bad ? 1 : 0;
    if (bad) {
        for (int n = tid; n <= n_seqs; n += 256) {
            chunk_off[n] = 0;
            if (range_off) range_off[n] = 0;
        }
        return;   // uniform over the workgroup
    }
    if (tid < 2) carry[tid] = 0;
    __syncthreads();
    for (int base = 0; base < n_seqs; base += 256) {
        const int n = base + tid;
        int32_t c = 0, rr = 0;
        if (n < n_seqs) {
            const int32_t len = cu[n + 1] - cu[n];
            c = len > 0 ? (len + C - 1) / C : 0;
            rr = range_off ? max(1, (c + L - 1) / L) : 0;
        }
        part[0][tid] = c;
        part[1][tid] = rr;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {  // inclusive Hillis-Steele scans
            const int32_t add0 = tid >= off ? part[0][tid - off] : 0;
            const int32_t add1 = tid >= off ? part[1][tid - off] : 0;
            __syncthreads();
            part[0][tid] += add0;
            part[1][tid] += add1;
            __syncthreads();
        }
        if (n < n_seqs) {
            chunk_off[n] = carry[0] + part[0][tid] - c;
            if (range_off) range_off[n] = carry[1] + part[1][tid] - rr;
        }
        __syncthreads();
        if (tid == 255) {
            carry[0] += part[0][255];
            carry[1] += part[1][255];
        }
        __syncthreads();
    }
    if (tid == 0) {
        chunk_off[n_seqs] = carry[0];
        if (range_off) range_off[n_seqs] = carry[1];
    }
}

// The packed sequences by decreasing chunk count (ties by index), one
// workgroup: a bitonic sort of (chunk count, index) keys in LDS.  The
// whole-row pass takes its (sequence, head) pairs in this order, so that the
// longest chains start first and the pass does not end on a long one started
// late (packed workload of 64 sequences of 1 to 32,768 tokens, 16 heads:
// 1,201 chunk steps on the busiest CU in input order, 977 in this order).
__global__ __launch_bounds__(1024) void kda_seq_order(const int32_t* __restrict__ cu, int32_t n_seqs, int32_t C,
                                                      int32_t* __restrict__ order) {
    __shared__ unsigned long long key[kSeqOrderMax];
    const int tid = threadIdx.x;
    if (n_seqs > kSeqOrderMax) {   // input order
        for (int i = tid; i < n_seqs; i += 1024) order[i] = i;
        return;
    }
    int P = 1;
    while (P < n_seqs) P <<= 1;
    for (int i = tid; i < P; i += 1024) {
        unsigned long long kv = ~0ull;   // padding sorts last
        if (i < n_seqs) {
            const int32_t len = cu[i + 1] - cu[i];
            const unsigned ch = len > 0 ? (unsigned)((len + C - 1) / C) : 0u;
            kv = ((unsigned long long)(~ch) << 32) | (unsigned)i;   // ascending: more chunks first, then index
        }
        key[i] = kv;
    }
    __syncthreads();
    for (int k = 2; k <= P; k <<= 1)
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = tid; i < P; i += 1024) {
                const int l = i ^ j;
                if (l > i) {
                    const unsigned long long x = key[i], y = key[l];
                    if ((x > y) == ((i & k) == 0)) {
                        key[i] = y;
                        key[l] = x;
                    }
                }
            }
            __syncthreads();
        }
    for (int i = tid; i < n_seqs; i += 1024) order[i] = (int32_t)(key[i] & 0xffffffffull);
}

// Where chunk x of the (flattened) chunk list lives.
struct ChunkPos {
    int64_t tok0;  // first token (row of the flattened [B*T] token axis)
    int valid;     // tokens of the chunk inside the sequence (1..C)
};

__device__ __forceinline__ bool locate_chunk(const PrefillArgs& a, int C, int x, ChunkPos& pos) {
    if (a.cu_seqlens) {
        const int32_t* off = a.chunk_off;
        if (x >= off[a.N]) return false;
        int lo = 0, hi = a.N;  // off[lo] <= x < off[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (off[mid] <= x) lo = mid; else hi = mid;
        }
        const int j = x - off[lo];
        const int64_t s = a.cu_seqlens[lo], e = a.cu_seqlens[lo + 1];
        pos.tok0 = s + (int64_t)j * C;
        pos.valid = (int)min((int64_t)C, e - pos.tok0);
    } else {
        if (x >= a.N * a.chunks_per_seq) return false;
        const int n = x / a.chunks_per_seq, j = x % a.chunks_per_seq;
        pos.tok0 = (int64_t)n * a.T + (int64_t)j * C;
        pos.valid = (int)min((int64_t)C, a.T - (int64_t)j * C);
    }
    return true;
}

// Where range x of the (flattened) range list lives: sequence n, its range r of
// nr, and the chunk window [c0, c1) inside the sequence's chunks starting at
// c_seq (indices of the flattened chunk list).
struct RangePos {
    int n, r, nr;
    int c_seq, c0, c1;
};

__device__ __forceinline__ bool locate_range(const PrefillArgs& a, int x, RangePos& rp) {
    const int L = a.range_len;
    int cb, ce;
    if (a.cu_seqlens) {
        const int32_t* off = a.range_off;
        if (x >= off[a.N]) return false;
        int lo = 0, hi = a.N;  // off[lo] <= x < off[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (off[mid] <= x) lo = mid; else hi = mid;
        }
        rp.n = lo;
        rp.r = x - off[lo];
        rp.nr = off[lo + 1] - off[lo];
        cb = a.chunk_off[lo];
        ce = a.chunk_off[lo + 1];
    } else {
        const int R = a.ranges_per_seq;
        if (x >= a.N * R) return false;
        rp.n = x / R;
        rp.r = x % R;
        rp.nr = R;
        cb = rp.n * a.chunks_per_seq;
        ce = cb + a.chunks_per_seq;
    }
    rp.c_seq = cb;
    rp.c0 = min(cb + rp.r * L, ce);
    rp.c1 = min(rp.c0 + L, ce);
    return true;
}

// ---------------------------------------------------------------------------
// K1: intra-chunk work.  256 threads (4 waves) per (chunk, head).
//
// Gram products on the matrix cores need factors 2^{+-g} that stay inside the
// operand format.  The chunk is cut into 16-token blocks; with G_R the decay
// exponent at the first token of block R and h_R half of the block's own
// decay range (per channel), the products k_r k_i 2^{g_r - g_i} are split as
//   row side   (r in block R)   k_r 2^{g_r - G_R + h_R}                 in 2^[-h_R, h_R]
//   column side (i in block I)  k_i 2^{G_I - h_I - g_i}                 in 2^[-h_I, h_I]
//                               times 2^{G_R - G_I + h_I - h_R} <= 1 when I < R
// which keeps every factor within 2^[-6, 6] while each block decays by less
// than 2^-12 in every channel.  Inside such blocks no alpha is floored, so the
// factors are running products of alpha scaled by a few per-channel powers of
// two.  Chunks beyond that take the exact pairwise path (decay products in
// linear space, fp32).
// ---------------------------------------------------------------------------
template <int DK, int C, typename T> struct Intra {
    static constexpr int kThreads = 256;
    static constexpr int NSEG = C / 4;   // 4-token segments
    static constexpr int NCG = DK / 8;   // 8-channel groups
    static constexpr int NB = C / 16;    // 16-token blocks
    static constexpr int NOFF = NB * (NB - 1) / 2;  // off-diagonal block pairs
    static constexpr int NQK = DK / 16;  // quads along dk
    static constexpr int LD_ROW = DK + 8;  // row-major [*][DK] tiles (elements)
    static constexpr int LD_CT = C + 4;    // [*][C] tiles (elements): a row stride of 2C + 8 bytes
                                           // spreads 32 consecutive rows over distinct bank pairs
    static constexpr int LD_F = C + 4;     // fp32 [C][C] matrices
    static constexpr int kDvMax = 128;
    static constexpr size_t a16(size_t x) { return (x + 15) / 16 * 16; }
    static constexpr size_t cmax(size_t x, size_t y) { return x > y ? x : y; }
    // region 1, in turn: fused-input norms -> {Ak, Aq, Bd} -> {P, MX, Tm, XD} -> {P, VT, Tm}
    static constexpr size_t kSeg = 8ull * C * 4;   // per-wave partial norms of the fused inputs
    static constexpr size_t kTile = (size_t)C * LD_ROW * sizeof(T);
    static constexpr size_t kMat = (size_t)C * LD_F * 4;
    static constexpr size_t oP = 0, oMX = kMat, oY = 2 * kMat;   // oY: end of P and MX
    static constexpr size_t kTb = (size_t)C * LD_CT * sizeof(T);
    static constexpr size_t kVT = (size_t)kDvMax * LD_CT * sizeof(T);
    static constexpr size_t oVT = kMat;                       // over MX once X is consumed
    static constexpr size_t oTb = a16(cmax(oY, oVT + kVT));
    static constexpr size_t oXD = a16(oTb + kTb);            // [NB][16][16] fp32 diagonal blocks of X
    static constexpr size_t kXD = (size_t)NB * 256 * 4;
    static constexpr size_t kR1 = a16(cmax(cmax(kSeg, 3 * kTile), cmax(oXD + kXD, oVT + kVT)));
    static constexpr size_t kKtT = (size_t)DK * LD_CT * sizeof(T);
    // small: beta, block exponents at first / last token, pair factors, range flag
    static constexpr size_t kSmall = (size_t)C * 4 + 2ull * NB * DK * 4 + (size_t)(NOFF > 0 ? NOFF : 1) * DK * 4 + 16 +
                                     2ull * C * 4;
    static constexpr size_t kLds = kR1 + kKtT + kSmall;
    static constexpr bool kFits = kLds <= 163840;
    static constexpr int kMinBlocks = kLds <= 81920 ? 2 : 1;
};

// Input modes of the intra-chunk kernel; each is its own instance, so a
// plain call runs none of the option code (the first build with the options
// compiled into every call cost 24 VGPRs and 6 %).
enum InMode {
    kInPlain = 0,    // alpha per key channel as given
    kInOpts = 1,     // per-channel alpha; floor and fused transforms at run time
    kInFloor = 2,    // per-channel alpha floored at >= 2^-0.75 (no other option)
    kInScalar = 3,   // one alpha per (token, head); floor and fused transforms at run time
};
// A decay floor of at least 2^-0.75 bounds the decay of a 16-token block by
// 2^-12 in every channel, which is the factored Gram path's range: the
// floored instance needs neither the per-chunk range check nor the exact path.
constexpr float kFloorFast = 0.59460356f;   // 2^-0.75

template <int DK, int C, typename In, int kIn>
__global__ __launch_bounds__(256, (Intra<DK, C, typename OperandOf<In>::type>::kMinBlocks))
void kda_intra_kernel(const PrefillArgs a) {
    // kOpts: floor and fused transforms applied at run time; kScalar: one decay
    // per token (the Gram is plain Q K^T and K K^T with a rank-1 decay mask);
    // kSureFast: every chunk takes the factored / masked Gram
    constexpr bool kOpts = kIn == kInOpts || kIn == kInScalar;
    constexpr bool kScalar = kIn == kInScalar;
    constexpr bool kSureFast = kIn == kInFloor || kIn == kInScalar;
    using T = typename OperandOf<In>::type;
    using I = Intra<DK, C, T>;
    static_assert(I::kFits, "LDS budget of one gfx950 workgroup exceeded");
    static_assert(I::NSEG * I::NCG <= I::kThreads, "thread mapping");
    using Q = quad_t<T>;
    constexpr int NB = I::NB, NQK = I::NQK, LD_ROW = I::LD_ROW, LD_CT = I::LD_CT, LD_F = I::LD_F;
    __shared__ __attribute__((aligned(16))) char smem[I::kLds];
    T* Ak = reinterpret_cast<T*>(smem);                       // [C][LD_ROW]  row side, k
    T* Aq = Ak + C * LD_ROW;                                  // [C][LD_ROW]  row side, q
    T* Bd = Aq + C * LD_ROW;                                  // [C][LD_ROW]  column side
    float* Pm = reinterpret_cast<float*>(smem + I::oP);      // [C][LD_F]  P (lower)
    float* MX = reinterpret_cast<float*>(smem + I::oMX);     // [C][LD_F]  M strictly lower, X^T strictly upper
    float* XD = reinterpret_cast<float*>(smem + I::oXD);     // [NB][16][16] X_RR, row-major
    T* Tb = reinterpret_cast<T*>(smem + I::oTb);             // [C][LD_CT] Tm = X diag(beta)
    T* VT = reinterpret_cast<T*>(smem + I::oVT);             // [DV][LD_CT] V^T
    T* KtT = reinterpret_cast<T*>(smem + I::kR1);            // [DK][LD_CT] Ktilde^T
    float* sbeta = reinterpret_cast<float*>(smem + I::kR1 + I::kKtT);
    float* Gs = sbeta + C;                      // [NB][DK] exponent at each block's first token
    float* Ge = Gs + NB * DK;                   // [NB][DK] exponent at each block's last token
    float* sIR = Ge + NB * DK;                  // [NOFF][DK] pair factors 2^{G_R - G_I + h_I - h_R}
    float* swmax = sIR + (I::NOFF > 0 ? I::NOFF : 1) * DK;   // [4] largest block decay range per wave
    float* sinv = swmax + 4;                                  // [2][C] inverse norms of q and k (fused inputs)

    const int tid = threadIdx.x;
    const int lane = tid & 63, g = lane >> 4, cl = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // one-dimensional grid, heads fastest: the workgroups in flight read
    // neighbouring rows of q, k, v, alpha and write neighbouring blocks
    // (1.365 ms against 1.448 ms per launch with chunks fastest on the
    // long-context workload)
    const int x = (int)(blockIdx.x / (unsigned)a.H), h = (int)(blockIdx.x % (unsigned)a.H);
    // the call's range status starts clear; the inter-chunk kernel, which runs
    // after this one on the stream, may set it.  Fixed-length calls have no
    // cu_seqlens to check: their layout status is clear too (packed calls have
    // theirs from the chunk-offset kernel).
    if (blockIdx.x == 0 && tid == 0) {
        a.status[0] = 0;
        if (!a.cu_seqlens) a.status[kLayoutWord] = 0;
    }
    ChunkPos pos;
    if (!locate_chunk(a, C, x, pos)) return;  // uniform over the workgroup
    const int valid = pos.valid;
    const int H = a.H, DV = a.DV;
    const In* __restrict__ qg = reinterpret_cast<const In*>(a.q);
    const In* __restrict__ kg = reinterpret_cast<const In*>(a.k);
    const In* __restrict__ vg = reinterpret_cast<const In*>(a.v);

    const ChunkBlock<T> cb(DK, C, DV, a.gsl);
    char* blk = a.ws_chunks + ((int64_t)x * H + h) * cb.bytes;
    T* Wf = reinterpret_cast<T*>(blk + cb.w);
    T* Qf = reinterpret_cast<T*>(blk + cb.q);
    T* Kbf = reinterpret_cast<T*>(blk + cb.kb);
    T* Pf = reinterpret_cast<T*>(blk + cb.p);
    float* gam = reinterpret_cast<float*>(blk + cb.gam);

    // ---- phase 1: every global load first ------------------------------------
    // thread -> 8 channels (group cg) x 4 consecutive tokens (segment sgi, block
    // Rb = sgi/4).  The NSEG segments of a channel group are adjacent lanes of
    // one wave: the prefix over segments is a shuffle scan, and the transposed
    // tile stores below (4 tokens of one channel per lane) land in consecutive
    // quads of a row instead of 8-way bank conflicts.
    const bool p1 = tid < I::NSEG * I::NCG;
    const int cg = tid / I::NSEG, sgi = tid % I::NSEG, Rb = sgi >> 2, sp = sgi & 3;
    const int NCGV = DV / 8;
    const bool pv = tid < I::NSEG * NCGV;
    const int cgv = tid / I::NSEG, sgv = tid % I::NSEG;
    // All loads go out before any is used: tokens past the chunk's end (and
    // threads outside the mapping) read an in-bounds row (the chunk's first
    // token, channel group 0) and are masked after the loads land.
    // beta of token tid goes out with the other inputs (a row past the chunk's
    // end reads its first token and is masked where sbeta is written)
    const float braw = a.beta[(pos.tok0 + (tid < valid ? tid : 0)) * H + h];
    float kr[4][8], qr[4][8], al[4][8];
    Raw8<In> vraw[4];   // v as loaded; converted where V^T is staged
    {
        Raw8<In> kraw[4], qraw[4];
        Raw8<float> araw[4];
        float ascal[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = 4 * sgi + u;
            const bool ok = p1 && r < valid;
            const int64_t row = (pos.tok0 + (ok ? r : 0)) * H + h;
            const int64_t base = row * DK + 8 * (p1 ? cg : 0);
            kraw[u].load(kg + base);
            qraw[u].load(qg + base);
            if constexpr (kScalar) ascal[u] = a.alpha[row];
            else araw[u].load(a.alpha + base);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bool ok = p1 && 4 * sgi + u < valid;
            kraw[u].unpack(kr[u]);
            qraw[u].unpack(qr[u]);
            if constexpr (kScalar) {
                // one decay for the token, formed once and shared by the channels
                float as = ascal[u];
                if (a.fuse_inputs) as = sigmoid(as);
                as = fmaxf(as, a.alpha_floor);
#pragma unroll
                for (int e = 0; e < 8; ++e) al[u][e] = as;
            } else {
                araw[u].unpack(al[u]);
                if (kOpts && a.fuse_inputs) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) al[u][e] = sigmoid(al[u][e]);
                }
                if (kIn != kInPlain) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) al[u][e] = fmaxf(al[u][e], a.alpha_floor);
                }
            }
            if (!p1 || valid < C) {   // a partial chunk's tail, threads outside the mapping
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    kr[u][e] = ok ? kr[u][e] : 0.f;
                    qr[u][e] = ok ? qr[u][e] : 0.f;
                    al[u][e] = ok ? al[u][e] : 1.f;
                }
            }
        }
    }
    // v is needed only once the solve is done: its loads go out after the Gram
    // phase so that they do not queue behind the factor inputs
    auto load_v = [&]() {
#pragma unroll
        for (int u = 0; u < 4; ++u) {   // masked where V^T is staged
            const bool ok = pv && 4 * sgv + u < valid;
            vraw[u].load(vg + ((pos.tok0 + (ok ? 4 * sgv + u : 0)) * H + h) * DV + 8 * (pv ? cgv : 0));
        }
    };
    if (kOpts && a.fuse_inputs) {
        // L2 norm of q and k per token.  The channel groups of a token are the
        // lanes sgi + NSEG * cg, spread over up to four waves: reduce inside
        // each wave, then add the waves' partial sums in a fixed order.
        constexpr int kGroupsPerWave = 64 / I::NSEG;
        constexpr int kWaves = (I::NCG + kGroupsPerWave - 1) / kGroupsPerWave;
        float* pnorm = reinterpret_cast<float*>(smem);   // [kWaves][2][C], free until the tiles are written
        float nq4[4], nk4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float nq = 0.f, nk = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                nq += qr[u][e] * qr[u][e];
                nk += kr[u][e] * kr[u][e];
            }
#pragma unroll
            for (int m = I::NSEG; m < 64; m <<= 1) {
                nq += __shfl_xor(nq, m, 64);
                nk += __shfl_xor(nk, m, 64);
            }
            nq4[u] = nq;
            nk4[u] = nk;
        }
        if (p1 && cg % kGroupsPerWave == 0) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                pnorm[(wave * 2 + 0) * C + 4 * sgi + u] = nq4[u];
                pnorm[(wave * 2 + 1) * C + 4 * sgi + u] = nk4[u];
            }
        }
        lds_barrier();
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float nq = 0.f, nk = 0.f;
            for (int w2 = 0; w2 < kWaves; ++w2) {
                nq += pnorm[(w2 * 2 + 0) * C + 4 * sgi + u];
                nk += pnorm[(w2 * 2 + 1) * C + 4 * sgi + u];
            }
            const float iq = 1.f / fmaxf(sqrtf(nq), 1e-12f), ik = 1.f / fmaxf(sqrtf(nk), 1e-12f);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                qr[u][e] *= iq;
                kr[u][e] *= ik;
            }
            if (p1 && cg == 0) {
                sinv[4 * sgi + u] = iq;
                sinv[C + 4 * sgi + u] = ik;
            }
        }
    }
    if (tid < C) {
        float b = tid < valid ? braw : 0.f;
        if (kOpts && a.fuse_inputs && tid < valid) b = sigmoid(b);
        sbeta[tid] = b;
    }

    // segment sums of log2 alpha (floored), then the exclusive prefix over the
    // segments of the channel group (a shuffle scan over NSEG adjacent lanes)
    float lg[4][8];  // inclusive running sum inside the segment
    float off[8], tot[8];
    if constexpr (kScalar) {
        // one exponent per token: a single scan, shared by the 8 channels
        float run = 0.f, lgs[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            run += fmaxf(__builtin_amdgcn_logf(al[u][0]), kLog2Floor);
            lgs[u] = run;
        }
        float incl = run;
        if constexpr (I::NSEG == 16) {
            incl = row_scan16(incl);
        } else {
#pragma unroll
            for (int d = 1; d < I::NSEG; d <<= 1) {
                const float t = __shfl_up(incl, d, I::NSEG);
                if (sgi >= d) incl += t;
            }
        }
        const float offs = incl - run, tots = __shfl(incl, I::NSEG - 1, I::NSEG);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            off[e] = offs;
            tot[e] = tots;
#pragma unroll
            for (int u = 0; u < 4; ++u) lg[u][e] = lgs[u];
        }
        // the token exponents g_r, for the decay mask of the Gram (the block
        // exponent region is not used by this instance)
        if (p1 && cg == 0) {
#pragma unroll
            for (int u = 0; u < 4; ++u) Gs[4 * sgi + u] = offs + lgs[u];
        }
    } else {
        float run[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) run[e] = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                run[e] += fmaxf(__builtin_amdgcn_logf(al[u][e]), kLog2Floor);
                lg[u][e] = run[e];
            }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float incl = run[e];
            if constexpr (I::NSEG == 16) {   // a channel group is one DPP row
                incl = row_scan16(incl);
            } else {
#pragma unroll
                for (int d = 1; d < I::NSEG; d <<= 1) {
                    const float t = __shfl_up(incl, d, I::NSEG);
                    if (sgi >= d) incl += t;
                }
            }
            off[e] = incl - run[e];
            tot[e] = __shfl(incl, I::NSEG - 1, I::NSEG);
        }
    }
    if (!kScalar && p1 && sp == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) Gs[Rb * DK + 8 * cg + e] = off[e] + lg[0][e];
    }
    if (!kScalar && p1 && sp == 3) {
#pragma unroll
        for (int e = 0; e < 8; ++e) Ge[Rb * DK + 8 * cg + e] = off[e] + lg[3][e];
    }
    if constexpr (!kSureFast) {
        // decay range of each 16-token block (exponent at its first token minus
        // at its last), maximised over the wave's blocks and channels; the last
        // segment of a block is 3 lanes above its first
        // (lanes with sp == 0 count, by an arithmetic mask rather than a branch,
        // which would mask off the lanes the row_shl:3 move reads)
        float mx = 0.f;
        const float first = fmaxf(1.f - (float)sp, 0.f);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float ge = dpp<0x103>(off[e] + lg[3][e]);   // row_shl:3, 3 lanes above
            mx = fmaxf(mx, (off[e] + lg[0][e] - ge) * first);
        }
        // in-row maxima (row_shr, lanes below a row's start read 0 <= mx), then
        // the four rows' last lanes
        mx = fmaxf(mx, dpp<0x111>(mx));
        mx = fmaxf(mx, dpp<0x112>(mx));
        mx = fmaxf(mx, dpp<0x114>(mx));
        mx = fmaxf(mx, dpp<0x118>(mx));
        mx = fmaxf(fmaxf(lane_value(mx, 15), lane_value(mx, 31)), fmaxf(lane_value(mx, 47), lane_value(mx, 63)));
        if (lane == 0) swmax[wave] = mx;
    }
    lds_barrier();
    const bool fast = kSureFast || fmaxf(fmaxf(swmax[0], swmax[1]), fmaxf(swmax[2], swmax[3])) <= kFastRange;

    // ---- phase 1 (cont.): operand factors, tiles and the workspace quads ----
    if (!kScalar && fast && p1 && sp < Rb) {
        // pair factors 2^{G_R - G_I + h_I - h_R} (<= 1) of the off-diagonal tiles (R = Rb, I = sp)
        const int Ib = sp;
        float* dst = sIR + (Rb * (Rb - 1) / 2 + Ib) * DK + 8 * cg;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int c = 8 * cg + e;
            const float hR = 0.5f * (Gs[Rb * DK + c] - Ge[Rb * DK + c]);
            const float hI = 0.5f * (Gs[Ib * DK + c] - Ge[Ib * DK + c]);
            dst[e] = __builtin_amdgcn_exp2f(fminf(Gs[Rb * DK + c] - Gs[Ib * DK + c] + hI - hR, 0.f));
        }
    }
    // The factor loops are instantiated once per path (fast is uniform over the
    // workgroup): a per-element choice was if-converted, so both paths' exp2
    // and products ran for every element.
    auto factor_phase = [&](auto path) {
        constexpr bool fast = decltype(path)::value;
        // fast path, per channel of block R: the row factor fa = 2^{g_r - G_R + h_R}
        // runs as a product of alpha from pre; Ktilde and Qtilde are the row-side
        // operands times cq = 2^{G_R - h_R}, and Kbar = k 2^{g_C - g_r} is the
        // column-side operand times dq = 2^{g_C - G_R + h_R}
        float sh[8], cq[8], pre[8], dq[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int c = 8 * cg + e;
            const float G0 = Gs[Rb * DK + c];
            const float hR = 0.5f * (G0 - Ge[Rb * DK + c]);
            sh[e] = __builtin_amdgcn_exp2f(fminf(hR, 30.f));          // 2^{h_R}
            cq[e] = __builtin_amdgcn_exp2f(G0 - hR);                   // 2^{G_R - h_R}
            pre[e] = sp == 0 ? 1.f : __builtin_amdgcn_exp2f(off[e] - G0);  // decay from the block's first token
            dq[e] = __builtin_amdgcn_exp2f(fminf(tot[e] - G0 + hR, 30.f));  // 2^{g_C - G_R + h_R}
        }
        // Kbar quads (4 tokens of a channel); the exact path forms them here, the
        // fast path in the forward pass below
        const int ut = sgi >> 2, gq = sgi & 3;
        f32x4 kbq[8];
        if constexpr (!fast) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    kbq[e][u] = kr[u][e] * __builtin_amdgcn_exp2f(fminf(tot[e] - (off[e] + lg[u][e]), 0.f));
        }
        // forward pass: prefix products give the row / column factors and 2^{g_r}
        float ktil[4][8];
        float pr[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pr[e] = pre[e];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = 4 * sgi + u;
            float ak[8], aq[8], bd[8], qt[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if (fast) {
                    if (!(sp == 0 && u == 0)) pr[e] *= al[u][e];   // 2^{g_r - G_R}
                    const float fa = pr[e] * sh[e];                // in 2^[-h, h]
                    const float fb = __builtin_amdgcn_rcpf(fa);
                    ak[e] = kr[u][e] * fa;
                    aq[e] = qr[u][e] * fa;
                    bd[e] = kr[u][e] * fb;
                    kbq[e][u] = bd[e] * dq[e];                     // k 2^{g_C - g_r}
                    ktil[u][e] = ak[e] * cq[e];                    // k 2^{g_r}
                    qt[e] = aq[e] * cq[e];
                } else {
                    const float gm = __builtin_amdgcn_exp2f(off[e] + lg[u][e]);   // 2^{g_r}
                    ktil[u][e] = kr[u][e] * gm;
                    qt[e] = qr[u][e] * gm;
                }
            }
            if (fast) {
                store8(Ak + r * LD_ROW + 8 * cg, ak);
                store8(Aq + r * LD_ROW + 8 * cg, aq);
                store8(Bd + r * LD_ROW + 8 * cg, bd);
            } else if (kScalar) {
                // one decay per token: the Gram operands are k and q as they are
                // (the decay enters as a mask on the fp32 products)
                store8(Ak + r * LD_ROW + 8 * cg, kr[u]);
                store8(Aq + r * LD_ROW + 8 * cg, qr[u]);
            }
            if constexpr (sizeof(T) == 2 && I::NSEG == 16 && I::NCG % 4 == 0) {
                // (four channel groups per wave, so every lane has its partner)
                // Qtilde quads of token r, channel groups 2cg and 2cg + 1.  A fragment
                // lane's 16 bytes hold the quads of groups a4 and a4 + 4, i.e. of this
                // thread and the one 32 lanes away (channel group cg +- 2): the lower
                // lane writes the slot of its group 2cg, the upper lane that of 2cg + 1,
                // each taking the partner's quad from one permlane32 swap per dword.
                typedef int i32x2 __attribute__((ext_vector_type(2)));
                typedef int i32x4 __attribute__((ext_vector_type(4)));
                const bool upper = (cg & 2) != 0;
                const i32x2 h0 = __builtin_bit_cast(i32x2, make_quad<T>(f32x4{qt[0], qt[1], qt[2], qt[3]}));
                const i32x2 h1 = __builtin_bit_cast(i32x2, make_quad<T>(f32x4{qt[4], qt[5], qt[6], qt[7]}));
                const auto s0 = __builtin_amdgcn_permlane32_swap(h0[0], h1[0], false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(h0[1], h1[1], false, false);
                // lower lanes: s*[1] is the upper partner's group-2cg quad; upper lanes:
                // s*[0] is the lower partner's group-(2cg + 1) quad
                const i32x4 v = upper ? i32x4{(int)s0[0], (int)s1[0], h1[0], h1[1]}
                                      : i32x4{h0[0], h0[1], (int)s0[1], (int)s1[1]};
                const int a4 = 2 * (upper ? cg - 2 : cg) + (upper ? 1 : 0);   // the slot's even group
                *reinterpret_cast<i32x4*>(Qf + Frag<T>::off(r >> 4, a4 >> 2, 16 * (a4 & 3) + (r & 15), DK)) = v;
            } else {
#pragma unroll
                for (int hq = 0; hq < 2; ++hq) {  // Qtilde quads: token r, channel groups 2cg, 2cg+1
                    const int a4 = 2 * cg + hq, ut = a4 >> 2, gq = a4 & 3;
                    store_q<T>(Qf + Frag<T>::off(r >> 4, ut, 16 * gq + (r & 15), DK),
                               f32x4{qt[4 * hq], qt[4 * hq + 1], qt[4 * hq + 2], qt[4 * hq + 3]});
                }
            }
        }
        if constexpr (sizeof(T) == 2 && I::NSEG == 16) {
            // Kbar to the workspace: a fragment lane's 16 bytes hold the token quads
            // ut and ut ^ 1 of one channel, which lie with this thread and the one 4
            // lanes away (same DPP row).  Per channel pair the even-ut thread writes
            // channel e0 and the odd-ut thread channel e1, each fetching the partner's
            // quad by DPP (moves unconditional, the choice by select).
            const bool odd = (ut & 1) != 0;
#pragma unroll
            for (int e0 = 0; e0 < 8; e0 += 2) {
                const Q q0 = make_quad<T>(kbq[e0]), q1 = make_quad<T>(kbq[e0 + 1]);
                typedef int i32x2 __attribute__((ext_vector_type(2)));
                const i32x2 w0 = __builtin_bit_cast(i32x2, q0), w1 = __builtin_bit_cast(i32x2, q1);
                i32x2 up, dn;   // partner's e0 quad (from 4 lanes above), e1 quad (from 4 below)
                up[0] = __builtin_amdgcn_update_dpp(0, w0[0], 0x104, 0xf, 0xf, true);
                up[1] = __builtin_amdgcn_update_dpp(0, w0[1], 0x104, 0xf, 0xf, true);
                dn[0] = __builtin_amdgcn_update_dpp(0, w1[0], 0x114, 0xf, 0xf, true);
                dn[1] = __builtin_amdgcn_update_dpp(0, w1[1], 0x114, 0xf, 0xf, true);
                typedef int i32x4 __attribute__((ext_vector_type(4)));
                const i32x4 v = odd ? i32x4{dn[0], dn[1], w1[0], w1[1]} : i32x4{w0[0], w0[1], up[0], up[1]};
                const int c = 8 * cg + e0 + (odd ? 1 : 0);
                *reinterpret_cast<i32x4*>(Kbf + Frag<T>::off(c >> 4, ut & ~1, 16 * gq + (c & 15), C)) = v;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int c = 8 * cg + e;
                store_q<T>(Kbf + Frag<T>::off(c >> 4, ut, 16 * gq + (c & 15), C), kbq[e]);
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)   // Ktilde^T: channel c, tokens 4*sgi .. +3
            store_q<T>(KtT + (8 * cg + e) * LD_CT + 4 * sgi, f32x4{ktil[0][e], ktil[1][e], ktil[2][e], ktil[3][e]});
        if (sgi == 0) {
            *reinterpret_cast<f32x4*>(gam + 8 * cg) =
                f32x4{__builtin_amdgcn_exp2f(tot[0]), __builtin_amdgcn_exp2f(tot[1]), __builtin_amdgcn_exp2f(tot[2]),
                      __builtin_amdgcn_exp2f(tot[3])};
            *reinterpret_cast<f32x4*>(gam + 8 * cg + 4) =
                f32x4{__builtin_amdgcn_exp2f(tot[4]), __builtin_amdgcn_exp2f(tot[5]), __builtin_amdgcn_exp2f(tot[6]),
                      __builtin_amdgcn_exp2f(tot[7])};
        }
    };
    if (p1) {
        // the scalar gate takes the per-token exponents of the exact path's
        // formulas (one exp2 per token: the channels share them) and the
        // plain operands
        if (kScalar) factor_phase(BoolTag<false>{});
        else if (fast) factor_phase(BoolTag<true>{});
        else factor_phase(BoolTag<false>{});
    }
    lds_barrier();

    // ---- phase 2: Gram matrices M (strictly lower) and P (lower) ------------
    if (fast) {
        // tile pairs (Ib, R), Ib <= R: M'^T(Ib,R) = Bcol_Ib Ak_R^T and P^T(Ib,R) = Bcol_Ib Aq_R^T
        constexpr int NP = NB * (NB + 1) / 2;
        constexpr int MAXP = (NP + 3) / 4;
        f32x4 mres[MAXP], pres[MAXP];
        int pI[MAXP], pR[MAXP];
#pragma unroll
        for (int pi = 0; pi < MAXP; ++pi) {
            const int p = wave + 4 * pi;
            int R = 0;
            while ((R + 1) * (R + 2) / 2 <= p) ++R;
            const int Ib = p - R * (R + 1) / 2;
            pI[pi] = Ib;
            pR[pi] = R;
            mres[pi] = zero4();
            pres[pi] = zero4();
            if (p < NP) {
                Q aq[NQK], bk[NQK], bq[NQK];
                if (kScalar) {   // plain k rows of block Ib
#pragma unroll
                    for (int u = 0; u < NQK; ++u)
                        aq[u] = *reinterpret_cast<const Q*>(Ak + (16 * Ib + cl) * LD_ROW + 16 * u + 4 * g);
                } else if (Ib == R) {
#pragma unroll
                    for (int u = 0; u < NQK; ++u)
                        aq[u] = *reinterpret_cast<const Q*>(Bd + (16 * Ib + cl) * LD_ROW + 16 * u + 4 * g);
                } else {
                    const float* sp4 = sIR + (R * (R - 1) / 2 + Ib) * DK;
#pragma unroll
                    for (int u = 0; u < NQK; ++u) {
                        const f32x4 b4 = from_quad(*reinterpret_cast<const Q*>(Bd + (16 * Ib + cl) * LD_ROW + 16 * u + 4 * g));
                        const f32x4 sf = *reinterpret_cast<const f32x4*>(sp4 + 16 * u + 4 * g);
                        aq[u] = make_quad<T>(b4 * sf);
                    }
                }
#pragma unroll
                for (int u = 0; u < NQK; ++u) {
                    bk[u] = *reinterpret_cast<const Q*>(Ak + (16 * R + cl) * LD_ROW + 16 * u + 4 * g);
                    bq[u] = *reinterpret_cast<const Q*>(Aq + (16 * R + cl) * LD_ROW + 16 * u + 4 * g);
                }
                // the M and P chains share A and are issued alternately
                mma_quads_pair(aq, bk, bq, mres[pi], pres[pi]);
            }
        }
        lds_barrier();  // the operand tiles are dead from here on
#pragma unroll
        for (int pi = 0; pi < MAXP; ++pi) {
            const int p = wave + 4 * pi;
            if (p < NP) {
                // lane holds M'^T[i = 16Ib + 4g + j][r = 16R + cl] for j = 0..3
                const int r = 16 * pR[pi] + cl, i0 = 16 * pI[pi] + 4 * g;
                const float br = sbeta[r];
                if constexpr (kScalar) {
                    // rank-1 decay mask 2^{g_r - g_i} (<= 1 where i <= r); Gs holds
                    // the token exponents in this instance
                    const float gr = Gs[r];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float dm = __builtin_amdgcn_exp2f(fminf(gr - Gs[i0 + j], 0.f));
                        mres[pi][j] *= dm;
                        pres[pi][j] *= dm;
                    }
                }
                // the accumulator is P's fragment (row tile R, quad Ib) as the
                // workspace stores it: it goes out from here
                if (pI[pi] < pR[pi]) {
                    *reinterpret_cast<f32x4*>(MX + r * LD_F + i0) = br * mres[pi];
                } else {   // diagonal tile: keep the strictly lower (M) / lower (P) part
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if (i0 + j < r) MX[r * LD_F + i0 + j] = br * mres[pi][j];
                        if (i0 + j > r) pres[pi][j] = 0.f;
                    }
                }
                *reinterpret_cast<Q*>(Pf + Frag<T>::off(pR[pi], pI[pi], lane, C)) = make_quad<T>(pres[pi]);
            }
        }
    } else {
        // exact pairwise path: decay products taken in linear space
        for (int e = tid; e < 2 * C * LD_F; e += I::kThreads) Pm[e] = 0.f;  // P and MX
        lds_barrier();
        constexpr int PARTS = I::kThreads / C;
        constexpr int CPP = DK / PARTS;
        const int i = tid % C, part = tid / C, c0 = part * CPP;
        if (i < valid) {
            float ki[CPP], prd[CPP];
            const int64_t bi = ((pos.tok0 + i) * H + h) * DK + c0;
            const float iki = kOpts && a.fuse_inputs ? sinv[C + i] : 1.f;
#pragma unroll
            for (int c = 0; c < CPP; ++c) { ki[c] = iki * load_as_float(kg, bi + c); prd[c] = 1.f; }
            for (int r = i; r < valid; ++r) {
                const int64_t br = ((pos.tok0 + r) * H + h) * DK + c0;
                float m = 0.f, pp = 0.f;
#pragma unroll
                for (int c = 0; c < CPP; ++c) {
                    if (r > i) prd[c] *= kOpts ? alpha_at(a, pos.tok0 + r, h, DK, c0 + c) : a.alpha[br + c];
                    const float w = ki[c] * prd[c];
                    m += load_as_float(kg, br + c) * w;
                    pp += load_as_float(qg, br + c) * w;
                }
                if (kOpts && a.fuse_inputs) {
                    m *= sinv[C + r];
                    pp *= sinv[r];
                }
                if (r > i) atomicAdd(&MX[r * LD_F + i], sbeta[r] * m);
                atomicAdd(&Pm[r * LD_F + i], pp);
            }
        }
    }
    lds_barrier();

    load_v();

    // ---- phase 3: X = (I + M)^{-1}; X^T kept in the strictly upper part of MX
    if (tid < C) {  // diagonal blocks by forward substitution, one column each
        const int R = tid >> 4, ci = tid & 15, b0 = 16 * R;
        float xv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) xv[r] = (r == ci) ? 1.f : 0.f;
#pragma unroll
        for (int r = 1; r < 16; ++r) {
            const float* mrow = MX + (b0 + r) * LD_F + b0;
            float s = 0.f;
#pragma unroll
            for (int j4 = 0; j4 < r; j4 += 4) {
                const f32x4 m4 = *reinterpret_cast<const f32x4*>(mrow + j4);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    if (j4 + jj < r) s += m4[jj] * xv[j4 + jj];
            }
            if (r > ci) xv[r] = -s;
        }
        const float bc = sbeta[b0 + ci];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            XD[R * 256 + r * 16 + ci] = xv[r];                        // X_RR[r][ci], row-major
            if (r > ci) MX[(b0 + ci) * LD_F + b0 + r] = xv[r];       // X[b0+r][b0+ci], transposed
            Tb[(b0 + r) * LD_CT + b0 + ci] = (T)(xv[r] * bc);         // Tm = X diag(beta)
        }
    } else if (tid >= 64) {
        // meanwhile the other waves write the zero tiles above the diagonal: Tm's
        // (the solve writes the others; the Gram operands are dead) and, on the
        // fast path, P's in the workspace (the exact path converts all of P later)
        auto above = [](int q, int& Rt, int& It) {   // q-th tile (Rt < It) above the diagonal, by columns
            int R = 0;
            while ((R + 1) * (R + 2) / 2 <= q) ++R;
            Rt = q - R * (R + 1) / 2;
            It = R + 1;
        };
        for (int e = tid - 64; e < I::NOFF * 64; e += I::kThreads - 64) {
            int Rt, It;
            above(e >> 6, Rt, It);
            store_q<T>(Tb + (16 * Rt + ((e >> 2) & 15)) * LD_CT + 16 * It + 4 * (e & 3), zero4());
        }
        if (kSureFast || fast) {
            for (int q = wave - 1; q < I::NOFF; q += 3) {
                int Rt, It;
                above(q, Rt, It);
                *reinterpret_cast<Q*>(Pf + Frag<T>::off(Rt, It, lane, C)) = make_quad<T>(zero4());
            }
        }
    }
    lds_barrier();
    // Off-diagonal blocks, one block pair (R, Ib = R - d) per wave, on fp32 MFMA:
    //   Y = sum_{J=Ib}^{R-1} M_RJ X_JIb ;  X_RIb^T = -(Y^T X_RR^T)
    // Y's accumulator is already Y^T in operand layout (lane: row ii = cl,
    // quad over j = 4g..4g+3), so it feeds the second product directly.
    for (int d = 1; d < NB; ++d) {
        if (wave < NB - d) {
            const int Ib = wave, R = Ib + d;
            const int rowX = 16 * Ib + cl;                   // row of X^T = column of X
            f32x4 y = zero4();
            for (int J = Ib; J < R; ++J) {
                const f32x4 m4 = *reinterpret_cast<const f32x4*>(MX + (16 * R + cl) * LD_F + 16 * J + 4 * g);
                f32x4 x4 = *reinterpret_cast<const f32x4*>(MX + rowX * LD_F + 16 * J + 4 * g);
                if (J == Ib) {   // diagonal block: X[j][ii] is 1 at j == ii, 0 above it
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int j = 4 * g + jj;
                        x4[jj] = j == cl ? 1.f : (j > cl ? x4[jj] : 0.f);
                    }
                }
                // A = M_RJ (lane row cl), B = X_JIb (lane column cl): both quads over j
                y = mma_step(m4, x4, y);
            }
            // Z^T = Y^T X_RR^T: A = Y^T (lane row ii = cl; the C layout of y), B = X_RR^T (lane column rr = cl)
            const f32x4 yt = f32x4{y[0], y[1], y[2], y[3]};
            const f32x4 xr = *reinterpret_cast<const f32x4*>(XD + R * 256 + cl * 16 + 4 * g);  // X_RR[rr=cl][4g..]
            const f32x4 z = mma_step(yt, xr, zero4());
            // lane holds Z^T[ii = 4g + j][rr = cl]; X_RIb^T[ii][rr] = -Z^T[ii][rr]
            f32x4 t4;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                MX[(16 * Ib + 4 * g + jj) * LD_F + 16 * R + cl] = -z[jj];
                t4[jj] = -z[jj] * sbeta[16 * Ib + 4 * g + jj];
            }
            store_q<T>(Tb + (16 * R + cl) * LD_CT + 16 * Ib + 4 * g, t4);   // Tm row 16R + cl
        }
        lds_barrier();
    }

    // ---- phase 4: value tile, P fragments, W = Tm Ktilde, Utilde = Tm V ------
    if (pv) {
        float vr[4][8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            vraw[u].unpack(vr[u]);
            if (4 * sgv + u >= valid) {
#pragma unroll
                for (int e = 0; e < 8; ++e) vr[u][e] = 0.f;
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
            store_q<T>(VT + (8 * cgv + e) * LD_CT + 4 * sgv, f32x4{vr[0][e], vr[1][e], vr[2][e], vr[3][e]});
    }
    if (kSureFast || fast) {
        // P went out from the Gram accumulators
    } else if constexpr (sizeof(T) == 2 && NB % 2 == 0) {   // both quads of a 16-byte slot per thread
        for (int e = tid; e < NB * (NB / 2) * 64; e += I::kThreads) {
            const int ct = e / (NB / 2 * 64), ut = 2 * ((e / 64) % (NB / 2)), ln = e & 63;
            const int r = 16 * ct + (ln & 15), i0 = 16 * ut + 4 * (ln >> 4);
            const f32x4 va = ut <= ct ? *reinterpret_cast<const f32x4*>(Pm + r * LD_F + i0) : zero4();
            const f32x4 vb = ut + 1 <= ct ? *reinterpret_cast<const f32x4*>(Pm + r * LD_F + i0 + 16) : zero4();
            store_pair(reinterpret_cast<_Float16*>(Pf) + Frag<T>::off(ct, ut, ln, C), va, vb);
        }
    } else {
        for (int e = tid; e < NB * NB * 64; e += I::kThreads) {
            const int ct = e / (NB * 64), ut = (e / 64) % NB, ln = e & 63;
            const int r = 16 * ct + (ln & 15), i0 = 16 * ut + 4 * (ln >> 4);
            const f32x4 v4 = ut <= ct ? *reinterpret_cast<const f32x4*>(Pm + r * LD_F + i0) : zero4();
            *reinterpret_cast<Q*>(Pf + Frag<T>::off(ct, ut, ln, C)) = make_quad<T>(v4);
        }
    }
    lds_barrier();
    // W^T(channel tile t, token tile tb) = Ktilde^T Tm^T: lane holds W[16tb+cl][16t+4g+j].
    // The waves take every fourth tile and 4 is a multiple of NB, so a wave's
    // token tile tb is fixed: its Tm rows are read from LDS once.
    {
        const int tb = wave % NB;
        Q bq[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) bq[u] = *reinterpret_cast<const Q*>(Tb + (16 * tb + cl) * LD_CT + 16 * u + 4 * g);
#pragma unroll 1
        for (int t = wave / NB; t < NQK; t += 4 / NB) {
            Q aq[NB];
#pragma unroll
            for (int u = 0; u < NB; ++u) aq[u] = *reinterpret_cast<const Q*>(KtT + (16 * t + cl) * LD_CT + 16 * u + 4 * g);
            const f32x4 res = mma_quads_upto(aq, bq, tb, zero4());
            *reinterpret_cast<Q*>(Wf + Frag<T>::off(tb, t, lane, DK)) = make_quad<T>(res);
        }
    }
    // Utilde(token tile tb, value tile s) = Tm V: lane holds U[16tb+4g+j][16s+cl].
    // A wave owns value tiles s = wave, wave + 4 (V^T rows read once) and walks
    // the token tiles (Tm rows read once per tile).
    {
        const int NSV = DV / 16;
        constexpr int kSW = (I::kDvMax / 16 + 3) / 4;   // value tiles per wave
        Q vq[kSW][NB];
#pragma unroll
        for (int j = 0; j < kSW; ++j) {
            const int sv = min(wave + 4 * j, NSV - 1);   // in bounds; unused past NSV
#pragma unroll
            for (int u = 0; u < NB; ++u) vq[j][u] = *reinterpret_cast<const Q*>(VT + (16 * sv + cl) * LD_CT + 16 * u + 4 * g);
        }
#pragma unroll 1
        for (int tb = 0; tb < NB; ++tb) {
            Q aq[NB];
#pragma unroll
            for (int u = 0; u < NB; ++u) aq[u] = *reinterpret_cast<const Q*>(Tb + (16 * tb + cl) * LD_CT + 16 * u + 4 * g);
#pragma unroll
            for (int j = 0; j < kSW; ++j) {
                const int sv = wave + 4 * j;
                if (sv < NSV) {
                    const f32x4 res = mma_quads_upto(aq, vq[j], tb, zero4());
                    T* Us = reinterpret_cast<T*>(blk + cb.u_slice(sv));
                    *reinterpret_cast<Q*>(Us + (lane * NB + tb) * 4) = make_quad<T>(res);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// K2: inter-chunk pass.  One workgroup per (sequence, head, group of up to 4
// value slices of 16 columns):
//   waves 0 .. ncw-1  compute: each holds its dk x 16 slice of S in MFMA
//                     accumulator registers (fp32) and walks the chunks;
//   waves ncw ..      I/O (kIoWaves of them): copy the next chunk's block from
//                     the workspace into the other half of a double-buffered
//                     LDS ring with direct-to-LDS loads, so compute waves only
//                     read LDS and only write global memory (they never wait
//                     on a load);
// One s_barrier per chunk hands the ring over.  The slice groups of one
// (sequence, head) are placed on one XCD (blocks are dealt round-robin over
// the 8 XCDs) so the block is fetched from HBM once per XCD.
// Plain calls with one slice per workgroup split the compute over two waves
// instead: the state wave forms U and updates S (the serial chain), and an
// output wave forms the outputs of the previous chunk from the S and U the
// state wave left in LDS, so the chain no longer waits for the output tile.
// ---------------------------------------------------------------------------
// All N quads of row tile rt of a fragment matrix (K = 16 N), read as whole
// 16-byte vectors per lane.
template <int N>
__device__ __forceinline__ void load_frag(f16x4 (&q)[N], const char* base, int rt, int lane) {
    const _Float16* p = reinterpret_cast<const _Float16*>(base) + Frag<_Float16>::off(rt, 0, lane, 16 * N);
    constexpr int NG = (N + 1) / 2;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        const _Float16* pg = p + gi * 64 * 8;
        if (2 * gi + 1 < N) {
            const f16x8 v = *reinterpret_cast<const f16x8*>(pg);
            q[2 * gi] = __builtin_shufflevector(v, v, 0, 1, 2, 3);
            q[2 * gi + 1] = __builtin_shufflevector(v, v, 4, 5, 6, 7);
        } else {
            q[2 * gi] = *reinterpret_cast<const f16x4*>(pg);
        }
    }
}
template <int N>
__device__ __forceinline__ void load_frag(f32x4 (&q)[N], const char* base, int rt, int lane) {
    const float* p = reinterpret_cast<const float*>(base) + Frag<float>::off(rt, 0, lane, 16 * N);
#pragma unroll
    for (int u = 0; u < N; ++u) q[u] = *reinterpret_cast<const f32x4*>(p + u * 64 * 4);
}

// Whole-row workgroups (plain calls with at least as many (sequence, head)
// pairs as compute units or with chunk ranges, and gated calls there) keep all
// dv / 16 slices (8 at dv = 128) in one workgroup.  Each chunk's shared
// operands (W, Q~, Kbar^T, P) are then fetched once for the whole row instead
// of once per slice: a compute unit takes in about 26 bytes per cycle from L2,
// and a one-slice workgroup needs ~57 KiB of shared operands per chunk, which
// caps it near 1 us per chunk whatever the number of workgroups in flight.
// Plain workgroups run two slices per compute wave (8 waves: two per SIMD).
// Gated ones hold a chunk's outputs across the barrier that completes the
// row norm and run one slice per wave (12 waves): 2.33 against 2.64 ms with
// two for the gated long-context call (and 2.44 ms with two slices per wave
// forming the outputs twice, once for the row sums and once to store them),
// where the plain call is 0.6 % faster with two.
constexpr int kRowSlices = 8;
constexpr int kRowSlicesPerWave = 2;
constexpr int kGatedSlicesPerWave = 1;

// Waves per workgroup that copy chunk blocks into LDS (they split the 1 KiB
// units), both beside the compute waves of whole rows and beside the state
// and output waves of the one-slice form.  One-slice form on the long-context
// workload with the ring B wait deferred: 4 waves 1.036 ms, 6: 1.039, 8: 1.059
// (before the deferral 8 waves were best: 1.26 against 1.33 ms with 4).
constexpr int kIoWaves = 4;

template <int DK, int C, typename T, bool kWhole = false, bool kGated = false> struct Inter {
    static constexpr int G = kWhole ? kRowSlices : kGroupSlices;   // most slices per workgroup
    static constexpr int SPW = kWhole ? (kGated ? kGatedSlicesPerWave : kRowSlicesPerWave) : 1;
    static constexpr int kMaxCompute = (G + SPW - 1) / SPW;
    static constexpr int64_t kShared = (2 * Frag<T>::elems(C, DK) + Frag<T>::elems(DK, C) + Frag<T>::elems(C, C)) *
                                           (int64_t)sizeof(T) + round_kib(DK * 4);
    static constexpr int64_t kGroupMax = round_kib((int64_t)G * C * 16 * sizeof(T));
    static constexpr int64_t kBuf = kShared + kGroupMax;
    static constexpr int64_t kPart = kGated ? 2ll * kMaxCompute * C * 4 : 0;   // output-norm partial sums
    // Output-wave layout (one value slice per workgroup): ring A (W, Kbar^T,
    // gamma_C, the slice of U~) has two slots, ring B (Q~, P) three, since the
    // output wave reads a chunk one interval after the state wave; the state
    // wave hands S and U to it through two LDS slots in its own lane layout.
    static constexpr int64_t kSzW = Frag<T>::elems(C, DK) * (int64_t)sizeof(T);
    static constexpr int64_t kSzK = Frag<T>::elems(DK, C) * (int64_t)sizeof(T);
    static constexpr int64_t kSzP = Frag<T>::elems(C, C) * (int64_t)sizeof(T);
    static constexpr int64_t kSzG = round_kib(DK * 4);
    static constexpr int64_t kBufA = 2 * kSzW + kSzG + round_kib((int64_t)C * 16 * sizeof(T));
    static constexpr int64_t kBufB = kSzW + kSzP;
    static constexpr int64_t kHand = (int64_t)(DK / 16 + C / 16) * 64 * sizeof(quad_t<T>);
    static constexpr int64_t kOWaveLds = 2 * kBufA + 3 * kBufB + 2 * kHand;
    static constexpr bool kOWave = !kWhole && G == 1 && SPW == 1 && kSzW % 1024 == 0 &&
                                   kSzP % 1024 == 0 && kSzK == kSzW && kOWaveLds <= 163840;
    static constexpr int kComputeWaves = kOWave ? 2 : kMaxCompute;
    static constexpr int kIo = kIoWaves;
    // 1 KiB copies of ring B issued by each I/O wave per chunk (they are dealt
    // evenly only when the I/O waves divide them)
    static constexpr int kDeferB = (int)((kSzW + kSzP) / 1024 / kIo);
    static constexpr bool kDeferOk = (kSzW + kSzP) / 1024 % kIo == 0 && kDeferB + 1 <= 63;
    static constexpr int kThreads = 64 * (kComputeWaves + kIo);
    // one-dword L2 prefetch loads per I/O lane that cover a whole block
    static constexpr int kPfLoads = (int)((kShared + kGroupMax) / 128 + kIo * 64 - 1) / (kIo * 64);
    static constexpr int64_t kLds = kOWave ? kOWaveLds : 2 * kBuf;
    static constexpr bool kFits = kOWave || 2 * kBuf + kPart <= 163840;
};

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

// The I/O waves also pull the block kL2Ahead chunks past the one they copy
// into L2 (one-slice form on the long-context workload: 1 chunk 1.047 ms,
// 2: 1.056, 3: 1.077; without any prefetch the copies are exposed).  The
// ranged walk issues none: its blocks are its own and would not stay in L2.
constexpr int kL2Ahead = 1;

// Copy the 1 KiB units first, first + step, ... of `bytes` (a multiple of
// 1 KiB) from global to LDS, 16 bytes per lane per instruction.
__device__ __forceinline__ void dma_to_lds(const char* src, char* dst, int64_t bytes, int lane, int first, int step) {
    for (int64_t off = (int64_t)first * 1024; off < bytes; off += (int64_t)step * 1024)
        __builtin_amdgcn_global_load_lds((gbl_void_t*)(src + off + lane * 16), (lds_void_t*)(dst + off), 16, 0, 0);
}

// Output modes of the inter-chunk kernel.
enum OutMode { kOutPlain = 0, kOutGate = 1, kOutSplit = 2, kOutRow = 3 };

// kMode kOutPlain: one-slice workgroups, o stored per chunk; kOutGate: all
// slices of a row in this workgroup, norm and gate applied here; kOutSplit:
// one-slice workgroups write un-normalised fp32 outputs and per-slice sums of
// squares for the epilogue; kOutRow: all slices of a row in this workgroup, o
// stored per chunk.
template <int kMode> constexpr bool whole_row_mode() { return kMode == kOutGate || kMode == kOutRow; }

template <int DK, int C, typename In, int kMode>
__global__ __launch_bounds__((Inter<DK, C, typename OperandOf<In>::type, whole_row_mode<kMode>(),
                                   kMode == kOutGate>::kThreads))
void kda_inter_kernel(const PrefillArgs a) {
    constexpr bool kGate = kMode == kOutGate;
    using T = typename OperandOf<In>::type;
    using Q = quad_t<T>;
    using X = Inter<DK, C, T, whole_row_mode<kMode>(), kGate>;
    static_assert(X::kFits, "LDS ring of the inter-chunk kernel exceeds one workgroup");
    constexpr int NB = C / 16, NQK = DK / 16, SPW = X::SPW;
    __shared__ __attribute__((aligned(1024))) char ring[X::kLds];
    // target of the I/O waves' one-dword L2 prefetch loads (never read)
    __shared__ __attribute__((aligned(256))) int pf_sink[64];
    // per-token sums of squares of each compute wave's outputs (double-buffered
    // by chunk parity) for the output norm of gated calls
    __shared__ float part[kGate ? 2 : 1][kGate ? X::kMaxCompute : 1][kGate ? C : 1];

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, cl = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS targets go to M0
    const int H = a.H, DV = a.DV;
    const ChunkBlock<T> cb(DK, C, DV, a.gsl);
    const int ncw = (cb.gsl + SPW - 1) / SPW, ngroups = DV / 16 / cb.gsl;
    // blocks are dealt round-robin over the 8 XCDs: keep the slice groups of
    // one (sequence, head) on one XCD so they share its L2
    const int b = blockIdx.x, xcd = b & 7, jx = b >> 3;
    int grp = jx % ngroups;
    int unit = (jx / ngroups) * 8 + xcd;
    // chunk-range scan (whole-row calls with range_len > 0): workgroup b runs
    // range b / H of head b % H
    RangePos rp{};
    const bool ranged = whole_row_mode<kMode>() && a.range_len > 0;
    if (ranged) {
        grp = 0;
        if (!locate_range(a, b / H, rp)) return;   // whole workgroup
        unit = rp.n * H + b % H;
    } else if (unit >= a.N * a.H) {
        return;  // whole workgroup
    } else if (whole_row_mode<kMode>() && a.seq_order) {
        unit = a.seq_order[unit / H] * H + unit % H;   // longest sequences first
    }
    const int n = unit / H, h = unit % H, seq = n;

    int c_begin, c_end;
    int64_t tok_begin, seq_len;
    if (a.cu_seqlens) {
        c_begin = a.chunk_off[n];
        c_end = a.chunk_off[n + 1];
        tok_begin = a.cu_seqlens[n];
        seq_len = (int64_t)a.cu_seqlens[n + 1] - tok_begin;
    } else {
        c_begin = n * a.chunks_per_seq;
        c_end = c_begin + a.chunks_per_seq;
        tok_begin = (int64_t)n * a.T;
        seq_len = a.T;
    }
    // the chunks this workgroup walks, the state it starts from and whether it
    // ends the sequence (a range other than the last hands over to the next)
    const int cw_begin = ranged ? rp.c0 : c_begin, cw_end = ranged ? rp.c1 : c_end;
    const float* s_init = ranged && rp.r > 0 ? a.range_start + ((int64_t)(b / H) * H + h) * DK * DV
                          : a.s0 ? a.s0 + (int64_t)unit * DK * DV
                                 : nullptr;
    const bool ends_seq = !ranged || rp.r == rp.nr - 1;

    if constexpr (X::kOWave) {
        // ---- two compute waves: wave 0 walks the state chain, wave 1 forms the
        // outputs of the chunk before; waves 2.. are I/O waves.  Interval jn
        // (between two barriers): the state wave takes chunk jn from ring A slot
        // jn & 1 and leaves S_jn and U_jn in hand-off slot jn & 1; the output
        // wave takes chunk jn - 1 (ring B slot (jn - 1) % 3, hand-off slot
        // (jn - 1) & 1); the I/O waves fill both rings with chunk jn + 1.
        const int nch = c_end - c_begin;
        const int nint = nch + (nch > 0);   // one extra interval for the last chunk's outputs
        char* const ringB = ring + 2 * X::kBufA;
        char* const hand = ringB + 3 * X::kBufB;
        const int sl = grp;   // the value slice of this workgroup
        if (wave >= 2) {
            const int io = wave - 2;
            auto fetch = [&](int jn) {
                const char* src = a.ws_chunks + ((int64_t)(c_begin + jn) * H + h) * cb.bytes;
                char* A = ring + (jn & 1) * X::kBufA;
                char* Bq = ringB + (jn % 3) * X::kBufB;
                int first = io;   // 1 KiB units dealt round-robin over the I/O waves across segments
                auto seg = [&](const char* sp, char* dp, int64_t bytes) {
                    dma_to_lds(sp, dp, bytes, lane, first, X::kIo);
                    first = ((first - (int)(bytes / 1024)) % X::kIo + X::kIo) % X::kIo;
                };
                seg(src + cb.w, A, X::kSzW);
                seg(src + cb.kb, A + X::kSzW, X::kSzK);
                seg(src + cb.gam, A + 2 * X::kSzW, X::kSzG);
                seg(src + cb.u + grp * cb.group, A + 2 * X::kSzW + X::kSzG, cb.group);
                seg(src + cb.q, Bq, X::kSzW);
                seg(src + cb.p, Bq + X::kSzW, X::kSzP);
            };
            if (nch > 0) fetch(0);
            asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
            // one dword per 128-byte line of a chunk kL2Ahead past the copy (see
            // the one-wave path below)
            const int64_t shared_lines = cb.shared / 128, group_lines = cb.group / 128;
            const int64_t my_shared = (shared_lines - grp + ngroups - 1) / ngroups;
            const int64_t pl = (int64_t)io * 64 + lane;
            const int64_t pf_off = pl < my_shared ? (grp + pl * ngroups) * 128
                                   : pl < my_shared + group_lines ? cb.u + grp * cb.group + (pl - my_shared) * 128
                                   : 0;
            for (int jn = 0; jn < nint; ++jn) {
                const bool more = jn + 1 < nch;
                if (more) fetch(jn + 1);
                asm volatile("" ::: "memory");   // the line load stays after the copies
                const int xp = c_begin + min(jn + 1 + kL2Ahead, nch - 1);
                if constexpr (X::kDeferOk) {
                // the line load lands in a scratch LDS word (no register, so no
                // compiler wait); ring B of the chunk just issued is first read
                // an interval later, so the wait leaves its copies (kDeferB per
                // wave) and the line load in flight: loads complete in order, so
                // everything issued before them, ring A included, has landed
                __builtin_amdgcn_global_load_lds((gbl_void_t*)(a.ws_chunks + ((int64_t)xp * H + h) * cb.bytes + pf_off),
                                                 (lds_void_t*)pf_sink, 4, 0, 0);
                if (more) asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(X::kDeferB + 1) : "memory");
                else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
                } else {
                typedef __attribute__((address_space(1))) const int gbl_int_t;
                const int pv = *(gbl_int_t*)(a.ws_chunks + ((int64_t)xp * H + h) * cb.bytes + pf_off);
                asm volatile("s_waitcnt vmcnt(1)\n\ts_barrier" ::: "memory");
                asm volatile("" ::"v"(pv));
                }
            }
            return;
        }
        const int64_t sbase = (int64_t)unit * DK * DV;
        if (wave == 0) {
            // ---- state wave: acc[t][j] = S[16t + 4g + j][16 sl + cl] --------------
            f32x4 acc[NQK];
#pragma unroll
            for (int t = 0; t < NQK; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[t][j] = a.s0 ? a.s0[sbase + (int64_t)(16 * t + 4 * g + j) * DV + 16 * sl + cl] : 0.f;
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            for (int jn = 0; jn < nint; ++jn) {
                if (jn < nch) {
                    const char* A = ring + (jn & 1) * X::kBufA;
                    const char* Wl = A;
                    const char* Kl = A + X::kSzW;
                    const float* gl = reinterpret_cast<const float*>(A + 2 * X::kSzW);
                    const T* Ul = reinterpret_cast<const T*>(A + 2 * X::kSzW + X::kSzG);
                    Q* hq = reinterpret_cast<Q*>(hand + (jn & 1) * X::kHand);
                    Q sb[NQK];
#pragma unroll
                    for (int t = 0; t < NQK; ++t) {
                        sb[t] = make_quad<T>(acc[t]);
                        hq[t * 64 + lane] = sb[t];
                    }
                    // U = Utilde - W S
                    Q ub[NB];
#pragma unroll
                    for (int tb = 0; tb < NB; ++tb) {
                        Q wq[NQK];
                        load_frag(wq, Wl, tb, lane);
                        const f32x4 xw = mma_quads(wq, sb, zero4());
                        const f32x4 ut = from_quad(*reinterpret_cast<const Q*>(Ul + (lane * NB + tb) * 4));
                        ub[tb] = make_quad<T>(ut - xw);
                        hq[(NQK + tb) * 64 + lane] = ub[tb];
                    }
                    // S <- diag(gamma_C) S + Kbar^T U
#pragma unroll
                    for (int t = 0; t < NQK; ++t) {
                        const f32x4 gv = *reinterpret_cast<const f32x4*>(gl + 16 * t + 4 * g);
                        Q kq[NB];
                        load_frag(kq, Kl, t, lane);
                        acc[t] = mma_quads(kq, ub, acc[t] * gv);
                    }
                    if (a.ckpt) {   // S after the first (jn + 1) C tokens, at multiples of ckpt_every
                        const int64_t done = (int64_t)(jn + 1) * C;
                        if (done <= seq_len && done % a.ckpt_every == 0 && done / a.ckpt_every <= a.max_ckpts) {
                            float* cp = a.ckpt + (((int64_t)seq * a.max_ckpts + done / a.ckpt_every - 1) * H + h) * DK * DV;
#pragma unroll
                            for (int t = 0; t < NQK; ++t)
#pragma unroll
                                for (int j = 0; j < 4; ++j)
                                    cp[(int64_t)(16 * t + 4 * g + j) * DV + 16 * sl + cl] = acc[t][j];
                        }
                    }
                }
                asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            }
            if (a.s_final) {
#pragma unroll
                for (int t = 0; t < NQK; ++t)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        a.s_final[sbase + (int64_t)(16 * t + 4 * g + j) * DV + 16 * sl + cl] = acc[t][j];
            }
            // a non-finite state element stays non-finite through every later
            // chunk (and reaches its checkpoints), so the final one tells
            bool fin = true;
#pragma unroll
            for (int t = 0; t < NQK; ++t) fin &= finite4(acc[t]);
            if (!fin) *a.status = 1;
            return;
        }
        // ---- output wave: O^T = S^T Qtilde^T + U^T P^T of chunk jn - 1 ------------
        // (lane: columns 16 sl + 4g + j, token 16tb + cl)
        bool fin = true;   // every output this lane formed was finite
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        for (int jn = 0; jn < nint; ++jn) {
            if (jn >= 1) {
                const int jp = jn - 1;
                const int64_t tok0 = tok_begin + (int64_t)jp * C;
                const int valid = (int)min((int64_t)C, seq_len - (int64_t)jp * C);
                const char* Bq = ringB + (jp % 3) * X::kBufB;
                const char* Ql = Bq;
                const char* Pl = Bq + X::kSzW;
                const Q* hq = reinterpret_cast<const Q*>(hand + (jp & 1) * X::kHand);
                Q sb[NQK], ub[NB];
#pragma unroll
                for (int t = 0; t < NQK; ++t) sb[t] = hq[t * 64 + lane];
#pragma unroll
                for (int tb = 0; tb < NB; ++tb) ub[tb] = hq[(NQK + tb) * 64 + lane];
#pragma unroll
                for (int tb = 0; tb < NB; ++tb) {
                    Q qq[NQK], pq[NB];
                    load_frag(qq, Ql, tb, lane);
                    load_frag(pq, Pl, tb, lane);
                    const int r = 16 * tb + cl;
                    // two chains summed on the VALU (no K=16 step accumulates onto a K=32 result)
                    const f32x4 sc = (mma_quads(sb, qq, zero4()) + mma_quads_upto(ub, pq, tb, zero4())) * a.scale;
                    fin &= finite4(sc);
                    if constexpr (kMode == kOutSplit) {
                        float sn = sc[0] * sc[0] + sc[1] * sc[1] + sc[2] * sc[2] + sc[3] * sc[3];
                        sn += __shfl_xor(sn, 16, 64);
                        sn += __shfl_xor(sn, 32, 64);
                        if (r < valid) {
                            const int64_t row = (tok0 + r) * H + h;
                            *reinterpret_cast<f32x4*>(a.o_scratch + row * DV + 16 * sl + 4 * g) = sc;
                            if (g == 0) a.part_scratch[row * (DV / 16) + sl] = sn;
                        }
                    } else if (r < valid) {
                        const int64_t oi = ((tok0 + r) * H + h) * DV + 16 * sl + 4 * g;
                        if (a.o_f32) store4(reinterpret_cast<float*>(a.o) + oi, sc);
                        else store4(reinterpret_cast<__bf16*>(a.o) + oi, sc);
                    }
                }
            }
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        }
        if (!fin) *a.status = 1;
    } else {
        if (wave >= ncw) {
            // ---- I/O waves -----------------------------------------------------------
            const int io = wave - ncw;
            auto fetch = [&](int x, int slot) {
                const char* src = a.ws_chunks + ((int64_t)x * H + h) * cb.bytes;
                char* dst = ring + slot * X::kBuf;
                dma_to_lds(src, dst, cb.shared, lane, io, kIoWaves);
                dma_to_lds(src + cb.u + grp * cb.group, dst + X::kShared, cb.group, lane, io, kIoWaves);
            };
            if (cw_begin < cw_end) fetch(cw_begin, 0);
            asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
            // The ring holds two chunks, so the copy of chunk x + 1 is issued only
            // one chunk ahead and would pay the full HBM latency.  One dword per
            // 128-byte line of chunk x + 1 + kL2Ahead is loaded as well, into a
            // scratch LDS word (no register the compiler would wait for), which
            // brings that block into this XCD's L2 early: the shared part is
            // split over the slice groups of the (sequence, head), each group
            // touches its own value slices.  Every lane issues kPfLoads such
            // loads (a lane without a line re-reads the block's first line), so
            // the wait below leaves exactly those outstanding.
            const int64_t shared_lines = cb.shared / 128, group_lines = cb.group / 128;
            const int64_t my_shared = (shared_lines - grp + ngroups - 1) / ngroups;
            int64_t pf_off[X::kPfLoads];
#pragma unroll
            for (int i = 0; i < X::kPfLoads; ++i) {
                const int64_t pl = ((int64_t)i * X::kIo + io) * 64 + lane;
                pf_off[i] = pl < my_shared ? (grp + pl * ngroups) * 128
                            : pl < my_shared + group_lines ? cb.u + grp * cb.group + (pl - my_shared) * 128
                            : 0;
            }
            for (int x = cw_begin; x < cw_end; ++x) {
                if (x + 1 < cw_end) fetch(x + 1, (x + 1 - cw_begin) & 1);
                if (ranged) {
                    // a range's blocks are read by its workgroup alone, and with
                    // one workgroup per CU the blocks a chunk ahead of all of an
                    // XCD's ranges exceed its L2: the line loads were evicted
                    // before use (25 % more HBM reads, no gain in time)
                    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
                    continue;
                }
                asm volatile("" ::: "memory");   // the line loads stay after the copies
                const char* pblk = a.ws_chunks + ((int64_t)min(x + 1 + kL2Ahead, cw_end - 1) * H + h) * cb.bytes;
#pragma unroll
                for (int i = 0; i < X::kPfLoads; ++i)
                    __builtin_amdgcn_global_load_lds((gbl_void_t*)(pblk + pf_off[i]), (lds_void_t*)pf_sink, 4, 0, 0);
                asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(X::kPfLoads) : "memory");
            }
            return;
        }

        // ---- compute waves: SPW value slices (16 columns each) per wave ----------------
        const int s0 = grp * cb.gsl + wave * SPW;   // first value slice of this wave
        // slices this wave owns (a group may hold fewer than SPW * waves); the
        // accumulators of a missing slice are computed on stale LDS and never stored
        const int nsl = min(SPW, cb.gsl - wave * SPW);
        // S slices in accumulator layout: acc[n][t][j] = S[16t + 4g + j][16 (s0 + n) + cl]
        f32x4 acc[SPW][NQK];
        const int64_t sbase = (int64_t)unit * DK * DV;
#pragma unroll
        for (int n = 0; n < SPW; ++n)
#pragma unroll
            for (int t = 0; t < NQK; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[n][t][j] = (s_init && n < nsl) ? s_init[(int64_t)(16 * t + 4 * g + j) * DV + 16 * (s0 + n) + cl] : 0.f;

        bool fin = true;   // every output this lane formed was finite
        // gated calls: a chunk's outputs wait in registers until every wave's
        // partial sums of squares are in LDS (after the chunk's barrier); the
        // norm, weight and gate are then applied and the outputs stored
        f32x4 opend[kGate ? NB : 1][kGate ? SPW : 1];
        int64_t ptok0 = 0;
        int pvalid = 0, pbuf = 0;
        bool pending = false;
        // the gate logits of the pending outputs, as loaded: they are loaded
        // when the chunk's interval begins and used when its outputs are
        // stored, one interval later (loading them there exposed an HBM round
        // trip per chunk: 2.58 against 2.34 ms for the gated long-context call)
        typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
        using GRaw = typename std::conditional<sizeof(In) == 2, u32x2, f32x4>::type;
        GRaw gpend[kGate ? NB : 1][kGate ? SPW : 1];
        const bool gvec = (reinterpret_cast<uintptr_t>(a.gate) & (4 * sizeof(In) - 1)) == 0;
        auto gate_load = [&](int64_t tok0, int valid) {
            if constexpr (kGate) {
#pragma unroll
                for (int tb = 0; tb < NB; ++tb) {
                    const int r = 16 * tb + cl;
#pragma unroll
                    for (int n = 0; n < SPW; ++n) {
                        if (r < valid && n < nsl) {
                            const int64_t oi = ((tok0 + r) * H + h) * DV + 16 * (s0 + n) + 4 * g;
                            const In* gp = reinterpret_cast<const In*>(a.gate) + oi;
                            if constexpr (sizeof(In) == 2) {
                                const unsigned short* gs = reinterpret_cast<const unsigned short*>(gp);
                                gpend[tb][n] = gvec ? *reinterpret_cast<const u32x2*>(gp)
                                                    : u32x2{gs[0] | ((unsigned)gs[1] << 16), gs[2] | ((unsigned)gs[3] << 16)};
                            } else {
                                const float* gf = reinterpret_cast<const float*>(gp);
                                gpend[tb][n] = gvec ? *reinterpret_cast<const f32x4*>(gf)
                                                    : f32x4{gf[0], gf[1], gf[2], gf[3]};
                            }
                        }
                    }
                }
            }
        };
        auto flush = [&]() {
            if constexpr (kGate) {
#pragma unroll
                for (int tb = 0; tb < NB; ++tb) {
                    const int r = 16 * tb + cl;
                    float ss = 0.f;
                    for (int w2 = 0; w2 < ncw; ++w2) ss += part[pbuf][w2][r];
                    const float inv = rsqrtf(ss / (float)DV + a.norm_eps);
#pragma unroll
                    for (int n = 0; n < SPW; ++n) {
                        if (r < pvalid && n < nsl) {
                            const int col = 16 * (s0 + n) + 4 * g;
                            const int64_t oi = ((ptok0 + r) * H + h) * DV + col;
                            float gl4[4];
                            if constexpr (sizeof(In) == 2) {
                                const u32x2 w2 = gpend[tb][n];
                                gl4[0] = __uint_as_float(w2[0] << 16);
                                gl4[1] = __uint_as_float(w2[0] & 0xffff0000u);
                                gl4[2] = __uint_as_float(w2[1] << 16);
                                gl4[3] = __uint_as_float(w2[1] & 0xffff0000u);
                            } else {
#pragma unroll
                                for (int j = 0; j < 4; ++j) gl4[j] = gpend[tb][n][j];
                            }
                            f32x4 o4 = opend[tb][n] * inv;
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                o4[j] *= (a.norm_w ? a.norm_w[col + j] : 1.f) * sigmoid(gl4[j]);
                            if (a.o_f32) store4(reinterpret_cast<float*>(a.o) + oi, o4);
                            else store4(reinterpret_cast<__bf16*>(a.o) + oi, o4);
                        }
                    }
                }
            }
        };
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

        for (int x = cw_begin; x < cw_end; ++x) {
            const int jc = x - c_begin;   // chunk index inside the sequence
            const int64_t tok0 = tok_begin + (int64_t)jc * C;
            const int valid = (int)min((int64_t)C, seq_len - (int64_t)jc * C);
            const char* buf = ring + ((x - cw_begin) & 1) * X::kBuf;
            const char* Wl = buf + cb.w;
            const char* Ql = buf + cb.q;
            const char* Kl = buf + cb.kb;
            const char* Pl = buf + cb.p;
            const float* gl = reinterpret_cast<const float*>(buf + cb.gam);
            const T* Ul = reinterpret_cast<const T*>(buf + X::kShared + (s0 - grp * cb.gsl) * cb.slice);
            if (kGate && pending) flush();   // the previous chunk: its partial sums are complete
            if (kGate) gate_load(tok0, valid);

            Q sb[SPW][NQK];
#pragma unroll
            for (int n = 0; n < SPW; ++n)
#pragma unroll
                for (int t = 0; t < NQK; ++t) sb[n][t] = make_quad<T>(acc[n][t]);

            // U = Utilde - W S   (lane: tokens 16tb + 4g + j, column of slice n)
            Q ub[SPW][NB];
#pragma unroll
            for (int tb = 0; tb < NB; ++tb) {
                Q wq[NQK];
                load_frag(wq, Wl, tb, lane);
#pragma unroll
                for (int n = 0; n < SPW; ++n) {
                    const f32x4 xw = mma_quads(wq, sb[n], zero4());
                    const f32x4 ut = from_quad(*reinterpret_cast<const Q*>(Ul + n * (cb.slice / sizeof(T)) + (lane * NB + tb) * 4));
                    ub[n][tb] = make_quad<T>(ut - xw);
                }
            }
            // S <- diag(gamma_C) S + Kbar^T U
#pragma unroll
            for (int t = 0; t < NQK; ++t) {
                const f32x4 gv = *reinterpret_cast<const f32x4*>(gl + 16 * t + 4 * g);
                Q kq[NB];
                load_frag(kq, Kl, t, lane);
#pragma unroll
                for (int n = 0; n < SPW; ++n) acc[n][t] = mma_quads(kq, ub[n], acc[n][t] * gv);
            }
            // state checkpoint: S after the first (jc + 1) C tokens when that is a
            // multiple of ckpt_every inside the sequence (a full chunk)
            if (a.ckpt) {
                const int64_t done = (int64_t)(jc + 1) * C;
                if (done <= seq_len && done % a.ckpt_every == 0 && done / a.ckpt_every <= a.max_ckpts) {
                    float* cp = a.ckpt + (((int64_t)seq * a.max_ckpts + done / a.ckpt_every - 1) * H + h) * DK * DV;
#pragma unroll
                    for (int sl = 0; sl < SPW; ++sl)
                        if (sl < nsl)
#pragma unroll
                            for (int t = 0; t < NQK; ++t)
#pragma unroll
                                for (int j = 0; j < 4; ++j)
                                    cp[(int64_t)(16 * t + 4 * g + j) * DV + 16 * (s0 + sl) + cl] = acc[sl][t][j];
                }
            }
            // O^T = S^T Qtilde^T + U^T P^T   (lane: columns 4g + j, token 16tb + cl); S^T from sb (pre-update)
#pragma unroll
            for (int tb = 0; tb < NB; ++tb) {
                Q qq[NQK], pq[NB];
                load_frag(qq, Ql, tb, lane);
                load_frag(pq, Pl, tb, lane);
                const int r = 16 * tb + cl;
                float ss = 0.f;
#pragma unroll
                for (int n = 0; n < SPW; ++n) {
                    // two chains summed on the VALU: with dk or C of 16 one of them is a
                    // single K=16 step, which must not accumulate onto a K=32 result
                    const f32x4 ot = mma_quads(sb[n], qq, zero4()) + mma_quads_upto(ub[n], pq, tb, zero4());
                    const f32x4 sc = ot * a.scale;
                    if (n < nsl) fin &= finite4(sc);
                    if constexpr (kGate) {
                        opend[tb][n] = sc;
                        if (n < nsl) ss += sc[0] * sc[0] + sc[1] * sc[1] + sc[2] * sc[2] + sc[3] * sc[3];
                    } else if constexpr (kMode == kOutSplit) {
                        float sn = sc[0] * sc[0] + sc[1] * sc[1] + sc[2] * sc[2] + sc[3] * sc[3];
                        sn += __shfl_xor(sn, 16, 64);
                        sn += __shfl_xor(sn, 32, 64);
                        if (r < valid && n < nsl) {
                            const int64_t row = (tok0 + r) * H + h;
                            *reinterpret_cast<f32x4*>(a.o_scratch + row * DV + 16 * (s0 + n) + 4 * g) = sc;
                            if (g == 0) a.part_scratch[row * (DV / 16) + s0 + n] = sn;
                        }
                    } else if (r < valid && n < nsl) {
                        const int64_t oi = ((tok0 + r) * H + h) * DV + 16 * (s0 + n) + 4 * g;
                        if (a.o_f32) store4(reinterpret_cast<float*>(a.o) + oi, sc);
                        else store4(reinterpret_cast<__bf16*>(a.o) + oi, sc);
                    }
                }
                if constexpr (kGate) {   // this wave's columns of token r: lanes cl, cl + 16, cl + 32, cl + 48
                    ss += __shfl_xor(ss, 16, 64);
                    ss += __shfl_xor(ss, 32, 64);
                    if (g == 0) part[jc & 1][wave][r] = ss;
                }
            }
            if constexpr (kGate) {
                ptok0 = tok0;
                pvalid = valid;
                pbuf = jc & 1;
                pending = true;
            }
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        }
        if (kGate && pending) flush();   // the last chunk, past its barrier
#pragma unroll
        for (int n = 0; n < SPW; ++n)
            if (n < nsl)
#pragma unroll
                for (int t = 0; t < NQK; ++t) fin &= finite4(acc[n][t]);
        if (!fin) *a.status = 1;
        if (a.s_final && ends_seq) {
#pragma unroll
            for (int n = 0; n < SPW; ++n)
                if (n < nsl)
#pragma unroll
                for (int t = 0; t < NQK; ++t)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        a.s_final[sbase + (int64_t)(16 * t + 4 * g + j) * DV + 16 * (s0 + n) + cl] = acc[n][t][j];
        }
    }   // one compute wave per slice group
}

// ---------------------------------------------------------------------------
// Chunk-range scan.  Over a range of chunks the chain is affine in its start
// state: S_end = A S_start + B, with A = prod_c (diag(gamma_c) - Kbar_c^T W_c)
// (dk x dk) and B the state reached from zero.  Both are the chain itself run
// on the (dk + dv)-column state [I | 0]: for A's columns U = -W X, for B's
// U = U~ - W X; then X <- diag(gamma) X + Kbar^T U.  With the maps of every
// range but each sequence's last, the ranges' start states follow from a
// short scan, and every range's outputs can be formed at once.
// ---------------------------------------------------------------------------
template <int DK, int C, typename T> struct RangeSum {
    static constexpr int kSlices = 2 * DK / 16;   // A's DK/16 column slices, then B's (dv == dk)
    static constexpr int SPW = 2;                 // slices per compute wave
    static constexpr int kCompute = kSlices / SPW;
    static constexpr int kIo = 4;
    static constexpr int kThreads = 64 * (kCompute + kIo);
    static constexpr int64_t kSzW = Frag<T>::elems(C, DK) * (int64_t)sizeof(T);
    static constexpr int64_t kSzK = Frag<T>::elems(DK, C) * (int64_t)sizeof(T);
    static constexpr int64_t kSzG = round_kib(DK * 4);
    static constexpr int64_t kSzU = round_kib((int64_t)(DK / 16) * C * 16 * sizeof(T));   // the row's U~ slices
    // ring slot: [W | Kbar^T | gamma_C | U~]; Q~ and P are not needed here
    static constexpr int64_t kSlot = kSzW + kSzK + kSzG + kSzU;
    static constexpr int64_t kLds = 2 * kSlot;
    static constexpr int kPfLoads = (int)((kSlot / 128 + kIo * 64 - 1) / (kIo * 64));
    static constexpr bool kFits = kLds <= 163840 && kSzW % 1024 == 0 && kSzK % 1024 == 0;
};

template <int DK, int C, typename In>
__global__ __launch_bounds__((RangeSum<DK, C, typename OperandOf<In>::type>::kThreads))
void kda_range_kernel(const PrefillArgs a) {
    using T = typename OperandOf<In>::type;
    using Q = quad_t<T>;
    using X = RangeSum<DK, C, T>;
    static_assert(X::kFits, "LDS ring of the range kernel exceeds one workgroup");
    constexpr int NB = C / 16, NQK = DK / 16, SPW = X::SPW;
    __shared__ __attribute__((aligned(1024))) char ring[X::kLds];
    __shared__ __attribute__((aligned(256))) int pf_sink[64];   // L2 prefetch target (never read)

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, cl = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = a.H, DV = a.DV;
    const ChunkBlock<T> cb(DK, C, DV, a.gsl);
    const int xr = blockIdx.x / H, h = blockIdx.x % H;
    RangePos rp;
    // the last range of a sequence needs no map (nothing follows it)
    if (!locate_range(a, xr, rp) || rp.r == rp.nr - 1) return;   // whole workgroup
    const int cw_begin = rp.c0, cw_end = rp.c1;   // a range before the last is full: L chunks

    if (wave >= X::kCompute) {
        // ---- I/O waves: W, Kbar^T, gamma_C and the row's U~ of chunk x + 1 ----
        const int io = wave - X::kCompute;
        auto fetch = [&](int x, int slot) {
            const char* src = a.ws_chunks + ((int64_t)x * H + h) * cb.bytes;
            char* dst = ring + slot * X::kSlot;
            int first = io;   // 1 KiB units dealt round-robin over the I/O waves across segments
            auto seg = [&](const char* sp, char* dp, int64_t bytes) {
                dma_to_lds(sp, dp, bytes, lane, first, X::kIo);
                first = ((first - (int)(bytes / 1024)) % X::kIo + X::kIo) % X::kIo;
            };
            seg(src + cb.w, dst, X::kSzW);
            seg(src + cb.kb, dst + X::kSzW, X::kSzK);
            seg(src + cb.gam, dst + X::kSzW + X::kSzK, X::kSzG);
            seg(src + cb.u, dst + X::kSzW + X::kSzK + X::kSzG, X::kSzU);
        };
        // one dword of each 128-byte line of the slot's four regions, kL2Ahead
        // chunks past the copy, into an LDS sink: brings them into L2 early
        int64_t pf_off[X::kPfLoads];
#pragma unroll
        for (int i = 0; i < X::kPfLoads; ++i) {
            const int64_t pl = ((int64_t)i * X::kIo + io) * 64 + lane;
            const int64_t lw = X::kSzW / 128, lk = X::kSzK / 128, lg = X::kSzG / 128, lu = X::kSzU / 128;
            pf_off[i] = pl < lw ? cb.w + pl * 128
                        : pl < lw + lk ? cb.kb + (pl - lw) * 128
                        : pl < lw + lk + lg ? cb.gam + (pl - lw - lk) * 128
                        : pl < lw + lk + lg + lu ? cb.u + (pl - lw - lk - lg) * 128
                        : cb.w;
        }
        if (cw_begin < cw_end) fetch(cw_begin, 0);
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        for (int x = cw_begin; x < cw_end; ++x) {
            if (x + 1 < cw_end) fetch(x + 1, (x + 1 - cw_begin) & 1);
            asm volatile("" ::: "memory");   // the line loads stay after the copies
            const char* pblk = a.ws_chunks + ((int64_t)min(x + 1 + kL2Ahead, cw_end - 1) * H + h) * cb.bytes;
#pragma unroll
            for (int i = 0; i < X::kPfLoads; ++i)
                __builtin_amdgcn_global_load_lds((gbl_void_t*)(pblk + pf_off[i]), (lds_void_t*)pf_sink, 4, 0, 0);
            asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(X::kPfLoads) : "memory");
        }
        return;
    }

    // ---- compute waves: slices s0, s0 + 1 of [A | B] (16 columns each) ---------
    const int s0 = wave * SPW;
    const bool partB = s0 >= NQK;   // wave-uniform: a wave's slices are all of A or all of B
    // acc[n][t][j] = X[16t + 4g + j][16 (s0 + n) + cl]; A starts as the identity, B as zero
    f32x4 acc[SPW][NQK];
#pragma unroll
    for (int n = 0; n < SPW; ++n)
#pragma unroll
        for (int t = 0; t < NQK; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[n][t][j] = (!partB && 16 * t + 4 * g + j == 16 * (s0 + n) + cl) ? 1.f : 0.f;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    for (int x = cw_begin; x < cw_end; ++x) {
        const char* buf = ring + ((x - cw_begin) & 1) * X::kSlot;
        const char* Wl = buf;
        const char* Kl = buf + X::kSzW;
        const float* gl = reinterpret_cast<const float*>(buf + X::kSzW + X::kSzK);
        const T* Ul = reinterpret_cast<const T*>(buf + X::kSzW + X::kSzK + X::kSzG);
        Q sb[SPW][NQK];
#pragma unroll
        for (int n = 0; n < SPW; ++n)
#pragma unroll
            for (int t = 0; t < NQK; ++t) sb[n][t] = make_quad<T>(acc[n][t]);
        // U = (U~ for B's columns, 0 for A's) - W X
        Q ub[SPW][NB];
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
            Q wq[NQK];
            load_frag(wq, Wl, tb, lane);
#pragma unroll
            for (int n = 0; n < SPW; ++n) {
                const f32x4 xw = mma_quads(wq, sb[n], zero4());
                f32x4 ut = zero4();
                if (partB)
                    ut = from_quad(*reinterpret_cast<const Q*>(Ul + (s0 + n - NQK) * (cb.slice / sizeof(T)) +
                                                               (lane * NB + tb) * 4));
                ub[n][tb] = make_quad<T>(ut - xw);
            }
        }
        // X <- diag(gamma_C) X + Kbar^T U
#pragma unroll
        for (int t = 0; t < NQK; ++t) {
            const f32x4 gv = *reinterpret_cast<const f32x4*>(gl + 16 * t + 4 * g);
            Q kq[NB];
            load_frag(kq, Kl, t, lane);
#pragma unroll
            for (int n = 0; n < SPW; ++n) acc[n][t] = mma_quads(kq, ub[n], acc[n][t] * gv);
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    // the map, row-major [dk][dk + dv]: A in columns [0, dk), B in [dk, dk + dv)
    float* ab = a.range_ab + ((int64_t)xr * H + h) * DK * (DK + DV);
    bool fin = true;
#pragma unroll
    for (int n = 0; n < SPW; ++n)
#pragma unroll
        for (int t = 0; t < NQK; ++t) {
            fin &= finite4(acc[n][t]);
#pragma unroll
            for (int j = 0; j < 4; ++j) ab[(int64_t)(16 * t + 4 * g + j) * (DK + DV) + 16 * (s0 + n) + cl] = acc[n][t][j];
        }
    if (!fin) *a.status = 1;
}

// Start states of the ranges of one (sequence, head), 16 value columns per
// workgroup: S_{r+1} = A_r S_r + B_r in fp32 from S_0 = the initial state,
// written for ranges 1 .. nr - 1.  The products run on fp32 MFMA
// (16x16x4): each of the four waves forms dk/64 16-row tiles of S_{r+1}.
// The contraction order is permuted so that a lane's A operand is a run of
// consecutive columns: in K-step 4m + u, lane (g, c) contracts column
// 16m + 4g + u, so it reads its row of A_r as float4 loads.  Only S is
// serial, so the operands of step r + 1 are loaded while step r runs.
template <int DK>
__global__ __launch_bounds__(256) void kda_range_scan_kernel(const PrefillArgs a) {
    constexpr int DV = DK, NSL = DV / 16, KQ = DK / 16, TW = DK / 64, RS = DK + DV;
    // blocks are dealt round-robin over the 8 XCDs: the slices of one
    // (sequence, head) share its range maps, so they go to one XCD
    const int xcd = blockIdx.x & 7, jx = blockIdx.x >> 3;
    const int unit = (jx / NSL) * 8 + xcd, sl = jx % NSL;
    const int H = a.H;
    if (unit >= a.N * H) return;
    const int n = unit / H, h = unit % H;
    int x0, nr;
    if (a.cu_seqlens) {
        x0 = a.range_off[n];
        nr = a.range_off[n + 1] - x0;
    } else {
        x0 = n * a.ranges_per_seq;
        nr = a.ranges_per_seq;
    }
    if (nr <= 1) return;   // uniform over the workgroup
    __shared__ float sS[DK][17];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, cl = lane & 15;
    for (int e = tid; e < DK * 16; e += 256) {
        const int c = e >> 4, j = e & 15;
        sS[c][j] = a.s0 ? a.s0[((int64_t)unit * DK + c) * DV + 16 * sl + j] : 0.f;
    }
    f32x4 aN[TW][KQ], cN[TW];   // operands of the next step: A rows, B tile
    auto fetch = [&](int r) {
        const float* ab = a.range_ab + ((int64_t)(x0 + r) * H + h) * DK * RS;
#pragma unroll
        for (int i = 0; i < TW; ++i) {
            const int t = wave * TW + i;
#pragma unroll
            for (int m = 0; m < KQ; ++m) aN[i][m] = *(const f32x4*)(ab + (int64_t)(16 * t + cl) * RS + 16 * m + 4 * g);
#pragma unroll
            for (int j = 0; j < 4; ++j) cN[i][j] = ab[(int64_t)(16 * t + 4 * g + j) * RS + DK + 16 * sl + cl];
        }
    };
    fetch(0);
    __syncthreads();
    bool fin = true;
    for (int r = 0; r + 1 < nr; ++r) {
        f32x4 aC[TW][KQ], acc[TW];
#pragma unroll
        for (int i = 0; i < TW; ++i) {
            acc[i] = cN[i];
#pragma unroll
            for (int m = 0; m < KQ; ++m) aC[i][m] = aN[i][m];
        }
        if (r + 2 < nr) fetch(r + 1);
#pragma unroll
        for (int m = 0; m < KQ; ++m)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float b = sS[16 * m + 4 * g + u][cl];
#pragma unroll
                for (int i = 0; i < TW; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(aC[i][m][u], b, acc[i], 0, 0, 0);
            }
        __syncthreads();   // every wave has read S_r
        float* out = a.range_start + ((int64_t)(x0 + r + 1) * H + h) * DK * DV;
#pragma unroll
        for (int i = 0; i < TW; ++i) {
            const int t = wave * TW + i;
            fin &= finite4(acc[i]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = 16 * t + 4 * g + j;
                sS[c][cl] = acc[i][j];
                out[(int64_t)c * DV + 16 * sl + cl] = acc[i][j];
            }
        }
        __syncthreads();
    }
    if (!fin) *a.status = 1;
}

// ---------------------------------------------------------------------------
// Host-side launchers (called from the C ABI after validation).
// ---------------------------------------------------------------------------
template <int DK, int C, typename In>
static hipError_t launch_phase_t(const PrefillArgs& a, int max_chunks, bool intra, hipStream_t stream) {
    if constexpr (!Intra<DK, C, typename OperandOf<In>::type>::kFits ||
                  !Inter<DK, C, typename OperandOf<In>::type>::kFits ||
                  !Inter<DK, C, typename OperandOf<In>::type, true>::kFits ||
                  !Inter<DK, C, typename OperandOf<In>::type, true, true>::kFits) {
        return hipErrorInvalidValue;  // effective_chunk() never selects this
    } else {
        if (intra) {
            if (max_chunks > 0) {
                const dim3 grid((unsigned)max_chunks * (unsigned)a.H);
                if (a.alpha_scalar)
                    hipLaunchKernelGGL((kda_intra_kernel<DK, C, In, kInScalar>), grid, dim3(256), 0, stream, a);
                else if (!a.fuse_inputs && a.alpha_floor >= kFloorFast)
                    hipLaunchKernelGGL((kda_intra_kernel<DK, C, In, kInFloor>), grid, dim3(256), 0, stream, a);
                else if (a.fuse_inputs || a.alpha_floor != 0.f)
                    hipLaunchKernelGGL((kda_intra_kernel<DK, C, In, kInOpts>), grid, dim3(256), 0, stream, a);
                else
                    hipLaunchKernelGGL((kda_intra_kernel<DK, C, In, kInPlain>), grid, dim3(256), 0, stream, a);
            }
        } else {
            const int units = a.N * a.H;
            const int blocks = ((units + 7) / 8) * 8 * (a.DV / 16 / a.gsl);
            if (a.whole_rows && a.range_len > 0) {
                // chunk-range scan: range maps, the ranges' start states, then
                // every range's whole-row pass (gated calls finish the output
                // norm in that pass)
                using T = typename OperandOf<In>::type;
                if constexpr (C == 64 && (DK == 64 || DK == 128) && sizeof(T) == 2 && RangeSum<DK, C, T>::kFits) {
                    const int spw = a.gate ? Inter<DK, C, T, true, true>::SPW : Inter<DK, C, T, true>::SPW;
                    const dim3 grid((unsigned)a.max_ranges * (unsigned)a.H);
                    const dim3 threads(64 * ((a.gsl + spw - 1) / spw + kIoWaves));
                    hipLaunchKernelGGL((kda_range_kernel<DK, C, In>), grid, dim3(RangeSum<DK, C, T>::kThreads), 0,
                                       stream, a);
                    hipLaunchKernelGGL((kda_range_scan_kernel<DK>), dim3((unsigned)(((units + 7) / 8) * 8 * (a.DV / 16))),
                                       dim3(256), 0, stream, a);
                    if (a.gate)
                        hipLaunchKernelGGL((kda_inter_kernel<DK, C, In, kOutGate>), grid, threads, 0, stream, a);
                    else
                        hipLaunchKernelGGL((kda_inter_kernel<DK, C, In, kOutRow>), grid, threads, 0, stream, a);
                } else {
                    return hipErrorInvalidValue;   // range_length() never selects this
                }
            } else if (a.gate && !a.gate_split) {
                constexpr int spw = Inter<DK, C, typename OperandOf<In>::type, true, true>::SPW;
                hipLaunchKernelGGL((kda_inter_kernel<DK, C, In, kOutGate>), dim3(blocks),
                                   dim3(64 * ((a.gsl + spw - 1) / spw + kIoWaves)), 0, stream, a);
            } else if (a.whole_rows) {
                constexpr int spw = Inter<DK, C, typename OperandOf<In>::type, true>::SPW;
                hipLaunchKernelGGL((kda_inter_kernel<DK, C, In, kOutRow>), dim3(blocks),
                                   dim3(64 * ((a.gsl + spw - 1) / spw + kIoWaves)), 0, stream, a);
            } else {
                using XP = Inter<DK, C, typename OperandOf<In>::type, false>;
                const int threads = XP::kOWave ? XP::kThreads : 64 * ((a.gsl + XP::SPW - 1) / XP::SPW + kIoWaves);
                if (a.gate)
                    hipLaunchKernelGGL((kda_inter_kernel<DK, C, In, kOutSplit>), dim3(blocks), dim3(threads), 0,
                                       stream, a);
                else
                    hipLaunchKernelGGL((kda_inter_kernel<DK, C, In, kOutPlain>), dim3(blocks), dim3(threads), 0,
                                       stream, a);
            }
        }
        return hipGetLastError();
    }
}

template <int DK, typename In>
static hipError_t launch_phase_c(const PrefillArgs& a, int C, int max_chunks, bool intra, hipStream_t s) {
    switch (C) {
        case 16: return launch_phase_t<DK, 16, In>(a, max_chunks, intra, s);
        case 32: return launch_phase_t<DK, 32, In>(a, max_chunks, intra, s);
        case 64: return launch_phase_t<DK, 64, In>(a, max_chunks, intra, s);
    }
    return hipErrorInvalidValue;
}

template <typename In>
static hipError_t launch_phase_k(const PrefillArgs& a, int DK, int C, int max_chunks, bool intra, hipStream_t s) {
    switch (DK) {
        case 16: return launch_phase_c<16, In>(a, C, max_chunks, intra, s);
        case 32: return launch_phase_c<32, In>(a, C, max_chunks, intra, s);
        case 64: return launch_phase_c<64, In>(a, C, max_chunks, intra, s);
        case 128: return launch_phase_c<128, In>(a, C, max_chunks, intra, s);
    }
    return hipErrorInvalidValue;
}

template <typename T> static bool fits(int DK, int C) {
#define KDA_FITS_CASE(D, CC)                                                                  \
    if (DK == D && C == CC)                                                                   \
        return Intra<D, CC, T>::kFits && Inter<D, CC, T>::kFits && Inter<D, CC, T, true>::kFits && \
               Inter<D, CC, T, true, true>::kFits;
    KDA_FITS_CASE(16, 16) KDA_FITS_CASE(16, 32) KDA_FITS_CASE(16, 64)
    KDA_FITS_CASE(32, 16) KDA_FITS_CASE(32, 32) KDA_FITS_CASE(32, 64)
    KDA_FITS_CASE(64, 16) KDA_FITS_CASE(64, 32) KDA_FITS_CASE(64, 64)
    KDA_FITS_CASE(128, 16) KDA_FITS_CASE(128, 32) KDA_FITS_CASE(128, 64)
#undef KDA_FITS_CASE
    return false;
}

int effective_chunk(int DK, int C, bool bf16) {
    while (C > 16 && !(bf16 ? fits<_Float16>(DK, C) : fits<float>(DK, C))) C /= 2;
    return C;
}

__global__ __launch_bounds__(64) void kda_clear_status(int32_t* status) {
    if (threadIdx.x == 0) {
        status[0] = 0;
        status[kLayoutWord] = 0;
    }
}

hipError_t launch_clear_status(int32_t* status, hipStream_t s) {
    hipLaunchKernelGGL(kda_clear_status, dim3(1), dim3(64), 0, s, status);
    return hipGetLastError();
}

// The range status of a call made of several calls (kda_chunk_fwd_windowed):
// each call clears and sets word 0; word 1 collects them.  kFoldClear clears
// word 1, kFoldOr adds word 0 to it, kFoldBack copies it to word 0.
__global__ __launch_bounds__(64) void kda_fold_status(int32_t* status, int32_t mode) {
    if (threadIdx.x == 0) {
        if (mode == kFoldClear) status[1] = 0;
        else if (mode == kFoldOr) status[1] |= status[0];
        else status[0] = status[1];
    }
}

hipError_t launch_fold_status(int32_t* status, int mode, hipStream_t s) {
    hipLaunchKernelGGL(kda_fold_status, dim3(1), dim3(64), 0, s, status, (int32_t)mode);
    return hipGetLastError();
}

hipError_t launch_chunk_offsets(const int32_t* cu, int32_t n, int32_t C, int32_t* chunk_off, int64_t T,
                                int32_t* status, hipStream_t s) {
    hipLaunchKernelGGL(kda_chunk_offsets, dim3(1), dim3(256), 0, s, cu, n, C, 1, chunk_off, (int32_t*)nullptr, T,
                       status);
    return hipGetLastError();
}

hipError_t launch_chunk_range_offsets(const int32_t* cu, int32_t n, int32_t C, int32_t L, int32_t* chunk_off,
                                      int32_t* range_off, int64_t T, int32_t* status, hipStream_t s) {
    hipLaunchKernelGGL(kda_chunk_offsets, dim3(1), dim3(256), 0, s, cu, n, C, L, chunk_off, range_off, T, status);
    return hipGetLastError();
}

hipError_t launch_seq_order(const int32_t* cu, int32_t n, int32_t C, int32_t* order, hipStream_t s) {
    hipLaunchKernelGGL(kda_seq_order, dim3(1), dim3(1024), 0, s, cu, n, C, order);
    return hipGetLastError();
}

hipError_t launch_intra(const PrefillArgs& a, int DK, int C, bool bf16, int max_chunks, hipStream_t s) {
    return bf16 ? launch_phase_k<__bf16>(a, DK, C, max_chunks, true, s)
                : launch_phase_k<float>(a, DK, C, max_chunks, true, s);
}

hipError_t launch_inter(const PrefillArgs& a, int DK, int C, bool bf16, hipStream_t s) {
    return bf16 ? launch_phase_k<__bf16>(a, DK, C, 0, false, s) : launch_phase_k<float>(a, DK, C, 0, false, s);
}

// Epilogue of split gated calls: one thread per (row = token * H + head, 4
// columns); the per-slice sums of squares are added in a fixed order.
template <typename In>
__global__ __launch_bounds__(256) void kda_gate_epilogue(const PrefillArgs a, const int64_t rows) {
    const int DV = a.DV, CG = DV / 4, NS = DV / 16;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = t / CG;
    if (row >= rows) return;
    const int c4 = (int)(t % CG) * 4;
    const float* ps = a.part_scratch + row * NS;
    const In* __restrict__ gt = reinterpret_cast<const In*>(a.gate) + row * DV + c4;
    // vector loads where the layout allows (the partial sums of a row are 32-byte
    // aligned in the workspace when NS is a multiple of 4; gate and weight
    // pointers need only element alignment, so they are tested, uniformly)
    const f32x4 o_raw = *reinterpret_cast<const f32x4*>(a.o_scratch + row * DV + c4);
    f32x4 gv, wv = f32x4{1.f, 1.f, 1.f, 1.f};
    if ((reinterpret_cast<uintptr_t>(a.gate) & (4 * sizeof(In) - 1)) == 0) {
        if constexpr (sizeof(In) == 4) {
            gv = *reinterpret_cast<const f32x4*>(gt);
        } else {
            const bf16x4 g4 = *reinterpret_cast<const bf16x4*>(gt);
#pragma unroll
            for (int j = 0; j < 4; ++j) gv[j] = (float)g4[j];
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) gv[j] = load_as_float(gt, j);
    }
    if (a.norm_w) {
        if ((reinterpret_cast<uintptr_t>(a.norm_w) & 15) == 0) {
            wv = *reinterpret_cast<const f32x4*>(a.norm_w + c4);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) wv[j] = a.norm_w[c4 + j];
        }
    }
    float ss = 0.f;
    if (NS % 4 == 0) {
        for (int sl = 0; sl < NS; sl += 4) {   // in a fixed order: the same sum for every column
            const f32x4 p4 = *reinterpret_cast<const f32x4*>(ps + sl);
            ss += p4[0];
            ss += p4[1];
            ss += p4[2];
            ss += p4[3];
        }
    } else {
        for (int sl = 0; sl < NS; ++sl) ss += ps[sl];
    }
    const float inv = rsqrtf(ss / (float)DV + a.norm_eps);
    f32x4 o4 = o_raw * inv;
#pragma unroll
    for (int j = 0; j < 4; ++j) o4[j] *= wv[j] * sigmoid(gv[j]);
    if (a.o_f32) store4(reinterpret_cast<float*>(a.o) + row * DV + c4, o4);
    else store4(reinterpret_cast<__bf16*>(a.o) + row * DV + c4, o4);
}

hipError_t launch_gate_epilogue(const PrefillArgs& a, int64_t rows, bool bf16, hipStream_t s) {
    const int64_t threads = rows * (a.DV / 4);
    if (threads <= 0) return hipSuccess;
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    if (bf16) hipLaunchKernelGGL(kda_gate_epilogue<__bf16>, dim3((unsigned)blocks), dim3(256), 0, s, a, rows);
    else hipLaunchKernelGGL(kda_gate_epilogue<float>, dim3((unsigned)blocks), dim3(256), 0, s, a, rows);
    return hipGetLastError();
}

// Compute units of each device, queried once per device (0: not yet).  A
// racing first query stores the same value twice.
constexpr int kMaxDevices = 64;
static std::atomic<int> g_cu_count[kMaxDevices];

static int cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int cus = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cus == 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        g_cu_count[dev].store(cus, std::memory_order_relaxed);
    }
    return cus;
}

bool whole_rows(int64_t units) { return units >= cu_count(); }

int range_length(int DK, int DV, int C, bool bf16, int64_t units, int64_t chunks_per_unit) {
    if (!bf16 || DK != DV || (DK != 64 && DK != 128) || C != 64) return 0;
    const int64_t cus = cu_count();
    if (units <= 0 || units >= cus) return 0;
    // about one range per compute unit, and no range shorter than 16 chunks
    int64_t L = (chunks_per_unit * units + cus - 1) / cus;
    if (L < 16) L = 16;
    // with fewer than three ranges per sequence the maps would cost as much as
    // the walk they shorten
    if (chunks_per_unit < 3 * L || L > (1 << 24)) return 0;
    return (int)L;
}

int slice_group(int DV, bool whole) { return whole ? DV / 16 : group_slices(DV); }

int64_t chunk_block_bytes(int DK, int C, int DV, bool bf16, int gsl) {
    return bf16 ? ChunkBlock<_Float16>(DK, C, DV, gsl).bytes : ChunkBlock<float>(DK, C, DV, gsl).bytes;
}

}  // namespace kda
