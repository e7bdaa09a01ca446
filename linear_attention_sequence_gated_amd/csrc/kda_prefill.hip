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
//   kda_inter_kernel   : one wave per (sequence, head, 16 value columns);
//                        walks the chunks in order with its slice of S held
//                        in MFMA accumulator registers (fp32)
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_kernels.h"
#include "kda_quads.h"

namespace kda {

// log2(alpha) is floored here: alpha below 2^-40 is treated as 2^-40, a
// relative change of the decayed terms far below fp32 resolution.
constexpr float kLog2Floor = -40.f;
// Largest decay (log2 units) a 16-token block may show in any channel for the
// factored Gram path; see the intra-chunk kernel.
constexpr float kFastRange = 12.f;

// ---------------------------------------------------------------------------
// K0: exclusive prefix of ceil(len_n / C) over the packed sequences.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kda_chunk_offsets(const int32_t* __restrict__ cu, int32_t n_seqs,
                                                         int32_t C, int32_t* __restrict__ chunk_off) {
    __shared__ int32_t part[256];
    __shared__ int32_t carry;
    const int tid = threadIdx.x;
    if (tid == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base < n_seqs; base += 256) {
        const int n = base + tid;
        int32_t c = 0;
        if (n < n_seqs) {
            const int32_t len = cu[n + 1] - cu[n];
            c = len > 0 ? (len + C - 1) / C : 0;
        }
        part[tid] = c;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {  // inclusive Hillis-Steele scan
            const int32_t add = tid >= off ? part[tid - off] : 0;
            __syncthreads();
            part[tid] += add;
            __syncthreads();
        }
        if (n < n_seqs) chunk_off[n] = carry + part[tid] - c;
        __syncthreads();
        if (tid == 255) carry += part[255];
        __syncthreads();
    }
    if (tid == 0) chunk_off[n_seqs] = carry;
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

// ---------------------------------------------------------------------------
// K1: intra-chunk work.  256 threads (4 waves) per (chunk, head).
//
// Gram products on the matrix cores need factors 2^{+-g} that stay inside the
// operand format.  The chunk is cut into 16-token blocks; with G_R the decay
// exponent at the first token of block R and h_R half of the block's own
// decay range (per channel), the products k_r k_i 2^{g_r - g_i} are split as
//   row side   (r in block R)  k_r 2^{g_r - G_R + h_R}             in 2^[-h_R, h_R]
//   diagonal   (i in block R)  k_i 2^{G_R - h_R - g_i}             in 2^[-h_R, h_R]
//   off-diag.  (i in block I<R) k_i 2^{G_{I+1} - g_i} * 2^{G_R - G_{I+1} - h_R}   <= 1
// which keeps every factor within 2^[-6, 6] while each block decays by less
// than 2^-12 in every channel.  Chunks beyond that take the exact pairwise
// path (decay products in linear space, fp32).
// ---------------------------------------------------------------------------
template <int DK, int C, typename T> struct Intra {
    static constexpr int kThreads = 256;
    static constexpr int NSEG = C / 4;   // 4-token segments
    static constexpr int NCG = DK / 8;   // 8-channel groups
    static constexpr int NB = C / 16;    // 16-token blocks
    static constexpr int NOFF = NB * (NB - 1) / 2;  // off-diagonal block pairs
    static constexpr int NQK = DK / 16;  // quads along dk
    static constexpr int LD_ROW = DK + 8;  // row-major [*][DK] tiles (elements)
    static constexpr int LD_CT = C + 8;    // [*][C] tiles (elements)
    static constexpr int LD_F = C + 4;     // fp32 [C][C] matrices
    static constexpr int kDvMax = 128;
    // region 1: {Ak, Aq, Bd, Bo} -> {P, M, X} -> {P, VT}
    static constexpr size_t kTiles = (size_t)(4 * C - 16) * LD_ROW * sizeof(T);
    static constexpr size_t kMPX = 3ull * C * LD_F * sizeof(float);
    static constexpr size_t kPVT = 1ull * C * LD_F * sizeof(float) + (size_t)kDvMax * LD_CT * sizeof(T);
    static constexpr size_t cmax(size_t x, size_t y) { return x > y ? x : y; }
    static constexpr size_t kR1 = (cmax(cmax(kTiles, kMPX), kPVT) + 15) / 16 * 16;
    static constexpr size_t kKtT = (size_t)DK * LD_CT * sizeof(T);
    // region 3: {segment sums} -> {Y} -> {Tm}
    static constexpr size_t kTb = (size_t)C * LD_CT * sizeof(T);
    static constexpr size_t kSeg = (size_t)NSEG * DK * sizeof(float);
    static constexpr size_t kY = (size_t)(NB > 1 ? NB - 1 : 1) * 256 * sizeof(float);
    static constexpr size_t kR3 = (cmax(cmax(kTb, kSeg), kY) + 15) / 16 * 16;
    // small: beta, block exponents G/E, pair factors, range flag
    static constexpr size_t kSmall = (size_t)C * 4 + 2ull * NB * DK * 4 + (size_t)(NOFF > 0 ? NOFF : 1) * DK * 4 + 16;
    static constexpr size_t kLds = kR1 + kKtT + kR3 + kSmall;
    static constexpr bool kFits = kLds <= 163840;
};

template <int DK, int C, typename In>
__global__ __launch_bounds__(256) void kda_intra_kernel(const PrefillArgs a) {
    using T = typename OperandOf<In>::type;
    using I = Intra<DK, C, T>;
    static_assert(I::kFits, "LDS budget of one gfx950 workgroup exceeded");
    static_assert(I::NSEG * I::NCG <= I::kThreads, "thread mapping");
    using Q = quad_t<T>;
    constexpr int NB = I::NB, NQK = I::NQK, LD_ROW = I::LD_ROW, LD_CT = I::LD_CT, LD_F = I::LD_F;
    __shared__ __attribute__((aligned(16))) char smem[I::kLds];
    T* Ak = reinterpret_cast<T*>(smem);         // [C][LD_ROW]   row side, k
    T* Aq = Ak + C * LD_ROW;                    // [C][LD_ROW]   row side, q
    T* Bd = Aq + C * LD_ROW;                    // [C][LD_ROW]   diagonal-block column side
    T* Bo = Bd + C * LD_ROW;                    // [C-16][LD_ROW] off-diagonal column side
    float* Pm = reinterpret_cast<float*>(smem);
    float* Mm = Pm + C * LD_F;
    float* Xm = Mm + C * LD_F;
    T* VT = reinterpret_cast<T*>(smem + (size_t)C * LD_F * sizeof(float));
    T* KtT = reinterpret_cast<T*>(smem + I::kR1);
    char* r3 = smem + I::kR1 + I::kKtT;
    float* seg = reinterpret_cast<float*>(r3);
    float* Ys = reinterpret_cast<float*>(r3);
    T* Tb = reinterpret_cast<T*>(r3);
    float* sbeta = reinterpret_cast<float*>(r3 + I::kR3);
    float* Gs = sbeta + C;                      // [NB][DK] exponent at each block's first token
    float* Ge = Gs + NB * DK;                   // [NB][DK] exponent at each block's last token
    float* sIR = Ge + NB * DK;                  // [NOFF][DK] pair factors 2^{G_R - G_{I+1} - h_R}
    unsigned* srange = reinterpret_cast<unsigned*>(sIR + (I::NOFF > 0 ? I::NOFF : 1) * DK);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, g = lane >> 4, cl = lane & 15;
    const int x = blockIdx.x, h = blockIdx.y;
    ChunkPos pos;
    if (!locate_chunk(a, C, x, pos)) return;  // uniform over the workgroup
    const int valid = pos.valid;
    const int H = a.H, DV = a.DV;
    const In* __restrict__ qg = reinterpret_cast<const In*>(a.q);
    const In* __restrict__ kg = reinterpret_cast<const In*>(a.k);
    const In* __restrict__ vg = reinterpret_cast<const In*>(a.v);

    const ChunkBlock<T> cb(DK, C, DV);
    char* blk = a.ws_chunks + ((int64_t)x * H + h) * cb.bytes;
    T* Wf = reinterpret_cast<T*>(blk + cb.w);
    T* Qf = reinterpret_cast<T*>(blk + cb.q);
    T* Kbf = reinterpret_cast<T*>(blk + cb.kb);
    T* Pf = reinterpret_cast<T*>(blk + cb.p);
    T* Uf = reinterpret_cast<T*>(blk + cb.u);
    float* gam = reinterpret_cast<float*>(blk + cb.gam);

    if (tid == 0) *srange = 0u;
    if (tid < C) sbeta[tid] = tid < valid ? a.beta[(pos.tok0 + tid) * H + h] : 0.f;

    // ---- phase 1: decay exponents and operand factors ------------------------
    // thread -> 4 consecutive tokens (segment sgi, block R = sgi/4) x 8 channels
    const bool p1 = tid < I::NSEG * I::NCG;
    const int sgi = tid / I::NCG, cg = tid % I::NCG, Rb = sgi >> 2;
    float kr[4][8], qr[4][8], gv[4][8];
    {
        float run[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) run[e] = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = 4 * sgi + u;
            const bool in = p1 && r < valid;
            const int64_t base = ((pos.tok0 + r) * H + h) * DK + 8 * cg;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                kr[u][e] = in ? load_as_float(kg, base + e) : 0.f;
                qr[u][e] = in ? load_as_float(qg, base + e) : 0.f;
                const float al = in ? a.alpha[base + e] : 1.f;
                run[e] += fmaxf(__builtin_amdgcn_logf(al), kLog2Floor);
                gv[u][e] = run[e];
            }
        }
        if (p1) {
#pragma unroll
            for (int e = 0; e < 8; ++e) seg[sgi * DK + 8 * cg + e] = run[e];
        }
    }
    // v of this thread's tokens, kept in registers until the value tile is built
    const int NCGV = DV / 8;
    const bool pv = tid < I::NSEG * NCGV;
    const int sgv = tid / NCGV, cgv = tid % NCGV;
    float vr[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int r = 4 * sgv + u;
        const bool in = pv && r < valid;
        const int64_t base = ((pos.tok0 + r) * H + h) * DV + 8 * cgv;
#pragma unroll
        for (int e = 0; e < 8; ++e) vr[u][e] = in ? load_as_float(vg, base + e) : 0.f;
    }
    __syncthreads();
    float tot[8];
    if (p1) {
        float off[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) { off[e] = 0.f; tot[e] = 0.f; }
        for (int s = 0; s < I::NSEG; ++s) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float t = seg[s * DK + 8 * cg + e];
                if (s < sgi) off[e] += t;
                tot[e] += t;
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) gv[u][e] += off[e];   // inclusive exponent g_r
        if ((sgi & 3) == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) Gs[Rb * DK + 8 * cg + e] = gv[0][e];
        }
        if ((sgi & 3) == 3) {
#pragma unroll
            for (int e = 0; e < 8; ++e) Ge[Rb * DK + 8 * cg + e] = gv[3][e];
        }
    }
    __syncthreads();
    // block ranges decide the path; pair factors for the off-diagonal tiles
    if (p1 && (sgi & 3) == 0) {
        float mx = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, Gs[Rb * DK + 8 * cg + e] - Ge[Rb * DK + 8 * cg + e]);
        atomicMax(srange, __float_as_uint(mx));  // non-negative floats order like their bits
    }
    for (int e = tid; e < I::NOFF * DK; e += I::kThreads) {
        const int p = e / DK, c = e % DK;
        int R = 1;
        while (R * (R + 1) / 2 <= p) ++R;          // off-diagonal pair p = R(R-1)/2 + Ib
        const int Ib = p - R * (R - 1) / 2;
        const float hR = 0.5f * (Gs[R * DK + c] - Ge[R * DK + c]);
        sIR[e] = __builtin_amdgcn_exp2f(fminf(Gs[R * DK + c] - Gs[(Ib + 1) * DK + c] - hR, 0.f));
    }
    __syncthreads();
    const bool fast = __uint_as_float(*srange) <= kFastRange;
    if (p1) {
        float kbar[4][8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int c = 8 * cg + e;
            const float G0 = Gs[Rb * DK + c];
            const float hR = 0.5f * (G0 - Ge[Rb * DK + c]);
            const bool last = Rb == NB - 1;
            const float Gn = last ? 0.f : Gs[(Rb + 1) * DK + c];
            // 2^{g_C - G_{R+1}} links the off-diagonal column factor to Kbar
            const float link = last ? 1.f : __builtin_amdgcn_exp2f(fminf(tot[e] - Gn, 0.f));
            const float gb = __builtin_amdgcn_exp2f(fminf(G0 - hR, 0.f));
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int r = 4 * sgi + u;
                const float gr = gv[u][e];
                float gam_r, kb_f;
                if (fast) {
                    const float fa = __builtin_amdgcn_exp2f(gr - G0 + hR);   // in 2^[-h, h]
                    const float fb = __builtin_amdgcn_rcpf(fa);
                    Ak[r * LD_ROW + c] = (T)(kr[u][e] * fa);
                    Aq[r * LD_ROW + c] = (T)(qr[u][e] * fa);
                    Bd[r * LD_ROW + c] = (T)(kr[u][e] * fb);
                    gam_r = fa * gb;                                        // 2^{g_r}
                    if (!last) {
                        const float fo = __builtin_amdgcn_exp2f(fminf(Gn - gr, 0.f));
                        Bo[r * LD_ROW + c] = (T)(kr[u][e] * fo);
                        kb_f = fo * link;                                    // 2^{g_C - g_r}
                    } else {
                        kb_f = __builtin_amdgcn_exp2f(fminf(tot[e] - gr, 0.f));
                    }
                } else {
                    gam_r = __builtin_amdgcn_exp2f(gr);
                    kb_f = __builtin_amdgcn_exp2f(fminf(tot[e] - gr, 0.f));
                }
                KtT[c * LD_CT + r] = (T)(kr[u][e] * gam_r);   // Ktilde, transposed
                qr[u][e] *= gam_r;                            // Qtilde
                kbar[u][e] = kr[u][e] * kb_f;                 // Kbar
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = 4 * sgi + u;
#pragma unroll
            for (int hq = 0; hq < 2; ++hq) {  // Qtilde quads: token r, channel groups 2cg, 2cg+1
                const int a4 = 2 * cg + hq, ut = a4 >> 2, gq = a4 & 3;
                const f32x4 v4{qr[u][4 * hq], qr[u][4 * hq + 1], qr[u][4 * hq + 2], qr[u][4 * hq + 3]};
                *reinterpret_cast<Q*>(Qf + Frag<T>::off(r >> 4, ut, 16 * gq + (r & 15), DK)) = make_quad<T>(v4);
            }
        }
        {   // Kbar^T quads: channel c, tokens 4*sgi .. 4*sgi+3
            const int ut = sgi >> 2, gq = sgi & 3;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int c = 8 * cg + e;
                const f32x4 v4{kbar[0][e], kbar[1][e], kbar[2][e], kbar[3][e]};
                *reinterpret_cast<Q*>(Kbf + Frag<T>::off(c >> 4, ut, 16 * gq + (c & 15), C)) = make_quad<T>(v4);
            }
        }
        if (sgi == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) gam[8 * cg + e] = __builtin_amdgcn_exp2f(tot[e]);
        }
    }
    __syncthreads();

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
                if (Ib == R) {
#pragma unroll
                    for (int u = 0; u < NQK; ++u)
                        aq[u] = *reinterpret_cast<const Q*>(Bd + (16 * Ib + cl) * LD_ROW + 16 * u + 4 * g);
                } else {
                    const float* sp = sIR + (R * (R - 1) / 2 + Ib) * DK;
#pragma unroll
                    for (int u = 0; u < NQK; ++u) {
                        const f32x4 bo = from_quad(*reinterpret_cast<const Q*>(Bo + (16 * Ib + cl) * LD_ROW + 16 * u + 4 * g));
                        const f32x4 sf = *reinterpret_cast<const f32x4*>(sp + 16 * u + 4 * g);
                        aq[u] = make_quad<T>(bo * sf);
                    }
                }
#pragma unroll
                for (int u = 0; u < NQK; ++u) {
                    bk[u] = *reinterpret_cast<const Q*>(Ak + (16 * R + cl) * LD_ROW + 16 * u + 4 * g);
                    bq[u] = *reinterpret_cast<const Q*>(Aq + (16 * R + cl) * LD_ROW + 16 * u + 4 * g);
                }
                mres[pi] = mma_quads(aq, bk, zero4());
                pres[pi] = mma_quads(aq, bq, zero4());
            }
        }
        __syncthreads();  // the operand tiles are dead from here on; P/M/X reuse them
#pragma unroll
        for (int pi = 0; pi < MAXP; ++pi) {
            const int p = wave + 4 * pi;
            if (p < NP) {
                // lane holds M'^T[i = 16Ib + 4g + j][r = 16R + cl] for j = 0..3
                const int r = 16 * pR[pi] + cl, i0 = 16 * pI[pi] + 4 * g;
                const float br = sbeta[r];
                f32x4 mv, pvv;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    mv[j] = (i0 + j < r) ? br * mres[pi][j] : 0.f;
                    pvv[j] = (i0 + j <= r) ? pres[pi][j] : 0.f;
                }
                *reinterpret_cast<f32x4*>(Mm + r * LD_F + i0) = mv;
                *reinterpret_cast<f32x4*>(Pm + r * LD_F + i0) = pvv;
            }
        }
    } else {
        // exact pairwise path: decay products taken in linear space
        for (int e = tid; e < 2 * C * LD_F; e += I::kThreads) Pm[e] = 0.f;  // P and M
        __syncthreads();
        constexpr int PARTS = I::kThreads / C;
        constexpr int CPP = DK / PARTS;
        const int i = tid % C, part = tid / C, c0 = part * CPP;
        if (i < valid) {
            float ki[CPP], pr[CPP];
            const int64_t bi = ((pos.tok0 + i) * H + h) * DK + c0;
#pragma unroll
            for (int c = 0; c < CPP; ++c) { ki[c] = load_as_float(kg, bi + c); pr[c] = 1.f; }
            for (int r = i; r < valid; ++r) {
                const int64_t br = ((pos.tok0 + r) * H + h) * DK + c0;
                float m = 0.f, pp = 0.f;
#pragma unroll
                for (int c = 0; c < CPP; ++c) {
                    if (r > i) pr[c] *= a.alpha[br + c];
                    const float w = ki[c] * pr[c];
                    m += load_as_float(kg, br + c) * w;
                    pp += load_as_float(qg, br + c) * w;
                }
                if (r > i) atomicAdd(&Mm[r * LD_F + i], sbeta[r] * m);
                atomicAdd(&Pm[r * LD_F + i], pp);
            }
        }
    }
    __syncthreads();

    // ---- phase 3: X = (I + M)^{-1}, blocked over 16-token blocks -------------
    if (tid < C) {  // diagonal blocks by forward substitution, one column each
        const int R = tid >> 4, ci = tid & 15, b0 = 16 * R;
        float xv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) xv[r] = (r == ci) ? 1.f : 0.f;
#pragma unroll
        for (int r = 1; r < 16; ++r) {
            if (r > ci) {
                float s = 0.f;
#pragma unroll
                for (int j = 0; j < r; ++j) s += Mm[(b0 + r) * LD_F + b0 + j] * xv[j];
                xv[r] = -s;
            }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) Xm[(b0 + r) * LD_F + b0 + ci] = xv[r];
    }
    __syncthreads();
#pragma unroll
    for (int d = 1; d < NB; ++d) {
        // Y_RI = sum_{J=I}^{R-1} M_RJ X_JI, then X_RI = -X_RR Y_RI, for R - I = d
        const int nel = (NB - d) * 256;
        for (int e = tid; e < nel; e += I::kThreads) {
            const int Ib = e >> 8, R = Ib + d, rr = (e >> 4) & 15, ii = e & 15;
            float y = 0.f;
            for (int J = Ib; J < R; ++J)
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    y += Mm[(16 * R + rr) * LD_F + 16 * J + j] * Xm[(16 * J + j) * LD_F + 16 * Ib + ii];
            Ys[e] = y;
        }
        __syncthreads();
        for (int e = tid; e < nel; e += I::kThreads) {
            const int Ib = e >> 8, R = Ib + d, rr = (e >> 4) & 15, ii = e & 15;
            float xs = 0.f;
#pragma unroll
            for (int j = 0; j < 16; ++j)
                xs += Xm[(16 * R + rr) * LD_F + 16 * R + j] * Ys[(Ib << 8) + (j << 4) + ii];
            Xm[(16 * R + rr) * LD_F + 16 * Ib + ii] = -xs;
        }
        __syncthreads();
    }
    // Tm = X diag(beta), lower triangle, in the operand type
    for (int e = tid; e < C * C; e += I::kThreads) {
        const int r = e / C, i = e % C;
        Tb[r * LD_CT + i] = (T)(i <= r ? Xm[r * LD_F + i] * sbeta[i] : 0.f);
    }
    __syncthreads();

    // ---- phase 4: value tile, P fragments, W = Tm Ktilde, Utilde = Tm V ------
    if (pv) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int u = 0; u < 4; ++u) VT[(8 * cgv + e) * LD_CT + 4 * sgv + u] = (T)vr[u][e];
    }
    for (int e = tid; e < NB * NB * 64; e += I::kThreads) {
        const int ct = e / (NB * 64), ut = (e / 64) % NB, ln = e & 63;
        const int r = 16 * ct + (ln & 15), i0 = 16 * ut + 4 * (ln >> 4);
        const f32x4 v4 = ut <= ct ? *reinterpret_cast<const f32x4*>(Pm + r * LD_F + i0) : zero4();
        *reinterpret_cast<Q*>(Pf + Frag<T>::off(ct, ut, ln, C)) = make_quad<T>(v4);
    }
    __syncthreads();
    // W^T(channel tile t, token tile tb) = Ktilde^T Tm^T: lane holds W[16tb+cl][16t+4g+j]
    for (int tile = wave; tile < NQK * NB; tile += 4) {
        const int t = tile / NB, tb = tile % NB;
        Q aq[NB], bq[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            aq[u] = *reinterpret_cast<const Q*>(KtT + (16 * t + cl) * LD_CT + 16 * u + 4 * g);
            bq[u] = *reinterpret_cast<const Q*>(Tb + (16 * tb + cl) * LD_CT + 16 * u + 4 * g);
        }
        const f32x4 res = mma_quads_upto(aq, bq, tb, zero4());
        *reinterpret_cast<Q*>(Wf + Frag<T>::off(tb, t, lane, DK)) = make_quad<T>(res);
    }
    // Utilde(token tile tb, value tile s) = Tm V: lane holds U[16tb+4g+j][16s+cl]
    const int NSV = DV / 16;
    for (int tile = wave; tile < NB * NSV; tile += 4) {
        const int tb = tile / NSV, s = tile % NSV;
        Q aq[NB], bq[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            aq[u] = *reinterpret_cast<const Q*>(Tb + (16 * tb + cl) * LD_CT + 16 * u + 4 * g);
            bq[u] = *reinterpret_cast<const Q*>(VT + (16 * s + cl) * LD_CT + 16 * u + 4 * g);
        }
        const f32x4 res = mma_quads_upto(aq, bq, tb, zero4());
        *reinterpret_cast<Q*>(Uf + ((int64_t)(s * 64 + lane) * NB + tb) * 4) = make_quad<T>(res);
    }
}

// ---------------------------------------------------------------------------
// K2: inter-chunk pass.  One wave per (sequence, head, 16 value columns).
// ---------------------------------------------------------------------------
template <int DK, int C, typename In>
__global__ __launch_bounds__(64) void kda_inter_kernel(const PrefillArgs a) {
    using T = typename OperandOf<In>::type;
    using Q = quad_t<T>;
    constexpr int NB = C / 16, NQK = DK / 16;
    const int lane = threadIdx.x, g = lane >> 4, cl = lane & 15;
    const int NS = a.DV / 16;
    // blocks are dealt round-robin over the 8 XCDs: keep the slices of one
    // (sequence, head) on one XCD so they share its L2
    const int b = blockIdx.x, xcd = b & 7, jx = b >> 3;
    const int s = jx % NS;
    const int unit = (jx / NS) * 8 + xcd;
    if (unit >= a.N * a.H) return;
    const int n = unit / a.H, h = unit % a.H;
    const int H = a.H, DV = a.DV;
    const int col = 16 * s + cl;

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

    // S slice in accumulator layout: acc[t][j] = S[16t + 4g + j][col]
    f32x4 acc[NQK];
    const int64_t sbase = (int64_t)unit * DK * DV;
#pragma unroll
    for (int t = 0; t < NQK; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[t][j] = a.s0 ? a.s0[sbase + (int64_t)(16 * t + 4 * g + j) * DV + col] : 0.f;

    const ChunkBlock<T> cb(DK, C, DV);
    for (int x = c_begin; x < c_end; ++x) {
        const int jc = x - c_begin;
        const int64_t tok0 = tok_begin + (int64_t)jc * C;
        const int valid = (int)min((int64_t)C, seq_len - (int64_t)jc * C);
        const char* blk = a.ws_chunks + ((int64_t)x * H + h) * cb.bytes;
        const T* Wf = reinterpret_cast<const T*>(blk + cb.w);
        const T* Qf = reinterpret_cast<const T*>(blk + cb.q);
        const T* Kbf = reinterpret_cast<const T*>(blk + cb.kb);
        const T* Pf = reinterpret_cast<const T*>(blk + cb.p);
        const T* Uf = reinterpret_cast<const T*>(blk + cb.u);
        const float* gam = reinterpret_cast<const float*>(blk + cb.gam);

        Q sb[NQK];
#pragma unroll
        for (int t = 0; t < NQK; ++t) sb[t] = make_quad<T>(acc[t]);

        // U = Utilde - W S   (lane: tokens 16tb + 4g + j, column col)
        Q ub[NB];
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
            Q wq[NQK];
#pragma unroll
            for (int u = 0; u < NQK; ++u) wq[u] = *reinterpret_cast<const Q*>(Wf + Frag<T>::off(tb, u, lane, DK));
            const f32x4 xw = mma_quads(wq, sb, zero4());
            const f32x4 ut = from_quad(*reinterpret_cast<const Q*>(Uf + ((int64_t)(s * 64 + lane) * NB + tb) * 4));
            ub[tb] = make_quad<T>(ut - xw);
        }
        // O^T = S^T Qtilde^T + U^T P^T   (lane: columns 4g + j, token 16tb + cl)
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
            Q qq[NQK], pq[NB];
#pragma unroll
            for (int u = 0; u < NQK; ++u) qq[u] = *reinterpret_cast<const Q*>(Qf + Frag<T>::off(tb, u, lane, DK));
#pragma unroll
            for (int u = 0; u < NB; ++u) pq[u] = *reinterpret_cast<const Q*>(Pf + Frag<T>::off(tb, u, lane, C));
            f32x4 ot = mma_quads(sb, qq, zero4());
            ot = mma_quads_upto(ub, pq, tb, ot);
            const int r = 16 * tb + cl;
            if (r < valid) {
                const f32x4 sc = ot * a.scale;
                const int64_t oi = ((tok0 + r) * H + h) * DV + 16 * s + 4 * g;
                if (a.o_f32) store4(reinterpret_cast<float*>(a.o) + oi, sc);
                else store4(reinterpret_cast<__bf16*>(a.o) + oi, sc);
            }
        }
        // S <- diag(gamma_C) S + Kbar^T U
#pragma unroll
        for (int t = 0; t < NQK; ++t) {
            const f32x4 gv = *reinterpret_cast<const f32x4*>(gam + 16 * t + 4 * g);
            Q kq[NB];
#pragma unroll
            for (int u = 0; u < NB; ++u) kq[u] = *reinterpret_cast<const Q*>(Kbf + Frag<T>::off(t, u, lane, C));
            acc[t] = mma_quads(kq, ub, acc[t] * gv);
        }
    }
    if (a.s_final) {
#pragma unroll
        for (int t = 0; t < NQK; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) a.s_final[sbase + (int64_t)(16 * t + 4 * g + j) * DV + col] = acc[t][j];
    }
}

// ---------------------------------------------------------------------------
// Host-side launchers (called from the C ABI after validation).
// ---------------------------------------------------------------------------
template <int DK, int C, typename In>
static hipError_t launch_phase_t(const PrefillArgs& a, int max_chunks, bool intra, hipStream_t stream) {
    if constexpr (!Intra<DK, C, typename OperandOf<In>::type>::kFits) {
        return hipErrorInvalidValue;  // effective_chunk() never selects this
    } else {
        if (intra) {
            if (max_chunks > 0) {
                hipLaunchKernelGGL((kda_intra_kernel<DK, C, In>), dim3(max_chunks, a.H), dim3(256), 0, stream, a);
            }
        } else {
            const int units = a.N * a.H;
            const int blocks = ((units + 7) / 8) * 8 * (a.DV / 16);
            hipLaunchKernelGGL((kda_inter_kernel<DK, C, In>), dim3(blocks), dim3(64), 0, stream, a);
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
#define KDA_FITS_CASE(D, CC) if (DK == D && C == CC) return Intra<D, CC, T>::kFits;
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

hipError_t launch_chunk_offsets(const int32_t* cu, int32_t n, int32_t C, int32_t* chunk_off, hipStream_t s) {
    hipLaunchKernelGGL(kda_chunk_offsets, dim3(1), dim3(256), 0, s, cu, n, C, chunk_off);
    return hipGetLastError();
}

hipError_t launch_intra(const PrefillArgs& a, int DK, int C, bool bf16, int max_chunks, hipStream_t s) {
    return bf16 ? launch_phase_k<__bf16>(a, DK, C, max_chunks, true, s)
                : launch_phase_k<float>(a, DK, C, max_chunks, true, s);
}

hipError_t launch_inter(const PrefillArgs& a, int DK, int C, bool bf16, hipStream_t s) {
    return bf16 ? launch_phase_k<__bf16>(a, DK, C, 0, false, s) : launch_phase_k<float>(a, DK, C, 0, false, s);
}

int64_t chunk_block_bytes(int DK, int C, int DV, bool bf16) {
    return bf16 ? ChunkBlock<_Float16>(DK, C, DV).bytes : ChunkBlock<float>(DK, C, DV).bytes;
}

}  // namespace kda
