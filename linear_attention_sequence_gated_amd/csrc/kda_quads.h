// kda_quads.h -- matrix-core building blocks for the KDA kernels (gfx950).
//
// Every contraction in the chunked KDA form is expressed on 16x16 output
// tiles with the CDNA4 MFMA instructions.  One lane of a wave64 holds, for
// the row (A operand) or column (B operand) l % 16 of its tile, "quads": four
// consecutive k-indices 16*u + 4*(l/16) + {0,1,2,3} of the u-th 16-wide slice
// of the contraction axis.  This is exactly what the accumulator of a 16x16
// MFMA tile holds per lane (rows 4*(l/16) + i of column l % 16), so a result
// tile can feed the next contraction as a B operand (or as the A operand of
// the transposed product) without moving data between lanes.
//
// Operand precision.  bf16 inputs are computed with fp16 operands: the
// max-abs/RMS parity bound of 2e-2 leaves no room for the 8-bit bf16
// mantissa in the intermediates (every bf16 rounding of an intermediate costs
// about 1-3e-2 in that measure on its own), while fp16's 11 bits keep the
// whole chain near 1e-2 and run at the same MFMA rate on gfx950.  fp32 inputs
// are computed in fp32 throughout.
//  * fp16 operands: two quads (u, u+1) form the 8 halves of one
//    v_mfma_f32_16x16x32_f16 k-step; a trailing single quad uses
//    v_mfma_f32_16x16x16_f16.
//  * fp32 operands: one quad is four v_mfma_f32_16x16x4_f32 k-steps.
// Accumulation is fp32 in both cases.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef _Float16 f16x4 __attribute__((__vector_size__(4 * sizeof(_Float16))));
typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));

template <typename T> struct QuadOf;
template <> struct QuadOf<float> { using type = f32x4; static constexpr int kPerStep = 1; };
template <> struct QuadOf<_Float16> { using type = f16x4; static constexpr int kPerStep = 2; };
template <typename T> using quad_t = typename QuadOf<T>::type;

// Storage type of the inputs q, k, v and the operand type they are computed in.
template <typename In> struct OperandOf;
template <> struct OperandOf<float> { using type = float; };
template <> struct OperandOf<__bf16> { using type = _Float16; };

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// fp32 -> quad (round to nearest even).
__device__ __forceinline__ void to_quad(const f32x4& x, f32x4& q) { q = x; }
__device__ __forceinline__ void to_quad(const f32x4& x, f16x4& q) {
    q = f16x4{(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
}
__device__ __forceinline__ void to_quad(const f32x4& x, bf16x4& q) {
    q = bf16x4{(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
}
template <typename T> __device__ __forceinline__ quad_t<T> make_quad(const f32x4& x) {
    quad_t<T> q;
    to_quad(x, q);
    return q;
}
__device__ __forceinline__ f32x4 from_quad(const f32x4& q) { return q; }
__device__ __forceinline__ f32x4 from_quad(const f16x4& q) {
    return f32x4{(float)q[0], (float)q[1], (float)q[2], (float)q[3]};
}

// c += A(quads a[0..n)) * B(quads b[0..n)) over one 16x16 tile.
__device__ __forceinline__ f32x4 mma_step(const f32x4& a, const f32x4& b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    return c;
}
__device__ __forceinline__ f32x4 mma_step(const f16x4& a, const f16x4& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_step2(const f16x4& a0, const f16x4& a1, const f16x4& b0,
                                           const f16x4& b1, f32x4 c) {
    const f16x8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
    const f16x8 b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_step2(const f32x4& a0, const f32x4& a1, const f32x4& b0,
                                           const f32x4& b1, f32x4 c) {
    return mma_step(a1, b1, mma_step(a0, b0, c));
}

// A K=16 fp16 step never takes its accumulator from a K=32 step: when the two
// opcodes (of different pass counts) issue back to back as one accumulation
// chain, gfx950 returned stale rows in the short step's result.  An odd
// trailing quad therefore accumulates from zero and is added on the VALU.
template <typename Q>
__device__ __forceinline__ f32x4 mma_tail(const Q& a, const Q& b, f32x4 c) {
    if constexpr (sizeof(Q) == sizeof(f16x4)) return c + mma_step(a, b, zero4());
    else return mma_step(a, b, c);
}

// c += sum over quads u in [0, N) of A_u * B_u, with N a compile-time count.
template <int N, typename Q>
__device__ __forceinline__ f32x4 mma_quads(const Q (&a)[N], const Q (&b)[N], f32x4 c) {
#pragma unroll
    for (int u = 0; u + 1 < N; u += 2) c = mma_step2(a[u], a[u + 1], b[u], b[u + 1], c);
    if constexpr (N % 2 == 1) c = mma_tail(a[N - 1], b[N - 1], c);
    return c;
}

// Same, but only quads u <= last contribute (lower-triangular operands whose
// quads above `last` are zero in memory; pairs are kept whole).
template <int N, typename Q>
__device__ __forceinline__ f32x4 mma_quads_upto(const Q (&a)[N], const Q (&b)[N], int last, f32x4 c) {
#pragma unroll
    for (int u = 0; u + 1 < N; u += 2)
        if (u <= last) c = mma_step2(a[u], a[u + 1], b[u], b[u + 1], c);
    if constexpr (N % 2 == 1) {
        if (N - 1 <= last) c = mma_tail(a[N - 1], b[N - 1], c);
    }
    return c;
}

// c0 += A B0 and c1 += A B1 over N quads, the two chains issued alternately.
template <int N, typename Q>
__device__ __forceinline__ void mma_quads_pair(const Q (&a)[N], const Q (&b0)[N], const Q (&b1)[N], f32x4& c0,
                                               f32x4& c1) {
#pragma unroll
    for (int u = 0; u + 1 < N; u += 2) {
        c0 = mma_step2(a[u], a[u + 1], b0[u], b0[u + 1], c0);
        c1 = mma_step2(a[u], a[u + 1], b1[u], b1[u + 1], c1);
    }
    if constexpr (N % 2 == 1) {
        c0 = mma_tail(a[N - 1], b0[N - 1], c0);
        c1 = mma_tail(a[N - 1], b1[N - 1], c1);
    }
}

// c[i] += sum over quads u in [0, N) of A_i,u * B_u for NT tiles that share
// their B quads, issued K-step by K-step across the tiles: consecutive MFMAs
// then write different accumulators, where the tile-by-tile order makes each
// MFMA wait for the one before it.
template <int NT, int N, typename Q>
__device__ __forceinline__ void mma_tiles(const Q (&a)[NT][N], const Q (&b)[N], f32x4 (&c)[NT]) {
#pragma unroll
    for (int u = 0; u + 1 < N; u += 2)
#pragma unroll
        for (int i = 0; i < NT; ++i) c[i] = mma_step2(a[i][u], a[i][u + 1], b[u], b[u + 1], c[i]);
    if constexpr (N % 2 == 1) {
#pragma unroll
        for (int i = 0; i < NT; ++i) c[i] = mma_tail(a[i][N - 1], b[N - 1], c[i]);
    }
}

// Fragment storage in global memory: a matrix of `rows` (multiple of 16) by
// K (multiple of 16) stored so that lane l of the wave that consumes row tile
// rt reads its quads of k-slices [kPerStep*gq, kPerStep*gq + kPerStep) as one
// contiguous 8- or 16-byte vector.  Offsets are in elements of T.
template <typename T> struct Frag {
    static constexpr int kPerStep = QuadOf<T>::kPerStep;
    __host__ __device__ static constexpr int groups(int K) { return (K / 16 + kPerStep - 1) / kPerStep; }
    __host__ __device__ static constexpr int64_t elems(int rows, int K) {
        return (int64_t)(rows / 16) * groups(K) * 64 * 4 * kPerStep;
    }
    __host__ __device__ static constexpr int64_t off(int rt, int u, int lane, int K) {
        return (((int64_t)rt * groups(K) + u / kPerStep) * 64 + lane) * (4 * kPerStep) + (u % kPerStep) * 4;
    }
};

// Per-(chunk, head) block that the intra-chunk kernel writes and the
// inter-chunk kernel reads.  Offsets in bytes; every region is a multiple of
// 1 KiB so that one wave moves it with whole 64-lane x 16-byte transfers.
//   [W | Qtilde | Kbar^T | P | gamma_C (padded)]  shared by all value slices
//   [Utilde of slice group 0 | group 1 | ...]      gsl slices of 16 columns each
// A slice group is what one inter-chunk workgroup owns: it copies the shared
// region and its group's Utilde slices into LDS for every chunk.  The chunk
// chain of a (sequence, head) is serial, so one slice per workgroup spreads a
// few long sequences over every CU (32 heads x 8 slices fill 256 CUs); the
// price is that each slice's workgroup reads the shared region from L2 itself.
constexpr int kGroupSlices = 1;
__host__ __device__ constexpr int64_t round_kib(int64_t x) { return (x + 1023) / 1024 * 1024; }
__host__ __device__ constexpr int group_slices(int DV) { return DV / 16 < kGroupSlices ? DV / 16 : kGroupSlices; }

template <typename T> struct ChunkBlock {
    int64_t w, q, kb, p, gam, shared, u, slice, group, bytes;
    int gsl;
    __host__ __device__ ChunkBlock(int DK, int C, int DV, int slices_per_group) {
        const int64_t s = sizeof(T);
        w = 0;                                   // W = T Ktilde      : C x DK frag
        q = w + Frag<T>::elems(C, DK) * s;       // Qtilde            : C x DK frag
        kb = q + Frag<T>::elems(C, DK) * s;      // Kbar^T            : DK x C frag
        p = kb + Frag<T>::elems(DK, C) * s;      // P (as P^T B-frag) : C x C frag
        gam = p + Frag<T>::elems(C, C) * s;      // gamma_C           : DK fp32
        shared = gam + round_kib((int64_t)DK * 4);
        gsl = slices_per_group;
        slice = (int64_t)C * 16 * s;             // Utilde slice      : [64 lanes][C/16][4]
        group = round_kib(gsl * slice);
        u = shared;
        bytes = shared + (int64_t)(DV / 16 / gsl) * group;
    }
    __host__ __device__ int64_t u_slice(int sl) const { return u + (sl / gsl) * group + (sl % gsl) * slice; }
};

__device__ __forceinline__ float load_as_float(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_as_float(const __bf16* p, int64_t i) { return (float)p[i]; }

// Eight consecutive elements (16-byte aligned) as fp32, in as few vector loads as possible.
__device__ __forceinline__ void load8(const float* p, float (&o)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { o[i] = a[i]; o[4 + i] = b[i]; }
}
__device__ __forceinline__ void load8(const __bf16* p, float (&o)[8]) {
    typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (float)a[i];
}
// Eight consecutive elements kept as loaded (one or two 16-byte vectors) and
// converted to fp32 where they are used, so that the wait for a load sits at
// its first use rather than right after it is issued.
template <typename In> struct Raw8;
template <> struct Raw8<__bf16> {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    u32x4 w;  // element 2i in the low half of word i
    __device__ __forceinline__ void load(const __bf16* p) { w = *reinterpret_cast<const u32x4*>(p); }
    __device__ __forceinline__ void zero() { w = u32x4{0u, 0u, 0u, 0u}; }
    __device__ __forceinline__ void unpack(float (&o)[8]) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = __uint_as_float(w[i] << 16);
            o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
};
template <> struct Raw8<float> {
    f32x4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = *reinterpret_cast<const f32x4*>(p);
        b = *reinterpret_cast<const f32x4*>(p + 4);
    }
    __device__ __forceinline__ void zero() { a = f32x4{0.f, 0.f, 0.f, 0.f}; b = a; }
    __device__ __forceinline__ void unpack(float (&o)[8]) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) { o[i] = a[i]; o[4 + i] = b[i]; }
    }
};

// Eight consecutive values to LDS in the operand type (16- or 32-byte vector stores).
__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}
__device__ __forceinline__ void store8(_Float16* p, const float (&v)[8]) {
    *reinterpret_cast<f16x8*>(p) = f16x8{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3],
                                         (_Float16)v[4], (_Float16)v[5], (_Float16)v[6], (_Float16)v[7]};
}
template <typename T> __device__ __forceinline__ void store_q(T* p, const f32x4& v) {
    *reinterpret_cast<quad_t<T>*>(p) = make_quad<T>(v);
}

// Store four fp32 values as fp32 (16 bytes) or bf16 (8 bytes, round to nearest even).
__device__ __forceinline__ void store4(float* p, const f32x4& v) { *reinterpret_cast<f32x4*>(p) = v; }
__device__ __forceinline__ void store4(__bf16* p, const f32x4& v) {
    bf16x4 q;
    to_quad(v, q);
    *reinterpret_cast<bf16x4*>(p) = q;
}

}  // namespace kda
