// kda_decode.hip -- one KDA decode step on gfx950.
//
// Per (sequence, head), with the state S (dk x dv, fp32) updated in place:
//   S' = diag(alpha) S ;  r = S'^T k ;  S = S' + beta k (v - r)^T ;  o = scale S^T q
// ("Kimi K3 Architecture Teardown", Visual 5: decay, erase, write;
// "Kimi K3 architecture: KDA, MLA and MoE", section "KDA is a writable state,
// not a smaller KV cache": a query reads the current matrix instead of a
// growing cache).  Since S^T q = S'^T q + beta (q.k) (v - r), the output
// needs only the decayed state and two column reductions, so every state
// element is read once and written once: the step is bound by HBM bandwidth.
//
// The reductions r = S'^T k and y = S'^T q run over rows, independently per
// value column, so a state can split by columns without any exchange: one
// workgroup per (sequence, head, block of DVW columns).  Thread (row group r0,
// column group cg) owns float4 columns [4cg, 4cg+4) of the block in rows r0,
// r0 + RPP, ... and keeps them in registers between the reduction and the
// write-back.  The write-back uses nontemporal (streaming) stores.  On MI355X
// the in-place step over 512 MiB of state measured 6.5 TB/s with whole
// 128 x 128 states per 256-thread workgroup (16 float4 of state per thread)
// and streaming stores (512 threads: 6.2-6.3 TB/s; 1,024: 6.4; 128: 5.5),
// against 5.1 TB/s with ordinary stores; streaming loads and smaller column
// blocks (64 columns: 5.0 TB/s) were slower.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_kernels.h"
#include "kda_quads.h"

namespace kda {

// Columns per workgroup (a whole 128-column row) and threads per workgroup.
constexpr int kDecodeCols = 128;
constexpr int kDecodeThreads = 256;

template <int DK, int DV> struct DecodeShape {
    static constexpr int DVW = DV < kDecodeCols ? DV : kDecodeCols;  // columns per workgroup
    static constexpr int CB = DV / DVW;                                     // column blocks per state
    static constexpr int CG = DVW / 4;                                      // threads per state row
    static constexpr int NT = (DK * DVW / 4) < kDecodeThreads ? (DK * DVW / 4) : kDecodeThreads;
    static constexpr int RPP = NT / CG;                                     // rows per pass
    static constexpr int PASSES = DK / RPP;
    static constexpr int NW = (NT + 63) / 64;
    static_assert(CG <= 64 && NT % CG == 0 && RPP * PASSES == DK, "decode thread mapping");
};

__device__ __forceinline__ float sigmoid(float x) { return 1.f / (1.f + __expf(-x)); }

template <int DK, int DV, typename T>
__global__ __launch_bounds__((DecodeShape<DK, DV>::NT)) void kda_decode_kernel(const DecodeArgs a) {
    using D = DecodeShape<DK, DV>;
    constexpr int CG = D::CG, RPP = D::RPP, PASSES = D::PASSES, NW = D::NW, DVW = D::DVW;
    __shared__ float sq[DK], sk[DK], sa[DK], sv[DVW];
    __shared__ f32x4 red_r[NW][CG], red_y[NW][CG];
    __shared__ float sqk, siq, sik;

    const int unit = blockIdx.x / D::CB;        // n * H + h
    const int col0 = (blockIdx.x % D::CB) * DVW;  // first value column of this workgroup
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cg = tid % CG, r0 = tid / CG;
    // state of this (sequence, head): its own, or a pool entry
    const int slot = a.slots ? a.slots[unit / a.H] : 0;
    if (a.slots && a.pool_entries > 0 && (slot < 0 || slot >= a.pool_entries)) {
        // a slot outside the pool: no state is touched, o reads NaN (uniform over the workgroup)
        if (r0 == 0) {
            const f32x4 nan4 = zero4() + __builtin_nanf("");
            const int64_t oi = (int64_t)unit * DV + col0 + 4 * cg;
            if (a.o_f32) store4(reinterpret_cast<float*>(a.o) + oi, nan4);
            else store4(reinterpret_cast<__bf16*>(a.o) + oi, nan4);
        }
        return;
    }
    const int64_t sidx = a.slots ? (int64_t)slot * a.H + unit % a.H : (int64_t)unit;
    float* __restrict__ S = a.state + sidx * DK * DV + col0;

    // state rows of this thread: issue every load before anything else
    f32x4 s[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
        s[p] = *reinterpret_cast<const f32x4*>(S + (r0 + p * RPP) * DV + 4 * cg);

    const T* __restrict__ q = reinterpret_cast<const T*>(a.q) + (int64_t)unit * DK;
    const T* __restrict__ k = reinterpret_cast<const T*>(a.k) + (int64_t)unit * DK;
    const T* __restrict__ v = reinterpret_cast<const T*>(a.v) + (int64_t)unit * DV + col0;
    for (int i = tid; i < DK; i += D::NT) {
        sq[i] = load_as_float(q, i);
        sk[i] = load_as_float(k, i);
        float al = a.alpha_scalar ? a.alpha[unit] : a.alpha[(int64_t)unit * DK + i];
        if (a.fuse_inputs) al = sigmoid(al);
        sa[i] = fmaxf(al, a.alpha_floor);
    }
    for (int i = tid; i < DVW; i += D::NT) sv[i] = load_as_float(v, i);
    float beta = a.beta[unit];
    if (a.fuse_inputs) beta = sigmoid(beta);
    __syncthreads();
    if (wave == 0) {  // q.k and, for fused inputs, the inverse norms of q and k
        float t = 0.f, nq = 0.f, nk = 0.f;
        for (int i = lane; i < DK; i += 64) {
            t += sq[i] * sk[i];
            nq += sq[i] * sq[i];
            nk += sk[i] * sk[i];
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            t += __shfl_xor(t, m, 64);
            nq += __shfl_xor(nq, m, 64);
            nk += __shfl_xor(nk, m, 64);
        }
        if (lane == 0) {
            const float iq = a.fuse_inputs ? 1.f / fmaxf(sqrtf(nq), 1e-12f) : 1.f;
            const float ik = a.fuse_inputs ? 1.f / fmaxf(sqrtf(nk), 1e-12f) : 1.f;
            sqk = t * iq * ik;
            siq = iq;
            sik = ik;
        }
    }

    // decay, then the two column reductions r = S'^T k and y = S'^T q
    f32x4 racc = zero4(), yacc = zero4();
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int c = r0 + p * RPP;
        s[p] = s[p] * sa[c];
        racc += sk[c] * s[p];
        yacc += sq[c] * s[p];
    }
#pragma unroll
    for (int m = CG; m < 64 && m < D::NT; m <<= 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            racc[j] += __shfl_xor(racc[j], m, 64);
            yacc[j] += __shfl_xor(yacc[j], m, 64);
        }
    }
    if (lane < CG) {
        red_r[wave][cg] = racc;
        red_y[wave][cg] = yacc;
    }
    __syncthreads();
    f32x4 r = zero4(), y = zero4();
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        r += red_r[w][cg];
        y += red_y[w][cg];
    }
    // normalised q and k enter linearly: scale the reductions once
    const float iq = siq, ik = sik;
    r = r * ik;
    y = y * iq;
    const f32x4 vv{sv[4 * cg], sv[4 * cg + 1], sv[4 * cg + 2], sv[4 * cg + 3]};
    const f32x4 e = vv - r;  // correction towards the new value

    // erase and write with the same beta, back to the same addresses
    const float bk = beta * ik;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        const int c = r0 + p * RPP;
        const f32x4 ns = s[p] + (bk * sk[c]) * e;
        __builtin_nontemporal_store(ns, reinterpret_cast<f32x4*>(S + c * DV + 4 * cg));
    }
    if (r0 == 0) {  // the CG threads of the first row group: lanes 0 .. CG-1 of wave 0
        f32x4 o4 = (y + (beta * sqk) * e) * a.scale;
        const int64_t oi = (int64_t)unit * DV + col0 + 4 * cg;
        if (a.gate) {  // norm over the row (this workgroup holds all of it), weight, sigmoid gate
            float ss = o4[0] * o4[0] + o4[1] * o4[1] + o4[2] * o4[2] + o4[3] * o4[3];
#pragma unroll
            for (int m = 1; m < CG; m <<= 1) ss += __shfl_xor(ss, m, 64);
            const float inv = rsqrtf(ss / (float)DV + a.norm_eps);
            const T* __restrict__ gt = reinterpret_cast<const T*>(a.gate) + oi;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float w = a.norm_w ? a.norm_w[col0 + 4 * cg + j] : 1.f;
                o4[j] = o4[j] * inv * w * sigmoid(load_as_float(gt, j));
            }
        }
        if (a.o_f32) store4(reinterpret_cast<float*>(a.o) + oi, o4);
        else store4(reinterpret_cast<__bf16*>(a.o) + oi, o4);
    }
}

template <int DK, int DV, typename T>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s) {
    using D = DecodeShape<DK, DV>;
    hipLaunchKernelGGL((kda_decode_kernel<DK, DV, T>), dim3(a.units * D::CB), dim3(D::NT), 0, s, a);
    return hipGetLastError();
}

template <int DK, typename T>
static hipError_t launch_decode_v(const DecodeArgs& a, int DV, hipStream_t s) {
    switch (DV) {
        case 16: return launch_decode_t<DK, 16, T>(a, s);
        case 32: return launch_decode_t<DK, 32, T>(a, s);
        case 64: return launch_decode_t<DK, 64, T>(a, s);
        case 128: return launch_decode_t<DK, 128, T>(a, s);
    }
    return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_decode_k(const DecodeArgs& a, int DK, int DV, hipStream_t s) {
    switch (DK) {
        case 16: return launch_decode_v<16, T>(a, DV, s);
        case 32: return launch_decode_v<32, T>(a, DV, s);
        case 64: return launch_decode_v<64, T>(a, DV, s);
        case 128: return launch_decode_v<128, T>(a, DV, s);
    }
    return hipErrorInvalidValue;
}

int decode_columns(int DV) { return DV < kDecodeCols ? DV : kDecodeCols; }

hipError_t launch_decode(const DecodeArgs& a, int DK, int DV, bool bf16, hipStream_t s) {
    return bf16 ? launch_decode_k<__bf16>(a, DK, DV, s) : launch_decode_k<float>(a, DK, DV, s);
}

}  // namespace kda
