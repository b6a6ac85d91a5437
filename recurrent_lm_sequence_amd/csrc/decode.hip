// Single-token recurrent decode step on a persistent fp32 state.
//
// "Simple linear attention language models balance the recall-throughput
// tradeoff" notes, §2.5: decoding fuses the outer-product write into the state
// with the query read-out, and still reads and writes the whole persistent
// state every step -- the step is bound by HBM bandwidth.  §2.2 gives the
// step (s += phi(k) v^T, z += phi(k), y = s^T phi(q) / z^T phi(q)), §2.3 phi.
//
// One workgroup per (batch, head).  The D x DV fp32 state is streamed once:
// every thread owns 4 adjacent columns of rows rr, rr + RPP, ... (16-byte
// loads and stores; a wavefront covers whole contiguous rows), issues all its
// loads before any arithmetic so each CU keeps many rows in flight, updates
// them in registers, writes them back and accumulates its part of phi(q)^T S.
// The partial sums over rows are reduced through LDS.
//
// With the compact layout (kDc = 153 rows: each unordered feature pair once,
// holding S[a][b] + S[b][a]) the same step reads and writes 44% fewer bytes:
// the query feature of pair row {a, b} is xb_a xb_b / sqrt 2 and the key
// feature written into it carries the pair's multiplicity (2 off the
// diagonal), so phi_c(q)^T S_c equals phi(q)^T S of the full layout.
#include "common.h"

namespace bla {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

template <int DV, bool COMPACT>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a, int in_bf16)
{
    constexpr int T = 256;
    constexpr int ND = COMPACT ? kDc : kD;     // state rows
    constexpr int TPR = DV / 4;                // threads per state row
    constexpr int RPP = T / TPR;               // rows per pass
    constexpr int NP = (ND + RPP - 1) / RPP;   // passes
    constexpr int ZP = (ND + T - 1) / T;       // z rows per thread
    constexpr int NPAIR = kDc - 1 - kFeat;     // 136 unordered pairs
    __shared__ float xq[kFeat], xk[kFeat], vsh[DV];
    __shared__ f4 red[RPP][TPR];
    __shared__ float dred[T / 64];
    __shared__ unsigned char pa[COMPACT ? NPAIR : 1], pb[COMPACT ? NPAIR : 1];

    const int tid = threadIdx.x, cq = tid % TPR, rr = tid / TPR;
    const long head = blockIdx.x;
    f4 *Sh = (f4 *)(a.S + head * ND * DV);
    float *zh = a.z + head * ND;
    if (COMPACT && tid < NPAIR) {  // pair row -> (a, b), row-major upper triangle
        int ia = 0;
        while (ia + 1 < kFeat && compact_pair(ia + 1, ia + 1) <= tid) ++ia;
        pa[tid] = (unsigned char)ia;
        pb[tid] = (unsigned char)(ia + tid - compact_pair(ia, ia));
    }

    // issue every state load first
    f4 sv[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int d = rr + RPP * p;
        if (d < ND) sv[p] = Sh[d * TPR + cq];
    }
    float zv[ZP];
#pragma unroll
    for (int p = 0; p < ZP; ++p) {
        const int d = tid + T * p;
        if (d < ND) zv[p] = zh[d];
    }
    if (tid < 2 * kFeat) {
        const int f = tid % kFeat;
        const void *src = tid < kFeat ? a.q : a.k;
        const long idx = head * kFeat + f;
        const float x = in_bf16 ? bf16_to_f32(((const uint16_t *)src)[idx])
                                : ((const float *)src)[idx];
        (tid < kFeat ? xq : xk)[f] = 0.5f * x;  // x / d'^(1/4), d' = 16
    } else if (tid >= 64 && tid < 64 + DV) {
        const int c = tid - 64;
        const long idx = head * DV + c;
        vsh[c] = in_bf16 ? bf16_to_f32(((const uint16_t *)a.v)[idx]) : ((const float *)a.v)[idx];
    }
    __syncthreads();

    const float r2 = 0.70710678118654752440f;
    // feature of row d (full layout: pair (ab/16, ab%16); compact: pair row)
    auto phi = [&](int d, const float *x) -> float {
        if (d == 0) return 1.f;
        if (d <= kFeat) return x[d - 1];
        const int ab = d - 1 - kFeat;
        if (COMPACT) return x[pa[ab]] * x[pb[ab]] * r2;
        return x[ab >> 4] * x[ab & 15] * r2;
    };
    // multiplicity of row d among the full layout's rows (2 for an off-diagonal compact pair)
    auto mult = [&](int d) -> float {
        if (!COMPACT || d <= kFeat) return 1.f;
        return pa[d - 1 - kFeat] == pb[d - 1 - kFeat] ? 1.f : 2.f;
    };

    const f4 v4 = *(const f4 *)(vsh + 4 * cq);
    f4 num = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int d = rr + RPP * p;
        if (d < ND) {
            const float fk = mult(d) * phi(d, xk), fq = phi(d, xq);
            const f4 s = sv[p] + fk * v4;
            Sh[d * TPR + cq] = s;
            num += fq * s;
        }
    }
    float den = 0.f;
#pragma unroll
    for (int p = 0; p < ZP; ++p) {
        const int d = tid + T * p;
        if (d < ND) {
            const float zn = zv[p] + mult(d) * phi(d, xk);
            zh[d] = zn;
            den += phi(d, xq) * zn;
        }
    }
    red[rr][cq] = num;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) den += __shfl_xor(den, o);
    if ((tid & 63) == 0) dred[tid >> 6] = den;
    __syncthreads();
    if (tid < DV) {
        const int q4 = tid / 4, e = tid % 4;
        float sum = 0.f;
        for (int r = 0; r < RPP; ++r) sum += red[r][q4][e];
        float dn = 0.f;
#pragma unroll
        for (int wv = 0; wv < T / 64; ++wv) dn += dred[wv];
        const float yv = sum / (dn + a.eps);
        if (a.y) {
            const long o = head * DV + tid;
            if (a.y_bf16)
                ((uint16_t *)a.y)[o] = f32_to_bf16_rne(yv);
            else
                ((float *)a.y)[o] = yv;
        }
    }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, int in_bf16, hipStream_t s)
{
    const dim3 grid((unsigned)(a.B * a.H));
    if (a.compact) {
        switch (a.dv) {
        case 16: hipLaunchKernelGGL((decode_kernel<16, true>), grid, dim3(256), 0, s, a, in_bf16); break;
        case 32: hipLaunchKernelGGL((decode_kernel<32, true>), grid, dim3(256), 0, s, a, in_bf16); break;
        default: hipLaunchKernelGGL((decode_kernel<64, true>), grid, dim3(256), 0, s, a, in_bf16); break;
        }
    } else {
        switch (a.dv) {
        case 16: hipLaunchKernelGGL((decode_kernel<16, false>), grid, dim3(256), 0, s, a, in_bf16); break;
        case 32: hipLaunchKernelGGL((decode_kernel<32, false>), grid, dim3(256), 0, s, a, in_bf16); break;
        default: hipLaunchKernelGGL((decode_kernel<64, false>), grid, dim3(256), 0, s, a, in_bf16); break;
        }
    }
    return hipGetLastError();
}

}  // namespace bla
