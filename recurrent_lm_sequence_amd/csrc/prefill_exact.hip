// Token-sequential Taylor linear-attention prefill with fp64 accumulation.
//
// This is the precision path of the library, used for fp32 inputs: it runs
// the recurrence of the "Simple linear attention language models balance the
// recall-throughput tradeoff" notes, §2.2, token by token (update with k_i,
// v_i, then read with q_i), with phi from §2.3, the JRT prefix sums of the
// "Just read twice" notes §2.6 first, and an optional initial state
// (length-generalization notes §2.5, Eq. (4)).
//
// One workgroup per (batch, head).  Thread t owns value column t % DV and the
// feature rows d = t/DV + NRG*p of S and z, in fp64 registers.  Per block of
// TB tokens the features phi(k), phi(q) of every row are computed once into
// LDS, and the per-thread partial numerators/denominators go through LDS and
// are reduced once, so there are three barriers per TB tokens.
// COMPACT: the state is held and exchanged in the compact layout (kDc rows,
// each unordered feature pair once; see common.h), where the key feature of an
// off-diagonal pair row carries multiplicity 2.
#include "common.h"

namespace bla {
namespace {

constexpr int TB = 8;  // tokens per reduction block


template <int DV, int T, bool COMPACT>
__global__ __launch_bounds__(T) void prefill_exact_kernel(PrefillArgs a, int in_bf16)
{
    constexpr int ND = COMPACT ? kDc : kD;      // state rows
    constexpr int NRG = T / DV;                 // row groups
    constexpr int R = (ND + NRG - 1) / NRG;     // rows per thread (upper bound)
    constexpr int NPAIR = kDc - 1 - kFeat;      // 136 unordered pairs
    __shared__ double part[TB][T];
    __shared__ double dpart[TB][NRG];
    // the block's q and k / d'^(1/4), then 1.0 and a pad (16-byte rows): every feature is
    // x[ia] * x[ib] * sc, with no branch on the feature row
    __shared__ double xs_q[TB][kFeat + 2], xs_k[TB][kFeat + 2], vs[TB][DV];
    __shared__ double phk[TB][ND], phq[TB][ND];  // phi of the block's keys (times multiplicity), queries
    __shared__ unsigned char pa[COMPACT ? NPAIR : 1], pb[COMPACT ? NPAIR : 1];

    const int tid = threadIdx.x, c = tid % DV, rg = tid / DV;
    const long head = blockIdx.x;
    const int dv = DV;
    const double r2 = 0.70710678118654752440;  // 1/sqrt(2)

    if (COMPACT && tid < NPAIR) {  // pair row -> (a, b), row-major upper triangle
        int ia = 0;
        while (ia + 1 < kFeat && compact_pair(ia + 1, ia + 1) <= tid) ++ia;
        pa[tid] = (unsigned char)ia;
        pb[tid] = (unsigned char)(ia + tid - compact_pair(ia, ia));
    }
    double S[R], z[R];
#pragma unroll
    for (int p = 0; p < R; ++p) {
        const int d = rg + NRG * p;
        S[p] = 0.0;
        z[p] = 0.0;
        if (d < ND && a.S0) {
            S[p] = a.S0[(head * ND + d) * dv + c];
            z[p] = a.z0[head * ND + d];
        }
    }

    // multiplicity of row d among the full layout's rows (2 for an off-diagonal compact pair)
    auto mult = [&](int d) -> double {
        if (!COMPACT || d <= kFeat) return 1.0;
        return pa[d - 1 - kFeat] == pb[d - 1 - kFeat] ? 1.0 : 2.0;
    };

    // the constant 1.0 column of the staged q and k rows (never overwritten; the first
    // barrier of the block loop orders it before any read)
    if (tid < TB) {
        xs_k[tid][kFeat] = 1.0;
        xs_q[tid][kFeat] = 1.0;
    }
    for (int phase = 0; phase < 2; ++phase) {
        const bool causal = phase == 1;
        // rows of this phase; the JRT prefix skips its left padding (the first M - mv rows)
        const int mv = valid_prefix(a, (int)(head / a.H));
        const int len = causal ? a.N : mv;
        const long row0 = causal ? head * (long)a.N : head * (long)a.M + (a.M - mv);
        const void *kp = causal ? a.k : a.ke;
        const void *vp = causal ? a.v : a.ve;
        // a block's inputs are at most one key/query feature and one value per thread
        // (TB * kFeat and TB * DV <= T); the next block's are loaded while this one runs
        static_assert(TB * kFeat <= T && TB * DV <= T, "one staged input of each kind per thread");
        // They are held as raw bits (fp32, or bf16 zero-extended) and converted only
        // when stored, so that no wait for them comes before the block's arithmetic.
        uint32_t nk = 0, nq = 0, nv = 0;
        const int sh = in_bf16 ? 16 : 0;  // bf16 bits are the high half of the fp32 value
        auto fetch = [&](int b0) {
            const int nbb = min(TB, len - b0);
            const long src = (row0 + b0 + tid / kFeat) * kFeat + tid % kFeat;
            const long vsrc = (row0 + b0 + tid / DV) * dv + tid % DV;
            if (in_bf16) {
                if (tid < nbb * kFeat) {
                    nk = ((const uint16_t *)kp)[src];
                    if (causal) nq = ((const uint16_t *)a.q)[src];
                }
                if (tid < nbb * DV) nv = ((const uint16_t *)vp)[vsrc];
            } else {
                if (tid < nbb * kFeat) {
                    nk = ((const uint32_t *)kp)[src];
                    if (causal) nq = ((const uint32_t *)a.q)[src];
                }
                if (tid < nbb * DV) nv = ((const uint32_t *)vp)[vsrc];
            }
        };
        if (len > 0) fetch(0);
        for (int t0 = 0; t0 < len; t0 += TB) {
            const int nb = min(TB, len - t0);
            __syncthreads();
            if (tid < nb * kFeat) {
                xs_k[tid / kFeat][tid % kFeat] = 0.5 * (double)__uint_as_float(nk << sh);
                if (causal) xs_q[tid / kFeat][tid % kFeat] = 0.5 * (double)__uint_as_float(nq << sh);
            }
            if (tid < nb * DV) vs[tid / DV][tid % DV] = (double)__uint_as_float(nv << sh);
            __syncthreads();
            if (t0 + TB < len) fetch(t0 + TB);
            // every feature of the block's tokens once (the DV threads of a row share it);
            // the products by 1.0 are exact, so these are the values phi() gives
            for (int i = tid; i < nb * ND; i += T) {
                const int tt = i / ND, d = i % ND;
                int ia, ib;
                double sc;
                if (d == 0) {
                    ia = kFeat; ib = kFeat; sc = 1.0;
                } else if (d <= kFeat) {
                    ia = d - 1; ib = kFeat; sc = 1.0;
                } else {
                    const int ab = d - 1 - kFeat;
                    ia = COMPACT ? pa[ab] : ab >> 4;
                    ib = COMPACT ? pb[ab] : ab & 15;
                    sc = r2;
                }
                phk[tt][d] = mult(d) * (xs_k[tt][ia] * xs_k[tt][ib] * sc);
                if (causal) phq[tt][d] = xs_q[tt][ia] * xs_q[tt][ib] * sc;
            }
            __syncthreads();
            for (int tt = 0; tt < nb; ++tt) {
                const double vc = vs[tt][c];
                double num = 0.0, den = 0.0;
#pragma unroll
                for (int p = 0; p < R; ++p) {
                    const int d = rg + NRG * p;
                    if (d < ND) {
                        const double fk = phk[tt][d];
                        S[p] += fk * vc;
                        z[p] += fk;
                        if (causal) {
                            const double fq = phq[tt][d];
                            num += fq * S[p];
                            den += fq * z[p];
                        }
                    }
                }
                if (causal) {
                    part[tt][tid] = num;
                    if (c == 0) dpart[tt][rg] = den;
                }
            }
            if (causal) {
                __syncthreads();
                for (int o = tid; o < nb * DV; o += T) {
                    const int tt = o / DV, cc = o % DV;
                    double num = 0.0, den = 0.0;
                    for (int r = 0; r < NRG; ++r) {
                        num += part[tt][r * DV + cc];
                        den += dpart[tt][r];
                    }
                    const double yv = num / (den + (double)a.eps);
                    const long oi = (head * a.N + t0 + tt) * dv + cc;
                    if (a.y) {
                        if (a.y_bf16)
                            ((uint16_t *)a.y)[oi] = f32_to_bf16_rne((float)yv);
                        else
                            ((float *)a.y)[oi] = (float)yv;
                    }
                }
            }
        }
    }

#pragma unroll
    for (int p = 0; p < R; ++p) {
        const int d = rg + NRG * p;
        if (d < ND) {
            if (a.S_out) a.S_out[(head * ND + d) * dv + c] = (float)S[p];
            if (a.z_out && c == 0) a.z_out[head * ND + d] = (float)z[p];
        }
    }
}


// ---------------------------------------------------------------------------
// Short sequences without a JRT prefix: the attention form of the same
// recurrence ("Simple linear attention language models..." notes, §2.2: y_i is
// sum_{j<=i} K(q_i,k_j) v_j / sum_{j<=i} K(q_i,k_j) with K = phi(q).phi(k) =
// 1 + t + t^2/2, t = q.k/4, §2.3), plus the read-out of the initial state
// phi(q_i)^T S0 / phi(q_i)^T z0 (length-generalization notes §2.5, Eq. (4)), in
// fp64 and spread over one workgroup per kQuadQ queries of a head instead of one
// token-sequential workgroup per head.  Workgroup g of a head also writes the
// final-state rows [g * rpb, (g + 1) * rpb): S0 plus mult(d) phi_d(k_j) v_j summed
// in token order, the same expressions in the same order as the kernel above.
constexpr int kQuadMaxN = 256;  // longest sequence handled this way
constexpr int kQuadQ = 16;      // queries per workgroup
constexpr int kQuadT = 1024;    // threads per workgroup

template <int DV, bool COMPACT>
__global__ __launch_bounds__(kQuadT) void prefill_quad_kernel(PrefillArgs a, int in_bf16, int nblk)
{
    constexpr int ND = COMPACT ? kDc : kD;
    constexpr int NPAIR = kDc - 1 - kFeat;
    // k / d'^(1/4) of every token of the head, then 1.0 (and a pad to 16-byte rows): every
    // feature is then x[ia] * x[ib] * sc with (ia, ib, sc) fixed per feature row
    __shared__ double xk[kQuadMaxN][kFeat + 2];
    // v, as doubles where they fit the LDS (d_v <= 32: no conversion in the token loops);
    // fp32 and bf16 values are exact in either type
    typedef typename std::conditional<(DV <= 32), double, float>::type VT;
    __shared__ __attribute__((aligned(32))) VT vs[kQuadMaxN][DV];
    __shared__ double xq[kQuadQ][kFeat];      // q / d'^(1/4) of this workgroup's queries
    __shared__ double Kq[kQuadQ][kQuadMaxN];  // K(q_i, k_j) for j <= i, zero after
    __shared__ unsigned char pa[COMPACT ? NPAIR : 1], pb[COMPACT ? NPAIR : 1];

    const int tid = threadIdx.x;
    const long head = blockIdx.x / nblk;
    const int g = blockIdx.x % nblk;
    const int N = a.N, dv = DV, q0 = g * kQuadQ;
    const double r2 = 0.70710678118654752440;  // 1/sqrt(2)

    if (COMPACT && tid < NPAIR) {  // pair row -> (a, b), row-major upper triangle
        int ia = 0;
        while (ia + 1 < kFeat && compact_pair(ia + 1, ia + 1) <= tid) ++ia;
        pa[tid] = (unsigned char)ia;
        pb[tid] = (unsigned char)(ia + tid - compact_pair(ia, ia));
    }
    auto phi = [&](int d, const double *x) -> double {
        if (d == 0) return 1.0;
        if (d <= kFeat) return x[d - 1];
        const int ab = d - 1 - kFeat;
        if (COMPACT) return x[pa[ab]] * x[pb[ab]] * r2;
        return x[ab >> 4] * x[ab & 15] * r2;
    };
    auto mult = [&](int d) -> double {
        if (!COMPACT || d <= kFeat) return 1.0;
        return pa[d - 1 - kFeat] == pb[d - 1 - kFeat] ? 1.0 : 2.0;
    };

    {   // every load of the head's keys, values and queries is issued before the first
        // conversion or LDS store, as raw bits (fp32, or bf16 zero-extended), with one
        // branch on the input type around all of them
        constexpr int KPT = kQuadMaxN * kFeat / kQuadT, VPT = kQuadMaxN * DV / kQuadT;
        static_assert(kQuadQ * kFeat <= kQuadT, "one query feature per thread");
        uint32_t kb[KPT], vb[VPT], qb = 0;
        const int qi = tid / kFeat, f = tid % kFeat;
        const bool qok = tid < kQuadQ * kFeat && q0 + qi < N;
        const long kbase = head * N * kFeat, vbase = head * N * DV, qidx = (head * N + q0 + qi) * kFeat + f;
        if (in_bf16) {
            const uint16_t *k16 = (const uint16_t *)a.k, *v16 = (const uint16_t *)a.v, *q16 = (const uint16_t *)a.q;
#pragma unroll
            for (int r = 0; r < KPT; ++r) {
                const int i = tid + r * kQuadT;
                kb[r] = i < N * kFeat ? (uint32_t)k16[kbase + i] : 0u;
            }
#pragma unroll
            for (int r = 0; r < VPT; ++r) {
                const int i = tid + r * kQuadT;
                vb[r] = i < N * DV ? (uint32_t)v16[vbase + i] : 0u;
            }
            if (qok) qb = (uint32_t)q16[qidx];
        } else {
            const uint32_t *k32 = (const uint32_t *)a.k, *v32 = (const uint32_t *)a.v, *q32 = (const uint32_t *)a.q;
#pragma unroll
            for (int r = 0; r < KPT; ++r) {
                const int i = tid + r * kQuadT;
                kb[r] = i < N * kFeat ? k32[kbase + i] : 0u;
            }
#pragma unroll
            for (int r = 0; r < VPT; ++r) {
                const int i = tid + r * kQuadT;
                vb[r] = i < N * DV ? v32[vbase + i] : 0u;
            }
            if (qok) qb = q32[qidx];
        }
        const int sh = in_bf16 ? 16 : 0;  // bf16 bits are the high half of the fp32 value
#pragma unroll
        for (int r = 0; r < KPT; ++r) {
            const int i = tid + r * kQuadT;
            if (i < N * kFeat) xk[i / kFeat][i % kFeat] = 0.5 * (double)__uint_as_float(kb[r] << sh);
        }
#pragma unroll
        for (int r = 0; r < VPT; ++r) {
            const int i = tid + r * kQuadT;
            if (i < N * DV) vs[i / DV][i % DV] = (VT)__uint_as_float(vb[r] << sh);
        }
        if (tid < kQuadQ * kFeat) xq[qi][f] = qok ? 0.5 * (double)__uint_as_float(qb << sh) : 0.0;
        for (int j = tid; j < N; j += kQuadT) xk[j][kFeat] = 1.0;
    }
    __syncthreads();
    {   // K(q_i, k_j): thread t takes key j = t mod kQuadMaxN, read once into registers,
        // and the queries qi = t / kQuadMaxN + QG r of the workgroup
        constexpr int QG = kQuadT / kQuadMaxN;
        static_assert(kQuadT % kQuadMaxN == 0 && kQuadQ % QG == 0, "whole query groups");
        const int j = tid % kQuadMaxN, qg = tid / kQuadMaxN;
        if (j < N) {
            double xr[kFeat];
#pragma unroll
            for (int f = 0; f < kFeat; ++f) xr[f] = xk[j][f];
#pragma unroll
            for (int r = 0; r < kQuadQ / QG; ++r) {
                const int qi = qg + QG * r, i = q0 + qi;
                double kv = 0.0;
                if (j <= i && i < N) {
                    double t = 0.0;
#pragma unroll
                    for (int f = 0; f < kFeat; ++f) t += xq[qi][f] * xr[f];
                    kv = 1.0 + t + 0.5 * t * t;
                }
                Kq[qi][j] = kv;
            }
        }
    }
    __syncthreads();

    // y: kQuadQ * DV outputs.  Where they would fill at most a quarter of the
    // workgroup (d_v = 16), each output's sums are split over YS = 2 adjacent
    // threads (alternate initial-state rows and tokens), added in a fixed order.
    // The final-state rows below start on the threads after the YT that compute
    // y, so that the two run at once.
    constexpr int NY = kQuadQ * DV;
    constexpr int YS = NY * 4 <= kQuadT ? 2 : 1;
    constexpr int YT = NY * YS;
    if (a.y) {
        for (int o2 = tid; o2 < YT; o2 += kQuadT) {
            const int o = o2 / YS, part = o2 % YS;
            const int qi = o / DV, c = o % DV, i = q0 + qi;
            double num = 0.0, den = 0.0;
            if (i < N) {
                if (a.S0) {
                    for (int d = part; d < ND; d += YS) {
                        const double f = phi(d, xq[qi]);
                        num += f * a.S0[(head * ND + d) * dv + c];
                        den += f * a.z0[head * ND + d];
                    }
                }
                for (int j = part; j <= i; j += YS) {
                    const double kv = Kq[qi][j];
                    num += kv * vs[j][c];
                    den += kv;
                }
            }
            if constexpr (YS == 2) {  // every lane of the pair takes part; the even part adds first
                const double num1 = __shfl_xor(num, 1), den1 = __shfl_xor(den, 1);
                num += num1;
                den += den1;
            }
            if (part != 0 || i >= N) continue;
            const double yv = num / (den + (double)a.eps);
            const long oi = (head * N + i) * dv + c;
            if (a.y_bf16)
                ((uint16_t *)a.y)[oi] = f32_to_bf16_rne((float)yv);
            else
                ((float *)a.y)[oi] = (float)yv;
        }
    }
    if (a.S_out || a.z_out) {
        // Each lane sums CPL adjacent columns of one row (two at d_v = 16, so that the
        // rows spread over three wavefronts; four otherwise): the feature value
        // phi_d(k_j) is formed once per token for them, and every entry keeps its
        // value and token order.
        constexpr int CPL = DV == 16 ? 2 : 4, NCG = DV / CPL;
        typedef VT vcpl __attribute__((ext_vector_type(CPL)));
        const int rpb = (ND + nblk - 1) / nblk, d0 = g * rpb, d1 = min(ND, d0 + rpb);
        for (int o = (tid + kQuadT - YT % kQuadT) % kQuadT; o < (d1 - d0) * NCG; o += kQuadT) {
            const int d = d0 + o / NCG, c0 = (o % NCG) * CPL;
            double sv[CPL];
#pragma unroll
            for (int e = 0; e < CPL; ++e) sv[e] = a.S0 ? a.S0[(head * ND + d) * dv + c0 + e] : 0.0;
            double zv = a.S0 ? a.z0[head * ND + d] : 0.0;
            // phi_d(x) = x[ia] * x[ib] * sc without a branch in the token loop (its lanes
            // hold different rows d); the products by 1.0 are exact, so fk is the value
            // phi() gives.  The multiplicity m (1 or 2) is folded into the scale:
            // (x[ia] x[ib]) (m sc) equals m ((x[ia] x[ib]) sc) exactly, m being a power of 2
            int ia, ib;
            double sc;
            if (d == 0) {
                ia = kFeat; ib = kFeat; sc = 1.0;
            } else if (d <= kFeat) {
                ia = d - 1; ib = kFeat; sc = 1.0;
            } else {
                const int ab = d - 1 - kFeat;
                ia = COMPACT ? pa[ab] : ab >> 4;
                ib = COMPACT ? pb[ab] : ab & 15;
                sc = r2;
            }
            const double msc = mult(d) * sc;
            for (int j = 0; j < N; ++j) {
                const double fk = xk[j][ia] * xk[j][ib] * msc;
                const vcpl vv = *(const vcpl *)&vs[j][c0];
#pragma unroll
                for (int e = 0; e < CPL; ++e) sv[e] += fk * (double)vv[e];
                zv += fk;
            }
#pragma unroll
            for (int e = 0; e < CPL; ++e)
                if (a.S_out) a.S_out[(head * ND + d) * dv + c0 + e] = (float)sv[e];
            if (a.z_out && c0 == 0) a.z_out[head * ND + d] = (float)zv;
        }
    }
}

template <int DV, bool COMPACT>
void launch_quad_dv(const PrefillArgs &a, int in_bf16, int nblk, hipStream_t s)
{
    hipLaunchKernelGGL((prefill_quad_kernel<DV, COMPACT>), dim3((unsigned)((long)a.B * a.H * nblk)),
                       dim3(kQuadT), 0, s, a, in_bf16, nblk);
}

// Threads per workgroup: 1024 for d_v <= 32 (each thread then keeps 5 or 9 state
// rows of one column in fp64 registers, within the 128 registers of 16 waves
// per CU); 512 for d_v = 64, whose 18 rows per thread need the larger budget.
template <int DV>
constexpr int exact_threads() { return DV <= 32 ? 1024 : 512; }

template <int DV, bool COMPACT>
void launch_exact_dv(const PrefillArgs &a, int in_bf16, hipStream_t s)
{
    constexpr int T = exact_threads<DV>();
    hipLaunchKernelGGL((prefill_exact_kernel<DV, T, COMPACT>), dim3((unsigned)(a.B * a.H)), dim3(T), 0, s, a,
                       in_bf16);
}

}  // namespace

hipError_t launch_prefill_exact(const PrefillArgs &a, int in_bf16, hipStream_t s)
{
    // short sequences without a prefix: the parallel attention-form kernel, unless the
    // state is updated in place (its workgroups read S0 while others write S_out) or
    // the grid would exceed 2^21 workgroups
    const int nblk = (a.N + kQuadQ - 1) / kQuadQ;
    const bool in_place = (a.S_out && a.S_out == a.S0) || (a.z_out && a.z_out == a.z0);
    if (a.M == 0 && a.N >= 1 && a.N <= kQuadMaxN && !in_place && (long long)a.B * a.H * nblk <= (1LL << 21)) {
        if (a.compact) {
            switch (a.dv) {
            case 16: launch_quad_dv<16, true>(a, in_bf16, nblk, s); break;
            case 32: launch_quad_dv<32, true>(a, in_bf16, nblk, s); break;
            default: launch_quad_dv<64, true>(a, in_bf16, nblk, s); break;
            }
        } else {
            switch (a.dv) {
            case 16: launch_quad_dv<16, false>(a, in_bf16, nblk, s); break;
            case 32: launch_quad_dv<32, false>(a, in_bf16, nblk, s); break;
            default: launch_quad_dv<64, false>(a, in_bf16, nblk, s); break;
            }
        }
        return hipGetLastError();
    }
    if (a.compact) {
        switch (a.dv) {
        case 16: launch_exact_dv<16, true>(a, in_bf16, s); break;
        case 32: launch_exact_dv<32, true>(a, in_bf16, s); break;
        default: launch_exact_dv<64, true>(a, in_bf16, s); break;
        }
    } else {
        switch (a.dv) {
        case 16: launch_exact_dv<16, false>(a, in_bf16, s); break;
        case 32: launch_exact_dv<32, false>(a, in_bf16, s); break;
        default: launch_exact_dv<64, false>(a, in_bf16, s); break;
        }
    }
    return hipGetLastError();
}

}  // namespace bla
