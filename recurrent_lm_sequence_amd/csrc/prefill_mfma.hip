// Chunked causal Taylor linear-attention prefill on gfx950 matrix cores.
//
// Method: "Simple linear attention language models balance the recall-throughput
// tradeoff" notes, §2.5 (chunked form): for chunk b of 64 tokens
//   U_b = (M_b o Phi_Qb Phi_Kb^T) V_b + Phi_Qb S_<b,   S_<b = sum_{a<b} Phi_Ka^T V_a,
// with the same split for the denominator, and the Taylor-order split of the
// state: order 0 is a running sum of v, order 1 a 16-wide product, order 2 the
// 256-row block.  §2.3 gives phi and K; §2.2 the recurrence this equals.
// "Just read twice" notes §2.6/§2.8: the JRT prefix state (non-causal sum over
// the M prefix tokens) is accumulated first and seeds the causal scan.
// Length-generalization notes §2.5 Eq. (4): an initial state is added to S, z.
//
// gfx950 design (not the H100 kernel's):
//  * one workgroup = one (batch, head) x a block of CW = 16*NW value columns;
//    wave w owns state columns [16w, 16w+16) of that block: its 256x16 order-2
//    slice (16 accumulator tiles), the 16x16 order-1 slice and the order-0 row
//    stay in MFMA accumulator registers across all chunks -- the state never
//    leaves the register file between chunks;
//  * the inter-chunk product Phi_Q S feeds those accumulators, converted to
//    fp16, straight back in as the B operand of v_mfma_f32_16x16x32_f16 (the
//    accumulator layout of two stacked 16x16 tiles is the B-operand layout of
//    one 32-deep slab, as long as the A operand lists its 32 features in the
//    same order);
//  * phi(q), phi(k) are never materialised in memory: the order-2 operands are
//    built in registers with packed fp16 multiplies from the 16-wide q, k rows;
//  * the intra-chunk score tile T^T = K Q^T is produced in the accumulator
//    layout that is exactly the A-operand layout of the following (A o mask) V
//    product; the V operand is stored in LDS in the matching token order;
//  * the denominator keeps z in fp32: order 0 is a count, order 1 and 2 are a
//    16-vector and a symmetric 16x16 matrix, so phi(q).z = z0 + q.z1 + q^T Z q;
//  * inputs are prefetched one chunk ahead into registers and staged through a
//    triple-buffered LDS ring; one workgroup barrier per chunk.
//
// Operand scales (powers of two, exact): the LDS copy of q holds q/8, the
// order-2 key operand holds k/16 per factor, the numerator accumulator runs at
// 2^-9 of the true value, and the state accumulators hold
//   acc2 = sum k_a k_b v / 2^8, acc1 = sum k_a v / 2^4, acc0 = sum v,
//   Z2 = sum k_a k_b / 2^8, z1 = sum k_a / 2^4, z0 = count.
// These keep every fp16 operand inside its normal range for realistic inputs.
#include "common.h"

namespace bla {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int CH = 64;  // tokens per chunk
constexpr int TS = 72;  // halves per LDS row of the token-slot arrays (64 slots + 8 pad)

// abi state <-> accumulator scales (see the header comment)
constexpr float kS2ToAcc = 0.022097086912079608f;  // 1 / (32 sqrt 2)
constexpr float kAccToS2 = 45.254833995939045f;    // 32 sqrt 2
constexpr float kS1ToAcc = 0.125f;
constexpr float kAccToS1 = 8.0f;

// Token order inside a 64-token chunk as seen by the 16x16x32 MFMA operands:
// the score accumulator tile rows are 4g+r (g = lane/16); two 16-row tiles form
// one 32-deep slab in which lane group g holds rows {4g..4g+3, 16+4g..16+4g+3}.
// Storing V and k in this "slot" order makes every operand a 16-byte LDS read.
__device__ __forceinline__ int slot_of(int j) {
    return (j & 32) + ((j >> 2) & 3) * 8 + ((j >> 4) & 1) * 4 + (j & 3);
}

__device__ __forceinline__ f4 mfma32(h8 a, h8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mfma16(h4 a, h4 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    h2 h = __builtin_convertvector((f2){a, b}, h2);
    return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ h4 to_h4(f4 x) { return __builtin_convertvector(x, h4); }

template <int NW>
struct Layout {
    static constexpr int CW = 16 * NW;                 // value columns per workgroup
    static constexpr int T = 64 * NW;                  // threads
    static constexpr int QS = 0;                       // [64][16] q/8
    static constexpr int KS = 2048;                    // [64][16] k
    static constexpr int KT = 4096;                    // [16][TS] k/16, slot order
    static constexpr int VT = KT + 16 * TS * 2;        // [CW][TS] v, slot order
    static constexpr int BUF = VT + CW * TS * 2;       // bytes per ring buffer
    static constexpr int ABUF = 3 * BUF;               // 2 x [4 it][2 slab][64 lane][8] fp16
    static constexpr int RDEN = ABUF + 2 * 8192;       // 2 x [64] fp32
    static constexpr int TOTAL = RDEN + 2 * 256;
    static constexpr int QKU = (128 + T - 1) / T;      // q/k staging units per thread
};

template <int NW>
__global__ __launch_bounds__(64 * NW, 1) void prefill_mfma_kernel(PrefillArgs a, int n_cb)
{
    using L = Layout<NW>;
    constexpr int CW = L::CW;
    __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];

    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63, g = l >> 4, lr = l & 15;
    const int heads = a.B * a.H;

    // XCD-aware block -> (head, column block): blocks dispatch round-robin over
    // the 8 XCDs, so the column blocks of one head share an XCD (and its L2).
    int head, cb;
    if (n_cb == 1) {
        head = blockIdx.x;
        cb = 0;
    } else if ((heads & 7) == 0) {
        const int xcd = blockIdx.x & 7, u = blockIdx.x >> 3;
        head = (u / n_cb) * 8 + xcd;
        cb = u % n_cb;
    } else {
        head = blockIdx.x / n_cb;
        cb = blockIdx.x % n_cb;
    }
    const int dv = a.dv;
    const int col = cb * CW + 16 * w + lr;  // this lane's state / output column
    const int P = (a.M + CH - 1) / CH;      // prefix chunks
    const int NC = (a.N + CH - 1) / CH;     // causal chunks
    const int total = P + NC;

    // ---------------- state (MFMA accumulator layout) ----------------
    f4 S2[16], S1, S0acc, dZ2, dz1, Z2i, z1i;
    float z0i = 0.f, dz0 = 0.f;
    const long sbase = (long)head * kD * dv;
    const long zbase = (long)head * kD;
    if (a.S0) {
#pragma unroll
        for (int m = 0; m < 16; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S2[m][r] = a.S0[sbase + (long)(17 + 16 * m + 4 * g + r) * dv + col] * kS2ToAcc;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            S1[r] = a.S0[sbase + (long)(1 + 4 * g + r) * dv + col] * kS1ToAcc;
            S0acc[r] = a.S0[sbase + col];
            const int ra = 4 * g + r;
            Z2i[r] = 0.5f * (a.z0[zbase + 17 + 16 * ra + lr] + a.z0[zbase + 17 + 16 * lr + ra]) *
                     kS2ToAcc;
            z1i[r] = a.z0[zbase + 1 + ra] * kS1ToAcc;
        }
        z0i = a.z0[zbase];
    } else {
#pragma unroll
        for (int m = 0; m < 16; ++m) S2[m] = (f4){0.f, 0.f, 0.f, 0.f};
        S1 = S0acc = Z2i = z1i = (f4){0.f, 0.f, 0.f, 0.f};
    }
    dZ2 = dz1 = (f4){0.f, 0.f, 0.f, 0.f};

    // ---------------- global -> register staging ----------------
    const uint16_t *qp = (const uint16_t *)a.q, *kp = (const uint16_t *)a.k,
                   *vp = (const uint16_t *)a.v, *kep = (const uint16_t *)a.ke,
                   *vep = (const uint16_t *)a.ve;
    const int jq = tid / (CW / 4), cq = tid % (CW / 4);  // v unit: 4 tokens x 4 columns
    u2 sv[4];
    u4 sqk[L::QKU][2];

    auto load_chunk = [&](int c) {
        const bool pre = c < P;
        const int len = pre ? a.M : a.N;
        const int tok0 = (pre ? c : c - P) * CH;
        const uint16_t *vsrc = pre ? vep : vp;
        const uint16_t *ksrc = pre ? kep : kp;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = tok0 + 4 * jq + r;
            sv[r] = (u2){0u, 0u};
            if (j < len)
                sv[r] = *(const u2 *)(vsrc + ((long)head * len + j) * dv + cb * CW + 4 * cq);
        }
#pragma unroll
        for (int i = 0; i < L::QKU; ++i) {
            const int u = tid + i * L::T;
            sqk[i][0] = sqk[i][1] = (u4){0u, 0u, 0u, 0u};
            if (u < 64) {  // q unit: token u, 16 features
                const int j = tok0 + u;
                if (!pre && j < len) {
                    const u4 *src = (const u4 *)(qp + ((long)head * len + j) * 16);
                    sqk[i][0] = src[0];
                    sqk[i][1] = src[1];
                }
            } else if (u < 128) {  // k unit: tokens 2p, 2p+1, features 8hh..8hh+7
                const int p = (u - 64) >> 1, hh = (u - 64) & 1;
                const int j = tok0 + 2 * p;
                if (j < len) sqk[i][0] = *(const u4 *)(ksrc + ((long)head * len + j) * 16 + 8 * hh);
                if (j + 1 < len)
                    sqk[i][1] = *(const u4 *)(ksrc + ((long)head * len + j + 1) * 16 + 8 * hh);
            }
        }
    };

    auto store_chunk = [&](int c) {
        unsigned char *buf = smem + (c % 3) * L::BUF;
        _Float16 *Qs = (_Float16 *)(buf + L::QS);
        _Float16 *Ks = (_Float16 *)(buf + L::KS);
        _Float16 *Kt = (_Float16 *)(buf + L::KT);
        _Float16 *Vt = (_Float16 *)(buf + L::VT);
        // v: tokens 4jq..4jq+3 (consecutive slots) x columns 4cq..4cq+3
        const int s0 = slot_of(4 * jq);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float f[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t wd = (e < 2) ? sv[r].x : sv[r].y;
                f[r] = (e & 1) ? bf16_hi(wd) : bf16_lo(wd);
            }
            *(u2 *)(Vt + (4 * cq + e) * TS + s0) = (u2){pack2(f[0], f[1]), pack2(f[2], f[3])};
        }
#pragma unroll
        for (int i = 0; i < L::QKU; ++i) {
            const int u = tid + i * L::T;
            if (u < 64) {
                u4 o[2];
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int x = 0; x < 4; ++x)
                        o[h][x] = pack2(bf16_lo(sqk[i][h][x]) * 0.125f, bf16_hi(sqk[i][h][x]) * 0.125f);
                *(u4 *)(Qs + u * 16) = o[0];
                *(u4 *)(Qs + u * 16 + 8) = o[1];
            } else if (u < 128) {
                const int p = (u - 64) >> 1, hh = (u - 64) & 1;
                const int jl = 2 * p;
                u4 o0, o1;
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    o0[x] = pack2(bf16_lo(sqk[i][0][x]), bf16_hi(sqk[i][0][x]));
                    o1[x] = pack2(bf16_lo(sqk[i][1][x]), bf16_hi(sqk[i][1][x]));
                }
                *(u4 *)(Ks + jl * 16 + 8 * hh) = o0;
                *(u4 *)(Ks + (jl + 1) * 16 + 8 * hh) = o1;
                const int sl = slot_of(jl);
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    *(uint32_t *)(Kt + (8 * hh + 2 * x) * TS + sl) =
                        pack2(bf16_lo(sqk[i][0][x]) * 0.0625f, bf16_lo(sqk[i][1][x]) * 0.0625f);
                    *(uint32_t *)(Kt + (8 * hh + 2 * x + 1) * TS + sl) =
                        pack2(bf16_hi(sqk[i][0][x]) * 0.0625f, bf16_hi(sqk[i][1][x]) * 0.0625f);
                }
            }
        }
    };

    const h8 ones = (h8){1, 1, 1, 1, 1, 1, 1, 1};
    const f4 zero4 = (f4){0.f, 0.f, 0.f, 0.f};

    // ---------------- stage 1: score tile, A operands, 1/denominator ----------------
    auto stage1 = [&](int c) {  // c: a causal chunk index (>= P)
        const unsigned char *buf = smem + (c % 3) * L::BUF;
        const _Float16 *Qs = (const _Float16 *)(buf + L::QS);
        const _Float16 *Ks = (const _Float16 *)(buf + L::KS);
        _Float16 *Ab = (_Float16 *)(smem + L::ABUF + (c & 1) * 8192);
        float *rden = (float *)(smem + L::RDEN + (c & 1) * 256);
        const h4 z2op = to_h4(Z2i + dZ2);
        const f4 z1t = z1i + dz1;
        const float z0t = z0i + dz0;
        for (int it = w; it < 4; it += NW) {
            const h4 qB = *(const h4 *)(Qs + (16 * it + lr) * 16 + 4 * g);
            float rowsum = 0.f;
            h8 aop;
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) {
                if (jt > it) break;
                const h4 kA = *(const h4 *)(Ks + (16 * jt + lr) * 16 + 4 * g);
                const f4 T = mfma16(kA, qB, zero4);  // [j = 16jt+4g+r][i = 16it+lr] = (q/8).k
                float av[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float cc = T[r];
                    // A/2^9 = (1 + t/4 + t^2/32)/2^9 with t = 8 cc
                    float x = __builtin_fmaf(cc * 0.00390625f, 1.0f + cc, 0.001953125f);
                    if (jt == it && 4 * g + r > lr) x = 0.f;  // causal mask j > i
                    rowsum += x;
                    av[r] = x;
                }
                const h4 hv = to_h4((f4){av[0], av[1], av[2], av[3]});
                if (jt & 1) {
                    aop[4] = hv[0]; aop[5] = hv[1]; aop[6] = hv[2]; aop[7] = hv[3];
                } else {
                    aop[0] = hv[0]; aop[1] = hv[1]; aop[2] = hv[2]; aop[3] = hv[3];
                    aop[4] = aop[5] = aop[6] = aop[7] = (_Float16)0.f;
                }
                if ((jt & 1) || jt == it)
                    *(h8 *)(Ab + ((it * 2 + (jt >> 1)) * 64 + l) * 8) = aop;
            }
            // phi(q).z for order 1 and 2: W = Z q, then sum_b q_b (16 W_b + z1_b), x32
            const f4 W = mfma16(z2op, qB, zero4);
            float p = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) p += (float)qB[r] * (16.f * W[r] + z1t[r]);
            float s = rowsum * 512.f + 32.f * p;
            s += __shfl_xor(s, 16);
            s += __shfl_xor(s, 32);
            const float den = s + z0t + a.eps;
            if (g == 0) rden[16 * it + lr] = 512.f / den;
        }
    };

    // ---------------- prologue ----------------
    if (total > 0) {
        load_chunk(0);
        store_chunk(0);
        if (total > 1) load_chunk(1);
    }
    __syncthreads();
    if (total > 0 && P == 0) stage1(0);

    float *yf = (float *)a.y;
    uint16_t *yh = (uint16_t *)a.y;
    const int wcol = 16 * w + lr;  // column inside this block's Vt rows

    for (int c = 0; c < total; ++c) {
        if (c + 1 < total) store_chunk(c + 1);
        if (c + 2 < total) load_chunk(c + 2);
        __syncthreads();

        const unsigned char *buf = smem + (c % 3) * L::BUF;
        const _Float16 *Kt = (const _Float16 *)(buf + L::KT);
        const _Float16 *Vt = (const _Float16 *)(buf + L::VT);
        h8 vop[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) vop[s] = *(const h8 *)(Vt + wcol * TS + 32 * s + 8 * g);

        if (c >= P) {
            // -------- stage 3: numerator = inter-chunk (state) + intra-chunk, output --------
            const _Float16 *Qs = (const _Float16 *)(buf + L::QS);
            const _Float16 *Ab = (const _Float16 *)(smem + L::ABUF + (c & 1) * 8192);
            const float *rden = (const float *)(smem + L::RDEN + (c & 1) * 256);
            h8 S2op[8];
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const h4 lo = to_h4(S2[2 * s]), hi = to_h4(S2[2 * s + 1]);
                S2op[s] = (h8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
            const h4 S1op = to_h4(S1 * 0.0625f);
            const float s0 = S0acc[0] * 0.001953125f;
            const int tok0 = (c - P) * CH;
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                f4 acc = (f4){s0, s0, s0, s0};
                const _Float16 *qrow = Qs + (16 * it + lr) * 16;
                const h8 qlo = *(const h8 *)qrow, qhi = *(const h8 *)(qrow + 8);
                const h4 qb = *(const h4 *)(qrow + 4 * g);
                acc = mfma16(qb, S1op, acc);  // order 1
                const h2 b01 = (h2){qb[0], qb[1]}, b23 = (h2){qb[2], qb[3]};
#pragma unroll
                for (int s = 0; s < 8; ++s) {  // order 2: features (2s, 4g+r), (2s+1, 4g+r)
                    const _Float16 qa0 = s < 4 ? qlo[2 * s] : qhi[2 * s - 8];
                    const _Float16 qa1 = s < 4 ? qlo[2 * s + 1] : qhi[2 * s - 7];
                    const h2 x0 = (h2){qa0, qa0} * b01, x1 = (h2){qa0, qa0} * b23;
                    const h2 x2 = (h2){qa1, qa1} * b01, x3 = (h2){qa1, qa1} * b23;
                    const h8 aop = (h8){x0[0], x0[1], x1[0], x1[1], x2[0], x2[1], x3[0], x3[1]};
                    acc = mfma32(aop, S2op[s], acc);
                }
#pragma unroll
                for (int s = 0; s < 2; ++s) {  // intra-chunk (A o mask) V
                    if (s > (it >> 1)) break;
                    const h8 aop = *(const h8 *)(Ab + ((it * 2 + s) * 64 + l) * 8);
                    acc = mfma32(aop, vop[s], acc);
                }
                const f4 rd = *(const f4 *)(rden + 16 * it + 4 * g);
                if (a.y) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = tok0 + 16 * it + 4 * g + r;
                        if (row < a.N) {
                            const long o = ((long)head * a.N + row) * dv + col;
                            const float yv = acc[r] * rd[r];
                            if (a.y_bf16)
                                yh[o] = f32_to_bf16_rne(yv);
                            else
                                yf[o] = yv;
                        }
                    }
                }
            }
        }

        // -------- stage 4: state update with this chunk --------
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const h8 kt = *(const h8 *)(Kt + lr * TS + 32 * s + 8 * g);
            S0acc = mfma32(ones, vop[s], S0acc);
            S1 = mfma32(kt, vop[s], S1);
            dZ2 = mfma32(kt, kt, dZ2);
            dz1 = mfma32(kt, ones, dz1);
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                const h8 km = *(const h8 *)(Kt + m * TS + 32 * s + 8 * g);
                S2[m] = mfma32(km * kt, vop[s], S2[m]);
            }
        }
        {
            const bool pre = c < P;
            const int len = pre ? a.M : a.N;
            const int tok0 = (pre ? c : c - P) * CH;
            dz0 += (float)min(CH, len - tok0);
        }

        if (c + 1 < total && c + 1 >= P) stage1(c + 1);
    }

    // ---------------- final state ----------------
    if (a.S_out) {
#pragma unroll
        for (int m = 0; m < 16; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                a.S_out[sbase + (long)(17 + 16 * m + 4 * g + r) * dv + col] = S2[m][r] * kAccToS2;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            a.S_out[sbase + (long)(1 + 4 * g + r) * dv + col] = S1[r] * kAccToS1;
        if (g == 0) a.S_out[sbase + col] = S0acc[0];
    }
    if (a.z_out && cb == 0 && w == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int ra = 4 * g + r;
            const long o2 = zbase + 17 + 16 * ra + lr;
            a.z_out[o2] = (a.z0 ? a.z0[o2] : 0.f) + dZ2[r] * kAccToS2;
            if (lr == 0) {
                const long o1 = zbase + 1 + ra;
                a.z_out[o1] = (a.z0 ? a.z0[o1] : 0.f) + dz1[r] * kAccToS1;
            }
        }
        if (l == 0) a.z_out[zbase] = (a.z0 ? a.z0[zbase] : 0.f) + dz0;
    }
}

}  // namespace

hipError_t launch_prefill_mfma(const PrefillArgs &a, int col_split_allowed, hipStream_t s)
{
    const int heads = a.B * a.H;
    // columns per workgroup: fill the 256 CUs with at least ~256 workgroups
    int cw = a.dv;
    if (col_split_allowed) {
        while (cw > 16 && (long)heads * (a.dv / cw) < 256) cw >>= 1;
    }
    const int n_cb = a.dv / cw;
    const dim3 grid((unsigned)(heads * n_cb));
    switch (cw) {
    case 64:
        hipLaunchKernelGGL(prefill_mfma_kernel<4>, grid, dim3(256), 0, s, a, n_cb);
        break;
    case 32:
        hipLaunchKernelGGL(prefill_mfma_kernel<2>, grid, dim3(128), 0, s, a, n_cb);
        break;
    default:
        hipLaunchKernelGGL(prefill_mfma_kernel<1>, grid, dim3(64), 0, s, a, n_cb);
        break;
    }
    return hipGetLastError();
}

}  // namespace bla
