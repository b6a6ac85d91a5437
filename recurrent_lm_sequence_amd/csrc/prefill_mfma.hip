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
// gfx950 design (not the H100 kernel's).  One workgroup of 4 wavefronts owns one
// (batch, head) and a block of CW = 16*NCT value columns; it walks the sequence
// in 64-token chunks.  The 4 waves form an MS x NS grid (MS*NS = 4): wave
// (m, n) owns feature rows ab with a in [16m/MS, 16(m+1)/MS) of the 256-row
// order-2 state, for the n-th group of NCW = NCT/NS 16-column tiles.
//  * Its slice of S stays in MFMA accumulator registers across all chunks.  The
//    state update S += phi2(K)^T V and the inter-chunk product phi2(Q) S run only
//    over the wave's own rows, and the accumulators feed the inter-chunk product
//    directly as B operands (two stacked 16x16 accumulator tiles are one 32-deep
//    B slab of v_mfma_f32_16x16x32_f16 when the A operand lists its features in
//    that order).  phi is never materialised in memory: the order-2 operands are
//    built in registers with packed fp16 multiplies from the 16-wide q, k rows.
//  * The MS waves of a column group split the chunk's four 16-token tiles for
//    everything per output row (causal score tile, intra-chunk product,
//    denominator, output); their partial inter-chunk sums meet once per chunk in
//    LDS.  MS = 2 halves both that exchange and the duplicated phi2 work of a
//    column-only split.
// The order-0/1 state (17 rows) of a column tile is owned by one wave of its
// group; the denominator state (a count, a 16-vector and a symmetric 16x16
// matrix, so phi(q).z = z0 + q.z1 + q^T Z q) is kept by every wave in fp32.
// Inputs are prefetched a chunk ahead into registers and staged through a
// triple-buffered LDS ring; two workgroup barriers per chunk.
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
#ifndef PREFILL_MS64
#define PREFILL_MS64 4     // wave grid for 64-column blocks: MS row blocks x 4/MS column groups
#endif
#ifndef PREFILL_MS32
#define PREFILL_MS32 4
#endif
#ifndef PREFILL_MIN_WG
#define PREFILL_MIN_WG 512  // minimum workgroups before the value columns are split
#endif
constexpr int QST = 20;  // halves per LDS row of q / k (16 + 4 pad: conflict-free 8-byte reads)
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit dwords (gfx9 family)

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
// Rows of the token-slot arrays are 64 halves (128 B = 8 blocks of 16 B); the
// block index is XOR-swizzled with the row so that both the 16-byte operand
// reads (8 consecutive rows, same block) and the staging writes (rows 4 apart)
// hit distinct banks.
__device__ __forceinline__ int tsw(int row) { return (row ^ (row >> 2)) & 7; }
__device__ __forceinline__ int ts_idx(int row, int x) {  // half index of (row, slot x)
    return row * 64 + (((x >> 3) ^ tsw(row)) << 3) + (x & 7);
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
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, bytes, kRsrcWord3);
}
__device__ __forceinline__ h4 to_h4(f4 x) { return __builtin_convertvector(x, h4); }
__device__ __forceinline__ h8 cat8(h4 lo, h4 hi) {
    return (h8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

template <typename OutT> __device__ __forceinline__ OutT to_out(float x);
template <> __device__ __forceinline__ float to_out<float>(float x) { return x; }
template <> __device__ __forceinline__ uint16_t to_out<uint16_t>(float x) { return f32_to_bf16_rne(x); }

extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

template <int NCT, int MS = 4>
struct Layout {
    static constexpr int NS = 4 / MS;                  // column groups
    static constexpr int NCW = NCT / NS;               // 16-column tiles per wave
    static constexpr int NT = 4 / MS;                  // token tiles finished per wave
    static constexpr int CW = 16 * NCT;                // value columns per workgroup
    static constexpr int QS = 0;                       // [64][QST] q/8
    static constexpr int KS = QS + 64 * QST * 2;       // [64][QST] k
    static constexpr int KT = KS + 64 * QST * 2;       // [16][64] k/16, slot order, swizzled
    static constexpr int VT = KT + 16 * 64 * 2;        // [CW][64] v, slot order, swizzled
    static constexpr int BUF = VT + CW * 64 * 2;       // bytes per ring buffer
    // partial numerators: [4 token tiles][NS groups][MS feature-row blocks][NCW][64 lanes] f4
    static constexpr int PBUF = 3 * BUF;
    // finished output tiles of each wave, held until the next chunk stores them
    static constexpr int YST = 16 * NCW + 4;           // floats per row (16-byte aligned pad)
    static constexpr int YBUF = PBUF + 4 * NS * MS * NCW * 1024;  // [4 wave][NT][16 rows][YST]
    static constexpr int TOTAL = YBUF + 4 * NT * 16 * YST * 4;
};

template <int NCT, int MS>
constexpr int lds_bytes() { return Layout<NCT, MS>::TOTAL; }

// Uniform (per-workgroup) description of where chunk c's tokens come from.
// All helpers take it and every other input by value: the kernel keeps no
// addressable locals, so nothing is placed in scratch memory.
struct Src {
    int N, M, P, dv, colb, w;
    const char *qb, *kb, *vb, *keb, *veb;  // this head's rows of q, k, v, k_e, v_e
};

struct Staged {  // one chunk's raw bf16 inputs held by one lane
    u2 v[4];
    u4 qk[2];
};

// Raw buffer accesses, one resource per tensor and head: loads past the end of a
// head's tokens return 0 and stores past it are dropped by the range check, so
// the chunk loop has no bounds branches.  Every wave issues the same six loads
// per chunk (a wave without a role, and q during the prefix, reads a zero-size
// resource), so the number of memory operations in flight never depends on
// the path taken.
template <int NCT>
__device__ __forceinline__ Staged load_chunk(const Src s, int c, int l, int jq, int cq)
{
    Staged o;
    const bool pre = c < s.P;
    const int tok0 = (pre ? c : c - s.P) * CH;
    const int len = pre ? s.M : s.N;
    const char *vb = pre ? s.veb : s.vb;
    const __amdgpu_buffer_rsrc_t vr = rsrc(vb, s.w < NCT ? len * s.dv * 2 : 0);
#pragma unroll
    for (int r = 0; r < 4; ++r)
        o.v[r] = __builtin_amdgcn_raw_buffer_load_b64(
            vr, ((tok0 + 4 * jq + r) * s.dv + s.colb + 4 * cq) * 2, 0, 0);
    // wave 0: q of token tok0 + l; wave 1: k of tokens 2p, 2p+1, features 8hh..8hh+7
    const int p = l >> 1, hh = l & 1;
    const char *qkb = s.w == 0 ? s.qb : (pre ? s.keb : s.kb);
    const int qkbytes = s.w == 0 ? (pre ? 0 : s.N * 32) : (s.w == 1 ? len * 32 : 0);
    const __amdgpu_buffer_rsrc_t qkr = rsrc(qkb, qkbytes);
    const int o0 = s.w == 0 ? (tok0 + l) * 32 : (tok0 + 2 * p) * 32 + 16 * hh;
    const int o1 = s.w == 0 ? (tok0 + l) * 32 + 16 : (tok0 + 2 * p + 1) * 32 + 16 * hh;
    o.qk[0] = __builtin_amdgcn_raw_buffer_load_b128(qkr, o0, 0, 0);
    o.qk[1] = __builtin_amdgcn_raw_buffer_load_b128(qkr, o1, 0, 0);
    return o;
}

// Converts one lane's staged chunk to fp16 and writes it into ring buffer `buf`:
// q/8 rows, k rows, (k/16)^T and V^T in token-slot order.
template <int NCT>
__device__ __forceinline__ void store_chunk(unsigned char *buf, const Staged in, int w, int l,
                                            int jq, int cq)
{
    using L = Layout<NCT>;
    _Float16 *Qs = (_Float16 *)(buf + L::QS);
    _Float16 *Ks = (_Float16 *)(buf + L::KS);
    _Float16 *Kt = (_Float16 *)(buf + L::KT);
    _Float16 *Vt = (_Float16 *)(buf + L::VT);
    if (w < NCT) {  // v: tokens 4jq..4jq+3 (consecutive slots) x columns 4cq..4cq+3
        const int s0 = slot_of(4 * jq);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float f[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t wd = (e < 2) ? in.v[r].x : in.v[r].y;
                f[r] = (e & 1) ? bf16_hi(wd) : bf16_lo(wd);
            }
            *(u2 *)(Vt + ts_idx(4 * cq + e, s0)) = (u2){pack2(f[0], f[1]), pack2(f[2], f[3])};
        }
    }
    if (w == 0) {  // q row l, scaled by 1/8
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 2; ++i)
                *(u2 *)(Qs + l * QST + 8 * h + 4 * i) =
                    (u2){pack2(bf16_lo(in.qk[h][2 * i]) * 0.125f, bf16_hi(in.qk[h][2 * i]) * 0.125f),
                         pack2(bf16_lo(in.qk[h][2 * i + 1]) * 0.125f,
                               bf16_hi(in.qk[h][2 * i + 1]) * 0.125f)};
    } else if (w == 1) {  // k rows 2p, 2p+1 (features 8hh..), and their k/16 columns
        const int p = l >> 1, hh = l & 1;
        const int jl = 2 * p;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 2; ++i)
                *(u2 *)(Ks + (jl + t) * QST + 8 * hh + 4 * i) =
                    (u2){pack2(bf16_lo(in.qk[t][2 * i]), bf16_hi(in.qk[t][2 * i])),
                         pack2(bf16_lo(in.qk[t][2 * i + 1]), bf16_hi(in.qk[t][2 * i + 1]))};
        const int sl = slot_of(jl);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            *(uint32_t *)(Kt + ts_idx(8 * hh + 2 * x, sl)) =
                pack2(bf16_lo(in.qk[0][x]) * 0.0625f, bf16_lo(in.qk[1][x]) * 0.0625f);
            *(uint32_t *)(Kt + ts_idx(8 * hh + 2 * x + 1, sl)) =
                pack2(bf16_hi(in.qk[0][x]) * 0.0625f, bf16_hi(in.qk[1][x]) * 0.0625f);
        }
    }
}

struct Stage1Out {
    h8 aop0, aop1;  // intra-chunk A operands of one token tile (slabs 0, 1)
    float rden;     // 2^9 / denominator of token 16t + lr
};

// Token tile t of the chunk in `buf`: causal score tile -> A operands of the
// intra-chunk product, and the reciprocal denominator from the score row sums
// and the denominator state (Z2, z1, z0 before this chunk).
template <int NCT>
__device__ __forceinline__ Stage1Out stage1(const unsigned char *buf, int t, int g, int lr, f4 Z2,
                                            f4 z1, float z0, float eps)
{
    using L = Layout<NCT>;
    const _Float16 *Qs = (const _Float16 *)(buf + L::QS);
    const _Float16 *Ks = (const _Float16 *)(buf + L::KS);
    const f4 zero4 = (f4){0.f, 0.f, 0.f, 0.f};
    const h4 qB = *(const h4 *)(Qs + (16 * t + lr) * QST + 4 * g);
    float rowsum = 0.f;
    h4 part[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
        part[jt] = (h4){0, 0, 0, 0};
        if (jt > t) continue;
        const h4 kA = *(const h4 *)(Ks + (16 * jt + lr) * QST + 4 * g);
        const f4 T = mfma16(kA, qB, zero4);  // [j = 16jt+4g+r][i = 16t+lr] = (q/8).k
        float av[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float cc = T[r];
            // A/2^9 = (1 + t/4 + t^2/32)/2^9 with t = 8 cc
            float x = __builtin_fmaf(cc * 0.00390625f, 1.0f + cc, 0.001953125f);
            if (jt == t && 4 * g + r > lr) x = 0.f;  // causal mask j > i
            rowsum += x;
            av[r] = x;
        }
        part[jt] = to_h4((f4){av[0], av[1], av[2], av[3]});
    }
    // phi(q).z for order 1 and 2: W = Z q, then sum_b q_b (16 W_b + z1_b), x32
    const f4 W = mfma16(to_h4(Z2), qB, zero4);
    float p = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) p += (float)qB[r] * (16.f * W[r] + z1[r]);
    float s = rowsum * 512.f + 32.f * p;
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    Stage1Out o;
    o.aop0 = cat8(part[0], part[1]);
    o.aop1 = cat8(part[2], part[3]);
    o.rden = 512.f / (s + z0 + eps);
    return o;
}

// Stores one finished 16-row output tile held in LDS (rows row0..row0+15 of
// this wave's NCW*16 columns): whole row segments, 16 bytes per lane.
template <int NCW, typename OutT>
__device__ __forceinline__ void flush_y(const float *ytile, const char *ybase, int ybytes, int row0,
                                       int dv, int col0, int l)
{
    constexpr int W4 = 4 * NCW;  // float4 per row
    constexpr int YST = 16 * NCW + 4;
    const __amdgpu_buffer_rsrc_t ry = rsrc(ybase, ybytes);
#pragma unroll
    for (int i = 0; i < NCW; ++i) {
        const int idx = i * 64 + l, row = idx / W4, c4 = idx % W4;
        const f4 v = *(const f4 *)(ytile + row * YST + 4 * c4);
        const int off = ((row0 + row) * dv + col0 + 4 * c4) * (int)sizeof(OutT);
        if constexpr (sizeof(OutT) == 4) {
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), ry, off, 0, 0);
        } else {
            const u2 h = (u2){(uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16),
                              (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16)};
            __builtin_amdgcn_raw_buffer_store_b64(h, ry, off, 0, 0);
        }
    }
}

template <int NCT, int MS>
struct State {
    static constexpr int MT = 16 / MS, NCW = Layout<NCT, MS>::NCW;
    f4 S2[MT][NCW];  // rows ab = 16(a0+mt) + 4g + r, column col0 + 16j + lr
    f4 S1, S0acc;    // order 1 / order 0 of the wave's owned column tile
    f4 Z2, z1;       // denominator state (initial + tokens so far)
    float z0;
};

// State update with the chunk in `buf` (the wave's feature rows; order 0/1 of
// its owned column tile; denominator state).
template <int NCT, int MS>
__device__ __forceinline__ void update(State<NCT, MS> &st, const unsigned char *buf, int a0,
                                       int ct0, int own_ct, bool owner, int g, int lr, float valid)
{
    using L = Layout<NCT, MS>;
    constexpr int MT = 16 / MS, NCW = L::NCW;
    const _Float16 *Kt = (const _Float16 *)(buf + L::KT);
    const _Float16 *Vt = (const _Float16 *)(buf + L::VT);
    const h8 ones = (h8){1, 1, 1, 1, 1, 1, 1, 1};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const h8 kt = *(const h8 *)(Kt + ts_idx(lr, 32 * s + 8 * g));
        h8 vs[NCW];
#pragma unroll
        for (int j = 0; j < NCW; ++j)
            vs[j] = *(const h8 *)(Vt + ts_idx(16 * (ct0 + j) + lr, 32 * s + 8 * g));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const h8 km = *(const h8 *)(Kt + ts_idx(a0 + mt, 32 * s + 8 * g));
            const h8 phk = km * kt;  // k_a k_b / 2^8, a = a0+mt, b = lr
#pragma unroll
            for (int j = 0; j < NCW; ++j) st.S2[mt][j] = mfma32(phk, vs[j], st.S2[mt][j]);
        }
        if (owner) {
            const h8 vw = *(const h8 *)(Vt + ts_idx(16 * own_ct + lr, 32 * s + 8 * g));
            st.S1 = mfma32(kt, vw, st.S1);
            st.S0acc = mfma32(ones, vw, st.S0acc);
        }
        st.Z2 = mfma32(kt, kt, st.Z2);
        st.z1 = mfma32(kt, ones, st.z1);
    }
    st.z0 += valid;
}

template <int NCT, int MS, typename OutT>
__global__ __launch_bounds__(256, 1) void prefill_mfma_kernel(PrefillArgs args, int n_cb)
{
    using L = Layout<NCT, MS>;
    constexpr int CW = L::CW, NS = L::NS, NCW = L::NCW, NT = L::NT, MT = 16 / MS;
    static_assert(NCW >= 1 && MS * NS == 4, "bad wave grid");

    const int aN = args.N, aM = args.M, dv = args.dv;
    const int tid = threadIdx.x;
    // the wave index is uniform: keep it in a scalar register so every branch on
    // it is a scalar branch
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, g = l >> 4, lr = l & 15;
    const int m = w / NS, n = w % NS;   // feature-row block, column group
    const int a0 = m * MT;              // first order-2 feature a of this wave
    const int ct0 = n * NCW;            // first 16-column tile of this wave (in the block)
    const bool owner = m < NCW;         // owns order 0/1 of column tile ct0 + m
    const int own_ct = ct0 + (owner ? m : 0);
    // token tiles finished by this wave: m, and 3 - m when two waves share a group
    const int t0 = m, t1 = MS == 2 ? 3 - m : m;
    const int heads = args.B * args.H;

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
    const int colb = cb * CW;            // first column of this block
    const int P = (aM + CH - 1) / CH;    // prefix chunks
    const int NC = (aN + CH - 1) / CH;   // causal chunks
    const int total = P + NC;

    // ---------------- state ----------------
    const long sbase = (long)head * kD * dv;
    const long zbase = (long)head * kD;
    const f4 zero4 = (f4){0.f, 0.f, 0.f, 0.f};
    State<NCT, MS> st;
    st.S1 = st.S0acc = st.Z2 = st.z1 = zero4;
    st.z0 = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < NCW; ++j) st.S2[mt][j] = zero4;
    if (args.S0) {
        const float *S0 = args.S0, *z0 = args.z0;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int j = 0; j < NCW; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    st.S2[mt][j][r] = S0[sbase + (long)(17 + 16 * (a0 + mt) + 4 * g + r) * dv + colb +
                                         16 * (ct0 + j) + lr] * kS2ToAcc;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int ra = 4 * g + r;
            if (owner) {
                st.S1[r] = S0[sbase + (long)(1 + ra) * dv + colb + 16 * own_ct + lr] * kS1ToAcc;
                st.S0acc[r] = S0[sbase + colb + 16 * own_ct + lr];
            }
            st.Z2[r] = 0.5f * (z0[zbase + 17 + 16 * ra + lr] + z0[zbase + 17 + 16 * lr + ra]) *
                       kS2ToAcc;
            st.z1[r] = z0[zbase + 1 + ra] * kS1ToAcc;
        }
        st.z0 = z0[zbase];
    }

    Src src;
    src.N = aN;
    src.M = aM;
    src.P = P;
    src.dv = dv;
    src.colb = colb;
    src.w = w;
    src.qb = (const char *)args.q + (long)head * aN * 32;
    src.kb = (const char *)args.k + (long)head * aN * 32;
    src.vb = (const char *)args.v + (long)head * aN * dv * 2;
    src.keb = (const char *)args.ke + (long)head * aM * 32;
    src.veb = (const char *)args.ve + (long)head * aM * dv * 2;
    const int jq = tid / (CW / 4), cq = tid % (CW / 4);  // v unit: 4 tokens x 4 columns
    const char *ybase = (const char *)args.y + (long)head * aN * dv * (int)sizeof(OutT);
    const int ybytes = args.y ? aN * dv * (int)sizeof(OutT) : 0;
    // ring slot of chunk c: (c - P) mod 3, so the first causal chunk uses slot 0
    auto ring = [P](int c) { return smem + (((c - P) % 3 + 3) % 3) * L::BUF; };
    f4 *const pbuf = (f4 *)(smem + L::PBUF);
    float *const ytiles = (float *)(smem + L::YBUF) + w * NT * 16 * L::YST;
    // pbuf slot of (token tile t, source row block mm, tile j) in this column group
    auto pslot = [n](int t, int mm, int j) { return (((t * NS + n) * MS + mm) * NCW + j) * 64; };

    // ---------------- prologue ----------------
    Staged stg = load_chunk<NCT>(src, 0, l, jq, cq);
    store_chunk<NCT>(ring(0), stg, w, l, jq, cq);
    stg = load_chunk<NCT>(src, 1, l, jq, cq);
    __syncthreads();
    Stage1Out s1a = stage1<NCT>(ring(0), t0, g, lr, st.Z2, st.z1, st.z0, args.eps);
    Stage1Out s1b = s1a;
    if (MS == 2) s1b = stage1<NCT>(ring(0), t1, g, lr, st.Z2, st.z1, st.z0, args.eps);

    // ---------------- JRT prefix: state update only ----------------
    for (int c = 0; c < P; ++c) {
        store_chunk<NCT>(ring(c + 1), stg, w, l, jq, cq);  // past the end: zeros, never used
        stg = load_chunk<NCT>(src, c + 2, l, jq, cq);
        __syncthreads();
        update<NCT, MS>(st, ring(c), a0, ct0, own_ct, owner, g, lr, (float)min(CH, aM - c * CH));
        if (c + 1 == P) {
            s1a = stage1<NCT>(ring(c + 1), t0, g, lr, st.Z2, st.z1, st.z0, args.eps);
            if (MS == 2) s1b = stage1<NCT>(ring(c + 1), t1, g, lr, st.Z2, st.z1, st.z0, args.eps);
        }
    }

    // ---------------- causal chunks ----------------
    // Memory-operation order inside one chunk: consume the prefetched inputs
    // (their loads are a whole chunk old), store the previous chunk's output,
    // then issue the next prefetch.  Loads and stores share one counter, so
    // waiting for a load also waits for every store issued before it; in this
    // order those stores are a whole chunk old too.
    for (int c = P; c < total; ++c) {
        store_chunk<NCT>(ring(c + 1), stg, w, l, jq, cq);
        if (c > P) {
            const int rb = (c - 1 - P) * CH;
            flush_y<NCW, OutT>(ytiles, ybase, ybytes, rb + 16 * t0, dv, colb + 16 * ct0, l);
            if (MS == 2)
                flush_y<NCW, OutT>(ytiles + 16 * L::YST, ybase, ybytes, rb + 16 * t1, dv,
                                   colb + 16 * ct0, l);
        }
        stg = load_chunk<NCT>(src, c + 2, l, jq, cq);
        __syncthreads();  // chunk c+1 staged; everyone is past chunk c-1

        const unsigned char *buf = ring(c);
        const _Float16 *Qs = (const _Float16 *)(buf + L::QS);
        const _Float16 *Vt = (const _Float16 *)(buf + L::VT);

        // -------- inter-chunk partial sums over this wave's feature rows --------
        {
            h8 S2op[MT / 2][NCW];
#pragma unroll
            for (int h = 0; h < MT / 2; ++h)
#pragma unroll
                for (int j = 0; j < NCW; ++j)
                    S2op[h][j] = cat8(to_h4(st.S2[2 * h][j]), to_h4(st.S2[2 * h + 1][j]));
            const h4 S1op = to_h4(st.S1 * 0.0625f);
            const float s0 = st.S0acc[0] * 0.001953125f;
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const _Float16 *qrow = Qs + (16 * it + lr) * QST;
                const h4 qb = *(const h4 *)(qrow + 4 * g);  // features 4g..4g+3
                const h2 b01 = (h2){qb[0], qb[1]}, b23 = (h2){qb[2], qb[3]};
                f4 acc[NCW];
#pragma unroll
                for (int j = 0; j < NCW; ++j) acc[j] = zero4;
#pragma unroll
                for (int h = 0; h < MT / 2; ++h) {
                    // slab: features (a0+2h, 4g+r) then (a0+2h+1, 4g+r)
                    const h2 qa = *(const h2 *)(qrow + a0 + 2 * h);
                    const h2 x0 = (h2){qa[0], qa[0]} * b01, x1 = (h2){qa[0], qa[0]} * b23;
                    const h2 x2 = (h2){qa[1], qa[1]} * b01, x3 = (h2){qa[1], qa[1]} * b23;
                    const h8 phq = (h8){x0[0], x0[1], x1[0], x1[1], x2[0], x2[1], x3[0], x3[1]};
#pragma unroll
                    for (int j = 0; j < NCW; ++j) acc[j] = mfma32(phq, S2op[h][j], acc[j]);
                }
                if (owner) {  // orders 0 and 1 of the owned column tile
                    const f4 o01 = mfma16(qb, S1op, (f4){s0, s0, s0, s0});
#pragma unroll
                    for (int j = 0; j < NCW; ++j)
                        if (j == m) acc[j] += o01;
                }
#pragma unroll
                for (int j = 0; j < NCW; ++j) pbuf[pslot(it, m, j) + l] = acc[j];
            }
        }

        update<NCT, MS>(st, buf, a0, ct0, own_ct, owner, g, lr, (float)min(CH, aN - (c - P) * CH));

        // A operands / denominators of this chunk; then stage 1 of the next one
        // (a chunk past the end is zeros: its result is never used)
        const Stage1Out ca = s1a, cb2 = s1b;
        s1a = stage1<NCT>(ring(c + 1), t0, g, lr, st.Z2, st.z1, st.z0, args.eps);
        if (MS == 2) s1b = stage1<NCT>(ring(c + 1), t1, g, lr, st.Z2, st.z1, st.z0, args.eps);
        __syncthreads();  // partial sums of chunk c are in LDS

        // -------- finish the wave's token tiles: partials + intra-chunk + normalise --------
#pragma unroll
        for (int ti = 0; ti < NT; ++ti) {
            const int t = ti == 0 ? t0 : t1;
            const Stage1Out &cs = ti == 0 ? ca : cb2;
            float *yt = ytiles + ti * 16 * L::YST;
            f4 part[NCW];
#pragma unroll
            for (int j = 0; j < NCW; ++j) {
                part[j] = pbuf[pslot(t, 0, j) + l];
#pragma unroll
                for (int mm = 1; mm < MS; ++mm) part[j] += pbuf[pslot(t, mm, j) + l];
                part[j] = mfma32(cs.aop0, *(const h8 *)(Vt + ts_idx(16 * (ct0 + j) + lr, 8 * g)), part[j]);
                if (t >= 2)
                    part[j] = mfma32(cs.aop1, *(const h8 *)(Vt + ts_idx(16 * (ct0 + j) + lr, 32 + 8 * g)),
                                     part[j]);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * g + r;
                const float rd = __shfl(cs.rden, row);
#pragma unroll
                for (int j = 0; j < NCW; ++j) yt[row * L::YST + 16 * j + lr] = part[j][r] * rd;
            }
        }
    }
    if (NC > 0) {
        const int rb = (NC - 1) * CH;
        flush_y<NCW, OutT>(ytiles, ybase, ybytes, rb + 16 * t0, dv, colb + 16 * ct0, l);
        if (MS == 2)
            flush_y<NCW, OutT>(ytiles + 16 * L::YST, ybase, ybytes, rb + 16 * t1, dv, colb + 16 * ct0, l);
    }

    // ---------------- final state ----------------
    if (args.S_out) {
        float *So = args.S_out;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int j = 0; j < NCW; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    So[sbase + (long)(17 + 16 * (a0 + mt) + 4 * g + r) * dv + colb + 16 * (ct0 + j) + lr] =
                        st.S2[mt][j][r] * kAccToS2;
        if (owner) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                So[sbase + (long)(1 + 4 * g + r) * dv + colb + 16 * own_ct + lr] = st.S1[r] * kAccToS1;
            if (g == 0) So[sbase + colb + 16 * own_ct + lr] = st.S0acc[0];
        }
    }
    if (args.z_out && cb == 0 && w == 0) {
        // z_out = z0 + (this call's tokens); the accumulator holds symmetrised z0.
        // All reads of z0 come before any write, so z_out may alias z0.
        const float *z0 = args.z0;
        float *zo = args.z_out;
        float z2v[4], z1v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int ra = 4 * g + r;
            float z2i = 0.f, zin = 0.f, z1in = 0.f;
            if (z0) {
                zin = z0[zbase + 17 + 16 * ra + lr];
                z2i = 0.5f * (zin + z0[zbase + 17 + 16 * lr + ra]) * kS2ToAcc;
                z1in = z0[zbase + 1 + ra];
            }
            z2v[r] = zin + (st.Z2[r] - z2i) * kAccToS2;
            z1v[r] = z1in + (st.z1[r] - z1in * kS1ToAcc) * kAccToS1;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int ra = 4 * g + r;
            zo[zbase + 17 + 16 * ra + lr] = z2v[r];
            if (lr == 0) zo[zbase + 1 + ra] = z1v[r];
        }
        if (l == 0) zo[zbase] = st.z0;
    }
}

template <int NCT, int MS, typename OutT>
hipError_t launch_one(const PrefillArgs &a, int n_cb, hipStream_t s)
{
    auto *k = prefill_mfma_kernel<NCT, MS, OutT>;
    constexpr int lds = lds_bytes<NCT, MS>();
    // more than 64 KiB of LDS per workgroup must be requested explicitly
    const hipError_t e =
        hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3((unsigned)(a.B * a.H * n_cb)), dim3(256), lds, s, a, n_cb);
    return hipGetLastError();
}

template <typename OutT>
hipError_t launch_cw(const PrefillArgs &a, int cw, hipStream_t s)
{
    const int n_cb = a.dv / cw;
    switch (cw) {
    case 64: return launch_one<4, PREFILL_MS64, OutT>(a, n_cb, s);
    case 32: return launch_one<2, PREFILL_MS32, OutT>(a, n_cb, s);
    default: return launch_one<1, 4, OutT>(a, n_cb, s);
    }
}

}  // namespace

hipError_t launch_prefill_mfma(const PrefillArgs &a, int col_split_allowed, hipStream_t s)
{
    const int heads = a.B * a.H;
    // columns per workgroup: split the value columns across workgroups until
    // the grid has at least PREFILL_MIN_WG workgroups
    int cw = a.dv;
    if (col_split_allowed) {
        while (cw > 16 && (long)heads * (a.dv / cw) < PREFILL_MIN_WG) cw >>= 1;
    }
    return a.y_bf16 ? launch_cw<uint16_t>(a, cw, s) : launch_cw<float>(a, cw, s);
}

}  // namespace bla
