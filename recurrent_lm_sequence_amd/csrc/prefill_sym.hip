// Chunked causal Taylor linear-attention prefill on gfx950 matrix cores, with
// the order-2 state held in compact symmetric form.
//
// Method: "Simple linear attention language models balance the recall-throughput
// tradeoff" notes, §2.5 (chunked form): for chunk b of 64 tokens
//   U_b = (M_b o Phi_Qb Phi_Kb^T) V_b + Phi_Qb S_<b,   S_<b = sum_{a<b} Phi_Ka^T V_a,
// with the same split for the denominator; §2.3 gives phi and the kernel
// K = 1 + q.k/4 + (q.k)^2/32 (d' = 16), §2.2 the recurrence this equals.
// "Just read twice" notes §2.6/§2.8: the JRT prefix state (non-causal sum over
// the M prefix tokens) is accumulated first and seeds the causal scan.
// Length-generalization notes §2.5 Eq. (4): an initial state is added to S, z.
// The same notes (§2.3) observe that vec(x x^T) repeats every off-diagonal
// product; the state here keeps each unordered pair once.
//
// Compact state.  (q.k)^2 = sum_a q_a^2 k_a^2 + 2 sum_{r=1..7} sum_a (q_a q_{a+r})(k_a k_{a+r})
// + 2 sum_{a<8} (q_a q_{a+8})(k_a k_{a+8}), indices mod 16: every unordered pair
// {a, b} appears once as (a, a + r) with r the circular distance.  The state is
// ten 16-row feature tiles:
//   T0        rows a: sum (k_a/128)^2 v                       (diagonal)
//   T1..T7    rows a: sum (k_a/64)(k_{a+r}/128) v              (pairs at distance r)
//   T8        rows a < 8: the same for r = 8; row 8: sum v / 16 (order 0); rows 9-15 zero
//   T9        rows a: sum (k_a/16) v                           (order 1)
// and the matching query features are q_a q_{a+r} (raw), 2^-5 for order 0 and
// q_a 2^-7 for order 1, so that every product of a query feature with a state
// row is 2^-9 times its term of phi(q).S.  Against the full 273-row state this
// is 160 rows: 41% fewer matrix-core operations in the two state products.
// Denominator state: count, sum k/16 and the symmetric 16x16 matrix
// sum (k/16)(k/16)^T, so phi(q).z = z0 + 4 q.z1 + 8 q^T Z2 q.
//
// gfx950 design.  One workgroup (4 wavefronts) owns one (batch, head) and a
// block of CW = 16*NCJ value columns and walks the sequence in 64-token
// chunks.  Wave w finishes token tile w (16 rows) of every chunk and owns the
// state tiles {T0-T2}, {T3-T5}, {T6,T7} or {T8,T9} (fp32 MFMA accumulators).
// Per chunk, wave w
//  * builds its query features in registers (one 32-byte q row per lane,
//    rotated with alignbit; no phi in memory) and multiplies them with the fp16
//    copy of the whole state in LDS (written by all waves after the previous
//    chunk) -- the inter-chunk term, as y^T tiles so that each lane ends with
//    4 adjacent output columns of one token;
//  * adds the causal intra-chunk term (score tiles q k^T on the matrix cores,
//    the polynomial on the vector ALUs) and normalises;
//  * updates its own state tiles with the chunk and writes their fp16 copy for
//    the next chunk into the other half of a double-buffered LDS area.
// Inputs are prefetched two chunks ahead into registers and staged through a
// two-slot LDS ring; one workgroup barrier per chunk.
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

constexpr int CH = 64;     // tokens per chunk
constexpr int QST = 24;    // halves per LDS row of raw q / k (48 B: conflict-free 16-byte row reads)
constexpr int NTILE = 10;  // feature tiles of the compact state
constexpr int KROWS = 51;  // key-operand rows: k/16, k/64, k/128 (16 each), ones, 2^-4, zero
constexpr int ROW_K16 = 0, ROW_K64 = 16, ROW_K128 = 32, ROW_ONE = 48, ROW_C4 = 49, ROW_ZERO = 50;
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit dwords (gfx9 family)

// ABI state row -> accumulator scales
constexpr float kPairToAcc = 6.9053396600248772e-04f;  // 2^-13 * 4 sqrt 2 (pair rows, T1..T8)
constexpr float kDiagToAcc = 3.4526698300124386e-04f;  // 2^-14 * 4 sqrt 2 (T0)
constexpr float kAccToPair = 1448.1546878700494f;      // 1 / kPairToAcc
constexpr float kAccToDiag = 2896.3093757400989f;      // 1 / kDiagToAcc
constexpr float kO1ToAcc = 0.125f, kAccToO1 = 8.0f;    // order 1 (T9)
constexpr float kO0ToAcc = 0.0625f, kAccToO0 = 16.0f;  // order 0 (T8 row 8)
constexpr float kZ2ToAcc = 0.022097086912079608f;      // sqrt 2 / 64
constexpr float kAccToZ2 = 45.254833995939045f;        // 32 sqrt 2
constexpr float kZ1ToAcc = 0.125f, kAccToZ1 = 8.0f;

// Token order inside a chunk as seen by the 16x16x32 operands (score tile rows
// are 4g+r with g = lane/16; two 16-row tiles form one 32-deep slab in which
// lane group g holds rows {4g..4g+3, 16+4g..16+4g+3}).  V and the key operand
// rows are stored in this "slot" order so every operand is one 16-byte read.
__device__ __forceinline__ int slot_of(int j) {
    return (j & 32) + ((j >> 2) & 3) * 8 + ((j >> 4) & 1) * 4 + (j & 3);
}
// Token-slot rows are 64 halves (8 blocks of 16 B), block index XOR-swizzled
// with the row so that operand reads and staging writes hit distinct banks.
__device__ __forceinline__ int tsw(int row) { return (row ^ (row >> 2)) & 7; }
__device__ __forceinline__ int ts_idx(int row, int x) {
    return row * 64 + (((x >> 3) ^ tsw(row)) << 3) + (x & 7);
}

__device__ __forceinline__ f4 mfma32(h8 a, h8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mfma16(h4 a, h4 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, h2));
}
__device__ __forceinline__ h2 as_h2(uint32_t x) { return __builtin_bit_cast(h2, x); }
__device__ __forceinline__ uint32_t as_u(h2 x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, bytes, kRsrcWord3);
}
__device__ __forceinline__ h4 to_h4(f4 x) { return __builtin_convertvector(x, h4); }
__device__ __forceinline__ h8 cat8(h4 lo, h4 hi) {
    return (h8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
__device__ __forceinline__ h8 mul8(h8 a, h8 b) { return a * b; }
__device__ __forceinline__ h8 h8_of(u4 x) { return __builtin_bit_cast(h8, x); }

extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

template <int NCJ>
struct Lay {
    static constexpr int CW = 16 * NCJ;                  // value columns per workgroup
    static constexpr int QR = 0;                         // [64][QST] raw q (fp16)
    static constexpr int KR = QR + 64 * QST * 2;         // [64][QST] raw k (fp16)
    static constexpr int KT = KR + 64 * QST * 2;         // [KROWS][64 slots] key operand rows
    static constexpr int VT = KT + KROWS * 128;          // [CW][64 slots] v
    static constexpr int SLOT = VT + CW * 128;           // bytes per ring slot
    static constexpr int SB = 2 * SLOT;                  // 2 x fp16 state copy [NTILE][CW][16]
    static constexpr int SBSZ = NTILE * CW * 32;
    static constexpr int TOTAL = SB + 2 * SBSZ;
};

// byte offset of the 16-byte block (key-operand row `row`, slab s, lane group g)
__device__ __forceinline__ int kt_off(int row, int s, int g) {
    return row * 128 + ((((4 * s + g)) ^ tsw(row)) << 4);
}
// half index in the state copy of (tile, column c, rows 8hb..8hb+7 of the tile)
__device__ __forceinline__ int sb_idx(int tile, int CW, int c, int hb) {
    return (tile * CW + c) * 16 + ((hb ^ ((c >> 3) & 1)) << 3);
}

struct Src {
    int N, M, P, dv, colb, tid, w;  // w: wave index (uniform, in a scalar register)
    const char *qb, *kb, *vb, *keb, *veb;  // this head's rows of q, k, v, k_e, v_e
};

struct Staged {  // one chunk's raw bf16 inputs held by one lane
    u2 v[4];
    u2 qk[2];
};

// Loads of chunk c (prefix chunks first): every lane issues the same six buffer
// loads; past the end of a head's tokens, or where the lane has no role, they
// read zeros (range-checked or zero-size resource).
template <int NCJ>
__device__ __forceinline__ Staged load_chunk(const Src s, int c)
{
    constexpr int CW = 16 * NCJ;
    Staged o;
    const bool pre = c < s.P;
    const int tok0 = (pre ? c : c - s.P) * CH;
    const int len = pre ? s.M : s.N;
    // v: unit (4 tokens x 4 columns), units 0 .. 16*CW/4 - 1
    const int jq = s.tid / (CW / 4), cq = s.tid % (CW / 4);
    const bool vrole = s.w < NCJ;  // 16 * CW / 4 units: the first NCJ waves
    const __amdgpu_buffer_rsrc_t vr = rsrc(pre ? s.veb : s.vb, vrole ? len * s.dv * 2 : 0);
#pragma unroll
    for (int r = 0; r < 4; ++r)
        o.v[r] = __builtin_amdgcn_raw_buffer_load_b64(
            vr, ((tok0 + 4 * jq + r) * s.dv + s.colb + 4 * cq) * 2, 0, 0);
    // threads 0-127: q of token t>>1, features 8(t&1)..+7 (causal chunks only);
    // threads 128-255: k of tokens 2p, 2p+1, features 4fq..4fq+3
    int o0, o1, bytes;
    const char *base;
    if (s.w < 2) {
        base = s.qb;
        bytes = pre ? 0 : s.N * 32;
        o0 = (tok0 + (s.tid >> 1)) * 32 + 16 * (s.tid & 1);
        o1 = o0 + 8;
    } else {
        const int l2 = s.tid - 128, p = l2 >> 2, fq = l2 & 3;
        base = pre ? s.keb : s.kb;
        bytes = len * 32;
        o0 = (tok0 + 2 * p) * 32 + 8 * fq;
        o1 = o0 + 32;
    }
    const __amdgpu_buffer_rsrc_t qr = rsrc(base, bytes);
    o.qk[0] = __builtin_amdgcn_raw_buffer_load_b64(qr, o0, 0, 0);
    o.qk[1] = __builtin_amdgcn_raw_buffer_load_b64(qr, o1, 0, 0);
    return o;
}

// Converts one lane's staged chunk to fp16 and writes it into ring slot `buf`.
template <int NCJ>
__device__ __forceinline__ void store_chunk(unsigned char *buf, const Staged in, int tid, int w)
{
    using L = Lay<NCJ>;
    constexpr int CW = L::CW;
    _Float16 *Vt = (_Float16 *)(buf + L::VT);
    if (w < NCJ) {  // v: tokens 4jq..4jq+3 (consecutive slots) x columns 4cq..4cq+3
        const int jq = tid / (CW / 4), cq = tid % (CW / 4);
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
    if (w < 2) {  // raw q, token t>>1, features 8(t&1)..
        const int tq = tid >> 1, h = tid & 1;
        u4 w;
        w.x = pack2(bf16_lo(in.qk[0].x), bf16_hi(in.qk[0].x));
        w.y = pack2(bf16_lo(in.qk[0].y), bf16_hi(in.qk[0].y));
        w.z = pack2(bf16_lo(in.qk[1].x), bf16_hi(in.qk[1].x));
        w.w = pack2(bf16_lo(in.qk[1].y), bf16_hi(in.qk[1].y));
        *(u4 *)(buf + L::QR + tq * QST * 2 + 16 * h) = w;
    } else {  // k of tokens 2p, 2p+1, features 4fq..4fq+3: raw rows and the key-operand rows
        const int l2 = tid - 128, p = l2 >> 2, fq = l2 & 3;
        float k0[4], k1[4];
        k0[0] = bf16_lo(in.qk[0].x); k0[1] = bf16_hi(in.qk[0].x);
        k0[2] = bf16_lo(in.qk[0].y); k0[3] = bf16_hi(in.qk[0].y);
        k1[0] = bf16_lo(in.qk[1].x); k1[1] = bf16_hi(in.qk[1].x);
        k1[2] = bf16_lo(in.qk[1].y); k1[3] = bf16_hi(in.qk[1].y);
        *(u2 *)(buf + L::KR + (2 * p) * QST * 2 + 8 * fq) = (u2){pack2(k0[0], k0[1]), pack2(k0[2], k0[3])};
        *(u2 *)(buf + L::KR + (2 * p + 1) * QST * 2 + 8 * fq) = (u2){pack2(k1[0], k1[1]), pack2(k1[2], k1[3])};
        _Float16 *Kt = (_Float16 *)(buf + L::KT);
        const int sl = slot_of(2 * p);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int a = 4 * fq + e;
            *(uint32_t *)(Kt + ts_idx(ROW_K16 + a, sl)) = pack2(k0[e] * 0.0625f, k1[e] * 0.0625f);
            *(uint32_t *)(Kt + ts_idx(ROW_K64 + a, sl)) = pack2(k0[e] * 0.015625f, k1[e] * 0.015625f);
            *(uint32_t *)(Kt + ts_idx(ROW_K128 + a, sl)) = pack2(k0[e] * 0.0078125f, k1[e] * 0.0078125f);
        }
    }
}

// key-operand rows (own, partner) of state tile `tile` for lane row a
__device__ __forceinline__ int own_row(int tile, int a) {
    if (tile == 0) return ROW_K128 + a;
    if (tile == 9) return ROW_K16 + a;
    if (tile == 8 && a >= 8) return a == 8 ? ROW_C4 : ROW_ZERO;
    return ROW_K64 + a;
}
__device__ __forceinline__ int part_row(int tile, int a) {
    if (tile == 9 || (tile == 8 && a >= 8)) return ROW_ONE;
    return ROW_K128 + ((a + tile) & 15);
}

// wave w owns state tiles TB(w) .. TB(w) + NT(w) - 1
__host__ __device__ constexpr int tile_base(int w) { return w == 0 ? 0 : w == 1 ? 3 : w == 2 ? 6 : 8; }
__host__ __device__ constexpr int tile_count(int w) { return w < 2 ? 3 : 2; }

template <int NCJ>
struct WaveState {
    f4 S[3][NCJ];  // own state tiles: rows a = 4g + r, column 16j + lr
    f4 Z2, z1;     // denominator state (initial + tokens so far), rows a = 4g + r
    float z0;
};

// State update with the chunk in ring slot `buf`: own state tiles, denominator.
template <int NCJ, int NT>
__device__ __forceinline__ void update(WaveState<NCJ> &st, const unsigned char *buf,
                                       const h8 (&vop)[2][NCJ], const int (&own)[3],
                                       const int (&part)[3], int g, int lr, float valid)
{
    using L = Lay<NCJ>;
    const h8 ones = (h8){1, 1, 1, 1, 1, 1, 1, 1};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            const h8 ko = *(const h8 *)(buf + L::KT + (own[tt] ^ (64 * s)));
            const h8 kp = *(const h8 *)(buf + L::KT + (part[tt] ^ (64 * s)));
            const h8 A = mul8(ko, kp);
#pragma unroll
            for (int j = 0; j < NCJ; ++j) st.S[tt][j] = mfma32(A, vop[s][j], st.S[tt][j]);
        }
        const h8 kt = *(const h8 *)(buf + L::KT + kt_off(ROW_K16 + lr, s, g));  // k/16 row a = lr
        st.Z2 = mfma32(kt, kt, st.Z2);
        st.z1 = mfma32(kt, ones, st.z1);
    }
    st.z0 += valid;
}

// fp16 copy of the own state tiles into state buffer `sb`
template <int NCJ, int NT>
__device__ __forceinline__ void write_state(const WaveState<NCJ> &st, _Float16 *sb, int tb, int g,
                                            int lr)
{
    constexpr int CW = 16 * NCJ;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int j = 0; j < NCJ; ++j)
            *(h4 *)(sb + sb_idx(tb + tt, CW, 16 * j + lr, g >> 1) + 4 * (g & 1)) = to_h4(st.S[tt][j]);
}

// One causal chunk for wave W (token tile W).
template <int NCJ, int W, typename OutT>
__device__ __forceinline__ void causal_chunk(WaveState<NCJ> &st, const unsigned char *buf,
                                             const _Float16 *sb_cur, _Float16 *sb_nxt,
                                             const int (&own)[3], const int (&part)[3],
                                             const __amdgpu_buffer_rsrc_t yr, int tok0, int ycol0,
                                             int dv, int g, int lr, float valid, float eps)
{
    using L = Lay<NCJ>;
    constexpr int CW = L::CW, NT = tile_count(W), TB = tile_base(W), T = W;
    const f4 zero4 = (f4){0.f, 0.f, 0.f, 0.f};
    const int h = g & 1;

    // value operands of both slabs (intra A operands and update B operands)
    h8 vop[2][NCJ];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int j = 0; j < NCJ; ++j)
            vop[s][j] = *(const h8 *)(buf + L::VT + 2 * ts_idx(16 * j + lr, 32 * s + 8 * g));

    // -------- inter-chunk term: y^T += S^T phi(q), slab by slab --------
    const unsigned char *qrow = buf + L::QR + (16 * T + lr) * QST * 2;
    uint32_t qr[8];  // this lane's q row rotated by 8h halves
    {
        const u4 lo = *(const u4 *)(qrow + 16 * h), hi = *(const u4 *)(qrow + 16 * (1 - h));
        qr[0] = lo.x; qr[1] = lo.y; qr[2] = lo.z; qr[3] = lo.w;
        qr[4] = hi.x; qr[5] = hi.y; qr[6] = hi.z; qr[7] = hi.w;
    }
    const uint32_t shift = g >= 2 ? 16u : 0u;
    f4 yacc[NCJ];
#pragma unroll
    for (int j = 0; j < NCJ; ++j) yacc[j] = zero4;
#pragma unroll
    for (int s = 0; s < 5; ++s) {
        uint32_t bq[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            uint32_t win = __builtin_amdgcn_alignbit(qr[(s + m + 1) & 7], qr[(s + m) & 7], shift);
            if (s == 4) {
                // lanes g=0: pairs at distance 8; g=1: order 0 (2^-5 at row 8);
                // g=2,3: order 1 (q_a 2^-7)
                if (g >= 2) win = 0x20002000u;  // (2^-7, 2^-7)
            }
            uint32_t p = as_u(as_h2(qr[m]) * as_h2(win));
            if (s == 4 && g == 1) p = m == 0 ? 0x00002800u : 0u;  // (2^-5, 0)
            bq[m] = p;
        }
        const h8 B = h8_of((u4){bq[0], bq[1], bq[2], bq[3]});
#pragma unroll
        for (int j = 0; j < NCJ; ++j) {
            const h8 A = *(const h8 *)(sb_cur + sb_idx(2 * s + (g >> 1), CW, 16 * j + lr, h));
            yacc[j] = mfma32(A, B, yacc[j]);
        }
    }

    // -------- intra-chunk scores and the denominator --------
    const h4 qB = *(const h4 *)(qrow + 8 * g);  // raw q features 4g..4g+3 of token 16T + lr
    float rowsum = 0.f;
    h4 part4[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
        part4[jt] = (h4){0, 0, 0, 0};
        if (jt > T) continue;
        const h4 kA = *(const h4 *)(buf + L::KR + (16 * jt + lr) * QST * 2 + 8 * g);
        const f4 cc = mfma16(kA, qB, zero4);  // [j = 16jt + 4g + r][i = 16T + lr] = q.k
        float xv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            // K / 2^9 = 2^-9 + 2^-11 cc + 2^-14 cc^2
            float x = __builtin_fmaf(cc[r], __builtin_fmaf(cc[r], 6.103515625e-05f, 4.8828125e-04f),
                                     1.953125e-03f);
            if (jt == T && 4 * g + r > lr) x = 0.f;  // causal mask j > i
            rowsum += x;
            xv[r] = x;
        }
        part4[jt] = to_h4((f4){xv[0], xv[1], xv[2], xv[3]});
    }
    // phi(q).z (orders 1, 2): sum_b q_b (4 z1_b + 8 (Z2 q)_b)
    const f4 Wz = mfma16(to_h4(st.Z2), qB, zero4);
    float pz = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) pz += (float)qB[r] * (4.f * st.z1[r] + 8.f * Wz[r]);
    float den = rowsum * 512.f + pz;
    den += __shfl_xor(den, 16);
    den += __shfl_xor(den, 32);
    const float rden = 512.f * __builtin_amdgcn_rcpf(den + st.z0 + eps);  // 1-ulp reciprocal

    // intra-chunk term: y^T += V^T A^T
#pragma unroll
    for (int s = 0; s < (T >= 2 ? 2 : 1); ++s) {
        const h8 B = cat8(part4[2 * s], part4[2 * s + 1]);
#pragma unroll
        for (int j = 0; j < NCJ; ++j) yacc[j] = mfma32(vop[s][j], B, yacc[j]);
    }

    // -------- state update with this chunk; fp16 copy for the next chunk --------
    update<NCJ, NT>(st, buf, vop, own, part, g, lr, valid);
    write_state<NCJ, NT>(st, sb_nxt, TB, g, lr);

    // -------- normalise and store: lane holds y[token 16T + lr][16j + 4g .. +3] --------
    const int tok = tok0 + 16 * T + lr;
#pragma unroll
    for (int j = 0; j < NCJ; ++j) {
        const f4 yv = yacc[j] * rden;
        const int off = (tok * dv + ycol0 + 16 * j + 4 * g) * (int)sizeof(OutT);
        if constexpr (sizeof(OutT) == 4) {
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, yv), yr, off, 0, 0);
        } else {
            const u2 hv = (u2){(uint32_t)f32_to_bf16_rne(yv[0]) | ((uint32_t)f32_to_bf16_rne(yv[1]) << 16),
                               (uint32_t)f32_to_bf16_rne(yv[2]) | ((uint32_t)f32_to_bf16_rne(yv[3]) << 16)};
            __builtin_amdgcn_raw_buffer_store_b64(hv, yr, off, 0, 0);
        }
    }
}

template <int NCJ>
struct Ctx {
    Src src;
    int tid, g, lr, P, NC, total, colb;
    float eps;
    __amdgpu_buffer_rsrc_t yr;
    int dv;
};

__device__ __forceinline__ unsigned char *ring(int slot_parity, int slot_bytes) {
    return smem + (slot_parity & 1) * slot_bytes;
}

// One JRT prefix chunk: stage the next chunk, prefetch, update the state.
template <int NCJ, int NT>
__device__ __forceinline__ void prefix_chunk(WaveState<NCJ> &st, const Ctx<NCJ> &x, int c, Staged &nx,
                                             const int (&own)[3], const int (&part)[3])
{
    using L = Lay<NCJ>;
    store_chunk<NCJ>(ring(c + 1, L::SLOT), nx, x.tid, x.src.w);
    nx = load_chunk<NCJ>(x.src, c + 3);
    const unsigned char *buf = ring(c, L::SLOT);
    h8 vop[2][NCJ];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int j = 0; j < NCJ; ++j)
            vop[s][j] = *(const h8 *)(buf + L::VT + 2 * ts_idx(16 * j + x.lr, 32 * s + 8 * x.g));
    update<NCJ, NT>(st, buf, vop, own, part, x.g, x.lr, (float)min(CH, x.src.M - c * CH));
    __syncthreads();
}

// The whole chunk walk of wave W: JRT prefix chunks (update only), then the
// causal chunks.  Register sets A and B alternate as the prefetch buffers.
template <int NCJ, int W, typename OutT>
__device__ __forceinline__ void walk(WaveState<NCJ> &st, const Ctx<NCJ> &x, Staged &rA, Staged &rB,
                                     const int (&own)[3], const int (&part)[3])
{
    using L = Lay<NCJ>;
    constexpr int NT = tile_count(W), TB = tile_base(W);
    const int g = x.g, lr = x.lr, tid = x.tid;
    _Float16 *const sb0 = (_Float16 *)(smem + L::SB);
    _Float16 *const sb1 = (_Float16 *)(smem + L::SB + L::SBSZ);

    // prefix: before chunk c the register set X (B for even c) holds chunk c+1
    // and the other set chunk c+2; chunk c is in ring slot c&1
    int c = 0;
    for (; c + 1 < x.P; c += 2) {
        prefix_chunk<NCJ, NT>(st, x, c, rB, own, part);
        prefix_chunk<NCJ, NT>(st, x, c + 1, rA, own, part);
    }
    if (c < x.P) {  // odd number of prefix chunks: the causal walk starts with set A
        prefix_chunk<NCJ, NT>(st, x, c, rB, own, part);
        const Staged t = rA;
        rA = rB;
        rB = t;
    }
    if (x.P > 0) {  // state after the prefix: the copy the first causal chunk reads
        write_state<NCJ, NT>(st, sb0, TB, g, lr);
        __syncthreads();
    }

    // causal chunks: chunk c (= P + i) in ring slot c&1, state copy i&1
    for (int i = 0; i < x.NC; i += 2) {
        const int c0 = x.P + i;
        store_chunk<NCJ>(ring(c0 + 1, L::SLOT), rB, tid, x.src.w);
        rB = load_chunk<NCJ>(x.src, c0 + 3);
        causal_chunk<NCJ, W, OutT>(st, ring(c0, L::SLOT), sb0, sb1, own, part, x.yr, i * CH, x.colb,
                                   x.dv, g, lr, (float)min(CH, x.src.N - i * CH), x.eps);
        __syncthreads();
        if (i + 1 < x.NC) {
            store_chunk<NCJ>(ring(c0 + 2, L::SLOT), rA, tid, x.src.w);
            rA = load_chunk<NCJ>(x.src, c0 + 4);
            causal_chunk<NCJ, W, OutT>(st, ring(c0 + 1, L::SLOT), sb1, sb0, own, part, x.yr,
                                       (i + 1) * CH, x.colb, x.dv, g, lr,
                                       (float)min(CH, x.src.N - (i + 1) * CH), x.eps);
            __syncthreads();
        }
    }
}

template <int NCJ, typename OutT>
__global__ __launch_bounds__(256, 1) void prefill_sym_kernel(PrefillArgs args, int n_cb)
{
    using L = Lay<NCJ>;
    constexpr int CW = L::CW;
    const int aN = args.N, aM = args.M, dv = args.dv;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, g = l >> 4, lr = l & 15;
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
    const int colb = cb * CW;
    const int P = (aM + CH - 1) / CH;
    const int NC = (aN + CH - 1) / CH;

    const int tb = tile_base(w), nt = tile_count(w);
    int own[3], part[3];
#pragma unroll
    for (int tt = 0; tt < 3; ++tt) {
        const int tile = min(tb + tt, NTILE - 1);
        own[tt] = kt_off(own_row(tile, lr), 0, g);
        part[tt] = kt_off(part_row(tile, lr), 0, g);
    }
    // slab s of a row is at kt_off(row, 0, g) ^ (64 s): the block index 4s + g
    // = 4s ^ g is XOR-swizzled, so slab 1 flips bit 2 of the block

    // ---------------- state ----------------
    const long sbase = (long)head * kD * dv;
    const long zbase = (long)head * kD;
    const f4 zero4 = (f4){0.f, 0.f, 0.f, 0.f};
    WaveState<NCJ> st;
#pragma unroll
    for (int tt = 0; tt < 3; ++tt)
#pragma unroll
        for (int j = 0; j < NCJ; ++j) st.S[tt][j] = zero4;
    st.Z2 = st.z1 = zero4;
    st.z0 = 0.f;
    if (args.S0) {
        const float *S0 = args.S0, *z0 = args.z0;
#pragma unroll
        for (int tt = 0; tt < 3; ++tt) {
            if (tt >= nt) break;
            const int tile = tb + tt;
#pragma unroll
            for (int j = 0; j < NCJ; ++j) {
                const long col = colb + 16 * j + lr;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int a = 4 * g + r;
                    float val = 0.f;
                    if (tile == 0) {
                        val = S0[sbase + (17 + 17 * a) * dv + col] * kDiagToAcc;
                    } else if (tile == 9) {
                        val = S0[sbase + (1 + a) * dv + col] * kO1ToAcc;
                    } else if (tile == 8 && a >= 8) {
                        if (a == 8) val = S0[sbase + col] * kO0ToAcc;
                    } else {
                        const int b = (a + tile) & 15;
                        val = 0.5f * (S0[sbase + (17 + 16 * a + b) * dv + col] +
                                      S0[sbase + (17 + 16 * b + a) * dv + col]) * kPairToAcc;
                    }
                    st.S[tt][j][r] = val;
                }
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int a = 4 * g + r;
            st.Z2[r] = 0.5f * (z0[zbase + 17 + 16 * a + lr] + z0[zbase + 17 + 16 * lr + a]) * kZ2ToAcc;
            st.z1[r] = z0[zbase + 1 + a] * kZ1ToAcc;
        }
        st.z0 = z0[zbase];
    }

    Ctx<NCJ> x;
    x.src.N = aN;
    x.src.M = aM;
    x.src.P = P;
    x.src.dv = dv;
    x.src.colb = colb;
    x.src.tid = tid;
    x.src.w = w;
    x.src.qb = (const char *)args.q + (long)head * aN * 32;
    x.src.kb = (const char *)args.k + (long)head * aN * 32;
    x.src.vb = (const char *)args.v + (long)head * aN * dv * 2;
    x.src.keb = (const char *)args.ke + (long)head * aM * 32;
    x.src.veb = (const char *)args.ve + (long)head * aM * dv * 2;
    x.tid = tid;
    x.g = g;
    x.lr = lr;
    x.P = P;
    x.NC = NC;
    x.total = P + NC;
    x.colb = colb;
    x.eps = args.eps;
    x.dv = dv;
    x.yr = rsrc((const char *)args.y + (long)head * aN * dv * (int)sizeof(OutT),
                args.y ? aN * dv * (int)sizeof(OutT) : 0);

    // ---------------- prologue ----------------
    // constant key-operand rows in both ring slots
    for (int i = tid; i < 2 * 3 * 64; i += 256) {
        const int slot = i / 192, rr = (i / 64) % 3, xx = i % 64;
        const float cv = rr == 0 ? 1.f : (rr == 1 ? 0.0625f : 0.f);
        ((_Float16 *)(smem + slot * L::SLOT + L::KT))[ts_idx(ROW_ONE + rr, xx)] = (_Float16)cv;
    }
    Staged rA = load_chunk<NCJ>(x.src, 0);
    Staged rB = load_chunk<NCJ>(x.src, 1);
    store_chunk<NCJ>(ring(0, L::SLOT), rA, tid, w);
    rA = load_chunk<NCJ>(x.src, 2);
    if (P == 0) {
        _Float16 *sb0 = (_Float16 *)(smem + L::SB);
        if (w == 0) write_state<NCJ, 3>(st, sb0, 0, g, lr);
        else if (w == 1) write_state<NCJ, 3>(st, sb0, 3, g, lr);
        else if (w == 2) write_state<NCJ, 2>(st, sb0, 6, g, lr);
        else write_state<NCJ, 2>(st, sb0, 8, g, lr);
    }
    __syncthreads();

    switch (w) {
    case 0: walk<NCJ, 0, OutT>(st, x, rA, rB, own, part); break;
    case 1: walk<NCJ, 1, OutT>(st, x, rA, rB, own, part); break;
    case 2: walk<NCJ, 2, OutT>(st, x, rA, rB, own, part); break;
    default: walk<NCJ, 3, OutT>(st, x, rA, rB, own, part); break;
    }

    // ---------------- final state ----------------
    // Pair rows are written as S0 + (accumulated - initial) so that an initial
    // state that is not symmetric in (a, b) keeps its antisymmetric part; every
    // entry is read and written by one lane (in place is safe).
    if (args.S_out) {
        const float *S0 = args.S0;
        float *So = args.S_out;
#pragma unroll
        for (int tt = 0; tt < 3; ++tt) {
            if (tt >= nt) break;
            const int tile = tb + tt;
#pragma unroll
            for (int j = 0; j < NCJ; ++j) {
                const long col = colb + 16 * j + lr;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int a = 4 * g + r;
                    const float acc = st.S[tt][j][r];
                    if (tile == 0) {
                        const long o = sbase + (17 + 17 * a) * dv + col;
                        const float s0 = S0 ? S0[o] : 0.f;
                        So[o] = s0 + (acc - s0 * kDiagToAcc) * kAccToDiag;
                    } else if (tile == 9) {
                        const long o = sbase + (1 + a) * dv + col;
                        const float s0 = S0 ? S0[o] : 0.f;
                        So[o] = s0 + (acc - s0 * kO1ToAcc) * kAccToO1;
                    } else if (tile == 8 && a >= 8) {
                        if (a == 8) {
                            const long o = sbase + col;
                            const float s0 = S0 ? S0[o] : 0.f;
                            So[o] = s0 + (acc - s0 * kO0ToAcc) * kAccToO0;
                        }
                    } else {
                        const int b = (a + tile) & 15;
                        const long o1 = sbase + (17 + 16 * a + b) * dv + col;
                        const long o2 = sbase + (17 + 16 * b + a) * dv + col;
                        const float s1 = S0 ? S0[o1] : 0.f, s2 = S0 ? S0[o2] : 0.f;
                        const float d = (acc - 0.5f * (s1 + s2) * kPairToAcc) * kAccToPair;
                        So[o1] = s1 + d;
                        So[o2] = s2 + d;
                    }
                }
            }
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
                z2i = 0.5f * (zin + z0[zbase + 17 + 16 * lr + ra]) * kZ2ToAcc;
                z1in = z0[zbase + 1 + ra];
            }
            z2v[r] = zin + (st.Z2[r] - z2i) * kAccToZ2;
            z1v[r] = z1in + (st.z1[r] - z1in * kZ1ToAcc) * kAccToZ1;
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

template <int NCJ, typename OutT>
hipError_t launch_one(const PrefillArgs &a, int n_cb, hipStream_t s)
{
    auto *k = prefill_sym_kernel<NCJ, OutT>;
    constexpr int lds = Lay<NCJ>::TOTAL;
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
    case 64: return launch_one<4, OutT>(a, n_cb, s);
    case 32: return launch_one<2, OutT>(a, n_cb, s);
    default: return launch_one<1, OutT>(a, n_cb, s);
    }
}

}  // namespace

hipError_t launch_prefill_sym(const PrefillArgs &a, int col_split_allowed, hipStream_t s)
{
    const int heads = a.B * a.H;
    // columns per workgroup: split the value columns across workgroups until
    // there are at least 256 workgroups (one per compute unit)
    int cw = a.dv;
    if (col_split_allowed) {
        while (cw > 16 && (long)heads * (a.dv / cw) < 256) cw >>= 1;
    }
    return a.y_bf16 ? launch_cw<uint16_t>(a, cw, s) : launch_cw<float>(a, cw, s);
}

}  // namespace bla
