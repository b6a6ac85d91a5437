// Chunked causal Taylor linear-attention prefill on gfx950 matrix cores, with
// the order-2 state held in compact symmetric form.
//
// Method: "Simple linear attention language models balance the recall-throughput
// tradeoff" notes, §2.5 (chunked form): for chunk b of C tokens
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
//   T0        rows a: sum (k_a/16)^2 v                        (diagonal)
//   T1..T7    rows a: sum (k_a/16)(k_{a+r}/16) v               (pairs at distance r)
//   T8        rows a < 8: the same for r = 8; row 8: sum v / 16 (order 0); rows 9-15 zero
//   T9        rows a: sum (k_a/16) v                           (order 1)
// and the matching query features are 2^-5 q_a q_{a+r} (2^-6 q_a^2 on the
// diagonal), 2^-5 for order 0 and 2^-7 q_a for order 1, so that every product
// of a query feature with a state row is 2^-9 times its term of phi(q).S.
// Against the full 273-row state this is 160 rows: 41% fewer matrix-core
// operations in the two state products.  Denominator state: count, sum k/16
// and the symmetric 16x16 matrix sum (k/16)(k/16)^T, so that
// phi(q).z = z0 + 4 q.z1 + 8 q^T Z2 q.
//
// gfx950 design.  One workgroup of sixteen wavefronts (four per SIMD) owns
// one (batch, head) and a block of CW = 16*NCJ value columns and walks the
// sequence in chunks of C = 128 tokens (8 token tiles of 16).  The waves take
// two roles, so that every SIMD interleaves two independent instruction
// streams per chunk:
//  * token wave w (0-7) finishes token tile t of every chunk (t = w for w < 4,
//    11 - w otherwise: the two token waves of a SIMD share 9 causal score
//    tiles): it builds its query features in registers (one 32-byte q row per
//    lane, rotated with alignbit; phi is never stored) and multiplies them
//    with the fp16 copy of the whole state in LDS (the inter-chunk term), in
//    the same straight-line block as its score tiles (q k^T on the matrix
//    cores, the Taylor polynomial on the vector ALUs), then adds the causal
//    intra-chunk term and normalises.  Outputs are y^T tiles, so each lane
//    stores 4 adjacent columns of one token straight from registers;
//  * state wave u (waves 8-15) owns state tiles {T0,T1}, {T2,T3} (u = 0, 1)
//    or T(u+2) (u = 2-7) for all CW columns in fp32 MFMA accumulators (and
//    the denominator state on u = ZW); it stages each causal chunk into a
//    two-slot LDS ring, prefetching two chunks ahead, updates its tiles with
//    the chunk and writes their fp16 copy for the next chunk into the other
//    half of a double-buffered LDS area.  Update-only prefix chunks (a JRT
//    prefix, or the tokens before a sequence segment) are staged by the token
//    waves, which have no other work then.
// The per-wave token tile and state tiles are uniform values; one workgroup
// barrier per chunk.  A call with few heads splits the value columns (two
// workgroups per head) and then the sequence, so that the grid still covers the
// compute units: segments either walk the head's earlier tokens as prefix
// chunks, or start from prefix sums of per-segment partial states (the
// chunk-parallel split, which with long segments keeps one column block per
// head and doubles the segments instead).
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

constexpr int CH = 128;    // tokens per chunk
constexpr int TT = 8;      // 16-token tiles per chunk = wavefronts per workgroup
constexpr int QST = 24;    // halves per LDS row of raw q (48 B: conflict-free 16-byte row reads)
constexpr int KPT = 56;    // bytes per token of raw k rows (32 + 24 pad: conflict-free 8-byte reads)
constexpr int NTILE = 10;  // feature tiles of the compact state
constexpr int KROWS = 19;  // key-operand rows: k/16 (16 rows), ones, 2^-4, zero
constexpr int ROW_K16 = 0, ROW_ONE = 16, ROW_C4 = 17, ROW_ZERO = 18;
constexpr int SLOTS = CH;  // token slots per key / value operand row
constexpr int ROWH = SLOTS + 16;  // halves per token-slot row (32-byte pad, see the note on LDS banks)
constexpr int ZW = 2;      // wave that keeps the denominator state (one state tile, light causal work)
constexpr int ZBSZ = 64 * (8 + 16);  // shared denominator state: Z2 operand (h4) + z1 (f4) per lane
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit dwords (gfx9 family)

// ABI state row -> accumulator scales
constexpr float kPairToAcc = 0.022097086912079608f;  // 2^-8 * 4 sqrt 2 (T0..T8 rows)
constexpr float kAccToPair = 45.254833995939045f;    // 1 / kPairToAcc
constexpr float kO1ToAcc = 0.125f, kAccToO1 = 8.0f;  // order 1 (T9)
constexpr float kO0ToAcc = 0.0625f, kAccToO0 = 16.0f;  // order 0 (T8 row 8)
constexpr float kZ2ToAcc = 0.022097086912079608f;    // sqrt 2 / 64
constexpr float kAccToZ2 = 45.254833995939045f;      // 32 sqrt 2
constexpr float kZ1ToAcc = 0.125f, kAccToZ1 = 8.0f;

// Token order inside a chunk as seen by the 16x16x32 operands: the score tile
// rows are 4g+r (g = lane/16), and two 16-row tiles form one 32-deep slab in
// which lane group g holds rows {4g..4g+3, 16+4g..16+4g+3}.  V and the key
// operand rows are stored in this "slot" order so every operand is one
// 16-byte read.
__device__ __forceinline__ int slot_of(int j) {
    return (j & ~31) + ((j >> 2) & 3) * 8 + ((j >> 4) & 1) * 4 + (j & 3);
}
// LDS banks (measured on gfx950 with the bank-conflict counter and timed
// access loops): a 16-byte read is served in four cycles of 16 lanes each,
// lanes {0-7, 16-23}, {8-15, 24-31}, {32-39, 48-55}, {40-47, 56-63}; a cycle is
// conflict-free when its lanes touch 16 distinct 16-byte bank groups, the group
// of byte address a being bits 4-7 of a with address bit 8 folded into bit 7.
// Token-slot rows are padded to ROWH halves (288 bytes: 2 groups + 256 bytes),
// so the operand reads of 8 consecutive rows x 2 adjacent 16-byte blocks cover
// all 16 groups, and every operand address is a per-lane base plus a constant.
__device__ __forceinline__ int ts_idx(int row, int x) { return row * ROWH + x; }

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
__device__ __forceinline__ h8 h8_of(u4 x) { return __builtin_bit_cast(h8, x); }
// Sum over the four 16-lane rows of a wavefront (lanes l, l^16, l^32, l^48):
// two row-swap permutes on the vector ALU, no LDS round trip.
__device__ __forceinline__ float sum_rows4(float x) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float s = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}
// Value select.  (A conditional expression on two lvalues selects their
// addresses; on struct fields that forces the struct into scratch memory.)
template <typename T> __device__ __forceinline__ T pick(bool c, T a, T b) { return c ? a : b; }
// A uniform value the compiler must treat as recomputed here: keeps per-wave
// constants (and the branch conditions derived from them) from being hoisted
// out of the chunk loop, where they would exhaust the scalar registers.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+s"(x));
    return x;
}

template <int NCJ>
struct Lay {
    static constexpr int CW = 16 * NCJ;               // value columns per workgroup
    static constexpr int QR = 0;                      // [CH][QST] raw q (fp16)
    static constexpr int KR = QR + CH * QST * 2;      // [CH][KPT bytes] raw k (fp16)
    static constexpr int KT = KR + CH * KPT;          // [KROWS][ROWH] key operand rows
    static constexpr int VT = KT + KROWS * ROWH * 2;  // [CW][ROWH] v
    static constexpr int SLOT = VT + CW * ROWH * 2;   // bytes per ring slot
    static constexpr int SB = 2 * SLOT;               // 2 x fp16 state copy [NTILE][CW][16]
    static constexpr int SBSZ = NTILE * CW * 32;
    static constexpr int ZB = SB + 2 * SBSZ;           // 2 x shared denominator state
    static constexpr int TOTAL = ZB + 2 * ZBSZ;
};

// The workgroup's LDS, statically sized for the widest column block so that
// its address is known at compile time and every constant part of an LDS
// address folds into the instruction offset.
__shared__ __attribute__((aligned(16))) unsigned char smem[Lay<4>::TOTAL];

// byte offset of the 16-byte block (key-operand row `row`, slab 0, lane group g);
// slab s of the same row is 64 s bytes further
__device__ __forceinline__ int kt_off(int row, int g) { return row * ROWH * 2 + 16 * g; }
// half index in the state copy of (tile, column c, rows 8hb..8hb+7 of the tile);
// the two 16-byte halves are swapped on columns with bit 2 set (conflict-free reads)
__device__ __forceinline__ int sb_idx(int tile, int CW, int c, int hb) {
    return (tile * CW + c) * 16 + ((hb ^ ((c >> 2) & 1)) << 3);
}
// byte offset of raw k (token j, features 4g..4g+3): one padded row per token
__device__ __forceinline__ int kr_off(int j, int g) { return j * KPT + 8 * g; }

// v staging unit (4 tokens x 4 columns) of thread t.  Each group of 16 lanes
// holds two column quads of opposite parity and eight token quads (all
// combinations of bits 0-2), so its 8-byte writes of rows 4cq+e (68 dwords
// apart per row) cover 16 distinct bank pairs.
template <int NCQ>
__device__ __forceinline__ void v_unit(int t, int &jq, int &cq) {
    const int jlo = (t >> 1) & 7;  // token quad bits 0-2
    if constexpr (NCQ == 16) {
        cq = (t & 1) | (((t >> 4) & 7) << 1);
        jq = jlo | (((t >> 7) & 3) << 3);
    } else if constexpr (NCQ == 8) {
        cq = (t & 1) | (((t >> 4) & 3) << 1);
        jq = jlo | (((t >> 6) & 3) << 3);
    } else {
        cq = (t & 1) | (((t >> 4) & 1) << 1);
        jq = jlo | (((t >> 5) & 3) << 3);
    }
}

struct Staged {  // one chunk's raw bf16 inputs held by one lane
    u2 v[4];
    u2 qk[2];
};

// Lane-constant byte offsets of one chunk's loads, relative to the chunk's
// first token (the chunk's base and remaining length go into the buffer
// descriptors, built on the scalar unit per chunk):
//   v: unit (4 tokens x 4 columns), waves 0 .. 2 NCJ - 1 (others read nothing);
//   waves 0-3: q of token t>>1, features 8(t&1)..+7 (causal chunks only);
//   waves 4-7: k of tokens 2p, 2p+1 (p = t & 63), features 4fq..4fq+3.
struct LoadOff {
    int v[4], qk[2];
};

template <int NCJ>
__device__ __forceinline__ LoadOff load_offsets(int tid, int w, int dv, int colb)
{
    LoadOff o;
    int jq, cq;
    v_unit<4 * NCJ>(tid, jq, cq);
#pragma unroll
    for (int r = 0; r < 4; ++r) o.v[r] = ((4 * jq + r) * dv + colb + 4 * cq) * 2;
    if (w < 4) {
        o.qk[0] = (tid >> 1) * 32 + 16 * (tid & 1);
        o.qk[1] = o.qk[0] + 8;
    } else {
        const int l2 = tid - 256, p = l2 & 63, fq = l2 >> 6;
        o.qk[0] = (2 * p) * 32 + 8 * fq;
        o.qk[1] = o.qk[0] + 32;
    }
    return o;
}

// Descriptor of the rows [tok0, len) of a tensor with `row_bytes` per token:
// loads past the end read zeros, stores past the end are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const char *base, int tok0, int len, int row_bytes)
{
    const int rows = len - tok0;
    return rsrc(base + (long)tok0 * row_bytes, rows > 0 ? rows * row_bytes : 0);
}

__device__ __forceinline__ Staged load_chunk(const LoadOff &o, __amdgpu_buffer_rsrc_t vr,
                                             __amdgpu_buffer_rsrc_t qkr)
{
    Staged st;
#pragma unroll
    for (int r = 0; r < 4; ++r) st.v[r] = __builtin_amdgcn_raw_buffer_load_b64(vr, o.v[r], 0, 0);
    st.qk[0] = __builtin_amdgcn_raw_buffer_load_b64(qkr, o.qk[0], 0, 0);
    st.qk[1] = __builtin_amdgcn_raw_buffer_load_b64(qkr, o.qk[1], 0, 0);
    return st;
}

// Converts one lane's staged chunk to fp16 and writes it into ring slot `buf`.
template <int NCJ>
__device__ __forceinline__ void store_chunk(unsigned char *buf, const Staged in, int tid, int w)
{
    using L = Lay<NCJ>;
    constexpr int CW = L::CW;
    _Float16 *Vt = (_Float16 *)(buf + L::VT);
    if (w < 2 * NCJ) {  // v: tokens 4jq..4jq+3 (consecutive slots) x columns 4cq..4cq+3
        int jq, cq;
        v_unit<CW / 4>(tid, jq, cq);
        const int s0 = slot_of(4 * jq);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float f[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t wd = pick<uint32_t>(e < 2, in.v[r].x, in.v[r].y);
                f[r] = (e & 1) ? bf16_hi(wd) : bf16_lo(wd);
            }
            *(u2 *)(Vt + ts_idx(4 * cq + e, s0)) = (u2){pack2(f[0], f[1]), pack2(f[2], f[3])};
        }
    }
    if (w < 4) {  // raw q, token t>>1, features 8(t&1)..
        const int tq = tid >> 1, h = tid & 1;
        u4 wv;
        wv.x = pack2(bf16_lo(in.qk[0].x), bf16_hi(in.qk[0].x));
        wv.y = pack2(bf16_lo(in.qk[0].y), bf16_hi(in.qk[0].y));
        wv.z = pack2(bf16_lo(in.qk[1].x), bf16_hi(in.qk[1].x));
        wv.w = pack2(bf16_lo(in.qk[1].y), bf16_hi(in.qk[1].y));
        *(u4 *)(buf + L::QR + tq * QST * 2 + 16 * h) = wv;
    } else {  // k of tokens 2p, 2p+1, features 4fq..4fq+3: raw rows and k/16 operand rows
        const int l2 = tid - 256, p = l2 & 63, fq = l2 >> 6;
        float k0[4], k1[4];
        k0[0] = bf16_lo(in.qk[0].x); k0[1] = bf16_hi(in.qk[0].x);
        k0[2] = bf16_lo(in.qk[0].y); k0[3] = bf16_hi(in.qk[0].y);
        k1[0] = bf16_lo(in.qk[1].x); k1[1] = bf16_hi(in.qk[1].x);
        k1[2] = bf16_lo(in.qk[1].y); k1[3] = bf16_hi(in.qk[1].y);
        *(u2 *)(buf + L::KR + kr_off(2 * p, fq)) = (u2){pack2(k0[0], k0[1]), pack2(k0[2], k0[3])};
        *(u2 *)(buf + L::KR + kr_off(2 * p + 1, fq)) = (u2){pack2(k1[0], k1[1]), pack2(k1[2], k1[3])};
        _Float16 *Kt = (_Float16 *)(buf + L::KT);
        const int sl = slot_of(2 * p);
#pragma unroll
        for (int e = 0; e < 4; ++e)  // (token 2p, token 2p+1) of feature 4fq+e, times 1/16 (exact)
            *(uint32_t *)(Kt + ts_idx(ROW_K16 + 4 * fq + e, sl)) =
                as_u(as_h2(pack2(k0[e], k1[e])) * as_h2(0x2c002c00u));
    }
}

// key-operand rows (own, partner) of state tile `tile` for lane row a
__device__ __forceinline__ int own_row(int tile, int a) {
    if (tile == 8 && a >= 8) return a == 8 ? ROW_C4 : ROW_ZERO;
    return ROW_K16 + a;
}
__device__ __forceinline__ int part_row(int tile, int a) {
    if (tile == 9 || (tile == 8 && a >= 8)) return ROW_ONE;
    return ROW_K16 + ((a + tile) & 15);
}

// state tiles of wave w: {0,1}, {2,3}, then one tile each (w + 2)
__device__ __forceinline__ int tile_base(int w) { return w < 2 ? 2 * w : w + 2; }
__device__ __forceinline__ int tile_count(int w) { return w < 2 ? 2 : 1; }

template <int NCJ>
struct WaveState {
    f4 S[2][NCJ];  // own state tiles: rows a = 4g + r, column 16j + lr
    f4 Z2, z1;     // denominator state (initial + tokens so far), rows a = 4g + r
    float z0;
};

// Per-lane constants of a wave.
struct Lane {
    int w, t, g, lr, tb, nt;
    int own[2], part[2];  // key-operand byte offsets (slab 0) of the own state tiles
    int kt;               // key-operand byte offset (slab 0) of k/16 row lr
};

template <int NCJ>
__device__ __forceinline__ void write_state(const WaveState<NCJ> &st, _Float16 *sb, const Lane &ln)
{
    constexpr int CW = 16 * NCJ;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        if (tt >= ln.nt) break;
#pragma unroll
        for (int j = 0; j < NCJ; ++j)
            *(h4 *)(sb + sb_idx(ln.tb + tt, CW, 16 * j + ln.lr, ln.g >> 1) + 4 * (ln.g & 1)) =
                to_h4(st.S[tt][j]);
    }
}

// Shared denominator state (sum (k/16)(k/16)^T as the fp16 operand of the
// Z2 q product, and sum k/16), written by its owner wave for the next chunk.
__device__ __forceinline__ void write_z(const f4 Z2, const f4 z1, unsigned char *zb, int l)
{
    *(h4 *)(zb + 8 * l) = to_h4(Z2);
    *(f4 *)(zb + 512 + 16 * l) = z1;
}

// Uniform description of where each chunk's inputs live: P update-only prefix
// chunks over M tokens (keys and values at keb, veb), then the causal tokens.
struct Ctx {
    int P, N, M, dv, w;
    const char *qb, *kb, *vb, *keb, *veb;  // this head's rows
    int vrole;                             // this wave stages v
};

// Descriptors of chunk c (prefix chunks first) for this wave's loads.
__device__ __forceinline__ void chunk_srcs(const Ctx &x, int c, __amdgpu_buffer_rsrc_t &vr,
                                           __amdgpu_buffer_rsrc_t &qkr)
{
    if (c < x.P) {
        const int tok0 = c * CH;
        vr = chunk_rsrc(x.veb, tok0, x.vrole ? x.M : 0, x.dv * 2);
        qkr = chunk_rsrc(pick<const char *>(x.w < 4, x.qb, x.keb), tok0, x.w < 4 ? 0 : x.M, 32);
    } else {
        const int tok0 = (c - x.P) * CH;
        vr = chunk_rsrc(x.vb, tok0, x.vrole ? x.N : 0, x.dv * 2);
        qkr = chunk_rsrc(pick<const char *>(x.w < 4, x.qb, x.kb), tok0, x.N, 32);
    }
}

// Ring slot of chunk c (prefix chunks first) is (c + P) & 1, so that causal
// chunk i sits in slot i & 1: in the causal loop (unrolled by two) the slot is
// a compile-time constant and folds into the LDS instruction offsets.
__device__ __forceinline__ unsigned char *ring(int parity, int slot_bytes) {
    return smem + (parity & 1) * slot_bytes;
}

// Initial state of the wave's state tiles and (wave ZW) the denominator state:
// S0/z0 converted to the accumulator scales, or zeros.  Pair rows take the
// symmetrised (S[a][b] + S[b][a]) / 2 of the full layout, or the compact pair
// row / 2 (the diagonal itself).
// Initial value, in the accumulator domain, of state element (tile, row a,
// column col): symmetrised pair rows (S[a][b] + S[b][a]) / 2 from the full layout,
// or the compact pair row (which holds the sum) / 2 (diagonal: itself).
__device__ __forceinline__ float init_S(const PrefillArgs &args, long sbase, int tile, int a, long col)
{
    const float *S0 = args.S0;
    const int dv = args.dv;
    if (tile == 9) return S0[sbase + (1 + a) * dv + col] * kO1ToAcc;
    if (tile == 8 && a >= 8) return a == 8 ? S0[sbase + col] * kO0ToAcc : 0.f;
    const int b = (a + tile) & 15;
    if (args.compact) {
        const float sc = S0[sbase + (17 + compact_pair(min(a, b), max(a, b))) * dv + col];
        return (a == b ? sc : 0.5f * sc) * kPairToAcc;
    }
    return 0.5f * (S0[sbase + (17 + 16 * a + b) * dv + col] + S0[sbase + (17 + 16 * b + a) * dv + col]) * kPairToAcc;
}
__device__ __forceinline__ float init_Z2(const PrefillArgs &args, long zbase, int a, int b)
{
    const float *z0 = args.z0;
    if (args.compact) {
        const float zc = z0[zbase + 17 + compact_pair(min(a, b), max(a, b))];
        return (a == b ? zc : 0.5f * zc) * kZ2ToAcc;
    }
    return 0.5f * (z0[zbase + 17 + 16 * a + b] + z0[zbase + 17 + 16 * b + a]) * kZ2ToAcc;
}
__device__ __forceinline__ float init_z1(const PrefillArgs &args, long zbase, int a)
{
    return args.z0[zbase + 1 + a] * kZ1ToAcc;
}

template <int NCJ>
__device__ __forceinline__ void load_state(WaveState<NCJ> &st, const PrefillArgs &args, const Lane &ln, int colb,
                                           long sbase, long zbase)
{
    const int g = ln.g, lr = ln.lr;
    const f4 zero4 = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int j = 0; j < NCJ; ++j) st.S[tt][j] = zero4;
    st.Z2 = st.z1 = zero4;
    st.z0 = 0.f;
    if (args.S0) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            if (tt >= ln.nt) break;
#pragma unroll
            for (int j = 0; j < NCJ; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    st.S[tt][j][r] = init_S(args, sbase, ln.tb + tt, 4 * g + r, colb + 16 * j + lr);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            st.Z2[r] = init_Z2(args, zbase, 4 * g + r, lr);
            st.z1[r] = init_z1(args, zbase, 4 * g + r);
        }
        st.z0 = args.z0[zbase];
    }
}

// Full-layout rows of element (tile, row a) of the compact state: the pair's two
// orders (r2 < 0 when there is one row: the diagonal, order 0 and order 1; r1 < 0
// for the unused rows 9-15 of T8), with the scales between the ABI rows and the
// accumulator.
__device__ __forceinline__ void full_rows(int tile, int a, int &r1, int &r2, float &to_acc, float &from_acc)
{
    if (tile == 9) {
        r1 = 1 + a;
        r2 = -1;
        to_acc = kO1ToAcc;
        from_acc = kAccToO1;
    } else if (tile == 8 && a >= 8) {
        r1 = a == 8 ? 0 : -1;
        r2 = -1;
        to_acc = kO0ToAcc;
        from_acc = kAccToO0;
    } else if (tile == 0) {
        r1 = 17 + 17 * a;
        r2 = -1;
        to_acc = kPairToAcc;
        from_acc = kAccToPair;
    } else {
        const int b = (a + tile) & 15;
        r1 = 17 + 16 * a + b;
        r2 = 17 + 16 * b + a;
        to_acc = kPairToAcc;
        from_acc = kAccToPair;
    }
}

// The final state in the full layout: the wave's state tiles and (wave ZW,
// first column block) z.  Each row is written as S0 + (accumulated - initial),
// where the accumulator started from the pair's symmetrised initial value
// (S0[a][b] + S0[b][a]) / 2, so that an initial state that is not symmetric keeps
// its antisymmetric part; z likewise.  With an initial state a tile's initial
// values are loaded first, by every lane (an element with one row or none reads
// a dummy row of its own head and discards it, so that no load sits under a
// divergent branch), then one wait, then the tile's stores: on gfx9 the
// vector-memory counter also counts stores, so a wait between stores would hold
// each store until the earlier ones complete.  Every entry is read and written
// by one lane, after its reads, so the state may be updated in place.
template <int NCJ, bool HAS_INIT>
__device__ __forceinline__ void store_full(const WaveState<NCJ> &st, const PrefillArgs &args, const Lane &ln,
                                           int colb, int cb, long sbase, long zbase)
{
    const int g = ln.g, lr = ln.lr, dv = args.dv, l = 16 * g + lr;
    const bool want_z = args.z_out != nullptr && cb == 0 && ln.w == ZW;
    const float *S0 = args.S0, *z0 = args.z0;
    float *So = args.S_out, *zo = args.z_out;
    float zin[4], ztr[4], z1in[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) zin[r] = ztr[r] = z1in[r] = 0.f;
    if (HAS_INIT && want_z) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int ra = 4 * g + r;
            zin[r] = z0[zbase + 17 + 16 * ra + lr];
            ztr[r] = z0[zbase + 17 + 16 * lr + ra];
            z1in[r] = z0[zbase + 1 + ra];
        }
    }
    // one tile at a time: its initial values, one wait, its stores
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        if (!So || tt >= ln.nt) break;
        int r1[4], r2[4];
        float ta[4], fa[4], s1[NCJ][4], s2[NCJ][4];
#pragma unroll
        for (int r = 0; r < 4; ++r) full_rows(ln.tb + tt, 4 * g + r, r1[r], r2[r], ta[r], fa[r]);
#pragma unroll
        for (int j = 0; j < NCJ; ++j) {
            const long col = colb + 16 * j + lr;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                s1[j][r] = HAS_INIT ? S0[sbase + (long)max(r1[r], 0) * dv + col] : 0.f;
                s2[j][r] = HAS_INIT ? S0[sbase + (long)max(r2[r], 0) * dv + col] : 0.f;
            }
        }
        if (HAS_INIT) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0) expcnt(7) lgkmcnt(15)
#pragma unroll
        for (int j = 0; j < NCJ; ++j) {
            const long col = colb + 16 * j + lr;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float acc = st.S[tt][j][r], i1 = s1[j][r], i2 = s2[j][r];
                if (r2[r] >= 0) {  // a pair: one rounded change added to both orders
                    const float d = (acc - 0.5f * (i1 + i2) * ta[r]) * fa[r];
                    So[sbase + (long)r1[r] * dv + col] = i1 + d;
                    So[sbase + (long)r2[r] * dv + col] = i2 + d;
                } else if (r1[r] >= 0) {
                    So[sbase + (long)r1[r] * dv + col] = i1 + (acc - i1 * ta[r]) * fa[r];
                }
            }
        }
    }
    if (want_z) {
        if (HAS_INIT) __builtin_amdgcn_s_waitcnt(0x0F70);  // z0 read before z_out is written
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int ra = 4 * g + r;
            zo[zbase + 17 + 16 * ra + lr] = zin[r] + (st.Z2[r] - 0.5f * (zin[r] + ztr[r]) * kZ2ToAcc) * kAccToZ2;
            if (lr == 0) zo[zbase + 1 + ra] = z1in[r] + (st.z1[r] - z1in[r] * kZ1ToAcc) * kAccToZ1;
        }
        if (l == 0) zo[zbase] = st.z0;
    }
}

// Final state of the wave's state tiles and (wave ZW, first column block) z.
template <int NCJ>
__device__ __forceinline__ void store_state(const WaveState<NCJ> &st, const PrefillArgs &args, const Lane &ln,
                                            int colb, int cb, long sbase, long zbase)
{
    if (!args.compact) {
        if (args.S0)
            store_full<NCJ, true>(st, args, ln, colb, cb, sbase, zbase);
        else
            store_full<NCJ, false>(st, args, ln, colb, cb, sbase, zbase);
        return;
    }
    const int g = ln.g, lr = ln.lr, dv = args.dv, l = 16 * g + lr;
    if (args.S_out) {
        // compact rows: the pair row is the sum of both orders, 2 * acc / scale
        // (the accumulator already holds half the initial pair row)
        float *So = args.S_out;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            if (tt >= ln.nt) break;
            const int tile = ln.tb + tt;
#pragma unroll
            for (int j = 0; j < NCJ; ++j) {
                const long col = colb + 16 * j + lr;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int a = 4 * g + r;
                    const float acc = st.S[tt][j][r];
                    if (tile == 9) {
                        So[sbase + (1 + a) * dv + col] = acc * kAccToO1;
                    } else if (tile == 8 && a >= 8) {
                        if (a == 8) So[sbase + col] = acc * kAccToO0;
                    } else {
                        const int b = (a + tile) & 15;
                        So[sbase + (17 + compact_pair(min(a, b), max(a, b))) * dv + col] =
                            (a == b ? 1.f : 2.f) * acc * kAccToPair;
                    }
                }
            }
        }
    }
    if (args.z_out && cb == 0 && ln.w == ZW) {
        // compact z: the accumulators hold z0 (pair entries halved) plus this call's sums
        float *zo = args.z_out;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int ra = 4 * g + r;
            if (ra <= lr) zo[zbase + 17 + compact_pair(ra, lr)] = (ra == lr ? 1.f : 2.f) * st.Z2[r] * kAccToZ2;
            if (lr == 0) zo[zbase + 1 + ra] = st.z1[r] * kAccToZ1;
        }
        if (l == 0) zo[zbase] = st.z0;
    }
}

// The inter-chunk term and the score tiles of token tile T in one
// straight-line block: the matrix-core products of slab s of the state and
// the vector-ALU Taylor weights of key tile s are independent, so one wave
// keeps both units busy.  Every LDS operand is read in the step that uses it
// (the four waves of a SIMD cover the latency), which keeps the wave within
// the register budget of four waves per SIMD.  Returns the row sum of the
// fp16 weights.
template <int NCJ, int T>
__device__ __forceinline__ float inter_scores(f4 (&yacc)[NCJ], h4 (&part4)[TT], const uint32_t (&qr)[8],
                                              const uint32_t (&own5)[4], uint32_t diag_sc, uint32_t shift,
                                              const _Float16 *sb_cur, const unsigned char *kr, h4 qB7,
                                              int g, int lr)
{
    constexpr int CW = 16 * NCJ;
    constexpr int STEPS = T + 1 > 5 ? T + 1 : 5;
    const int h = g & 1;
    const f4 c5 = (f4){0.03125f, 0.03125f, 0.03125f, 0.03125f};
    const h2 one2 = (h2){1, 1};
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
        if (st < 5) {
            h8 A[NCJ];
#pragma unroll
            for (int j = 0; j < NCJ; ++j) A[j] = *(const h8 *)(sb_cur + sb_idx(2 * st + (g >> 1), CW, 16 * j + lr, h));
            uint32_t bq[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                uint32_t win = __builtin_amdgcn_alignbit(qr[(st + m + 1) & 7], qr[(st + m) & 7], shift);
                if (st == 0) win = as_u(as_h2(win) * as_h2(diag_sc));
                if (st == 4 && g >= 2) win = 0x34003400u;
                uint32_t pq = as_u(as_h2(own5[m]) * as_h2(win));
                if (st == 4 && g == 1) pq = m == 0 ? 0x00002800u : 0u;
                bq[m] = pq;
            }
            const h8 B = h8_of((u4){bq[0], bq[1], bq[2], bq[3]});
#pragma unroll
            for (int j = 0; j < NCJ; ++j) yacc[j] = mfma32(A[j], B, yacc[j]);
        }
        if (st <= T) {
            const h4 kA = *(const h4 *)(kr + kr_off(16 * st + lr, g));
            const f4 dd = mfma16(kA, qB7, c5);
            float xv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float x = __builtin_fmaf(dd[r], dd[r], 9.765625e-04f);
                if (st == T && 4 * g + r > lr) x = 0.f;
                xv[r] = x;
            }
            part4[st] = to_h4((f4){xv[0], xv[1], xv[2], xv[3]});
            rs0 = __builtin_amdgcn_fdot2((h2){part4[st][0], part4[st][1]}, one2, rs0, false);
            rs1 = __builtin_amdgcn_fdot2((h2){part4[st][2], part4[st][3]}, one2, rs1, false);
        }
    }
    if constexpr (T + 1 < TT) part4[T + 1] = (h4){0, 0, 0, 0};
    return rs0 + rs1;
}

constexpr int TW = TT;                  // token waves (one per token tile)
constexpr int NTHR_WS = 64 * (TW + 8);  // token + state waves

// Token-wave part of causal chunk (token tile ln.t).  zprev: order-0
// denominator state (initial count plus the tokens before this chunk).
template <int NCJ, typename OutT>
__device__ __forceinline__ void token_chunk(const unsigned char *buf, const _Float16 *sb_cur,
                                            const unsigned char *zb_cur, const Lane &ln,
                                            const __amdgpu_buffer_rsrc_t yr, int dv, float zprev, float eps)
{
    using L = Lay<NCJ>;
    const f4 zero4 = (f4){0.f, 0.f, 0.f, 0.f};
    const int g = ln.g, lr = ln.lr, t = ln.t, h = g & 1;

    const unsigned char *qrow = buf + L::QR + (16 * t + lr) * QST * 2;
    uint32_t qr[8];  // this lane's q row rotated by 8h halves
    {
        const u4 lo = *(const u4 *)(qrow + 16 * h), hi = *(const u4 *)(qrow + 16 * (1 - h));
        qr[0] = lo.x; qr[1] = lo.y; qr[2] = lo.z; qr[3] = lo.w;
        qr[4] = hi.x; qr[5] = hi.y; qr[6] = hi.z; qr[7] = hi.w;
    }
    const uint32_t shift = g >= 2 ? 16u : 0u;
    uint32_t own5[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) own5[m] = as_u(as_h2(qr[m]) * as_h2(0x28002800u));
    const uint32_t diag_sc = g < 2 ? 0x38003800u : 0x3c003c00u;
    f4 yacc[NCJ];
#pragma unroll
    for (int j = 0; j < NCJ; ++j) yacc[j] = zero4;
    const h4 qB = *(const h4 *)(qrow + 8 * g);
    const h4 qB7 = qB * (h4){0.0078125f16, 0.0078125f16, 0.0078125f16, 0.0078125f16};
    h4 part4[TT];
    float rowsum = 0.f;
    const unsigned char *kr = buf + L::KR;
    switch (t) {
    case 0: rowsum = inter_scores<NCJ, 0>(yacc, part4, qr, own5, diag_sc, shift, sb_cur, kr, qB7, g, lr); break;
    case 1: rowsum = inter_scores<NCJ, 1>(yacc, part4, qr, own5, diag_sc, shift, sb_cur, kr, qB7, g, lr); break;
    case 2: rowsum = inter_scores<NCJ, 2>(yacc, part4, qr, own5, diag_sc, shift, sb_cur, kr, qB7, g, lr); break;
    case 3: rowsum = inter_scores<NCJ, 3>(yacc, part4, qr, own5, diag_sc, shift, sb_cur, kr, qB7, g, lr); break;
    case 4: rowsum = inter_scores<NCJ, 4>(yacc, part4, qr, own5, diag_sc, shift, sb_cur, kr, qB7, g, lr); break;
    case 5: rowsum = inter_scores<NCJ, 5>(yacc, part4, qr, own5, diag_sc, shift, sb_cur, kr, qB7, g, lr); break;
    case 6: rowsum = inter_scores<NCJ, 6>(yacc, part4, qr, own5, diag_sc, shift, sb_cur, kr, qB7, g, lr); break;
    default: rowsum = inter_scores<NCJ, 7>(yacc, part4, qr, own5, diag_sc, shift, sb_cur, kr, qB7, g, lr); break;
    }
    const h4 Z2op = *(const h4 *)(zb_cur + 8 * (16 * g + lr));
    const f4 z1v = *(const f4 *)(zb_cur + 512 + 16 * (16 * g + lr));
    const f4 Wz = mfma16(Z2op, qB, zero4);
    float pz = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) pz += (float)qB[r] * (4.f * z1v[r] + 8.f * Wz[r]);
    const float den = sum_rows4(rowsum * 512.f + pz);
    const float rden = 512.f * __builtin_amdgcn_rcpf(den + zprev + eps);

    // intra-chunk term: the value slabs of the key tiles at or before tile t
#pragma unroll
    for (int sl = 0; sl < CH / 32; ++sl) {
        if (2 * sl > t) break;
        h8 vop[NCJ];
#pragma unroll
        for (int j = 0; j < NCJ; ++j) vop[j] = *(const h8 *)(buf + L::VT + 2 * ts_idx(16 * j + lr, 32 * sl + 8 * g));
        const h8 B = cat8(part4[2 * sl], part4[2 * sl + 1]);
#pragma unroll
        for (int j = 0; j < NCJ; ++j) yacc[j] = mfma32(vop[j], B, yacc[j]);
    }

    const int yoff = ((16 * t + lr) * dv + 4 * g) * (int)sizeof(OutT);
#pragma unroll
    for (int j = 0; j < NCJ; ++j) {
        const f4 yv = yacc[j] * rden;
        const int off = yoff + 16 * j * (int)sizeof(OutT);
        if constexpr (sizeof(OutT) == 4) {
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, yv), yr, off, 0, 0);
        } else {
            const u2 hv = (u2){f32x2_to_bf16x2(yv[0], yv[1]), f32x2_to_bf16x2(yv[2], yv[3])};
            __builtin_amdgcn_raw_buffer_store_b64(hv, yr, off, 0, 0);
        }
    }
}

// State-wave part of a chunk in ring slot `buf`: the update of the wave's NT
// state tiles and (HASZ: wave ZW) the denominator state, one 32-token slab at a
// time (32 or 16 columns).  The operands of slab s + 1 are read from LDS while
// slab s's products run (two register sets), so that the LDS latency is not
// exposed at every slab.
template <int NCJ, int NT, bool HASZ>
__device__ __forceinline__ void state_update_t(WaveState<NCJ> &st, const unsigned char *buf, const Lane &ln)
{
    using L = Lay<NCJ>;
    const h8 ones = (h8){1, 1, 1, 1, 1, 1, 1, 1};
    struct Ops {
        h8 v[NCJ], own[NT], part[NT], kt;
    };
    auto load = [&](Ops &o, int s) {
#pragma unroll
        for (int j = 0; j < NCJ; ++j) o.v[j] = *(const h8 *)(buf + L::VT + 2 * ts_idx(16 * j + ln.lr, 32 * s + 8 * ln.g));
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            o.own[tt] = *(const h8 *)(buf + L::KT + ln.own[tt] + 64 * s);
            o.part[tt] = *(const h8 *)(buf + L::KT + ln.part[tt] + 64 * s);
        }
        if constexpr (HASZ) o.kt = *(const h8 *)(buf + L::KT + ln.kt + 64 * s);
    };
    Ops o[2];
    load(o[0], 0);
#pragma unroll
    for (int s = 0; s < CH / 32; ++s) {
        if (s + 1 < CH / 32) load(o[(s + 1) & 1], s + 1);
        __builtin_amdgcn_sched_barrier(0);  // the next slab's reads stay ahead of these products
        const Ops &c = o[s & 1];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            const h8 A = c.own[tt] * c.part[tt];
#pragma unroll
            for (int j = 0; j < NCJ; ++j) st.S[tt][j] = mfma32(A, c.v[j], st.S[tt][j]);
        }
        if constexpr (HASZ) {
            st.Z2 = mfma32(c.kt, c.kt, st.Z2);
            st.z1 = mfma32(c.kt, ones, st.z1);
        }
    }
}

// The update of this wave's state tiles.  64 columns: one loop over the wave's
// one or two tiles, each slab's operands read where they are used (a second
// register set would spill).  32 or 16 columns: one of three straight-line
// variants (two tiles, or one with or without the denominator state), chosen
// by one uniform branch per chunk with no loads under it, double-buffered.
template <int NCJ>
__device__ __forceinline__ void state_update(WaveState<NCJ> &st, const unsigned char *buf, const Lane &ln)
{
    // At 64 columns the state waves are the last at the chunk barrier: while they
    // update, their SIMD issues their instructions before the token waves'.
    if constexpr (NCJ == 4) __builtin_amdgcn_s_setprio(2);
    if constexpr (NCJ == 4) {
        using L = Lay<NCJ>;
        const h8 ones = (h8){1, 1, 1, 1, 1, 1, 1, 1};
#pragma unroll
        for (int s = 0; s < CH / 32; ++s) {
            h8 v[NCJ];
#pragma unroll
            for (int j = 0; j < NCJ; ++j)
                v[j] = *(const h8 *)(buf + L::VT + 2 * ts_idx(16 * j + ln.lr, 32 * s + 8 * ln.g));
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                if (tt >= ln.nt) break;
                const h8 A = *(const h8 *)(buf + L::KT + ln.own[tt] + 64 * s) *
                             *(const h8 *)(buf + L::KT + ln.part[tt] + 64 * s);
#pragma unroll
                for (int j = 0; j < NCJ; ++j) st.S[tt][j] = mfma32(A, v[j], st.S[tt][j]);
            }
            if (ln.w == ZW) {
                const h8 kt = *(const h8 *)(buf + L::KT + ln.kt + 64 * s);
                st.Z2 = mfma32(kt, kt, st.Z2);
                st.z1 = mfma32(kt, ones, st.z1);
            }
        }
    } else if (ln.nt == 2)
        state_update_t<NCJ, 2, false>(st, buf, ln);
    else if (ln.w == ZW)
        state_update_t<NCJ, 1, true>(st, buf, ln);
    else
        state_update_t<NCJ, 1, false>(st, buf, ln);
    if constexpr (NCJ == 4) __builtin_amdgcn_s_setprio(0);
}

// Chunk-parallel form of the sequence split (three launches, for few heads and
// long sequences): pass 1 (kModePartial) has every segment but the last sum its
// own tokens' contribution to the state, starting from zero; pass 2
// (scan_partials_kernel) replaces those, in segment order, by exclusive prefix
// sums; pass 3 (kModeSeeded) starts each segment's causal walk from S0 plus its
// prefix sum instead of walking the earlier tokens again ([LG] §2.5: a state
// carried into the scan; the sum over a sequence is the sum of its segments'
// sums).  The partials stay in the accumulator domain of the compact tiles.
// Each workgroup keeps its partial in its own rows and columns of y (segment
// rows, its CW columns), which pass 3 overwrites with y after reading it, so no
// other memory is needed and no two workgroups touch the same bytes.
constexpr int kModeWalk = 0, kModePartial = 1, kModeSeeded = 2;
// kModeSeededFold: pass 3 of a call that updates its state in place.  Pass 2 has
// already added the initial state (and its order-0 count) to every prefix sum, so
// no segment reads S0 or z0 except the last one's lanes, each reading the entries
// it then overwrites; the column split is then safe with z in place too.
constexpr int kModeSeededFold = 3;
// kModeStateOnly: a call that wants no y (and has no JRT prefix) only needs the
// sum over all its tokens: they are walked as update-only chunks from S0, like a
// partial, and the final state is stored.
constexpr int kModeStateOnly = 4;
// The chunk-parallel split costs two more launches and the scan, about the time of
// walking 1000-2000 tokens of prefix; it replaces the walk of (nseg - 2) * seglen
// tokens on the longest segment.
constexpr int kScanMinSaved = 2048;
constexpr int kPartialZ = NTILE * 16;  // partial float index of Z2 (256 values), then z1 (16): x CW

// Float f of the partial of the workgroup whose first token row is trow and
// first column colb: row f / fpr of its segment, 4-byte slot f % fpr of its
// columns (fpr = floats per row in those columns).
__device__ __forceinline__ float *partial_ptr(const PrefillArgs &a, long trow, int colb, int fpr, int f)
{
    const int ysz = a.y_bf16 ? 2 : 4;
    char *base = (char *)a.y + (trow * a.dv + colb) * ysz;
    return (float *)(base + (long)(f / fpr) * a.dv * ysz + (f % fpr) * 4);
}

// Partial index of state element (tile, row a, column c) of a CW-column block,
// and of the denominator entries.
__device__ __forceinline__ int pidx_S(int tile, int a, int c, int CW) { return (tile * 16 + a) * CW + c; }
__device__ __forceinline__ int pidx_Z2(int a, int b, int CW) { return kPartialZ * CW + a * 16 + b; }
__device__ __forceinline__ int pidx_z1(int a, int CW) { return kPartialZ * CW + 256 + a; }
__device__ __forceinline__ int pidx_z0(int CW) { return kPartialZ * CW + 272; }  // order-0 count (pass 2 only)
constexpr int partial_floats(int CW) { return kPartialZ * CW + 256 + 16 + 1; }

// Floats per row of a workgroup's columns of y, and the rows one partial takes.
__device__ __forceinline__ int partial_fpr(const PrefillArgs &a, int CW) { return CW * (a.y_bf16 ? 2 : 4) / 4; }
__device__ __forceinline__ int partial_rows(const PrefillArgs &a, int CW)
{
    const int fpr = partial_fpr(a, CW);
    return (partial_floats(CW) + fpr - 1) / fpr;
}

// Stores the wave's accumulators as the partial in slot `slot` (0, or 1 for a JRT
// prefix partial, rows [rows, 2 rows) of the segment).
template <int NCJ>
__device__ __forceinline__ void store_partial(const WaveState<NCJ> &st, const PrefillArgs &args, const Lane &ln,
                                              long trow, int colb, int slot)
{
    constexpr int CW = 16 * NCJ;
    const int g = ln.g, lr = ln.lr, fpr = partial_fpr(args, CW);
    trow += (long)slot * partial_rows(args, CW);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        if (tt >= ln.nt) break;
#pragma unroll
        for (int j = 0; j < NCJ; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                *partial_ptr(args, trow, colb, fpr, pidx_S(ln.tb + tt, 4 * g + r, 16 * j + lr, CW)) = st.S[tt][j][r];
    }
    if (ln.w == ZW) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            *partial_ptr(args, trow, colb, fpr, pidx_Z2(4 * g + r, lr, CW)) = st.Z2[r];
            if (lr == 0) *partial_ptr(args, trow, colb, fpr, pidx_z1(4 * g + r, CW)) = st.z1[r];
        }
    }
}

// Adds the segment's prefix sum (pass 2's output) to the initial accumulators:
// every load first, then the additions.
template <int NCJ>
__device__ __forceinline__ void add_partial(WaveState<NCJ> &st, const PrefillArgs &args, const Lane &ln, long trow,
                                            int colb)
{
    constexpr int CW = 16 * NCJ;
    const int g = ln.g, lr = ln.lr, fpr = partial_fpr(args, CW);
    const bool zw = ln.w == ZW;
    float p[2][NCJ][4], pz2[4], pz1[4];
    const float pz0 = *partial_ptr(args, trow, colb, fpr, pidx_z0(CW));
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int j = 0; j < NCJ; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                p[tt][j][r] = tt < ln.nt
                                  ? *partial_ptr(args, trow, colb, fpr, pidx_S(ln.tb + tt, 4 * g + r, 16 * j + lr, CW))
                                  : 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        pz2[r] = zw ? *partial_ptr(args, trow, colb, fpr, pidx_Z2(4 * g + r, lr, CW)) : 0.f;
        pz1[r] = zw ? *partial_ptr(args, trow, colb, fpr, pidx_z1(4 * g + r, CW)) : 0.f;
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int j = 0; j < NCJ; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) st.S[tt][j][r] += p[tt][j][r];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        st.Z2[r] += pz2[r];
        st.z1[r] += pz1[r];
    }
    st.z0 += pz0;
}

// Column split (ncb = 2): workgroup (head, cb) owns value columns
// [cb * CW, (cb + 1) * CW) of its head; both walk every token, and only cb = 0
// writes the denominator state.
// Sequence split (nseg > 1): workgroup (head, seg) produces the outputs of tokens
// [seg * seglen, (seg + 1) * seglen) of its head.  The state before its first
// token is either the sum over the earlier tokens, which it accumulates itself by
// walking them as update-only prefix chunks (kModeWalk, no JRT prefix: the same
// path a JRT prefix takes), or S0 plus the prefix sum that passes 1 and 2 of the
// chunk-parallel split left in its rows of y (kModeSeeded / kModeSeededFold);
// only the last segment writes the final state.  In the partial pass
// (kModePartial) a workgroup instead sums its segment, or a part of the JRT
// prefix, from zero and stores the sum as a partial.
template <int NCJ, typename OutT>
__global__ __launch_bounds__(NTHR_WS, 1) void prefill_ws_kernel(PrefillArgs args, int ncb, int nseg, int seglen,
                                                             int mode, int ncp, int pseglen)
{
    using L = Lay<NCJ>;
    const int aM = args.M, dv = args.dv;
    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool token_wave = w < TW;
    const int u = w - TW;        // state-wave index
    const int utid = tid - 64 * TW;  // thread index among the state waves
    Lane ln;
    ln.g = l >> 4;
    ln.lr = l & 15;
    ln.w = token_wave ? w : u;
    ln.t = w < 4 ? w : 11 - w;
    ln.tb = tile_base(max(u, 0));
    ln.nt = token_wave ? 0 : tile_count(u);
    const int g = ln.g, lr = ln.lr;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        const int tile = min(ln.tb + tt, NTILE - 1);
        ln.own[tt] = kt_off(own_row(tile, lr), g);
        ln.part[tt] = kt_off(part_row(tile, lr), g);
    }
    ln.kt = kt_off(ROW_K16 + lr, g);
    // XCD-aware block -> (head, column block, segment): blocks dispatch
    // round-robin over the 8 XCDs, so the column blocks and segments of one head
    // (which read the same queries and keys) share an XCD and its L2
    const int heads = args.B * args.H, nsub = ncb * nseg;
    int head, sub;
    if (nsub == 1) {
        head = blockIdx.x;
        sub = 0;
    } else if ((heads & 7) == 0) {
        const int xcd = blockIdx.x & 7, r = blockIdx.x >> 3;
        head = (r / nsub) * 8 + xcd;
        sub = r % nsub;
    } else {
        head = blockIdx.x / nsub;
        sub = blockIdx.x % nsub;
    }
    const int cb = sub % ncb, seg = sub / ncb;
    const int colb = cb * L::CW;                        // first value column of this workgroup
    // in the partial pass, segments ncp.. sum parts of the JRT prefix and keep them
    // in the rows of causal segment seg - ncp
    const bool pre_part = mode == kModePartial && seg >= ncp;
    const bool own_walk = mode == kModePartial || mode == kModeStateOnly;  // the segment's tokens, update only
    const int cseg = pre_part ? seg - ncp : seg;        // causal segment (its rows of y)
    const int tok0 = cseg * seglen;                     // first token of that segment
    const int segN = min(args.N - tok0, seglen);        // tokens of that segment
    const int aN = own_walk ? 0 : segN;                 // causal tokens
    const bool last_seg = seg == nseg - 1;
    int pstart = 0, pcnt = 0;                           // a prefix partial's valid tokens
    if (pre_part) {
        const int j = seg - ncp;
        pstart = min(args.M, max(j * pseglen, args.M - valid_prefix(args, head / args.H)));
        pcnt = max(0, min(args.M, (j + 1) * pseglen) - pstart);
    }
    // update-only prefix: the JRT prefix (unsplit), the head's tokens before the
    // segment (walk), or in the partial pass the segment's own tokens or its part
    // of the JRT prefix; mv also counts the tokens before the causal ones for the
    // order-0 denominator (a seeded segment walks no prefix)
    const bool fold = mode == kModeSeededFold, seeded = mode == kModeSeeded || fold;
    const int mv = __builtin_amdgcn_readfirstlane(
        own_walk             ? (pre_part ? pcnt : segN)
        : seeded             ? valid_prefix(args, head / args.H) + tok0
        : nseg == 1          ? valid_prefix(args, head / args.H)
                             : tok0);
    const int P = seeded ? 0 : (mv + CH - 1) / CH;
    const int NC = (aN + CH - 1) / CH;
    const int ND = args.compact ? kDc : kD;
    const long sbase = (long)head * ND * dv;
    const long zbase = (long)head * ND;
    const long trow = (long)head * args.N + tok0;       // row of the segment's first token

    // constant key-operand rows (ones, 2^-4, zero) in both ring slots
    for (int i = tid; i < 2 * 3 * SLOTS; i += NTHR_WS) {
        const int slot = i / (3 * SLOTS), rr = (i / SLOTS) % 3, xx = i % SLOTS;
        const float cv = rr == 0 ? 1.f : (rr == 1 ? 0.0625f : 0.f);
        ((_Float16 *)(smem + slot * L::SLOT + L::KT))[ts_idx(ROW_ONE + rr, xx)] = (_Float16)cv;
    }

    if (token_wave) {
        // At 32 and 16 columns the token waves with the most causal tiles (t = 4-7)
        // are the last at the chunk barrier: they issue first on their SIMD.
        if (NCJ < 4 && w >= 4) __builtin_amdgcn_s_setprio(1);
        // order-0 denominator state before the first causal chunk
        float zc = (args.S0 && !fold ? args.z0[zbase] : 0.f) + (float)mv;
        if (fold) zc += *partial_ptr(args, trow, colb, partial_fpr(args, L::CW), pidx_z0(L::CW));
        const int ybpt = dv * (int)sizeof(OutT);
        const char *yb = (const char *)args.y + trow * ybpt + colb * (int)sizeof(OutT);
        const int ylen = args.y ? aN : 0;
        if (P == 0) {
            __syncthreads();                  // prologue
        } else {
            // Prefix: the token waves stage the prefix chunks and the first causal
            // chunk (chunk c in ring slot (c + P) & 1, loaded one chunk ahead) while
            // the state waves only update the state.
            Ctx xt;
            xt.P = P;
            xt.M = mv;
            xt.N = aN;
            xt.dv = dv;
            xt.w = w;
            xt.vrole = w < 2 * NCJ;  // the waves that stage v (all at 64 columns)
            xt.qb = (const char *)args.q + trow * 32;
            xt.kb = (const char *)args.k + trow * 32;
            xt.vb = (const char *)args.v + trow * dv * 2;
            if (pre_part) {
                xt.keb = (const char *)args.ke + ((long)head * aM + pstart) * 32;
                xt.veb = (const char *)args.ve + ((long)head * aM + pstart) * dv * 2;
            } else if (own_walk) {
                xt.keb = xt.kb;
                xt.veb = xt.vb;
            } else if (nseg == 1) {
                xt.keb = (const char *)args.ke + ((long)head * aM + (aM - mv)) * 32;
                xt.veb = (const char *)args.ve + ((long)head * aM + (aM - mv)) * dv * 2;
            } else {
                xt.keb = (const char *)args.k + (long)head * args.N * 32;
                xt.veb = (const char *)args.v + (long)head * args.N * dv * 2;
            }
            const LoadOff lo = load_offsets<NCJ>(tid, w, dv, colb);
            __amdgpu_buffer_rsrc_t vr, qkr;
            chunk_srcs(xt, 0, vr, qkr);
            Staged tx = load_chunk(lo, vr, qkr);
            store_chunk<NCJ>(ring(P, L::SLOT), tx, tid, w);
            chunk_srcs(xt, 1, vr, qkr);
            tx = load_chunk(lo, vr, qkr);
            __syncthreads();                  // prologue
            for (int c = 0; c < P; ++c) {
                store_chunk<NCJ>(ring(c + 1 + P, L::SLOT), tx, tid, opaque(w));
                if (c + 2 <= P) {
                    chunk_srcs(xt, c + 2, vr, qkr);
                    tx = load_chunk(lo, vr, qkr);
                }
                __syncthreads();
            }
            __syncthreads();                  // the state copy after the prefix
        }
        for (int i = 0; i < NC; ++i) {
            Lane lw = ln;
            lw.t = opaque(ln.t);
            const __amdgpu_buffer_rsrc_t yr = chunk_rsrc(yb, i * CH, ylen, ybpt);
            token_chunk<NCJ, OutT>(ring(i, L::SLOT), (const _Float16 *)(smem + L::SB + (i & 1) * L::SBSZ),
                              smem + L::ZB + (i & 1) * ZBSZ, lw, yr, dv, zc, args.eps);
            zc += (float)min(CH, aN - i * CH);
            if (i + 1 < NC) __syncthreads();  // nothing is staged after the last chunk
        }
        return;
    }

    // ---------------- state waves ----------------
    WaveState<NCJ> st;
    {
        PrefillArgs a0 = args;  // folded: the initial state is in the prefix sum
        if (fold) a0.S0 = a0.z0 = nullptr;
        load_state<NCJ>(st, a0, ln, colb, sbase, zbase);
    }
    if (seeded) {
        st.z0 += (float)mv;
        add_partial<NCJ>(st, args, ln, trow, colb);
    }
    Ctx x;
    x.P = P;
    x.N = aN;
    x.M = mv;
    x.dv = dv;
    x.w = u;
    x.vrole = u < 2 * NCJ;  // the waves that stage v (all at 64 columns)
    x.qb = (const char *)args.q + trow * 32;
    x.kb = (const char *)args.k + trow * 32;
    x.vb = (const char *)args.v + trow * dv * 2;
    if (pre_part) {
        x.keb = (const char *)args.ke + ((long)head * aM + pstart) * 32;
        x.veb = (const char *)args.ve + ((long)head * aM + pstart) * dv * 2;
    } else if (own_walk) {
        x.keb = x.kb;
        x.veb = x.vb;
    } else if (nseg == 1) {
        x.keb = (const char *)args.ke + ((long)head * aM + (aM - mv)) * 32;
        x.veb = (const char *)args.ve + ((long)head * aM + (aM - mv)) * dv * 2;
    } else {
        x.keb = (const char *)args.k + (long)head * args.N * 32;
        x.veb = (const char *)args.v + (long)head * args.N * dv * 2;
    }
    const LoadOff lo = load_offsets<NCJ>(utid, u, dv, colb);

    // Causal chunks: one chunk of staged inputs in registers; chunk c + 2 is loaded
    // while chunk c is computed and stored into the ring at the start of the next
    // chunk.
    __amdgpu_buffer_rsrc_t vr, qkr;
    Staged nx;
    if (P == 0) {
        chunk_srcs(x, 0, vr, qkr);
        nx = load_chunk(lo, vr, qkr);
        store_chunk<NCJ>(ring(0, L::SLOT), nx, utid, u);
        chunk_srcs(x, 1, vr, qkr);
        nx = load_chunk(lo, vr, qkr);
        write_state<NCJ>(st, (_Float16 *)(smem + L::SB), ln);
        if (u == ZW) write_z(st.Z2, st.z1, smem + L::ZB, l);
    }
    __syncthreads();

    // prefix chunks (update only; the token waves stage them); chunk c (prefix
    // chunks first) sits in ring slot (c + P) & 1.  The state waves take over the
    // staging with causal chunk 1, loaded during the last prefix chunk.
    for (int c = 0; c < P; ++c) {
        Lane lw = ln;
        lw.w = opaque(ln.w);
        lw.tb = opaque(ln.tb);
        lw.nt = opaque(ln.nt);
        if (c == P - 1) {
            chunk_srcs(x, P + 1, vr, qkr);
            nx = load_chunk(lo, vr, qkr);
        }
        state_update<NCJ>(st, ring(c + P, L::SLOT), lw);
        st.z0 += (float)min(CH, mv - c * CH);
        __syncthreads();
    }
    if (P > 0) {
        write_state<NCJ>(st, (_Float16 *)(smem + L::SB), ln);
        if (u == ZW) write_z(st.Z2, st.z1, smem + L::ZB, l);
        __syncthreads();
    }
    for (int i = 0; i < NC; i += 2) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            const int ii = i + k2;
            if (ii >= NC) break;
            Lane lw = ln;
            lw.w = opaque(ln.w);
            lw.tb = opaque(ln.tb);
            lw.nt = opaque(ln.nt);
            store_chunk<NCJ>(ring(ii + 1, L::SLOT), nx, utid, lw.w);
            const int tl = (ii + 2) * CH;
            nx = load_chunk(lo, chunk_rsrc(x.vb, tl, x.vrole ? x.N : 0, dv * 2),
                            chunk_rsrc(pick<const char *>(lw.w < 4, x.qb, x.kb), tl, x.N, 32));
            state_update<NCJ>(st, ring(ii, L::SLOT), lw);
            st.z0 += (float)min(CH, aN - ii * CH);
            write_state<NCJ>(st, (_Float16 *)(smem + L::SB + ((ii + 1) & 1) * L::SBSZ), lw);
            if (lw.w == ZW) write_z(st.Z2, st.z1, smem + L::ZB + ((ii + 1) & 1) * ZBSZ, 16 * g + lr);
            // after the last chunk the final state is stored while the token waves
            // finish that chunk (they read LDS the state waves no longer write)
            if (ii + 1 < NC) __syncthreads();
        }
    }
    // The last prefetch (past the end: range-checked, no memory access) completes
    // here, before the first store, so that no wait lands between the stores (the
    // vector-memory counter also counts stores).  vmcnt(0) expcnt(7) lgkmcnt(15).
    __builtin_amdgcn_s_waitcnt(0x0F70);
    if (mode == kModePartial)
        store_partial<NCJ>(st, args, ln, trow, colb, pre_part ? 1 : 0);
    else if (last_seg)
        store_state<NCJ>(st, args, ln, colb, cb, sbase, zbase);
}

// Pass 2 of the chunk-parallel split: for each (head, column block) and partial
// float f, P_s = (prefix partials 0 .. m-1) + Delta_0 + ... + Delta_{s-1}, added
// in that order, replaces Delta_s in slot 0 of causal segment s, for s = 0 ..
// nseg - 1 (the last segment has no Delta).  The m JRT prefix partials sit in
// slot 1 (slot1 floats further) of causal segments 0 .. m-1.  Loads go in groups
// before the group's stores, so that they are in flight together.
__global__ __launch_bounds__(256) void scan_partials_kernel(PrefillArgs a, int ncb, int cw, int nseg, int seglen,
                                                            int nelem, int m, int slot1, int fold)
{
    const long t = (long)blockIdx.x * 256 + threadIdx.x;
    if (t >= (long)a.B * a.H * ncb * nelem) return;
    const int f = (int)(t % nelem);
    const long hc = t / nelem;
    const int cb = (int)(hc % ncb);
    const long head = hc / ncb;
    const int fpr = cw * (a.y_bf16 ? 2 : 4) / 4;
    const bool count = f == pidx_z0(cw);  // no partial holds it: zero, or z0's count when folded
    constexpr int G = 16;
    float acc = 0.f;
    if (fold && a.S0) {  // the initial state joins every prefix sum (pass 3 then reads no S0)
        const int ND = a.compact ? kDc : kD;
        const long sbase = head * ND * a.dv, zbase = head * ND;
        if (f < kPartialZ * cw)
            acc = init_S(a, sbase, f / (16 * cw), (f / cw) % 16, cb * cw + f % cw);
        else if (f < kPartialZ * cw + 256)
            acc = init_Z2(a, zbase, (f - kPartialZ * cw) / 16, (f - kPartialZ * cw) % 16);
        else if (!count)
            acc = init_z1(a, zbase, f - kPartialZ * cw - 256);
        else
            acc = a.z0[zbase];
    }
    for (int j0 = 0; j0 < m; j0 += G) {
        float d[G];
#pragma unroll
        for (int i = 0; i < G; ++i)
            d[i] = j0 + i < m && !count ? *partial_ptr(a, head * a.N + (long)(j0 + i) * seglen, cb * cw, fpr, f + slot1)
                                        : 0.f;
#pragma unroll
        for (int i = 0; i < G; ++i) acc += d[i];
    }
    for (int s0 = 0; s0 < nseg; s0 += G) {
        float d[G];
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const int sg = s0 + i;
            d[i] = sg < nseg - 1 && !count ? *partial_ptr(a, head * a.N + (long)sg * seglen, cb * cw, fpr, f) : 0.f;
        }
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const int sg = s0 + i;
            if (sg < nseg) *partial_ptr(a, head * a.N + (long)sg * seglen, cb * cw, fpr, f) = acc;
            acc += d[i];
        }
    }
}

// ncj: 16-column tiles per workgroup (dv / 16 / ncb); ncb: column blocks per head;
// nseg segments of seglen tokens (the last possibly shorter)
template <typename OutT>
hipError_t launch_ws_grid(const PrefillArgs &a, int ncj, int ncb, int nseg, int seglen, int mode, hipStream_t s,
                          int ncp = 0, int pseglen = 0)
{
    const dim3 grid((unsigned)((long)a.B * a.H * ncb * nseg));
    if (ncj == 4)
        hipLaunchKernelGGL((prefill_ws_kernel<4, OutT>), grid, dim3(NTHR_WS), 0, s, a, ncb, nseg, seglen, mode, ncp,
                           pseglen);
    else if (ncj == 2)
        hipLaunchKernelGGL((prefill_ws_kernel<2, OutT>), grid, dim3(NTHR_WS), 0, s, a, ncb, nseg, seglen, mode, ncp,
                           pseglen);
    else
        hipLaunchKernelGGL((prefill_ws_kernel<1, OutT>), grid, dim3(NTHR_WS), 0, s, a, ncb, nseg, seglen, mode, ncp,
                           pseglen);
    return hipGetLastError();
}

// Segments of whole chunks for a split into (at most) nseg parts, none empty.
void segments(int N, int nseg, int &seglen, int &nseg_eff)
{
    const int nch = (N + CH - 1) / CH;
    seglen = nseg > 1 ? (nch + nseg - 1) / nseg * CH : (N > 0 ? N : 1);
    nseg_eff = nseg > 1 ? (N + seglen - 1) / seglen : 1;
}

template <typename OutT>
hipError_t launch_ws(const PrefillArgs &a, int ncj, int ncb, int nseg, hipStream_t s)
{
    int seglen, nseg_eff;
    segments(a.N, nseg, seglen, nseg_eff);
    return launch_ws_grid<OutT>(a, ncj, ncb, nseg_eff, seglen, kModeWalk, s);
}

// The three launches of the chunk-parallel split: nseg causal segments of seglen
// tokens and m JRT prefix parts of pseglen tokens (m = 0 without a prefix).
template <typename OutT>
hipError_t launch_scan3(const PrefillArgs &a, int ncj, int ncb, int nseg, int seglen, int m, int pseglen,
                        int fold, hipStream_t s)
{
    PrefillArgs p1 = a;  // partial sums start from zero and write no state
    p1.S0 = nullptr;
    p1.z0 = nullptr;
    p1.S_out = nullptr;
    p1.z_out = nullptr;
    hipError_t e = launch_ws_grid<OutT>(p1, ncj, ncb, nseg - 1 + m, seglen, kModePartial, s, nseg - 1, pseglen);
    if (e != hipSuccess) return e;
    const int cw = 16 * ncj, nelem = partial_floats(cw), fpr = cw * (a.y_bf16 ? 2 : 4) / 4;
    const int slot1 = (nelem + fpr - 1) / fpr * fpr;
    const long threads = (long)a.B * a.H * ncb * nelem;
    hipLaunchKernelGGL(scan_partials_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, a, ncb, cw,
                       nseg, seglen, nelem, m, slot1, fold);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_ws_grid<OutT>(a, ncj, ncb, nseg, seglen, fold ? kModeSeededFold : kModeSeeded, s);
}

// A launch plan of the chunk-parallel split: ncb column blocks, nseg causal
// segments of seglen tokens, m JRT prefix parts of pseglen tokens.
struct Scan3Plan {
    int ncb, ncj, nseg, seglen, m, pseglen;
};

// The split for ncb column blocks per head if it pays (it needs y, with room in
// every segment for its partials); false leaves the call to the walk.
bool plan_scan3(const PrefillArgs &a, int ncb, Scan3Plan &p)
{
    if (!a.y) return false;
    const long heads = (long)a.B * a.H;
    const int nch = (a.N + CH - 1) / CH, ncj = a.dv / 16 / ncb;
    const int cw = 16 * ncj, fpr = cw * (a.y_bf16 ? 2 : 4) / 4;
    const int rows = (partial_floats(cw) + fpr - 1) / fpr;
    int ns = 1;
    while (ns < nch && heads * ncb * (ns * 2) <= 256) ns *= 2;
    for (; ns >= 3; ns /= 2) {
        int seglen, nseg;
        segments(a.N, ns, seglen, nseg);
        if (nseg < 3 || a.N - (nseg - 1) * seglen < rows) continue;
        int m = 0, pseglen = 0;
        long saved = (long)(nseg - 2) * seglen;  // the walk's longest prefix less the split's
        if (a.M > 0) {
            // JRT: the prefix is summed in parts whose partials sit in a second
            // slot of the first m causal segments' rows ([JRT] §2.8: the prefix
            // state is one sum over the prefix tokens)
            m = nseg - 1;
            pseglen = ((a.M + CH - 1) / CH + m - 1) / m * CH;
            saved = (long)a.M + a.N - max(seglen, pseglen) - seglen;
            if (seglen < 2 * rows) continue;
        }
        if (saved < kScanMinSaved) continue;
        p = Scan3Plan{ncb, ncj, nseg, seglen, m, pseglen};
        return true;
    }
    return false;
}

// Where the split with two column blocks per head applies, one block per head
// is faster if it halves every workgroup's tokens (twice the segments) and each
// segment still holds kScanWideMinSeg tokens: a 64-column chunk costs about 1.3
// times a 32-column one (measured 95 -> 81 us for one 16-head sequence of 32768
// tokens).  With 256- or 512-token segments the fixed costs per segment, and
// with the segment length held by the room the partials need half as many
// workgroups, made it up to 30% slower.
constexpr int kScanWideMinSeg = 1024;

bool try_scan3(const PrefillArgs &a, int ncb, int fold, hipStream_t s, hipError_t &err)
{
    Scan3Plan p;
    if (!plan_scan3(a, ncb, p)) return false;
    Scan3Plan wide;
    if (ncb == 2 && plan_scan3(a, 1, wide) && wide.seglen >= kScanWideMinSeg && 2 * wide.seglen <= p.seglen)
        p = wide;
    err = a.y_bf16 ? launch_scan3<uint16_t>(a, p.ncj, p.ncb, p.nseg, p.seglen, p.m, p.pseglen, fold, s)
                   : launch_scan3<float>(a, p.ncj, p.ncb, p.nseg, p.seglen, p.m, p.pseglen, fold, s);
    return true;
}

}  // namespace

hipError_t launch_prefill_sym(const PrefillArgs &a, int col_split_allowed, hipStream_t s)
{
    const bool in_place = (a.S_out && a.S_out == a.S0) || (a.z_out && a.z_out == a.z0);
    const long heads = (long)a.B * a.H;
    const int nch = (a.N + CH - 1) / CH;
    // With 128 heads or fewer, 64 or 32 value columns go to two workgroups per
    // head (each walks the whole sequence: no prefix to recompute; measured 31.9
    // against 33.8 us for two sequence segments at 128 heads, N = 2048,
    // d_v = 64).  A state updated in place keeps its z in one column block,
    // except in the folded split, where only the last segment reads the state.
    const int ncb_free = a.dv >= 32 && heads * 2 <= 256 ? 2 : 1;
    const int ncb = col_split_allowed ? ncb_free : 1;
    // Then the sequence is split in segments (powers of two) while the workgroups
    // still fit one per compute unit: chunk-parallel when that saves enough (the
    // initial state folded into the prefix sums when it is updated in place),
    // else by walking the earlier tokens (not for a JRT prefix, whose walk is the
    // segment's own, nor in place, where a segment would read S0 after the last
    // one has written S_out).
    hipError_t err = hipSuccess;
    if (!a.y && a.M == 0) {
        // state only: one update-only walk per head and column block (a split
        // would only repeat the walk of earlier tokens)
        const int ncj = a.dv / 16 / ncb, seglen = a.N > 0 ? a.N : 1;
        return a.y_bf16 ? launch_ws_grid<uint16_t>(a, ncj, ncb, 1, seglen, kModeStateOnly, s)
                        : launch_ws_grid<float>(a, ncj, ncb, 1, seglen, kModeStateOnly, s);
    }
    if (try_scan3(a, in_place ? ncb_free : ncb, in_place ? 1 : 0, s, err)) return err;
    int nseg = 1;
    if (!in_place && a.M == 0)
        while (nseg < nch && heads * ncb * (nseg * 2) <= 256) nseg *= 2;
    const int ncj = a.dv / 16 / ncb;
    return a.y_bf16 ? launch_ws<uint16_t>(a, ncj, ncb, nseg, s) : launch_ws<float>(a, ncj, ncb, nseg, s);
}

}  // namespace bla
