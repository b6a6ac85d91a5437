// Sliding-window softmax attention (SWA): prefill on gfx950 matrix cores and
// the fused decode step on a ring KV cache.
//
// "Simple linear attention language models balance the recall-throughput
// tradeoff" notes, §2.4: SWA is standard softmax attention over the keys
// j in [i - w + 1, i] only, keeping the w most recent keys/values per head;
// the pages pick w in 64..128 to match matrix-core tile sizes.  §2.5: decoding
// fuses the dot products, the softmax and the weighted sum over the window.
// Scores are q.k / sqrt(d) (standard attention); no rotary embedding.
//
// Prefill (w <= 64 and w > 128; 64 < w <= 128 uses the ring kernel further
// down): one workgroup of 8 wavefronts per (batch, head) and tile of 128
// queries; the keys of the tile's windows (at most 128 + w - 1, rounded out to
// 32-key slabs) are staged in LDS -- keys as the bf16 they arrive in, values
// converted to fp16 in token-slot order (one 16-byte read per 32-key operand).
// Wave wv owns queries 16 wv .. 16 wv + 15: score tiles K Q^T on the matrix
// cores (16 keys x 16 queries, two bf16 16x16x32 products over d = 64, exact
// products in fp32), the masked softmax in fp32 with the 1/sqrt(64) scale
// folded into the exp2 argument (max, exp2, row sums of the fp16 weights),
// then y^T += V^T P^T on the fp16 matrix cores and one divide.
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
typedef __bf16 b8 __attribute__((ext_vector_type(8)));

constexpr int kQueryTile = 128;  // queries per workgroup (one wavefront per 16)
constexpr int DK = 64;       // key / query width
constexpr int DV = 64;       // value width
constexpr uint32_t kRsrcWord3 = 0x00020000u;

// LDS layouts, in 16-byte units: key rows of 144 bytes (64 bf16 + 16 bytes of
// padding that staggers consecutive rows across the bank groups) and value rows
// (one per value column) of the staged keys plus 8 halves.  A 128-query tile
// then stages 52 KB (w <= 64: three workgroups per compute unit) or 69 KB
// (w <= 128: two).  Swizzled unpadded rows were measured slower here.
__device__ __forceinline__ int k_unit(int j, int u) { return 9 * j + u; }
__device__ __forceinline__ int v_unit(int c, int u, int vst) { return c * (vst / 8) + u; }

__device__ __forceinline__ f4 mfma32(h8 a, h8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mfma32_bf16(u4 a, u4 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, a), __builtin_bit_cast(b8, b), c,
                                                    0, 0, 0);
}
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, h2));
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, bytes, kRsrcWord3);
}
// token order inside a 32-key slab as seen by the 16x16x32 operands (lane group
// g holds keys {4g..4g+3, 16+4g..16+4g+3}); values are stored in this order
__device__ __forceinline__ int slot_of(int j) {
    return (j & ~31) + ((j >> 2) & 3) * 8 + ((j >> 4) & 1) * 4 + (j & 3);
}
// reductions over the four 16-lane rows of a wavefront (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float max_rows4(float x) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float s = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ float sum_rows4(float x) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float s = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

template <int WMAX, int QT>
struct SwaLay {
    static_assert(QT % 32 == 0 && WMAX % 32 == 0, "tiles and windows in whole 32-key slabs");
    // staged keys: a tile starts on a slab, so its windows begin at most
    // ceil((w - 1) / 32) slabs earlier: QT + WMAX keys in whole slabs
    static constexpr int NK = QT + WMAX;
    static constexpr int VST = NK + 8;             // halves per value row
    static constexpr int K = 0;                    // [NK][72] bf16 (64 used)
    static constexpr int V = K + NK * 144;         // [DV][VST] fp16, slot order
    static constexpr int TOTAL = V + DV * VST * 2;
    static_assert(TOTAL >= (QT / 16) * 16 * 72 * 4, "the y tiles reuse the staging area");
    // score tiles per wave: 16 queries need w + 15 keys, and the slab-aligned
    // first tile starts at most 17 keys before the window: WMAX / 16 + 2 tiles
    static constexpr int NT = WMAX / 16 + 2;
};

template <int WMAX, int QT, typename OutT>
__global__ __launch_bounds__(4 * QT) void swa_prefill_kernel(SwaArgs a)
{
    constexpr int NTH = 4 * QT;  // one wavefront per 16 queries
    using L = SwaLay<WMAX, QT>;
    __shared__ __attribute__((aligned(16))) unsigned char sm[L::TOTAL];
    const int tid = threadIdx.x, l = tid & 63, g = l >> 4, lr = l & 15;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int N = a.N, w = a.window;
    const int ntile = (N + QT - 1) / QT;
    const int heads = a.B * a.H;
    // XCD-aware: consecutive query tiles of one head (overlapping windows) share an XCD
    int head, qt;
    if ((heads & 7) == 0) {
        const int xcd = blockIdx.x & 7, u = blockIdx.x >> 3;
        head = (u / ntile) * 8 + xcd;
        qt = u % ntile;
    } else {
        head = blockIdx.x / ntile;
        qt = blockIdx.x % ntile;
    }
    const int q0 = qt * QT;
    const int kt0 = max(0, q0 - w + 1) & ~31;            // first staged key
    const int kend = min(N, q0 + QT);                     // one past the last key any query here sees
    const int nks = ((kend - kt0 + 31) >> 5) << 5;        // staged keys, whole slabs (<= L::NK)
    const char *qb = (const char *)a.q + (long)head * N * DK * 2;
    const char *kb = (const char *)a.k + ((long)head * N + kt0) * DK * 2;
    const char *vb = (const char *)a.v + ((long)head * N + kt0) * DV * 2;
    const __amdgpu_buffer_rsrc_t kr = rsrc(kb, (kend - kt0) * DK * 2);  // keys past kend read 0
    const __amdgpu_buffer_rsrc_t vr = rsrc(vb, (kend - kt0) * DV * 2);

    // ---- stage K rows (bf16) and V (fp16) in slot order ----
    u4 *Ks = (u4 *)(sm + L::K);  // 16-byte units of bf16 keys
    _Float16 *Vs = (_Float16 *)(sm + L::V);
    // every load of the tile is issued before the first LDS store; loads past the
    // staged keys read zeros (buffer range check) and are not stored
    {
        constexpr int KIT = (L::NK * 8 + NTH - 1) / NTH;            // 16 bytes of one key per item
        constexpr int VIT = ((L::NK >> 2) * (DV / 4) + NTH - 1) / NTH;  // 4 keys x 4 columns per item
        u4 kx[KIT];
        u2 vx[VIT][4];
#pragma unroll
        for (int it = 0; it < KIT; ++it) {
            const int u = tid + it * NTH, j = u >> 3, part = u & 7;
            kx[it] = __builtin_amdgcn_raw_buffer_load_b128(kr, j * DK * 2 + 16 * part, 0, 0);
        }
#pragma unroll
        for (int it = 0; it < VIT; ++it) {
            const int u = tid + it * NTH, jq = u >> 4, cq = u & 15;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                vx[it][r] = __builtin_amdgcn_raw_buffer_load_b64(vr, ((4 * jq + r) * DV + 4 * cq) * 2, 0, 0);
        }
#pragma unroll
        for (int it = 0; it < KIT; ++it) {
            const int u = tid + it * NTH, j = u >> 3, part = u & 7;
            if (u < nks * 8) Ks[k_unit(j, part)] = kx[it];
        }
#pragma unroll
        for (int it = 0; it < VIT; ++it) {
            const int u = tid + it * NTH, jq = u >> 4, cq = u & 15;
            if (u < (nks >> 2) * (DV / 4)) {
                const int s0 = slot_of(4 * jq);
#pragma unroll
                for (int e = 0; e < 4; ++e) {  // value column 4 cq + e of keys 4 jq .. 4 jq + 3
                    float f[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const uint32_t wd = e < 2 ? vx[it][r].x : vx[it][r].y;
                        f[r] = (e & 1) ? bf16_hi(wd) : bf16_lo(wd);
                    }
                    *(u2 *)(Vs + 8 * v_unit(4 * cq + e, s0 >> 3, L::VST) + (s0 & 7)) =
                        (u2){pack2(f[0], f[1]), pack2(f[2], f[3])};
                }
            }
        }
    }
    // ---- this lane's query operand (bf16 as stored): features 8g..8g+7 and 32+8g.. (i = q0 + 16 wv + lr) ----
    const int qi = q0 + 16 * wv + lr;
    const __amdgpu_buffer_rsrc_t qr = rsrc(qb, N * DK * 2);
    u4 qop[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
        qop[hh] = __builtin_amdgcn_raw_buffer_load_b128(qr, qi * DK * 2 + 64 * hh + 16 * g, 0, 0);
    __syncthreads();

    // ---- scores of this wave's 16 queries against its key tiles ----
    const int qw0 = q0 + 16 * wv;                                   // first query of the wave
    const int tlo = (max(kt0, qw0 - w + 1) - kt0) >> 5 << 1;       // first 16-key tile (slab aligned)
    const int thi = min((qw0 + 15 - kt0) >> 4, (nks >> 4) - 1);    // last tile
    const int ntl = __builtin_amdgcn_readfirstlane(thi - tlo + 1);  // <= L::NT
    const float c2 = 0.125f * 1.4426950408889634f;                  // log2(e) / sqrt(64)
    f4 sc[L::NT];
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < L::NT; ++tt) {
        sc[tt] = (f4){-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        if (tt >= ntl) continue;
        const int kt = tlo + tt;
        const int kj = 16 * kt + lr;  // staged key row this lane supplies
        f4 s = mfma32_bf16(Ks[k_unit(kj, g)], qop[0], (f4){0.f, 0.f, 0.f, 0.f});
        s = mfma32_bf16(Ks[k_unit(kj, 4 + g)], qop[1], s);  // s = q.k (unscaled)
        // the window / causal / length mask, only on tiles that cross a boundary for
        // some query of the wave (a uniform test: interior tiles skip it)
        const int jlo = kt0 + 16 * kt;
        const bool interior = jlo + 15 <= qw0 && jlo > qw0 + 15 - w && jlo + 15 < N;
        if (!interior) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = jlo + 4 * g + r;  // key of this entry; query is qi
                const bool ok = j <= qi && j > qi - w && j < N;
                s[r] = ok ? s[r] : -INFINITY;
            }
        }
        mx = fmaxf(mx, fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
        sc[tt] = s;
    }
    mx = max_rows4(mx);
    if (mx == -INFINITY) mx = 0.f;  // query rows past the sequence end (not stored)
    const float mc = mx * c2;
    h4 pw[L::NT];
    float rs = 0.f;
    const h2 one2 = (h2){1, 1};
#pragma unroll
    for (int tt = 0; tt < L::NT; ++tt) {
        float e[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) e[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[tt][r], c2, -mc));
        pw[tt] = __builtin_convertvector((f4){e[0], e[1], e[2], e[3]}, h4);
        rs = __builtin_amdgcn_fdot2((h2){pw[tt][0], pw[tt][1]}, one2, rs, false);
        rs = __builtin_amdgcn_fdot2((h2){pw[tt][2], pw[tt][3]}, one2, rs, false);
    }
    rs = sum_rows4(rs);

    // ---- y^T += V^T P^T, one 32-key slab (two score tiles) per product ----
    f4 yacc[DV / 16];
#pragma unroll
    for (int j = 0; j < DV / 16; ++j) yacc[j] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tt = 0; tt < L::NT; tt += 2) {
        if (tt >= ntl) continue;
        const h4 p1 = tt + 1 < L::NT ? pw[tt + 1] : (h4){0, 0, 0, 0};
        const h8 B = (h8){pw[tt][0], pw[tt][1], pw[tt][2], pw[tt][3], p1[0], p1[1], p1[2], p1[3]};
        const int slab0 = 16 * (tlo + tt);  // first key (relative to kt0) of this slab
#pragma unroll
        for (int j = 0; j < DV / 16; ++j)
            yacc[j] = mfma32(*(const h8 *)(Vs + 8 * v_unit(16 * j + lr, (slab0 >> 3) + g, L::VST)), B, yacc[j]);
    }

    // ---- normalise and store ----
    // lane (lr, g) holds y[qi][16 j + 4 g .. + 3].  Stored as is, one instruction would
    // write 64-byte pieces of 16 rows; instead, once every wave is done with the staged
    // keys and values, each wave passes its 16 x 64 tile through LDS (rows of 72 floats)
    // and reads it back row-major, so that one store instruction writes 4 whole rows.
    if (a.y) {
        const float inv = 1.f / rs;
        __syncthreads();
        float *yt = (float *)sm + wv * (16 * 72);
#pragma unroll
        for (int j = 0; j < DV / 16; ++j) *(f4 *)(yt + lr * 72 + 16 * j + 4 * g) = yacc[j] * inv;
        __syncthreads();
        const int c = 4 * (l & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = (l >> 4) + 4 * i, qr = q0 + 16 * wv + r;
            const f4 yv = *(const f4 *)(yt + r * 72 + c);
            if (qr < N) {
                const long o = ((long)head * N + qr) * DV + c;
                if constexpr (sizeof(OutT) == 4) {
                    *(f4 *)((float *)a.y + o) = yv;
                } else {
                    *(u2 *)((uint16_t *)a.y + o) =
                        (u2){f32x2_to_bf16x2(yv[0], yv[1]), f32x2_to_bf16x2(yv[2], yv[3])};
                }
            }
        }
    }
    // ---- ring cache of the last w tokens (token p in slot p mod w) ----
    if (a.k_cache) {
        for (int u = tid; u < QT * (DK / 8); u += NTH) {
            const int p = q0 + u / (DK / 8), part = u % (DK / 8);
            if (p < N && p >= N - w) {
                const long src = ((long)head * N + p) * DK + 8 * part;
                const long dst = ((long)head * w + p % w) * DK + 8 * part;
                *(u4 *)((uint16_t *)a.k_cache + dst) = *(const u4 *)((const uint16_t *)a.k + src);
                *(u4 *)((uint16_t *)a.v_cache + dst) = *(const u4 *)((const uint16_t *)a.v + src);
            }
        }
    }
}

template <int WMAX, typename OutT>
hipError_t launch_swa_w(const SwaArgs &a, hipStream_t s)
{
    constexpr int QT = kQueryTile;
    const long tiles = (long)a.B * a.H * ((a.N + QT - 1) / QT);
    hipLaunchKernelGGL((swa_prefill_kernel<WMAX, QT, OutT>), dim3((unsigned)tiles), dim3(4 * QT), 0, s,
                       a);
    return hipGetLastError();
}

// ---------------- ring prefill (window <= 128) ----------------
// One workgroup of 8 wavefronts walks a run of consecutive 128-query tiles of one
// head.  Every window reaches back at most 127 keys, so tile t reads key blocks
// t - 1 and t (128 keys each) only; they sit in an LDS ring of two slots (block b
// in slot b & 1).  While tile t is computed, block t + 1's keys and values and
// tile t + 1's queries are already loading into registers; they are written over
// block t - 1 once every wave is done with it.  Within a run each block is
// staged once; a run also stages the block before its first tile.
//
// Score tiles start on 16-key boundaries: the 16 queries of a wave see
// w + 15 keys, so at most w / 16 + 1 tiles.  Values are stored transposed in
// natural key order; the product y^T += V^T P^T pairs consecutive score tiles
// into one 16x16x32 operand (two 8-byte reads per lane) and takes a last
// unpaired tile through the 16x16x16 product.  At w = 128 every wave whose
// window lies inside the sequence takes a path with the tile count and the two
// masked tiles fixed at compile time (wave_attend<NT, true>).
struct RingLay {
    static constexpr int BK = 128;             // keys per block = queries per tile
    static constexpr int VST = 2 * BK + 8;     // halves per value row (both slots)
    static constexpr int K = 0;                // [2 * BK][72] bf16 (64 used), 144-byte rows
    static constexpr int V = K + 2 * BK * 144; // [DV][VST] fp16: slot s holds keys at s * BK
    static constexpr int TOTAL = V + DV * VST * 2;
};
constexpr int kRingThreads = 512;

__device__ __forceinline__ f4 mfma16(h4 a, h4 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
// ring position of key j (absolute index)
__device__ __forceinline__ int ring_key(int j) { return (j & RingLay::BK) + (j & (RingLay::BK - 1)); }

// registers of one 128-key block in flight: 2 x 16 bytes of key rows and, for 4
// keys x 4 value columns, four 8-byte value pieces per thread
struct BlockRegs {
    u4 k[2];
    u2 v[4];
};
__device__ __forceinline__ void load_block_k(BlockRegs &r, __amdgpu_buffer_rsrc_t kr, int blk, int tid) {
    const int j0 = blk * RingLay::BK;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int u = tid + it * kRingThreads, j = u >> 3, part = u & 7;
        r.k[it] = __builtin_amdgcn_raw_buffer_load_b128(kr, (j0 + j) * DK * 2 + 16 * part, 0, 0);
    }
}
__device__ __forceinline__ void load_block_v(BlockRegs &r, __amdgpu_buffer_rsrc_t vr, int blk, int tid) {
    const int j0 = blk * RingLay::BK, jq = tid >> 4, cq = tid & 15;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        r.v[q] = __builtin_amdgcn_raw_buffer_load_b64(vr, ((j0 + 4 * jq + q) * DV + 4 * cq) * 2, 0, 0);
}
__device__ __forceinline__ void load_block(BlockRegs &r, __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                           int blk, int tid) {
    load_block_k(r, kr, blk, tid);
    load_block_v(r, vr, blk, tid);
}
__device__ __forceinline__ void store_block(const BlockRegs &r, unsigned char *sm, int blk, int tid) {
    u4 *Ks = (u4 *)(sm + RingLay::K);
    _Float16 *Vs = (_Float16 *)(sm + RingLay::V);
    const int row0 = (blk & 1) * RingLay::BK;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int u = tid + it * kRingThreads, j = u >> 3, part = u & 7;
        Ks[9 * (row0 + j) + part] = r.k[it];
    }
    const int jq = tid >> 4, cq = tid & 15;
#pragma unroll
    for (int e = 0; e < 4; ++e) {  // value column 4 cq + e of keys 4 jq .. 4 jq + 3
        float f[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t wd = e < 2 ? r.v[q].x : r.v[q].y;
            f[q] = (e & 1) ? bf16_hi(wd) : bf16_lo(wd);
        }
        *(u2 *)(Vs + (4 * cq + e) * RingLay::VST + row0 + 4 * jq) = (u2){pack2(f[0], f[1]), pack2(f[2], f[3])};
    }
}

// One wave's 16 queries (qw0 .. qw0 + 15, this lane's query qw0 + lr) against
// the key tiles tlo .. tlo + ntl - 1 in the ring: scores K Q^T (16 keys x 16
// queries per tile, bf16 products), the masked softmax in fp32 (max, exp2 with the
// 1/sqrt(64) scale folded in, fp16 weights), y^T = V^T P^T into yacc; returns the
// row sum of the fp16 weights for query lr (a product with an all-ones operand).
// FULL: ntl = NT, every key < N, only tile 0 (window start) and tile NT - 1 (the
// diagonal) partly masked -- for w a multiple of 16 that is 4 g + r > lr and its
// complement.
template <int NT, bool FULL>
__device__ __forceinline__ float wave_attend(const u4 *Ks, const _Float16 *Vs, const u4 (&qop)[2], int qw0,
                                             int tlo, int ntl, int w, int N, int g, int lr, f4 (&yacc)[DV / 16])
{
    const float c2 = 0.125f * 1.4426950408889634f;  // log2(e) / sqrt(64)
    const int qi = qw0 + lr;
    f4 sc[NT];
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
        if (!FULL) {
            sc[tt] = (f4){-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            if (tt >= ntl) continue;
        }
        const int jlo = 16 * (tlo + tt);
        const int row = ring_key(jlo + lr);
        f4 s = mfma32_bf16(Ks[9 * row + g], qop[0], (f4){0.f, 0.f, 0.f, 0.f});
        s = mfma32_bf16(Ks[9 * row + 4 + g], qop[1], s);  // s = q.k (unscaled)
        if (FULL) {
            if (tt == 0 || tt == NT - 1) {
#pragma unroll
                for (int r = 0; r < 4; ++r) s[r] = ((4 * g + r > lr) == (tt == 0)) ? s[r] : -INFINITY;
            }
        } else {
            const bool interior = jlo + 15 <= qw0 && jlo > qw0 + 15 - w && jlo + 15 < N;
            if (!interior) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = jlo + 4 * g + r;  // key of this entry; query is qi
                    const bool ok = j <= qi && j > qi - w && j < N;
                    s[r] = ok ? s[r] : -INFINITY;
                }
            }
        }
        mx = __builtin_elementwise_maximum(
            mx, __builtin_elementwise_maximum(__builtin_elementwise_maximum(s[0], s[1]),
                                              __builtin_elementwise_maximum(s[2], s[3])));
        sc[tt] = s;
    }
    mx = max_rows4(mx);
    if (mx == -INFINITY) mx = 0.f;  // query rows past the sequence end (not stored)
    const float mc = mx * c2;
    h4 pw[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
        float e[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) e[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[tt][r], c2, -mc));
        pw[tt] = __builtin_convertvector((f4){e[0], e[1], e[2], e[3]}, h4);
    }
    // row sums of the fp16 weights: in the generic case on the vector ALU (fewer
    // registers), in the full case as a product with ones next to y's
    float rs = 0.f;
    if (!FULL) {
        const h2 one2 = (h2){1, 1};
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            rs = __builtin_amdgcn_fdot2((h2){pw[tt][0], pw[tt][1]}, one2, rs, false);
            rs = __builtin_amdgcn_fdot2((h2){pw[tt][2], pw[tt][3]}, one2, rs, false);
        }
        rs = sum_rows4(rs);
    }
    // y^T += V^T P^T over pairs of score tiles (one 16x16x32 product), a last
    // unpaired tile through the 16x16x16 product
    const h8 ones8 = (h8){1, 1, 1, 1, 1, 1, 1, 1};
    const h4 ones4 = (h4){1, 1, 1, 1};
    f4 rsum = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < DV / 16; ++jj) yacc[jj] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tt = 0; tt < NT; tt += 2) {
        if (!FULL && tt >= ntl) continue;
        const int ka = ring_key(16 * (tlo + tt) + 4 * g);
        if (tt + 1 < NT && (FULL || tt + 1 < ntl)) {
            const int kb = ring_key(16 * (tlo + tt + 1) + 4 * g);
            const h8 B = (h8){pw[tt][0], pw[tt][1], pw[tt][2], pw[tt][3],
                              pw[tt + 1][0], pw[tt + 1][1], pw[tt + 1][2], pw[tt + 1][3]};
#pragma unroll
            for (int jj = 0; jj < DV / 16; ++jj) {
                const _Float16 *vrow = Vs + (16 * jj + lr) * RingLay::VST;
                const h4 lo = *(const h4 *)(vrow + ka), hi = *(const h4 *)(vrow + kb);
                const h8 A = (h8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                yacc[jj] = mfma32(A, B, yacc[jj]);
            }
            if (FULL) rsum = mfma32(ones8, B, rsum);
        } else {
#pragma unroll
            for (int jj = 0; jj < DV / 16; ++jj)
                yacc[jj] = mfma16(*(const h4 *)(Vs + (16 * jj + lr) * RingLay::VST + ka), pw[tt], yacc[jj]);
            if (FULL) rsum = mfma16(ones4, pw[tt], rsum);
        }
    }
    return FULL ? rsum[0] : rs;
}

template <typename OutT>
__device__ __forceinline__ void store_y4(__amdgpu_buffer_rsrc_t yr, uint32_t off, f4 v) {
    if constexpr (sizeof(OutT) == 4)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), yr, off, 0, 0);
    else
        __builtin_amdgcn_raw_buffer_store_b64((u2){f32x2_to_bf16x2(v[0], v[1]), f32x2_to_bf16x2(v[2], v[3])}, yr,
                                              off, 0, 0);
}

template <int WMAX, typename OutT>
__global__ __launch_bounds__(kRingThreads) __attribute__((amdgpu_waves_per_eu(4)))
void swa_ring_kernel(SwaArgs a, int nseg, int seg_tiles)
{
    constexpr int NT = WMAX / 16 + 1;  // score tiles per wave
    __shared__ __attribute__((aligned(16))) unsigned char sm[RingLay::TOTAL];
    const int tid = threadIdx.x, l = tid & 63, g = l >> 4, lr = l & 15;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int N = a.N, w = a.window;
    const int head = blockIdx.x / nseg, seg = blockIdx.x % nseg;
    const int ntile = (N + RingLay::BK - 1) / RingLay::BK;
    const int t0 = seg * seg_tiles, t1 = min(ntile, t0 + seg_tiles);
    const long hoff = (long)head * N;
    const __amdgpu_buffer_rsrc_t qr = rsrc((const char *)a.q + hoff * DK * 2, N * DK * 2);
    const __amdgpu_buffer_rsrc_t kr = rsrc((const char *)a.k + hoff * DK * 2, N * DK * 2);
    const __amdgpu_buffer_rsrc_t vr = rsrc((const char *)a.v + hoff * DV * 2, N * DV * 2);
    const u4 *Ks = (const u4 *)(sm + RingLay::K);
    const _Float16 *Vs = (const _Float16 *)(sm + RingLay::V);

    // this lane's query operand for tile t (bf16 as stored; rows past N read 0)
    auto load_q = [&](u4 *qo, int t) {
        const int qi = t * RingLay::BK + 16 * wv + lr;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
            qo[hh] = __builtin_amdgcn_raw_buffer_load_b128(qr, qi * DK * 2 + 64 * hh + 16 * g, 0, 0);
    };
    u4 qop[2];
    {
        // the queries are loaded first: once the blocks are stored they are in too,
        // and nothing the loop waits for is still pending from here
        load_q(qop, t0);
        BlockRegs b0, b1;
        if (t0 > 0) load_block(b0, kr, vr, t0 - 1, tid);
        load_block(b1, kr, vr, t0, tid);
        if (t0 > 0) store_block(b0, sm, t0 - 1, tid);
        store_block(b1, sm, t0, tid);
        __syncthreads();
    }
    // y rows of this head; stores to rows past N (or with y absent) are dropped by
    // the range check, so the stores need no branch
    constexpr int YB = sizeof(OutT);
    const __amdgpu_buffer_rsrc_t yr = rsrc(a.y ? (const char *)a.y + hoff * DV * YB : nullptr, a.y ? N * DV * YB : 0);
    const bool lo = lr < 8;
    const int cb = (lo ? 0 : 16) + 4 * g;  // first column this lane stores (plus 32 hh)
    for (int t = t0; t < t1; ++t) {
        // block t + 1 and tile t + 1's queries, in flight while tile t is computed
        const bool pre = t + 1 < t1;
        BlockRegs nb;
        u4 qn[2];
        if (pre) {
            load_block(nb, kr, vr, t + 1, tid);
            load_q(qn, t + 1);
        }
        const int qw0 = t * RingLay::BK + 16 * wv;  // first query of the wave
        const int rlo = qw0 + (lr & 7), rhi = rlo + 8;  // the rows this lane stores
        {
            f4 yacc[DV / 16];
            float rs;
            // waves whose windows are whole and inside the sequence (all but the first
            // w / 128 tiles and the last one) at w = WMAX: NT tiles, the first and last
            // masked by a fixed per-lane pattern
            if (w == WMAX && qw0 >= w - 1 && qw0 + 15 < N)
                rs = wave_attend<NT, true>(Ks, Vs, qop, qw0, (qw0 - w + 1) >> 4, NT, w, N, g, lr, yacc);
            else {
                const int tlo = max(0, qw0 - w + 1) >> 4;  // first 16-key tile
                const int ntl = __builtin_amdgcn_readfirstlane((min(qw0 + 15, N - 1) >> 4) - tlo + 1);
                rs = wave_attend<NT, false>(Ks, Vs, qop, qw0, tlo, ntl, w, N, g, lr, yacc);
            }
            // lane (lr, g) holds y[qi][16 jj + 4 g .. + 3].  Stored as is, one store
            // instruction would write 64-byte pieces of 16 rows.  Lanes lr and lr ^ 8
            // swap half of the registers instead (a DPP rotate by 8 within each 16-lane
            // row), so that each instruction writes whole 32-column pieces of 8 rows.
            const float inv = 1.f / rs;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const f4 y0 = yacc[2 * hh] * inv, y1 = yacc[2 * hh + 1] * inv;
                const f4 send = lo ? y1 : y0;
                f4 recv;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    recv[r] = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(send[r]), 0x128, 0xf, 0xf, false));
                store_y4<OutT>(yr, (uint32_t)(rlo * DV + 32 * hh + cb) * YB, lo ? y0 : recv);
                store_y4<OutT>(yr, (uint32_t)(rhi * DV + 32 * hh + cb) * YB, lo ? recv : y1);
            }
        }
        // ring cache of the last w tokens (token p in slot p mod w)
        if (a.k_cache) {
            for (int u = tid; u < RingLay::BK * (DK / 8); u += kRingThreads) {
                const int p = t * RingLay::BK + u / (DK / 8), part = u % (DK / 8);
                if (p < N && p >= N - w) {
                    const long src = (hoff + p) * DK + 8 * part;
                    const long dst = ((long)head * w + p % w) * DK + 8 * part;
                    *(u4 *)((uint16_t *)a.k_cache + dst) = *(const u4 *)((const uint16_t *)a.k + src);
                    *(u4 *)((uint16_t *)a.v_cache + dst) = *(const u4 *)((const uint16_t *)a.v + src);
                }
            }
        }
        __syncthreads();  // every wave is done with block t - 1
        if (pre) {
            store_block(nb, sm, t + 1, tid);
            qop[0] = qn[0];
            qop[1] = qn[1];
        }
        __syncthreads();
    }
}

// runs of two tiles per workgroup, numbered head-major: the workgroups in flight
// then sweep a few heads' rows together.  Measured at B = H = 16, N = 32768,
// w = 128 against runs of 1, 3, 4, 8 ... 128 tiles and against an XCD-aware
// numbering, two tiles in this order was the fastest (longer runs keep fewer
// bytes in flight per workgroup than a new workgroup's first loads do).
constexpr int kRunTiles = 2;

template <int WMAX, typename OutT>
hipError_t launch_swa_ring(const SwaArgs &a, hipStream_t s)
{
    const long heads = (long)a.B * a.H;
    const int ntile = (a.N + RingLay::BK - 1) / RingLay::BK;
    const int seg_tiles = std::min(ntile, kRunTiles);
    const int nseg = (ntile + seg_tiles - 1) / seg_tiles;
    hipLaunchKernelGGL((swa_ring_kernel<WMAX, OutT>), dim3((unsigned)(heads * nseg)), dim3(kRingThreads), 0, s,
                       a, nseg, seg_tiles);
    return hipGetLastError();
}

// w <= 64: one workgroup per tile (three resident per compute unit) measured
// slightly ahead of the ring; 64 < w <= 128: the ring kernel, whose fixed tile
// count and masks cut the arithmetic that bounds the per-tile kernel there
template <typename OutT>
hipError_t launch_swa_t(const SwaArgs &a, hipStream_t s)
{
    if (a.window <= 64) return launch_swa_w<64, OutT>(a, s);
    if (a.window <= 128) return launch_swa_ring<128, OutT>(a, s);
    return launch_swa_w<256, OutT>(a, s);
}

// ---------------- decode ----------------
// One workgroup of 256 threads per (batch, head).  Every cache load of the step
// is issued first, before any arithmetic: TPS = 1, 2 or 4 threads per cache
// slot (window <= 256, 128, 64) read their share of the slot's key row with
// 16-byte loads, and thread (column quad cq, slot group sg) reads 4 value
// columns of slots sg, sg + 16, ... (8- or 16-byte loads).  The slot that the
// new token overwrites is never read from the cache: its key and value come
// from LDS.  The softmax is reduced through wavefront shuffles and LDS; each
// thread then accumulates its value columns and the 16 partial sums per column
// are reduced through LDS.  The new key/value is written into its slot last.
template <typename InT>
__device__ __forceinline__ float ld1(const void *p, long i) {
    if constexpr (sizeof(InT) == 2) return bf16_to_f32(((const uint16_t *)p)[i]);
    else return ((const float *)p)[i];
}
template <int Bytes> struct VRawT;             // 4 value columns as loaded
template <> struct VRawT<2> { typedef u2 T; };
template <> struct VRawT<4> { typedef u4 T; };
__device__ __forceinline__ f4 unpack4(u2 r) {
    return (f4){bf16_lo(r.x), bf16_hi(r.x), bf16_lo(r.y), bf16_hi(r.y)};
}
__device__ __forceinline__ f4 unpack4(u4 r) { return __builtin_bit_cast(f4, r); }

// fp32 caches at 64 < window <= 128 (two threads per slot): left to itself the
// compiler spends 230 registers here (one wave per SIMD); a floor of four waves
// per SIMD gives 96 registers without spills.  Every other instance keeps its
// own allocation.
template <typename InT, int TPS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(sizeof(InT) == 4 && TPS == 2 ? 4 : 1)))
void swa_decode_kernel(SwaArgs a)
{
    constexpr int FPT = DK / TPS;                    // key features per thread
    constexpr int KU = FPT * (int)sizeof(InT) / 16;  // 16-byte key loads per thread
    constexpr int NS = 16 / TPS;                     // value slots per thread ((256 / TPS) / 16)
    typedef typename VRawT<sizeof(InT)>::T VRaw;
    __shared__ float qs[DK], ks[DK], vs[DV], ps[256], red[8];
    __shared__ f4 part[16][DV / 4];
    const int tid = threadIdx.x;
    const long head = blockIdx.x;
    const int w = a.window, pos = a.pos, slot = pos % w;
    const int nvalid = min(pos + 1, w);
    const InT *kc = (const InT *)a.k_cache + head * w * DK;
    const InT *vc = (const InT *)a.v_cache + head * w * DV;
    // a cache slot s holds one of the last nvalid tokens iff (slot - s) mod w < nvalid
    // ---- cache loads: key slot t = tid / TPS (features f0 ..); value slots sg + 16 i (columns 4 cq ..) ----
    const int t = tid / TPS, f0 = FPT * (tid % TPS);
    const bool live = t < w && (slot - t + w) % w < nvalid;
    u4 kraw[KU];
    if (live && t != slot) {
#pragma unroll
        for (int i = 0; i < KU; ++i) kraw[i] = *(const u4 *)((const char *)(kc + (long)t * DK + f0) + 16 * i);
    }
    const int cq = tid & 15, sg = tid >> 4;
    VRaw vraw[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const int sl = sg + 16 * i;
        if (sl < w && sl != slot && (slot - sl + w) % w < nvalid)
            vraw[i] = *(const VRaw *)(vc + (long)sl * DV + 4 * cq);
    }
    if (tid < DK) {
        qs[tid] = ld1<InT>(a.q, head * DK + tid) * 0.125f;  // 1/sqrt(64)
        ks[tid] = ld1<InT>(a.k, head * DK + tid);
    } else if (tid < DK + DV) {
        vs[tid - DK] = ld1<InT>(a.v, head * DV + tid - DK);
    }
    __syncthreads();
    // ---- scores ----
    float acc = 0.f;
    if (live) {
        if (t == slot) {
#pragma unroll
            for (int f = 0; f < FPT; ++f) acc = __builtin_fmaf(qs[f0 + f], ks[f0 + f], acc);
        } else {
#pragma unroll
            for (int f = 0; f < FPT; ++f) {
                float x;
                if constexpr (sizeof(InT) == 2) {
                    const uint32_t wd = kraw[f / 8][(f % 8) / 2];
                    x = (f & 1) ? bf16_hi(wd) : bf16_lo(wd);
                } else {
                    x = __uint_as_float(kraw[f / 4][f % 4]);
                }
                acc = __builtin_fmaf(qs[f0 + f], x, acc);
            }
        }
    }
#pragma unroll
    for (int o = 1; o < TPS; o <<= 1) acc += __shfl_xor(acc, o);
    const float sc = live ? acc : -INFINITY;
    float m = sc;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float p = live ? __expf(sc - m) : 0.f;
    if (tid % TPS == 0) ps[t] = p;
    float sum = (tid % TPS == 0) ? p : 0.f;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
    __syncthreads();
    if ((tid & 63) == 0) red[4 + (tid >> 6)] = sum;
    // ---- weighted sum: column quad cq over slots sg, sg + 16, ... ----
    f4 y4 = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const int sl = sg + 16 * i;
        if (sl < w) {
            const float ptt = ps[sl];
            if (ptt != 0.f) {  // non-zero only for the last nvalid tokens
                const f4 v4 = sl == slot ? (f4){vs[4 * cq], vs[4 * cq + 1], vs[4 * cq + 2], vs[4 * cq + 3]}
                                         : unpack4(vraw[i]);
                y4 += ptt * v4;
            }
        }
    }
    part[sg][cq] = y4;
    __syncthreads();
    if (tid < DV) {
        const float tot = red[4] + red[5] + red[6] + red[7];
        float num = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) num += part[r][tid >> 2][tid & 3];
        const float yv = num / tot;
        if (a.y) {
            if (a.y_bf16) ((uint16_t *)a.y)[head * DV + tid] = f32_to_bf16_rne(yv);
            else ((float *)a.y)[head * DV + tid] = yv;
        }
        // append the new token to the cache (no thread reads this slot from the cache)
        InT *kw = (InT *)a.k_cache + (head * w + slot) * DK;
        InT *vw = (InT *)a.v_cache + (head * w + slot) * DV;
        if constexpr (sizeof(InT) == 2) {
            ((uint16_t *)kw)[tid] = f32_to_bf16_rne(ks[tid]);
            ((uint16_t *)vw)[tid] = f32_to_bf16_rne(vs[tid]);
        } else {
            kw[tid] = ks[tid];
            vw[tid] = vs[tid];
        }
    }
}

template <typename InT>
hipError_t launch_decode_t(const SwaArgs &a, hipStream_t s)
{
    const dim3 grid((unsigned)(a.B * a.H));
    if (a.window <= 64)
        hipLaunchKernelGGL((swa_decode_kernel<InT, 4>), grid, dim3(256), 0, s, a);
    else if (a.window <= 128)
        hipLaunchKernelGGL((swa_decode_kernel<InT, 2>), grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((swa_decode_kernel<InT, 1>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_swa_prefill(const SwaArgs &a, hipStream_t s)
{
    return a.y_bf16 ? launch_swa_t<uint16_t>(a, s) : launch_swa_t<float>(a, s);
}

hipError_t launch_swa_decode(const SwaArgs &a, int in_bf16, hipStream_t s)
{
    return in_bf16 ? launch_decode_t<uint16_t>(a, s) : launch_decode_t<float>(a, s);
}

}  // namespace bla
