// C-ABI entry points of libbasedla.so: argument validation and dispatch.
// Declarations, semantics and citations: include/based_la.h.
#include "../../include/based_la.h"

#include <stdint.h>

#include "common.h"

namespace {

struct Range {
    uintptr_t lo = 0, hi = 0;  // [lo, hi)
    bool empty() const { return hi <= lo; }
};

Range range_of(const void *p, long long bytes)
{
    Range r;
    if (p && bytes > 0) {
        r.lo = (uintptr_t)p;
        r.hi = r.lo + (uintptr_t)bytes;
    }
    return r;
}

bool overlap(const Range &a, const Range &b)
{
    return !a.empty() && !b.empty() && a.lo < b.hi && b.lo < a.hi;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// One dispatch carries at most 2^31 work-items (HIP counts them in 32 bits):
// the grid has at most 2^22 workgroups of at most 512 threads, except two
// prefill kernels that run 1024 threads per workgroup and are therefore held
// to 2^21 heads: the bf16-input kernel (sixteen wavefronts per head; it splits
// a head over several workgroups only when there are 128 heads or fewer) and
// the fp32-input token-sequential kernel at d_v <= 32.
constexpr long long kMaxBlocks = 1LL << 22;
constexpr long long kMaxBlocks1024 = 1LL << 21;

bool dtype_ok(int t) { return t == BLA_F32 || t == BLA_BF16; }
int dtype_bytes(int t) { return t == BLA_F32 ? 4 : 2; }

// common shape checks; returns BLA_OK or the status to report
bla_status check_dims(int B, int H, int N, int M, int d_feat, int d_v, int in_dtype, int out_dtype)
{
    if (B < 1 || H < 1 || N < 0 || M < 0 || d_feat < 1 || d_v < 1) return BLA_ERR_INVALID;
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return BLA_ERR_INVALID;
    if ((long long)B * H * (long long)(N > M ? N : M) * 64 > (1LL << 46)) return BLA_ERR_INVALID;
    if ((long long)B * H > kMaxBlocks) return BLA_ERR_UNSUPPORTED;  // one workgroup per head
    if (d_feat != bla::kFeat) return BLA_ERR_UNSUPPORTED;
    // per-head byte ranges are addressed with 32-bit buffer offsets
    if ((long long)(N > M ? N : M) * d_v * 4 >= (1LL << 31)) return BLA_ERR_UNSUPPORTED;
    if (d_v != 16 && d_v != 32 && d_v != 64) return BLA_ERR_UNSUPPORTED;
    return BLA_OK;
}

// Output ranges must not overlap each other or any input, except an exact
// in-place state (same pointer as its input).
bla_status check_aliasing(const Range *outs, int n_out, const Range *ins, int n_in,
                          const void *S_out, const void *S0, const void *z_out, const void *z0)
{
    for (int i = 0; i < n_out; ++i) {
        for (int j = i + 1; j < n_out; ++j)
            if (overlap(outs[i], outs[j])) return BLA_ERR_INVALID;
        for (int j = 0; j < n_in; ++j) {
            if (!overlap(outs[i], ins[j])) continue;
            const bool same = outs[i].lo == ins[j].lo && outs[i].hi == ins[j].hi;
            const bool state_pair = (outs[i].lo == (uintptr_t)S_out && ins[j].lo == (uintptr_t)S0) ||
                                    (outs[i].lo == (uintptr_t)z_out && ins[j].lo == (uintptr_t)z0);
            if (!(same && state_pair)) return BLA_ERR_INVALID;
        }
    }
    return BLA_OK;
}

bla_status run_prefill(int B, int H, int N, int M, int d_feat, int d_v, int in_dtype,
                       int out_dtype, float eps, const void *q, const void *k, const void *v,
                       const void *k_e, const void *v_e, const float *S0, const float *z0,
                       void *y, float *S_out, float *z_out, void *stream, int compact,
                       const int *prefix_len = nullptr)
{
    bla_status st = check_dims(B, H, N, M, d_feat, d_v, in_dtype, out_dtype);
    if (st != BLA_OK) return st;
    if ((in_dtype == BLA_BF16 || d_v <= 32) && (long long)B * H > kMaxBlocks1024) return BLA_ERR_UNSUPPORTED;
    if (prefix_len && ((uintptr_t)prefix_len & 3u)) return BLA_ERR_INVALID;
    if (N > 0 && (!q || !k || !v)) return BLA_ERR_INVALID;
    if (M > 0 && (!k_e || !v_e)) return BLA_ERR_INVALID;
    if ((S0 == nullptr) != (z0 == nullptr)) return BLA_ERR_INVALID;
    const void *ptrs[] = {q, k, v, k_e, v_e, S0, z0, y, S_out, z_out};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return BLA_ERR_INVALID;

    const long long heads = (long long)B * H;
    const long long D = compact ? bla::kDc : bla::kD;
    const int ib = dtype_bytes(in_dtype), ob = dtype_bytes(out_dtype);
    const Range in_r[] = {
        range_of(q, heads * N * d_feat * ib),   range_of(k, heads * N * d_feat * ib),
        range_of(v, heads * N * d_v * ib),      range_of(k_e, heads * M * d_feat * ib),
        range_of(v_e, heads * M * d_v * ib),    range_of(S0, heads * D * d_v * 4),
        range_of(z0, heads * D * 4)};
    const Range out_r[] = {range_of(N > 0 ? y : nullptr, heads * N * d_v * ob),
                           range_of(S_out, heads * D * d_v * 4), range_of(z_out, heads * D * 4)};
    st = check_aliasing(out_r, 3, in_r, 7, S_out, S0, z_out, z0);
    if (st != BLA_OK) return st;
    const Range len_r[] = {range_of(prefix_len, (long long)B * 4)};
    st = check_aliasing(out_r, 3, len_r, 1, nullptr, nullptr, nullptr, nullptr);
    if (st != BLA_OK) return st;

    const bool want_y = y && N > 0;
    if (!want_y && !S_out && !z_out) return BLA_OK;  // nothing to produce

    bla::PrefillArgs a;
    a.B = B;
    a.H = H;
    a.N = N;
    a.M = M;
    a.dv = d_v;
    a.eps = eps;
    a.q = q;
    a.k = k;
    a.v = v;
    a.ke = k_e;
    a.ve = v_e;
    a.S0 = S0;
    a.z0 = z0;
    a.y = want_y ? y : nullptr;
    a.y_bf16 = out_dtype == BLA_BF16;
    a.S_out = S_out;
    a.z_out = z_out;
    a.compact = compact;
    a.prefix_len = M > 0 ? prefix_len : nullptr;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (in_dtype == BLA_BF16) {
        // in-place z with several column blocks per head would let one block
        // overwrite z before another has read it: keep one block per head then
        const int split_ok = !(z_out && z_out == z0);
        e = bla::launch_prefill_sym(a, split_ok, s);
    } else {
        e = bla::launch_prefill_exact(a, 0, s);
    }
    return e == hipSuccess ? BLA_OK : BLA_ERR_HIP;
}

bla_status run_decode(int B, int H, int d_feat, int d_v, int in_dtype, int out_dtype, float eps,
                      const void *q, const void *k, const void *v, float *S, float *z, void *y,
                      void *stream, int compact)
{
    bla_status st = check_dims(B, H, 1, 0, d_feat, d_v, in_dtype, out_dtype);
    if (st != BLA_OK) return st;
    if (!q || !k || !v || !S || !z) return BLA_ERR_INVALID;
    const void *ptrs[] = {q, k, v, S, z, y};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return BLA_ERR_INVALID;
    const long long heads = (long long)B * H;
    const int ib = dtype_bytes(in_dtype), ob = dtype_bytes(out_dtype);
    const Range in_r[] = {range_of(q, heads * d_feat * ib), range_of(k, heads * d_feat * ib),
                          range_of(v, heads * d_v * ib)};
    const long long D = compact ? bla::kDc : bla::kD;
    const Range out_r[] = {range_of(y, heads * d_v * ob), range_of(S, heads * D * d_v * 4),
                           range_of(z, heads * D * 4)};
    st = check_aliasing(out_r, 3, in_r, 3, nullptr, nullptr, nullptr, nullptr);
    if (st != BLA_OK) return st;

    bla::DecodeArgs a;
    a.B = B;
    a.H = H;
    a.dv = d_v;
    a.eps = eps;
    a.q = q;
    a.k = k;
    a.v = v;
    a.S = S;
    a.z = z;
    a.y = y;
    a.y_bf16 = out_dtype == BLA_BF16;
    a.compact = compact;
    const hipError_t e = bla::launch_decode(a, in_dtype == BLA_BF16, (hipStream_t)stream);
    return e == hipSuccess ? BLA_OK : BLA_ERR_HIP;
}

bla_status check_swa(int B, int H, int N, int d, int d_v, int window, int in_dtype, int out_dtype)
{
    if (B < 1 || H < 1 || N < 0 || d < 1 || d_v < 1 || window < 1) return BLA_ERR_INVALID;
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return BLA_ERR_INVALID;
    // one workgroup per head and 128-query tile (per head for a decode step)
    if ((long long)B * H * (N > 128 ? (N + 127) / 128 : 1) > kMaxBlocks) return BLA_ERR_UNSUPPORTED;
    if (d != 64 || d_v != 64 || window > 256) return BLA_ERR_UNSUPPORTED;
    if ((long long)N * 64 * 4 >= (1LL << 31)) return BLA_ERR_UNSUPPORTED;  // 32-bit per-head offsets
    return BLA_OK;
}

}  // namespace

extern "C" {

int bla_feature_dim(int d_feat)
{
    if (d_feat < 1 || d_feat > 4096) return -1;
    return 1 + d_feat + d_feat * d_feat;
}

const char *bla_status_string(bla_status status)
{
    switch (status) {
    case BLA_OK: return "BLA_OK";
    case BLA_ERR_INVALID: return "BLA_ERR_INVALID: invalid argument";
    case BLA_ERR_UNSUPPORTED: return "BLA_ERR_UNSUPPORTED: valid but not implemented";
    case BLA_ERR_HIP: return "BLA_ERR_HIP: HIP runtime error at launch";
    default: return "unknown bla_status";
    }
}

bla_status based_prefill(int B, int H, int N, int d_feat, int d_v, bla_dtype in_dtype, bla_dtype out_dtype,
                         float eps, const void *q, const void *k, const void *v, const float *S0,
                         const float *z0, void *y, float *S_out, float *z_out, void *stream)
{
    return run_prefill(B, H, N, 0, d_feat, d_v, in_dtype, out_dtype, eps, q, k, v, nullptr,
                       nullptr, S0, z0, y, S_out, z_out, stream, 0);
}

bla_status jrt_prefix_prefill(int B, int H, int N, int M, int d_feat, int d_v, bla_dtype in_dtype,
                              bla_dtype out_dtype, float eps, const void *q, const void *k,
                              const void *v, const void *k_e, const void *v_e, const float *S0,
                              const float *z0, void *y, float *S_out, float *z_out, void *stream)
{
    return run_prefill(B, H, N, M, d_feat, d_v, in_dtype, out_dtype, eps, q, k, v, k_e, v_e, S0,
                       z0, y, S_out, z_out, stream, 0);
}

bla_status based_decode_step(int B, int H, int d_feat, int d_v, bla_dtype in_dtype, bla_dtype out_dtype,
                             float eps, const void *q, const void *k, const void *v, float *S,
                             float *z, void *y, void *stream)
{
    return run_decode(B, H, d_feat, d_v, in_dtype, out_dtype, eps, q, k, v, S, z, y, stream, 0);
}

int bla_compact_dim(int d_feat)
{
    if (d_feat < 1 || d_feat > 4096) return -1;
    return 1 + d_feat + d_feat * (d_feat + 1) / 2;
}

bla_status based_prefill_compact(int B, int H, int N, int d_feat, int d_v, bla_dtype in_dtype,
                                 bla_dtype out_dtype, float eps, const void *q, const void *k,
                                 const void *v, const float *S0, const float *z0, void *y,
                                 float *S_out, float *z_out, void *stream)
{
    return run_prefill(B, H, N, 0, d_feat, d_v, in_dtype, out_dtype, eps, q, k, v, nullptr,
                       nullptr, S0, z0, y, S_out, z_out, stream, 1);
}

bla_status jrt_prefix_prefill_compact(int B, int H, int N, int M, int d_feat, int d_v,
                                      bla_dtype in_dtype, bla_dtype out_dtype, float eps, const void *q,
                                      const void *k, const void *v, const void *k_e,
                                      const void *v_e, const float *S0, const float *z0, void *y,
                                      float *S_out, float *z_out, void *stream)
{
    return run_prefill(B, H, N, M, d_feat, d_v, in_dtype, out_dtype, eps, q, k, v, k_e, v_e, S0,
                       z0, y, S_out, z_out, stream, 1);
}

bla_status jrt_prefix_prefill_ex(int B, int H, int N, int M, int d_feat, int d_v, bla_dtype in_dtype,
                                 bla_dtype out_dtype, float eps, const void *q, const void *k,
                                 const void *v, const void *k_e, const void *v_e,
                                 const int *prefix_len, const float *S0, const float *z0, void *y,
                                 float *S_out, float *z_out, bla_state_layout state_layout, void *stream)
{
    if (state_layout != BLA_STATE_FULL && state_layout != BLA_STATE_COMPACT) return BLA_ERR_INVALID;
    return run_prefill(B, H, N, M, d_feat, d_v, in_dtype, out_dtype, eps, q, k, v, k_e, v_e, S0,
                       z0, y, S_out, z_out, stream, state_layout == BLA_STATE_COMPACT, prefix_len);
}

bla_status based_decode_step_compact(int B, int H, int d_feat, int d_v, bla_dtype in_dtype,
                                     bla_dtype out_dtype, float eps, const void *q, const void *k,
                                     const void *v, float *S, float *z, void *y, void *stream)
{
    return run_decode(B, H, d_feat, d_v, in_dtype, out_dtype, eps, q, k, v, S, z, y, stream, 1);
}

}  // extern "C"

extern "C" {

bla_status swa_prefill(int B, int H, int N, int d, int d_v, int window, bla_dtype in_dtype, bla_dtype out_dtype,
                       const void *q, const void *k, const void *v, void *y, void *k_cache,
                       void *v_cache, void *stream)
{
    bla_status st = check_swa(B, H, N, d, d_v, window, in_dtype, out_dtype);
    if (st != BLA_OK) return st;
    if (in_dtype != BLA_BF16) return BLA_ERR_UNSUPPORTED;
    if (N > 0 && (!q || !k || !v)) return BLA_ERR_INVALID;
    if ((k_cache == nullptr) != (v_cache == nullptr)) return BLA_ERR_INVALID;
    const void *ptrs[] = {q, k, v, y, k_cache, v_cache};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return BLA_ERR_INVALID;
    const long long heads = (long long)B * H;
    const int ob = dtype_bytes(out_dtype);
    const Range in_r[] = {range_of(q, heads * N * d * 2), range_of(k, heads * N * d * 2),
                          range_of(v, heads * N * d_v * 2)};
    const Range out_r[] = {range_of(N > 0 ? y : nullptr, heads * N * d_v * ob),
                           range_of(k_cache, heads * window * d * 2),
                           range_of(v_cache, heads * window * d_v * 2)};
    st = check_aliasing(out_r, 3, in_r, 3, nullptr, nullptr, nullptr, nullptr);
    if (st != BLA_OK) return st;
    if (N == 0 || (!y && !k_cache)) return BLA_OK;
    bla::SwaArgs a;
    a.B = B;
    a.H = H;
    a.N = N;
    a.window = window;
    a.pos = 0;
    a.q = q;
    a.k = k;
    a.v = v;
    a.y = y;
    a.y_bf16 = out_dtype == BLA_BF16;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    const hipError_t e = bla::launch_swa_prefill(a, (hipStream_t)stream);
    return e == hipSuccess ? BLA_OK : BLA_ERR_HIP;
}

bla_status swa_decode_step(int B, int H, int d, int d_v, int window, int pos, bla_dtype in_dtype,
                           bla_dtype out_dtype, const void *q, const void *k, const void *v,
                           void *k_cache, void *v_cache, void *y, void *stream)
{
    bla_status st = check_swa(B, H, 1, d, d_v, window, in_dtype, out_dtype);
    if (st != BLA_OK) return st;
    if (pos < 0) return BLA_ERR_INVALID;
    if (!q || !k || !v || !k_cache || !v_cache) return BLA_ERR_INVALID;
    const void *ptrs[] = {q, k, v, y, k_cache, v_cache};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return BLA_ERR_INVALID;
    const long long heads = (long long)B * H;
    const int ib = dtype_bytes(in_dtype), ob = dtype_bytes(out_dtype);
    const Range in_r[] = {range_of(q, heads * d * ib), range_of(k, heads * d * ib),
                          range_of(v, heads * d_v * ib)};
    const Range out_r[] = {range_of(y, heads * d_v * ob), range_of(k_cache, heads * window * d * ib),
                           range_of(v_cache, heads * window * d_v * ib)};
    st = check_aliasing(out_r, 3, in_r, 3, nullptr, nullptr, nullptr, nullptr);
    if (st != BLA_OK) return st;
    bla::SwaArgs a;
    a.B = B;
    a.H = H;
    a.N = 1;
    a.window = window;
    a.pos = pos;
    a.q = q;
    a.k = k;
    a.v = v;
    a.y = y;
    a.y_bf16 = out_dtype == BLA_BF16;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    const hipError_t e = bla::launch_swa_decode(a, in_dtype == BLA_BF16, (hipStream_t)stream);
    return e == hipSuccess ? BLA_OK : BLA_ERR_HIP;
}

}  // extern "C"
