/*
 * based_la.h -- C ABI of the MI355X (gfx950) causal Taylor linear-attention
 * library: BASED prefill, JRT-RNN prefix prefill and the state-passing decode
 * step.
 *
 * The method (cited from the reading-notes pages it is built from):
 *   [BASED] "Simple linear attention language models balance the
 *     recall-throughput tradeoff" notes.  §2.2: s_i = s_{i-1} + phi(k_i) v_i^T,
 *     z_i = z_{i-1} + phi(k_i), y_i = s_i^T phi(q_i) / z_i^T phi(q_i), equal to
 *     the attention form sum_{j<=i} K(q_i,k_j) v_j / sum_{j<=i} K(q_i,k_j).
 *     §2.3, Eq. (4): K(q,k) = 1 + q.k/sqrt(d') + (q.k)^2/(2 d'), realised by
 *     phi(x) = [1, xb, vec(xb xb^T)/sqrt(2)], xb = x / d'^(1/4), of dimension
 *     D = 1 + d' + d'^2 (273 for d' = 16).  §2.5: chunked prefill and the
 *     recurrent decode step that reads and writes the persistent state.
 *   [JRT] "Just read twice: closing the recall gap for recurrent language
 *     models" notes.  §2.6, Eq. (3): a non-causal prefix state s_E, z_E summed
 *     over M prefix tokens (own keys/values k_e, v_e) is added to the causal
 *     state at every position; Eq. (4): the cached state is s_E + s_{D,N}.
 *     §2.8: the prefix state seeds the causal scan.
 *   [LG] "Understanding and Improving Length Generalization in Recurrent
 *     Models" notes.  §2.5, Eq. (4): a non-zero initial state is carried by the
 *     same scan (for linear attention it is added to s and z); §2.6: the final
 *     state of one call is the initial state of the next (state passing).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller, contiguous
 *     row-major, 16-byte aligned.  Nothing is allocated or freed here.
 *   - Shapes: q, k [B][H][N][d_feat]; v [B][H][N][d_v] (in_dtype);
 *             y [B][H][N][d_v] (out_dtype);
 *             S [B][H][D][d_v] fp32, z [B][H][D] fp32, D = bla_feature_dim(d_feat),
 *             feature order [1 | xb (d_feat) | vec(xb xb^T)/sqrt2 (d_feat^2,
 *             index 1 + d_feat + a*d_feat + b)].
 *   - Inputs are taken raw: the kernel applies the 1/d'^(1/4) scale.
 *   - y_i includes token i itself (update first, then read).
 *   - eps is added to every denominator (0 is fine: K >= 1/2 > 0).
 *   - stream is a hipStream_t passed as void* (NULL = default stream).  Calls
 *     are asynchronous: they return after the launch is enqueued; device
 *     faults surface at the caller's next synchronisation.
 *   - The library keeps no state between calls; calls are thread-safe.  Calls
 *     that write overlapping memory must not run concurrently.
 *   - Every argument is validated before anything is launched, so a call that
 *     returns an error has changed nothing.
 *
 * Supported on the GPU: d_feat == 16; d_v in {16, 32, 64}; B * H <= 2^21
 * (2,097,152) heads, whose kernels run 1024 threads per head, except F32
 * inputs with d_v = 64 (512 threads per head): B * H <= 2^22; so that one
 * dispatch carries at most 2^31 work-items;
 * N * d_v * 4 and M * d_v * 4 below 2^31 (N <= 8,388,607 tokens at d_v = 64); in_dtype BF16
 * (the fp16-MFMA chunked kernel) or F32 (fp64 arithmetic for fp32-exact results:
 * the attention form over several workgroups per head when N <= 256, there is no
 * prefix and the state is not updated in place; otherwise a token-sequential
 * kernel).  Anything else that is valid returns BLA_ERR_UNSUPPORTED.
 * Numerics of the BF16 path: operands of the matrix-core products are fp16
 * (bf16 inputs are exact in fp16), accumulation, state and denominators fp32;
 * the relative error per output row is ~5e-4.  Internally the order-2 state is
 * kept with each unordered feature pair once (160 rows instead of 273),
 * whichever ABI layout (full or compact, below) the call uses.  Power-of-two
 * operand scales keep the fp16 operands in range for |q.k| <= 3.2e4, |q_a| < 255, |k_a| < 4095,
 * |v| <= 65504, and per state entry sum_j |k_ja k_jb v_jc|, sum_j |k_ja k_jb|
 * below 1.6e7 and sum_j |k_ja v_jc|, |sum_j v_jc| below 1e6; inputs outside
 * this range overflow to inf/NaN (not checked).
 * NaN/Inf inputs propagate unchecked.
 */
#ifndef BASED_LA_H
#define BASED_LA_H

#ifdef __cplusplus
extern "C" {
#endif

/* The RANGE_ enumerators are not values of the type: they make every int a
 * representable value of it, so that an out-of-range code passed by a caller
 * is a defined value the library can reject (C++ otherwise limits an enum to
 * the bit width of its enumerators). */
typedef enum {
    BLA_OK = 0,
    BLA_ERR_INVALID = 1,     /* NULL required pointer, bad size, misalignment, bad aliasing */
    BLA_ERR_UNSUPPORTED = 2, /* valid but not implemented (d_feat != 16, d_v not 16/32/64, dtype) */
    BLA_ERR_HIP = 3,         /* the HIP runtime reported an error at launch */
    BLA_STATUS_RANGE_MIN = -2147483647 - 1,
    BLA_STATUS_RANGE_MAX = 2147483647
} bla_status;

typedef enum {
    BLA_F32 = 0,
    BLA_BF16 = 1,
    BLA_DTYPE_RANGE_MIN = -2147483647 - 1,
    BLA_DTYPE_RANGE_MAX = 2147483647
} bla_dtype;

/* D = 1 + d + d*d, the feature dimension of the Taylor map ([BASED] §2.3).
 * Returns -1 for d < 1. */
int bla_feature_dim(int d_feat);

/* Static, human-readable name of a status code ("unknown bla_status" for any
 * other value). */
const char *bla_status_string(bla_status status);

/* Causal Taylor linear-attention prefill with explicit initial state
 * ([BASED] §2.2/§2.5, [LG] §2.5 Eq. (4)).
 *   B, H >= 1; N >= 0 (tokens); d_feat == 16; d_v in {16, 32, 64}.
 *   q, k, v : inputs (in_dtype).  Required when N > 0.
 *   S0, z0  : initial state, or both NULL for the zero state (one NULL and
 *             the other not is BLA_ERR_INVALID).
 *   y       : output [B][H][N][d_v] in out_dtype, or NULL to skip it.  Until
 *             the call completes, y's memory may hold intermediate values: with
 *             few heads and a long sequence (BF16 inputs), each segment of a
 *             head's sequence keeps its partial state in its own rows of y
 *             before its outputs overwrite them.
 *   S_out, z_out : final state S_N, z_N (each may be NULL to skip it).
 *             S_out may be exactly S0 and z_out exactly z0 (in place); any
 *             other overlap between outputs and inputs is BLA_ERR_INVALID.
 *   Returns BLA_OK after enqueueing the work on `stream`. */
bla_status based_prefill(int B, int H, int N, int d_feat, int d_v, bla_dtype in_dtype, bla_dtype out_dtype,
                         float eps, const void *q, const void *k, const void *v, const float *S0,
                         const float *z0, void *y, float *S_out, float *z_out, void *stream);

/* JRT-RNN prefix linear attention ([JRT] §2.6 Eqs. (3)-(4), §2.8): the
 * non-causal prefix state from (k_e, v_e) over M tokens is added to the
 * initial state, then the causal scan runs over all N positions with the
 * same queries.  y_i = phi(q_i)^T (S0 + s_E + s_{D,i}) / phi(q_i)^T (z0 + z_E + z_{D,i}).
 *   M >= 0 (M == 0 is exactly based_prefill); k_e [B][H][M][d_feat],
 *   v_e [B][H][M][d_v] (in_dtype), required when M > 0.
 *   S_out/z_out receive the merged state S0 + s_E + s_{D,N} (Eq. (4)).
 *   Other arguments, aliasing and errors as based_prefill. */
bla_status jrt_prefix_prefill(int B, int H, int N, int M, int d_feat, int d_v, bla_dtype in_dtype,
                              bla_dtype out_dtype, float eps, const void *q, const void *k,
                              const void *v, const void *k_e, const void *v_e, const float *S0,
                              const float *z0, void *y, float *S_out, float *z_out, void *stream);

/* One recurrent decode step per (b, h) on a persistent fp32 state
 * ([BASED] §2.5: the fused outer-product write and query read; [LG] §2.6:
 * state passing).  q, k [B][H][d_feat], v [B][H][d_v] (in_dtype);
 * S [B][H][D][d_v] and z [B][H][D] are read and updated in place
 * (S += phi(k) v^T, z += phi(k)); then y [B][H][d_v] (out_dtype) =
 * S^T phi(q) / (z^T phi(q) + eps).  y may be NULL.  All fp32 arithmetic.
 *   Errors as based_prefill. */
bla_status based_decode_step(int B, int H, int d_feat, int d_v, bla_dtype in_dtype, bla_dtype out_dtype,
                             float eps, const void *q, const void *k, const void *v, float *S,
                             float *z, void *y, void *stream);

/* ---------------- compact (folded) state layout ----------------
 * The quadratic features of phi are symmetric in (a, b) ([BASED] §2.3: the
 * entries of vec(xb xb^T) repeat), so phi(q)^T S depends on S only through
 * S[a][b] + S[b][a].  The compact layout keeps one row per unordered pair:
 *   Dc = bla_compact_dim(d_feat) = 1 + d + d(d+1)/2 rows (153 for d = 16):
 *   row 0: order 0 (as in the full layout); rows 1..d: xb (as in the full
 *   layout); row 1 + d + P(a,b) for a <= b, P(a,b) = a*d - a*(a-1)/2 + (b-a)
 *   (row-major upper triangle), holding S[a][b] + S[b][a] for a < b and
 *   S[a][a] for a == b.  z uses the same rows.
 * This fold is exact for every output: with phi_c(q) = [1, xb,
 * xb_a xb_b / sqrt2 (a <= b)], phi(q)^T S == phi_c(q)^T fold(S) and
 * phi(q)^T z == phi_c(q)^T fold(z) for any S, z (symmetric or not).  A full
 * state that is folded and passed to a *_compact call gives the same y as the
 * full state passed to the full-layout call; the compact final state is the
 * fold of the full one.  The decode step reads and writes Dc/D = 56% of the
 * bytes. */

/* Dc = 1 + d + d(d+1)/2, rows of the compact state; -1 for d < 1. */
int bla_compact_dim(int d_feat);

/* based_prefill with S0, z0, S_out, z_out in the compact layout
 * ([B][H][Dc][d_v] and [B][H][Dc] fp32).  Everything else (arguments,
 * aliasing, in-place state, errors) as based_prefill. */
bla_status based_prefill_compact(int B, int H, int N, int d_feat, int d_v, bla_dtype in_dtype,
                                 bla_dtype out_dtype, float eps, const void *q, const void *k,
                                 const void *v, const float *S0, const float *z0, void *y,
                                 float *S_out, float *z_out, void *stream);

/* jrt_prefix_prefill with the state in the compact layout; S_out/z_out
 * receive fold(S0 + s_E + s_{D,N}) ([JRT] Eq. (4)). */
bla_status jrt_prefix_prefill_compact(int B, int H, int N, int M, int d_feat, int d_v,
                                      bla_dtype in_dtype, bla_dtype out_dtype, float eps, const void *q,
                                      const void *k, const void *v, const void *k_e,
                                      const void *v_e, const float *S0, const float *z0, void *y,
                                      float *S_out, float *z_out, void *stream);

typedef enum {
    BLA_STATE_FULL = 0,
    BLA_STATE_COMPACT = 1,
    BLA_STATE_RANGE_MIN = -2147483647 - 1,
    BLA_STATE_RANGE_MAX = 2147483647
} bla_state_layout;

/* JRT-RNN prefix prefill with left-padded prefixes ([JRT] §2.7: a prompt
 * shorter than M is left-padded to M and the padding is masked in the prefix
 * linear attention, so that it never enters the state).
 *   prefix_len: DEVICE array of B int32, the number of valid prefix tokens of
 *     each batch element; its prefix is then rows [M - prefix_len[b], M) of
 *     k_e/v_e, and rows [0, M - prefix_len[b]) are padding that is never read.
 *     Values are clamped to [0, M].  NULL: every prefix row is valid (exactly
 *     jrt_prefix_prefill).  Must be 4-byte aligned and not overlap an output.
 *   state_layout: BLA_STATE_FULL (S0/z0/S_out/z_out with D rows) or
 *     BLA_STATE_COMPACT (Dc rows); anything else is BLA_ERR_INVALID.
 *   Everything else as jrt_prefix_prefill. */
bla_status jrt_prefix_prefill_ex(int B, int H, int N, int M, int d_feat, int d_v, bla_dtype in_dtype,
                                 bla_dtype out_dtype, float eps, const void *q, const void *k,
                                 const void *v, const void *k_e, const void *v_e,
                                 const int *prefix_len, const float *S0, const float *z0, void *y,
                                 float *S_out, float *z_out, bla_state_layout state_layout, void *stream);

/* based_decode_step on a compact state S [B][H][Dc][d_v], z [B][H][Dc]
 * (updated in place: pair row {a,b} += m_ab xb_a xb_b / sqrt2 * v^T with
 * m_ab = 2 for a < b, 1 for a == b; y = S^T phi_c(q) / (z^T phi_c(q) + eps)). */
bla_status based_decode_step_compact(int B, int H, int d_feat, int d_v, bla_dtype in_dtype,
                                     bla_dtype out_dtype, float eps, const void *q, const void *k,
                                     const void *v, float *S, float *z, void *y, void *stream);

/* ---------------- sliding-window softmax attention ----------------
 * [BASED] §2.4: the second mixer of the BASED architecture is standard
 * softmax attention restricted to the w most recent keys:
 *   y_i = sum_{j = max(0, i-w+1)}^{i} softmax_j(q_i . k_j / sqrt(d)) v_j,
 * with a per-head state of the w most recent keys and values; §2.5: the
 * decode step fuses the dot products, the softmax and the weighted sum.
 * No rotary embedding is applied (the caller applies any position encoding).
 * Supported: d == d_v == 64, 1 <= window <= 256, and B * H * ceil(N / 128) <= 2^22
 * (one workgroup per head and 128-query tile); BLA_ERR_UNSUPPORTED above.
 * The KV cache is a ring of `window` slots: token p (0-based) sits in slot
 * p % window; k_cache [B][H][window][d], v_cache [B][H][window][d_v] in the
 * input dtype. */

/* SWA prefill over N tokens: q, k [B][H][N][d], v [B][H][N][d_v], BF16 only
 * (BLA_ERR_UNSUPPORTED for F32 inputs); y [B][H][N][d_v] in out_dtype, or
 * NULL.  k_cache/v_cache (both or neither): receive the ring cache of the last
 * min(N, window) tokens (other slots untouched), ready for swa_decode_step at
 * pos = N.  Outputs must not overlap inputs or each other.  Numerics: the
 * scores are exact products of the bf16 inputs summed in fp32, the softmax is
 * fp32, and its weights are rounded to fp16 for the value product (fp32
 * accumulation); the worst row error against fp64 is about 4e-4 of the row's
 * largest output. */
bla_status swa_prefill(int B, int H, int N, int d, int d_v, int window, bla_dtype in_dtype, bla_dtype out_dtype,
                       const void *q, const void *k, const void *v, void *y, void *k_cache,
                       void *v_cache, void *stream);

/* One SWA decode step for the token at position pos (pos >= 0 tokens before
 * it): writes k, v [B][H][d|d_v] into slot pos % window of the caches (in
 * place), then y [B][H][d_v] (out_dtype, or NULL) = softmax attention of q
 * over the min(pos + 1, window) most recent tokens.  BF16 or F32 inputs; the
 * caches have the input dtype; fp32 arithmetic. */
bla_status swa_decode_step(int B, int H, int d, int d_v, int window, int pos, bla_dtype in_dtype,
                           bla_dtype out_dtype, const void *q, const void *k, const void *v,
                           void *k_cache, void *v_cache, void *y, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BASED_LA_H */
