// Internal declarations shared by the kernels and the C-ABI layer of
// libbasedla.so (gfx950).  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bla {

constexpr int kFeat = 16;                          // d' (query/key feature width)
constexpr int kD = 1 + kFeat + kFeat * kFeat;      // 273: Taylor feature dimension
constexpr int kDc = 1 + kFeat + kFeat * (kFeat + 1) / 2;  // 153: compact (folded) state rows

// Compact state layout: rows [1 | xb (kFeat) | one row per unordered pair
// {a, b}, a <= b, in row-major upper-triangle order]; the pair row holds
// S[a][b] + S[b][a] of the full layout (S[a][a] on the diagonal).  Because the
// quadratic features of phi are symmetric in (a, b), phi(q)^T S equals
// phi_c(q)^T fold(S) with phi_c(q)_ab = xb_a xb_b / sqrt 2.
__host__ __device__ constexpr int compact_pair(int a, int b)  // a <= b
{
    return a * kFeat - a * (a - 1) / 2 + (b - a);
}

// bf16 <-> fp32 helpers (bit-level; bf16 is the upper half of an fp32)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
// fp32 -> bf16, round to nearest even (NaN stays NaN): gfx950's packed
// conversion instruction
typedef __bf16 bla_bf16x2 __attribute__((ext_vector_type(2)));
typedef float bla_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((bla_f32x2){lo, hi}, bla_bf16x2));
}
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) { return (uint16_t)f32x2_to_bf16x2(f, 0.f); }

struct PrefillArgs {
    int B, H, N, M, dv;
    float eps;
    const void *q, *k, *v, *ke, *ve;  // bf16 or fp32 according to the kernel
    const float *S0, *z0;
    void *y;
    int y_bf16;                       // 1: y is bf16, 0: fp32
    float *S_out, *z_out;
    int compact;                      // 1: S0/z0/S_out/z_out in the compact layout (kDc rows)
    const int *prefix_len;            // [B] valid prefix tokens (left padding), or null: all M
};

// Valid (unpadded) prefix tokens of batch element b: the last m of the M prefix
// rows; the first M - m rows are left padding and never read.
__device__ __forceinline__ int valid_prefix(const PrefillArgs &a, int b)
{
    if (!a.prefix_len) return a.M;
    const int m = a.prefix_len[b];
    return m < 0 ? 0 : (m > a.M ? a.M : m);
}

// fp16-MFMA chunked prefill with the compact symmetric state (bf16 inputs);
// returns hipSuccess or the launch error
hipError_t launch_prefill_sym(const PrefillArgs &a, int col_split_allowed, hipStream_t s);
// exact fp32 token-sequential prefill (fp32 or bf16 inputs)
hipError_t launch_prefill_exact(const PrefillArgs &a, int in_bf16, hipStream_t s);

struct DecodeArgs {
    int B, H, dv;
    float eps;
    const void *q, *k, *v;
    float *S, *z;
    void *y;
    int y_bf16;
    int compact;  // 1: S, z in the compact layout (kDc rows)
};
hipError_t launch_decode(const DecodeArgs &a, int in_bf16, hipStream_t s);

struct SwaArgs {
    int B, H, N, window, pos;  // pos: decode only (tokens before this one)
    const void *q, *k, *v;     // prefill [B][H][N][64] / decode [B][H][64]
    void *y;
    int y_bf16;
    void *k_cache, *v_cache;   // [B][H][window][64] in the input dtype (decode: in place)
};
// sliding-window softmax attention (bf16 inputs, d = d_v = 64, window <= 256)
hipError_t launch_swa_prefill(const SwaArgs &a, hipStream_t s);
hipError_t launch_swa_decode(const SwaArgs &a, int in_bf16, hipStream_t s);

}  // namespace bla
