// Peak-rate micro-kernels (include/based_la_probe.h): a matrix-core loop with
// no memory traffic and a 16-byte-vector streaming copy.  They carry none of
// the method's arithmetic; they give the measured ceilings stated beside the
// vendor peaks.
#include "../../include/based_la_probe.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kChains = 8;  // independent accumulators per wavefront

__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(int iters, float *sink)
{
    const int t = threadIdx.x;
    // operands that depend on the lane, so nothing folds at compile time
    const _Float16 x = (_Float16)(1.0f + 0.0009765625f * (float)(t & 63));
    h8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = x;
        b[i] = (_Float16)(0.5f) - x * (_Float16)0.001f;
    }
    f4 acc[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j) acc[j] = (f4){0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kChains; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kChains; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    sink[(long)blockIdx.x * kProbeThreads + t] = s;
}

__global__ __launch_bounds__(kProbeThreads) void copy_probe_kernel(const u4 *__restrict__ src, u4 *__restrict__ dst,
                                                                   long n)
{
    const long stride = (long)gridDim.x * kProbeThreads;
    long i = (long)blockIdx.x * kProbeThreads + threadIdx.x;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const u4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        dst[i] = a;
        dst[i + stride] = b;
        dst[i + 2 * stride] = c;
        dst[i + 3 * stride] = d;
    }
    for (; i < n; i += stride) dst[i] = src[i];
}

}  // namespace

extern "C" {

bla_status bla_probe_mfma_f16(int blocks, int iters, float *sink, void *stream)
{
    if (blocks < 1 || blocks > 65536 || iters < 1 || iters > (1 << 20) || !sink || ((uintptr_t)sink & 3u))
        return BLA_ERR_INVALID;
    hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, (hipStream_t)stream,
                       iters, sink);
    return hipGetLastError() == hipSuccess ? BLA_OK : BLA_ERR_HIP;
}

bla_status bla_probe_copy(const void *src, void *dst, long long bytes, void *stream)
{
    if (!src || !dst || bytes <= 0 || (bytes & 15) || ((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u))
        return BLA_ERR_INVALID;
    const uintptr_t s = (uintptr_t)src, d = (uintptr_t)dst;
    if (s < d + (uintptr_t)bytes && d < s + (uintptr_t)bytes) return BLA_ERR_INVALID;
    const long n = (long)(bytes / 16);
    // enough workgroups to fill every compute unit several times over
    long blocks = (n + kProbeThreads * 4 - 1) / (kProbeThreads * 4);
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(copy_probe_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, (hipStream_t)stream,
                       (const u4 *)src, (u4 *)dst, n);
    return hipGetLastError() == hipSuccess ? BLA_OK : BLA_ERR_HIP;
}

}  // extern "C"
