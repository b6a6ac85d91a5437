/*
 * based_la_probe.h -- peak-rate micro-kernels of libbasedla.so.
 *
 * These are not part of the method.  They measure what the GPU delivers on
 * the two resources the method's kernels are bound by, so that a measured
 * rate can be stated beside the vendor peak: matrix-core throughput on the
 * fp16 16x16x32 product the prefill uses, and HBM bandwidth of a plain
 * 16-byte-vector streaming copy.  (The BASED notes, §4.5, compare efficiency
 * only with the kernel that realises the architecture; these probes give the
 * ceilings a kernel's achieved rate is read against.)
 *
 * Both are asynchronous on `stream` (a hipStream_t passed as void*, NULL =
 * default stream) and return BLA_ERR_INVALID for bad arguments (checked
 * before anything is launched) or BLA_ERR_HIP for a launch error.
 */
#ifndef BASED_LA_PROBE_H
#define BASED_LA_PROBE_H

#include "based_la.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Matrix-core probe: `blocks` workgroups of 256 threads (4 wavefronts); each
 * wavefront issues iters x 8 independent v_mfma_f32_16x16x32_f16 products
 * (16,384 FLOP each) with no memory traffic, then writes one float per thread
 * to sink [blocks * 256] (DEVICE pointer, 4-byte aligned) so that the work is
 * kept.  FLOP per call = blocks * 4 * iters * 8 * 16384.
 * 1 <= blocks <= 65536, 1 <= iters <= 1048576. */
bla_status bla_probe_mfma_f16(int blocks, int iters, float *sink, void *stream);

/* HBM probe: copies `bytes` bytes from src to dst (DEVICE pointers, 16-byte
 * aligned, not overlapping; bytes a positive multiple of 16) with 16-byte
 * vector loads and stores, four in flight per thread.  Bytes moved per call =
 * 2 * bytes (read + write). */
bla_status bla_probe_copy(const void *src, void *dst, long long bytes, void *stream);

/* Prefill-traffic probe: the HBM traffic of a bf16-input, fp32-output prefill
 * over `heads` heads of N tokens (d' = 16, d_v = 64) with none of its
 * arithmetic.  One workgroup per head walks the tokens in chunks of 128, reads
 * q, k [heads][N][16] and v [heads][N][64] (bf16, 192 B per token) two chunks
 * ahead and writes y [heads][N][64] (fp32, 256 B per token, whole rows), with
 * one workgroup barrier per chunk.  Its time is the floor the memory system
 * sets for that traffic when each head is streamed by one compute unit.
 *   mode 0: reads and writes; 1: reads only; 2: writes only.
 *   sink: DEVICE float [heads * 512] (keeps the loaded data live).
 *   Pointers 16-byte aligned (sink 4-byte); y must not overlap the inputs.
 *   N * 256 below 2^31; 1 <= heads <= 2^22. */
bla_status bla_probe_prefill_traffic(int heads, int N, const void *q, const void *k, const void *v, void *y,
                                     float *sink, int mode, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BASED_LA_PROBE_H */
