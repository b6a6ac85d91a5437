"""GPU parity of the sliding-window softmax attention kernels (swa_prefill,
swa_decode_step) against the fp64 oracle (oracle/swa.py) on seeded inputs.
"""
import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch
from threadpoolctl import threadpool_limits

import oracle
from recurrent_lm_sequence_amd import inputs as gen
from tests.parity_util import TOL_BF16, assert_rows, worst_row_error

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def swa_inputs(B, H, N, seed, dtype="bf16", device=DEV):
    w = gen.Workload("swa", B=B, H=H, N=N, d_feat=64, d_v=64, dtype=dtype, seed=seed)
    return gen.make_prefill_inputs(w, device)


@pytest.mark.parametrize("window", [1, 16, 64, 100, 128, 200, 256])
@pytest.mark.parametrize("N", [1, 37, 130, 300])
def test_swa_prefill(gpu_lib, window, N):
    print(f"swa prefill w={window} N={N}", flush=True)
    q, k, v = swa_inputs(2, 3, N, seed=400 + window + N)
    y, kc, vc = gpu_lib.swa_prefill(q, k, v, window, want_cache=True)
    torch.cuda.synchronize()
    yr = oracle.swa_prefill(q.double().cpu().numpy(), k.double().cpu().numpy(),
                            v.double().cpu().numpy(), window)
    assert_rows(y, yr, TOL_BF16)
    kr, vr = oracle.swa_cache_from_prefill(k.double().cpu().numpy(), v.double().cpu().numpy(), window)
    assert np.array_equal(kc.double().cpu().numpy(), kr)
    assert np.array_equal(vc.double().cpu().numpy(), vr)


@pytest.mark.parametrize("window", [64, 128])
def test_swa_prefill_and_decode_large_scores(gpu_lib, window):
    # q and k scaled by 8 (a power of two: the bf16 values stay exact): the scaled scores
    # q.k / 8 reach about +-100, so the softmax weights are nearly one-hot and exercise the
    # max subtraction and the fp16 weights at their extremes
    print(f"swa large scores w={window}", flush=True)
    q, k, v = swa_inputs(2, 3, 300, seed=470 + window)
    q, k = q * 8, k * 8
    y, kc, vc = gpu_lib.swa_prefill(q, k, v, window, want_cache=True)
    torch.cuda.synchronize()
    qd, kd, vd = (t.double().cpu().numpy() for t in (q, k, v))
    assert_rows(y, oracle.swa_prefill(qd, kd, vd, window), TOL_BF16)
    # one decode step (token 300, reusing token 299's large q and k) on the prefill's cache,
    # against the oracle's step on the oracle's cache
    qs, ks, vs = q[:, :, -1].contiguous(), k[:, :, -1].contiguous(), v[:, :, -1].contiguous()
    yd = gpu_lib.swa_decode_step(qs, ks, vs, kc, vc, 300, window)
    torch.cuda.synchronize()
    kr, vr = oracle.swa_cache_from_prefill(kd, vd, window)
    ydr, _, _ = oracle.swa_decode_step(qs.double().cpu().numpy(), ks.double().cpu().numpy(),
                                       vs.double().cpu().numpy(), kr, vr, 300, window)
    assert_rows(yd, ydr, TOL_BF16)


@pytest.mark.parametrize("window", [1, 17, 64, 100, 128])
def test_swa_prefill_tile_walk_all_heads(gpu_lib, window):
    # 256 heads of 4 full 128-query tiles and a ragged tail: at this head count a
    # workgroup walks a run of consecutive tiles of one head, one run starting
    # mid-sequence; every head and row is compared, and the ring cache
    B, H, N = 4, 64, 4 * 128 + 77
    print(f"swa tile walk w={window} B={B} H={H} N={N}", flush=True)
    q, k, v = swa_inputs(B, H, N, seed=480 + window)
    y, kc, vc = gpu_lib.swa_prefill(q, k, v, window, want_cache=True)
    torch.cuda.synchronize()
    qd, kd, vd = (t.double().cpu().numpy() for t in (q, k, v))
    e = assert_rows(y, oracle.swa_prefill(qd, kd, vd, window), TOL_BF16)
    kr, vr = oracle.swa_cache_from_prefill(kd, vd, window)
    assert np.array_equal(kc.double().cpu().numpy(), kr)
    assert np.array_equal(vc.double().cpu().numpy(), vr)
    print(f"worst row error {e:.3e}", flush=True)


def test_swa_prefill_many_heads_bf16_output(gpu_lib):
    q, k, v = swa_inputs(3, 8, 257, seed=450)
    y, _, _ = gpu_lib.swa_prefill(q, k, v, 128, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    yr = oracle.swa_prefill(q.double().cpu().numpy(), k.double().cpu().numpy(),
                            v.double().cpu().numpy(), 128)
    # bf16 rounding of the output (8 significant bits) adds up to 2^-8 of a row's largest entry
    assert_rows(y, yr, TOL_BF16 + 2.0 ** -8)


@pytest.mark.parametrize("window", [16, 64, 256])
def test_swa_decode_continues_prefill(gpu_lib, window):
    # prefill N tokens (cache out), then decode steps that wrap the ring
    print(f"swa decode after prefill w={window}", flush=True)
    B, H, N, n = 2, 3, 150, 2 * window + 3 if window < 64 else 5
    q, k, v = swa_inputs(B, H, N + n, seed=460 + window)
    _, kc, vc = gpu_lib.swa_prefill(q[:, :, :N].contiguous(), k[:, :, :N].contiguous(),
                                    v[:, :, :N].contiguous(), window, want_cache=True)
    qn, kn, vn = (t.double().cpu().numpy() for t in (q, k, v))
    kr, vr = oracle.swa_cache_from_prefill(kn[:, :, :N], vn[:, :, :N], window)
    for p in range(N, N + n):
        y = gpu_lib.swa_decode_step(q[:, :, p].contiguous(), k[:, :, p].contiguous(),
                                    v[:, :, p].contiguous(), kc, vc, p, window)
        torch.cuda.synchronize()
        yr, kr, vr = oracle.swa_decode_step(qn[:, :, p], kn[:, :, p], vn[:, :, p], kr, vr, p, window)
        assert_rows(y, yr, 1e-5)
    assert np.array_equal(kc.double().cpu().numpy(), kr)
    assert np.array_equal(vc.double().cpu().numpy(), vr)


@pytest.mark.parametrize("w", [8, 100, 200])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_swa_decode_from_empty_cache(gpu_lib, dtype, w):
    # positions 0..w+2 from an empty ring: the first steps see fewer than w tokens;
    # the windows reach the three launch shapes (4, 2 and 1 threads per cache slot)
    B, H = 2, 2
    q, k, v = swa_inputs(B, H, w + 3, seed=470, dtype=dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kc = torch.zeros((B, H, w, 64), dtype=tdt, device=DEV)
    vc = torch.zeros((B, H, w, 64), dtype=tdt, device=DEV)
    qn, kn, vn = (t.double().cpu().numpy() for t in (q, k, v))
    yr_all = oracle.swa_prefill(qn, kn, vn, w)
    for p in range(w + 3):
        y = gpu_lib.swa_decode_step(q[:, :, p].contiguous(), k[:, :, p].contiguous(),
                                    v[:, :, p].contiguous(), kc, vc, p, w)
        torch.cuda.synchronize()
        assert_rows(y, yr_all[:, :, p], 1e-5)


# full sizes, in the launch configuration bench.py times


@pytest.mark.parametrize("window", [64, 128])
def test_swa_prefill_long_prefill_all_heads(gpu_lib, record_parity, window):
    """B=16, H=16, N=32768: every head and row against the oracle's blocked form
    (pinned to the per-row form), one batch entry at a time."""
    print(f"swa long prefill B=16 H=16 N=32768 w={window}", flush=True)
    q, k, v = swa_inputs(16, 16, 32768, seed=1200)
    y = torch.empty((16, 16, 32768, 64), dtype=torch.float32, device=DEV)
    gpu_lib.swa_prefill(q, k, v, window, y=y)
    torch.cuda.synchronize()
    qc, kc, vc, yc = (t.cpu() for t in (q, k, v, y))

    def batch_error(b):
        qd, kd, vd = (t[b].double().numpy() for t in (qc, kc, vc))
        return worst_row_error(yc[b:b + 1], oracle.swa_prefill_blocked(qd, kd, vd, window, block=128)[None])

    # one BLAS thread per worker: the products are small, and nested BLAS threads
    # oversubscribe the host many times over
    with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        errs = list(ex.map(batch_error, range(16)))
    assert np.all(np.isfinite(yc.numpy()))
    worst = max(errs)
    print(f"worst row error {worst:.3e}", flush=True)
    assert worst <= TOL_BF16, f"worst row error {worst:.3e} (batch {int(np.argmax(errs))}) > {TOL_BF16:.1e}"
    record_parity(f"swa prefill w={window} B=16 H=16 N=32768 (all 256 heads)", worst, TOL_BF16)


def test_swa_decode_full_size_all_heads(gpu_lib):
    # B=256, H=16, window 128: ring cache from a 128-token prefill, then steps that
    # overwrite slots 0, 1, 2; every head against the oracle, cache included
    B, H, w = 256, 16, 128
    print(f"swa decode B={B} H={H} w={w}", flush=True)
    q, k, v = swa_inputs(B, H, w + 3, seed=1201)
    _, kc, vc = gpu_lib.swa_prefill(q[:, :, :w].contiguous(), k[:, :, :w].contiguous(),
                                    v[:, :, :w].contiguous(), w, want_cache=True)
    qn, kn, vn = (t.double().cpu().numpy() for t in (q, k, v))
    kr, vr = oracle.swa_cache_from_prefill(kn[:, :, :w], vn[:, :, :w], w)
    worst = 0.0
    for p in range(w, w + 3):
        y = gpu_lib.swa_decode_step(q[:, :, p].contiguous(), k[:, :, p].contiguous(),
                                    v[:, :, p].contiguous(), kc, vc, p, w)
        torch.cuda.synchronize()
        yr, kr, vr = oracle.swa_decode_step(qn[:, :, p], kn[:, :, p], vn[:, :, p], kr, vr, p, w)
        worst = max(worst, assert_rows(y, yr, 1e-5))
    assert np.array_equal(kc.double().cpu().numpy(), kr)
    assert np.array_equal(vc.double().cpu().numpy(), vr)
    print(f"worst row error {worst:.3e}", flush=True)


def test_swa_prefill_million_tokens_per_head(gpu_lib):
    # maximum-size edge: 2^20 + 37 tokens in one head; rows at the start, the middle and
    # the end against the oracle on the same rows with the w - 1 keys before them
    N, w, L = (1 << 20) + 37, 128, 300
    print(f"swa prefill N={N} w={w}", flush=True)
    q, k, v = swa_inputs(1, 1, N, seed=480)
    y, kc, vc = gpu_lib.swa_prefill(q, k, v, w, want_cache=True)
    torch.cuda.synchronize()
    qn, kn, vn = (t[0, 0].double().cpu().numpy() for t in (q, k, v))
    for a in (0, N // 2 + 3, N - L):
        lo = max(0, a - w + 1)
        yr = oracle.swa_prefill(qn[lo:a + L], kn[lo:a + L], vn[lo:a + L], w)[a - lo:]
        assert_rows(y[0, 0, a:a + L], yr, TOL_BF16)
    kr, vr = oracle.swa_cache_from_prefill(kn, vn, w)
    assert np.array_equal(kc[0, 0].double().cpu().numpy(), kr)
    assert np.array_equal(vc[0, 0].double().cpu().numpy(), vr)


def test_swa_prefill_zero_tokens_and_cache_only(gpu_lib):
    # N = 0 is a no-op that leaves the caches untouched; y = NULL with caches writes only them
    q, k, v = swa_inputs(2, 2, 0, seed=490)
    kc = torch.full((2, 2, 16, 64), 7.0, dtype=torch.bfloat16, device=DEV)
    vc = torch.full((2, 2, 16, 64), 7.0, dtype=torch.bfloat16, device=DEV)
    P = ctypes.c_void_p
    st = gpu_lib.lib.swa_prefill(2, 2, 0, 64, 64, 16, gpu_lib.BLA_BF16, gpu_lib.BLA_F32, None, None,
                                 None, None, P(kc.data_ptr()), P(vc.data_ptr()), None)
    torch.cuda.synchronize()
    assert st == gpu_lib.BLA_OK and bool((kc == 7).all()) and bool((vc == 7).all())
    q, k, v = swa_inputs(2, 2, 40, seed=491)
    st = gpu_lib.lib.swa_prefill(2, 2, 40, 64, 64, 16, gpu_lib.BLA_BF16, gpu_lib.BLA_F32,
                                 P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()), None,
                                 P(kc.data_ptr()), P(vc.data_ptr()), None)
    torch.cuda.synchronize()
    assert st == gpu_lib.BLA_OK
    kr, vr = oracle.swa_cache_from_prefill(k.double().cpu().numpy(), v.double().cpu().numpy(), 16)
    assert np.array_equal(kc.double().cpu().numpy(), kr)
    assert np.array_equal(vc.double().cpu().numpy(), vr)
