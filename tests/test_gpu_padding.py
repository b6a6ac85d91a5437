"""GPU parity of jrt_prefix_prefill_ex (left-padded JRT prefixes, "Just read
twice" notes §2.7) against the oracle's jrt_padded.  The padding rows are
filled with NaN: any read of them would poison the outputs.
"""
import numpy as np
import pytest
import torch

import oracle
from recurrent_lm_sequence_amd import inputs as gen
from tests.parity_util import TOL_BF16, TOL_F32, assert_rows, assert_state

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def padded_inputs(B, H, N, M, dv, dtype, seed, lens):
    w = gen.Workload("pad", B=B, H=H, N=N, d_feat=16, d_v=dv, dtype=dtype, seed=seed, M=M)
    q, k, v = gen.make_prefill_inputs(w, DEV)
    ke, ve = gen.make_prefix_inputs(w, DEV)
    ke_nan, ve_nan = ke.clone(), ve.clone()
    for b, m in enumerate(lens):
        ke_nan[b, :, : M - m] = float("nan")
        ve_nan[b, :, : M - m] = float("nan")
    return q, k, v, ke, ve, ke_nan, ve_nan


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("compact", [False, True])
def test_jrt_left_padded_prefix(gpu_lib, dtype, compact):
    print(f"jrt padded {dtype} compact={compact}", flush=True)
    B, H, N, M, dv = 4, 3, 190, 300, 64
    lens = [0, 1, 130, 300]
    q, k, v, ke, ve, ke_nan, ve_nan = padded_inputs(B, H, N, M, dv, dtype, 300, lens)
    plen = torch.tensor(lens, dtype=torch.int32, device=DEV)
    y, S, z = gpu_lib.jrt_prefix_prefill(q, k, v, ke_nan, ve_nan, prefix_len=plen,
                                         compact=compact)
    torch.cuda.synchronize()
    yr, Sr, zr = oracle.jrt_padded(q, k, v, ke, ve, lens, compact=compact)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    assert_rows(y, yr, tol)
    assert_state(S, Sr, tol, "S")
    assert_state(z, zr, tol, "z")


def test_jrt_left_padded_prefix_256_heads(gpu_lib):
    # 16 batch entries x 16 heads take the wave-specialised kernel; valid prefix
    # lengths from 0 to 4 chunks per batch entry (a different prefix chunk count
    # in each workgroup)
    print("jrt padded 256 heads", flush=True)
    B, H, N, M, dv = 16, 16, 150, 512, 64
    lens = [0, 1, 2, 127, 128, 129, 200, 255, 256, 257, 300, 383, 384, 385, 500, 512]
    q, k, v, ke, ve, ke_nan, ve_nan = padded_inputs(B, H, N, M, dv, "bf16", 310, lens)
    plen = torch.tensor(lens, dtype=torch.int32, device=DEV)
    y, S, z = gpu_lib.jrt_prefix_prefill(q, k, v, ke_nan, ve_nan, prefix_len=plen)
    torch.cuda.synchronize()
    yr, Sr, zr = oracle.jrt_padded(q, k, v, ke, ve, lens)
    assert_rows(y, yr, TOL_BF16)
    assert_state(S, Sr, TOL_BF16, "S")
    assert_state(z, zr, TOL_BF16, "z")


def test_jrt_padded_full_lengths_equal_unpadded_call(gpu_lib):
    B, H, N, M, dv = 2, 2, 150, 200, 64
    q, k, v, ke, ve, _, _ = padded_inputs(B, H, N, M, dv, "bf16", 310, [M, M])
    plen = torch.full((B,), M, dtype=torch.int32, device=DEV)
    y1, S1, z1 = gpu_lib.jrt_prefix_prefill(q, k, v, ke, ve, prefix_len=plen)
    y0, S0, z0 = gpu_lib.jrt_prefix_prefill(q, k, v, ke, ve)
    torch.cuda.synchronize()
    assert torch.equal(y1, y0) and torch.equal(S1, S0) and torch.equal(z1, z0)


def test_jrt_padded_lengths_are_clamped(gpu_lib):
    # out-of-range lengths are clamped to [0, M]
    B, H, N, M, dv = 2, 1, 64, 96, 32
    q, k, v, ke, ve, _, _ = padded_inputs(B, H, N, M, dv, "bf16", 320, [M, 0])
    plen = torch.tensor([10 * M, -5], dtype=torch.int32, device=DEV)
    y, S, z = gpu_lib.jrt_prefix_prefill(q, k, v, ke, ve, prefix_len=plen)
    torch.cuda.synchronize()
    yr, Sr, zr = oracle.jrt_padded(q, k, v, ke, ve, [M, 0])
    assert_rows(y, yr, TOL_BF16)
    assert_state(S, Sr, TOL_BF16, "S")
