"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

The GPU runs every head of each workload; the fp64 oracle recomputes all heads
where that takes seconds, and a fixed sample of heads (all tokens of each)
where it would not.  Tolerance and metric: tests/parity_util.py.
"""
import numpy as np
import pytest
import torch

import oracle
from recurrent_lm_sequence_amd import inputs as gen
from tests.parity_util import TOL_BF16, assert_rows, assert_state

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# sampled (b, h) heads: spread over batch and head indices, including the corners
SAMPLE_LONG = [(0, 0), (3, 7), (7, 15), (8, 1), (12, 9), (15, 15)]
SAMPLE_JRT = [(0, 0), (2, 11), (5, 3), (9, 14), (13, 6), (15, 15)]
SAMPLE_DECODE = [(0, 0), (37, 5), (128, 15), (200, 8), (255, 15)]


def take(t, heads):
    """Rows of the sampled heads as one [1, len(heads), ...] host tensor."""
    return torch.stack([t[b, h] for b, h in heads]).unsqueeze(0).cpu()


def test_layer_prefill_all_heads(gpu_lib):
    w = gen.LAYER_PREFILL
    print(f"workload {w}", flush=True)
    q, k, v = gen.make_prefill_inputs(w, DEV)
    y, S, z = gpu_lib.based_prefill(q, k, v)
    torch.cuda.synchronize()
    yr, Sr, zr = oracle.prefill(q, k, v)
    e = assert_rows(y, yr, TOL_BF16)
    assert_state(S, Sr, TOL_BF16, "S")
    assert_state(z, zr, TOL_BF16, "z")
    print(f"worst row error {e:.3e}", flush=True)


def test_long_prefill_sampled_heads(gpu_lib):
    w = gen.LONG_PREFILL
    print(f"workload {w}", flush=True)
    q, k, v = gen.make_prefill_inputs(w, DEV)
    y, S, z = gpu_lib.based_prefill(q, k, v)
    torch.cuda.synchronize()
    yr, Sr, zr = oracle.prefill(take(q, SAMPLE_LONG), take(k, SAMPLE_LONG), take(v, SAMPLE_LONG))
    e = assert_rows(take(y, SAMPLE_LONG), yr, TOL_BF16)
    assert_state(take(S, SAMPLE_LONG), Sr, TOL_BF16, "S")
    assert_state(take(z, SAMPLE_LONG), zr, TOL_BF16, "z")
    print(f"worst row error {e:.3e}", flush=True)


def test_jrt_prefix_sampled_heads(gpu_lib):
    w = gen.JRT_PREFIX
    print(f"workload {w}", flush=True)
    q, k, v = gen.make_prefill_inputs(w, DEV)
    ke, ve = gen.make_prefix_inputs(w, DEV)
    y, S, z = gpu_lib.jrt_prefix_prefill(q, k, v, ke, ve)
    torch.cuda.synchronize()
    sm = SAMPLE_JRT
    yr, Sr, zr = oracle.jrt(take(q, sm), take(k, sm), take(v, sm), take(ke, sm), take(ve, sm))
    e = assert_rows(take(y, sm), yr, TOL_BF16)
    assert_state(take(S, sm), Sr, TOL_BF16, "S")
    assert_state(take(z, sm), zr, TOL_BF16, "z")
    print(f"worst row error {e:.3e}", flush=True)


def test_state_passing_decode_chain_sampled_heads(gpu_lib):
    """GPU: 8192-token prefill -> 512 decode steps, all 4096 heads.  Oracle: the
    same chain from the same seeded inputs for the sampled heads (its own
    prefill state; nothing computed on the GPU enters the oracle)."""
    w = gen.STATE_DECODE
    sm = SAMPLE_DECODE
    print(f"workload {w}", flush=True)
    q, k, v = gen.make_prefill_inputs(w, DEV)
    _, S, z = gpu_lib.based_prefill(q, k, v, want_y=False)
    _, Sr, zr = oracle.prefill(take(q, sm), take(k, sm), take(v, sm))
    del q, k, v
    torch.cuda.empty_cache()
    assert_state(take(S, sm), Sr, TOL_BF16, "S after prefill")
    worst = 0.0
    for step in range(w.decode_steps):
        qd, kd, vd = gen.make_decode_step_inputs(w, step, DEV)
        y = gpu_lib.based_decode_step(qd, kd, vd, S, z)
        yr, Sr, zr = oracle.decode_step(take(qd, sm), take(kd, sm), take(vd, sm), Sr, zr)
        worst = max(worst, assert_rows(take(y, sm), yr, TOL_BF16, f"y step {step}"))
    torch.cuda.synchronize()
    assert_state(take(S, sm), Sr, TOL_BF16, "S after decode")
    assert_state(take(z, sm), zr, TOL_BF16, "z after decode")
    print(f"worst row error over {w.decode_steps} steps {worst:.3e}", flush=True)


@pytest.mark.parametrize("N", [1, 63, 65, 64 * 3 + 17])
def test_ragged_lengths_full_head_count(gpu_lib, N):
    """All 256 heads of the long-prefill shape at short ragged lengths (tail chunk)."""
    w = gen.Workload("ragged", B=16, H=16, N=N, d_feat=16, d_v=64, dtype="bf16", seed=77 + N)
    q, k, v = gen.make_prefill_inputs(w, DEV)
    y, S, z = gpu_lib.based_prefill(q, k, v)
    torch.cuda.synchronize()
    yr, Sr, zr = oracle.prefill(q, k, v)
    assert_rows(y, yr, TOL_BF16)
    assert_state(S, Sr, TOL_BF16, "S")
    assert_state(z, zr, TOL_BF16, "z")
