"""GPU parity of the compact-state entry points (based_prefill_compact,
jrt_prefix_prefill_compact, based_decode_step_compact) against the fp64
oracle's compact wrappers (oracle/compact.py: fold / unfold around the
token-by-token recurrence).  Compact initial states given to the GPU are
folds of oracle states; nothing the GPU computes becomes an oracle input.
"""
import numpy as np
import pytest
import torch

import oracle
from recurrent_lm_sequence_amd import inputs as gen
from tests.parity_util import TOL_BF16, TOL_F32, assert_rows, assert_state

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
D_FEAT = 16


def small(B, H, N, dv, seed, dtype="bf16", M=0):
    w = gen.Workload("small", B=B, H=H, N=N, d_feat=D_FEAT, d_v=dv, dtype=dtype, seed=seed, M=M)
    q, k, v = gen.make_prefill_inputs(w, DEV)
    if M:
        ke, ve = gen.make_prefix_inputs(w, DEV)
        return q, k, v, ke, ve
    return q, k, v


def compact_state(B, H, dv, seed, noise=0.5):
    """Fold of an oracle prefill state plus seeded non-symmetric noise, as fp32."""
    w = gen.Workload("init", B=B, H=H, N=96, d_feat=D_FEAT, d_v=dv, dtype="bf16", seed=seed)
    q, k, v = gen.make_prefill_inputs(w, "cpu")
    _, S, z = oracle.prefill(q, k, v)
    nS, nz = gen.state_noise(B, H, S.shape[2], dv, seed + 1)
    S = S + noise * nS.double().numpy()
    z = z + noise * np.abs(nz.double().numpy())
    Sc = torch.tensor(oracle.fold(S, D_FEAT, axis=-2), dtype=torch.float32)
    zc = torch.tensor(oracle.fold(z, D_FEAT, axis=-1), dtype=torch.float32)
    return Sc.to(DEV), zc.to(DEV), Sc.double().numpy(), zc.double().numpy()


@pytest.mark.parametrize("dv", [16, 32, 64])
@pytest.mark.parametrize("N", [37, 300])
def test_prefill_compact_bf16(gpu_lib, dv, N):
    print(f"prefill compact bf16 dv={dv} N={N}", flush=True)
    q, k, v = small(2, 3, N, dv, seed=200 + N + dv)
    y, S, z = gpu_lib.based_prefill(q, k, v, compact=True)
    torch.cuda.synchronize()
    assert S.shape[2] == 153 and z.shape[2] == 153
    yr, Sr, zr = oracle.prefill_compact(q, k, v)
    assert_rows(y, yr, TOL_BF16)
    assert_state(S, Sr, TOL_BF16, "S")
    assert_state(z, zr, TOL_BF16, "z")


def test_prefill_compact_bf16_column_split_and_initial_state(gpu_lib):
    # 40 heads at d_v = 64: several column blocks per head read the compact S0
    print("prefill compact bf16 column split + S0", flush=True)
    q, k, v = small(5, 8, 200, 64, seed=231)
    S0, z0, S0r, z0r = compact_state(5, 8, 64, seed=232)
    y, S, z = gpu_lib.based_prefill(q, k, v, S0, z0, compact=True)
    torch.cuda.synchronize()
    yr, Sr, zr = oracle.prefill_compact(q, k, v, S0r, z0r)
    assert_rows(y, yr, TOL_BF16)
    assert_state(S, Sr, TOL_BF16, "S")
    assert_state(z, zr, TOL_BF16, "z")


def test_prefill_compact_bf16_in_place_split_resume(gpu_lib):
    print("prefill compact bf16 in place / split-resume", flush=True)
    q, k, v = small(2, 2, 250, 64, seed=233)
    yr, Sr, zr = oracle.prefill_compact(q, k, v)
    S = torch.zeros((2, 2, 153, 64), device=DEV)
    z = torch.zeros((2, 2, 153), device=DEV)
    parts = []
    for a, b in [(0, 100), (100, 250)]:
        ys, _, _ = gpu_lib.based_prefill(q[:, :, a:b].contiguous(), k[:, :, a:b].contiguous(),
                                         v[:, :, a:b].contiguous(), S, z, S_out=S, z_out=z,
                                         compact=True)
        parts.append(ys)
    torch.cuda.synchronize()
    assert_rows(torch.cat(parts, dim=2), yr, TOL_BF16)
    assert_state(S, Sr, TOL_BF16, "S")
    assert_state(z, zr, TOL_BF16, "z")


def test_prefill_compact_same_outputs_as_full_layout(gpu_lib):
    # same inputs, zero state: the compact call runs the same kernel -> identical y;
    # its final state is the fold of the full one
    q, k, v = small(2, 4, 190, 64, seed=234)
    yf, Sf, zf = gpu_lib.based_prefill(q, k, v)
    yc, Sc, zc = gpu_lib.based_prefill(q, k, v, compact=True)
    torch.cuda.synchronize()
    assert torch.equal(yf, yc)
    assert_state(Sc, oracle.fold(Sf.double().cpu().numpy(), D_FEAT, axis=-2), 1e-6, "S")
    assert_state(zc, oracle.fold(zf.double().cpu().numpy(), D_FEAT, axis=-1), 1e-6, "z")


@pytest.mark.parametrize("dv", [16, 64])
def test_prefill_compact_f32_exact(gpu_lib, dv):
    print(f"prefill compact f32 dv={dv}", flush=True)
    q, k, v = small(2, 2, 133, dv, seed=240 + dv, dtype="f32")
    S0, z0, S0r, z0r = compact_state(2, 2, dv, seed=241)
    y, S, z = gpu_lib.based_prefill(q, k, v, S0, z0, compact=True)
    torch.cuda.synchronize()
    yr, Sr, zr = oracle.prefill_compact(q, k, v, S0r, z0r)
    assert_rows(y, yr, TOL_F32)
    assert_state(S, Sr, TOL_F32, "S")
    assert_state(z, zr, TOL_F32, "z")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_jrt_compact(gpu_lib, dtype):
    print(f"jrt compact {dtype}", flush=True)
    q, k, v, ke, ve = small(2, 2, 170, 64, seed=250, dtype=dtype, M=90)
    S0, z0, S0r, z0r = compact_state(2, 2, 64, seed=251)
    y, S, z = gpu_lib.jrt_prefix_prefill(q, k, v, ke, ve, S0, z0, compact=True)
    torch.cuda.synchronize()
    yr, Sr, zr = oracle.jrt_compact(q, k, v, ke, ve, S0r, z0r)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    assert_rows(y, yr, tol)
    assert_state(S, Sr, tol, "S")
    assert_state(z, zr, tol, "z")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dv", [16, 32, 64])
def test_decode_compact_steps(gpu_lib, dtype, dv):
    print(f"decode compact {dtype} dv={dv}", flush=True)
    B, H, steps = 3, 5, 6
    S, z, Sr, zr = compact_state(B, H, dv, seed=260 + dv)
    w = gen.Workload("dec", B=B, H=H, N=steps, d_feat=D_FEAT, d_v=dv, dtype=dtype, seed=261 + dv)
    q, k, v = gen.make_prefill_inputs(w, DEV)
    for i in range(steps):
        qi, ki, vi = (t[:, :, i].contiguous() for t in (q, k, v))
        y = gpu_lib.based_decode_step(qi, ki, vi, S, z, compact=True)
        torch.cuda.synchronize()
        yr, Sr, zr = oracle.decode_step_compact(qi, ki, vi, Sr, zr)
        # all-fp32 arithmetic on exact inputs (as the full-layout decode test)
        assert_rows(y, yr, 2e-5)
    assert_state(S, Sr, 2e-6, "S")
    assert_state(z, zr, 2e-6, "z")


def test_decode_compact_after_jrt_compact(gpu_lib):
    # state passing in the compact layout: JRT prefill, then decode steps on its merged state
    q, k, v, ke, ve = small(2, 2, 100, 64, seed=280, M=64)
    _, S, z = gpu_lib.jrt_prefix_prefill(q, k, v, ke, ve, compact=True)
    _, Sr, zr = oracle.jrt_compact(q, k, v, ke, ve)
    wd = gen.Workload("dec", B=2, H=2, N=0, d_feat=D_FEAT, d_v=64, dtype="bf16", seed=281)
    for step in range(3):
        qd, kd, vd = gen.make_decode_step_inputs(wd, step, DEV)
        y = gpu_lib.based_decode_step(qd, kd, vd, S, z, compact=True)
        torch.cuda.synchronize()
        yr, Sr, zr = oracle.decode_step_compact(qd, kd, vd, Sr, zr)
        assert_rows(y, yr, TOL_BF16)


def test_compact_entry_points_reject_bad_arguments(gpu_lib):
    q, k, v = small(1, 1, 8, 64, seed=270)
    with pytest.raises(gpu_lib.BlaError):
        # S0 without z0
        S0 = torch.zeros((1, 1, 153, 64), device=DEV)
        gpu_lib.based_prefill(q, k, v, S0, None, compact=True)
