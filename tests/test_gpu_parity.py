"""GPU parity: the HIP kernels, called through the C ABI, against the fp64 oracle.

Inputs come from the seeded generator (recurrent_lm_sequence_amd.inputs) and
are fed unchanged to both sides.  Initial states given to the GPU are either
zero or produced by the oracle; nothing the GPU computes ever becomes an
oracle input.  Tolerances and the row-wise metric: tests/parity_util.py.
"""
import numpy as np
import pytest
import torch

import oracle
from recurrent_lm_sequence_amd import inputs as gen
from tests.parity_util import TOL_BF16, TOL_F32, assert_rows, assert_state

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def small(B, H, N, dv, seed, dtype="bf16", M=0):
    w = gen.Workload("small", B=B, H=H, N=N, d_feat=16, d_v=dv, dtype=dtype, seed=seed, M=M)
    q, k, v = gen.make_prefill_inputs(w, DEV)
    if M:
        ke, ve = gen.make_prefix_inputs(w, DEV)
        return w, q, k, v, ke, ve
    return w, q, k, v


def oracle_state(B, H, dv, seed, N=96, noise=0.0):
    """A physical initial state from an oracle prefill of seeded tokens, optionally
    plus seeded noise (non-symmetric order-2 block)."""
    w = gen.Workload("init", B=B, H=H, N=N, d_feat=16, d_v=dv, dtype="bf16", seed=seed)
    q, k, v = gen.make_prefill_inputs(w, "cpu")
    _, S, z = oracle.prefill(q, k, v)
    if noise:
        nS, nz = gen.state_noise(B, H, S.shape[2], dv, seed + 1)
        S = S + noise * nS.double().numpy()
        z = z + noise * np.abs(nz.double().numpy())
    S32 = torch.tensor(S, dtype=torch.float32)
    z32 = torch.tensor(z, dtype=torch.float32)
    return S32.to(DEV), z32.to(DEV), S32.double().numpy(), z32.double().numpy()


# ---------------- BASED prefill, bf16 (fp16-MFMA kernel) ----------------

@pytest.mark.parametrize("dv", [16, 32, 64])
@pytest.mark.parametrize("N", [1, 37, 64, 357])
def test_prefill_bf16_small(gpu_lib, dv, N):
    print(f"prefill bf16 dv={dv} N={N}", flush=True)
    w, q, k, v = small(2, 3, N, dv, seed=10 + N + dv)
    y, S, z = gpu_lib.based_prefill(q, k, v)
    torch.cuda.synchronize()
    yr, Sr, zr = oracle.prefill(q, k, v)
    assert_rows(y, yr, TOL_BF16)
    assert_state(S, Sr, TOL_BF16, "S")
    assert_state(z, zr, TOL_BF16, "z")


@pytest.mark.parametrize("dv", [32, 64])
def test_prefill_bf16_many_heads_column_split(gpu_lib, dv):
    # 40 heads -> several column blocks per head; 40 is not a multiple of 8
    print(f"prefill bf16 column split dv={dv}", flush=True)
    w, q, k, v = small(5, 8, 200, dv, seed=30 + dv)
    y, S, z = gpu_lib.based_prefill(q, k, v)
    torch.cuda.synchronize()
    yr, Sr, zr = oracle.prefill(q, k, v)
    assert_rows(y, yr, TOL_BF16)
    assert_state(S, Sr, TOL_BF16, "S")
    assert_state(z, zr, TOL_BF16, "z")


def test_prefill_bf16_large_magnitudes_within_documented_range(gpu_lib):
    # q, k scaled by 8 and v by 128 (powers of two: the bf16 values stay exact and both sides
    # see the same inputs).  |q.k| then has a standard deviation of 256, and the per-entry
    # sums are ~4e6 (sum |k_a k_b v_c|) and ~6.5e5 (sum |k_a v_c|): inside the range
    # include/based_la.h documents for the fp16 operands of the bf16 path
    print("prefill bf16 large magnitudes", flush=True)
    w, q, k, v = small(2, 4, 1000, 64, seed=91)
    q, k, v = q * 8, k * 8, v * 128
    y, S, z = gpu_lib.based_prefill(q, k, v)
    torch.cuda.synchronize()
    yr, Sr, zr = oracle.prefill(q, k, v)
    assert_rows(y, yr, TOL_BF16)
    assert_state(S, Sr, TOL_BF16, "S")
    assert_state(z, zr, TOL_BF16, "z")


@pytest.mark.parametrize("noise", [0.0, 0.5])
def test_prefill_bf16_initial_state(gpu_lib, noise):
    print(f"prefill bf16 initial state noise={noise}", flush=True)
    w, q, k, v = small(2, 4, 300, 64, seed=41)
    S0, z0, S0r, z0r = oracle_state(2, 4, 64, seed=42, noise=noise)
    y, S, z = gpu_lib.based_prefill(q, k, v, S0, z0)
    torch.cuda.synchronize()
    yr, Sr, zr = oracle.prefill(q, k, v, S0r, z0r)
    assert_rows(y, yr, TOL_BF16)
    assert_state(S, Sr, TOL_BF16, "S")
    assert_state(z, zr, TOL_BF16, "z")


@pytest.mark.parametrize("dv", [16, 32, 64])
def test_prefill_bf16_in_place_state_and_split_resume(gpu_lib, dv):
    print(f"prefill bf16 in place / split-resume, d_v={dv}", flush=True)
    w, q, k, v = small(2, 2, 250, dv, seed=43)
    yr, Sr, zr = oracle.prefill(q, k, v)
    D = 273
    S = torch.zeros((2, 2, D, dv), device=DEV)
    z = torch.zeros((2, 2, D), device=DEV)
    ya, _, _ = gpu_lib.based_prefill(q[:, :, :100].contiguous(), k[:, :, :100].contiguous(),
                                     v[:, :, :100].contiguous(), S, z, S_out=S, z_out=z)
    yb, _, _ = gpu_lib.based_prefill(q[:, :, 100:].contiguous(), k[:, :, 100:].contiguous(),
                                     v[:, :, 100:].contiguous(), S, z, S_out=S, z_out=z)
    torch.cuda.synchronize()
    assert_rows(torch.cat([ya, yb], dim=2), yr, TOL_BF16)
    assert_state(S, Sr, TOL_BF16, "S")
    assert_state(z, zr, TOL_BF16, "z")


@pytest.mark.parametrize("dv", [16, 32, 64])
@pytest.mark.parametrize("B,H", [(2, 2), (8, 16)])
def test_prefill_bf16_state_in_place_z_separate(gpu_lib, B, H, dv):
    # S_out == S0 with a separate z_out: with 128 heads or fewer 64 or 32 value columns
    # go to two workgroups per head, each reading and then writing only its own columns
    # of the state in place, and only column block 0 writing z; split-resume over 300 + 213
    print(f"prefill bf16 S in place, z separate, B={B} H={H} d_v={dv}", flush=True)
    w, q, k, v = small(B, H, 513, dv, seed=47 + H)
    S0, z0, S0r, z0r = oracle_state(B, H, dv, seed=48 + H, noise=0.2)
    yr, Sr, zr = oracle.prefill(q, k, v, S0r, z0r)
    S = S0.clone()
    z1 = torch.empty_like(z0)
    ya, _, _ = gpu_lib.based_prefill(q[:, :, :300].contiguous(), k[:, :, :300].contiguous(),
                                     v[:, :, :300].contiguous(), S, z0, S_out=S, z_out=z1)
    z2 = torch.empty_like(z0)
    yb, _, _ = gpu_lib.based_prefill(q[:, :, 300:].contiguous(), k[:, :, 300:].contiguous(),
                                     v[:, :, 300:].contiguous(), S, z1, S_out=S, z_out=z2)
    torch.cuda.synchronize()
    assert_rows(torch.cat([ya, yb], dim=2), yr, TOL_BF16)
    assert_state(S, Sr, TOL_BF16, "S")
    assert_state(z2, zr, TOL_BF16, "z")


def test_prefill_bf16_output_only_and_state_only(gpu_lib):
    w, q, k, v = small(1, 4, 130, 64, seed=44)
    y_full, S_full, z_full = gpu_lib.based_prefill(q, k, v)
    y_only, S_none, z_none = gpu_lib.based_prefill(q, k, v, want_state=False)
    y_none, S_only, z_only = gpu_lib.based_prefill(q, k, v, want_y=False)
    torch.cuda.synchronize()
    assert S_none is None and y_none is None
    assert torch.equal(y_only, y_full)
    assert torch.equal(S_only, S_full) and torch.equal(z_only, z_full)


def test_prefill_bf16_bf16_output(gpu_lib):
    w, q, k, v = small(2, 2, 150, 64, seed=45)
    y, _, _ = gpu_lib.based_prefill(q, k, v, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    yr, _, _ = oracle.prefill(q, k, v)
    # bf16 rounding of the output (8 significant bits) adds up to 2^-8 of a row's largest
    # entry on top of the kernel error
    assert_rows(y, yr, TOL_BF16 + 2.0 ** -8)


def test_prefill_bf16_zero_tokens_copies_state(gpu_lib):
    S0, z0, S0r, z0r = oracle_state(1, 2, 64, seed=46)
    q = torch.empty((1, 2, 0, 16), dtype=torch.bfloat16, device=DEV)
    v = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device=DEV)
    y, S, z = gpu_lib.based_prefill(q, q, v, S0, z0)
    torch.cuda.synchronize()
    assert_state(S, S0r, 1e-6, "S")
    assert_state(z, z0r, 1e-6, "z")


def test_prefill_bf16_deterministic(gpu_lib):
    w, q, k, v = small(2, 4, 333, 64, seed=47)
    y1, S1, z1 = gpu_lib.based_prefill(q, k, v)
    y2, S2, z2 = gpu_lib.based_prefill(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(S1, S2) and torch.equal(z1, z2)


def test_prefill_bf16_eps(gpu_lib):
    w, q, k, v = small(1, 2, 90, 64, seed=48)
    y, _, _ = gpu_lib.based_prefill(q, k, v, eps=3.0)
    torch.cuda.synchronize()
    yr, _, _ = oracle.prefill(q, k, v, eps=3.0)
    assert_rows(y, yr, TOL_BF16)


# ---------------- JRT prefix ----------------

@pytest.mark.parametrize("M,N", [(1, 1), (100, 200), (128, 64), (77, 333)])
def test_jrt_bf16_small(gpu_lib, M, N):
    print(f"jrt bf16 M={M} N={N}", flush=True)
    w, q, k, v, ke, ve = small(2, 3, N, 64, seed=50 + M, M=M)
    y, S, z = gpu_lib.jrt_prefix_prefill(q, k, v, ke, ve)
    torch.cuda.synchronize()
    yr, Sr, zr = oracle.jrt(q, k, v, ke, ve)
    assert_rows(y, yr, TOL_BF16)
    assert_state(S, Sr, TOL_BF16, "S")
    assert_state(z, zr, TOL_BF16, "z")


@pytest.mark.parametrize("M", [1, 128, 200, 300, 511])
def test_jrt_short_prefixes_256_heads(gpu_lib, M):
    # one workgroup per head: the token waves stage the prefix chunks and the state
    # waves take the staging over with causal chunk 1; prefixes of one to four chunks
    # reach every hand-over between the prefix walk and the causal loop
    print(f"jrt bf16 256 heads M={M}", flush=True)
    w, q, k, v, ke, ve = small(16, 16, 300, 64, seed=700 + M, M=M)
    y, S, z = gpu_lib.jrt_prefix_prefill(q, k, v, ke, ve)
    torch.cuda.synchronize()
    yr, Sr, zr = oracle.jrt(q, k, v, ke, ve)
    assert_rows(y, yr, TOL_BF16)
    assert_state(S, Sr, TOL_BF16, "S")
    assert_state(z, zr, TOL_BF16, "z")


def test_jrt_bf16_with_initial_state(gpu_lib):
    w, q, k, v, ke, ve = small(2, 2, 170, 32, seed=60, M=90)
    S0, z0, S0r, z0r = oracle_state(2, 2, 32, seed=61, noise=0.3)
    y, S, z = gpu_lib.jrt_prefix_prefill(q, k, v, ke, ve, S0, z0)
    torch.cuda.synchronize()
    yr, Sr, zr = oracle.jrt(q, k, v, ke, ve, S0r, z0r)
    assert_rows(y, yr, TOL_BF16)
    assert_state(S, Sr, TOL_BF16, "S")
    assert_state(z, zr, TOL_BF16, "z")


@pytest.mark.parametrize("dv", [16, 32, 64])
@pytest.mark.parametrize("B,H", [(2, 3), (8, 16)])
def test_jrt_bf16_in_place_state(gpu_lib, B, H, dv):
    # a JRT prefix with the state updated in place (S and z): no split of any kind, one
    # workgroup per head whatever the head count
    print(f"jrt bf16 in place B={B} H={H} d_v={dv}", flush=True)
    w, q, k, v, ke, ve = small(B, H, 301, dv, seed=64 + dv, M=260)
    S0, z0, S0r, z0r = oracle_state(B, H, dv, seed=65 + dv, noise=0.2)
    yr, Sr, zr = oracle.jrt(q, k, v, ke, ve, S0r, z0r)
    S, z = S0.clone(), z0.clone()
    y, _, _ = gpu_lib.jrt_prefix_prefill(q, k, v, ke, ve, S, z, S_out=S, z_out=z)
    torch.cuda.synchronize()
    assert_rows(y, yr, TOL_BF16)
    assert_state(S, Sr, TOL_BF16, "S")
    assert_state(z, zr, TOL_BF16, "z")


def test_jrt_without_prefix_is_based_prefill(gpu_lib):
    w, q, k, v = small(2, 2, 140, 64, seed=62)
    ke = torch.empty((2, 2, 0, 16), dtype=torch.bfloat16, device=DEV)
    ve = torch.empty((2, 2, 0, 64), dtype=torch.bfloat16, device=DEV)
    y1, S1, z1 = gpu_lib.jrt_prefix_prefill(q, k, v, ke, ve)
    y2, S2, z2 = gpu_lib.based_prefill(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(S1, S2) and torch.equal(z1, z2)


# ---------------- fp32 inputs (fp64-accumulating precision kernel) ----------------

def test_tiny_f32_workload(gpu_lib):
    w = gen.TINY_F32
    q, k, v = gen.make_prefill_inputs(w, DEV)
    y, S, z = gpu_lib.based_prefill(q, k, v)
    torch.cuda.synchronize()
    yr, Sr, zr = oracle.prefill(q, k, v)
    assert y.shape == (1, 1, 256, 16)
    assert_rows(y, yr, TOL_F32)
    assert_state(S, Sr, TOL_F32, "S")
    assert_state(z, zr, TOL_F32, "z")


@pytest.mark.parametrize("dv", [16, 32, 64])
def test_f32_state_and_jrt(gpu_lib, dv):
    w, q, k, v, ke, ve = small(2, 2, 75, dv, seed=70 + dv, dtype="f32", M=19)
    S0, z0, S0r, z0r = oracle_state(2, 2, dv, seed=71, noise=0.2)
    y, S, z = gpu_lib.jrt_prefix_prefill(q, k, v, ke, ve, S0, z0)
    torch.cuda.synchronize()
    yr, Sr, zr = oracle.jrt(q, k, v, ke, ve, S0r, z0r)
    assert_rows(y, yr, TOL_F32)
    assert_state(S, Sr, TOL_F32, "S")
    assert_state(z, zr, TOL_F32, "z")


@pytest.mark.parametrize("dv", [16, 32, 64])
@pytest.mark.parametrize("N", [1, 100, 256, 300])
def test_f32_prefill_with_initial_state(gpu_lib, dv, N):
    # fp32 inputs without a prefix: N <= 256 runs the parallel attention-form kernel,
    # N = 300 the token-sequential one; both against the oracle from a non-symmetric
    # initial state
    print(f"prefill f32 initial state dv={dv} N={N}", flush=True)
    w, q, k, v = small(2, 2, N, dv, seed=80 + dv + N, dtype="f32")
    S0, z0, S0r, z0r = oracle_state(2, 2, dv, seed=81 + dv, noise=0.5)
    y, S, z = gpu_lib.based_prefill(q, k, v, S0, z0)
    torch.cuda.synchronize()
    yr, Sr, zr = oracle.prefill(q, k, v, S0r, z0r)
    assert_rows(y, yr, TOL_F32)
    assert_state(S, Sr, TOL_F32, "S")
    assert_state(z, zr, TOL_F32, "z")


def test_f32_prefill_in_place_bf16_output_and_eps(gpu_lib):
    # the same call in place (token-sequential kernel) and out of place (parallel kernel):
    # the final states are the same sums in the same order, so they agree exactly
    print("prefill f32 in place vs out of place, bf16 y, eps", flush=True)
    w, q, k, v = small(2, 3, 200, 64, seed=95, dtype="f32")
    S0, z0, S0r, z0r = oracle_state(2, 3, 64, seed=96, noise=0.2)
    y1, S1, z1 = gpu_lib.based_prefill(q, k, v, S0, z0)
    Si, zi = S0.clone(), z0.clone()
    y2, _, _ = gpu_lib.based_prefill(q, k, v, Si, zi, S_out=Si, z_out=zi)
    torch.cuda.synchronize()
    assert torch.equal(S1, Si) and torch.equal(z1, zi)
    yr, _, _ = oracle.prefill(q, k, v, S0r, z0r)
    assert_rows(y1, yr, TOL_F32)
    assert_rows(y2, yr, TOL_F32)
    # bf16 output (8 significant bits: rounding adds up to 2^-8 of a row's largest entry) and eps
    y3, _, _ = gpu_lib.based_prefill(q, k, v, S0, z0, eps=0.25, out_dtype=torch.bfloat16,
                                     want_state=False)
    torch.cuda.synchronize()
    yr3, _, _ = oracle.prefill(q, k, v, S0r, z0r, eps=0.25)
    assert_rows(y3.float(), yr3, TOL_F32 + 2.0 ** -8)


# ---------------- decode step ----------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dv", [16, 32, 64])
def test_decode_steps_from_oracle_state(gpu_lib, dtype, dv):
    print(f"decode {dtype} dv={dv}", flush=True)
    B, H = 3, 5
    S0, z0, Sr, zr = oracle_state(B, H, dv, seed=80 + dv, noise=0.2)
    S, z = S0.clone(), z0.clone()
    w = gen.Workload("dec", B=B, H=H, N=0, d_feat=16, d_v=dv, dtype=dtype, seed=81)
    for step in range(6):
        q, k, v = gen.make_decode_step_inputs(w, step, DEV)
        y = gpu_lib.based_decode_step(q, k, v, S, z)
        torch.cuda.synchronize()
        yr, Sr, zr = oracle.decode_step(q, k, v, Sr, zr)
        # all-fp32 arithmetic on exact inputs
        assert_rows(y, yr, 2e-5)
    assert_state(S, Sr, 2e-6, "S")
    assert_state(z, zr, 2e-6, "z")


def test_decode_after_jrt_continues_the_merged_state(gpu_lib):
    w, q, k, v, ke, ve = small(2, 2, 100, 64, seed=90, M=64)
    _, S, z = gpu_lib.jrt_prefix_prefill(q, k, v, ke, ve)
    _, Sr, zr = oracle.jrt(q, k, v, ke, ve)
    wd = gen.Workload("dec", B=2, H=2, N=0, d_feat=16, d_v=64, dtype="bf16", seed=91)
    for step in range(3):
        qd, kd, vd = gen.make_decode_step_inputs(wd, step, DEV)
        y = gpu_lib.based_decode_step(qd, kd, vd, S, z)
        torch.cuda.synchronize()
        yr, Sr, zr = oracle.decode_step(qd, kd, vd, Sr, zr)
        assert_rows(y, yr, TOL_BF16)


def _prefix_state(kn, vn, upto, chunk=1 << 16):
    """sum_{j < upto} phi(k_j) v_j^T and sum_{j < upto} phi(k_j) for one head (fp64), the
    state's definition, built in chunks from the oracle's numpy feature map."""
    D = oracle.feature_dim(kn.shape[-1])
    S = np.zeros((D, vn.shape[-1]))
    z = np.zeros(D)
    for a in range(0, upto, chunk):
        b = min(upto, a + chunk)
        phi = oracle.feature_map_np(kn[a:b])
        S += phi.T @ vn[a:b]
        z += phi.sum(axis=0)
    return S, z


def _prefix_states(kn, vn, points, chunk=1 << 16):
    """The state's definition at each token count p in `points` (sum_{j < p} phi(k_j) v_j^T
    and sum_{j < p} phi(k_j), fp64) for one head, in one chunked pass over the tokens."""
    D = oracle.feature_dim(kn.shape[-1])
    S = np.zeros((D, vn.shape[-1]))
    z = np.zeros(D)
    out, pos = {}, 0
    for p in sorted(set(points)):
        while pos < p:
            b = min(p, pos + chunk)
            phi = oracle.feature_map_np(kn[pos:b])
            S += phi.T @ vn[pos:b]
            z += phi.sum(axis=0)
            pos = b
        out[p] = (S.copy(), z.copy())
    return out


def test_prefill_bf16_at_the_length_limit(gpu_lib):
    # the longest head the ABI accepts at d_v = 64: y takes N * d_v * 4 = 2^31 - 256 bytes
    # per head.  One head splits into 128 segments of 65536 tokens, the last one a token
    # short.  Row blocks at the start, across the boundary of segments 63 and 64 and at
    # the end are checked against the oracle recurrence seeded with the fp64 state of
    # every token before them, and the final state against its definition
    B, H, N, L = 1, 1, ((1 << 31) - 1) // 256, 300
    print(f"prefill B={B} H={H} N={N}", flush=True)
    w = gen.Workload("nmax", B=B, H=H, N=N, d_feat=16, d_v=64, dtype="bf16", seed=137)
    q, k, v = gen.make_prefill_inputs(w, DEV)
    y, S, z = gpu_lib.based_prefill(q, k, v)
    torch.cuda.synchronize()
    qn, kn, vn = (t[0, 0].cpu().double().numpy() for t in (q, k, v))
    starts = (0, 64 * 65536 - L // 2, N - L)
    states = _prefix_states(kn, vn, starts + (N,))
    for a in starts:
        S0, z0 = states[a]
        yr, _, _ = oracle.prefill(qn[None, None, a:a + L], kn[None, None, a:a + L],
                                  vn[None, None, a:a + L], S0[None, None], z0[None, None])
        assert_rows(y[:, :, a:a + L], yr, TOL_BF16)
    SN, zN = states[N]
    assert_state(S, SN[None, None], TOL_BF16, "S")
    assert_state(z, zN[None, None], TOL_BF16, "z")


def test_jrt_bf16_prefix_at_the_length_limit(gpu_lib):
    # the longest JRT prefix the ABI accepts at d_v = 64 (M = 8,388,607) before 65536 causal
    # tokens of one head: the chunk-parallel split sums the prefix in 63 parts.  Row blocks at
    # the start, across a segment boundary and at the end are checked against the oracle
    # recurrence seeded with the fp64 state of the prefix and every earlier causal token
    # ([JRT] §2.6 Eq. (3)), and the merged final state against its definition (Eq. (4))
    B, H, N, M, L = 1, 1, 1 << 16, ((1 << 31) - 1) // 256, 300
    print(f"jrt B={B} H={H} N={N} M={M}", flush=True)
    w = gen.Workload("mmax", B=B, H=H, N=N, d_feat=16, d_v=64, dtype="bf16", seed=141, M=M)
    q, k, v = gen.make_prefill_inputs(w, DEV)
    ke, ve = gen.make_prefix_inputs(w, DEV)
    y, S, z = gpu_lib.jrt_prefix_prefill(q, k, v, ke, ve)
    torch.cuda.synchronize()
    qn, kn, vn = (t[0, 0].cpu().double().numpy() for t in (q, k, v))
    ken, ven = (t[0, 0].cpu().double().numpy() for t in (ke, ve))
    Sp, zp = _prefix_states(ken, ven, (M,))[M]
    del ken, ven
    starts = (0, N // 2 - L // 2, N - L)
    states = _prefix_states(kn, vn, starts + (N,))
    for a in starts:
        Sa, za = states[a]
        yr, _, _ = oracle.prefill(qn[None, None, a:a + L], kn[None, None, a:a + L],
                                  vn[None, None, a:a + L], (Sp + Sa)[None, None], (zp + za)[None, None])
        assert_rows(y[:, :, a:a + L], yr, TOL_BF16)
    SN, zN = states[N]
    assert_state(S, (Sp + SN)[None, None], TOL_BF16, "S")
    assert_state(z, (zp + zN)[None, None], TOL_BF16, "z")


def test_prefill_bf16_at_the_head_limit(gpu_lib):
    # the most heads the bf16 prefill accepts: 2^21 workgroups of 1024 threads, 2^31
    # work-items in one dispatch.  Short sequences, y only; the first, the last and a
    # random sample of heads are checked against the oracle
    B, H, N = 1 << 11, 1 << 10, 5
    print(f"prefill B={B} H={H} N={N}", flush=True)
    w = gen.Workload("hmax", B=B, H=H, N=N, d_feat=16, d_v=64, dtype="bf16", seed=139)
    q, k, v = gen.make_prefill_inputs(w, DEV)
    y, _, _ = gpu_lib.based_prefill(q, k, v, want_state=False)
    torch.cuda.synchronize()
    rng = np.random.default_rng(139)
    heads = np.unique(np.concatenate([[0, 1, B * H - 2, B * H - 1], rng.integers(0, B * H, 60)]))
    flat = [t.reshape(B * H, N, -1) for t in (q, k, v, y)]
    qs, ks, vs, ys = (t[torch.as_tensor(heads, device=DEV)][None] for t in flat)
    yr, _, _ = oracle.prefill(qs, ks, vs)
    assert_rows(ys, yr, TOL_BF16)


def test_prefill_bf16_million_tokens_per_head(gpu_lib):
    # maximum-size edge: 2^20 + 77 tokens per head (element offsets past 2^26).  The oracle
    # recurrence runs on three row blocks, each seeded with the state of everything before
    # it; the final state is the last block's
    B, H, N, L = 1, 2, (1 << 20) + 77, 300
    print(f"prefill B={B} H={H} N={N}", flush=True)
    w = gen.Workload("long1m", B=B, H=H, N=N, d_feat=16, d_v=64, dtype="bf16", seed=131)
    q, k, v = gen.make_prefill_inputs(w, DEV)
    y, S, z = gpu_lib.based_prefill(q, k, v)
    torch.cuda.synchronize()
    for h in range(H):
        qn, kn, vn = (t[0, h].double().cpu().numpy() for t in (q, k, v))
        for a in (0, N // 2 + 5, N - L):
            S0, z0 = _prefix_state(kn, vn, a)
            yr, Sr, zr = oracle.prefill(qn[None, None, a:a + L], kn[None, None, a:a + L],
                                        vn[None, None, a:a + L], S0[None, None], z0[None, None])
            assert_rows(y[0:1, h:h + 1, a:a + L], yr, TOL_BF16)
        assert_state(S[0:1, h:h + 1], Sr, TOL_BF16, "S")
        assert_state(z[0:1, h:h + 1], zr, TOL_BF16, "z")
