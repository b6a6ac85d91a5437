"""GPU parity of the bf16 prefill when a call has few heads and a long sequence.

Such a call splits each head's sequence into segments so that the grid still
covers the compute units.  When that spares the longest segment a walk over at
least 2048 earlier tokens, and y is requested with room for a segment's partial
state in that segment's own rows of y, the split runs as a chunk-parallel scan in
three launches: each segment sums its own tokens' state, the partial sums become
exclusive prefix sums in segment order, and each segment then walks its tokens
causally from S0 plus its prefix sum (a JRT prefix is summed in parts in the
same launches; a state updated in place is folded into the prefix sums, so that
only the last segment reads it).  Where segments stay long, one column block per
head with twice the segments replaces two column blocks.  Otherwise every segment walks the tokens
before it again (here: the 1000-, 700- and 2048-token cases and the state-only
call).  Both must match the fp64 oracle on every row and on the final state,
whatever the value width, output type, state layout and initial state.  Inputs come from the seeded generator; initial states
come from the oracle plus seeded non-symmetric noise.
"""
import numpy as np
import pytest
import torch

import oracle
from recurrent_lm_sequence_amd import inputs as gen
from tests.parity_util import TOL_BF16, assert_rows, assert_state

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _initial_state(B, H, dv, compact, seed):
    w = gen.Workload("init", B=B, H=H, N=80, d_feat=16, d_v=dv, dtype="bf16", seed=seed)
    q, k, v = gen.make_prefill_inputs(w, "cpu")
    _, S, z = oracle.prefill(q, k, v)
    nS, nz = gen.state_noise(B, H, S.shape[2], dv, seed + 1)
    S = S + 0.2 * nS.double().numpy()
    z = z + 0.2 * np.abs(nz.double().numpy())
    if compact:
        S, z = oracle.fold(S, 16, axis=-2), oracle.fold(z, 16, axis=-1)
    S0 = torch.tensor(S, dtype=torch.float32, device=DEV)
    z0 = torch.tensor(z, dtype=torch.float32, device=DEV)
    return S0, z0, S0.double().cpu().numpy(), z0.double().cpu().numpy()


# (B, H, N, d_v, bf16 y, initial state, compact): from 8 to 256 segments, ragged ends,
# every value width (two column blocks at 32 and 64), both output types
CASES = [
    (1, 2, 5000, 64, False, False, False),
    (1, 2, 5000, 64, True, True, False),
    (1, 1, 9001, 16, True, False, False),
    (1, 3, 7777, 32, False, True, True),
    (2, 1, 6000, 64, True, False, True),
    (3, 5, 9999, 16, False, True, False),
    (1, 1, 1000, 32, False, False, False),
    (1, 1, 700, 64, False, True, False),
    (1, 16, 2048, 64, True, True, False),
]


@pytest.mark.parametrize("B,H,N,dv,ybf16,init,compact", CASES)
def test_few_heads_long_sequence(gpu_lib, B, H, N, dv, ybf16, init, compact):
    print(f"sequence split B={B} H={H} N={N} d_v={dv} y={'bf16' if ybf16 else 'f32'} "
          f"initial={init} compact={compact}", flush=True)
    w = gen.Workload("split", B=B, H=H, N=N, d_feat=16, d_v=dv, dtype="bf16", seed=1200 + N % 97 + dv)
    q, k, v = gen.make_prefill_inputs(w, DEV)
    S0 = z0 = S0r = z0r = None
    if init:
        S0, z0, S0r, z0r = _initial_state(B, H, dv, compact, seed=1300 + N % 89)
    y, S, z = gpu_lib.based_prefill(q, k, v, S0, z0, compact=compact,
                                    out_dtype=torch.bfloat16 if ybf16 else torch.float32)
    torch.cuda.synchronize()
    yr, Sr, zr = (oracle.prefill_compact if compact else oracle.prefill)(q, k, v, S0r, z0r)
    # bf16 output rounding (8 significant bits) adds up to 2^-8 of a row's largest entry
    e = assert_rows(y.float(), yr, TOL_BF16 + (2.0 ** -8 if ybf16 else 0.0))
    print(f"worst row error {e:.3e}", flush=True)
    assert_state(S, Sr, TOL_BF16, "S")
    assert_state(z, zr, TOL_BF16, "z")


# Shapes where one column block per head with twice the segments replaces two column
# blocks (each segment >= 1024 tokens and half as long as with two blocks): the 64-column
# instance in the partial and seeded modes.  (B, H, N, M, d_v, bf16 y, initial state,
# compact, in place)
WIDE_CASES = [
    (1, 16, 32768, 0, 64, False, False, False, False),
    (2, 8, 16384, 0, 32, True, True, True, True),
    (1, 16, 32768, 16384, 64, False, True, False, False),
    (1, 4, 65536, 0, 64, False, True, False, True),
    (1, 32, 8192, 0, 64, True, False, True, False),
    (1, 8, 32768, 8000, 32, True, True, True, True),
]


@pytest.mark.parametrize("B,H,N,M,dv,ybf16,init,compact,in_place", WIDE_CASES)
def test_one_column_block_split(gpu_lib, B, H, N, M, dv, ybf16, init, compact, in_place):
    print(f"one-block split B={B} H={H} N={N} M={M} d_v={dv} y={'bf16' if ybf16 else 'f32'} "
          f"initial={init} compact={compact} in place={in_place}", flush=True)
    w = gen.Workload("wide", B=B, H=H, N=N, d_feat=16, d_v=dv, dtype="bf16", seed=1700 + N % 89 + dv,
                     M=max(M, 1))
    q, k, v = gen.make_prefill_inputs(w, DEV)
    S0 = z0 = S0r = z0r = None
    if init:
        S0, z0, S0r, z0r = _initial_state(B, H, dv, compact, seed=1800 + N % 83)
    out = dict(S_out=S0, z_out=z0) if in_place else {}
    od = torch.bfloat16 if ybf16 else torch.float32
    if M > 0:
        ke, ve = gen.make_prefix_inputs(w, DEV)
        y, S, z = gpu_lib.jrt_prefix_prefill(q, k, v, ke, ve, S0, z0, compact=compact, out_dtype=od, **out)
        torch.cuda.synchronize()
        yr, Sr, zr = (oracle.jrt_compact if compact else oracle.jrt)(q, k, v, ke, ve, S0r, z0r)
    else:
        y, S, z = gpu_lib.based_prefill(q, k, v, S0, z0, compact=compact, out_dtype=od, **out)
        torch.cuda.synchronize()
        yr, Sr, zr = (oracle.prefill_compact if compact else oracle.prefill)(q, k, v, S0r, z0r)
    e = assert_rows(y.float(), yr, TOL_BF16 + (2.0 ** -8 if ybf16 else 0.0))
    print(f"worst row error {e:.3e}", flush=True)
    assert_state(S, Sr, TOL_BF16, "S")
    assert_state(z, zr, TOL_BF16, "z")


def test_one_head_131072_tokens(gpu_lib):
    # 256 segments of 512 tokens at d_v = 16 (one column block), 128 of 1024 at 64
    for dv in (16, 64):
        print(f"sequence split B=1 H=1 N=131072 d_v={dv}", flush=True)
        w = gen.Workload("split1", B=1, H=1, N=131072, d_feat=16, d_v=dv, dtype="bf16", seed=1400 + dv)
        q, k, v = gen.make_prefill_inputs(w, DEV)
        y, S, z = gpu_lib.based_prefill(q, k, v)
        torch.cuda.synchronize()
        yr, Sr, zr = oracle.prefill(q, k, v)
        assert_rows(y, yr, TOL_BF16)
        assert_state(S, Sr, TOL_BF16, "S")
        assert_state(z, zr, TOL_BF16, "z")


def test_state_only_call_walks_the_prefix(gpu_lib):
    # no y: the call only needs the sum over its tokens, walked update-only in one
    # workgroup per head and column block; the final state must match
    print("state only, few heads", flush=True)
    w = gen.Workload("split2", B=1, H=2, N=5000, d_feat=16, d_v=64, dtype="bf16", seed=1500)
    q, k, v = gen.make_prefill_inputs(w, DEV)
    _, S, z = gpu_lib.based_prefill(q, k, v, want_y=False)
    torch.cuda.synchronize()
    _, Sr, zr = oracle.prefill(q, k, v)
    assert_state(S, Sr, TOL_BF16, "S")
    assert_state(z, zr, TOL_BF16, "z")


def test_split_and_unsplit_agree(gpu_lib):
    # the same tokens as one call over 2 heads x 6000 (split into segments) and as
    # 128 heads (64 copies of the batch: no sequence split).  The states are fp32 sums
    # in a different order (agreeing to 1e-4); y goes through the fp16 copy of the
    # state that each chunk's inter-chunk product reads, where such a difference can
    # flip a rounding, so y is held to half the parity tolerance
    print("sequence split against the unsplit launch", flush=True)
    w = gen.Workload("split3", B=1, H=2, N=6000, d_feat=16, d_v=64, dtype="bf16", seed=1600)
    q, k, v = gen.make_prefill_inputs(w, DEV)
    y1, S1, z1 = gpu_lib.based_prefill(q, k, v)
    rep = lambda t: t.repeat(64, 1, 1, 1).contiguous()
    y2, S2, z2 = gpu_lib.based_prefill(rep(q), rep(k), rep(v))
    torch.cuda.synchronize()
    rel = ((y1 - y2[:1]).abs().amax(-1) / y2[:1].abs().amax(-1).clamp_min(1e-30)).max().item()
    assert rel < TOL_BF16 / 2, rel
    for a, b in ((S1, S2[:1]), (z1, z2[:1])):
        assert ((a - b).abs().max() / b.abs().max()).item() < 1e-4


# JRT prefix with few heads: the prefix is summed in parts alongside the causal
# segments' partials, and every causal segment (the first included) starts from S0
# plus the prefix sum plus the segments before it.  (B, H, N, M, d_v, bf16 y,
# initial state, compact, left-padded prefix lengths or None)
JRT_CASES = [
    (1, 16, 4096, 2048, 64, False, False, False, None),
    (2, 3, 4096, 2048, 64, True, True, False, None),
    (1, 1, 8192, 8192, 16, True, False, True, None),
    (1, 2, 3000, 5000, 32, False, True, True, None),
    (1, 4, 20000, 300, 64, False, False, False, None),
    (3, 1, 5000, 3000, 64, False, True, False, [3000, 1, 1700]),
    (2, 2, 6000, 4000, 32, True, False, True, [0, 3999]),
    # long segments: one column block per head with twice the segments, padded prefixes
    (2, 4, 32768, 6000, 64, True, True, False, [6000, 2345]),
    (2, 8, 16384, 4000, 32, False, False, True, [0, 3999]),
]


@pytest.mark.parametrize("B,H,N,M,dv,ybf16,init,compact,lens", JRT_CASES)
def test_few_heads_jrt_prefix(gpu_lib, B, H, N, M, dv, ybf16, init, compact, lens):
    print(f"jrt split B={B} H={H} N={N} M={M} d_v={dv} y={'bf16' if ybf16 else 'f32'} initial={init} "
          f"compact={compact} prefix_len={lens}", flush=True)
    w = gen.Workload("jsplit", B=B, H=H, N=N, d_feat=16, d_v=dv, dtype="bf16", seed=1700 + N % 83 + M % 7, M=M)
    q, k, v = gen.make_prefill_inputs(w, DEV)
    ke, ve = gen.make_prefix_inputs(w, DEV)
    S0 = z0 = S0r = z0r = None
    if init:
        S0, z0, S0r, z0r = _initial_state(B, H, dv, compact, seed=1800 + M % 61)
    od = torch.bfloat16 if ybf16 else torch.float32
    if lens is not None:
        pl = torch.tensor(lens, dtype=torch.int32, device=DEV)
        y, S, z = gpu_lib.jrt_prefix_prefill(q, k, v, ke, ve, S0, z0, compact=compact, prefix_len=pl,
                                             out_dtype=od)
        torch.cuda.synchronize()
        yr, Sr, zr = oracle.jrt_padded(q, k, v, ke, ve, lens, S0r, z0r, compact=compact)
    else:
        y, S, z = gpu_lib.jrt_prefix_prefill(q, k, v, ke, ve, S0, z0, compact=compact, out_dtype=od)
        torch.cuda.synchronize()
        yr, Sr, zr = (oracle.jrt_compact if compact else oracle.jrt)(q, k, v, ke, ve, S0r, z0r)
    e = assert_rows(y.float(), yr, TOL_BF16 + (2.0 ** -8 if ybf16 else 0.0))
    print(f"worst row error {e:.3e}", flush=True)
    assert_state(S, Sr, TOL_BF16, "S")
    assert_state(z, zr, TOL_BF16, "z")


# State updated in place (S, z or both) with few heads: the initial state is folded
# into the segments' prefix sums, so only the last segment reads S0 and z0, each lane
# the entries it then overwrites.  (B, H, N, M, d_v, bf16 y, compact, S in place,
# z in place)
IN_PLACE_CASES = [
    (1, 2, 6000, 0, 64, False, False, True, True),
    (1, 3, 9000, 0, 32, True, True, True, True),
    (2, 1, 7000, 0, 16, False, False, True, False),
    (1, 2, 6000, 0, 64, False, False, False, True),
    (1, 4, 5000, 3000, 64, False, False, True, True),
    (1, 1, 8192, 8192, 16, True, True, True, True),
]


@pytest.mark.parametrize("B,H,N,M,dv,ybf16,compact,s_in,z_in", IN_PLACE_CASES)
def test_few_heads_in_place_state(gpu_lib, B, H, N, M, dv, ybf16, compact, s_in, z_in):
    print(f"in-place split B={B} H={H} N={N} M={M} d_v={dv} y={'bf16' if ybf16 else 'f32'} compact={compact} "
          f"S in place={s_in} z in place={z_in}", flush=True)
    w = gen.Workload("ipsplit", B=B, H=H, N=N, d_feat=16, d_v=dv, dtype="bf16", seed=1900 + N % 71 + dv,
                     M=max(M, 1))
    q, k, v = gen.make_prefill_inputs(w, DEV)
    S0, z0, S0r, z0r = _initial_state(B, H, dv, compact, seed=2000 + N % 53)
    S, z = S0.clone(), z0.clone()
    S_out = S if s_in else torch.empty_like(S0)
    z_out = z if z_in else torch.empty_like(z0)
    od = torch.bfloat16 if ybf16 else torch.float32
    if M > 0:
        ke, ve = gen.make_prefix_inputs(w, DEV)
        y, _, _ = gpu_lib.jrt_prefix_prefill(q, k, v, ke, ve, S, z, S_out=S_out, z_out=z_out, compact=compact,
                                             out_dtype=od)
        torch.cuda.synchronize()
        yr, Sr, zr = (oracle.jrt_compact if compact else oracle.jrt)(q, k, v, ke, ve, S0r, z0r)
    else:
        y, _, _ = gpu_lib.based_prefill(q, k, v, S, z, S_out=S_out, z_out=z_out, compact=compact, out_dtype=od)
        torch.cuda.synchronize()
        yr, Sr, zr = (oracle.prefill_compact if compact else oracle.prefill)(q, k, v, S0r, z0r)
    e = assert_rows(y.float(), yr, TOL_BF16 + (2.0 ** -8 if ybf16 else 0.0))
    print(f"worst row error {e:.3e}", flush=True)
    assert_state(S_out, Sr, TOL_BF16, "S")
    assert_state(z_out, zr, TOL_BF16, "z")


# State-only calls (y not requested, no JRT prefix): every token is walked as an
# update-only chunk from S0.  (B, H, N, d_v, initial state, compact, in place)
STATE_ONLY_CASES = [
    (16, 16, 1000, 64, False, False, False),
    (2, 3, 777, 32, True, False, False),
    (1, 1, 5000, 16, True, True, True),
    (8, 16, 2048, 64, True, False, True),
    (3, 2, 129, 32, False, True, False),
]


@pytest.mark.parametrize("B,H,N,dv,init,compact,in_place", STATE_ONLY_CASES)
def test_state_only_calls(gpu_lib, B, H, N, dv, init, compact, in_place):
    print(f"state only B={B} H={H} N={N} d_v={dv} initial={init} compact={compact} in place={in_place}",
          flush=True)
    w = gen.Workload("sonly", B=B, H=H, N=N, d_feat=16, d_v=dv, dtype="bf16", seed=2100 + N % 67 + dv)
    q, k, v = gen.make_prefill_inputs(w, DEV)
    S0 = z0 = S0r = z0r = None
    if init:
        S0, z0, S0r, z0r = _initial_state(B, H, dv, compact, seed=2200 + N % 59)
    if in_place:
        _, S, z = gpu_lib.based_prefill(q, k, v, S0, z0, S_out=S0, z_out=z0, want_y=False, compact=compact)
    else:
        _, S, z = gpu_lib.based_prefill(q, k, v, S0, z0, want_y=False, compact=compact)
    torch.cuda.synchronize()
    _, Sr, zr = (oracle.prefill_compact if compact else oracle.prefill)(q, k, v, S0r, z0r)
    assert_state(S, Sr, TOL_BF16, "S")
    assert_state(z, zr, TOL_BF16, "z")


def _draw_split_case(i):
    r = np.random.default_rng(9700 + i)
    B, H = int(r.integers(1, 3)), int(r.integers(1, 9))
    N = int(r.integers(3000, 12001))
    M = 0 if r.random() < 0.5 else int(r.integers(1, 5000))
    lens = [int(x) for x in r.integers(0, M + 1, size=B)] if M > 0 and r.random() < 0.5 else None
    dv = int(r.choice([16, 32, 64]))
    ybf16 = bool(r.random() < 0.3)
    compact = bool(r.integers(0, 2))
    init = bool(r.integers(0, 2))
    in_place = init and bool(r.integers(0, 2))
    return B, H, N, M, lens, dv, ybf16, compact, init, in_place


@pytest.mark.parametrize("i", range(10))
def test_random_split_configuration(gpu_lib, i):
    # seeded random combinations in the split's regime (few heads, thousands of tokens)
    B, H, N, M, lens, dv, ybf16, compact, init, in_place = _draw_split_case(i)
    print(f"random split case {i}: B={B} H={H} N={N} M={M} prefix_len={lens} d_v={dv} "
          f"y={'bf16' if ybf16 else 'f32'} compact={compact} initial={init} in place={in_place}", flush=True)
    w = gen.Workload("rsplit", B=B, H=H, N=N, d_feat=16, d_v=dv, dtype="bf16", seed=9800 + i, M=max(M, 1))
    q, k, v = gen.make_prefill_inputs(w, DEV)
    ke, ve = gen.make_prefix_inputs(w, DEV)
    ke, ve = ke[:, :, :M].contiguous(), ve[:, :, :M].contiguous()
    S0 = z0 = S0r = z0r = None
    if init:
        S0, z0, S0r, z0r = _initial_state(B, H, dv, compact, seed=9900 + i)
    out = dict(S_out=S0, z_out=z0) if in_place else {}
    od = torch.bfloat16 if ybf16 else torch.float32
    if M > 0:
        pl = torch.tensor(lens, dtype=torch.int32, device=DEV) if lens is not None else None
        y, S, z = gpu_lib.jrt_prefix_prefill(q, k, v, ke, ve, S0, z0, compact=compact, prefix_len=pl,
                                             out_dtype=od, **out)
        torch.cuda.synchronize()
        yr, Sr, zr = oracle.jrt_padded(q, k, v, ke, ve, lens if lens is not None else [M] * B, S0r, z0r,
                                       compact=compact)
    else:
        y, S, z = gpu_lib.based_prefill(q, k, v, S0, z0, compact=compact, out_dtype=od, **out)
        torch.cuda.synchronize()
        yr, Sr, zr = (oracle.prefill_compact if compact else oracle.prefill)(q, k, v, S0r, z0r)
    e = assert_rows(y.float(), yr, TOL_BF16 + (2.0 ** -8 if ybf16 else 0.0))
    print(f"worst row error {e:.3e}", flush=True)
    assert_state(S, Sr, TOL_BF16, "S")
    assert_state(z, zr, TOL_BF16, "z")
