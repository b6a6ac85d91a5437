"""Decode steps captured in a HIP graph (the pages time decode with CUDA graphs,
BASED notes §4.5): replays must equal the eager steps bit for bit.

The library's entry points launch on the caller's stream and neither allocate
nor synchronise, so torch's graph capture records them as they are.  The graph
is replayed several times from a restored state, with eager work and
synchronisations between the replays, and every replay is compared with the
eager run.
"""
import pytest
import torch

from recurrent_lm_sequence_amd import inputs as gen

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("compact", [False, True])
def test_decode_graph_replays_equal_eager(gpu_lib, compact):
    w = gen.Workload("graph", B=8, H=16, N=300, d_feat=16, d_v=64, dtype="bf16", seed=31)
    q, k, v = gen.make_prefill_inputs(w, DEV)
    _, S0, z0 = gpu_lib.based_prefill(q, k, v, want_y=False, compact=compact)
    steps = 8
    qs, ks, vs = zip(*(gen.make_decode_step_inputs(w, i, DEV) for i in range(steps)))
    ys = torch.empty((steps, w.B, w.H, w.d_v), dtype=torch.float32, device=DEV)
    S, z = S0.clone(), z0.clone()
    for i in range(steps):
        gpu_lib.based_decode_step(qs[i], ks[i], vs[i], S, z, y=ys[i], compact=compact)
    torch.cuda.synchronize()
    y_ref, S_ref, z_ref = ys.clone(), S.clone(), z.clone()

    S.copy_(S0)
    z.copy_(z0)
    ys.zero_()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up launch outside the capture
        gpu_lib.based_decode_step(qs[0], ks[0], vs[0], S.clone(), z.clone(), compact=compact)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            gpu_lib.based_decode_step(qs[i], ks[i], vs[i], S, z, y=ys[i], compact=compact)
    for rep in range(3):
        S.copy_(S0)  # eager work between the replays
        z.copy_(z0)
        ys.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ys, y_ref), f"replay {rep}: y differs from the eager steps"
        assert torch.equal(S, S_ref) and torch.equal(z, z_ref), f"replay {rep}: state differs"
