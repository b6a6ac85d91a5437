"""Decode steps and prefills captured in a HIP graph (the pages time decode with
CUDA graphs, BASED notes §4.5): replays must equal the eager calls bit for bit.

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


def _prefill_cases(bla):
    """(name, inputs, call(out)) for prefills of each launch shape; `out` holds
    preallocated y, S, z (S, z also the in-place initial state where used)."""
    D = bla.feature_dim(16)
    g = torch.Generator(device=DEV).manual_seed(33)
    cases = []
    w1 = gen.Workload("g_walk", B=8, H=16, N=700, d_feat=16, d_v=64, dtype="bf16", seed=34)
    q1, k1, v1 = gen.make_prefill_inputs(w1, DEV)
    cases.append(("walk B=8 H=16 N=700", (w1.B, w1.H, w1.N, 64), None,
                  lambda o: bla.based_prefill(q1, k1, v1, y=o["y"], S_out=o["S"], z_out=o["z"])))
    w2 = gen.Workload("g_split", B=1, H=4, N=9000, d_feat=16, d_v=64, dtype="bf16", seed=35)
    q2, k2, v2 = gen.make_prefill_inputs(w2, DEV)
    S0 = torch.randn((1, 4, D, 64), generator=g, device=DEV)
    z0 = torch.rand((1, 4, D), generator=g, device=DEV) + 1.0
    cases.append(("three-launch split B=1 H=4 N=9000 with S0", (1, 4, 9000, 64), None,
                  lambda o: bla.based_prefill(q2, k2, v2, S0, z0, y=o["y"], S_out=o["S"], z_out=o["z"])))
    w3 = gen.Workload("g_jrt", B=2, H=8, N=1200, d_feat=16, d_v=32, dtype="bf16", seed=36, M=500)
    q3, k3, v3 = gen.make_prefill_inputs(w3, DEV)
    ke3, ve3 = gen.make_prefix_inputs(w3, DEV)
    S3 = torch.randn((2, 8, D, 32), generator=g, device=DEV)
    z3 = torch.rand((2, 8, D), generator=g, device=DEV) + 1.0
    cases.append(("jrt in place B=2 H=8 N=1200 M=500", (2, 8, 1200, 32), (S3, z3),
                  lambda o: bla.jrt_prefix_prefill(q3, k3, v3, ke3, ve3, o["S"], o["z"], y=o["y"],
                                                   S_out=o["S"], z_out=o["z"])))
    return cases


def test_prefill_graph_replays_equal_eager(gpu_lib):
    """Prefills captured in a HIP graph: the walk, the chunk-parallel split (three
    launches whose partial sums live in y) and a JRT call with the state updated in
    place; every replay equals the eager call bit for bit."""
    D = gpu_lib.feature_dim(16)
    for name, (B, H, N, dv), init, call in _prefill_cases(gpu_lib):
        print(f"graph prefill: {name}", flush=True)
        o = {"y": torch.empty((B, H, N, dv), device=DEV), "S": torch.empty((B, H, D, dv), device=DEV),
             "z": torch.empty((B, H, D), device=DEV)}

        def restore():
            if init is not None:
                o["S"].copy_(init[0])
                o["z"].copy_(init[1])

        restore()
        call(o)
        torch.cuda.synchronize()
        ref = {key: t.clone() for key, t in o.items()}

        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        restore()
        with torch.cuda.stream(side):  # warm-up launch outside the capture
            call(o)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            call(o)
        for rep in range(3):
            for t in o.values():  # eager work between the replays
                t.fill_(float("nan"))
            restore()
            torch.cuda.synchronize()
            gr.replay()
            torch.cuda.synchronize()
            for key in o:
                assert torch.equal(o[key], ref[key]), f"{name}: replay {rep}, {key} differs from the eager call"
