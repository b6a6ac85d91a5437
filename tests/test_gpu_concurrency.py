"""Calls from several host threads, each on its own stream, give the same bits as the
same calls made one after another.

The library keeps no state between calls: the chunk-parallel split of a few-head call
keeps its partial sums in that call's own y, and nothing is allocated or cached.  So calls
that write disjoint memory may run at the same time.  Every kernel sums in a fixed order
with no atomics, so a call's outputs do not depend on what else runs, and the comparison
is exact.  The jobs cover the long walk (many heads), the three-launch split (few heads,
long sequence), a JRT prefix with the state updated in place, a state-only call and a
decode chain that updates its state in place step after step.
"""
import threading

import pytest
import torch

from recurrent_lm_sequence_amd import inputs as gen

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
D_FEAT = 16


def _inputs(B, H, N, dv, seed, M=0):
    w = gen.Workload("conc", B=B, H=H, N=N, d_feat=D_FEAT, d_v=dv, dtype="bf16", seed=seed, M=M)
    q, k, v = gen.make_prefill_inputs(w, DEV)
    ke = ve = None
    if M:
        ke, ve = gen.make_prefix_inputs(w, DEV)
    return w, q, k, v, ke, ve


def _make_jobs(bla):
    D = bla.feature_dim(D_FEAT)
    jobs = []

    # many heads: one walk per (head, column block)
    _, q1, k1, v1, _, _ = _inputs(8, 16, 1000, 64, 4401)

    def walk():
        return bla.based_prefill(q1, k1, v1)

    jobs.append(("walk B=8 H=16 N=1000", walk))

    # few heads, long sequence: the three-launch chunk-parallel split (partials in y)
    _, q2, k2, v2, _, _ = _inputs(1, 4, 16384, 64, 4402)
    g = torch.Generator(device=DEV).manual_seed(4403)
    S0 = torch.randn((1, 4, D, 64), generator=g, device=DEV)
    z0 = torch.rand((1, 4, D), generator=g, device=DEV) + 1.0

    def split():
        return bla.based_prefill(q2, k2, v2, S0, z0)

    jobs.append(("split B=1 H=4 N=16384 with S0", split))

    # JRT prefix, state updated in place (each call on its own copy of S0)
    _, q3, k3, v3, ke3, ve3 = _inputs(2, 8, 1500, 32, 4404, M=700)
    S3 = torch.randn((2, 8, D, 32), generator=g, device=DEV)
    z3 = torch.rand((2, 8, D), generator=g, device=DEV) + 1.0

    def jrt_in_place():
        S, z = S3.clone(), z3.clone()
        y, _, _ = bla.jrt_prefix_prefill(q3, k3, v3, ke3, ve3, S, z, S_out=S, z_out=z)
        return y, S, z

    jobs.append(("jrt in place B=2 H=8 N=1500 M=700", jrt_in_place))

    # state only (no y)
    _, q4, k4, v4, _, _ = _inputs(4, 4, 3000, 16, 4405)

    def state_only():
        _, S, z = bla.based_prefill(q4, k4, v4, want_y=False)
        return S, z

    jobs.append(("state only B=4 H=4 N=3000 dv=16", state_only))

    # a decode chain on the compact state, updated in place
    wd = gen.Workload("conc_dec", B=16, H=16, N=0, d_feat=D_FEAT, d_v=64, dtype="bf16", seed=4406,
                      decode_steps=6)
    steps = [gen.make_decode_step_inputs(wd, s, DEV) for s in range(6)]
    Dc = bla.compact_dim(D_FEAT)
    Sc = torch.randn((16, 16, Dc, 64), generator=g, device=DEV)
    zc = torch.rand((16, 16, Dc), generator=g, device=DEV) + 1.0

    def decode_chain():
        S, z = Sc.clone(), zc.clone()
        ys = [bla.based_decode_step(qs, ks, vs, S, z, compact=True) for qs, ks, vs in steps]
        return torch.stack(ys), S, z

    jobs.append(("decode chain B=16 H=16 compact", decode_chain))
    return jobs


def _as_list(out):
    if isinstance(out, torch.Tensor):
        return [out]
    return [t for t in out if t is not None]


def test_threads_on_separate_streams_match_serial_calls(gpu_lib):
    bla = gpu_lib
    jobs = _make_jobs(bla)
    torch.cuda.synchronize()
    serial = {}
    for name, fn in jobs:
        print(f"serial: {name}", flush=True)
        serial[name] = [t.clone() for t in _as_list(fn())]
    torch.cuda.synchronize()

    reps = 3
    results = {name: [] for name, _ in jobs}
    errors = []

    def worker(name, fn):
        try:
            s = torch.cuda.Stream(device=DEV)  # default priority
            with torch.cuda.stream(s):
                for _ in range(reps):
                    results[name].append([t.clone() for t in _as_list(fn())])
            s.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append((name, repr(e)))

    print("concurrent: " + ", ".join(n for n, _ in jobs), flush=True)
    threads = [threading.Thread(target=worker, args=(name, fn)) for name, fn in jobs]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    torch.cuda.synchronize()
    assert not errors, errors
    for name, _ in jobs:
        assert len(results[name]) == reps, name
        for r, outs in enumerate(results[name]):
            for i, (a, b) in enumerate(zip(outs, serial[name])):
                assert torch.equal(a, b), f"{name}: repetition {r}, output {i} differs from the serial call"
