#!/usr/bin/env python3
"""Benchmark of the causal Taylor linear-attention library on one MI355X.

Prints ONE JSON line on stdout (progress goes to stderr).

Headline ("step"): one based_prefill launch over the long-prefill workload
(B=16, H=16, N=32768, d'=16, D=273, d_v=64; bf16 q,k,v ~ N(0,1), zero initial
state, fp32 y and final state).  value = B*N / (time per launch), tokens/s.
In the same run:
  * jrt:    jrt_prefix_prefill, B=16, H=16, N=4096, M=2048 (tokens/s = B*N/t);
  * decode: state-passing decode, B=256, H=16, initial state from an untimed
            8192-token prefill, then 512 timed decode steps (tokens/s = B*512/t,
            state bytes streamed per second);
  * decode_compact: the same with the compact (folded, 153-row) state layout;
  * swa: sliding-window softmax attention prefill (B=16, H=16, N=32768,
            windows 64/128) and its ring-cache decode step (B=256, H=16, w=128);
  * table5: the pages' Table 5 sweep (L = 2048..32768, B=16): BASED prefill,
            JRT-Prompt (prefill over the prompt repeated, 2L tokens) and JRT-RNN
            (M = L/2 prefix + N = L causal), with the H100 figures as context;
  * cpu_baseline: the fp64 oracle on the machine's host cores over the whole
            long-prefill batch (256 heads x 32768 tokens, about 10-30 s of CPU
            work), which is also a parity check of every row the timed launch
            wrote.
Timing uses events on the stream the kernels are launched on (torch's current
stream is passed through the C ABI).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix peak
# the pages' H100 BASED prefill latency at batch 16, N=32768 (4.5 ms), as tokens/s
H100_BASED_TOKENS_PER_S = 16 * 32768 / 4.5e-3
METRIC = "prefill tokens/s + %MFMA peak (N=32k,B=16); decode tokens/s + HBM GB/s"

# algorithmic work per unit.  Prefill FLOP per token-head (the dense part of the chunked form of
#   the BASED notes, section 2.5): scores 2*C*d' + intra-chunk A.V 2*C*d_v on the full C = 64 tile
#   of the workload, plus the inter-chunk product phi(Q).S and the update phi(K)^T V, 2*D*d_v each,
#   counted with the D the kernel contracts: every unordered feature pair once, D = 1 + 16 + 136
#   = 153 (section 2.3 notes that vec(x x^T) repeats each off-diagonal product).  The matrix-core
#   work the kernel actually issues (a 160-row padded state, 128-token chunks and the denominator
#   products) is read from the rocprofv3 counter SQ_INSTS_VALU_MFMA_MOPS_F16 and reported beside.
#   Bytes: what one launch must read and write once.
BYTES_PER_TOKEN_HEAD = 2 * 16 * 2 + 64 * 2 + 64 * 4   # q, k, v bf16 in + y fp32 out = 448 B
STATE_BYTES_PER_HEAD = (273 * 64 + 273) * 4           # final S, z written once = 70,980 B
D_CONTRACTED = 153
FLOP_PER_TOKEN_HEAD = 2 * 64 * (16 + 64) + 2 * 2 * D_CONTRACTED * 64   # 49,408
DECODE_BYTES_PER_HEAD = 2 * STATE_BYTES_PER_HEAD + 16 * 2 * 2 + 64 * 2 + 64 * 4  # 142,408 B
# compact (folded) state: 153 rows instead of 273
COMPACT_STATE_BYTES_PER_HEAD = (153 * 64 + 153) * 4    # 39,780 B
DECODE_COMPACT_BYTES_PER_HEAD = 2 * COMPACT_STATE_BYTES_PER_HEAD + 16 * 2 * 2 + 64 * 2 + 64 * 4  # 80,008 B


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def committed_traffic(kernel_file: str, profile_name: str):
    """HBM bytes per launch measured with rocprofv3 counters (profiles/), if the
    kernel source still matches the digest recorded with the measurement."""
    p = os.path.join(ROOT, "profiles", profile_name)
    if not os.path.exists(p):
        return None
    text = open(p).read()
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    m_h = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    if not (m_b and m_h):
        return None
    if m_h.group(1) != source_digest(kernel_file):
        return None
    return float(m_b.group(1))


def committed_executed_flop(kernel_file: str, profile_name: str):
    """Matrix-core FLOP per launch the kernel executed (512 x SQ_INSTS_VALU_MFMA_MOPS_F16,
    from the committed rocprofv3 summary), if the kernel source still matches."""
    p = os.path.join(ROOT, "profiles", profile_name)
    if not os.path.exists(p):
        return None
    text = open(p).read()
    m_f = re.search(r"executed_mfma_flop_per_launch:\s*([0-9.eE+]+)", text)
    m_h = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    if not (m_f and m_h) or m_h.group(1) != source_digest(kernel_file):
        return None
    return float(m_f.group(1))


def measured_peaks(bl):
    """Ceilings measured on this GPU with the library's probe kernels: a matrix-core loop
    of fp16 16x16x32 products with no memory traffic, and a 16-byte-vector streaming copy
    of 4 GiB (read + write bytes per second).  Best of five timed launches each."""
    import torch

    sink = torch.empty(8192 * 256, dtype=torch.float32, device="cuda:0")
    blocks, iters = 8192, 2048
    flop = bl.probe_mfma_f16(sink, blocks, iters)  # warm-up
    best_mfma = 0.0
    for _ in range(5):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        bl.probe_mfma_f16(sink, blocks, iters)
        e.record()
        torch.cuda.synchronize()
        best_mfma = max(best_mfma, flop / (s.elapsed_time(e) / 1e3) / 1e12)
    n = 1 << 30  # 4 GiB of fp32
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    moved = bl.probe_copy(src, dst)
    best_copy = 0.0
    for _ in range(5):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        bl.probe_copy(src, dst)
        e.record()
        torch.cuda.synchronize()
        best_copy = max(best_copy, moved / (s.elapsed_time(e) / 1e3) / 1e9)
    del src, dst, sink
    torch.cuda.empty_cache()
    log(f"[peaks] matrix-core probe {best_mfma:.0f} TFLOP/s (fp16 16x16x32), copy probe {best_copy:.0f} GB/s")
    return {"mfma_f16_tflops": round(best_mfma, 1), "hbm_copy_gbs": round(best_copy, 1),
            "note": "best of 5 launches: bla_probe_mfma_f16 (8192 x 4 wavefronts x 2048 x 8 "
                    "independent 16x16x32 fp16 products, no memory traffic) and bla_probe_copy "
                    "(4 GiB, 16-byte vectors; read + write bytes)"}


def time_launches(fn, steps: int, warmup: int, per_launch: list | None = None):
    """Seconds for `steps` launches after `warmup` untimed ones, between two events on
    the stream.  With per_launch, an event also follows every launch and the list
    receives each launch's seconds (the bracket is unchanged: first to last event)."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1 if per_launch is not None else 2)]
    ev[0].record()
    for i in range(steps):
        fn()
        if per_launch is not None:
            ev[i + 1].record()
    if per_launch is None:
        ev[1].record()
    torch.cuda.synchronize()
    if per_launch is not None:
        per_launch.extend(ev[i].elapsed_time(ev[i + 1]) / 1e3 for i in range(steps))
    return ev[0].elapsed_time(ev[-1]) / 1e3  # seconds for `steps` launches


def bench_prefill(bl, gen, steps, warmup):
    import torch

    w = gen.LONG_PREFILL
    log(f"[prefill] generating inputs {w}")
    q, k, v = gen.make_prefill_inputs(w, "cuda:0")
    D = w.feature_dim
    y = torch.empty((w.B, w.H, w.N, w.d_v), dtype=torch.float32, device="cuda:0")
    S = torch.empty((w.B, w.H, D, w.d_v), dtype=torch.float32, device="cuda:0")
    z = torch.empty((w.B, w.H, D), dtype=torch.float32, device="cuda:0")

    def run():
        bl.based_prefill(q, k, v, y=y, S_out=S, z_out=z)

    log(f"[prefill] warmup {warmup}, timing {steps} launches")
    each = []
    t = time_launches(run, steps, warmup, per_launch=each)
    per = t / steps
    srt = sorted(each)
    med = (srt[(steps - 1) // 2] + srt[steps // 2]) / 2
    launch_stats = {"mean_ms": round(per * 1e3, 4), "median_ms": round(med * 1e3, 4),
                    "min_ms": round(srt[0] * 1e3, 4), "max_ms": round(srt[-1] * 1e3, 4)}
    log(f"[prefill] per launch: median {med * 1e3:.4f} ms, min {srt[0] * 1e3:.4f}, max {srt[-1] * 1e3:.4f}")
    token_heads = w.B * w.H * w.N
    alg_bytes = token_heads * BYTES_PER_TOKEN_HEAD + w.B * w.H * STATE_BYTES_PER_HEAD
    alg_flop = token_heads * FLOP_PER_TOKEN_HEAD
    log(f"[prefill] {per * 1e3:.4f} ms/launch, {w.B * w.N / per / 1e6:.1f} M tokens/s")
    # context: the same launch with bf16 y (half the output stream; not the headline, whose
    # y is fp32 because bf16 rounding alone can reach 2^-8 of a row)
    yb = torch.empty((w.B, w.H, w.N, w.d_v), dtype=torch.bfloat16, device="cuda:0")
    per_b = time_launches(lambda: bl.based_prefill(q, k, v, y=yb, S_out=S, z_out=z), steps,
                          warmup) / steps
    bytes_b = token_heads * (BYTES_PER_TOKEN_HEAD - 64 * 2) + w.B * w.H * STATE_BYTES_PER_HEAD
    log(f"[prefill] bf16 y: {per_b * 1e3:.4f} ms/launch")
    bf16_y = {"ms": round(per_b * 1e3, 4), "tokens_per_s": w.B * w.N / per_b,
              "roofline": {"bound": "hbm", "achieved": round(bytes_b / per_b / 1e9, 1),
                           "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(bytes_b / per_b / 1e9 / HBM_PEAK_GBS, 4), "traffic": None}}
    del yb
    floor = traffic_floor(bl, q, k, v, steps, warmup)
    return dict(w=w, q=q, k=k, v=v, y=y, per=per, alg_bytes=alg_bytes, alg_flop=alg_flop,
                bf16_y=bf16_y, traffic_floor=floor, launch_stats=launch_stats)


def traffic_floor(bl, q, k, v, steps, warmup):
    """The long prefill's HBM traffic with none of its arithmetic (bla_probe_prefill_traffic:
    one workgroup per head streams q, k, v in and fp32 y out in 128-token chunks), timed like
    the kernel: the floor the memory system sets for this traffic shape.  Also its read-only
    and write-only halves."""
    import torch

    B, H, N, _ = q.shape
    y2 = torch.empty((B, H, N, 64), dtype=torch.float32, device="cuda:0")
    sink = torch.empty(B * H * 512, dtype=torch.float32, device="cuda:0")
    out = {}
    for mode, key in ((0, "reads_and_writes"), (1, "reads_only"), (2, "writes_only")):
        nbytes = bl.probe_prefill_traffic(q, k, v, y2, sink, mode)
        per = time_launches(lambda: bl.probe_prefill_traffic(q, k, v, y2, sink, mode), steps, warmup) / steps
        out[key] = {"ms": round(per * 1e3, 4), "GBps": round(nbytes / per / 1e9, 1)}
    log(f"[prefill] traffic floor: {out['reads_and_writes']['ms']:.4f} ms "
        f"({out['reads_and_writes']['GBps']:.0f} GB/s); reads only {out['reads_only']['ms']:.4f} ms, "
        f"writes only {out['writes_only']['ms']:.4f} ms")
    del y2, sink
    torch.cuda.empty_cache()
    return out


def bench_jrt(bl, gen, steps, warmup):
    import torch

    w = gen.JRT_PREFIX
    log(f"[jrt] generating inputs {w}")
    q, k, v = gen.make_prefill_inputs(w, "cuda:0")
    ke, ve = gen.make_prefix_inputs(w, "cuda:0")
    D = w.feature_dim
    y = torch.empty((w.B, w.H, w.N, w.d_v), dtype=torch.float32, device="cuda:0")
    S = torch.empty((w.B, w.H, D, w.d_v), dtype=torch.float32, device="cuda:0")
    z = torch.empty((w.B, w.H, D), dtype=torch.float32, device="cuda:0")

    def run():
        bl.jrt_prefix_prefill(q, k, v, ke, ve, y=y, S_out=S, z_out=z)

    t = time_launches(run, steps, warmup)
    per = t / steps
    log(f"[jrt] {per * 1e3:.4f} ms/launch, {w.B * w.N / per / 1e6:.1f} M tokens/s")
    # algorithmic bytes: 448 B per causal token-head (q, k, v in, fp32 y out), 160 B per prefix
    # token-head (k_e, v_e in) and the merged final state once per head
    alg = (w.B * w.H * w.N * BYTES_PER_TOKEN_HEAD + w.B * w.H * w.M * (16 * 2 + 64 * 2)
           + w.B * w.H * STATE_BYTES_PER_HEAD)
    out = {"workload": f"jrt_prefix B={w.B} H={w.H} N={w.N} M={w.M} d'={w.d_feat} d_v={w.d_v}",
           "ms": round(per * 1e3, 4), "tokens_per_s": w.B * w.N / per,
           "roofline": {"bound": "hbm", "achieved": round(alg / per / 1e9, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(alg / per / 1e9 / HBM_PEAK_GBS, 4),
                        "traffic": committed_traffic(PREFILL_SRC, "prefill_ws_jrt_prefix.md")}}
    del q, k, v, ke, ve, y, S, z
    torch.cuda.empty_cache()
    return out


SINGLE_SEQUENCE = dict(B=1, H=16, N=32768, d_feat=16, d_v=64, dtype="bf16", seed=1005)


def bench_small_configs(bl, gen, steps, warmup, which=("layer_prefill", "tiny_f32")):
    """The smaller configurations reported beside the headline: the BASED-layer
    prefill (B=8, H=16, N=2048, bf16) with its HBM roofline, the latency of the
    tiny fp32 case (B=1, H=1, N=256, d_v=16) on the fp32-exact kernel, and (its own
    leg) one long sequence (B=1, H=16, N=32768, bf16), whose few heads take the
    chunk-parallel sequence split (three launches per call)."""
    import torch

    table = {"layer_prefill": gen.LAYER_PREFILL, "tiny_f32": gen.TINY_F32,
             "single_sequence": gen.Workload("single_sequence", **SINGLE_SEQUENCE)}
    out = {}
    for key in which:
        w = table[key]
        q, k, v = gen.make_prefill_inputs(w, "cuda:0")
        D = w.feature_dim
        y = torch.empty((w.B, w.H, w.N, w.d_v), dtype=torch.float32, device="cuda:0")
        S = torch.empty((w.B, w.H, D, w.d_v), dtype=torch.float32, device="cuda:0")
        z = torch.empty((w.B, w.H, D), dtype=torch.float32, device="cuda:0")

        def run():
            bl.based_prefill(q, k, v, y=y, S_out=S, z_out=z)

        per = time_launches(run, steps, warmup) / steps
        th = w.B * w.H * w.N
        entry = {"workload": f"{w.name} B={w.B} H={w.H} N={w.N} d'={w.d_feat} d_v={w.d_v} {w.dtype} in",
                 "us_per_launch": round(per * 1e6, 2), "tokens_per_s": w.B * w.N / per}
        if w.dtype == "bf16":
            alg = th * BYTES_PER_TOKEN_HEAD + w.B * w.H * STATE_BYTES_PER_HEAD
            entry["roofline"] = {"bound": "hbm", "achieved": round(alg / per / 1e9, 1),
                                 "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": round(alg / per / 1e9 / HBM_PEAK_GBS, 4),
                                 "traffic": (committed_traffic(PREFILL_SRC, "prefill_ws_layer_prefill.md")
                                             if key == "layer_prefill" else None)}
        log(f"[{key}] {per * 1e6:.2f} us/launch, {w.B * w.N / per / 1e6:.2f} M tokens/s")
        out[key] = entry
        del q, k, v, y, S, z
    torch.cuda.empty_cache()
    return out


# The pages' Table 5 (H100, batch 16, prefill latency in ms): BASED custom CUDA,
# JRT-Prompt (the prompt read twice: a prefill over 2L tokens, counted by the
# pages as twice the BASED cost) and JRT-RNN (prefix state plus causal scan,
# about 1.24x BASED).  Context from another machine, not a target.
TABLE5_H100_MS = {2048: (0.3, 0.6, 0.4), 8192: (1.2, 2.3, 1.5), 16384: (2.3, 4.5, 2.8),
                  32768: (4.5, 9.0, 5.6)}


TABLE5_ROUNDS = 3


def bench_table5(bl, gen, steps, warmup):
    """The Table 5 sweep on this GPU: for L in 2048..32768 at B=16, H=16, d'=16,
    d_v=64: BASED prefill over L tokens, JRT-Prompt = BASED prefill over the
    prompt repeated twice (2L tokens; the second copy equals the first), and
    JRT-RNN = jrt_prefix_prefill with an M = L/2 token prefix and N = L."""
    import torch

    rows = []
    for L, h100 in TABLE5_H100_MS.items():
        w = gen.Workload("table5", B=16, H=16, N=L, d_feat=16, d_v=64, dtype="bf16",
                         seed=1100 + L // 1024, M=L // 2)
        q, k, v = gen.make_prefill_inputs(w, "cuda:0")
        ke, ve = gen.make_prefix_inputs(w, "cuda:0")
        y = torch.empty((w.B, w.H, 2 * L, w.d_v), dtype=torch.float32, device="cuda:0")
        S = torch.empty((w.B, w.H, w.feature_dim, w.d_v), dtype=torch.float32, device="cuda:0")
        z = torch.empty((w.B, w.H, w.feature_dim), dtype=torch.float32, device="cuda:0")
        y1 = torch.empty((w.B, w.H, L, w.d_v), dtype=torch.float32, device="cuda:0")
        q2, k2, v2 = (torch.cat([t, t], dim=2).contiguous() for t in (q, k, v))
        # the three workloads interleaved over three rounds, median per workload: a single
        # back-to-back series is exposed to the clock drift of sustained prefill load
        runs = {"based": lambda: bl.based_prefill(q, k, v, y=y1, S_out=S, z_out=z),
                "prompt": lambda: bl.based_prefill(q2, k2, v2, y=y, S_out=S, z_out=z),
                "rnn": lambda: bl.jrt_prefix_prefill(q, k, v, ke, ve, y=y1, S_out=S, z_out=z)}
        # shorter sequences get proportionally more launches, so that every series spans
        # about the same GPU time as the longest one
        n = steps * max(1, max(TABLE5_H100_MS) // L)
        times = {key: [] for key in runs}
        for _ in range(TABLE5_ROUNDS):
            for key, fn in runs.items():
                times[key].append(time_launches(fn, n, warmup * max(1, max(TABLE5_H100_MS) // L)) / n)
        t_based, t_prompt, t_rnn = (sorted(times[key])[TABLE5_ROUNDS // 2] for key in runs)
        log(f"[table5] L={L}: based {t_based * 1e3:.3f} ms, jrt_prompt {t_prompt * 1e3:.3f} ms, "
            f"jrt_rnn {t_rnn * 1e3:.3f} ms")
        rows.append({"L": L, "based_ms": round(t_based * 1e3, 4),
                     "jrt_prompt_ms": round(t_prompt * 1e3, 4),
                     "jrt_rnn_ms": round(t_rnn * 1e3, 4),
                     "jrt_prompt_over_based": round(t_prompt / t_based, 3),
                     "jrt_rnn_over_based": round(t_rnn / t_based, 3),
                     "h100_ms_based_prompt_rnn": list(h100)})
        del q, k, v, ke, ve, q2, k2, v2, y, y1, S, z
        torch.cuda.empty_cache()
    return {"workload": "Table 5 sweep: B=16 H=16 d'=16 d_v=64 bf16 in, fp32 y; JRT-Prompt = "
                        "prefill over the prompt repeated (2L tokens); JRT-RNN = M=L/2 prefix + "
                        "N=L causal", "rows": rows}


SWA_SRC = os.path.join(ROOT, "recurrent_lm_sequence_amd", "csrc", "swa.hip")
PREFILL_SRC = os.path.join(ROOT, "recurrent_lm_sequence_amd", "csrc", "prefill_sym.hip")


def bench_swa(bl, gen, steps, warmup):
    """Sliding-window softmax attention at the long-prefill shape (B=16, H=16,
    N=32768, d=d_v=64, bf16 in, fp32 y) for windows 64 and 128, and its decode
    step on a ring cache at the decode shape (B=256, H=16, window 128)."""
    import torch

    out = {}
    w = gen.Workload("swa_prefill", B=16, H=16, N=32768, d_feat=64, d_v=64, dtype="bf16", seed=1200)
    q, k, v = gen.make_prefill_inputs(w, "cuda:0")
    y = torch.empty((w.B, w.H, w.N, 64), dtype=torch.float32, device="cuda:0")
    for window in (64, 128):
        per = time_launches(lambda: bl.swa_prefill(q, k, v, window, y=y), steps, warmup) / steps
        # HBM: q, k, v bf16 in (3 x 128 B) + y fp32 out (256 B) per token-head
        gbs = w.B * w.H * w.N * 640 / per / 1e9
        # matrix-core work actually issued: 16 queries x (window + 32) keys x 64 x 2 (scores)
        # and the same for the value product, per token
        log(f"[swa] prefill w={window}: {per * 1e3:.3f} ms, {w.B * w.N / per / 1e6:.1f} M tokens/s, "
            f"{gbs:.0f} GB/s")
        out[f"prefill_w{window}"] = {"ms": round(per * 1e3, 4), "tokens_per_s": w.B * w.N / per,
                                     "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                                                  "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                                  "frac": round(gbs / HBM_PEAK_GBS, 4),
                                                  "traffic": committed_traffic(
                                                      SWA_SRC, f"swa_prefill_w{window}.md")}}
    del q, k, v, y
    torch.cuda.empty_cache()
    B, H, window, nsteps = 256, 16, 128, 64
    wd = gen.Workload("swa_decode", B=B, H=H, N=window, d_feat=64, d_v=64, dtype="bf16", seed=1201)
    q, k, v = gen.make_prefill_inputs(wd, "cuda:0")
    _, kc, vc = bl.swa_prefill(q, k, v, window, want_cache=True)
    qs = torch.empty((nsteps, B, H, 64), dtype=torch.bfloat16, device="cuda:0")
    ks, vs = torch.empty_like(qs), torch.empty_like(qs)
    for i in range(nsteps):
        qs[i], ks[i], vs[i] = gen.make_decode_step_inputs(
            gen.Workload("swa_dec", B=B, H=H, N=0, d_feat=64, d_v=64, dtype="bf16", seed=1202), i,
            "cuda:0")
    yd = torch.empty((nsteps, B, H, 64), dtype=torch.float32, device="cuda:0")
    kc0, vc0 = kc.clone(), vc.clone()
    torch.cuda.synchronize()
    s0 = torch.cuda.Event(enable_timing=True)
    e0 = torch.cuda.Event(enable_timing=True)
    s0.record()
    for i in range(nsteps):
        bl.swa_decode_step(qs[i], ks[i], vs[i], kc, vc, window + i, window, y=yd[i])
    e0.record()
    torch.cuda.synchronize()
    per = s0.elapsed_time(e0) / 1e3 / nsteps
    # the same steps captured in one HIP graph, replayed from the cache they started from
    yg = torch.empty_like(yd)
    kcg, vcg = kc0.clone(), vc0.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        bl.swa_decode_step(qs[0], ks[0], vs[0], kc0.clone(), vc0.clone(), window, window)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(nsteps):
            bl.swa_decode_step(qs[i], ks[i], vs[i], kcg, vcg, window + i, window, y=yg[i])
    gt = []
    for _ in range(3):
        kcg.copy_(kc0)
        vcg.copy_(vc0)
        torch.cuda.synchronize()
        sg, eg = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        sg.record()
        g.replay()
        eg.record()
        torch.cuda.synchronize()
        if not (torch.equal(yg, yd) and torch.equal(kcg, kc)):
            raise SystemExit("SWA decode graph replay differs from the eager steps")
        gt.append(sg.elapsed_time(eg) / 1e3 / nsteps)
    per_graph = sorted(gt)[1]
    del g, kcg, vcg, yg, kc0, vc0
    # per head: the window's keys and values read (2 x 128 x 64 x 2 B), one slot of each written,
    # q, k, v in, y out
    bytes_head = 2 * window * 64 * 2 + 2 * 64 * 2 + 3 * 64 * 2 + 64 * 4
    gbs = B * H * bytes_head / per / 1e9
    log(f"[swa] decode w={window}: {per * 1e6:.2f} us/step, {B / per / 1e6:.3f} M tokens/s, {gbs:.0f} GB/s; "
        f"in a graph {per_graph * 1e6:.2f} us/step")
    out["decode_w128"] = {"workload": f"B={B} H={H} window={window} d=d_v=64 bf16 ring cache",
                          "us_per_step": round(per * 1e6, 3), "tokens_per_s": B / per,
                          "graph": {"us_per_step": round(per_graph * 1e6, 3), "tokens_per_s": B / per_graph,
                                    "roofline_frac": round(B * H * bytes_head / per_graph / 1e9 / HBM_PEAK_GBS, 4),
                                    "note": f"all {nsteps} steps captured in one HIP graph; outputs equal "
                                            "the eager steps"},
                          "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                                       "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                       "frac": round(gbs / HBM_PEAK_GBS, 4),
                                       "traffic": committed_traffic(SWA_SRC, "swa_decode_w128.md")}}
    out["workload"] = "swa_prefill B=16 H=16 N=32768 d=d_v=64 bf16 in fp32 y, windows 64/128"
    del q, k, v, kc, vc, qs, ks, vs, yd
    torch.cuda.empty_cache()
    return out


def bench_decode(bl, gen, warmup, compact=False, with_oracle=False):
    import torch

    w = gen.STATE_DECODE
    tag = "decode_compact" if compact else "decode"
    log(f"[{tag}] building the initial state with an untimed {w.N}-token prefill")
    q, k, v = gen.make_prefill_inputs(w, "cuda:0")
    _, S, z = bl.based_prefill(q, k, v, want_y=False, compact=compact)
    del q, k, v
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    steps = w.decode_steps
    log(f"[{tag}] generating {steps} steps of inputs")
    qs = torch.empty((steps, w.B, w.H, w.d_feat), dtype=torch.bfloat16, device="cuda:0")
    ks = torch.empty_like(qs)
    vs = torch.empty((steps, w.B, w.H, w.d_v), dtype=torch.bfloat16, device="cuda:0")
    for i in range(steps):
        qs[i], ks[i], vs[i] = gen.make_decode_step_inputs(w, i, "cuda:0")
    ys = torch.empty((steps, w.B, w.H, w.d_v), dtype=torch.float32, device="cuda:0")
    Sc, zc = S.clone(), z.clone()  # warm up on a scratch copy so the timed run starts from S0
    for i in range(warmup):
        bl.based_decode_step(qs[i], ks[i], vs[i], Sc, zc, y=ys[i], compact=compact)
    S0_host = S.cpu() if with_oracle else None  # the state the timed steps start from
    z0_host = z.cpu() if with_oracle else None
    del Sc, zc
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(steps):
        bl.based_decode_step(qs[i], ks[i], vs[i], S, z, y=ys[i], compact=compact)
    e.record()
    torch.cuda.synchronize()
    t = s.elapsed_time(e) / 1e3
    per = t / steps
    bytes_step = w.B * w.H * (DECODE_COMPACT_BYTES_PER_HEAD if compact else DECODE_BYTES_PER_HEAD)
    gbs = bytes_step / per / 1e9
    log(f"[{tag}] {per * 1e6:.2f} us/step, {w.B / per / 1e6:.3f} M tokens/s, {gbs:.0f} GB/s")
    out = {"workload": f"state_passing_decode B={w.B} H={w.H} d'={w.d_feat} d_v={w.d_v} "
                       f"{'compact 153-row' if compact else 'full 273-row'} state, "
                       f"S0 from {w.N}-token prefill, {steps} steps",
           "us_per_step": round(per * 1e6, 3), "tokens_per_s": w.B / per,
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "traffic": committed_traffic(
                            os.path.join(ROOT, "recurrent_lm_sequence_amd", "csrc", "decode.hip"),
                            "decode_compact_state_passing.md" if compact
                            else "decode_state_passing.md")}}
    out["graph"] = decode_graph(bl, qs, ks, vs, ys, S, z, compact, bytes_step)
    if with_oracle:
        out["cpu_baseline"] = decode_cpu_baseline(w, qs, ks, vs, ys, S0_host, z0_host)
    del qs, ks, vs, S, z, ys
    torch.cuda.empty_cache()
    return out


def decode_graph(bl, qs, ks, vs, ys, S, z, compact, bytes_step):
    """The same 512 decode steps captured in one HIP graph (the pages time decode with
    CUDA graphs) and replayed from the state the eager steps ended with; each replay's
    outputs are checked against an eager run of the same steps from that state."""
    import torch

    steps = qs.shape[0]
    S1, z1 = S.clone(), z.clone()
    y_eager = torch.empty_like(ys)
    Se, ze = S1.clone(), z1.clone()
    for i in range(steps):
        bl.based_decode_step(qs[i], ks[i], vs[i], Se, ze, y=y_eager[i], compact=compact)
    yg = torch.empty_like(ys)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        bl.based_decode_step(qs[0], ks[0], vs[0], S1.clone(), z1.clone(), compact=compact)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    Sg, zg = S1.clone(), z1.clone()
    with torch.cuda.graph(g):
        for i in range(steps):
            bl.based_decode_step(qs[i], ks[i], vs[i], Sg, zg, y=yg[i], compact=compact)
    times = []
    for _ in range(3):
        Sg.copy_(S1)
        zg.copy_(z1)
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        g.replay()
        e.record()
        torch.cuda.synchronize()
        if not (torch.equal(yg, y_eager) and torch.equal(Sg, Se)):
            raise SystemExit("decode graph replay differs from the eager steps")
        times.append(s.elapsed_time(e) / 1e3 / steps)
    per = sorted(times)[1]
    log(f"[decode graph] {per * 1e6:.2f} us/step (median of 3 replays of {steps} captured steps)")
    del g, Sg, zg, S1, z1, Se, ze, y_eager, yg
    return {"us_per_step": round(per * 1e6, 3), "tokens_per_s": qs.shape[1] / per,
            "roofline_frac": round(bytes_step / per / 1e9 / HBM_PEAK_GBS, 4),
            "note": "all steps captured in one HIP graph and replayed; outputs equal the eager steps"}


def decode_cpu_baseline(w, qs, ks, vs, ys, S0, z0):
    """The fp64 oracle's decode step over the same 512 steps and all heads, from the
    state the timed GPU steps started from, timed on the host cores; every step's y
    is also checked against the GPU's (2e-3 per row)."""
    import numpy as np

    import oracle
    from tests.parity_util import TOL_BF16, worst_row_error

    threads = oracle.default_threads()
    steps = qs.shape[0]
    Sr = np.ascontiguousarray(S0.double().numpy())
    zr = np.ascontiguousarray(z0.double().numpy())
    qh, kh, vh = qs.cpu(), ks.cpu(), vs.cpu()
    yg = ys.cpu()
    log(f"[decode cpu_baseline] oracle: {steps} steps x {w.B * w.H} heads, {threads} threads")
    worst, spent = 0.0, 0.0
    for i in range(steps):
        t0 = time.perf_counter()
        yr, Sr, zr = oracle.decode_step(qh[i], kh[i], vh[i], Sr, zr, nthreads=threads, in_place=True)
        spent += time.perf_counter() - t0
        worst = max(worst, worst_row_error(yg[i].numpy(), yr))
    log(f"[decode cpu_baseline] {spent:.2f} s, worst row error of the timed steps' y {worst:.3e}")
    if not worst <= TOL_BF16:
        raise SystemExit(f"decode parity failed: worst row error {worst:.3e} > {TOL_BF16}")
    return {"value": w.B * steps / spent, "unit": "tokens/s", "cores": threads,
            "nproc": oracle.host_cores(), "kind": "oracle",
            "sample": f"all {w.B} x {w.H} heads x {steps} decode steps (fp64 state, "
                      f"273 rows), from the state the timed GPU steps started from; {spent:.1f} s",
            "parity_worst_row_error": worst}


def cpu_baseline(pre):
    """The fp64 oracle on host cores over the whole long-prefill batch."""
    import oracle
    from tests.parity_util import worst_row_error

    from tests.parity_util import TOL_BF16

    w = pre["w"]
    threads = oracle.default_threads()
    q, k, v = pre["q"].cpu(), pre["k"].cpu(), pre["v"].cpu()
    log(f"[cpu_baseline] oracle on {w.B} x {w.H} heads x {w.N} tokens, {threads} threads "
        f"({oracle.host_cores()} cores in this process's affinity, os.cpu_count() {os.cpu_count()})")
    t0 = time.perf_counter()
    yr, _, _ = oracle.prefill(q, k, v, nthreads=threads)
    dt = time.perf_counter() - t0
    err = worst_row_error(pre["y"].cpu().numpy(), yr)
    log(f"[cpu_baseline] {dt:.2f} s, worst row error of the timed launch's output {err:.3e}")
    if not err <= TOL_BF16:
        raise SystemExit(f"long-prefill parity failed: worst row error {err:.3e} > {TOL_BF16}")
    return ({"value": w.B * w.N / dt, "unit": "tokens/s", "cores": threads,
             "nproc": oracle.host_cores(), "kind": "oracle",
             "sample": f"the whole long_prefill batch: {w.B} x {w.H} heads x {w.N} tokens "
                       f"({w.B * w.H * w.N} token-heads), fp64 token-by-token recurrence, "
                       f"{dt:.1f} s"},
            float(err))


def copy_probe():
    """A plain 1 GiB device copy: calibrates rocprofv3 FETCH_SIZE/WRITE_SIZE counters and
    gives the copy bandwidth of the box (read + write bytes per second)."""
    import torch

    n = 1 << 28
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(10):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    per = s.elapsed_time(e) / 1e3 / 10
    print(json.dumps({"copy_probe_bytes_read": 4 * n, "copy_probe_bytes_written": 4 * n,
                      "copy_ms": round(per * 1e3, 4), "copy_GBps_read_plus_write": round(8 * n / per / 1e9, 1)}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["all", "prefill", "jrt", "small", "single", "decode", "decode_compact",
                                       "table5", "swa", "peaks"], default="all")
    ap.add_argument("--copy-probe", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(--gpus {args.gpus} requested). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        copy_probe()
        return

    from recurrent_lm_sequence_amd import based_la as bl
    from recurrent_lm_sequence_amd import inputs as gen

    result = {"metric": METRIC}
    extra = {}
    pre = None
    if args.only in ("all", "prefill"):
        pre = bench_prefill(bl, gen, args.steps, args.warmup)
    if args.only in ("all", "jrt"):
        extra["jrt"] = bench_jrt(bl, gen, args.steps, args.warmup)
    if args.only in ("all", "small"):
        extra.update(bench_small_configs(bl, gen, args.steps, args.warmup))
    if args.only in ("all", "single"):
        extra.update(bench_small_configs(bl, gen, args.steps, args.warmup, which=("single_sequence",)))
    if args.only in ("all", "decode"):
        extra["decode"] = bench_decode(bl, gen, args.warmup,
                                       with_oracle=not args.no_cpu_baseline)
    if args.only in ("all", "decode_compact"):
        extra["decode_compact"] = bench_decode(bl, gen, args.warmup, compact=True)
    if args.only in ("all", "swa"):
        extra["swa"] = bench_swa(bl, gen, min(args.steps, 10), min(args.warmup, 2))
    if args.only in ("all", "table5"):
        extra["table5"] = bench_table5(bl, gen, min(args.steps, 10), min(args.warmup, 2))
    peaks = measured_peaks(bl) if args.only in ("all", "peaks") else None

    if pre is not None:
        w = pre["w"]
        per = pre["per"]
        gbs = pre["alg_bytes"] / per / 1e9
        tfl = pre["alg_flop"] / per / 1e12
        result.update({
            "value": w.B * w.N / per, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(per * 1e3, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": round(w.B * w.N / per / H100_BASED_TOKENS_PER_S, 3),
            "dtype": "f16",
            "dtype_detail": "bf16 inputs; fp16 matrix-core operands; fp32 accumulation, "
                            "state, denominators and y",
            "data": "synthetic (seeded N(0,1), bf16)",
            "config": {"workload": f"long_prefill B={w.B} H={w.H} N={w.N} d'={w.d_feat} "
                                   f"D={w.feature_dim} d_v={w.d_v} chunk=128 zero initial state"},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": committed_traffic(PREFILL_SRC, "prefill_ws_long_prefill.md")},
            "mfma": {"achieved": round(tfl, 1), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tfl / MFMA_F16_PEAK_TFLOPS, 4),
                     "flop_per_launch": pre["alg_flop"],
                     "formula": f"{FLOP_PER_TOKEN_HEAD} FLOP per token-head: 2*64*(16+64) "
                                f"intra-chunk (64-token tile) + 2*2*{D_CONTRACTED}*64 inter-chunk "
                                f"and update at the D the kernel contracts"},
            "launch_stats": dict(pre["launch_stats"], note="HIP events after every timed launch; "
                                 "ms_per_step is the mean over the bracket of all of them"),
            "prefill_bf16_y": pre["bf16_y"],
            "context_h100": {"based_custom_cuda_tokens_per_s": H100_BASED_TOKENS_PER_S,
                             "note": "vs_baseline divides by the pages' H100 prefill figure "
                                     "(custom CUDA kernel, 4.5 ms at batch 16, N=32768; heads "
                                     "and widths not printed): context from another machine, "
                                     "not a target"},
        })
    result.update(extra)
    if pre is not None:
        ex = committed_executed_flop(PREFILL_SRC, "prefill_ws_long_prefill.md")
        result["mfma"]["executed_flop_per_launch"] = ex
        result["mfma"]["executed_frac"] = (round(ex / pre["per"] / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)
                                           if ex else None)
        fl = pre["traffic_floor"]
        result["roofline"]["traffic_floor"] = dict(fl, note=(
            "bla_probe_prefill_traffic: this launch's HBM traffic (q, k, v bf16 in, fp32 y out, one "
            "workgroup per head in 128-token chunks) with none of its arithmetic"))
        result["roofline"]["frac_of_traffic_floor"] = round(fl["reads_and_writes"]["ms"] / (pre["per"] * 1e3), 4)
        if peaks:
            result["measured_peaks"] = peaks
            result["roofline"]["frac_of_measured_peak"] = round(
                result["roofline"]["achieved"] / peaks["hbm_copy_gbs"], 4)
            result["mfma"]["frac_of_measured_peak"] = round(
                result["mfma"]["achieved"] / peaks["mfma_f16_tflops"], 4)
    elif peaks:
        result["measured_peaks"] = peaks
    if pre is not None and not args.no_cpu_baseline:
        result["cpu_baseline"], result["parity_worst_row_error_sample"] = cpu_baseline(pre)
    if "value" not in result and ("decode" in result or "decode_compact" in result):
        d = result.get("decode") or result["decode_compact"]
        result.update({"value": d["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
                       "steps": 512, "warmup": args.warmup,
                       "ms_per_step": d["us_per_step"] / 1e3, "higher_is_better": True,
                       "scaling": "weak", "vs_baseline": None, "dtype": "f32",
                       "data": "synthetic", "config": {"workload": d["workload"]},
                       "roofline": d["roofline"]})
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
