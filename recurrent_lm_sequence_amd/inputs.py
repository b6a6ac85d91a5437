"""Seeded synthetic inputs and the workload table.

This module holds no arithmetic of the method: it only draws i.i.d. N(0,1)
values (fp32, then rounded to bf16 with round-to-nearest-even where the
workload asks for bf16) from a seeded generator.  Both the HIP path and the
CPU oracle consume exactly the tensors it returns; the oracle reads them as
exact fp64 values, so input quantisation never counts as error.

The workloads mirror the shapes the pages benchmark: BASED's linear-attention
layers use 16 heads with feature dimension d' = 16 (D = 1 + 16 + 256 = 273),
value width 64 ("Simple linear attention language models balance the
recall-throughput tradeoff" notes, Table 7 in §2.4), the prefill latency sweep
runs batch 16 up to N = 32768 ("Just read twice" notes, Table 5 in §4.8), and
JRT-RNN splits a sequence into a non-causal prefix of M tokens and the causal
rest (same notes, §2.6).  The pages benchmark on random inputs, not on a
dataset, so unstructured N(0,1) data is the plain stand-in.
"""
from __future__ import annotations

import dataclasses
import hashlib

import torch

# stream identifiers: one independent generator per tensor role
STREAM_Q, STREAM_K, STREAM_V, STREAM_KE, STREAM_VE = 0, 1, 2, 3, 4
STREAM_DECODE_BASE = 100  # per-step decode inputs use STREAM_DECODE_BASE + step


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int  # causal tokens (for decode: length of the prefill that builds S0)
    d_feat: int
    d_v: int
    dtype: str  # "f32" or "bf16"
    seed: int
    M: int = 0  # JRT prefix length
    decode_steps: int = 0  # >0: state-passing decode workload

    @property
    def feature_dim(self) -> int:
        return 1 + self.d_feat + self.d_feat * self.d_feat


TINY_F32 = Workload("tiny_causal_f32", B=1, H=1, N=256, d_feat=16, d_v=16, dtype="f32", seed=1001)
LAYER_PREFILL = Workload("based_layer_prefill", B=8, H=16, N=2048, d_feat=16, d_v=64,
                         dtype="bf16", seed=1002)
LONG_PREFILL = Workload("long_prefill", B=16, H=16, N=32768, d_feat=16, d_v=64, dtype="bf16",
                        seed=1003)
JRT_PREFIX = Workload("jrt_prefix", B=16, H=16, N=4096, M=2048, d_feat=16, d_v=64, dtype="bf16",
                      seed=1004)
STATE_DECODE = Workload("state_passing_decode", B=256, H=16, N=8192, d_feat=16, d_v=64,
                        dtype="bf16", seed=1005, decode_steps=512)

WORKLOADS = (TINY_F32, LAYER_PREFILL, LONG_PREFILL, JRT_PREFIX, STATE_DECODE)


def _stream_seed(seed: int, stream: int) -> int:
    h = hashlib.sha256(f"{seed}:{stream}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def normal(shape, seed: int, stream: int, dtype: str = "bf16", device="cpu") -> torch.Tensor:
    """i.i.d. N(0,1) drawn in fp32 from a generator seeded by (seed, stream),
    rounded to bf16 (round-to-nearest-even) when dtype == "bf16"."""
    g = torch.Generator(device=device)
    g.manual_seed(_stream_seed(seed, stream))
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    if dtype == "f32":
        return x
    raise ValueError(f"unknown dtype {dtype!r}")


def make_prefill_inputs(w: Workload, device="cpu", N: int | None = None):
    """(q, k, v) of shapes [B,H,N,d'], [B,H,N,d'], [B,H,N,d_v]."""
    N = w.N if N is None else N
    q = normal((w.B, w.H, N, w.d_feat), w.seed, STREAM_Q, w.dtype, device)
    k = normal((w.B, w.H, N, w.d_feat), w.seed, STREAM_K, w.dtype, device)
    v = normal((w.B, w.H, N, w.d_v), w.seed, STREAM_V, w.dtype, device)
    return q, k, v


def make_prefix_inputs(w: Workload, device="cpu"):
    """(k_e, v_e) of shapes [B,H,M,d'], [B,H,M,d_v] for the JRT prefix."""
    ke = normal((w.B, w.H, w.M, w.d_feat), w.seed, STREAM_KE, w.dtype, device)
    ve = normal((w.B, w.H, w.M, w.d_v), w.seed, STREAM_VE, w.dtype, device)
    return ke, ve


def make_decode_step_inputs(w: Workload, step: int, device="cpu"):
    """Fresh (q, k, v) for one decode step: [B,H,d'], [B,H,d'], [B,H,d_v]."""
    s = STREAM_DECODE_BASE + 3 * step
    q = normal((w.B, w.H, w.d_feat), w.seed, s, w.dtype, device)
    k = normal((w.B, w.H, w.d_feat), w.seed, s + 1, w.dtype, device)
    v = normal((w.B, w.H, w.d_v), w.seed, s + 2, w.dtype, device)
    return q, k, v


def state_noise(B: int, H: int, D: int, d_v: int, seed: int, device="cpu"):
    """i.i.d. N(0,1) fp32 arrays shaped like a state (S [B,H,D,d_v], z [B,H,D]).
    Tests add a scaled copy to a physical state to get a generic, non-symmetric
    initial state."""
    S = normal((B, H, D, d_v), seed, 10_000_000, "f32", device)
    z = normal((B, H, D), seed, 10_000_001, "f32", device)
    return S, z
