"""Compact (folded) state layout of the Taylor feature map, in fp64 numpy.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

"Simple linear attention language models balance the recall-throughput
tradeoff" notes, §2.3: phi(x) = [1, xb, vec(xb xb^T)/sqrt(2)], xb = x/d^(1/4);
the notes remark that the quadratic block repeats features (entry (a, b)
equals entry (b, a)).  Therefore phi(q)^T S = sum_{a,b} (xb_a xb_b/sqrt 2)
S[(a,b)] + (orders 0 and 1) depends on S only through S[(a,b)] + S[(b,a)].

The compact layout keeps, for every unordered pair a <= b (row-major upper
triangle), that sum, after the d + 1 rows of orders 0 and 1:
    rows: [1 | xb (d) | pair (a, b), a <= b]   (1 + d + d(d+1)/2 rows)
The compact oracle calls are the full fp64 recurrence of ``oracle`` wrapped
by these plain index maps: a compact initial state is unfolded into a
symmetric full state (any full state with the same fold gives the same
outputs), the full recurrence runs, and its final state is folded.
"""
from __future__ import annotations

import numpy as np


def compact_dim(d: int) -> int:
    return 1 + d + d * (d + 1) // 2


def pair_list(d: int) -> list[tuple[int, int]]:
    """Unordered pairs (a, b), a <= b, in the order of the compact pair rows."""
    return [(a, b) for a in range(d) for b in range(a, d)]


def _full_row(d: int, a: int, b: int) -> int:
    return 1 + d + a * d + b


def fold(S: np.ndarray, d: int, axis: int) -> np.ndarray:
    """Full layout (axis of length 1 + d + d*d) -> compact layout (sum of both orders)."""
    S = np.moveaxis(np.asarray(S, dtype=np.float64), axis, 0)
    out = np.zeros((compact_dim(d),) + S.shape[1:])
    out[: 1 + d] = S[: 1 + d]
    for p, (a, b) in enumerate(pair_list(d)):
        out[1 + d + p] = S[_full_row(d, a, b)]
        if a != b:
            out[1 + d + p] += S[_full_row(d, b, a)]
    return np.ascontiguousarray(np.moveaxis(out, 0, axis))


def unfold(Sc: np.ndarray, d: int, axis: int) -> np.ndarray:
    """Compact layout -> the symmetric full state with the same fold."""
    Sc = np.moveaxis(np.asarray(Sc, dtype=np.float64), axis, 0)
    out = np.zeros((1 + d + d * d,) + Sc.shape[1:])
    out[: 1 + d] = Sc[: 1 + d]
    for p, (a, b) in enumerate(pair_list(d)):
        if a == b:
            out[_full_row(d, a, a)] = Sc[1 + d + p]
        else:
            out[_full_row(d, a, b)] = 0.5 * Sc[1 + d + p]
            out[_full_row(d, b, a)] = 0.5 * Sc[1 + d + p]
    return np.ascontiguousarray(np.moveaxis(out, 0, axis))


def compact_feature_map(x: np.ndarray) -> np.ndarray:
    """phi_c(x) = [1, xb, xb_a xb_b / sqrt(2) for a <= b]: the query-side feature
    of the compact state, so that phi(q)^T S == phi_c(q)^T fold(S)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    xb = x / d ** 0.25
    pairs = [xb[..., a] * xb[..., b] / np.sqrt(2.0) for a, b in pair_list(d)]
    ones = np.ones(x.shape[:-1] + (1,))
    return np.concatenate([ones, xb, np.stack(pairs, axis=-1)], axis=-1)


def pair_multiplicity(d: int) -> np.ndarray:
    """How many full-layout rows each compact row stands for (2 off the diagonal)."""
    m = np.ones(compact_dim(d))
    for p, (a, b) in enumerate(pair_list(d)):
        if a != b:
            m[1 + d + p] = 2.0
    return m
