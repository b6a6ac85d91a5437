"""Sliding-window softmax attention (SWA), fp64 numpy.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

"Simple linear attention language models balance the recall-throughput
tradeoff" notes, §2.4: SWA computes standard softmax attention only over the
keys j in [max(1, i-w+1), i] (1-based) and keeps the most recent w keys and
values per head; §2.5: decoding fuses the dot products, the softmax and the
weighted sum over the window.  Readings taken here: the score scale is
1/sqrt(d) (standard softmax attention), no rotary embedding (the pages' SWA
kernel test excludes it), and the decode cache is a ring of w slots in which
token p (0-based) sits in slot p mod w.
"""
from __future__ import annotations

import numpy as np


def swa_prefill(q, k, v, window: int) -> np.ndarray:
    """y [..., N, dv]: y_i = sum_{j = max(0, i-w+1)}^{i} softmax_j(q_i.k_j / sqrt(d)) v_j.
    Written as the plain definition: one softmax per query row over its window."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    N, d = q.shape[-2], q.shape[-1]
    y = np.zeros(q.shape[:-1] + (v.shape[-1],))
    for i in range(N):
        lo = max(0, i - window + 1)
        s = np.einsum("...d,...jd->...j", q[..., i, :], k[..., lo:i + 1, :]) / np.sqrt(d)
        s = s - s.max(axis=-1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=-1, keepdims=True)
        y[..., i, :] = np.einsum("...j,...jc->...c", p, v[..., lo:i + 1, :])
    return y


def swa_prefill_blocked(q, k, v, window: int, block: int = 256) -> np.ndarray:
    """The same y as ``swa_prefill``, with one matrix product per block of
    queries instead of one per query (for full-size checks).  For the queries
    i in [i0, i1) the scores against the keys j in [max(0, i0-w+1), i1) are
    formed at once, every entry outside j in [i-w+1, i] is set to -inf, and
    each row is then the same max-shifted softmax and weighted sum."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    N, d = q.shape[-2], q.shape[-1]
    y = np.zeros(q.shape[:-1] + (v.shape[-1],))
    for i0 in range(0, N, block):
        i1 = min(N, i0 + block)
        lo = max(0, i0 - window + 1)
        s = np.matmul(q[..., i0:i1, :], np.swapaxes(k[..., lo:i1, :], -1, -2)) / np.sqrt(d)
        i = np.arange(i0, i1)[:, None]
        j = np.arange(lo, i1)[None, :]
        s = np.where((j <= i) & (j > i - window), s, -np.inf)
        s = s - s.max(axis=-1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=-1, keepdims=True)
        y[..., i0:i1, :] = np.matmul(p, v[..., lo:i1, :])
    return y


def swa_cache_from_prefill(k, v, window: int):
    """The ring cache after a prefill of N tokens: slot p mod w holds token p for
    the last min(N, w) tokens (other slots zero)."""
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    N = k.shape[-2]
    kc = np.zeros(k.shape[:-2] + (window, k.shape[-1]))
    vc = np.zeros(v.shape[:-2] + (window, v.shape[-1]))
    for p in range(max(0, N - window), N):
        kc[..., p % window, :] = k[..., p, :]
        vc[..., p % window, :] = v[..., p, :]
    return kc, vc


def swa_decode_step(q, k, v, k_cache, v_cache, pos: int, window: int):
    """One step for the token at position pos: write (k, v) into slot pos mod w,
    then attend over the min(pos+1, w) most recent tokens.  Returns
    (y [..., dv], k_cache', v_cache') without modifying the inputs."""
    q = np.asarray(q, np.float64)
    kc = np.array(k_cache, np.float64)
    vc = np.array(v_cache, np.float64)
    kc[..., pos % window, :] = np.asarray(k, np.float64)
    vc[..., pos % window, :] = np.asarray(v, np.float64)
    slots = [p % window for p in range(max(0, pos - window + 1), pos + 1)]
    d = q.shape[-1]
    s = np.einsum("...d,...jd->...j", q, kc[..., slots, :]) / np.sqrt(d)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    y = np.einsum("...j,...jc->...c", p, vc[..., slots, :])
    return y, kc, vc
