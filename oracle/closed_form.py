"""O(N^2) attention form of Taylor linear attention, in fp64 numpy.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

"Simple linear attention language models balance the recall-throughput
tradeoff" notes, §2.2: y_i = sum_{j<=i} K(q_i,k_j) v_j / sum_{j<=i} K(q_i,k_j);
§2.3, Eq. (4) with the dimension normalisation:
K(q,k) = 1 + q.k/sqrt(d') + (q.k)^2/(2 d').
"Just read twice" notes, §2.6, Eq. (3): the prefix keys/values enter every
position's sums (non-causal), the decoder keys/values causally.
A non-zero initial state adds phi(q_i)^T S0 to the numerator and
phi(q_i)^T z0 to the denominator (length-generalization notes, §2.5, Eq. (4),
with the identity transition of linear attention).
"""
from __future__ import annotations

import numpy as np


def taylor_kernel(q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """K(q_i, k_j) for all pairs: q [..., N, d], k [..., M, d] -> [..., N, M]."""
    d = q.shape[-1]
    t = np.matmul(q, np.swapaxes(k, -1, -2))
    return 1.0 + t / np.sqrt(d) + t * t / (2.0 * d)


def feature_map_np(x: np.ndarray) -> np.ndarray:
    """phi(x) = [1, x/d^(1/4), vec(xb xb^T)/sqrt(2)] with xb = x/d^(1/4), a-major vec.
    Written independently of the C oracle (numpy outer products)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    xb = x / d ** 0.25
    outer = xb[..., :, None] * xb[..., None, :]
    ones = np.ones(x.shape[:-1] + (1,))
    return np.concatenate([ones, xb, outer.reshape(x.shape[:-1] + (d * d,)) / np.sqrt(2.0)], axis=-1)


def closed_form_prefill(q, k, v, S0=None, z0=None, eps: float = 0.0) -> np.ndarray:
    """y [B,H,N,dv] from the quadratic (attention) form with a causal mask j <= i."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    N = q.shape[-2]
    A = taylor_kernel(q, k) * np.tril(np.ones((N, N)))
    num = A @ v
    den = A.sum(-1)
    if S0 is not None:
        phq = feature_map_np(q)
        num = num + phq @ np.asarray(S0, np.float64)
        den = den + np.einsum("...nf,...f->...n", phq, np.asarray(z0, np.float64))
    return num / (den[..., None] + eps)


def closed_form_jrt(q, k, v, ke, ve, S0=None, z0=None, eps: float = 0.0) -> np.ndarray:
    """Eq. (3) of the JRT notes in attention form: every prefix key counts for
    every position, decoder keys only for j <= i."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    ke = np.asarray(ke, np.float64)
    ve = np.asarray(ve, np.float64)
    N = q.shape[-2]
    A = taylor_kernel(q, k) * np.tril(np.ones((N, N)))
    E = taylor_kernel(q, ke)
    num = A @ v + E @ ve
    den = A.sum(-1) + E.sum(-1)
    if S0 is not None:
        phq = feature_map_np(q)
        num = num + phq @ np.asarray(S0, np.float64)
        den = den + np.einsum("...nf,...f->...n", phq, np.asarray(z0, np.float64))
    return num / (den[..., None] + eps)
