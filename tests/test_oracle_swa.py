"""Pins of the oracle's sliding-window softmax attention ("Simple linear
attention language models balance the recall-throughput tradeoff" notes, §2.4
and §2.5), against a library softmax over a dense banded mask, special cases
with closed forms, a hand-computed example and decode/prefill agreement.
"""
import numpy as np
import pytest
from scipy.special import softmax

import oracle


def rng(seed):
    return np.random.default_rng(seed)


def rel_err(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def banded_reference(q, k, v, w):
    # dense scores with a band mask, scipy's softmax (a different formulation)
    N, d = q.shape[-2], q.shape[-1]
    s = q @ np.swapaxes(k, -1, -2) / np.sqrt(d)
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    s = np.where((j <= i) & (j > i - w), s, -np.inf)
    return softmax(s, axis=-1) @ v


@pytest.mark.parametrize("w", [1, 3, 16, 64])
def test_prefill_matches_banded_softmax(w):
    r = rng(w)
    q, k = r.standard_normal((2, 3, 70, 8)), r.standard_normal((2, 3, 70, 8))
    v = r.standard_normal((2, 3, 70, 5))
    assert rel_err(oracle.swa_prefill(q, k, v, w), banded_reference(q, k, v, w)) < 1e-12


@pytest.mark.parametrize("w,block", [(1, 7), (5, 3), (16, 16), (64, 50), (64, 200), (100, 33), (128, 256)])
def test_blocked_prefill_matches_banded_softmax(w, block):
    # the blocked form (one product per block of queries, for full-size checks) against
    # scipy's softmax over the dense band and against the per-row form: blocks smaller
    # than, equal to and larger than the window, a ragged last block, scores near 40 (the
    # max shift matters)
    r = rng(100 + w + block)
    q, k = 3.0 * r.standard_normal((2, 2, 150, 8)), 3.0 * r.standard_normal((2, 2, 150, 8))
    v = r.standard_normal((2, 2, 150, 5))
    yb = oracle.swa_prefill_blocked(q, k, v, w, block=block)
    assert rel_err(yb, banded_reference(q, k, v, w)) < 1e-12
    assert rel_err(yb, oracle.swa_prefill(q, k, v, w)) < 1e-12


def test_window_one_returns_v():
    r = rng(1)
    q, k, v = r.standard_normal((20, 4)), r.standard_normal((20, 4)), r.standard_normal((20, 3))
    assert rel_err(oracle.swa_prefill(q, k, v, 1), v) < 1e-15


def test_equal_keys_give_window_mean():
    # identical keys -> uniform weights -> the mean of the window's values
    r = rng(2)
    N, w = 12, 5
    q = r.standard_normal((N, 4))
    k = np.tile(r.standard_normal((1, 4)), (N, 1))
    v = r.standard_normal((N, 3))
    y = oracle.swa_prefill(q, k, v, w)
    want = np.stack([v[max(0, i - w + 1):i + 1].mean(axis=0) for i in range(N)])
    assert rel_err(y, want) < 1e-14


def test_hand_example():
    # d = 1, w = 2: y_1 = (e^{q1 k0} v0 + e^{q1 k1} v1) / (e^{q1 k0} + e^{q1 k1})
    q = np.array([[0.0], [1.0]])
    k = np.array([[0.0], [np.log(3.0)]])
    v = np.array([[1.0], [5.0]])
    y = oracle.swa_prefill(q, k, v, 2)
    # weights 1 : 3 -> (1 + 15) / 4 = 4
    assert abs(y[0, 0] - 1.0) < 1e-15 and abs(y[1, 0] - 4.0) < 1e-14


def test_decode_steps_continue_the_prefill():
    r = rng(3)
    N, n, w = 40, 7, 16
    q, k = r.standard_normal((2, N + n, 8)), r.standard_normal((2, N + n, 8))
    v = r.standard_normal((2, N + n, 6))
    y_all = oracle.swa_prefill(q, k, v, w)
    kc, vc = oracle.swa_cache_from_prefill(k[:, :N], v[:, :N], w)
    for p in range(N, N + n):
        y, kc, vc = oracle.swa_decode_step(q[:, p], k[:, p], v[:, p], kc, vc, p, w)
        assert rel_err(y, y_all[:, p]) < 1e-13


def test_decode_from_empty_cache_short_prefix():
    # pos < w - 1: only the tokens so far count (the zero slots are not attended)
    r = rng(4)
    w = 8
    q, k, v = r.standard_normal((5, 4)), r.standard_normal((5, 4)), r.standard_normal((5, 2))
    kc, vc = np.zeros((w, 4)), np.zeros((w, 2))
    y_all = oracle.swa_prefill(q, k, v, w)
    for p in range(5):
        y, kc, vc = oracle.swa_decode_step(q[p], k[p], v[p], kc, vc, p, w)
        assert rel_err(y, y_all[p]) < 1e-13
