"""Pins of the oracle's left-padded JRT prefix ("Just read twice" notes, §2.7:
a prompt shorter than M is left-padded to M and the padding is masked out of
the prefix linear attention, so it never enters the state).  Checked against
the attention form on the valid rows, the unpadded call, the no-prefix call,
and invariance to whatever the padding rows hold.
"""
import numpy as np

import oracle
from oracle import closed_form_jrt, closed_form_prefill


def rng(seed):
    return np.random.default_rng(seed)


def rel_err(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def inputs(B=3, H=2, N=13, M=9, d=16, dv=5, seed=0):
    r = rng(seed)
    return (r.standard_normal((B, H, N, d)), r.standard_normal((B, H, N, d)),
            r.standard_normal((B, H, N, dv)), r.standard_normal((B, H, M, d)),
            r.standard_normal((B, H, M, dv)))


def test_full_length_equals_unpadded_jrt():
    q, k, v, ke, ve = inputs(seed=1)
    y, S, z = oracle.jrt_padded(q, k, v, ke, ve, [9, 9, 9])
    y0, S0, z0 = oracle.jrt(q, k, v, ke, ve)
    assert rel_err(y, y0) < 1e-14 and rel_err(S, S0) < 1e-14 and rel_err(z, z0) < 1e-14


def test_zero_length_is_plain_prefill_in_attention_form():
    q, k, v, ke, ve = inputs(seed=2)
    y, _, _ = oracle.jrt_padded(q, k, v, ke, ve, [0, 0, 0])
    assert rel_err(y, closed_form_prefill(q, k, v)) < 1e-11


def test_mixed_lengths_match_attention_form_on_valid_rows():
    q, k, v, ke, ve = inputs(seed=3)
    lens = [0, 4, 9]
    y, _, _ = oracle.jrt_padded(q, k, v, ke, ve, lens)
    for b, m in enumerate(lens):
        M = ke.shape[2]
        ref = closed_form_jrt(q[b:b + 1], k[b:b + 1], v[b:b + 1], ke[b:b + 1, :, M - m:],
                              ve[b:b + 1, :, M - m:])
        assert rel_err(y[b:b + 1], ref) < 1e-11


def test_padding_content_is_irrelevant():
    q, k, v, ke, ve = inputs(seed=4)
    lens = [2, 5, 7]
    y1, S1, z1 = oracle.jrt_padded(q, k, v, ke, ve, lens)
    ke2, ve2 = ke.copy(), ve.copy()
    for b, m in enumerate(lens):
        ke2[b, :, : ke.shape[2] - m] = 1e6
        ve2[b, :, : ke.shape[2] - m] = -3e5
    y2, S2, z2 = oracle.jrt_padded(q, k, v, ke2, ve2, lens)
    assert np.array_equal(y1, y2) and np.array_equal(S1, S2) and np.array_equal(z1, z2)


def test_padding_does_not_enter_the_state_count():
    # the order-0 entry of z is the number of tokens that entered the state
    q, k, v, ke, ve = inputs(seed=5)
    lens = [1, 3, 8]
    _, _, z = oracle.jrt_padded(q, k, v, ke, ve, lens)
    N = q.shape[2]
    assert [z[b, 0, 0] for b in range(3)] == [N + m for m in lens]


def test_compact_padded_is_fold_of_full_padded():
    q, k, v, ke, ve = inputs(seed=6)
    lens = [3, 0, 6]
    y, S, z = oracle.jrt_padded(q, k, v, ke, ve, lens)
    yc, Sc, zc = oracle.jrt_padded(q, k, v, ke, ve, lens, compact=True)
    assert rel_err(yc, y) < 1e-13
    assert rel_err(Sc, oracle.fold(S, 16, axis=-2)) < 1e-13
    assert rel_err(zc, oracle.fold(z, 16, axis=-1)) < 1e-13
