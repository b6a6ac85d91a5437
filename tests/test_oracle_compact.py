"""Pins of the compact (folded) state layout of the oracle (CPU only).

The compact layout keeps each unordered pair of the quadratic features once
("Simple linear attention language models balance the recall-throughput
tradeoff" notes, §2.3: the entries of vec(xb xb^T) repeat).  Every check here
ties the compact functions to something fixed independently: the Taylor kernel
in closed form (1 + t + t^2/2, t = q.k/sqrt(d)), the O(N^2) attention form, a
brute-force enumeration of pairs, or an algebraic identity with arbitrary
(non-symmetric) states.
"""
import itertools

import numpy as np
import pytest

import oracle
from oracle import closed_form_jrt, closed_form_prefill, taylor_kernel


def rng(seed):
    return np.random.default_rng(seed)


def rel_err(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


@pytest.mark.parametrize("d", [1, 2, 3, 16])
def test_compact_dim_and_pairs(d):
    pairs = oracle.pair_list(d)
    assert oracle.compact_dim(d) == 1 + d + d * (d + 1) // 2 == 1 + d + len(pairs)
    # every unordered pair exactly once, row-major upper triangle
    want = list(itertools.combinations_with_replacement(range(d), 2))
    assert pairs == want


def test_compact_index_formula_d16():
    # row 1 + d + P(a, b) with P(a, b) = a*d - a*(a-1)/2 + (b-a) (the documented ABI formula)
    d = 16
    for p, (a, b) in enumerate(oracle.pair_list(d)):
        assert p == a * d - a * (a - 1) // 2 + (b - a)


@pytest.mark.parametrize("d", [2, 16])
def test_compact_kernel_is_taylor_kernel(d):
    # phi_c(q) . (m * phi_c(k)) = 1 + t + t^2/2 (closed form), m = multiplicity (2 off the diagonal)
    r = rng(d)
    q = r.standard_normal((7, d))
    k = r.standard_normal((5, d))
    m = oracle.pair_multiplicity(d)
    got = oracle.compact_feature_map(q) @ (oracle.compact_feature_map(k) * m).T
    assert rel_err(got, taylor_kernel(q, k)) < 1e-13


@pytest.mark.parametrize("d", [3, 16])
def test_fold_preserves_readout_of_any_state(d):
    # phi(q)^T S == phi_c(q)^T fold(S) for an arbitrary, NON-symmetric S
    r = rng(10 + d)
    D = 1 + d + d * d
    S = r.standard_normal((D, 5))
    z = r.standard_normal(D)
    q = r.standard_normal((9, d))
    phi = oracle.feature_map_np(q)
    phic = oracle.compact_feature_map(q)
    assert rel_err(phic @ oracle.fold(S, d, axis=0), phi @ S) < 1e-13
    assert rel_err(phic @ oracle.fold(z, d, axis=0), phi @ z) < 1e-13


def test_fold_unfold_roundtrip_and_symmetry():
    d = 4
    r = rng(3)
    Sc = r.standard_normal((2, oracle.compact_dim(d), 3))
    S = oracle.unfold(Sc, d, axis=-2)
    assert np.array_equal(oracle.fold(S, d, axis=-2), Sc)
    quad = S[:, 1 + d:, :].reshape(2, d, d, 3)
    assert np.array_equal(quad, np.swapaxes(quad, 1, 2))


def test_fold_of_pair_rows_by_hand():
    # d = 2: full quadratic rows (0,0),(0,1),(1,0),(1,1) -> compact (0,0),(0,1),(1,1)
    S = np.arange(1 + 2 + 4, dtype=np.float64)  # rows 0..6
    got = oracle.fold(S, 2, axis=0)
    assert got.tolist() == [0.0, 1.0, 2.0, 3.0, 4.0 + 5.0, 6.0]


def test_prefill_compact_matches_attention_form_with_nonsymmetric_state():
    # y from the compact call equals the attention form with the full (non-symmetric) S0
    d, dv, N = 16, 8, 37
    r = rng(5)
    q = r.standard_normal((1, 2, N, d))
    k = r.standard_normal((1, 2, N, d))
    v = r.standard_normal((1, 2, N, dv))
    D = 1 + d + d * d
    S0 = r.standard_normal((1, 2, D, dv))
    z0 = np.abs(r.standard_normal((1, 2, D))) + 50.0
    y_ref = closed_form_prefill(q, k, v, S0, z0, eps=0.0)
    y, Sc, zc = oracle.prefill_compact(q, k, v, oracle.fold(S0, d, axis=-2), oracle.fold(z0, d, axis=-1))
    assert rel_err(y, y_ref) < 1e-11
    # final compact state = fold(S0) + sum_j (m * phi_c(k_j)) v_j^T
    m = oracle.pair_multiplicity(d)
    fk = oracle.compact_feature_map(k) * m
    S_ref = oracle.fold(S0, d, axis=-2) + np.einsum("bhnf,bhnc->bhfc", fk, v)
    z_ref = oracle.fold(z0, d, axis=-1) + fk.sum(axis=2)
    assert rel_err(Sc, S_ref) < 1e-12
    assert rel_err(zc, z_ref) < 1e-12


def test_jrt_compact_matches_attention_form():
    d, dv, N, M = 16, 4, 19, 11
    r = rng(6)
    q = r.standard_normal((1, 1, N, d))
    k = r.standard_normal((1, 1, N, d))
    v = r.standard_normal((1, 1, N, dv))
    ke = r.standard_normal((1, 1, M, d))
    ve = r.standard_normal((1, 1, M, dv))
    y_ref = closed_form_jrt(q, k, v, ke, ve)
    y, Sc, zc = oracle.jrt_compact(q, k, v, ke, ve)
    assert rel_err(y, y_ref) < 1e-11
    m = oracle.pair_multiplicity(d)
    S_ref = (np.einsum("bhnf,bhnc->bhfc", oracle.compact_feature_map(k) * m, v)
             + np.einsum("bhnf,bhnc->bhfc", oracle.compact_feature_map(ke) * m, ve))
    assert rel_err(Sc, S_ref) < 1e-12


def test_decode_compact_steps_match_attention_form():
    # n compact decode steps from the zero state give the causal attention form at every step
    d, dv, n = 16, 6, 9
    r = rng(7)
    q = r.standard_normal((1, 1, n, d))
    k = r.standard_normal((1, 1, n, d))
    v = r.standard_normal((1, 1, n, dv))
    y_ref = closed_form_prefill(q, k, v)
    Sc = np.zeros((1, 1, oracle.compact_dim(d), dv))
    zc = np.zeros((1, 1, oracle.compact_dim(d)))
    for i in range(n):
        y, Sc, zc = oracle.decode_step_compact(q[:, :, i], k[:, :, i], v[:, :, i], Sc, zc)
        assert rel_err(y, y_ref[:, :, i]) < 1e-12


def test_mutant_fold_without_second_order_fails():
    # a plausible mistake (folding only S[a][b], dropping S[b][a]) breaks the read-out pin
    d = 3
    r = rng(8)
    S = r.standard_normal((1 + d + d * d, 2))
    q = r.standard_normal((4, d))
    bad = oracle.fold(S, d, axis=0).copy()
    for p, (a, b) in enumerate(oracle.pair_list(d)):
        if a != b:
            bad[1 + d + p] = S[1 + d + a * d + b]
    assert rel_err(oracle.compact_feature_map(q) @ bad, oracle.feature_map_np(q) @ S) > 1e-3
