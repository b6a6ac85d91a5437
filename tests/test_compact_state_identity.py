"""The algebra behind the prefill kernel's compact order-2 state (CPU only).

The kernel keeps each unordered feature pair {a, b} of vec(x x^T) once, as
(a, a + r mod 16) with r the circular distance: r = 1..7 for every a, r = 8 for
a < 8, plus the diagonal.  These tests check, independently of any kernel, that
this enumeration covers every unordered pair exactly once and that it
reproduces (q.k)^2 with weights 1 (diagonal) and 2 (pairs); [BASED] notes §2.3
give K = 1 + t + t^2/2 and observe that the quadratic features repeat.
"""
import itertools

import numpy as np


def circulant_pairs(d=16):
    pairs = [(a, a) for a in range(d)]
    for r in range(1, d // 2):
        pairs += [(a, (a + r) % d) for a in range(d)]
    pairs += [(a, a + d // 2) for a in range(d // 2)]
    return pairs


def test_every_unordered_pair_once():
    pairs = circulant_pairs()
    assert len(pairs) == 16 * 17 // 2 == 136
    seen = [frozenset(p) for p in pairs]
    assert len(set(seen)) == len(seen)
    expected = {frozenset((a, b)) for a, b in itertools.combinations_with_replacement(range(16), 2)}
    assert set(seen) == expected


def test_square_of_dot_product_from_compact_pairs():
    rng = np.random.default_rng(7)
    for _ in range(20):
        q, k = rng.standard_normal(16), rng.standard_normal(16)
        total = 0.0
        for a, b in circulant_pairs():
            w = 1.0 if a == b else 2.0
            total += w * (q[a] * q[b]) * (k[a] * k[b])
        assert abs(total - (q @ k) ** 2) <= 1e-12 * max(1.0, (q @ k) ** 2)


def test_compact_rows_count():
    # ten 16-row tiles: diagonal, distances 1..7, distance 8 (8 rows) + order 0, order 1
    assert 16 + 7 * 16 + 8 + 1 + 16 <= 10 * 16
    assert 1 + 16 + len(circulant_pairs()) == 153
