"""The chunked form of the prefill equals the token-by-token recurrence for any chunk size.

"Simple linear attention language models balance the recall-throughput tradeoff"
notes, §2.5: the sequence is cut into chunks of C tokens; chunk b's outputs are
the masked intra-chunk term (M o Phi_Qb Phi_Kb^T) V_b plus the inter-chunk term
Phi_Qb S_<b, where S_<b sums phi(k) v^T over the earlier chunks (the denominator
splits the same way), and the state then absorbs the chunk.  The GPU kernels use
this form with C = 128; the oracle is the recurrence.  Here a plain fp64 NumPy
version of the chunked form, with the feature map materialised, is checked
against the oracle for chunk sizes from 1 to N, ones that do not divide N
included, with and without an initial state and eps: the result does not depend
on the chunk size.
"""
import numpy as np
import pytest

import oracle
from recurrent_lm_sequence_amd import inputs as gen


def _phi(x):
    """[1, x/d^(1/4), vec(x x^T)/(sqrt2 sqrt d)] for rows x [..., d]."""
    d = x.shape[-1]
    xb = x / d ** 0.25
    quad = (xb[..., :, None] * xb[..., None, :]).reshape(*x.shape[:-1], d * d) / np.sqrt(2.0)
    return np.concatenate([np.ones(x.shape[:-1] + (1,)), xb, quad], axis=-1)


def chunked_prefill(q, k, v, C, S0=None, z0=None, eps=0.0):
    """Chunked linear attention over one (b, h): q, k [N, d], v [N, dv]."""
    N, dv = v.shape
    D = _phi(q[:1]).shape[-1]
    S = np.zeros((D, dv)) if S0 is None else S0.copy()
    z = np.zeros(D) if z0 is None else z0.copy()
    y = np.empty((N, dv))
    for c0 in range(0, N, C):
        pq, pk, vb = _phi(q[c0:c0 + C]), _phi(k[c0:c0 + C]), v[c0:c0 + C]
        A = np.tril(pq @ pk.T)                      # intra-chunk, causal mask j <= i
        num = A @ vb + pq @ S                       # intra + inter (state of earlier chunks)
        den = A.sum(-1) + pq @ z
        y[c0:c0 + C] = num / (den + eps)[:, None]
        S += pk.T @ vb                              # the state absorbs the chunk
        z += pk.sum(0)
    return y, S, z


@pytest.mark.parametrize("C", [1, 7, 16, 64, 100, 128, 300])
@pytest.mark.parametrize("init", [False, True])
def test_chunked_form_equals_recurrence(C, init):
    w = gen.Workload("chunk", B=1, H=2, N=300, d_feat=4, d_v=3, dtype="f32", seed=77)
    q, k, v = gen.make_prefill_inputs(w, "cpu")
    qn, kn, vn = (t.double().numpy() for t in (q, k, v))
    D = oracle.feature_dim(4)
    S0 = z0 = None
    if init:
        rng = np.random.default_rng(78)
        S0 = rng.standard_normal((1, 2, D, 3))
        z0 = np.abs(rng.standard_normal((1, 2, D))) + 1.0
    eps = 1e-3 if init else 0.0
    yr, Sr, zr = oracle.prefill(qn, kn, vn, S0, z0, eps=eps)
    for h in range(2):
        y, S, z = chunked_prefill(qn[0, h], kn[0, h], vn[0, h], C,
                                  None if S0 is None else S0[0, h], None if z0 is None else z0[0, h], eps)
        np.testing.assert_allclose(y, yr[0, h], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(S, Sr[0, h], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(z, zr[0, h], rtol=1e-12, atol=1e-12)


def test_a_wrong_mask_is_caught():
    # the chunked form with the diagonal masked out (j < i) must not match
    w = gen.Workload("chunk", B=1, H=1, N=50, d_feat=4, d_v=3, dtype="f32", seed=79)
    q, k, v = gen.make_prefill_inputs(w, "cpu")
    qn, kn, vn = (t.double().numpy()[0, 0] for t in (q, k, v))
    yr, _, _ = oracle.prefill(qn[None, None], kn[None, None], vn[None, None])
    pq, pk = _phi(qn), _phi(kn)
    A = np.tril(pq @ pk.T, -1)
    y_bad = (A @ vn)[1:] / A.sum(-1)[1:, None]
    assert np.abs(y_bad - yr[0, 0, 1:]).max() > 1e-3
