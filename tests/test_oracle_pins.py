"""Pins of the fp64 CPU oracle against facts the pages and the mathematics fix.

Nothing here compares the oracle with itself: every check uses a different
formulation (the O(N^2) attention form, a numpy library routine, a
hand-computed worked example in tests/golden/, or an algebraic identity).

Pages: "Simple linear attention language models balance the recall-throughput
tradeoff" notes (BASED), §2.2-§2.3; "Just read twice" notes (JRT), §2.6,
Eqs. (3)-(4); length-generalization notes (LG), §2.5, Eq. (4).
"""
import numpy as np
import pytest

import oracle
from oracle import closed_form_jrt, closed_form_prefill, feature_map_np, taylor_kernel
from tests import golden_io

RTOL = 1e-11


def rng(seed):
    return np.random.default_rng(seed)


def assert_close(a, b, rtol=RTOL, atol=0.0):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    scale = max(np.max(np.abs(b)), 1e-300)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= rtol * scale + atol, f"max abs err {err:.3e} vs scale {scale:.3e}"


# --- feature map: phi(q).phi(k) = K(q,k)  (BASED §2.3, Eq. (4) with the d'^(1/4) scale) ---

@pytest.mark.parametrize("d", [1, 2, 4, 16])
def test_feature_dim(d):
    assert oracle.feature_dim(d) == 1 + d + d * d
    assert len(oracle.feature_map(np.ones(d))) == 1 + d + d * d


def test_feature_dim_273():
    # BASED §2.3: 1 + 16 + 16^2 = 273 for d' = 16
    assert oracle.feature_dim(16) == 273


@pytest.mark.parametrize("d", [1, 2, 4, 16])
def test_feature_map_reproduces_taylor_kernel(d):
    r = rng(d)
    for _ in range(20):
        q, k = r.normal(size=d) * 1.5, r.normal(size=d) * 1.5
        t = float(q @ k)
        K = 1.0 + t / np.sqrt(d) + t * t / (2.0 * d)
        assert abs(oracle.feature_map(q) @ oracle.feature_map(k) - K) <= 1e-13 * abs(K)
        assert abs(feature_map_np(q) @ feature_map_np(k) - K) <= 1e-13 * abs(K)


def test_feature_map_layout_d2():
    # explicit layout for d = 2: [1, x/2^(1/4), xb0^2, xb0 xb1, xb1 xb0, xb1^2] / sqrt2 on the last 4
    x = np.array([3.0, -5.0])
    xb = x / 2 ** 0.25
    want = [1.0, xb[0], xb[1], xb[0] ** 2 / np.sqrt(2), xb[0] * xb[1] / np.sqrt(2),
            xb[1] * xb[0] / np.sqrt(2), xb[1] ** 2 / np.sqrt(2)]
    assert_close(oracle.feature_map(x), want, rtol=1e-15)


def test_kernel_bounded_below_by_half():
    # K = ((t+1)^2 + 1)/2 >= 1/2, equality at t = -1 (BASED §2.3)
    r = rng(7)
    q, k = r.normal(size=(300, 16)) * 2, r.normal(size=(300, 16)) * 2
    assert taylor_kernel(q, k).min() >= 0.5
    q1 = np.zeros(16)
    q1[0] = 4.0
    k1 = np.zeros(16)
    k1[0] = -1.0  # q.k = -4 -> t = -4/sqrt(16) = -1
    assert abs(taylor_kernel(q1[None], k1[None])[0, 0] - 0.5) < 1e-15


# --- hand-computed worked examples (tests/golden/) ---

def test_golden_hand_d1():
    g = golden_io.load("hand_d1.txt")
    q = np.array(g["q"][0]).reshape(1, 1, -1, 1)
    k = np.array(g["k"][0]).reshape(1, 1, -1, 1)
    v = np.array(g["v"][0]).reshape(1, 1, -1, 1)
    y, S, z = oracle.prefill(q, k, v)
    assert_close(y.reshape(-1), g["y"][0], rtol=1e-15)
    assert_close(S.reshape(-1), g["S"][0], rtol=1e-15)
    assert_close(z.reshape(-1), g["z"][0], rtol=1e-15)


def test_golden_hand_d4():
    g = golden_io.load("hand_d4.txt")
    q = np.array(g["q"]).reshape(1, 1, 2, 4)
    k = np.array(g["k"]).reshape(1, 1, 2, 4)
    v = np.array(g["v"]).reshape(1, 1, 2, 2)
    y, S, z = oracle.prefill(q, k, v)
    assert_close(y.reshape(2, 2), np.array(g["y"]), rtol=1e-15)
    S_want = np.zeros((21, 2))
    z_want = np.zeros(21)
    for key, rows in g.items():
        if key.startswith("row"):
            idx = int(key.split()[1])
            S_want[idx] = rows[0][:2]
            z_want[idx] = rows[0][2]
    assert_close(S.reshape(21, 2), S_want, rtol=1e-15)
    assert_close(z.reshape(21), z_want, rtol=1e-15)


def test_golden_hand_jrt_d1():
    g = golden_io.load("hand_jrt_d1.txt")
    sh = lambda key: np.array(g[key][0]).reshape(1, 1, -1, 1)  # noqa: E731
    y, S, z = oracle.jrt(sh("q"), sh("k"), sh("v"), sh("ke"), sh("ve"))
    assert_close(y.reshape(-1), g["y"][0], rtol=1e-15)
    assert_close(S.reshape(-1), g["S"][0], rtol=1e-15)
    assert_close(z.reshape(-1), g["z"][0], rtol=1e-15)


def test_golden_hand_initial_state_d1():
    g = golden_io.load("hand_state_d1.txt")
    sh = lambda key: np.array(g[key][0]).reshape(1, 1, -1, 1)  # noqa: E731
    S0 = np.array(g["S0"][0]).reshape(1, 1, 3, 1)
    z0 = np.array(g["z0"][0]).reshape(1, 1, 3)
    y, S, z = oracle.prefill(sh("q"), sh("k"), sh("v"), S0, z0)
    assert_close(y.reshape(-1), g["y"][0], rtol=1e-15)
    assert_close(S.reshape(-1), g["S"][0], rtol=1e-15)
    assert_close(z.reshape(-1), g["z"][0], rtol=1e-15)
    # the decode step is the same single update-then-read
    yd, Sd, zd = oracle.decode_step(sh("q")[:, :, 0], sh("k")[:, :, 0], sh("v")[:, :, 0], S0, z0)
    assert_close(yd.reshape(-1), g["y"][0], rtol=1e-15)
    assert_close(Sd.reshape(-1), g["S"][0], rtol=1e-15)


# --- recurrence == attention form (BASED §2.2) ---

def _inputs(seed, B=2, H=2, N=150, d=16, dv=8, scale=1.0):
    r = rng(seed)
    q = r.normal(size=(B, H, N, d)) * scale
    k = r.normal(size=(B, H, N, d)) * scale
    v = r.normal(size=(B, H, N, dv))
    return q, k, v


@pytest.mark.parametrize("d,dv,N", [(16, 8, 150), (4, 3, 97), (1, 2, 60)])
def test_recurrence_equals_attention_form(d, dv, N):
    q, k, v = _inputs(11 + d, N=N, d=d, dv=dv)
    y, S, z = oracle.prefill(q, k, v)
    assert_close(y, closed_form_prefill(q, k, v))
    # the final state equals the feature-space sums phi(K)^T V, 1^T phi(K) (numpy)
    phk = feature_map_np(k)
    assert_close(S, np.einsum("bhnf,bhnc->bhfc", phk, v))
    assert_close(z, phk.sum(2))


def test_recurrence_with_eps():
    q, k, v = _inputs(5, N=40)
    y, _, _ = oracle.prefill(q, k, v, eps=0.37)
    assert_close(y, closed_form_prefill(q, k, v, eps=0.37))


def test_recurrence_with_initial_state_equals_attention_form():
    q, k, v = _inputs(21, N=120)
    q0, k0, v0 = _inputs(22, N=64)
    _, S0, z0 = oracle.prefill(q0, k0, v0)
    r = rng(23)
    S0 = S0 + 0.5 * r.normal(size=S0.shape)  # generic, non-symmetric in the vec block
    y, S, z = oracle.prefill(q, k, v, S0, z0)
    assert_close(y, closed_form_prefill(q, k, v, S0, z0))
    phk = feature_map_np(k)
    assert_close(S, S0 + np.einsum("bhnf,bhnc->bhfc", phk, v))
    assert_close(z, z0 + phk.sum(2))


# --- special cases ---

def test_zero_query_gives_running_mean():
    # q = 0 -> K = 1 for every key -> y_i = mean of v_1..v_i (numpy cumsum)
    q, k, v = _inputs(31, N=90)
    y, _, _ = oracle.prefill(np.zeros_like(q), k, v)
    want = np.cumsum(v, axis=2) / np.arange(1, 91)[None, None, :, None]
    assert_close(y, want, rtol=1e-13)


def test_first_output_is_first_value():
    q, k, v = _inputs(32, N=5)
    y, _, _ = oracle.prefill(q, k, v)
    assert_close(y[:, :, 0], v[:, :, 0], rtol=1e-14)


def test_constant_values_give_constant_output():
    q, k, v = _inputs(33, N=70)
    c = rng(34).normal(size=(2, 2, 1, 8))
    y, _, _ = oracle.prefill(q, k, np.broadcast_to(c, v.shape))
    assert_close(y, np.broadcast_to(c, y.shape), rtol=1e-13)


def test_linear_in_values():
    q, k, v1 = _inputs(35, N=80)
    v2 = rng(36).normal(size=v1.shape)
    y1, _, _ = oracle.prefill(q, k, v1)
    y2, _, _ = oracle.prefill(q, k, v2)
    y3, _, _ = oracle.prefill(q, k, 2.0 * v1 - 3.0 * v2)
    assert_close(y3, 2.0 * y1 - 3.0 * y2, rtol=1e-12)


def test_output_in_running_convex_hull():
    # K > 0, so y_i is a convex combination of v_1..v_i
    q, k, v = _inputs(37, N=100, scale=2.0)
    y, _, _ = oracle.prefill(q, k, v)
    lo = np.minimum.accumulate(v, axis=2)
    hi = np.maximum.accumulate(v, axis=2)
    assert np.all(y >= lo - 1e-12) and np.all(y <= hi + 1e-12)


# --- state passing (LG §2.5, Eq. (4)) ---

def test_split_and_resume_equals_uninterrupted():
    q, k, v = _inputs(41, N=160)
    y, S, z = oracle.prefill(q, k, v)
    ya, Sa, za = oracle.prefill(q[:, :, :61], k[:, :, :61], v[:, :, :61])
    yb, Sb, zb = oracle.prefill(q[:, :, 61:], k[:, :, 61:], v[:, :, 61:], Sa, za)
    assert_close(np.concatenate([ya, yb], axis=2), y)
    assert_close(Sb, S)
    assert_close(zb, z)


def test_decode_steps_equal_prefill():
    q, k, v = _inputs(42, N=40)
    _, S, z = oracle.prefill(q[:, :, :30], k[:, :, :30], v[:, :, :30])
    ys = []
    for i in range(30, 40):
        yi, S, z = oracle.decode_step(q[:, :, i], k[:, :, i], v[:, :, i], S, z)
        ys.append(yi)
    assert_close(np.stack(ys, axis=2), closed_form_prefill(q, k, v)[:, :, 30:])
    _, S_all, z_all = oracle.prefill(q, k, v)
    assert_close(S, S_all)
    assert_close(z, z_all)


# --- JRT prefix (JRT §2.6, Eqs. (3)-(4)) ---

def _prefix(seed, B=2, H=2, M=50, d=16, dv=8):
    r = rng(seed)
    return r.normal(size=(B, H, M, d)), r.normal(size=(B, H, M, dv))


def test_jrt_equals_attention_form():
    q, k, v = _inputs(51, N=90)
    ke, ve = _prefix(52)
    y, S, z = oracle.jrt(q, k, v, ke, ve)
    assert_close(y, closed_form_jrt(q, k, v, ke, ve))
    phe, phk = feature_map_np(ke), feature_map_np(k)
    assert_close(S, np.einsum("bhmf,bhmc->bhfc", phe, ve) + np.einsum("bhnf,bhnc->bhfc", phk, v))
    assert_close(z, phe.sum(2) + phk.sum(2))


def test_jrt_equals_based_with_prefix_state_as_initial_state():
    q, k, v = _inputs(53, N=70)
    ke, ve = _prefix(54, M=33)
    phe = feature_map_np(ke)
    S_pre = np.einsum("bhmf,bhmc->bhfc", phe, ve)
    z_pre = phe.sum(2)
    y, S, z = oracle.jrt(q, k, v, ke, ve)
    yb, Sb, zb = oracle.prefill(q, k, v, S_pre, z_pre)
    assert_close(y, yb)
    assert_close(S, Sb)
    assert_close(z, zb)


def test_jrt_with_initial_state_is_additive():
    q, k, v = _inputs(55, N=64)
    ke, ve = _prefix(56, M=20)
    _, S0, z0 = oracle.prefill(*_inputs(57, N=30))
    y, S, z = oracle.jrt(q, k, v, ke, ve, S0, z0)
    assert_close(y, closed_form_jrt(q, k, v, ke, ve, S0, z0))
    _, S_pre, z_pre = oracle.prefill(np.zeros((2, 2, 20, 16)), ke, ve)
    _, S_n, z_n = oracle.prefill(q, k, v)
    assert_close(S, S0 + S_pre + S_n)  # Eq. (4): merged state
    assert_close(z, z0 + z_pre + z_n)


def test_jrt_without_prefix_equals_based():
    q, k, v = _inputs(58, N=50)
    ke, ve = np.zeros((2, 2, 0, 16)), np.zeros((2, 2, 0, 8))
    y, S, z = oracle.jrt(q, k, v, ke, ve)
    yb, Sb, zb = oracle.prefill(q, k, v)
    assert_close(y, yb, rtol=0)
    assert_close(S, Sb, rtol=0)


def test_jrt_prefix_order_does_not_matter():
    q, k, v = _inputs(59, N=40)
    ke, ve = _prefix(60, M=45)
    perm = rng(61).permutation(45)
    y1, S1, _ = oracle.jrt(q, k, v, ke, ve)
    y2, S2, _ = oracle.jrt(q, k, v, ke[:, :, perm], ve[:, :, perm])
    assert_close(y2, y1, rtol=1e-12)
    assert_close(S2, S1, rtol=1e-12)


def test_threads_do_not_change_results():
    q, k, v = _inputs(62, B=3, H=3, N=30)
    y1, S1, _ = oracle.prefill(q, k, v, nthreads=1)
    y4, S4, _ = oracle.prefill(q, k, v, nthreads=4)
    assert np.array_equal(y1, y4) and np.array_equal(S1, S4)


def test_decode_threads_do_not_change_results():
    r = np.random.default_rng(11)
    q, k, v = r.normal(size=(3, 5, 16)), r.normal(size=(3, 5, 16)), r.normal(size=(3, 5, 8))
    _, S0, z0 = oracle.prefill(r.normal(size=(3, 5, 20, 16)), r.normal(size=(3, 5, 20, 16)),
                               r.normal(size=(3, 5, 20, 8)))
    y1, S1, z1 = oracle.decode_step(q, k, v, S0, z0, nthreads=1)
    y4, S4, z4 = oracle.decode_step(q, k, v, S0, z0, nthreads=4)
    assert np.array_equal(y1, y4) and np.array_equal(S1, S4) and np.array_equal(z1, z4)
    # in place: the same result, written into the given fp64 arrays
    S2, z2 = S0.copy(), z0.copy()
    y2, S2r, z2r = oracle.decode_step(q, k, v, S2, z2, nthreads=3, in_place=True)
    assert S2r is S2 and z2r is z2
    assert np.array_equal(y2, y1) and np.array_equal(S2, S1) and np.array_equal(z2, z1)
