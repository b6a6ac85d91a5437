"""Planted mistakes in the oracle (on the CPU) must be caught by the pins.

Each case copies oracle/based_oracle.c, plants one plausible mistake (a
dropped factor, a wrong index, a transposed operand, read-before-update, an
ignored initial state, a dropped prefix token), builds it with gcc into a
temporary library, and checks that the closed-form / hand-computed pins used
in test_oracle_pins.py reject it.  The unmodified source must pass the same
checks, so the harness itself is validated too.
"""
import ctypes
import os
import subprocess
import tempfile

import numpy as np
import pytest

from oracle import closed_form_jrt, closed_form_prefill
from tests import golden_io

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "based_oracle.c")

MUTANTS = {
    "drop_inv_sqrt2": ("(x[a] * s) * (x[b] * s) * r2;", "(x[a] * s) * (x[b] * s);"),
    "drop_feature_scale": ("phi[1 + a] = x[a] * s;", "phi[1 + a] = x[a];"),
    "cross_term_index": ("(x[a] * s) * (x[b] * s) * r2;", "(x[a] * s) * (x[a] * s) * r2;"),
    "transposed_state_read": ("num += phi[f] * S[(long)f * dv + c];",
                              "num += phi[f] * S[(long)c * D + f];"),
    "initial_z_ignored": ("memcpy(z, J->z0 + bh * D, sizeof(double) * D);",
                          "memset(z, 0, sizeof(double) * D);"),
    "drop_last_prefix_token": ("for (long j = 0; j < M; ++j) {", "for (long j = 0; j + 1 < M; ++j) {"),
    "eps_sign": ("den += eps;", "den -= eps;"),
}

READ_BEFORE_UPDATE = (
    """        oracle_feature_map(d, J->k + (bh * N + i) * d, phi);
        absorb(D, dv, phi, J->v + (bh * N + i) * dv, S, z);
        if (J->y) {
            oracle_feature_map(d, J->q + (bh * N + i) * d, phi);
            readout(D, dv, phi, S, z, J->eps, J->y + (bh * N + i) * dv);
        }""",
    """        if (J->y) {
            oracle_feature_map(d, J->q + (bh * N + i) * d, phi);
            readout(D, dv, phi, S, z, J->eps, J->y + (bh * N + i) * dv);
        }
        oracle_feature_map(d, J->k + (bh * N + i) * d, phi);
        absorb(D, dv, phi, J->v + (bh * N + i) * dv, S, z);""",
)
MUTANTS["read_before_update"] = READ_BEFORE_UPDATE


def _build(src_text, tmpdir, name):
    c = os.path.join(tmpdir, name + ".c")
    so = os.path.join(tmpdir, name + ".so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", "-O1", "-fPIC", "-shared", "-std=c99", "-o", so, c, "-lm",
                           "-lpthread"])
    lib = ctypes.CDLL(so)
    dp = ctypes.POINTER(ctypes.c_double)
    i = ctypes.c_int
    lib.oracle_prefill.argtypes = [i, i, i, i, i, dp, dp, dp, dp, dp, ctypes.c_double, dp, dp,
                                   dp, i]
    lib.oracle_jrt.argtypes = [i, i, i, i, i, i, dp, dp, dp, dp, dp, dp, dp, ctypes.c_double, dp,
                               dp, dp, i]
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _prefill(lib, q, k, v, S0=None, z0=None, eps=0.0):
    B, H, N, d = q.shape
    dv = v.shape[-1]
    D = 1 + d + d * d
    y = np.zeros((B, H, N, dv))
    S = np.zeros((B, H, D, dv))
    z = np.zeros((B, H, D))
    lib.oracle_prefill(B, H, N, d, dv, _p(q), _p(k), _p(v), _p(S0), _p(z0), eps, _p(y), _p(S),
                       _p(z), 1)
    return y, S, z


def _jrt(lib, q, k, v, ke, ve):
    B, H, N, d = q.shape
    M = ke.shape[2]
    dv = v.shape[-1]
    D = 1 + d + d * d
    y = np.zeros((B, H, N, dv))
    S = np.zeros((B, H, D, dv))
    z = np.zeros((B, H, D))
    lib.oracle_jrt(B, H, N, M, d, dv, _p(q), _p(k), _p(v), _p(ke), _p(ve), None, None, 0.0,
                   _p(y), _p(S), _p(z), 1)
    return y


def _close(a, b, rtol=1e-11):
    return np.max(np.abs(a - b)) <= rtol * np.max(np.abs(b))


def _pins_pass(lib) -> bool:
    """The subset of pins that every planted mistake should trip at least once."""
    r = np.random.default_rng(3)
    q, k = r.normal(size=(1, 2, 40, 16)), r.normal(size=(1, 2, 40, 16))
    v = r.normal(size=(1, 2, 40, 8))
    ok = True
    y, _, _ = _prefill(lib, q, k, v)
    ok &= _close(y, closed_form_prefill(q, k, v))
    y, _, _ = _prefill(lib, q, k, v, eps=0.5)
    ok &= _close(y, closed_form_prefill(q, k, v, eps=0.5))
    _, S0, z0 = _prefill(lib, q[:, :, :10] * 0.5, k[:, :, :10], v[:, :, :10])
    S0 = S0 + 0.3 * r.normal(size=S0.shape)
    y, _, _ = _prefill(lib, q, k, v, np.ascontiguousarray(S0), np.ascontiguousarray(z0))
    ok &= _close(y, closed_form_prefill(q, k, v, S0, z0))
    ke, ve = r.normal(size=(1, 2, 9, 16)), r.normal(size=(1, 2, 9, 8))
    ok &= _close(_jrt(lib, q, k, v, ke, ve), closed_form_jrt(q, k, v, ke, ve))
    g = golden_io.load("hand_state_d1.txt")
    sh = lambda key: np.ascontiguousarray(np.array(g[key][0]).reshape(1, 1, -1, 1))  # noqa
    y, _, _ = _prefill(lib, sh("q"), sh("k"), sh("v"),
                       np.ascontiguousarray(np.array(g["S0"][0]).reshape(1, 1, 3, 1)),
                       np.ascontiguousarray(np.array(g["z0"][0]).reshape(1, 1, 3)))
    ok &= _close(y.reshape(-1), np.array(g["y"][0]), rtol=1e-14)
    return bool(ok)


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


def test_unmodified_oracle_passes_harness(source):
    with tempfile.TemporaryDirectory() as td:
        assert _pins_pass(_build(source, td, "orig"))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(source, name):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    with tempfile.TemporaryDirectory() as td:
        assert not _pins_pass(_build(source.replace(old, new), td, name))
