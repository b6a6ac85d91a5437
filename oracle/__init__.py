"""fp64 CPU oracle for causal Taylor linear attention (BASED), the JRT-RNN
prefix variant and the single-token decode step.

TEST INFRASTRUCTURE ONLY: the test-suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only users.  The HIP library never
imports, links or calls anything here, and nothing here touches the HIP
library: both sides only share the seeded input generator.

Two independent formulations live here:

* ``prefill`` / ``jrt`` / ``decode_step`` -- the token-by-token fp64
  recurrence (``based_oracle.c``), following the "Simple linear attention
  language models balance the recall-throughput tradeoff" notes, §2.2
  (s_i = s_{i-1} + phi(k_i) v_i^T, z_i = z_{i-1} + phi(k_i),
  y_i = s_i^T phi(q_i) / z_i^T phi(q_i)) and §2.3 (the feature map), the
  "Just read twice" notes §2.6 (Eqs. (3)-(4), prefix state) and the
  length-generalization notes §2.5 (Eq. (4), non-zero initial state).
* ``closed_form`` -- the O(N^2) attention form of the same method
  (sum_j K(q_i,k_j) v_j / sum_j K(q_i,k_j), Taylor kernel of Eq. (4)),
  written with numpy, used to pin the recurrence.

Sliding-window softmax attention (the second mixer of BASED) is in
``swa.py``.  The compact state layout (each unordered feature pair once) is in
``compact.py``; ``prefill_compact`` / ``jrt_compact`` / ``decode_step_compact``
wrap the recurrence with its fold/unfold maps.

Pins for every function are in ``tests/test_oracle_pins.py`` and
``tests/test_oracle_compact.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .closed_form import (  # noqa: F401  (re-exported)
    closed_form_prefill,
    closed_form_jrt,
    feature_map_np,
    taylor_kernel,
)
from .swa import swa_cache_from_prefill, swa_decode_step, swa_prefill, swa_prefill_blocked  # noqa: F401
from .compact import (  # noqa: F401  (re-exported)
    compact_dim,
    compact_feature_map,
    fold,
    pair_list,
    pair_multiplicity,
    unfold,
)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "based_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build_oracle_library(force: bool = False) -> str:
    """Compile based_oracle.c into liboracle.so with gcc (plain -O2)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fPIC", "-shared", "-std=c99", "-o", tmp, _SRC, "-lm", "-lpthread"]
        )
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        # BLA_ORACLE_LIBRARY: a separately built copy of based_oracle.c (the sanitizer test
        # loads an AddressSanitizer/UBSan build through it)
        path = os.environ.get("BLA_ORACLE_LIBRARY") or build_oracle_library()
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        i = ctypes.c_int
        lib.oracle_feature_dim.argtypes = [i]
        lib.oracle_feature_dim.restype = i
        lib.oracle_feature_map.argtypes = [i, dp, dp]
        lib.oracle_feature_map.restype = None
        lib.oracle_prefill.argtypes = [i, i, i, i, i, dp, dp, dp, dp, dp, ctypes.c_double,
                                       dp, dp, dp, i]
        lib.oracle_prefill.restype = None
        lib.oracle_jrt.argtypes = [i, i, i, i, i, i, dp, dp, dp, dp, dp, dp, dp,
                                   ctypes.c_double, dp, dp, dp, i]
        lib.oracle_jrt.restype = None
        lib.oracle_decode_step.argtypes = [i, i, i, i, dp, dp, dp, dp, dp, ctypes.c_double, dp, i]
        lib.oracle_decode_step.restype = None
        _lib = lib
    return _lib


def _f64(x):
    """Exact fp64 copy of a numpy array or a torch tensor (bf16/fp32 values are exact in fp64)."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def host_cores() -> int:
    """Cores this process may run on (its CPU affinity, as `nproc` reports it)."""
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def default_threads() -> int:
    """Worker threads: one per core this process may run on, capped by
    OMP_NUM_THREADS when that is set (the CPU share a shared host gives one GPU)."""
    n = host_cores()
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def feature_dim(d: int) -> int:
    return int(_load().oracle_feature_dim(d))


def feature_map(x) -> np.ndarray:
    """phi(x) for one vector x of length d (C implementation)."""
    x = _f64(x).reshape(-1)
    d = x.shape[0]
    out = np.empty(feature_dim(d), dtype=np.float64)
    _load().oracle_feature_map(d, _ptr(x), _ptr(out))
    return out


def prefill(q, k, v, S0=None, z0=None, eps: float = 0.0, nthreads: int | None = None,
            want_y: bool = True):
    """Causal prefill.  q,k [B,H,N,d], v [B,H,N,dv]; S0 [B,H,D,dv], z0 [B,H,D] or None.
    Returns (y [B,H,N,dv], S_N [B,H,D,dv], z_N [B,H,D]) in fp64 (y is None when
    want_y is False: then only the state recurrence runs)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    dv = v.shape[-1]
    D = feature_dim(d)
    S0, z0 = _f64(S0), _f64(z0)
    y = np.zeros((B, H, N, dv)) if want_y else None
    S = np.zeros((B, H, D, dv))
    z = np.zeros((B, H, D))
    _load().oracle_prefill(B, H, N, d, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(S0), _ptr(z0),
                           float(eps), _ptr(y), _ptr(S), _ptr(z), nthreads or default_threads())
    return y, S, z


def jrt(q, k, v, ke, ve, S0=None, z0=None, eps: float = 0.0, nthreads: int | None = None):
    """JRT-RNN prefix linear attention.  ke [B,H,M,d], ve [B,H,M,dv].
    Returns (y [B,H,N,dv], S [B,H,D,dv], z [B,H,D]) with S = S0 + s_E + s_{D,N}."""
    q, k, v, ke, ve = _f64(q), _f64(k), _f64(v), _f64(ke), _f64(ve)
    B, H, N, d = q.shape
    M = ke.shape[2]
    dv = v.shape[-1]
    D = feature_dim(d)
    S0, z0 = _f64(S0), _f64(z0)
    y = np.zeros((B, H, N, dv))
    S = np.zeros((B, H, D, dv))
    z = np.zeros((B, H, D))
    _load().oracle_jrt(B, H, N, M, d, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(ke), _ptr(ve),
                       _ptr(S0), _ptr(z0), float(eps), _ptr(y), _ptr(S), _ptr(z),
                       nthreads or default_threads())
    return y, S, z


def decode_step(q, k, v, S, z, eps: float = 0.0, nthreads: int | None = None,
                in_place: bool = False):
    """One recurrent step.  q,k [B,H,d], v [B,H,dv]; S [B,H,D,dv], z [B,H,D].
    Returns (y [B,H,dv], S_new, z_new).  The inputs are not modified unless
    in_place=True and S, z are already contiguous fp64 numpy arrays (then they
    are updated and returned)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    if not (in_place and isinstance(S, np.ndarray) and S.dtype == np.float64
            and S.flags.c_contiguous and isinstance(z, np.ndarray) and z.dtype == np.float64
            and z.flags.c_contiguous):
        S = _f64(S).copy()
        z = _f64(z).copy()
    B, H, d = q.shape
    dv = v.shape[-1]
    y = np.zeros((B, H, dv))
    _load().oracle_decode_step(B, H, d, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(S), _ptr(z),
                               float(eps), _ptr(y), nthreads or default_threads())
    return y, S, z


# ---------------- compact state layout (see oracle/compact.py) ----------------

def _unfold_state(S0c, z0c, d):
    if S0c is None:
        return None, None
    return unfold(_f64(S0c), d, axis=-2), unfold(_f64(z0c), d, axis=-1)


def prefill_compact(q, k, v, S0c=None, z0c=None, eps: float = 0.0, nthreads: int | None = None):
    """prefill with the state in the compact layout: (y, fold(S_N), fold(z_N))."""
    d = q.shape[-1]
    S0, z0 = _unfold_state(S0c, z0c, d)
    y, S, z = prefill(q, k, v, S0, z0, eps=eps, nthreads=nthreads)
    return y, fold(S, d, axis=-2), fold(z, d, axis=-1)


def jrt_compact(q, k, v, ke, ve, S0c=None, z0c=None, eps: float = 0.0, nthreads: int | None = None):
    """jrt with the state in the compact layout: (y, fold(S), fold(z)) of the merged state."""
    d = q.shape[-1]
    S0, z0 = _unfold_state(S0c, z0c, d)
    y, S, z = jrt(q, k, v, ke, ve, S0, z0, eps=eps, nthreads=nthreads)
    return y, fold(S, d, axis=-2), fold(z, d, axis=-1)


def decode_step_compact(q, k, v, Sc, zc, eps: float = 0.0):
    """decode_step on a compact state: (y, fold(S_new), fold(z_new))."""
    d = q.shape[-1]
    S, z = _unfold_state(Sc, zc, d)
    y, S1, z1 = decode_step(q, k, v, S, z, eps=eps)
    return y, fold(S1, d, axis=-2), fold(z1, d, axis=-1)


def jrt_padded(q, k, v, ke, ve, prefix_len, S0=None, z0=None, eps: float = 0.0,
               compact: bool = False, nthreads: int | None = None):
    """JRT with left-padded prefixes ("Just read twice" notes, §2.7: a prompt
    shorter than M is left-padded to M and the padding is masked out of the
    prefix linear attention).  prefix_len[b] valid prefix tokens: the last
    prefix_len[b] rows of ke/ve[b]; the rows before are excluded.  Runs the
    recurrence per batch element on its valid prefix rows only."""
    q, k, v, ke, ve = _f64(q), _f64(k), _f64(v), _f64(ke), _f64(ve)
    B, M = q.shape[0], ke.shape[2]
    run = jrt_compact if compact else jrt
    outs = []
    for b in range(B):
        m = int(min(max(int(prefix_len[b]), 0), M))
        sl = slice(b, b + 1)
        s0 = None if S0 is None else _f64(S0)[sl]
        zz = None if z0 is None else _f64(z0)[sl]
        outs.append(run(q[sl], k[sl], v[sl], ke[sl, :, M - m:], ve[sl, :, M - m:], s0, zz,
                        eps=eps, nthreads=nthreads))
    return tuple(np.concatenate([o[i] for o in outs], axis=0) for i in range(3))
