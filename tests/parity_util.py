"""Tolerance metric shared by the GPU parity tests.

Per output row (b, h, i): max_c |y - y_ref| <= tol * max_c |y_ref|.
Per (b, h) state: max |S - S_ref| <= tol * max |S_ref| (same for z).
The bf16-input tolerance 2e-3 and the fp32-input tolerance 1e-5 are the
relative tolerances of the workloads these kernels are built for.
"""
import numpy as np

TOL_BF16 = 2e-3
TOL_F32 = 1e-5


def _np(x):
    if hasattr(x, "detach"):
        x = x.detach().float().cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def worst_row_error(y, y_ref):
    """Largest row-relative error over all rows (rows = all leading dims)."""
    y, y_ref = _np(y), _np(y_ref)
    assert y.shape == y_ref.shape, (y.shape, y_ref.shape)
    if y.size == 0:
        return 0.0
    d = np.abs(y - y_ref).max(-1)
    s = np.abs(y_ref).max(-1)
    return float((d / np.maximum(s, 1e-30)).max())


def worst_state_error(S, S_ref):
    """Largest per-(b,h) relative error of a state [B,H,...]."""
    S, S_ref = _np(S), _np(S_ref)
    assert S.shape == S_ref.shape, (S.shape, S_ref.shape)
    B, H = S.shape[:2]
    d = np.abs(S - S_ref).reshape(B, H, -1).max(-1)
    s = np.abs(S_ref).reshape(B, H, -1).max(-1)
    return float((d / np.maximum(s, 1e-30)).max())


def assert_rows(y, y_ref, tol, what="y"):
    e = worst_row_error(y, y_ref)
    assert np.all(np.isfinite(_np(y))), f"{what}: non-finite values"
    assert e <= tol, f"{what}: worst row error {e:.3e} > tol {tol:.1e}"
    return e


def assert_state(S, S_ref, tol, what="S"):
    e = worst_state_error(S, S_ref)
    assert np.all(np.isfinite(_np(S))), f"{what}: non-finite values"
    assert e <= tol, f"{what}: worst state error {e:.3e} > tol {tol:.1e}"
    return e
