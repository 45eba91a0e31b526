"""Error metrics and the acceptance bar for GPU-vs-oracle parity.

The bar for fp16/bf16 attention outputs: max-abs error <= 1e-2 AND relative
Frobenius error <= 2e-3, both against the fp64 oracle.
"""
import numpy as np

MAX_ABS_TOL = 1e-2
REL_FRO_TOL = 2e-3


def errors(test, ref):
    """(max_abs, rel_fro) of ``test`` against ``ref`` (any array-likes)."""
    t = np.asarray(test, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert t.shape == r.shape, (t.shape, r.shape)
    if t.size == 0:
        return 0.0, 0.0
    diff = t - r
    max_abs = float(np.max(np.abs(diff)))
    nr = float(np.linalg.norm(r.ravel()))
    rel = float(np.linalg.norm(diff.ravel()) / nr) if nr > 0 else float(np.linalg.norm(diff.ravel()))
    return max_abs, rel


def assert_parity(test, ref, what="", max_abs_tol=MAX_ABS_TOL, rel_fro_tol=REL_FRO_TOL):
    t = np.asarray(test, dtype=np.float64)
    assert np.all(np.isfinite(t)), f"{what}: non-finite values in the output"
    ma, rf = errors(t, ref)
    print(f"[parity] {what}: max_abs={ma:.3e} rel_fro={rf:.3e}", flush=True)
    assert ma <= max_abs_tol and rf <= rel_fro_tol, \
        f"{what}: max_abs={ma:.3e} (tol {max_abs_tol}) rel_fro={rf:.3e} (tol {rel_fro_tol})"
    return ma, rf
