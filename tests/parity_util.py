"""Tolerance checks shared by the GPU parity tests.

Acceptance bounds (max-abs error against the float64 oracle on identical inputs):
  * float32 inputs:            max|x_gpu - x_ref| <= 1e-4 * max|x_ref|
  * bfloat16 inputs, fp32 state: max|x_gpu - x_ref| <= 2e-2 * RMS(x_ref)
applied to the outputs o and, separately, to the final / updated states.
"""
import numpy as np

TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def bound(ref: np.ndarray, dtype: str) -> float:
    ref = np.asarray(ref, dtype=np.float64)
    if dtype == "f32":
        return TOL_F32 * float(np.max(np.abs(ref)))
    return TOL_BF16 * float(np.sqrt(np.mean(ref * ref)))


def check(name: str, got, ref, dtype: str) -> float:
    """Assert the bound; return err / bound (the fraction of the budget used)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    b = bound(ref, dtype) if ref.size else 0.0
    frac = err / b if b > 0 else (0.0 if err == 0 else float("inf"))
    print(f"  {name}: max err {err:.3e}  bound {b:.3e}  ({frac:.3f} of bound)", flush=True)
    assert err <= b, f"{name}: max err {err:.3e} exceeds bound {b:.3e}"
    return frac
