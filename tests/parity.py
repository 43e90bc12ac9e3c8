"""Comparison helpers for the GPU-vs-oracle parity tests.

Tolerances (per output element, against the fp64 oracle):
  fp32 inputs: max |gpu - oracle| <= 1e-5.
  bf16 inputs: max |gpu - oracle| <= 2e-2 and, per output row,
               ||gpu - oracle||_2 / ||oracle||_2 <= 1e-2.
A row whose oracle value is exactly zero (no allowed key) must be exactly zero.
"""
from __future__ import annotations

import numpy as np

TOL = {"f32": dict(abs=1e-5, rel=None), "bf16": dict(abs=2e-2, rel=1e-2)}


def errors(got: np.ndarray, want: np.ndarray):
    """(max abs error, max per-row relative-to-norm error) over the last axis."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    if got.size == 0:
        return 0.0, 0.0
    diff = got - want
    max_abs = float(np.abs(diff).max())
    dn = np.linalg.norm(diff, axis=-1)
    rn = np.linalg.norm(want, axis=-1)
    zero = rn == 0.0
    rel = np.where(zero, np.where(dn == 0.0, 0.0, np.inf), dn / np.where(zero, 1.0, rn))
    return max_abs, float(rel.max())


def assert_parity(got, want, dtype: str, what: str = ""):
    tol = TOL[dtype]
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    max_abs, max_rel = errors(got, want)
    msg = f"{what}: max abs {max_abs:.3e} (tol {tol['abs']}), max row rel {max_rel:.3e}"
    assert max_abs <= tol["abs"], msg
    if tol["rel"] is not None:
        assert max_rel <= tol["rel"], msg
    # rows the oracle leaves exactly zero (nothing allowed) must be zero
    zero_rows = np.all(np.asarray(want) == 0.0, axis=-1)
    if zero_rows.any():
        assert np.all(got[zero_rows] == 0.0), f"{what}: fully masked rows not zero"
    return max_abs, max_rel
