"""Comparison of GPU results with the float64 oracle.

Tolerance for fp16 K/V and fp16 output (the decode-attention accuracy bar):
  * max |out - ref| <= 1e-2 over all elements, and
  * row-normwise relative error max_{b,h} ||out - ref||_inf / ||ref||_inf
    <= 2e-3 (an element-wise relative error is meaningless for outputs that
    are averages of N(0, 1) values and sit near zero; fp16 rounding of the
    output alone contributes up to 2^-11 ~ 4.9e-4 of a row's scale).
Rows whose reference is exactly zero (empty contexts) must be exactly zero.
The log-sum-exp is compared absolutely: |lse - ref| <= 1e-4 (fp32 scores of
magnitude ~10 carry ~1e-6 of rounding).
"""
from __future__ import annotations

import numpy as np

ABS_TOL = 1e-2
ROW_REL_TOL = 2e-3
LSE_TOL = 1e-4


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def compare_out(out, ref, abs_tol=ABS_TOL, row_rel_tol=ROW_REL_TOL, what="out"):
    """out, ref: float arrays [..., D]; raises AssertionError with the worst figures."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert out.shape == ref.shape, (out.shape, ref.shape)
    assert np.all(np.isfinite(out)), f"{what}: non-finite values"
    diff = np.abs(out - ref)
    max_abs = float(diff.max()) if diff.size else 0.0
    row_scale = np.abs(ref).max(axis=-1)
    row_err = diff.max(axis=-1)
    zero_rows = row_scale == 0
    assert np.all(row_err[zero_rows] == 0), f"{what}: rows with an all-zero reference are not zero"
    rel = row_err[~zero_rows] / row_scale[~zero_rows]
    max_rel = float(rel.max()) if rel.size else 0.0
    assert max_abs <= abs_tol, f"{what}: max abs error {max_abs:.3e} > {abs_tol:.1e}"
    assert max_rel <= row_rel_tol, f"{what}: row-normwise rel error {max_rel:.3e} > {row_rel_tol:.1e}"
    return max_abs, max_rel


def compare_lse(lse, ref, tol=LSE_TOL, what="lse"):
    lse = np.asarray(lse, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert lse.shape == ref.shape
    neg = np.isneginf(ref)
    assert np.all(np.isneginf(lse[neg])), f"{what}: empty ranges must give -inf"
    d = np.abs(lse[~neg] - ref[~neg])
    worst = float(d.max()) if d.size else 0.0
    assert worst <= tol, f"{what}: max |lse error| {worst:.3e} > {tol:.1e}"
    return worst


def compare_ulps(a, b, ulps=2, rowwise=False, what="merge"):
    """|a - b| <= ulps fp16 ulps, element by element, or of each row's largest |b| (rowwise)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    ref = np.abs(b).max(axis=-1, keepdims=True) if rowwise else np.abs(b)
    unit = np.maximum(np.spacing(ref.astype(np.float16)).astype(np.float64), 2.0 ** -24)
    worst = float((np.abs(a - b) / unit).max())
    assert worst <= ulps, f"{what}: {worst:.1f} fp16 ulps > {ulps}"
    return worst


def p_rounding_bound(v):
    """Largest move of a normalised output from rounding p to fp16 before p.V.

    With p_i >= 0 and relative rounding |d_i| <= 2^-11,
    |sum d_i p_i v_i| / sum p_i <= 2^-11 max|v|; 1e-5 covers fp32 summation.
    Poison (NaN) slots in the pool are ignored.
    """
    return 2.0 ** -11 * float(np.nanmax(np.abs(np.asarray(v, dtype=np.float64)))) + 1e-5
