"""Comparison of GPU BF16 outputs with the CPU oracle.

Tolerance (the target's own): with R = bf16_rne(oracle float64) over the
valid rows,
    ||D - R||_F / ||R||_F <= 1e-3    and    max |D - R| <= 2^-7 * max |R|.
R is the BF16-rounded oracle because BF16 rounding alone puts the exact
result about 1.7e-3 (Frobenius) away from the unrounded float64 value, above
the 1e-3 bound; against R a correct float32-accumulating kernel differs
only where float32 summation order moves a value across a BF16 rounding
boundary (1 ulp on roughly 1e-4 of the elements).
Rows that must not be written are compared bit for bit with the sentinel.
"""

from __future__ import annotations

import numpy as np

from oracle import dg_oracle as O

REL_FROB = 1e-3
MAX_ABS_FRAC = 2.0 ** -7
SENTINEL = 0xFFFF


def check_close(d_bits: np.ndarray, ref_f64: np.ndarray, what: str = "") -> dict:
    """d_bits: uint16 GPU output; ref_f64: unrounded oracle values (same shape)."""
    d = O.bf16_bits_to_f64(d_bits)
    r = O.bf16_round(ref_f64)
    assert d.shape == r.shape, (d.shape, r.shape)
    assert np.all(np.isfinite(r)), f"{what}: non-finite reference"
    assert np.all(np.isfinite(d)), f"{what}: non-finite output at {np.argwhere(~np.isfinite(d))[:5].tolist()}"
    diff = d - r
    norm_r = float(np.linalg.norm(r))
    rel = float(np.linalg.norm(diff)) / max(norm_r, 1e-300)
    max_r = float(np.max(np.abs(r))) if r.size else 0.0
    max_err = float(np.max(np.abs(diff))) if r.size else 0.0
    stats = {"rel_frob": rel, "max_abs": max_err, "max_ref": max_r,
             "ulp_mismatch_frac": float(np.mean(d_bits != O.bf16_bits(ref_f64))) if r.size else 0.0}
    assert rel <= REL_FROB, f"{what}: relative Frobenius error {rel:.3e} > {REL_FROB}"
    assert max_err <= MAX_ABS_FRAC * max_r, f"{what}: max abs error {max_err:.3e} > 2^-7 * {max_r:.3e}"
    return stats


def check_untouched(d_bits: np.ndarray, what: str = "") -> None:
    bad = np.argwhere(d_bits != SENTINEL)
    assert bad.size == 0, f"{what}: {len(bad)} elements written outside the valid rows, first {bad[:5].tolist()}"
