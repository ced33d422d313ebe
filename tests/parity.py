"""Comparison of GPU BF16 outputs with the CPU oracle.

With R = bf16_rne(oracle float64) over the valid rows, every comparison
asserts the target's own tolerance
    ||D - R||_F / ||R||_F <= 1e-3    and    max |D - R| <= 2^-7 * max |R|,
and, per element, the bound that follows from the arithmetic of the kernels:
    |D - R| <= ulp(max(|D|, |R|)) + E,
    E = (2^-15 + (nkb + 3) * 2^-24) * sum_k |Ahat[m,k] Bhat[n,k]|.
The kernel computes a float32 value y with |y - x| <= E from the exact sum x
(the matrix cores sum one 128-K block of products to within 2^-15 of the sum
of their magnitudes -- measured up to 1.6e-5, about 2^-16 -- and each of the
nkb promotions into float32 rounds the scale product, the product and the
sum: three roundings of at most 2^-24 each, bounded by (nkb + 3) * 2^-24 of
the magnitudes in all), then rounds y once to BF16. D = bf16(y) and
R = bf16(x) are each within half an ulp of y and x, and the ulp of a BF16
rounding result is at least that of its argument, hence the bound. The same
argument fixes which elements may differ from R at all: if no BF16 rounding
midpoint lies within E of x, bf16(y) = bf16(x), so D must equal R bit for
bit; only elements whose exact value lies within E of a midpoint may round
to the other neighbour. (On random data that is of the order of 1% of the
elements: the matrix cores' sum of a block is only good to about 2^-16 of
the magnitudes, not to float32 rounding.)

R is the BF16-rounded oracle because BF16 rounding alone puts the exact
result about 1.7e-3 (Frobenius) away from the unrounded float64 value, above
the 1e-3 bound. Rows that must not be written are compared bit for bit with
the sentinel.
"""

from __future__ import annotations

import numpy as np

from oracle import dg_oracle as O

REL_FROB = 1e-3
MAX_ABS_FRAC = 2.0 ** -7
MFMA_BLOCK_REL = 2.0 ** -15
F32_ROUND = 2.0 ** -24
SENTINEL = 0xFFFF


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of BF16 values at magnitude |v| (8 significant bits, float32's
    exponent range: 2^(E - 7) for |v| in [2^E, 2^(E+1)), 2^-133 below 2^-126)."""
    _, e = np.frexp(np.abs(np.asarray(v, np.float64)))
    return np.ldexp(1.0, np.maximum(e - 1, -126) - 7)


def midpoint_distance(x: np.ndarray) -> np.ndarray:
    """Distance from each value to the nearest BF16 rounding midpoint (the
    point halfway between bf16(x) and either of its BF16 neighbours)."""
    ax = np.abs(np.asarray(x, np.float64))
    bits = O.bf16_bits(ax).astype(np.int64)
    r = O.bf16_bits_to_f64(bits.astype(np.uint16))
    up = O.bf16_bits_to_f64(np.minimum(bits + 1, 0x7F7F).astype(np.uint16))
    down = O.bf16_bits_to_f64(np.maximum(bits - 1, 0).astype(np.uint16))
    d_up = np.where(bits < 0x7F7F, np.abs(ax - (r + up) / 2), np.inf)
    d_down = np.where(bits > 0, np.abs(ax - (r + down) / 2), ax + 2.0 ** -134)  # below 0: -min/2
    return np.minimum(d_up, d_down)


def element_bound(mag: np.ndarray, k: int) -> np.ndarray:
    """E above for a K of k (k / 128 promotions)."""
    nkb = max(k // 128, 1)
    return (MFMA_BLOCK_REL + (nkb + 3) * F32_ROUND) * np.asarray(mag, np.float64)


def check_close(d_bits: np.ndarray, ref_f64: np.ndarray, what: str = "", mag=None, k=None) -> dict:
    """d_bits: uint16 GPU output; ref_f64: unrounded oracle values; mag: the
    oracle's sum of product magnitudes at the same elements; k: the GEMM's K.
    Without mag/k the per-element bound is skipped (used only where the
    reference is another GPU output rather than the oracle)."""
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
    mismatches = int(np.count_nonzero(np.asarray(d_bits, np.uint16) != O.bf16_bits(ref_f64)))
    stats = {"rel_frob": rel, "max_abs": max_err, "max_ref": max_r,
             "ulp_mismatch_frac": mismatches / max(r.size, 1)}
    assert rel <= REL_FROB, f"{what}: relative Frobenius error {rel:.3e} > {REL_FROB}"
    assert max_err <= MAX_ABS_FRAC * max_r, f"{what}: max abs error {max_err:.3e} > 2^-7 * {max_r:.3e}"
    if mag is not None:
        assert k is not None, "the per-element bound needs K"
        bound = bf16_ulp(np.maximum(np.abs(d), np.abs(r))) + element_bound(mag, k)
        bad = np.abs(diff) > bound
        assert not bad.any(), (f"{what}: {int(bad.sum())} elements beyond the per-element bound, "
                               f"first at {np.argwhere(bad)[:3].tolist()}")
        e = element_bound(mag, k)
        differs = np.asarray(d_bits, np.uint16) != O.bf16_bits(ref_f64)
        # f64 slack: the oracle's own sum is good to K * 2^-52 of the magnitudes
        near = midpoint_distance(ref_f64) <= e + (k + 2) * 2.0 ** -52 * np.asarray(mag, np.float64)
        wrong = differs & ~near
        assert not wrong.any(), (f"{what}: {int(wrong.sum())} elements differ from bf16(oracle) although no "
                                 f"rounding midpoint lies within the error bound, first at "
                                 f"{np.argwhere(wrong)[:3].tolist()}")
        stats["near_midpoint_frac"] = float(np.mean(near)) if r.size else 0.0
    return stats


def check_untouched(d_bits: np.ndarray, what: str = "") -> None:
    bad = np.argwhere(d_bits != SENTINEL)
    assert bad.size == 0, f"{what}: {len(bad)} elements written outside the valid rows, first {bad[:5].tolist()}"


def abs_e4m3(codes: np.ndarray) -> np.ndarray:
    """E4M3 codes of the magnitudes (sign bit cleared; NaN codes stay NaN)."""
    return (np.asarray(codes, np.uint8) & 0x7F).astype(np.uint8)


def abs_e2m1_packed(packed: np.ndarray) -> np.ndarray:
    """Packed E2M1 bytes of the magnitudes (the sign bit of both nibbles cleared)."""
    return (np.asarray(packed, np.uint8) & 0x77).astype(np.uint8)
