"""Pins for the oracle's GEMM, independent of the oracle itself.

Each pin checks the oracle against something other than its own code:
  * exact rational arithmetic (fractions.Fraction) on tiny inputs, with an
    exact round-to-nearest-even to BF16 written on rationals;
  * integer-exact inputs (codes in {-2..2}, power-of-two scales that differ
    per K block, per row and per N block) against a per-block integer closed
    form;
  * all scales 1: torch float64 matmul of the decoded operands;
  * constant operands: a closed form in the scales alone;
  * invariants: grouped == per-group dense, permuting segments permutes rows,
    masked and padding rows untouched, NaN-poisoned padding does not leak,
    the no-padding layout with 128-aligned counts == the contiguous layout;
  * a no-padding row owner map built by walking the counts row by row;
  * UE8M0 scales: a hand-derived table of float32 bit patterns and their
    E8M0 values (tests/golden/e8m0_scale_cases.txt), the float32 variants on
    power-of-two scales, and math.frexp rounding down for other scales;
  * K-grouped GEMM: exact rationals with the indices written out, K-range
    splitting additivity, empty groups, and the dense GEMM as the special
    case of one group with block-constant RHS scales;
  * FP8 x FP4: a hand-derived E2M1 table (tests/golden/e2m1_values.txt), a
    one-hot closed form fixing the packing order and the per-32 scale index,
    exact rationals, and the FP8 UE8M0 GEMM on the same values re-encoded.

test_planted_mistakes_are_caught plants plausible mistakes in a private copy
of the oracle (wrong scale index, transposed RHS scales, wrong FP8 flavour,
truncating or double rounding, dropped K block, missing sign, padding rows
written, off-by-one masks, no-padding groups that restart at row 0, negative
counts that move later groups back, unowned rows written) and checks that at
least one pin fails for each.
"""

import importlib.util
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import dg_oracle as O

ORACLE_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "dg_oracle.py")

CODE_OF = {0: 0x00, 1: 0x38, 2: 0x40, -1: 0xB8, -2: 0xC0}   # E4M3 codes of small integers
# E4M3 codes of the E2M1 values (sign bit 7, exponent bias 7, 3 mantissa bits)
CODE_OF_F = {0.0: 0x00, 0.5: 0x30, 1.0: 0x38, 1.5: 0x3C, 2.0: 0x40, 3.0: 0x44, 4.0: 0x48, 6.0: 0x4C,
             -0.5: 0xB0, -1.0: 0xB8, -1.5: 0xBC, -2.0: 0xC0, -3.0: 0xC4, -4.0: 0xC8, -6.0: 0xCC}


# ---------------------------------------------------------------------------
# Independent helpers
# ---------------------------------------------------------------------------

def _decode_torch(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _bf16_rne_exact(v: Fraction) -> int:
    """BF16 bits of a rational, rounded to nearest even, in exact arithmetic."""
    if v == 0:
        return 0
    neg = v < 0
    a = -v if neg else v
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    quantum = Fraction(2) ** (e - 7)
    t = a / quantum
    n = t.numerator // t.denominator
    rem = t - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = n * quantum
    if val >= Fraction(2) ** 128:
        bits = 0x7F80
    else:
        bits = int(np.array([float(val)], dtype=np.float32).view(np.uint32)[0] >> 16)
    return bits | (0x8000 if neg else 0)


def _random_inputs(rng, m, n, k, groups=None):
    """Random codes (finite, not NaN) and random positive float32 scales."""
    def codes(shape):
        c = rng.integers(0, 256, size=shape).astype(np.uint8)
        c[(c & 0x7F) == 0x7F] = 0x3C  # replace NaN codes
        return c

    def scales(shape):
        return (rng.uniform(0.25, 4.0, size=shape)).astype(np.float32)

    a = codes((m, k))
    sfa = scales((k // 128, (m + 3) // 4 * 4))
    if groups is None:
        return a, sfa, codes((n, k)), scales((n // 128, k // 128))
    return a, sfa, codes((groups, n, k)), scales((groups, n // 128, k // 128))


def _exact_gemm(a, sfa, b, sfb):
    """Exact rational sum_k dec(a) sa * dec(b) sb, as a list of lists of Fractions."""
    m, k = a.shape
    n = b.shape[0]
    av = _decode_torch(a)
    bv = _decode_torch(b)
    fa = [[Fraction(float(av[i, kk])) * Fraction(float(sfa[kk // 128, i])) for kk in range(k)] for i in range(m)]
    fb = [[Fraction(float(bv[j, kk])) * Fraction(float(sfb[j // 128, kk // 128])) for kk in range(k)] for j in range(n)]
    return [[sum(x * y for x, y in zip(fa[i], fb[j])) for j in range(n)] for i in range(m)], fa, fb


def _check_against_exact(oracle_f64, oracle_bits, exact, fa, fb):
    m, n = len(exact), len(exact[0])
    k = len(fa[0])
    checked = 0
    for i in range(m):
        for j in range(n):
            ex = exact[i][j]
            abs_terms = sum(abs(x * y) for x, y in zip(fa[i], fb[j]))
            bound = float(abs_terms) * 2 * k * 2.0 ** -53 + 1e-300
            assert abs(oracle_f64[i, j] - float(ex)) <= bound, (i, j)
            # skip elements so close to a BF16 midpoint that fp64 rounding may flip it
            lo = _bf16_rne_exact(ex - Fraction(bound))
            hi = _bf16_rne_exact(ex + Fraction(bound))
            if lo != hi:
                continue
            assert int(oracle_bits[i, j]) == _bf16_rne_exact(ex), (i, j)
            checked += 1
    assert checked >= 0.95 * m * n


# ---------------------------------------------------------------------------
# Pins, written as functions of an oracle module so that they can also run
# against planted-mistake copies.
# ---------------------------------------------------------------------------

def pin_exact_dense(orc):
    rng = np.random.default_rng(7)
    a, sfa, b, sfb = _random_inputs(rng, 3, 256, 256)
    exact, fa, fb = _exact_gemm(a, sfa, b, sfb)
    f64 = orc.gemm_nt_f64(a, sfa, b, sfb)
    bits = orc.fp8_gemm_nt(a, sfa, b, sfb)
    _check_against_exact(f64, bits, exact, fa, fb)


def pin_exact_brute_force_matches(orc):
    """The oracle's exact-rational brute force equals this file's, which
    decodes through torch instead of the OCP formula."""
    rng = np.random.default_rng(29)
    a, sfa, b, sfb = _random_inputs(rng, 2, 128, 256)
    exact, _, _ = _exact_gemm(a, sfa, b, sfb)
    assert orc.gemm_nt_exact(a, sfa, b, sfb) == exact


def pin_exact_grouped(orc):
    rng = np.random.default_rng(11)
    a, sfa, b, sfb = _random_inputs(rng, 256, 128, 256, groups=2)
    layout = np.full(256, -1, dtype=np.int32)
    layout[0:2] = 0
    layout[128:131] = 1
    d0 = np.full((256, 128), 0xFFFF, dtype=np.uint16)
    d = orc.m_grouped_fp8_gemm_nt_contiguous(a, sfa, b, sfb, layout, d0)
    for g, rows in ((0, [0, 1]), (1, [128, 129, 130])):
        sub_a = a[rows]
        sub_sfa = sfa[:, rows]
        sub_sfa = np.pad(sub_sfa, ((0, 0), (0, (-len(rows)) % 4)))
        exact, fa, fb = _exact_gemm(sub_a, sub_sfa, b[g], sfb[g])
        for ii, r in enumerate(rows):
            for j in range(128):
                assert int(d[r, j]) == _bf16_rne_exact(exact[ii][j]) or abs(
                    float(O.bf16_bits_to_f64(d[r, j])) - float(exact[ii][j])) <= 2.0 ** -7 * abs(float(exact[ii][j]))
    untouched = np.ones(256, bool)
    untouched[[0, 1, 128, 129, 130]] = False
    assert np.all(d[untouched] == 0xFFFF)


def _int_exact_case(rng, m, n, k):
    vals_a = rng.integers(-2, 3, size=(m, k))
    vals_b = rng.integers(-2, 3, size=(n, k))
    a = np.vectorize(CODE_OF.get)(vals_a).astype(np.uint8)
    b = np.vectorize(CODE_OF.get)(vals_b).astype(np.uint8)
    ld = (m + 3) // 4 * 4
    # exponents that differ with the K block and the row / N block
    ea = (np.arange(k // 128)[:, None] * 3 + np.arange(ld)[None, :]) % 3 - 1        # in {-1, 0, 1}
    eb = (np.arange(n // 128)[:, None] * 2 + np.arange(k // 128)[None, :] * 5) % 3 - 1
    sfa = np.ldexp(1.0, ea).astype(np.float32)
    sfb = np.ldexp(1.0, eb).astype(np.float32)
    return vals_a, vals_b, a, sfa, b, sfb, ea, eb


def pin_integer_closed_form(orc):
    rng = np.random.default_rng(3)
    m, n, k = 12, 256, 640
    vals_a, vals_b, a, sfa, b, sfb, ea, eb = _int_exact_case(rng, m, n, k)
    f64 = orc.gemm_nt_f64(a, sfa, b, sfb)
    bits = orc.fp8_gemm_nt(a, sfa, b, sfb)
    for i in range(m):
        for j in range(n):
            total = Fraction(0)
            for kb in range(k // 128):
                s = int(np.dot(vals_a[i, kb * 128:(kb + 1) * 128], vals_b[j, kb * 128:(kb + 1) * 128]))
                total += s * Fraction(2) ** int(ea[kb, i] + eb[j // 128, kb])
            assert f64[i, j] == float(total), (i, j, f64[i, j], total)
            assert int(bits[i, j]) == _bf16_rne_exact(total), (i, j)


def pin_unit_scales_matmul(orc):
    rng = np.random.default_rng(5)
    a, _, b, _ = _random_inputs(rng, 40, 256, 384)
    sfa = np.ones((3, 40), np.float32)
    sfb = np.ones((2, 3), np.float32)
    ref = torch.from_numpy(_decode_torch(a)) @ torch.from_numpy(_decode_torch(b)).T
    got = orc.gemm_nt_f64(a, sfa, b, sfb)
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-12)


def pin_constant_operands(orc):
    # A all 1.5 (code 0x3C), B all -3 (code 0xC4): D[m,n] = 128 * 1.5 * -3 * sum_kb sa[kb][m] sb[n//128][kb]
    m, n, k = 6, 384, 512
    a = np.full((m, k), 0x3C, np.uint8)
    b = np.full((n, k), 0xC4, np.uint8)
    sfa = (np.arange(k // 128)[:, None] + 1.0 + 0.25 * np.arange(8)[None, :]).astype(np.float32)
    sfb = (0.5 + np.arange(n // 128)[:, None] * 2.0 + np.arange(k // 128)[None, :] * 0.125).astype(np.float32)
    got = orc.gemm_nt_f64(a, sfa, b, sfb)
    for i in range(m):
        for j in range(n):
            expect = 128 * 1.5 * -3.0 * sum(float(sfa[kb, i]) * float(sfb[j // 128, kb]) for kb in range(k // 128))
            assert math.isclose(got[i, j], expect, rel_tol=1e-13), (i, j)


def pin_grouped_is_per_group_dense(orc):
    rng = np.random.default_rng(9)
    rows = [130, 0, 77, 256]
    layout = np.concatenate([np.r_[np.full(r, g), np.full((-r) % 128, -1)] for g, r in enumerate(rows)]).astype(np.int32)
    m = layout.size
    a, sfa, b, sfb = _random_inputs(rng, m, 256, 256, groups=len(rows))
    d0 = np.full((m, 256), 0xFFFF, np.uint16)
    d = orc.m_grouped_fp8_gemm_nt_contiguous(a, sfa, b, sfb, layout, d0)
    for g in range(len(rows)):
        idx = np.nonzero(layout == g)[0]
        if idx.size == 0:
            continue
        sub_sfa = np.pad(sfa[:, idx], ((0, 0), (0, (-idx.size) % 4)))
        dense = orc.fp8_gemm_nt(a[idx], sub_sfa, b[g], sfb[g])
        assert np.array_equal(d[idx], dense)
    assert np.all(d[layout < 0] == 0xFFFF)
    # permuting whole segments permutes the output rows
    segs, start = [], 0
    for g, r in enumerate(rows):
        p = r + (-r) % 128
        segs.append(np.arange(start, start + p))
        start += p
    order = [3, 0, 2, 1]
    perm = np.concatenate([segs[i] for i in order])
    sfa_p = np.pad(sfa[:, perm], ((0, 0), (0, sfa.shape[1] - perm.size)))
    d_p = orc.m_grouped_fp8_gemm_nt_contiguous(a[perm], sfa_p, b, sfb, layout[perm], d0)
    assert np.array_equal(d_p, d[perm])


def pin_masked_rows(orc):
    rng = np.random.default_rng(13)
    g_count, max_m, n, k = 4, 40, 128, 256
    a, _, b, sfb = _random_inputs(rng, g_count * max_m, n, k, groups=g_count)
    a = a.reshape(g_count, max_m, k).copy()
    sfa = rng.uniform(0.5, 2, size=(g_count, k // 128, max_m)).astype(np.float32)
    masked = np.array([0, 1, 40, 17], np.int32)
    for g in range(g_count):
        a[g, masked[g]:] = 0x7F   # NaN beyond the valid rows must not leak
    d0 = np.full((g_count, max_m, n), 0xFFFF, np.uint16)
    d = orc.m_grouped_fp8_gemm_nt_masked(a, sfa, b, sfb, masked, d0)
    for g in range(g_count):
        v = masked[g]
        assert np.all(d[g, v:] == 0xFFFF)
        if v:
            dense = orc.fp8_gemm_nt(a[g, :v], sfa[g], b[g], sfb[g])
            assert np.array_equal(d[g, :v], dense)
            assert not np.any(np.isnan(O.bf16_bits_to_f64(d[g, :v])))
    # out-of-range counts are clamped
    d2 = orc.m_grouped_fp8_gemm_nt_masked(a, sfa, b, sfb, np.array([-5, 1, 99, 17], np.int32), d0)
    assert np.array_equal(d2[1:3], d[1:3]) and np.all(d2[0] == 0xFFFF)


def _nopad_owner(counts, m_rows):
    """Group of each row of the no-padding layout, walked row by row: group
    g's max(c_g, 0) rows follow group g - 1's; rows no group reaches, and
    anything past m_rows, are -1."""
    owner = []
    for g, c in enumerate(counts):
        owner.extend([g] * max(int(c), 0))
    owner = owner[:m_rows]
    return np.array(owner + [-1] * (m_rows - len(owner)), dtype=np.int64)


def pin_exact_nopad(orc):
    """Tiny no-padding case against exact rationals, with a row owner map
    built by walking the counts one row at a time."""
    rng = np.random.default_rng(23)
    counts = [2, 0, 3, -1]
    m_rows = 7                      # rows 5 and 6 belong to no group
    a, sfa, b, sfb = _random_inputs(rng, m_rows, 128, 256, groups=len(counts))
    owner = _nopad_owner(counts, m_rows)
    d0 = np.full((m_rows, 128), 0xFFFF, dtype=np.uint16)
    d = orc.m_grouped_fp8_gemm_nt_nopad(a, sfa, b, sfb, np.array(counts, np.int32), d0)
    for r in range(m_rows):
        g = int(owner[r])
        if g < 0:
            assert np.all(d[r] == 0xFFFF), r
            continue
        sub_sfa = np.pad(sfa[:, [r]], ((0, 0), (0, 3)))
        exact, _, _ = _exact_gemm(a[[r]], sub_sfa, b[g], sfb[g])
        for j in range(128):
            ex = exact[0][j]
            assert int(d[r, j]) == _bf16_rne_exact(ex) or abs(
                float(O.bf16_bits_to_f64(d[r, j])) - float(ex)) <= 2.0 ** -7 * abs(float(ex)), (r, j)


def pin_nopad_layout_invariants(orc):
    """No-padding rows: (1) 128-aligned counts give the contiguous layout's
    result on the same rows; (2) each group equals a dense call on its rows;
    (3) counts past M are cut off at M and negative counts own nothing;
    (4) NaN-poisoned rows that no group owns never leak."""
    rng = np.random.default_rng(29)
    counts = [128, 0, 256]
    m_rows = 384
    a, sfa, b, sfb = _random_inputs(rng, m_rows, 128, 256, groups=3)
    d0 = np.full((m_rows, 128), 0xFFFF, np.uint16)
    layout = np.r_[np.zeros(128), np.full(256, 2)].astype(np.int32)
    d_np = orc.m_grouped_fp8_gemm_nt_nopad(a, sfa, b, sfb, np.array(counts, np.int32), d0)
    d_ct = orc.m_grouped_fp8_gemm_nt_contiguous(a, sfa, b, sfb, layout, d0)
    assert np.array_equal(d_np, d_ct)

    counts = [-4, 5, 0, 9, 100]
    m_rows = 20
    a, sfa, b, sfb = _random_inputs(rng, m_rows, 128, 256, groups=len(counts))
    d0 = np.full((m_rows, 128), 0xFFFF, np.uint16)
    d = orc.m_grouped_fp8_gemm_nt_nopad(a, sfa, b, sfb, np.array(counts, np.int32), d0)
    owner = _nopad_owner(counts, m_rows)
    assert list(owner[:5]) == [1] * 5 and list(owner[5:14]) == [3] * 9 and list(owner[14:]) == [4] * 6
    for g in range(len(counts)):
        rows = np.nonzero(owner == g)[0]
        if rows.size == 0:
            continue
        sub_sfa = np.pad(sfa[:, rows], ((0, 0), (0, (-rows.size) % 4)))
        assert np.array_equal(d[rows], orc.fp8_gemm_nt(a[rows], sub_sfa, b[g], sfb[g])), g

    counts = [3, 4]
    m_rows = 12
    a, sfa, b, sfb = _random_inputs(rng, m_rows, 128, 256, groups=2)
    a[7:] = 0x7F
    d0 = np.full((m_rows, 128), 0xFFFF, np.uint16)
    d = orc.m_grouped_fp8_gemm_nt_nopad(a, sfa, b, sfb, np.array(counts, np.int32), d0)
    assert np.all(d[7:] == 0xFFFF)
    assert not np.any(np.isnan(O.bf16_bits_to_f64(d[:7])))


def _pow2_inputs(rng, m, n, k, groups=None):
    a, sfa, b, sfb = _random_inputs(rng, m, n, k, groups)
    return (a, np.ldexp(1.0, rng.integers(-8, 3, size=sfa.shape)).astype(np.float32), b,
            np.ldexp(1.0, rng.integers(-8, 3, size=sfb.shape)).astype(np.float32))


def pin_ue8m0_power_of_two_identity(orc):
    """With scales that are powers of two the UE8M0 variants are the float32
    variants, bit for bit, for every layout."""
    rng = np.random.default_rng(41)
    a, sfa, b, sfb = _pow2_inputs(rng, 40, 256, 384)
    assert np.array_equal(orc.fp8_gemm_nt_ue8m0(a, sfa, b, sfb), orc.fp8_gemm_nt(a, sfa, b, sfb))
    a, sfa, b, sfb = _pow2_inputs(rng, 256, 128, 256, groups=2)
    d0 = np.full((256, 128), 0xFFFF, np.uint16)
    layout = np.r_[np.zeros(100), np.full(28, -1), np.ones(128)].astype(np.int32)
    assert np.array_equal(orc.m_grouped_fp8_gemm_nt_contiguous_ue8m0(a, sfa, b, sfb, layout, d0),
                          orc.m_grouped_fp8_gemm_nt_contiguous(a, sfa, b, sfb, layout, d0))
    counts = np.array([100, 120], np.int32)
    assert np.array_equal(orc.m_grouped_fp8_gemm_nt_nopad_ue8m0(a, sfa, b, sfb, counts, d0),
                          orc.m_grouped_fp8_gemm_nt_nopad(a, sfa, b, sfb, counts, d0))
    am = a.reshape(2, 128, 256)
    sfam = np.stack([sfa[:, :128], sfa[:, 128:]])
    d0m = np.full((2, 128, 128), 0xFFFF, np.uint16)
    assert np.array_equal(orc.m_grouped_fp8_gemm_nt_masked_ue8m0(am, sfam, b, sfb, counts, d0m),
                          orc.m_grouped_fp8_gemm_nt_masked(am, sfam, b, sfb, counts, d0m))
    kb_sfb = np.ldexp(1.0, rng.integers(-8, 3, size=(2, 128))).astype(np.float32)
    ks = [128, 128]
    np.testing.assert_array_equal(
        orc.k_grouped_fp8_gemm_nt_contiguous_ue8m0(a[:, :256], sfa[:2], b[0], kb_sfb, ks),
        orc.k_grouped_fp8_gemm_nt_contiguous(a[:, :256], sfa[:2], b[0], kb_sfb, ks))


def pin_ue8m0_drops_mantissa(orc):
    """Arbitrary positive scales: the UE8M0 variant equals the float32 one on
    scales rounded down to powers of two (math.frexp: s = f * 2^e, f in
    [0.5, 1), so the power of two at or below s is 2^(e - 1))."""
    rng = np.random.default_rng(43)
    a, sfa, b, sfb = _random_inputs(rng, 24, 256, 384)

    def floor_pow2(x):
        return np.vectorize(lambda v: math.ldexp(1.0, math.frexp(float(v))[1] - 1))(x).astype(np.float32)
    assert np.array_equal(orc.fp8_gemm_nt_ue8m0(a, sfa, b, sfb),
                          orc.fp8_gemm_nt(a, floor_pow2(sfa), b, floor_pow2(sfb)))


def pin_e8m0_golden(orc):
    import test_oracle_formats as F
    F.check_e8m0_golden(orc)


def pin_exact_k_grouped(orc):
    """Tiny K-grouped case against exact rationals, indices written out:
    D[g][i][j] = C[g][i][j] + sum over group g's k of
    dec(a[i,k]) sfa[k//128, i] dec(b[j,k]) sfb[k//128, j]."""
    rng = np.random.default_rng(47)
    ks = [128, 0, 256]
    m_rows, n, k = 3, 5, sum(ks)
    a = rng.integers(0, 256, size=(m_rows, k)).astype(np.uint8)
    b = rng.integers(0, 256, size=(n, k)).astype(np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x30
    b[(b & 0x7F) == 0x7F] = 0x30
    sfa = rng.uniform(0.25, 4.0, size=(k // 128, 4)).astype(np.float32)
    sfb = rng.uniform(0.25, 4.0, size=(k // 128, 8)).astype(np.float32)
    c = rng.standard_normal((3, m_rows, n)).astype(np.float32)
    av, bv = _decode_torch(a), _decode_torch(b)
    d = orc.k_grouped_fp8_gemm_nt_contiguous(a, sfa, b, sfb, ks, c)
    starts = [0, 128, 128]
    for g in range(3):
        for i in range(m_rows):
            for j in range(n):
                terms = [Fraction(float(av[i, kk])) * Fraction(float(sfa[kk // 128, i]))
                         * Fraction(float(bv[j, kk])) * Fraction(float(sfb[kk // 128, j]))
                         for kk in range(starts[g], starts[g] + ks[g])]
                exact = Fraction(float(c[g, i, j])) + sum(terms, Fraction(0))
                bound = (float(sum(abs(t) for t in terms)) + abs(float(c[g, i, j]))) * (k + 2) * 2.0 ** -52
                assert abs(d[g, i, j] - float(exact)) <= bound, (g, i, j)


def pin_k_grouped_invariants(orc):
    """(1) splitting a group's K range in two and adding the two outputs
    gives the merged group's; (2) an empty group returns C (zeros without
    C); (3) one group with RHS scales constant over 128-row blocks of N is
    the dense GEMM with those block scales."""
    rng = np.random.default_rng(53)
    m_rows, n = 6, 256
    a, _, b, _ = _random_inputs(rng, m_rows, n, 512)
    sfa = rng.uniform(0.5, 2, size=(4, 8)).astype(np.float32)
    sfb = rng.uniform(0.5, 2, size=(4, 256)).astype(np.float32)
    merged = orc.k_grouped_fp8_gemm_nt_contiguous(a, sfa, b, sfb, [128, 384])
    split = orc.k_grouped_fp8_gemm_nt_contiguous(a, sfa, b, sfb, [128, 128, 256])
    np.testing.assert_allclose(split[1] + split[2], merged[1], rtol=1e-12, atol=1e-9)
    np.testing.assert_array_equal(split[0], merged[0])
    c = rng.standard_normal((3, m_rows, n))
    with_empty = orc.k_grouped_fp8_gemm_nt_contiguous(a, sfa, b, sfb, [128, 0, 384], c)
    assert np.array_equal(with_empty[1], c[1])
    assert np.all(orc.k_grouped_fp8_gemm_nt_contiguous(a, sfa, b, sfb, [0, 512])[0] == 0)
    blocks = rng.uniform(0.5, 2, size=(n // 128, 4)).astype(np.float32)     # [N/128][K/128]
    sfb_rows = np.repeat(blocks.T, 128, axis=1)                            # [K/128][N]
    one = orc.k_grouped_fp8_gemm_nt_contiguous(a, sfa, b, sfb_rows, [512])[0]
    np.testing.assert_allclose(one, orc.gemm_nt_f64(a, sfa, b, blocks), rtol=1e-12, atol=1e-9)


E2M1_OF = {0.0: 0x0, 0.5: 0x1, 1.0: 0x2, 1.5: 0x3, 2.0: 0x4, 3.0: 0x5, 4.0: 0x6, 6.0: 0x7}


def _pack_e2m1(values):
    """Pack E2M1 values [N, K] two per byte, element 2j in the low nibble of byte j."""
    codes = np.vectorize(lambda v: E2M1_OF[abs(v)] | (0x8 if v < 0 else 0))(values).astype(np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def pin_e2m1_golden(orc):
    import test_oracle_formats as F
    F.check_e2m1_golden(orc)


def pin_fp4_element_positions(orc):
    """One nonzero E2M1 element per B row, at K position k_n (odd and even
    positions, in different 32-K scale blocks): D[m][n] = A[m][k_n] *
    sa * sb, a closed form that fixes the packing order and the scale index."""
    rng = np.random.default_rng(61)
    k, n, rows = 256, 128, 8
    vals_a = rng.integers(-2, 3, size=(rows, k))
    a = np.vectorize(CODE_OF.get)(vals_a).astype(np.uint8)
    pos = rng.integers(0, k, size=n)
    bvals = np.zeros((n, k))
    bvals[np.arange(n), pos] = 1.5
    b = _pack_e2m1(bvals)[None]
    sfa = np.ldexp(1.0, rng.integers(-3, 3, size=(k // 128, rows))).astype(np.float32)
    e_b = rng.integers(-3, 3, size=(k // 32, n))
    sfb = np.ldexp(1.0, e_b).astype(np.float32)[None]
    layout = np.zeros(rows, np.int32)
    a_pad = np.concatenate([a, np.zeros((128 - rows, k), np.uint8)])
    lay_pad = np.r_[layout, np.full(128 - rows, -1)].astype(np.int32)
    sfa_pad = np.pad(sfa, ((0, 0), (0, 128 - rows)))
    d = orc.m_grouped_fp8_fp4_gemm_nt_contiguous(a_pad, sfa_pad, b, sfb, lay_pad,
                                                 np.full((128, n), 0xFFFF, np.uint16))
    got = O.bf16_bits_to_f64(d[:rows])
    for i in range(rows):
        for j in range(n):
            kk = int(pos[j])
            expect = vals_a[i, kk] * 1.5 * float(sfa[kk // 128, i]) * 2.0 ** int(e_b[kk // 32, j])
            assert got[i, j] == expect, (i, j, kk)


def pin_exact_fp8_fp4(orc):
    """A tiny masked FP8 x FP4 case against exact rationals (values from a
    hand-written E2M1 table, scales 2^e)."""
    rng = np.random.default_rng(67)
    g_count, max_m, n, k = 2, 3, 128, 256
    a, _, _, _ = _random_inputs(rng, g_count * max_m, n, k)
    a = a.reshape(g_count, max_m, k)
    grid = np.array(sorted(E2M1_OF))
    bvals = rng.choice(grid, size=(g_count, n, k)) * rng.choice([-1.0, 1.0], size=(g_count, n, k))
    b = np.stack([_pack_e2m1(bvals[g]) for g in range(g_count)])
    ea = rng.integers(-4, 4, size=(g_count, k // 128, 4))
    eb = rng.integers(-4, 4, size=(g_count, k // 32, n))
    sfa, sfb = np.ldexp(1.0, ea).astype(np.float32), np.ldexp(1.0, eb).astype(np.float32)
    masked = np.array([3, 2], np.int32)
    d = orc.m_grouped_fp8_fp4_gemm_nt_masked(a, sfa, b, sfb, masked, np.full((g_count, max_m, n), 0xFFFF, np.uint16))
    av = _decode_torch(a.reshape(-1, k)).reshape(g_count, max_m, k)
    for g in range(g_count):
        for i in range(masked[g]):
            for j in range(0, n, 7):
                ex = sum(Fraction(float(av[g, i, kk])) * Fraction(2) ** int(ea[g, kk // 128, i])
                         * Fraction(float(bvals[g, j, kk])) * Fraction(2) ** int(eb[g, kk // 32, j])
                         for kk in range(k))
                assert int(d[g, i, j]) == _bf16_rne_exact(ex), (g, i, j)
    assert np.all(d[1, 2:] == 0xFFFF)


def pin_fp4_matches_fp8_on_shared_values(orc):
    """Every E2M1 value is an E4M3 value: with RHS scales constant over
    128 x 128 blocks, the FP8 x FP4 GEMM equals the FP8 UE8M0 GEMM on the same
    values re-encoded as E4M3."""
    rng = np.random.default_rng(71)
    n, k, m_rows = 256, 256, 128
    a, _, _, _ = _random_inputs(rng, m_rows, n, k)
    grid = np.array(sorted(E2M1_OF))
    bvals = rng.choice(grid, size=(n, k)) * rng.choice([-1.0, 1.0], size=(n, k))
    b4 = _pack_e2m1(bvals)[None]
    b8 = np.vectorize(lambda v: CODE_OF_F[v])(bvals).astype(np.uint8)[None]
    eblk = rng.integers(-3, 3, size=(n // 128, k // 128))
    sfb8 = np.ldexp(1.0, eblk).astype(np.float32)[None]
    sfb4 = np.ldexp(1.0, np.repeat(np.repeat(eblk.T, 4, axis=0), 128, axis=1)).astype(np.float32)[None]
    sfa = np.ldexp(1.0, rng.integers(-3, 3, size=(k // 128, m_rows))).astype(np.float32)
    layout = np.zeros(m_rows, np.int32)
    d0 = np.full((m_rows, n), 0xFFFF, np.uint16)
    assert np.array_equal(orc.m_grouped_fp8_fp4_gemm_nt_contiguous(a, sfa, b4, sfb4, layout, d0),
                          orc.m_grouped_fp8_gemm_nt_contiguous_ue8m0(a, sfa, b8, sfb8, layout, d0))


def pin_contiguous_poisoned_padding(orc):
    rng = np.random.default_rng(17)
    rows = [5, 128, 1]
    layout = np.concatenate([np.r_[np.full(r, g), np.full((-r) % 128, -1)] for g, r in enumerate(rows)]).astype(np.int32)
    m = layout.size
    a, sfa, b, sfb = _random_inputs(rng, m, 128, 256, groups=3)
    a[layout < 0] = 0x7F
    d = orc.m_grouped_fp8_gemm_nt_contiguous(a, sfa, b, sfb, layout, np.full((m, 128), 0xFFFF, np.uint16))
    assert np.all(d[layout < 0] == 0xFFFF)
    assert not np.any(np.isnan(O.bf16_bits_to_f64(d[layout >= 0])))


def pin_sampled_matches_full(orc):
    rng = np.random.default_rng(19)
    a, sfa, b, sfb = _random_inputs(rng, 64, 384, 384)
    full = orc.gemm_nt_f64(a, sfa, b, sfb)
    rows, cols = np.array([0, 5, 63]), np.array([1, 200, 383])
    # same sums, possibly a different BLAS summation order: equal to fp64 rounding
    np.testing.assert_allclose(orc.dense_f64_at(a, sfa, b, sfb, rows, cols), full[np.ix_(rows, cols)],
                               rtol=1e-12, atol=1e-9)


def pin_formats_golden(orc):
    """The hand-derived E4M3 and BF16 tables in tests/golden."""
    import test_oracle_formats as F
    F.check_e4m3_golden(orc)
    F.check_bf16_golden(orc)


def pin_near_tie_gemm(orc):
    """A product whose exact value is just above a BF16 tie: 1 + 2^-8 + 2^-34.

    Row 0 of A is [1, 2^-4, 0...] in block 0 and [2^-9, 0...] in block 1;
    row 0 of B is [1, 2^-4, 0...] in block 0 and [1, 0...] in block 1; the
    second K block carries scales 2^-10 (A) and 2^-15 (B). A single rounding
    gives 1 + 2^-7; rounding through float32 first gives 1.0.
    """
    k = 256
    a = np.zeros((1, k), np.uint8)
    b = np.zeros((128, k), np.uint8)
    a[0, 0], a[0, 1], a[0, 128] = 0x38, 0x18, 0x01        # 1, 2^-4, 2^-9
    b[0, 0], b[0, 1], b[0, 128] = 0x38, 0x18, 0x38        # 1, 2^-4, 1
    sfa = np.array([[1.0, 0, 0, 0], [2.0 ** -10, 0, 0, 0]], np.float32)
    sfb = np.array([[1.0, 2.0 ** -15]], np.float32)
    f64 = orc.gemm_nt_f64(a, sfa, b, sfb)
    assert f64[0, 0] == 1.0 + 2.0 ** -8 + 2.0 ** -34
    assert int(orc.fp8_gemm_nt(a, sfa, b, sfb)[0, 0]) == 0x3F81


# ---------------------------------------------------------------------------
# The contiguous layout's row rule, and the sampled-evaluation functions that
# the full-size GPU checks use as their reference
# ---------------------------------------------------------------------------

def _contiguous_owner_walk(layout, num_groups):
    """Owner of each row, walked block by block: a 128-row block takes the id
    of its first row; a row is computed for that id when its own id is the
    same and the id names a group."""
    owner = []
    for start in range(0, len(layout), 128):
        block_id = int(layout[start])
        for r in range(start, start + 128):
            ok = int(layout[r]) == block_id and 0 <= block_id < num_groups
            owner.append(block_id if ok else -1)
    return np.array(owner)


def pin_contiguous_block_rule(orc):
    """Ids that change inside a 128-row block: only rows whose id is their
    block's first-row id (and names a group) are written, each equal to a
    dense GEMM of its group; aligned layouts write every row with a valid id."""
    rng = np.random.default_rng(83)
    g_count, n, k = 3, 128, 256
    layout = np.full(512, -1, np.int32)
    layout[0:100] = 0          # block 0: group 0, rows 100..127 padding
    layout[100:128] = 1        # ... and rows of group 1 inside group 0's block (not written)
    layout[128:200] = 1        # block 1: group 1
    layout[200:256] = 2        # ... group 2 inside group 1's block (not written)
    layout[256] = -1           # block 2 starts with padding: nothing in it is written
    layout[257:300] = 2
    layout[384:500] = 5        # block 3: an id outside [0, G): nothing written
    a, sfa, b, sfb = _random_inputs(rng, 512, n, k, groups=g_count)
    d0 = np.full((512, n), 0xFFFF, np.uint16)
    d = orc.m_grouped_fp8_gemm_nt_contiguous(a, sfa, b, sfb, layout, d0)
    owner = _contiguous_owner_walk(layout, g_count)
    assert np.array_equal(orc.contiguous_row_groups(layout, g_count), owner)
    assert np.array_equal(np.nonzero(owner >= 0)[0], np.r_[0:100, 128:200])
    assert np.all(d[owner < 0] == 0xFFFF)
    for g in range(g_count):
        idx = np.nonzero(owner == g)[0]
        if idx.size:
            sub_sfa = np.pad(sfa[:, idx], ((0, 0), (0, (-idx.size) % 4)))
            assert np.array_equal(d[idx], orc.fp8_gemm_nt(a[idx], sub_sfa, b[g], sfb[g]))
    aligned = np.r_[np.zeros(100), np.full(28, -1), np.full(128, 2), np.ones(60), np.full(68, -1)].astype(np.int32)
    assert np.array_equal(orc.contiguous_row_groups(aligned, g_count), np.where(aligned >= 0, aligned, -1))
    fp4 = orc.m_grouped_fp8_fp4_gemm_nt_contiguous(
        a, np.ldexp(1.0, np.round(np.log2(sfa)).astype(np.int64)).astype(np.float32),
        rng.integers(0, 256, size=(g_count, n, k // 2)).astype(np.uint8),
        np.ones((g_count, k // 32, n), np.float32), layout, d0)
    assert np.all(fp4[owner < 0] == 0xFFFF) and np.all(fp4[owner >= 0] != 0xFFFF)


def _int_codes(rng, shape):
    return np.vectorize(CODE_OF.get)(rng.integers(-2, 3, size=shape)).astype(np.uint8)


def _pow2(rng, shape, lo=-2, hi=3):
    return np.ldexp(1.0, rng.integers(lo, hi, size=shape)).astype(np.float32)


def _abs_codes(c):
    return (np.asarray(c, np.uint8) & 0x7F).astype(np.uint8)


def pin_sampled_functions_match_full(orc):
    """Each *_f64_at function equals its full oracle counterpart on the rows
    and columns it is asked for (first and last rows of every group included),
    and is NaN exactly where the full function leaves D untouched; with
    abs_sum its magnitude equals the full function run on |operands|.
    Integer-valued codes and power-of-two scales make every sum exact, so the
    comparisons are exact."""
    rng = np.random.default_rng(89)
    n, k = 256, 384
    sentinel = 0xFFFF

    def bits_or_nan(vals):
        out = orc.bf16_bits(np.nan_to_num(vals))
        out[np.isnan(vals)] = sentinel
        return out

    # contiguous: three aligned segments with padding, one empty group
    rows_g = [130, 0, 77, 128]
    layout = np.concatenate([np.r_[np.full(r, g), np.full((-r) % 128, -1)] for g, r in enumerate(rows_g)])
    layout = layout.astype(np.int32)
    m = layout.size
    a, b = _int_codes(rng, (m, k)), _int_codes(rng, (4, n, k))
    sfa, sfb = _pow2(rng, (k // 128, m)), _pow2(rng, (4, n // 128, k // 128))
    full = orc.m_grouped_fp8_gemm_nt_contiguous(a, sfa, b, sfb, layout, np.full((m, n), sentinel, np.uint16))
    rows = np.r_[0, 1, 129, 130, 255, 256, 332, 333, 383, 384, 511]
    cols = np.r_[0, 5, 127, 128, 255]
    val, mag = orc.contiguous_f64_at(a, sfa, b, sfb, layout, rows, cols, abs_sum=True)
    assert np.array_equal(bits_or_nan(val), full[np.ix_(rows, cols)])
    full_abs = orc.m_grouped_fp8_gemm_nt_contiguous(_abs_codes(a), sfa, _abs_codes(b), sfb, layout,
                                                    np.full((m, n), sentinel, np.uint16))
    assert np.array_equal(bits_or_nan(mag), full_abs[np.ix_(rows, cols)])

    # masked: counts 0, 1, max, clamped from above and below
    g_count, max_m = 5, 40
    a = _int_codes(rng, (g_count, max_m, k))
    b = _int_codes(rng, (g_count, n, k))
    sfa, sfb = _pow2(rng, (g_count, k // 128, max_m)), _pow2(rng, (g_count, n // 128, k // 128))
    masked = np.array([0, 1, 40, 99, 17], np.int32)
    d0 = np.full((g_count, max_m, n), sentinel, np.uint16)
    full = orc.m_grouped_fp8_gemm_nt_masked(a, sfa, b, sfb, masked, d0)
    full_abs = orc.m_grouped_fp8_gemm_nt_masked(_abs_codes(a), sfa, _abs_codes(b), sfb, masked, d0)
    rows = np.r_[0, 1, 2, 16, 17, 39]
    for g in range(g_count):
        val, mag = orc.masked_f64_at(a, sfa, b, sfb, masked, g, rows, cols, abs_sum=True)
        assert np.array_equal(bits_or_nan(val), full[g][np.ix_(rows, cols)]), g
        assert np.array_equal(bits_or_nan(mag), full_abs[g][np.ix_(rows, cols)]), g

    # no-padding: unaligned groups, an empty one, rows no group owns
    counts = np.array([5, 0, 130, 1, 60], np.int32)
    m = 200
    a, b = _int_codes(rng, (m, k)), _int_codes(rng, (5, n, k))
    sfa, sfb = _pow2(rng, (k // 128, m)), _pow2(rng, (5, n // 128, k // 128))
    full = orc.m_grouped_fp8_gemm_nt_nopad(a, sfa, b, sfb, counts, np.full((m, n), sentinel, np.uint16))
    full_abs = orc.m_grouped_fp8_gemm_nt_nopad(_abs_codes(a), sfa, _abs_codes(b), sfb, counts,
                                               np.full((m, n), sentinel, np.uint16))
    rows = np.r_[0, 4, 5, 134, 135, 136, 137, 195, 196, 199]
    val, mag = orc.nopad_f64_at(a, sfa, b, sfb, counts, rows, cols, abs_sum=True)
    assert np.array_equal(bits_or_nan(val), full[np.ix_(rows, cols)])
    assert np.array_equal(bits_or_nan(mag), full_abs[np.ix_(rows, cols)])

    # K-grouped: per-row scales of both operands, an empty group, C
    ks = [128, 0, 256, 384]
    m, nk = 130, 260
    a, b = _int_codes(rng, (m, sum(ks))), _int_codes(rng, (nk, sum(ks)))
    sfa, sfb = _pow2(rng, (sum(ks) // 128, 132)), _pow2(rng, (sum(ks) // 128, 260))
    c = rng.integers(-8, 9, size=(len(ks), m, nk)).astype(np.float64)
    full = orc.k_grouped_fp8_gemm_nt_contiguous(a, sfa, b, sfb, ks, c)
    full_abs = orc.k_grouped_fp8_gemm_nt_contiguous(_abs_codes(a), sfa, _abs_codes(b), sfb, ks, np.abs(c))
    rows, kcols = np.r_[0, 1, 127, 128, 129], np.r_[0, 1, 127, 128, 200, 259]
    for g in range(len(ks)):
        val, mag = orc.k_grouped_f64_at(a, sfa, b, sfb, ks, g, rows, kcols, c, abs_sum=True)
        assert np.array_equal(val, full[g][np.ix_(rows, kcols)]), g
        assert np.array_equal(mag, full_abs[g][np.ix_(rows, kcols)]), g

    # FP8 x FP4: one group of a masked batch
    grid = np.array(sorted(E2M1_OF))
    g_count, max_m, kf = 2, 20, 256
    a = _int_codes(rng, (g_count, max_m, kf))
    bvals = rng.choice(grid, size=(g_count, n, kf)) * rng.choice([-1.0, 1.0], size=(g_count, n, kf))
    b = np.stack([_pack_e2m1(bvals[g]) for g in range(g_count)])
    b_abs = np.stack([_pack_e2m1(np.abs(bvals[g])) for g in range(g_count)])
    sfa, sfb = _pow2(rng, (g_count, kf // 128, max_m)), _pow2(rng, (g_count, kf // 32, n))
    masked = np.array([20, 20], np.int32)
    d0 = np.full((g_count, max_m, n), sentinel, np.uint16)
    full = orc.m_grouped_fp8_fp4_gemm_nt_masked(a, sfa, b, sfb, masked, d0)
    full_abs = orc.m_grouped_fp8_fp4_gemm_nt_masked(_abs_codes(a), sfa, b_abs, sfb, masked, d0)
    rows = np.r_[0, 1, 18, 19]
    for g in range(g_count):
        val, mag = orc.fp8_fp4_f64_at(a[g], sfa[g], b[g], sfb[g], rows, cols, abs_sum=True)
        assert np.array_equal(orc.bf16_bits(val), full[g][np.ix_(rows, cols)]), g
        assert np.array_equal(orc.bf16_bits(mag), full_abs[g][np.ix_(rows, cols)]), g


PINS = [
    pin_formats_golden,
    pin_near_tie_gemm,
    pin_exact_dense,
    pin_exact_brute_force_matches,
    pin_exact_grouped,
    pin_integer_closed_form,
    pin_unit_scales_matmul,
    pin_constant_operands,
    pin_grouped_is_per_group_dense,
    pin_masked_rows,
    pin_contiguous_poisoned_padding,
    pin_sampled_matches_full,
    pin_exact_nopad,
    pin_nopad_layout_invariants,
    pin_e8m0_golden,
    pin_ue8m0_power_of_two_identity,
    pin_ue8m0_drops_mantissa,
    pin_exact_k_grouped,
    pin_k_grouped_invariants,
    pin_e2m1_golden,
    pin_fp4_element_positions,
    pin_exact_fp8_fp4,
    pin_fp4_matches_fp8_on_shared_values,
    pin_contiguous_block_rule,
    pin_sampled_functions_match_full,
]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin_holds(pin):
    pin(O)


# ---------------------------------------------------------------------------
# Planted mistakes: each must break at least one pin
# ---------------------------------------------------------------------------

def _fresh_oracle():
    spec = importlib.util.spec_from_file_location("dg_oracle_mutant", ORACLE_PATH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _mut_lhs_scale_first_row(mod):
    orig = mod.dequant_lhs

    def f(a_codes, sfa):
        s = np.repeat(np.asarray(sfa)[:, :1], sfa.shape[1], axis=1)
        return orig(a_codes, s)
    mod.dequant_lhs = f


def _mut_rhs_scale_transposed(mod):
    def f(b_codes, sfb, rows=None):
        b_codes = np.asarray(b_codes, np.uint8) if rows is None else np.asarray(b_codes, np.uint8)[rows]
        n, k = b_codes.shape
        v = mod.e4m3_decode_table()[b_codes]
        s = np.asarray(sfb, np.float64)
        # reads sfb[kb][nb] instead of sfb[nb][kb] (wraps when the shape is not square)
        idx_n = np.arange(n) // 128
        idx_k = np.arange(k) // 128
        flat = s.reshape(-1)
        scale = flat[(idx_k[None, :] * s.shape[1] + idx_n[:, None]) % flat.size]
        return v * scale
    mod.dequant_rhs = f


def _mut_fnuz(mod):
    def table():
        t = np.empty(256)
        for c in range(256):
            s = -1.0 if c >> 7 else 1.0
            e, f = (c >> 3) & 15, c & 7
            t[c] = s * ((f / 8) * 2.0 ** -7 if e == 0 else (1 + f / 8) * 2.0 ** (e - 8))
        t[0x80] = np.nan
        return t
    mod.e4m3_decode_table = table


def _mut_truncate(mod):
    def bits(x):
        y = np.asarray(x, np.float64).astype(np.float32)
        return (y.view(np.uint32) >> 16).astype(np.uint16)
    mod.bf16_bits = bits


def _mut_double_round(mod):
    orig = mod.bf16_bits

    def bits(x):
        return orig(np.asarray(x, np.float64).astype(np.float32).astype(np.float64))
    mod.bf16_bits = bits


def _mut_drop_last_kblock(mod):
    orig = mod.dequant_lhs

    def f(a_codes, sfa):
        r = orig(a_codes, sfa)
        r[:, -128:] = 0.0
        return r
    mod.dequant_lhs = f


def _mut_no_sign(mod):
    orig = mod.e4m3_decode_table

    def table():
        return np.abs(orig())
    mod.e4m3_decode_table = table


def _mut_padding_written(mod):
    orig = mod.m_grouped_fp8_gemm_nt_contiguous

    def f(a_codes, sfa, b_codes, sfb, layout, d_init):
        lay = np.where(np.asarray(layout) < 0, 0, layout)
        return orig(a_codes, sfa, b_codes, sfb, lay, d_init)
    mod.m_grouped_fp8_gemm_nt_contiguous = f


def _mut_masked_off_by_one(mod):
    orig = mod.m_grouped_fp8_gemm_nt_masked

    def f(a_codes, sfa, b_codes, sfb, masked_m, d_init):
        return orig(a_codes, sfa, b_codes, sfb, np.asarray(masked_m) + 1, d_init)
    mod.m_grouped_fp8_gemm_nt_masked = f


def _mut_lhs_scale_by_k_only(mod):
    # applies sfa[kb][kb] (diagonal) instead of sfa[kb][m]
    def f(a_codes, sfa):
        m, k = a_codes.shape
        v = mod.e4m3_decode_table()[np.asarray(a_codes, np.uint8)]
        kb = np.arange(k) // 128
        s = np.asarray(sfa, np.float64)[kb, kb % sfa.shape[1]]
        return v * s[None, :]
    mod.dequant_lhs = f


def _mut_nopad_groups_restart(mod):
    # every group starts at row 0 (offsets dropped)
    def f(group_rows, m_rows):
        return [(0, min(max(int(c), 0), m_rows)) for c in np.asarray(group_rows)]
    mod.nopad_row_ranges = f


def _mut_nopad_negative_counts(mod):
    # negative counts move the next group's start backwards
    def f(group_rows, m_rows):
        out, s = [], 0
        for c in np.asarray(group_rows, np.int64):
            first = min(max(s, 0), m_rows)
            out.append((first, min(max(first + int(c), first), m_rows)))
            s += int(c)
        return out
    mod.nopad_row_ranges = f


def _mut_nopad_last_group_to_end(mod):
    # the last group also takes the rows no group owns
    orig = mod.nopad_row_ranges

    def f(group_rows, m_rows):
        r = orig(group_rows, m_rows)
        if r:
            r[-1] = (r[-1][0], m_rows)
        return r
    mod.nopad_row_ranges = f


def _mut_e8m0_rounds_up(mod):
    # the next power of two at or above the scale instead of its exponent field
    def f(scales):
        x = np.asarray(scales, np.float64)
        return np.ldexp(1.0, np.ceil(np.log2(np.abs(x))).astype(np.int64))
    mod.e8m0_value = f


def _mut_e8m0_bias_128(mod):
    orig = mod.e8m0_value

    def f(scales):
        return orig(scales) / 2.0
    mod.e8m0_value = f


def _mut_e8m0_keeps_mantissa(mod):
    def f(scales):
        return np.asarray(scales, np.float64)
    mod.e8m0_value = f


def _mut_k_grouped_restart(mod):
    # every group reads K from position 0
    def f(ks):
        return [(0, int(x)) for x in ks]
    mod.k_grouped_ranges = f


def _mut_k_grouped_rhs_block_scales(mod):
    # RHS scale of the 128-row block's first row instead of the row's own
    orig = mod._k_group_operands

    def f(a_codes, sfa, b_codes, sfb, k0, k1):
        sfb2 = np.repeat(np.asarray(sfb)[:, ::128], 128, axis=1)[:, :np.asarray(sfb).shape[1]]
        return orig(a_codes, sfa, b_codes, sfb2, k0, k1)
    mod._k_group_operands = f


def _mut_k_grouped_drops_c(mod):
    orig = mod.k_grouped_fp8_gemm_nt_contiguous

    def f(a_codes, sfa, b_codes, sfb, ks, c_init=None):
        return orig(a_codes, sfa, b_codes, sfb, ks, None)
    mod.k_grouped_fp8_gemm_nt_contiguous = f


def _mut_e2m1_nibbles_swapped(mod):
    def f(packed):
        packed = np.asarray(packed, dtype=np.uint8)
        out = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.uint8)
        out[..., 0::2] = packed >> 4
        out[..., 1::2] = packed & 0x0F
        return out
    mod.unpack_e2m1 = f


def _mut_fp4_scale_per_128(mod):
    # the RHS scale of the first 32-K block of each 128-K block for all four
    orig = mod.dequant_rhs_e2m1

    def f(b_packed, sfb):
        s = np.array(sfb, copy=True)
        s[:] = np.repeat(s[0::4], 4, axis=0)[:s.shape[0]]
        return orig(b_packed, s)
    mod.dequant_rhs_e2m1 = f


def _mut_e2m1_bias_0(mod):
    def table():
        return np.array([mod.e2m1_value(c) * (2.0 if (c >> 1) & 3 else 1.0) for c in range(16)])
    mod.e2m1_decode_table = table


def _mut_contiguous_any_valid_id(mod):
    # every row with an id in [0, G) is computed, whatever its block's id
    def f(layout, num_groups):
        lay = np.asarray(layout, np.int64)
        return np.where((lay >= 0) & (lay < num_groups), lay, -1)
    mod.contiguous_row_groups = f


def _mut_at_contiguous_wrong_group(mod):
    # the sampled contiguous reference uses the next group's B
    orig = mod.contiguous_f64_at

    def f(a_codes, sfa, b_codes, sfb, layout, rows, cols, abs_sum=False):
        return orig(a_codes, sfa, np.roll(b_codes, 1, axis=0), np.roll(sfb, 1, axis=0), layout, rows, cols, abs_sum)
    mod.contiguous_f64_at = f


def _mut_at_masked_off_by_one(mod):
    orig = mod.masked_f64_at

    def f(a_codes, sfa, b_codes, sfb, masked_m, group, rows, cols, abs_sum=False):
        return orig(a_codes, sfa, b_codes, sfb, np.asarray(masked_m) + 1, group, rows, cols, abs_sum)
    mod.masked_f64_at = f


def _mut_at_nopad_shifted(mod):
    # the sampled no-padding reference starts every group one row late
    orig = mod.nopad_f64_at

    def f(a_codes, sfa, b_codes, sfb, group_rows, rows, cols, abs_sum=False):
        return orig(a_codes, sfa, b_codes, sfb, group_rows, np.asarray(rows) - 1, cols, abs_sum)
    mod.nopad_f64_at = f


def _mut_at_k_grouped_rhs_block_scales(mod):
    # the sampled K-grouped reference reads the RHS scale of each 128-row block's first row
    orig = mod.k_grouped_f64_at

    def f(a_codes, sfa, b_codes, sfb, ks, group, rows, cols, c_init=None, abs_sum=False):
        s = np.asarray(sfb)
        s2 = np.repeat(s[:, ::128], 128, axis=1)[:, :s.shape[1]]
        return orig(a_codes, sfa, b_codes, s2, ks, group, rows, cols, c_init, abs_sum)
    mod.k_grouped_f64_at = f


def _mut_at_fp4_nibbles_swapped(mod):
    orig = mod.fp8_fp4_f64_at

    def f(a_codes, sfa, b_packed_g, sfb_g, rows, cols, abs_sum=False):
        p = np.asarray(b_packed_g, np.uint8)
        return orig(a_codes, sfa, ((p >> 4) | (p << 4)).astype(np.uint8), sfb_g, rows, cols, abs_sum)
    mod.fp8_fp4_f64_at = f


def _mut_at_magnitude_of_sum(mod):
    # |sum| instead of the sum of magnitudes for the error bound
    orig = mod._rows_cols_f64

    def f(a_codes, sfa, b_codes, sfb, rows, cols, abs_sum=False):
        v = orig(a_codes, sfa, b_codes, sfb, rows, cols, False)
        return (v, np.abs(v)) if abs_sum else v
    mod._rows_cols_f64 = f


MUTANTS = [
    _mut_lhs_scale_first_row,
    _mut_rhs_scale_transposed,
    _mut_fnuz,
    _mut_truncate,
    _mut_double_round,
    _mut_drop_last_kblock,
    _mut_no_sign,
    _mut_padding_written,
    _mut_masked_off_by_one,
    _mut_lhs_scale_by_k_only,
    _mut_nopad_groups_restart,
    _mut_nopad_negative_counts,
    _mut_nopad_last_group_to_end,
    _mut_e8m0_rounds_up,
    _mut_e8m0_bias_128,
    _mut_e8m0_keeps_mantissa,
    _mut_k_grouped_restart,
    _mut_k_grouped_rhs_block_scales,
    _mut_k_grouped_drops_c,
    _mut_e2m1_nibbles_swapped,
    _mut_fp4_scale_per_128,
    _mut_e2m1_bias_0,
    _mut_contiguous_any_valid_id,
    _mut_at_contiguous_wrong_group,
    _mut_at_masked_off_by_one,
    _mut_at_nopad_shifted,
    _mut_at_k_grouped_rhs_block_scales,
    _mut_at_fp4_nibbles_swapped,
    _mut_at_magnitude_of_sum,
]


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m.__name__ for m in MUTANTS])
def test_planted_mistakes_are_caught(mutant):
    mod = _fresh_oracle()
    mutant(mod)
    failures = 0
    for pin in PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError):
            failures += 1
    assert failures >= 1, f"no pin caught {mutant.__name__}"
