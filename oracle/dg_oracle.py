"""Plain CPU oracle for the fine-grained-scaled FP8 NT GEMM and its M-grouped
variants.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module. The GPU library never calls it, and
it shares no code with the GPU library: it reads raw bytes (uint8 FP8 codes,
float32 scales, int32 layouts, uint16 BF16 bit patterns) as numpy arrays.

What it computes is the plain definition of the operation, in float64:

    dec(q)     value of the OCP E4M3 byte q
    Ahat[m,k]  = dec(A[m,k]) * sfa[k // 128][m]          (LHS: one scale per 1x128)
    Bhat[n,k]  = dec(B[n,k]) * sfb[n // 128][k // 128]   (RHS: one scale per 128x128)
    D[m,n]     = bf16_rne( sum_k Ahat[m,k] * Bhat[n,k] )

Sources on the pages:
  * "DeepGEMM for PPU" README, "Interfaces > Notices": kernels are NT only
    (LHS row-major, RHS stored transposed, i.e. [N, K]); the LHS scaling
    factors are stored transposed (M-major) with an aligned leading dimension.
  * same page, "Normal dense GEMMs (non-grouped)": the dense FP8 x FP8 -> BF16
    NT GEMM.
  * same page, "Grouped GEMMs (contiguous layout)": only M is grouped, N and K
    are shared by every group; expert segments are concatenated along M and
    each is aligned to the M block size.
  * same page, "Grouped GEMMs (masked layout)": a per-group count of valid
    rows; only the valid part of each group is computed.
  * same page, "Grouped GEMMs (nopad layout)": the groups' rows are
    concatenated without alignment padding, and a tensor of per-group token
    counts says where each group's rows are.
  * "DeepGEMM Compatibility Wrapper (deep-gemm)" page, "0.2.7 Compatibility
    Additions" and "Contiguous Grouped GEMM Alignment": scale recipe
    (1, 128, 128) and the 128-row segment alignment; UE8M0 scale casting and
    the packed UE8M0 scale conversion (the *_ue8m0 variants below); the
    contiguous K-grouped FP8 NT GEMM with host K sizes, recipe (1, 1, 128)
    and a float32 C (k_grouped_fp8_gemm_nt_contiguous below); the FP8 x FP4
    grouped GEMMs with FP8 E4M3 A, packed E2M1 B, LHS scales per 1x128 and
    RHS scales per 1x32 (the *_fp8_fp4_* functions below).

The 128-K block structure of the scales does not change the definition: the
per-block sums scaled and added are algebraically the plain sum over the
dequantised operands, which is what is written here.

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):
  * FP8 flavour: OCP E4M3 (bias 7, max 448, codes 0x7F/0xFF are NaN, no inf).
  * BF16 rounding: round to nearest, ties to even, applied once to the exact
    float64 sum (no intermediate rounding to float32).
  * contiguous layout: the layout is a sequence of 128-row blocks, each
    holding one group's rows (segments are aligned to the M block). A
    block belongs to the group named by its first row's id; row m is
    computed, for group L[m], when L[m] is that id and lies in [0, G). Any
    other row (id -1 for padding, an id outside [0, G), or an id that
    differs from its block's) is left untouched. For layouts whose segments
    really are 128-row aligned this is simply "row m belongs to L[m] when
    0 <= L[m] < G".
  * masked layout: masked_m[g] is clamped to [0, max_m]; rows at or beyond it
    are left untouched.
  * no-padding layout: the count tensor holds one int32 row count per group;
    group 0's rows come first, then group 1's, and so on from row 0 of A and
    D. A negative count counts as zero; rows at or past M do not exist, so a
    group reaching past them is cut off there. Rows no group owns are left
    untouched.
  * UE8M0 variants: the scales are powers of two (a UE8M0 cast made at
    quantisation); a float32 scale is taken as 2^(e - 127), e being its
    biased exponent field, as the packed UE8M0 conversion reads it (sign and
    mantissa bits dropped; e = 255 is NaN). The GEMM is then the same
    definition with those scale values.
  * K-grouped GEMM: the groups split K into consecutive ranges in the order
    given; group g's output is D[g] = C[g] + (A restricted to its K range)
    times (B restricted to it) transposed, with one float32 scale per row
    and 128-wide K block for both operands (stored transposed like the LHS
    scales); C absent means zero; the result is float32 and is compared
    unrounded.
  * FP8 x FP4 GEMMs: B holds OCP E2M1 values packed two per byte along K,
    element 2j in the low nibble of byte j; its scales sfb[g][k // 32][n]
    (one per row and 32-wide K block, stored transposed); all scales are read
    as UE8M0 like the *_ue8m0 variants.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "BLOCK_K",
    "e4m3_value",
    "e4m3_decode_table",
    "bf16_round",
    "bf16_bits",
    "bf16_bits_to_f64",
    "dequant_lhs",
    "dequant_rhs",
    "gemm_nt_f64",
    "gemm_nt_exact",
    "dense_f64_at",
    "fp8_gemm_nt",
    "contiguous_row_groups",
    "m_grouped_fp8_gemm_nt_contiguous",
    "m_grouped_fp8_gemm_nt_masked",
    "nopad_row_ranges",
    "m_grouped_fp8_gemm_nt_nopad",
    "contiguous_f64_at",
    "masked_f64_at",
    "nopad_f64_at",
    "e8m0_value",
    "fp8_gemm_nt_ue8m0",
    "m_grouped_fp8_gemm_nt_contiguous_ue8m0",
    "m_grouped_fp8_gemm_nt_masked_ue8m0",
    "m_grouped_fp8_gemm_nt_nopad_ue8m0",
    "k_grouped_ranges",
    "k_grouped_fp8_gemm_nt_contiguous",
    "k_grouped_f64_at",
    "k_grouped_fp8_gemm_nt_contiguous_ue8m0",
    "e2m1_value",
    "e2m1_decode_table",
    "unpack_e2m1",
    "dequant_rhs_e2m1",
    "m_grouped_fp8_fp4_gemm_nt_contiguous",
    "m_grouped_fp8_fp4_gemm_nt_masked",
    "fp8_fp4_f64_at",
]

# Scale granularity along K for both operands: recipe (1, 128, 128).
BLOCK_K = 128


# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------

def e4m3_value(code: int) -> float:
    """Value of one OCP E4M3 byte (OCP 8-bit floating point specification).

    Layout: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0.
    Exponent field 0 encodes subnormals (f/8 * 2^-6); exponent field 15 with
    mantissa 7 is NaN; there is no infinity, so 0x7E (= 448) is the largest
    finite value.
    """
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp_field = (code >> 3) & 0xF
    man_field = code & 0x7
    if exp_field == 0xF and man_field == 0x7:
        return float("nan")
    if exp_field == 0:
        return sign * (man_field / 8.0) * 2.0 ** -6
    return sign * (1.0 + man_field / 8.0) * 2.0 ** (exp_field - 7)


def e4m3_decode_table() -> np.ndarray:
    """All 256 E4M3 values as float64, indexed by the byte."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 has 8 significant bits and float32's exponent range: a finite
    value with binary exponent E (|x| in [2^E, 2^(E+1))) is a multiple of
    2^(E-7); below 2^-126 the spacing stays 2^-133 (subnormals). A result of
    magnitude 2^128 or more is out of range and becomes infinity. The result
    is returned as float64 holding the exact bfloat16 value.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    finite = np.isfinite(x)
    ax = np.abs(x[finite])
    _, e = np.frexp(ax)                      # ax = mant * 2^e, mant in [0.5, 1)
    exponent = np.maximum(e - 1, -126)       # E with the subnormal floor
    quantum = np.ldexp(1.0, exponent - 7)
    y = np.rint(ax / quantum) * quantum      # rint rounds half to even
    y = np.where(y >= 2.0 ** 128, np.inf, y)
    out[finite] = np.copysign(y, x[finite])
    return out


def bf16_bits(x) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of float64 values, rounded to nearest even.

    The bfloat16 encoding is the upper half of the float32 encoding of the same
    value; every bfloat16 value is exact in float32. NaN maps to 0x7FC0.
    """
    y = bf16_round(x).astype(np.float32)
    bits = (y.view(np.uint32) >> 16).astype(np.uint16)
    bits[np.isnan(y)] = 0x7FC0
    return bits


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Values of bfloat16 bit patterns, as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Dequantisation
# ---------------------------------------------------------------------------

def dequant_lhs(a_codes: np.ndarray, sfa: np.ndarray) -> np.ndarray:
    """Ahat[m,k] = dec(A[m,k]) * sfa[k // 128][m].

    a_codes: uint8 [M, K] (row-major, K contiguous).
    sfa:     float32 [K/128, ld] with ld >= M: the LHS scales stored
             transposed (M-major) with an aligned leading dimension.
    """
    a_codes = np.asarray(a_codes, dtype=np.uint8)
    m_rows, k = a_codes.shape
    assert k % BLOCK_K == 0
    assert sfa.shape[0] == k // BLOCK_K and sfa.shape[1] >= m_rows
    values = e4m3_decode_table()[a_codes]                       # [M, K]
    scale = np.asarray(sfa, dtype=np.float64)[:, :m_rows].T     # [M, K/128]
    return values * np.repeat(scale, BLOCK_K, axis=1)


def dequant_rhs(b_codes: np.ndarray, sfb: np.ndarray, rows=None) -> np.ndarray:
    """Bhat[n,k] = dec(B[n,k]) * sfb[n // 128][k // 128].

    b_codes: uint8 [N, K] (the transposed RHS of the NT product).
    sfb:     float32 [ceil(N/128), K/128].
    rows:    None for all N rows, else the row indices n to dequantise (the
             result then has one row per index, in that order).
    """
    b_codes = np.asarray(b_codes, dtype=np.uint8)
    n, k = b_codes.shape
    assert k % BLOCK_K == 0
    assert sfb.shape == ((n + BLOCK_K - 1) // BLOCK_K, k // BLOCK_K)
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    values = e4m3_decode_table()[b_codes[rows]]                 # [len(rows), K]
    scale = np.asarray(sfb, dtype=np.float64)[rows // BLOCK_K]  # [len(rows), K/128]
    return values * np.repeat(scale, BLOCK_K, axis=1)


def gemm_nt_exact(a_codes, sfa, b_codes, sfb) -> list:
    """The dense result in exact rational arithmetic, element by element:
    sum_k dec(A[m,k]) sfa[k // 128][m] dec(B[n,k]) sfb[n // 128][k // 128]
    as a list of lists of fractions.Fraction (every E4M3 value and float32
    scale is a dyadic rational, so nothing is rounded). Brute force for tiny
    shapes only."""
    from fractions import Fraction
    a_codes = np.asarray(a_codes, dtype=np.uint8)
    b_codes = np.asarray(b_codes, dtype=np.uint8)
    m_rows, k = a_codes.shape
    n = b_codes.shape[0]
    dec = [Fraction(e4m3_value(c)) if c & 0x7F != 0x7F else None for c in range(256)]
    ahat = [[dec[a_codes[i, kk]] * Fraction(float(sfa[kk // BLOCK_K][i])) for kk in range(k)] for i in range(m_rows)]
    bhat = [[dec[b_codes[j, kk]] * Fraction(float(sfb[j // BLOCK_K][kk // BLOCK_K])) for kk in range(k)]
            for j in range(n)]
    return [[sum((x * y for x, y in zip(ahat[i], bhat[j])), Fraction(0)) for j in range(n)] for i in range(m_rows)]


def gemm_nt_f64(a_codes, sfa, b_codes, sfb) -> np.ndarray:
    """Unrounded float64 result sum_k Ahat[m,k] * Bhat[n,k], shape [M, N]."""
    ahat = dequant_lhs(a_codes, sfa)
    bhat = dequant_rhs(b_codes, sfb)
    return ahat @ bhat.T


# ---------------------------------------------------------------------------
# The three operations (output: uint16 BF16 bit patterns)
# ---------------------------------------------------------------------------

def fp8_gemm_nt(a_codes, sfa, b_codes, sfb, d_init=None) -> np.ndarray:
    """Dense FP8 NT GEMM: D[m,n] = bf16(sum_k Ahat[m,k] Bhat[n,k]) for all rows.

    d_init is accepted for a uniform interface; every element is written.
    """
    d = bf16_bits(gemm_nt_f64(a_codes, sfa, b_codes, sfb))
    if d_init is not None:
        assert d_init.shape == d.shape
    return d


def contiguous_row_groups(layout, num_groups: int) -> np.ndarray:
    """Group of each row of the contiguous layout, -1 for rows not computed.

    The rows form blocks of 128 (the M-block alignment of the segments); a
    block belongs to the group named by the id of its first row. Row m gets
    group L[m] when L[m] equals its block's id and 0 <= L[m] < G, else -1.
    M must be a multiple of 128.
    """
    layout = np.asarray(layout, dtype=np.int64)
    assert layout.size % BLOCK_K == 0, "contiguous layouts hold whole 128-row blocks"
    block_id = np.repeat(layout[::BLOCK_K], BLOCK_K)
    ok = (layout == block_id) & (layout >= 0) & (layout < num_groups)
    return np.where(ok, layout, -1)


def m_grouped_fp8_gemm_nt_contiguous(a_codes, sfa, b_codes, sfb, layout, d_init) -> np.ndarray:
    """M-grouped GEMM, contiguous layout.

    a_codes [M, K], sfa [K/128, ld], b_codes [G, N, K], sfb [G, N/128, K/128],
    layout int32 [M] (group of each row, -1 for padding), d_init uint16
    [M, N] (prior contents of D). Row m of D becomes
    bf16(Ahat[m] . Bhat_g^T) for g = contiguous_row_groups(layout, G)[m] >= 0
    and is copied from d_init otherwise.
    """
    num_groups = b_codes.shape[0]
    owner = contiguous_row_groups(layout, num_groups)
    d = np.array(d_init, dtype=np.uint16, copy=True)
    for g in range(num_groups):
        rows = np.nonzero(owner == g)[0]
        if rows.size == 0:
            continue
        ahat = dequant_lhs(a_codes[rows], sfa[:, rows])
        bhat = dequant_rhs(b_codes[g], sfb[g])
        d[rows] = bf16_bits(ahat @ bhat.T)
    return d


def m_grouped_fp8_gemm_nt_masked(a_codes, sfa, b_codes, sfb, masked_m, d_init) -> np.ndarray:
    """M-grouped GEMM, masked layout.

    a_codes [G, max_m, K], sfa [G, K/128, ld], b_codes [G, N, K],
    sfb [G, N/128, K/128], masked_m int32 [G], d_init uint16 [G, max_m, N].
    For each group g, rows m < clamp(masked_m[g], 0, max_m) of D[g] become
    bf16(Ahat_g[m] . Bhat_g^T); all other rows keep d_init's contents.
    """
    num_groups, max_m, _ = a_codes.shape
    d = np.array(d_init, dtype=np.uint16, copy=True)
    for g in range(num_groups):
        valid = int(min(max(int(masked_m[g]), 0), max_m))
        if valid == 0:
            continue
        ahat = dequant_lhs(a_codes[g, :valid], sfa[g])
        bhat = dequant_rhs(b_codes[g], sfb[g])
        d[g, :valid] = bf16_bits(ahat @ bhat.T)
    return d


def nopad_row_ranges(group_rows, m_rows: int) -> list:
    """[first, end) of each group's rows in the no-padding layout: the groups
    follow one another from row 0, a negative count counts as zero, and
    nothing lies at or past row m_rows."""
    ranges, start = [], 0
    for c in np.asarray(group_rows, dtype=np.int64):
        first = min(start, m_rows)
        end = min(start + max(int(c), 0), m_rows)
        ranges.append((first, end))
        start += max(int(c), 0)
    return ranges


def m_grouped_fp8_gemm_nt_nopad(a_codes, sfa, b_codes, sfb, group_rows, d_init) -> np.ndarray:
    """M-grouped GEMM, no-padding layout.

    a_codes [M, K], sfa [K/128, ld], b_codes [G, N, K], sfb [G, N/128, K/128],
    group_rows int32 [G] (rows of each group), d_init uint16 [M, N].
    Rows [first_g, end_g) of D (nopad_row_ranges) become
    bf16(Ahat[r] . Bhat_g^T); all other rows keep d_init's contents.
    """
    m_rows = a_codes.shape[0]
    d = np.array(d_init, dtype=np.uint16, copy=True)
    for g, (first, end) in enumerate(nopad_row_ranges(group_rows, m_rows)):
        if end == first:
            continue
        ahat = dequant_lhs(a_codes[first:end], sfa[:, first:end])
        bhat = dequant_rhs(b_codes[g], sfb[g])
        d[first:end] = bf16_bits(ahat @ bhat.T)
    return d


# ---------------------------------------------------------------------------
# Sampled evaluation for full-size checks: a subset of rows and columns.
# ---------------------------------------------------------------------------

def _rows_cols_f64(a_codes, sfa, b_codes, sfb, rows, cols, abs_sum=False):
    """sum_k Ahat[r,k] Bhat[c,k] for r in rows, c in cols (one group), from
    dequant_lhs and dequant_rhs on those rows; with abs_sum also
    sum_k |Ahat[r,k] Bhat[c,k]| (for error bounds)."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    ahat = dequant_lhs(np.asarray(a_codes)[rows], np.asarray(sfa)[:, rows])
    bhat = dequant_rhs(b_codes, sfb, cols)
    val = ahat @ bhat.T
    return (val, np.abs(ahat) @ np.abs(bhat).T) if abs_sum else val


def _nan_like(rows, cols, abs_sum):
    out = np.full((len(rows), len(cols)), np.nan)
    return (out, out.copy()) if abs_sum else out


def _put(out, sel, val, abs_sum):
    if abs_sum:
        out[0][sel], out[1][sel] = val
    else:
        out[sel] = val


def dense_f64_at(a_codes, sfa, b_codes, sfb, rows, cols, abs_sum=False):
    """Unrounded dense result at rows x cols (with abs_sum: (value, sum of
    the products' magnitudes))."""
    return _rows_cols_f64(a_codes, sfa, b_codes, sfb, rows, cols, abs_sum)


def contiguous_f64_at(a_codes, sfa, b_codes, sfb, layout, rows, cols, abs_sum=False):
    """Unrounded contiguous-layout result at rows x cols; NaN where a row is
    not computed (contiguous_row_groups gives it no group)."""
    owner = contiguous_row_groups(layout, b_codes.shape[0])
    rows = np.asarray(rows, dtype=np.int64)
    out = _nan_like(rows, cols, abs_sum)
    for g in range(b_codes.shape[0]):
        sel = np.nonzero(owner[rows] == g)[0]
        if sel.size:
            _put(out, sel, _rows_cols_f64(a_codes, sfa, b_codes[g], sfb[g], rows[sel], cols, abs_sum), abs_sum)
    return out


def masked_f64_at(a_codes, sfa, b_codes, sfb, masked_m, group, rows, cols, abs_sum=False):
    """Unrounded masked-layout result of one group at rows x cols; NaN for
    rows at or beyond the group's clamped valid count."""
    max_m = a_codes.shape[1]
    valid = int(min(max(int(masked_m[group]), 0), max_m))
    rows = np.asarray(rows, dtype=np.int64)
    out = _nan_like(rows, cols, abs_sum)
    sel = np.nonzero(rows < valid)[0]
    if sel.size:
        _put(out, sel, _rows_cols_f64(a_codes[group], sfa[group], b_codes[group], sfb[group], rows[sel], cols,
                                      abs_sum), abs_sum)
    return out


def nopad_f64_at(a_codes, sfa, b_codes, sfb, group_rows, rows, cols, abs_sum=False):
    """Unrounded no-padding-layout result at rows x cols; NaN for rows that
    no group owns."""
    rows = np.asarray(rows, dtype=np.int64)
    out = _nan_like(rows, cols, abs_sum)
    for g, (first, end) in enumerate(nopad_row_ranges(group_rows, a_codes.shape[0])):
        sel = np.nonzero((rows >= first) & (rows < end))[0]
        if sel.size:
            _put(out, sel, _rows_cols_f64(a_codes, sfa, b_codes[g], sfb[g], rows[sel], cols, abs_sum), abs_sum)
    return out


# ---------------------------------------------------------------------------
# Power-of-two (UE8M0) scales
# ---------------------------------------------------------------------------

def e8m0_value(scales) -> np.ndarray:
    """float64 value of each float32 scale read as an E8M0 code: the biased
    exponent field e (bits 30..23 of the float32 encoding) stands for
    2^(e - 127), and e = 255 for NaN (OCP Microscaling formats, E8M0). For a
    positive normal power of two this is the scale itself."""
    bits = np.ascontiguousarray(scales, dtype=np.float32).view(np.uint32)
    e = ((bits >> 23) & 0xFF).astype(np.int64)
    out = np.ldexp(1.0, e - 127)
    out[e == 255] = np.nan
    return out


def fp8_gemm_nt_ue8m0(a_codes, sfa, b_codes, sfb, d_init=None) -> np.ndarray:
    """Dense GEMM with every scale taken as its E8M0 value."""
    return fp8_gemm_nt(a_codes, e8m0_value(sfa), b_codes, e8m0_value(sfb), d_init)


def m_grouped_fp8_gemm_nt_contiguous_ue8m0(a_codes, sfa, b_codes, sfb, layout, d_init) -> np.ndarray:
    return m_grouped_fp8_gemm_nt_contiguous(a_codes, e8m0_value(sfa), b_codes, e8m0_value(sfb), layout, d_init)


def m_grouped_fp8_gemm_nt_masked_ue8m0(a_codes, sfa, b_codes, sfb, masked_m, d_init) -> np.ndarray:
    return m_grouped_fp8_gemm_nt_masked(a_codes, e8m0_value(sfa), b_codes, e8m0_value(sfb), masked_m, d_init)


def m_grouped_fp8_gemm_nt_nopad_ue8m0(a_codes, sfa, b_codes, sfb, group_rows, d_init) -> np.ndarray:
    return m_grouped_fp8_gemm_nt_nopad(a_codes, e8m0_value(sfa), b_codes, e8m0_value(sfb), group_rows, d_init)


# ---------------------------------------------------------------------------
# K-grouped GEMM (weight-gradient shape), recipe (1, 1, 128)
# ---------------------------------------------------------------------------

def k_grouped_ranges(ks) -> list:
    """[first, end) of each group's K positions: consecutive, in order."""
    out, start = [], 0
    for x in ks:
        out.append((start, start + int(x)))
        start += int(x)
    return out


def _k_group_operands(a_codes, sfa, b_codes, sfb, k0, k1):
    """Dequantised A[:, k0:k1] and B[:, k0:k1]: one scale per row and
    128-wide K block for both, sf[k // 128][row]."""
    kb0, kb1 = k0 // BLOCK_K, k1 // BLOCK_K
    ahat = dequant_lhs(a_codes[:, k0:k1], sfa[kb0:kb1])
    bhat = dequant_lhs(b_codes[:, k0:k1], sfb[kb0:kb1])
    return ahat, bhat


def k_grouped_fp8_gemm_nt_contiguous(a_codes, sfa, b_codes, sfb, ks, c_init=None) -> np.ndarray:
    """K-grouped FP8 NT GEMM, float64 result [G, M, N].

    a_codes [M, K], sfa [K/128, ld >= M], b_codes [N, K], sfb [K/128, ld >= N],
    ks: the groups' K sizes (multiples of 128, summing to K), c_init None or
    [G, M, N]. D[g] = c_init[g] (or 0) + sum_{k in group g} Ahat[:, k] Bhat[:, k]^T.
    """
    m_rows, k = a_codes.shape
    n = b_codes.shape[0]
    ranges = k_grouped_ranges(ks)
    assert ranges[-1][1] == k and all((e - f) % BLOCK_K == 0 for f, e in ranges)
    d = np.zeros((len(ranges), m_rows, n)) if c_init is None else np.array(c_init, dtype=np.float64, copy=True)
    for g, (k0, k1) in enumerate(ranges):
        if k1 > k0:
            ahat, bhat = _k_group_operands(a_codes, sfa, b_codes, sfb, k0, k1)
            d[g] += ahat @ bhat.T
    return d


def k_grouped_fp8_gemm_nt_contiguous_ue8m0(a_codes, sfa, b_codes, sfb, ks, c_init=None) -> np.ndarray:
    """The K-grouped GEMM with every scale taken as its E8M0 value."""
    return k_grouped_fp8_gemm_nt_contiguous(a_codes, e8m0_value(sfa), b_codes, e8m0_value(sfb), ks, c_init)


def k_grouped_f64_at(a_codes, sfa, b_codes, sfb, ks, group, rows, cols, c_init=None, abs_sum=False):
    """Group `group`'s result at rows x cols (float64), from _k_group_operands
    on those rows of A and B; with abs_sum also sum_k |Ahat[r, k] Bhat[c, k]|
    + |C| there (for error bounds)."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    k0, k1 = k_grouped_ranges(ks)[group]
    c = np.zeros((rows.size, cols.size)) if c_init is None else np.asarray(c_init, np.float64)[group][np.ix_(rows, cols)]
    if k1 == k0:
        val, mag = c.copy(), np.abs(c)
    else:
        ahat, bhat = _k_group_operands(np.asarray(a_codes)[rows], np.asarray(sfa)[:, rows],
                                       np.asarray(b_codes)[cols], np.asarray(sfb)[:, cols], k0, k1)
        val = c + ahat @ bhat.T
        mag = np.abs(c) + np.abs(ahat) @ np.abs(bhat).T
    return (val, mag) if abs_sum else val


# ---------------------------------------------------------------------------
# FP8 x FP4 (W4A8): packed E2M1 B with one scale per row and 32-wide K block
# ---------------------------------------------------------------------------

FP4_BLOCK_K = 32


def e2m1_value(code: int) -> float:
    """Value of one OCP E2M1 code (OCP Microscaling formats, FP4 E2M1): sign
    bit 3, exponent bits 2..1 with bias 1, mantissa bit 0; exponent field 0
    encodes subnormals (m/2 * 2^0). No infinity or NaN: 6 is the largest."""
    sign = -1.0 if (code >> 3) & 1 else 1.0
    e = (code >> 1) & 0x3
    mant = code & 0x1
    if e == 0:
        return sign * mant * 0.5
    return sign * (1.0 + mant / 2.0) * 2.0 ** (e - 1)


def e2m1_decode_table() -> np.ndarray:
    return np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def unpack_e2m1(packed) -> np.ndarray:
    """E2M1 codes [..., 2 * L] from bytes [..., L]: element 2j is the low
    nibble of byte j, element 2j + 1 its high nibble."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = packed & 0x0F
    out[..., 1::2] = packed >> 4
    return out


def dequant_rhs_e2m1(b_packed, sfb) -> np.ndarray:
    """Bhat[n,k] = e2m1(B[n,k]) * E8M0(sfb[k // 32][n]); b_packed [N, K/2]."""
    codes = unpack_e2m1(b_packed)
    n, k = codes.shape
    scale = e8m0_value(np.asarray(sfb)[:, :n]).T                 # [N, K/32]
    assert scale.shape[1] * FP4_BLOCK_K == k
    return e2m1_decode_table()[codes] * np.repeat(scale, FP4_BLOCK_K, axis=1)


def m_grouped_fp8_fp4_gemm_nt_contiguous(a_codes, sfa, b_packed, sfb, layout, d_init) -> np.ndarray:
    """Contiguous-layout FP8 x FP4 GEMM: as m_grouped_fp8_gemm_nt_contiguous
    with Bhat_g from dequant_rhs_e2m1 and every scale read as E8M0.
    b_packed [G, N, K/2], sfb [G, K/32, ld >= N]."""
    owner = contiguous_row_groups(layout, b_packed.shape[0])
    d = np.array(d_init, dtype=np.uint16, copy=True)
    sfa_v = e8m0_value(sfa)
    for g in range(b_packed.shape[0]):
        rows = np.nonzero(owner == g)[0]
        if rows.size == 0:
            continue
        ahat = dequant_lhs(a_codes[rows], sfa_v[:, rows])
        bhat = dequant_rhs_e2m1(b_packed[g], sfb[g])
        d[rows] = bf16_bits(ahat @ bhat.T)
    return d


def m_grouped_fp8_fp4_gemm_nt_masked(a_codes, sfa, b_packed, sfb, masked_m, d_init) -> np.ndarray:
    """Masked-layout FP8 x FP4 GEMM; a_codes [G, max_m, K], sfa [G, K/128, ld]."""
    num_groups, max_m, _ = a_codes.shape
    d = np.array(d_init, dtype=np.uint16, copy=True)
    for g in range(num_groups):
        valid = int(min(max(int(masked_m[g]), 0), max_m))
        if valid == 0:
            continue
        ahat = dequant_lhs(a_codes[g, :valid], e8m0_value(sfa[g]))
        bhat = dequant_rhs_e2m1(b_packed[g], sfb[g])
        d[g, :valid] = bf16_bits(ahat @ bhat.T)
    return d


def fp8_fp4_f64_at(a_codes, sfa, b_packed_g, sfb_g, rows, cols, abs_sum=False):
    """Unrounded FP8 x FP4 result of one group at rows x cols, from
    dequant_lhs (E8M0 LHS scales) and dequant_rhs_e2m1 on those rows:
    a_codes [M, K] and sfa [K/128, ld] of that group's rows,
    b_packed_g [N, K/2], sfb_g [K/32, ld]; with abs_sum also the sum of the
    products' magnitudes."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    ahat = dequant_lhs(np.asarray(a_codes)[rows], e8m0_value(np.asarray(sfa)[:, rows]))
    bhat = dequant_rhs_e2m1(np.asarray(b_packed_g)[cols], np.asarray(sfb_g)[:, cols])
    val = ahat @ bhat.T
    return (val, np.abs(ahat) @ np.abs(bhat).T) if abs_sum else val
