"""Pins for the oracle's number formats: OCP E4M3 decoding and BF16 rounding.

The oracle's E4M3 table is checked against the hand-written OCP table in
tests/golden and against torch's float8_e4m3fn conversion (a library routine
for the same format); its BF16 rounding against hand-derived tie/overflow/
subnormal cases and against torch's float32 -> bfloat16 conversion (round to
nearest even) on float32-exact inputs.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import dg_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line)
    return rows


def check_e4m3_golden(orc):
    table = orc.e4m3_decode_table()
    rows = _read_golden("e4m3_ocp_values.txt")
    assert len(rows) >= 20
    for row in rows:
        code_s, val_s = row.split()
        code = int(code_s, 16)
        if val_s == "nan":
            assert math.isnan(table[code])
            continue
        expected = float(Fraction(val_s.lstrip("-"))) * (-1.0 if val_s.startswith("-") else 1.0)
        assert table[code] == expected, (hex(code), table[code], expected)
        assert math.copysign(1.0, table[code]) == math.copysign(1.0, expected)


def test_e4m3_golden_table():
    check_e4m3_golden(O)


def test_e4m3_all_codes_match_torch():
    table = O.e4m3_decode_table()
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan_o = np.isnan(table)
    nan_r = np.isnan(ref)
    assert np.array_equal(nan_o, nan_r)
    assert nan_o.sum() == 2 and nan_o[0x7F] and nan_o[0xFF]
    assert np.array_equal(table[~nan_o], ref[~nan_r])
    assert np.array_equal(np.signbit(table[~nan_o]), np.signbit(ref[~nan_r]))


def test_e4m3_integers_exact():
    # every integer 0..16 has a code, which the integer-exact GEMM pins rely on
    table = O.e4m3_decode_table()
    finite = set(float(v) for v in table if np.isfinite(v))
    for i in range(17):
        assert float(i) in finite and float(-i) in finite


def check_bf16_golden(orc):
    rows = _read_golden("bf16_rne_cases.txt")
    assert len(rows) >= 15
    xs, expected = [], []
    for row in rows:
        expr, bits = row.rsplit(None, 1)
        xs.append(float(eval(expr, {"__builtins__": {}}, {})))  # dyadic literals only
        expected.append(int(bits, 16))
    got = orc.bf16_bits(np.array(xs))
    for x, e, g in zip(xs, expected, got):
        assert int(g) == e, (x, hex(e), hex(int(g)))


def test_bf16_golden_cases():
    check_bf16_golden(O)


def check_e8m0_golden(orc):
    rows = _read_golden("e8m0_scale_cases.txt")
    assert len(rows) >= 12
    for row in rows:
        bits_s, val_s = row.split("#")[0].split()
        bits = np.array([int(bits_s, 16)], dtype=np.uint32)
        got = orc.e8m0_value(bits.view(np.float32))[0]
        if val_s == "nan":
            assert math.isnan(got), bits_s
        else:
            assert got == float(eval(val_s, {"__builtins__": {}}, {})), (bits_s, got)


def test_e8m0_golden_cases():
    check_e8m0_golden(O)


def check_e2m1_golden(orc):
    rows = _read_golden("e2m1_values.txt")
    assert len(rows) == 16
    table = orc.e2m1_decode_table()
    for row in rows:
        code_s, val_s = row.split()
        code = int(code_s, 16)
        expected = float(Fraction(val_s.lstrip("-"))) * (-1.0 if val_s.startswith("-") else 1.0)
        assert table[code] == expected, (code_s, table[code])
        assert math.copysign(1.0, table[code]) == math.copysign(1.0, expected), code_s


def test_e2m1_golden_table():
    check_e2m1_golden(O)


def test_bf16_single_rounding_from_f64():
    # 1 + 2^-8 + 2^-40 is just above a tie; rounding through float32 first would
    # land exactly on the tie and then go down to 1.0
    x = np.array([1.0 + 2.0 ** -8 + 2.0 ** -40])
    assert O.bf16_round(x)[0] == 1.0 + 2.0 ** -7


def test_bf16_matches_torch_on_f32_values():
    rng = np.random.default_rng(12345)
    parts = [
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e30).astype(np.float32),
        (rng.standard_normal(20000) * 1e-38).astype(np.float32),   # subnormal range
        (rng.standard_normal(20000) * 1e-42).astype(np.float32),
        np.array([3.3e38, -3.3e38, 3.4e38, np.float32(np.finfo(np.float32).max)], dtype=np.float32),
    ]
    # exact ties in float32: 8 significant bits plus a half
    mant = rng.integers(0, 256, size=20000)
    ties = ((256 + mant) * 2 + 1).astype(np.float64) * 2.0 ** rng.integers(-20, 20, size=20000)
    parts.append(ties.astype(np.float32))
    x32 = np.concatenate(parts)
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.bf16_bits(x32.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_nan_and_roundtrip():
    bits = O.bf16_bits(np.array([np.nan, -np.nan, np.inf, -np.inf]))
    assert bits[0] == 0x7FC0 and bits[2] == 0x7F80 and bits[3] == 0xFF80
    all_bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = O.bf16_bits_to_f64(all_bits)
    finite = np.isfinite(vals)
    assert np.array_equal(O.bf16_bits(vals[finite]), all_bits[finite])
