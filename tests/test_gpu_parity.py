"""GPU parity: the gfx950 kernels against the CPU oracle, through the C ABI.

Small shapes (several tiles, ragged tails, empty groups) are compared in
full; the benchmark workloads at full size are compared on sampled
rows and columns, plus the invariant that no row outside the valid rows is
written. Integer-exact inputs are compared bit for bit.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from moe_grouped_gemm_amd import dg, synth
from oracle import dg_oracle as O
from parity import check_close, check_untouched

pytestmark = pytest.mark.gpu

NP = synth.to_numpy_bytes


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dg.lib()  # the native library must load: no fallback
    return torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)


# ---------------------------------------------------------------------------
# Dense
# ---------------------------------------------------------------------------

DENSE_SHAPES = [
    (128, 256, 512),     # the small benchmark workload
    (300, 384, 1024),    # ragged M, 3 N blocks
    (1, 128, 128),
    (17, 256, 256),
    (257, 128, 128),
    (64, 256, 4096),
    (1000, 640, 384),
    (2048, 1024, 1024),  # more tiles than CUs
    (300, 896, 1024),    # N = 3.5 tiles
    (1, 896, 128),
    # K of 32 blocks and more: the deep-prefetch pipeline
    (300, 384, 4096),
    (257, 1792, 8192),
]


@pytest.mark.parametrize("m,n,k", DENSE_SHAPES)
def test_dense_small(dev, m, n, k):
    _say(f"dense {m}x{n}x{k}")
    w = synth.make_dense(m, n, k, seed=m + n + k, device=dev)
    d = w.new_output()
    dg.fp8_gemm_nt(w.a, w.sfa, w.b, w.sfb, d)
    torch.cuda.synchronize()
    ref = O.gemm_nt_f64(NP(w.a), NP(w.sfa), NP(w.b), NP(w.sfb))
    check_close(NP(d), ref, f"dense {m}x{n}x{k}")


CODE_OF = {0: 0x00, 1: 0x38, 2: 0x40, -1: 0xB8, -2: 0xC0}


def _int_exact(m, n, k, seed):
    """Codes in {-2..2} and power-of-two scales varying per K block, row and
    N block: every float32 partial and promoted sum is exact."""
    rng = np.random.default_rng(seed)
    lut = np.zeros(5, np.uint8)
    for v, c in CODE_OF.items():
        lut[v + 2] = c
    a = lut[rng.integers(-2, 3, size=(m, k)) + 2]
    b = lut[rng.integers(-2, 3, size=(n, k)) + 2]
    ld = (m + 3) // 4 * 4
    sfa = np.ldexp(1.0, rng.integers(-2, 3, size=(k // 128, ld))).astype(np.float32)
    sfb = np.ldexp(1.0, rng.integers(-2, 3, size=(n // 128, k // 128))).astype(np.float32)
    return a, sfa, b, sfb


def _dev_fp8(x, dev):
    return torch.from_numpy(x).to(dev).view(torch.float8_e4m3fn)


@pytest.mark.parametrize("m,n,k", [(200, 256, 1024), (129, 384, 2048), (77, 896, 512), (65, 256, 4096)])
def test_dense_integer_exact_bitwise(dev, m, n, k):
    _say(f"dense integer-exact {m}x{n}x{k}")
    a, sfa, b, sfb = _int_exact(m, n, k, seed=m)
    d = synth.sentinel_output((m, n), dev)
    dg.fp8_gemm_nt(_dev_fp8(a, dev), torch.from_numpy(sfa).to(dev), _dev_fp8(b, dev),
                   torch.from_numpy(sfb).to(dev), d)
    torch.cuda.synchronize()
    ref_bits = O.fp8_gemm_nt(a, sfa, b, sfb)
    got = NP(d)
    assert np.array_equal(got, ref_bits), f"{np.sum(got != ref_bits)} mismatching elements"


def test_dense_deterministic(dev):
    w = synth.make_dense(1024, 2048, 1024, seed=5, device=dev)
    d1, d2 = w.new_output(), w.new_output()
    dg.fp8_gemm_nt(w.a, w.sfa, w.b, w.sfb, d1)
    dg.fp8_gemm_nt(w.a, w.sfa, w.b, w.sfb, d2)
    torch.cuda.synchronize()
    assert torch.equal(d1.view(torch.int16), d2.view(torch.int16))


# ---------------------------------------------------------------------------
# Contiguous layout
# ---------------------------------------------------------------------------

def _contig_ref(w):
    return O.m_grouped_fp8_gemm_nt_contiguous(NP(w.a), NP(w.sfa), NP(w.b), NP(w.sfb), NP(w.layout),
                                              np.full((w.m, w.n), 0xFFFF, np.uint16))


def _check_contiguous(w, d, what):
    got = NP(d)
    layout = NP(w.layout)
    valid = layout >= 0
    ref = np.full((w.m, w.n), np.nan)
    for g in range(w.num_groups):
        rows = np.nonzero(layout == g)[0]
        if rows.size:
            ref[rows] = O.dense_f64_at(NP(w.a), NP(w.sfa), NP(w.b)[g], NP(w.sfb)[g], rows, np.arange(w.n))
    check_close(got[valid], ref[valid], what)
    check_untouched(got[~valid], what + " padding rows")


@pytest.mark.parametrize("rows,n,k", [
    ([130, 0, 77, 256, 1], 256, 512),
    ([128], 128, 128),
    ([5, 300, 1, 129], 384, 1024),
    ([130, 0, 77, 256, 1], 896, 512),
    ([130, 0, 77, 256, 1], 256, 4096),
])
def test_contiguous_small(dev, rows, n, k):
    _say(f"contiguous rows={rows} n={n} k={k}")
    w = synth.make_contiguous(rows, n, k, seed=len(rows), device=dev, poison_padding=True)
    d = w.new_output()
    dg.m_grouped_fp8_gemm_nt_contiguous(w.a, w.sfa, w.b, w.sfb, d, w.layout)
    torch.cuda.synchronize()
    _check_contiguous(w, d, f"contiguous {rows}")


def test_contiguous_out_of_range_ids_and_padding_blocks(dev):
    w = synth.make_contiguous([200, 100, 128], 256, 256, seed=3, device=dev)
    layout = w.layout.clone()
    # a whole padding block in the middle and a segment with an id >= G
    lay = NP(layout).copy()
    lay[256:384] = -1
    lay[384:484] = 7
    lay[484:512] = -1
    layout.copy_(torch.from_numpy(lay))
    w.layout = layout
    d = w.new_output()
    dg.m_grouped_fp8_gemm_nt_contiguous(w.a, w.sfa, w.b, w.sfb, d, w.layout)
    torch.cuda.synchronize()
    got = NP(d)
    check_untouched(got[256:], "ids outside [0, G)")
    ref = O.m_grouped_fp8_gemm_nt_contiguous(NP(w.a), NP(w.sfa), NP(w.b), NP(w.sfb), lay,
                                             np.full((w.m, w.n), 0xFFFF, np.uint16))
    assert np.all(ref[256:] == 0xFFFF)
    valid = lay >= 0
    valid[256:] = False
    ref64 = np.zeros((int(valid.sum()), w.n))
    ref64[:] = O.dense_f64_at(NP(w.a), NP(w.sfa), NP(w.b)[0], NP(w.sfb)[0], np.nonzero(valid)[0], np.arange(w.n))
    check_close(got[valid], ref64, "group 0")


def test_contiguous_equals_dense_per_group(dev):
    """Same kernel arithmetic, so a group's rows match a dense call on them bit for bit."""
    w = synth.make_contiguous([256, 128, 384], 512, 1024, seed=9, device=dev)
    d = w.new_output()
    dg.m_grouped_fp8_gemm_nt_contiguous(w.a, w.sfa, w.b, w.sfb, d, w.layout)
    start = 0
    for g, r in enumerate(w.rows):
        a_g = w.a[start:start + r].contiguous()
        sfa_g = w.sfa[:, start:start + r].contiguous()
        d_g = synth.sentinel_output((r, w.n), dev)
        dg.fp8_gemm_nt(a_g, sfa_g, w.b[g].contiguous(), w.sfb[g].contiguous(), d_g)
        torch.cuda.synchronize()
        assert torch.equal(d[start:start + r].view(torch.int16), d_g.view(torch.int16)), f"group {g}"
        start += r


# ---------------------------------------------------------------------------
# Masked layout
# ---------------------------------------------------------------------------

def _check_masked(w, d, counts, what):
    got = NP(d)
    for g, c in enumerate(counts):
        v = min(max(int(c), 0), w.max_m)
        if v:
            ref = O.dense_f64_at(NP(w.a)[g], NP(w.sfa)[g], NP(w.b)[g], NP(w.sfb)[g], np.arange(v), np.arange(w.n))
            check_close(got[g, :v], ref, f"{what} group {g}")
        check_untouched(got[g, v:], f"{what} group {g} rows >= {v}")


@pytest.mark.parametrize("counts,max_m,n,k", [
    ([0, 1, 200, 77], 200, 256, 512),
    ([256, 129], 256, 384, 1024),
    ([3], 64, 128, 128),
    ([0, 1, 200, 77], 200, 896, 512),
    ([0, 1, 200, 77], 200, 256, 4096),
])
def test_masked_small(dev, counts, max_m, n, k):
    _say(f"masked counts={counts} max_m={max_m} n={n} k={k}")
    w = synth.make_masked(counts, max_m, n, k, seed=max_m, device=dev, poison_invalid=True)
    d = w.new_output()
    dg.m_grouped_fp8_gemm_nt_masked(w.a, w.sfa, w.b, w.sfb, d, w.masked_m)
    torch.cuda.synchronize()
    _check_masked(w, d, counts, "masked")


def test_masked_clamps_counts(dev):
    w = synth.make_masked([10, 10, 10], 96, 128, 256, seed=1, device=dev)
    w.masked_m.copy_(torch.tensor([-3, 500, 33], dtype=torch.int32))
    d = w.new_output()
    dg.m_grouped_fp8_gemm_nt_masked(w.a, w.sfa, w.b, w.sfb, d, w.masked_m)
    torch.cuda.synchronize()
    _check_masked(w, d, [-3, 500, 33], "clamped")


def test_masked_graph_replay_follows_device_counts(dev):
    """One captured graph serves changing masked_m contents; replays are
    checked against eager calls, with eager work between replays."""
    w = synth.make_masked([40, 100, 7, 64], 128, 256, 512, seed=2, device=dev)
    d = w.new_output()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        dg.m_grouped_fp8_gemm_nt_masked(w.a, w.sfa, w.b, w.sfb, d, w.masked_m)  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dg.m_grouped_fp8_gemm_nt_masked(w.a, w.sfa, w.b, w.sfb, d, w.masked_m)
    for counts in ([40, 100, 7, 64], [128, 0, 1, 127], [5, 5, 5, 5]):
        w.masked_m.copy_(torch.tensor(counts, dtype=torch.int32))
        d.view(torch.int16).fill_(-1)
        graph.replay()
        torch.cuda.synchronize()
        d_eager = w.new_output()
        dg.m_grouped_fp8_gemm_nt_masked(w.a, w.sfa, w.b, w.sfb, d_eager, w.masked_m)
        torch.cuda.synchronize()
        assert torch.equal(d.view(torch.int16), d_eager.view(torch.int16)), counts
        _check_masked(w, d, counts, f"graph {counts}")


def test_masked_many_groups(dev):
    """More groups than one 64-wide pass of the on-device group table."""
    rng = np.random.default_rng(31)
    counts = [int(c) for c in rng.integers(0, 40, size=150)]
    counts[64] = 0
    counts[127] = 33
    _say(f"masked {len(counts)} groups")
    w = synth.make_masked(counts, 40, 128, 256, seed=4, device=dev, poison_invalid=True)
    d = w.new_output()
    dg.m_grouped_fp8_gemm_nt_masked(w.a, w.sfa, w.b, w.sfb, d, w.masked_m)
    torch.cuda.synchronize()
    _check_masked(w, d, counts, "masked many groups")


@pytest.mark.parametrize("ue8m0", [False, True])
def test_masked_partial_band_copies(dev, ue8m0):
    """Valid rows ending at and next to the 64-row boundary of each wave's
    128 rows (below it the wave runs the K loop copy without bands 4-7).
    Three workgroups take all 24 tiles, so copies alternate within one
    workgroup; 5 K blocks make consecutive tiles start on alternating
    stages."""
    counts = [64, 65, 192, 193, 48, 80, 16, 17, 256, 0, 1, 129]
    _say(f"masked partial bands ue8m0={ue8m0}")
    w = synth.make_masked(counts, 256, 512, 640, seed=7, device=dev, poison_invalid=True, ue8m0=ue8m0)
    d = w.new_output()
    dg.set_num_cus(3)
    try:
        dg.m_grouped_fp8_gemm_nt_masked(w.a, w.sfa, w.b, w.sfb, d, w.masked_m, ue8m0=ue8m0)
        torch.cuda.synchronize()
    finally:
        dg.set_num_cus(0)
    _check_masked(w, d, counts, "masked partial bands")
    d_full = w.new_output()
    dg.m_grouped_fp8_gemm_nt_masked(w.a, w.sfa, w.b, w.sfb, d_full, w.masked_m, ue8m0=ue8m0)
    torch.cuda.synchronize()
    # the grid size changes which tiles share a workgroup, not the arithmetic
    assert torch.equal(d.view(torch.int16), d_full.view(torch.int16))


# ---------------------------------------------------------------------------
# No-padding layout
# ---------------------------------------------------------------------------

def _check_nopad(w, d, what):
    got = NP(d)
    owned = np.zeros(w.m, bool)
    for g, (first, end) in enumerate(O.nopad_row_ranges(NP(w.group_rows), w.m)):
        if end > first:
            ref = O.dense_f64_at(NP(w.a), NP(w.sfa), NP(w.b)[g], NP(w.sfb)[g], np.arange(first, end),
                                 np.arange(w.n))
            check_close(got[first:end], ref, f"{what} group {g}")
            owned[first:end] = True
    check_untouched(got[~owned], what + " rows no group owns")


@pytest.mark.parametrize("rows,n,k,tail", [
    ([130, 0, 77, 256, 1], 256, 512, 7),
    ([1], 128, 128, 0),
    ([5, 300, 1, 129], 384, 1024, 3),
    ([130, 0, 77, 256, 1], 896, 512, 0),
    ([130, 0, 77, 256, 1], 256, 4096, 5),
])
def test_nopad_small(dev, rows, n, k, tail):
    _say(f"nopad rows={rows} n={n} k={k} tail={tail}")
    w = synth.make_nopad(rows, n, k, seed=len(rows) + tail, device=dev, tail=tail, poison_tail=True)
    d = w.new_output()
    dg.m_grouped_fp8_gemm_nt_nopad(w.a, w.sfa, w.b, w.sfb, d, w.group_rows)
    torch.cuda.synchronize()
    _check_nopad(w, d, f"nopad {rows}")


def test_nopad_many_groups(dev):
    """Groups of 0-6 rows, more than one 64-wide pass of the group table."""
    rng = np.random.default_rng(37)
    rows = [int(c) for c in rng.integers(0, 7, size=300)]
    _say(f"nopad {len(rows)} groups, {sum(rows)} rows")
    w = synth.make_nopad(rows, 128, 256, seed=6, device=dev, tail=9, poison_tail=True)
    d = w.new_output()
    dg.m_grouped_fp8_gemm_nt_nopad(w.a, w.sfa, w.b, w.sfb, d, w.group_rows)
    torch.cuda.synchronize()
    _check_nopad(w, d, "nopad many groups")


def test_nopad_clips_counts(dev):
    """A negative count owns nothing; counts reaching past M are cut off."""
    _say("nopad clipped counts")
    w = synth.make_nopad([-3, 100, 50, 7], 256, 512, seed=8, device=dev, m=120)
    d = w.new_output()
    dg.m_grouped_fp8_gemm_nt_nopad(w.a, w.sfa, w.b, w.sfb, d, w.group_rows)
    torch.cuda.synchronize()
    assert O.nopad_row_ranges(NP(w.group_rows), w.m) == [(0, 0), (0, 100), (100, 120), (120, 120)]
    _check_nopad(w, d, "nopad clipped")


def test_nopad_equals_dense_per_group(dev):
    """Same kernel arithmetic, so a group's rows match a dense call on them bit for bit."""
    w = synth.make_nopad([200, 1, 383, 0, 130], 512, 1024, seed=10, device=dev)
    d = w.new_output()
    dg.m_grouped_fp8_gemm_nt_nopad(w.a, w.sfa, w.b, w.sfb, d, w.group_rows)
    for g, (first, end) in enumerate(w.row_ranges()):
        if end == first:
            continue
        a_g = w.a[first:end].contiguous()
        sfa_g = torch.zeros(w.k // 128, synth.tma_aligned_size(end - first), dtype=torch.float32, device=dev)
        sfa_g[:, :end - first] = w.sfa[:, first:end]
        d_g = synth.sentinel_output((end - first, w.n), dev)
        dg.fp8_gemm_nt(a_g, sfa_g, w.b[g].contiguous(), w.sfb[g].contiguous(), d_g)
        torch.cuda.synchronize()
        assert torch.equal(d[first:end].view(torch.int16), d_g.view(torch.int16)), f"group {g}"


def test_nopad_graph_replay_follows_device_counts(dev):
    """One captured graph serves changing group_rows contents; replays are
    checked against eager calls, with eager work between replays."""
    w = synth.make_nopad([100, 50, 7, 64], 256, 512, seed=12, device=dev, tail=35)
    d = w.new_output()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        dg.m_grouped_fp8_gemm_nt_nopad(w.a, w.sfa, w.b, w.sfb, d, w.group_rows)  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dg.m_grouped_fp8_gemm_nt_nopad(w.a, w.sfa, w.b, w.sfb, d, w.group_rows)
    for rows in ([100, 50, 7, 64], [0, 256, 0, 0], [1, 1, 1, 300]):
        w.group_rows.copy_(torch.tensor(rows, dtype=torch.int32))
        w.rows = list(rows)
        d.view(torch.int16).fill_(-1)
        graph.replay()
        torch.cuda.synchronize()
        d_eager = w.new_output()
        dg.m_grouped_fp8_gemm_nt_nopad(w.a, w.sfa, w.b, w.sfb, d_eager, w.group_rows)
        torch.cuda.synchronize()
        assert torch.equal(d.view(torch.int16), d_eager.view(torch.int16)), rows
        _check_nopad(w, d, f"graph {rows}")


# ---------------------------------------------------------------------------
# Power-of-two (UE8M0) scales: the *_ue8m0 entry points
# ---------------------------------------------------------------------------

def _assert_pow2(*scales):
    for s in scales:
        s = NP(s)
        s = s[s != 0]   # the zero padding of the aligned LHS-scale rows is never read
        assert np.array_equal(O.e8m0_value(s), s.astype(np.float64)), "scales are not powers of two"


@pytest.mark.parametrize("m,n,k", [(128, 256, 512), (300, 384, 1024), (1, 896, 128), (257, 1792, 8192)])
def test_ue8m0_dense(dev, m, n, k):
    _say(f"ue8m0 dense {m}x{n}x{k}")
    w = synth.make_dense(m, n, k, seed=m + k, device=dev, ue8m0=True)
    _assert_pow2(w.sfa, w.sfb)
    d = w.new_output()
    dg.fp8_gemm_nt(w.a, w.sfa, w.b, w.sfb, d, ue8m0=True)
    torch.cuda.synchronize()
    ref = O.gemm_nt_f64(NP(w.a), O.e8m0_value(NP(w.sfa)), NP(w.b), O.e8m0_value(NP(w.sfb)))
    check_close(NP(d), ref, f"ue8m0 dense {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(200, 256, 1024), (77, 896, 512), (65, 256, 4096)])
def test_ue8m0_integer_exact_bitwise(dev, m, n, k):
    _say(f"ue8m0 integer-exact {m}x{n}x{k}")
    a, sfa, b, sfb = _int_exact(m, n, k, seed=m + 1)
    d = synth.sentinel_output((m, n), dev)
    dg.fp8_gemm_nt(_dev_fp8(a, dev), torch.from_numpy(sfa).to(dev), _dev_fp8(b, dev),
                   torch.from_numpy(sfb).to(dev), d, ue8m0=True)
    torch.cuda.synchronize()
    ref_bits = O.fp8_gemm_nt_ue8m0(a, sfa, b, sfb)
    got = NP(d)
    assert np.array_equal(got, ref_bits), f"{np.sum(got != ref_bits)} mismatching elements"


@pytest.mark.parametrize("k", [512, 4096])
def test_ue8m0_grouped_layouts(dev, k):
    _say(f"ue8m0 grouped layouts k={k}")
    rows = [130, 0, 77, 256, 1]
    w = synth.make_contiguous(rows, 256, k, seed=21, device=dev, poison_padding=True, ue8m0=True)
    _assert_pow2(w.sfa, w.sfb)
    d = w.new_output()
    dg.m_grouped_fp8_gemm_nt_contiguous(w.a, w.sfa, w.b, w.sfb, d, w.layout, ue8m0=True)
    torch.cuda.synchronize()
    _check_contiguous(w, d, "ue8m0 contiguous")
    counts = [0, 1, 200, 77]
    w = synth.make_masked(counts, 200, 256, k, seed=22, device=dev, poison_invalid=True, ue8m0=True)
    _assert_pow2(w.sfa, w.sfb)
    d = w.new_output()
    dg.m_grouped_fp8_gemm_nt_masked(w.a, w.sfa, w.b, w.sfb, d, w.masked_m, ue8m0=True)
    torch.cuda.synchronize()
    _check_masked(w, d, counts, "ue8m0 masked")
    w = synth.make_nopad(rows, 256, k, seed=23, device=dev, tail=7, poison_tail=True, ue8m0=True)
    _assert_pow2(w.sfa, w.sfb)
    d = w.new_output()
    dg.m_grouped_fp8_gemm_nt_nopad(w.a, w.sfa, w.b, w.sfb, d, w.group_rows, ue8m0=True)
    torch.cuda.synchronize()
    _check_nopad(w, d, "ue8m0 nopad")


def test_ue8m0_drops_mantissa(dev):
    """Scales that are not powers of two: the mantissa bits are ignored, so the
    output equals the call on the scales rounded down to powers of two, bit
    for bit, and the oracle's UE8M0 variant within the tolerance."""
    w = synth.make_dense(256, 512, 1024, seed=3, device=dev)   # amax/448 scales
    floor_sfa = torch.from_numpy(O.e8m0_value(NP(w.sfa)).astype(np.float32)).to(dev)
    floor_sfb = torch.from_numpy(O.e8m0_value(NP(w.sfb)).astype(np.float32)).to(dev)
    d1, d2 = w.new_output(), w.new_output()
    dg.fp8_gemm_nt(w.a, w.sfa, w.b, w.sfb, d1, ue8m0=True)
    dg.fp8_gemm_nt(w.a, floor_sfa, w.b, floor_sfb, d2, ue8m0=True)
    torch.cuda.synchronize()
    assert torch.equal(d1.view(torch.int16), d2.view(torch.int16))
    ref = O.gemm_nt_f64(NP(w.a), O.e8m0_value(NP(w.sfa)), NP(w.b), O.e8m0_value(NP(w.sfb)))
    check_close(NP(d1), ref, "ue8m0 mantissa dropped")


def test_ue8m0_close_to_float32_path(dev):
    """On power-of-two scales both paths compute the same sum (float32
    accumulation, different order): they agree within the tolerance."""
    w = synth.make_dense(512, 1024, 2048, seed=4, device=dev, ue8m0=True)
    d1, d2 = w.new_output(), w.new_output()
    dg.fp8_gemm_nt(w.a, w.sfa, w.b, w.sfb, d1, ue8m0=True)
    dg.fp8_gemm_nt(w.a, w.sfa, w.b, w.sfb, d2)
    torch.cuda.synchronize()
    check_close(NP(d1), O.bf16_bits_to_f64(NP(d2)), "ue8m0 vs float32 scales")


# ---------------------------------------------------------------------------
# FP8 x FP4 (W4A8): packed E2M1 B, per-32 UE8M0 RHS scales
# ---------------------------------------------------------------------------

def _fp4_ref_rows(w, g, rows, cols, a=None, sfa=None):
    a = NP(w.a) if a is None else a
    sfa = NP(w.sfa) if sfa is None else sfa
    return O.fp8_fp4_f64_at(a, sfa, NP(w.b)[g], NP(w.sfb)[g], rows, cols)


@pytest.mark.parametrize("rows,n,k", [([130, 0, 77, 256, 1], 256, 512), ([5, 300, 1, 129], 384, 1024),
                                      ([130, 0, 77, 256, 1], 896, 4096)])
def test_fp8_fp4_contiguous_small(dev, rows, n, k):
    _say(f"w4a8 contiguous rows={rows} n={n} k={k}")
    w = synth.make_contiguous(rows, n, k, seed=len(rows) + 30, device=dev, poison_padding=True, fp4=True)
    d = w.new_output()
    dg.m_grouped_fp8_fp4_gemm_nt_contiguous(w.a, w.sfa, w.b, w.sfb, d, w.layout)
    torch.cuda.synchronize()
    got, layout = NP(d), NP(w.layout)
    for g in range(w.num_groups):
        idx = np.nonzero(layout == g)[0]
        if idx.size:
            check_close(got[idx], _fp4_ref_rows(w, g, idx, np.arange(w.n)), f"w4a8 contiguous group {g}")
    check_untouched(got[layout < 0], "w4a8 contiguous padding rows")
    ref_bits = O.m_grouped_fp8_fp4_gemm_nt_contiguous(NP(w.a), NP(w.sfa), NP(w.b), NP(w.sfb), layout,
                                                      np.full((w.m, w.n), 0xFFFF, np.uint16))
    assert np.all(ref_bits[layout < 0] == 0xFFFF)


@pytest.mark.parametrize("counts,max_m,n,k", [([0, 1, 200, 77], 200, 256, 512), ([0, 1, 200, 77], 200, 896, 4096)])
def test_fp8_fp4_masked_small(dev, counts, max_m, n, k):
    _say(f"w4a8 masked counts={counts} n={n} k={k}")
    w = synth.make_masked(counts, max_m, n, k, seed=max_m + 30, device=dev, poison_invalid=True, fp4=True)
    d = w.new_output()
    dg.m_grouped_fp8_fp4_gemm_nt_masked(w.a, w.sfa, w.b, w.sfb, d, w.masked_m)
    torch.cuda.synchronize()
    got = NP(d)
    for g, c in enumerate(counts):
        v = min(max(int(c), 0), max_m)
        if v:
            check_close(got[g, :v], _fp4_ref_rows(w, g, np.arange(v), np.arange(n), NP(w.a)[g], NP(w.sfa)[g]),
                        f"w4a8 masked group {g}")
        check_untouched(got[g, v:], f"w4a8 masked group {g} rows >= {v}")


def test_fp8_fp4_masked_partial_band_copies(dev):
    """Valid rows ending at and next to the 64-row boundary of each wave's 128
    rows (below it the wave runs the K loop copy without bands 4-7), with
    three workgroups taking all tiles so that both copies alternate in one
    workgroup."""
    counts = [64, 65, 192, 193, 48, 80, 16, 17, 256, 0, 1, 129]
    _say("w4a8 masked partial bands")
    w = synth.make_masked(counts, 256, 512, 640, seed=37, device=dev, poison_invalid=True, fp4=True)
    d = w.new_output()
    dg.set_num_cus(3)
    try:
        dg.m_grouped_fp8_fp4_gemm_nt_masked(w.a, w.sfa, w.b, w.sfb, d, w.masked_m)
        torch.cuda.synchronize()
    finally:
        dg.set_num_cus(0)
    got = NP(d)
    for g, c in enumerate(counts):
        v = min(max(int(c), 0), 256)
        if v:
            check_close(got[g, :v], _fp4_ref_rows(w, g, np.arange(v), np.arange(512), NP(w.a)[g], NP(w.sfa)[g]),
                        f"w4a8 masked partial bands group {g}")
        check_untouched(got[g, v:], f"w4a8 masked partial bands group {g} rows >= {v}")


def test_fp8_fp4_integer_exact_bitwise(dev):
    """A codes in {-2..2}, B any E2M1 value, scales 2^-1..2^1: every product
    and partial sum is exact in float32, so the output matches bit for bit."""
    rng = np.random.default_rng(73)
    n, k = 384, 1024
    m = 256
    a8, sfa, _, _ = _int_exact(m, 128, k, seed=74)
    sfa = np.ldexp(1.0, rng.integers(-1, 2, size=sfa.shape)).astype(np.float32)
    codes = rng.integers(0, 16, size=(2, n, k)).astype(np.uint8)
    b = (codes[:, :, 0::2] | (codes[:, :, 1::2] << 4)).astype(np.uint8)
    sfb = np.zeros((2, k // 32, synth.tma_aligned_size(n)), np.float32)
    sfb[:, :, :n] = np.ldexp(1.0, rng.integers(-1, 2, size=(2, k // 32, n)))
    layout = np.r_[np.zeros(128), np.ones(100), np.full(28, -1)].astype(np.int32)  # 128-row aligned segments
    d = synth.sentinel_output((m, n), dev)
    dg.m_grouped_fp8_fp4_gemm_nt_contiguous(_dev_fp8(a8, dev), torch.from_numpy(sfa).to(dev),
                                            torch.from_numpy(b).to(dev), torch.from_numpy(sfb).to(dev), d,
                                            torch.from_numpy(layout).to(dev))
    torch.cuda.synchronize()
    ref = O.m_grouped_fp8_fp4_gemm_nt_contiguous(a8, sfa, b, sfb, layout, np.full((m, n), 0xFFFF, np.uint16))
    got = NP(d)
    assert np.array_equal(got, ref), f"{np.sum(got != ref)} mismatching elements"


# ---------------------------------------------------------------------------
# K-grouped GEMM (float32 output)
# ---------------------------------------------------------------------------
#
# Tolerance. The MFMA does not sum a K block's 128 FP8 products as rounded
# float32 additions: measured on MI355X, one block's result is off by up to
# 1.6e-5 (about 2^-16) of the sum of the products' magnitudes (that limited
# accumulation precision is why the method promotes every 128-K block into
# float32 registers). Allowing 2^-15 of that per block, plus the float32
# promotion (sfb * sfa, the product and the add: 3 roundings per block) and
# the rounding of C, every element satisfies
#   |D - R| <= (2^-15 + (nkb + 3) * 2^-24) * sum_k |Ahat Bhat| + 2^-24 * |C|
# with R the float64 oracle and nkb the group's K blocks. The relative
# Frobenius error must stay below 5e-5 (measured: 1.35e-5).

def _check_k_grouped(w, d, c0, what, groups=None, rows=None, cols=None):
    got = d.detach().cpu().numpy().astype(np.float64)
    c_np = None if c0 is None else c0.detach().cpu().numpy()
    rows = np.arange(w.m) if rows is None else rows
    cols = np.arange(w.n) if cols is None else cols
    a, sfa, b, sfb = NP(w.a), NP(w.sfa), NP(w.b), NP(w.sfb)
    if w.ue8m0:
        sfa, sfb = O.e8m0_value(sfa), O.e8m0_value(sfb)
    for g in (range(w.num_groups) if groups is None else groups):
        ref, mag = O.k_grouped_f64_at(a, sfa, b, sfb, w.ks, g, rows, cols, c_np, abs_sum=True)
        cmag = 0.0 if c_np is None else np.abs(c_np[g][np.ix_(rows, cols)])
        out = got[g][np.ix_(rows, cols)]
        nkb = w.ks[g] // 128
        bound = (2.0 ** -15 + (nkb + 3) * 2.0 ** -24) * (mag - cmag) + 2.0 ** -24 * cmag + 1e-30
        bad = np.abs(out - ref) > bound
        assert not bad.any(), f"{what} group {g}: {int(bad.sum())} elements beyond the bound"
        nr = np.linalg.norm(ref)
        if nr > 0:
            assert np.linalg.norm(out - ref) <= 5e-5 * nr, f"{what} group {g}: relative Frobenius error"


@pytest.mark.parametrize("ks,m,n", [
    ([128, 0, 384, 256], 300, 384),
    ([4096], 130, 256),
    ([256, 128], 1, 128),
    ([512, 1024, 128], 520, 640),
])
@pytest.mark.parametrize("c_mode", ["none", "separate", "in_place"])
def test_k_grouped_small(dev, ks, m, n, c_mode):
    _say(f"k_grouped ks={ks} m={m} n={n} c={c_mode}")
    w = synth.make_k_grouped(ks, m, n, seed=m + len(ks), device=dev)
    d = w.new_output()
    c0 = None if c_mode == "none" else d.clone()
    if c_mode == "none":
        d.fill_(float("nan"))             # every element must be written
        dg.k_grouped_fp8_gemm_nt_contiguous(w.a, w.sfa, w.b, w.sfb, d, w.ks)
    elif c_mode == "separate":
        out = torch.full_like(d, float("nan"))
        dg.k_grouped_fp8_gemm_nt_contiguous(w.a, w.sfa, w.b, w.sfb, out, w.ks, c=d)
        torch.cuda.synchronize()
        assert torch.equal(d, c0), "C was modified"
        d = out
    else:
        dg.k_grouped_fp8_gemm_nt_contiguous(w.a, w.sfa, w.b, w.sfb, d, w.ks, c=d)
    torch.cuda.synchronize()
    _check_k_grouped(w, d, c0, f"k_grouped {ks} {c_mode}")


@pytest.mark.parametrize("ks,m,n", [([128, 0, 384, 256], 300, 384), ([4096], 130, 256)])
def test_k_grouped_ue8m0(dev, ks, m, n):
    _say(f"k_grouped ue8m0 ks={ks} m={m} n={n}")
    w = synth.make_k_grouped(ks, m, n, seed=m + 7, device=dev, ue8m0=True)
    _assert_pow2(w.sfa, w.sfb)
    d = w.new_output()
    c0 = d.clone()
    dg.k_grouped_fp8_gemm_nt_contiguous(w.a, w.sfa, w.b, w.sfb, d, w.ks, c=d, ue8m0=True)
    torch.cuda.synchronize()
    _check_k_grouped(w, d, c0, f"k_grouped ue8m0 {ks}")


def test_k_grouped_many_groups(dev):
    rng = np.random.default_rng(59)
    ks = [int(x) * 128 for x in rng.integers(0, 3, size=40)]
    _say(f"k_grouped {len(ks)} groups, K={sum(ks)}")
    w = synth.make_k_grouped(ks, 64, 128, seed=5, device=dev)
    d = w.new_output()
    c0 = d.clone()
    dg.k_grouped_fp8_gemm_nt_contiguous(w.a, w.sfa, w.b, w.sfb, d, w.ks, c=d)
    torch.cuda.synchronize()
    _check_k_grouped(w, d, c0, "k_grouped many groups")


# ---------------------------------------------------------------------------
# The benchmark workloads at full size (sampled comparison)
# ---------------------------------------------------------------------------

def _sample(n_total, count, rng, extra=()):
    idx = set(int(x) for x in rng.choice(n_total, size=min(count, n_total), replace=False))
    idx.update(int(e) for e in extra if 0 <= e < n_total)
    return np.array(sorted(idx), dtype=np.int64)


@pytest.mark.parametrize("index", list(range(synth.NUM_WORKLOADS)))
def test_workload_full_size(dev, index):
    spec = synth.workload_spec(index)
    _say(f"workload {index} {spec.name}")
    w = synth.make_workload(spec, seed=0, device=dev)
    d = w.new_output()
    c0 = d.clone() if spec.kind == "k_grouped" else None
    dg.run_workload(w, d)
    torch.cuda.synchronize()
    rng = np.random.default_rng(100 + index)
    if getattr(w, "fp4", False):
        got = NP(d)
        if spec.kind == "contiguous":
            layout = NP(w.layout)
            cols = _sample(w.n, 48, rng, (0, 127, 128, w.n - 1))
            for g in range(w.num_groups):
                idx = np.nonzero(layout == g)[0]
                rows = idx[_sample(idx.size, 12, rng, (0, idx.size - 1))]
                check_close(got[np.ix_(rows, cols)], _fp4_ref_rows(w, g, rows, cols), f"{spec.name} group {g}")
            check_untouched(got[layout < 0], spec.name + " padding rows")
        else:
            for g in range(w.num_groups):
                v = w.counts[g]
                rows = _sample(v, 8, rng, (0, v - 1))
                cols = _sample(w.n, 32, rng, (0, w.n - 1))
                ref = _fp4_ref_rows(w, g, rows, cols, NP(w.a)[g], NP(w.sfa)[g])
                check_close(got[g][np.ix_(rows, cols)], ref, f"{spec.name} group {g}")
                check_untouched(got[g, v:], f"{spec.name} group {g} rows >= {v}")
        return
    if spec.kind == "k_grouped":
        rows = _sample(w.m, 24, rng, (0, 255, 256, w.m - 1))
        cols = _sample(w.n, 24, rng, (0, 255, 256, w.n - 1))
        _check_k_grouped(w, d, c0, spec.name, rows=rows, cols=cols)
        return
    got = NP(d)
    a, sfa, b, sfb = NP(w.a), NP(w.sfa), NP(w.b), NP(w.sfb)
    if w.ue8m0:
        sfa, sfb = O.e8m0_value(sfa), O.e8m0_value(sfb)
    if spec.kind == "dense":
        rows = _sample(w.m, 96, rng, (0, 127, 128, 255, 256, w.m - 1))
        cols = _sample(w.n, 96, rng, (0, 127, 128, 255, w.n - 1))
        ref = O.dense_f64_at(a, sfa, b, sfb, rows, cols)
        check_close(got[np.ix_(rows, cols)], ref, spec.name)
    elif spec.kind == "contiguous":
        layout = NP(w.layout)
        valid_rows = np.nonzero(layout >= 0)[0]
        starts = np.nonzero(np.diff(np.r_[-2, layout]) != 0)[0]
        rows = np.union1d(valid_rows[rng.choice(valid_rows.size, 128, replace=False)],
                          np.intersect1d(starts, valid_rows))
        cols = _sample(w.n, 64, rng, (0, 127, 128, w.n - 1))
        ref = O.contiguous_f64_at(a, sfa, b, sfb, layout, rows, cols)
        check_close(got[np.ix_(rows, cols)], ref, spec.name)
        check_untouched(got[layout < 0], spec.name + " padding rows")
    elif spec.kind == "nopad":
        group_rows = NP(w.group_rows)
        ranges = O.nopad_row_ranges(group_rows, w.m)
        firsts = [f for f, e in ranges if e > f]
        lasts = [e - 1 for f, e in ranges if e > f]
        rows = _sample(w.m, 128, rng, firsts + lasts)
        cols = _sample(w.n, 64, rng, (0, 127, 128, w.n - 1))
        ref = O.nopad_f64_at(a, sfa, b, sfb, group_rows, rows, cols)
        check_close(got[np.ix_(rows, cols)], ref, spec.name)
        used = max(lasts) + 1
        check_untouched(got[used:], spec.name + " rows no group owns")
    else:
        counts = w.counts
        for g in range(w.num_groups):
            v = counts[g]
            rows = _sample(v, 8, rng, (0, v - 1))
            cols = _sample(w.n, 32, rng, (0, w.n - 1))
            ref = O.masked_f64_at(a, sfa, b, sfb, w.masked_m.cpu().numpy(), g, rows, cols)
            check_close(got[g][np.ix_(rows, cols)], ref, f"{spec.name} group {g}")
            check_untouched(got[g, v:], f"{spec.name} group {g} rows >= {v}")
