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
from parity import abs_e4m3, check_close, check_untouched

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
    (2048, 1024, 1024),
    (4096, 8192, 512),   # 512 tiles: two rounds of the persistent grid on 256 CUs
    (300, 896, 1024),    # N = 3.5 tiles
    (1, 896, 128),
    # K of 32 blocks and more: the deep-prefetch pipeline
    (300, 384, 4096),
    (257, 1792, 8192),
]


def _dense_ref(a, sfa, b, sfb):
    """The oracle's unrounded dense result and the sum of the products'
    magnitudes (the oracle on |A| and |B|), for the per-element bound."""
    return (O.gemm_nt_f64(a, sfa, b, sfb),
            O.gemm_nt_f64(abs_e4m3(a), np.abs(sfa), abs_e4m3(b), np.abs(sfb)))


@pytest.mark.parametrize("m,n,k", DENSE_SHAPES)
def test_dense_small(dev, m, n, k):
    _say(f"dense {m}x{n}x{k}")
    w = synth.make_dense(m, n, k, seed=m + n + k, device=dev)
    d = w.new_output()
    dg.fp8_gemm_nt(w.a, w.sfa, w.b, w.sfb, d)
    torch.cuda.synchronize()
    ref, mag = _dense_ref(NP(w.a), NP(w.sfa), NP(w.b), NP(w.sfb))
    check_close(NP(d), ref, f"dense {m}x{n}x{k}", mag, k)


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


def _check_contiguous(w, d, what, sfa=None, sfb=None):
    got = NP(d)
    layout = NP(w.layout)
    sfa = NP(w.sfa) if sfa is None else sfa
    sfb = NP(w.sfb) if sfb is None else sfb
    valid = O.contiguous_row_groups(layout, w.num_groups) >= 0
    rows = np.nonzero(valid)[0]
    ref, mag = O.contiguous_f64_at(NP(w.a), sfa, NP(w.b), sfb, layout, rows, np.arange(w.n), abs_sum=True)
    check_close(got[valid], ref, what, mag, w.k)
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
    ref64, mag = O.dense_f64_at(NP(w.a), NP(w.sfa), NP(w.b)[0], NP(w.sfb)[0], np.nonzero(valid)[0],
                                np.arange(w.n), abs_sum=True)
    check_close(got[valid], ref64, "group 0", mag, w.k)


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


def test_contiguous_ids_changing_inside_blocks(dev):
    """Layouts whose segments are not 128-row aligned: a row is written only
    when its id is the id of its 128-row block's first row (and names a
    group). Checked against the oracle's row rule and values, and rows it
    leaves out must keep the sentinel."""
    _say("contiguous ids changing inside 128-row blocks")
    w = synth.make_contiguous([256, 256, 256], 384, 512, seed=41, device=dev)
    lay = np.full(w.m, -1, np.int32)
    lay[0:100] = 0
    lay[100:128] = 1        # group 1 rows inside group 0's block
    lay[128:200] = 1
    lay[200:300] = 2        # crosses into block 2, whose first row says 2
    lay[300:384] = 0        # group 0 rows inside group 2's block
    lay[384] = -1           # block 3 starts with padding
    lay[385:500] = 1
    lay[512:640] = 2        # an aligned block in the second 256-row tile
    lay[640:700] = 9        # an id outside [0, G)
    w.layout.copy_(torch.from_numpy(lay))
    d = w.new_output()
    dg.m_grouped_fp8_gemm_nt_contiguous(w.a, w.sfa, w.b, w.sfb, d, w.layout)
    torch.cuda.synchronize()
    owner = O.contiguous_row_groups(lay, w.num_groups)
    assert np.array_equal(np.nonzero(owner >= 0)[0], np.r_[0:100, 128:200, 256:300, 512:640])
    _check_contiguous(w, d, "contiguous unaligned ids")
    ref_bits = O.m_grouped_fp8_gemm_nt_contiguous(NP(w.a), NP(w.sfa), NP(w.b), NP(w.sfb), lay,
                                                  np.full((w.m, w.n), 0xFFFF, np.uint16))
    assert np.all(ref_bits[owner < 0] == 0xFFFF)


def _int_exact_grouped(g_count, rows_a, n, k, seed):
    """Integer-exact operands for grouped layouts: codes in {-2..2}, B per
    group, power-of-two scales varying per K block, row and N block."""
    a, sfa, _, _ = _int_exact(rows_a, 128, k, seed)
    bs, sfbs = [], []
    for g in range(g_count):
        _, _, b, sfb = _int_exact(4, n, k, seed + 100 + g)
        bs.append(b)
        sfbs.append(sfb)
    return a, sfa, np.stack(bs), np.stack(sfbs)


@pytest.mark.parametrize("k", [1024, 4096])
def test_grouped_integer_exact_bitwise(dev, k):
    """Contiguous, masked and no-padding layouts with integer-exact inputs:
    every float32 intermediate is exact, so D equals the oracle bit for bit
    (K = 4096 runs the deep-prefetch pipeline)."""
    _say(f"grouped integer-exact k={k}")
    n = 384
    # contiguous: groups of 200, 0, 77 and 300 rows, each padded to 128
    rows = [200, 0, 77, 300]
    layout = synth.contiguous_layout(rows)
    m = layout.size
    a, sfa, b, sfb = _int_exact_grouped(len(rows), m, n, k, seed=k)
    d = synth.sentinel_output((m, n), dev)
    dg.m_grouped_fp8_gemm_nt_contiguous(_dev_fp8(a, dev), torch.from_numpy(sfa).to(dev), _dev_fp8(b, dev),
                                        torch.from_numpy(sfb).to(dev), d, torch.from_numpy(layout).to(dev))
    torch.cuda.synchronize()
    ref = O.m_grouped_fp8_gemm_nt_contiguous(a, sfa, b, sfb, layout, np.full((m, n), 0xFFFF, np.uint16))
    assert np.array_equal(NP(d), ref), f"contiguous: {np.sum(NP(d) != ref)} mismatching elements"
    # no-padding: the same rows without padding, and 9 rows no group owns
    m2 = sum(rows) + 9
    a2, sfa2, b2, sfb2 = _int_exact_grouped(len(rows), m2, n, k, seed=k + 1)
    counts = np.array(rows, np.int32)
    d = synth.sentinel_output((m2, n), dev)
    dg.m_grouped_fp8_gemm_nt_nopad(_dev_fp8(a2, dev), torch.from_numpy(sfa2).to(dev), _dev_fp8(b2, dev),
                                   torch.from_numpy(sfb2).to(dev), d, torch.from_numpy(counts).to(dev))
    torch.cuda.synchronize()
    ref = O.m_grouped_fp8_gemm_nt_nopad(a2, sfa2, b2, sfb2, counts, np.full((m2, n), 0xFFFF, np.uint16))
    assert np.array_equal(NP(d), ref), f"nopad: {np.sum(NP(d) != ref)} mismatching elements"
    # masked: counts below, at and past the 64-row band boundaries
    masked = np.array([1, 64, 65, 200, 0, 256], np.int32)
    g_count, max_m = masked.size, 256
    a3, _, b3, sfb3 = _int_exact_grouped(g_count, g_count * max_m, n, k, seed=k + 2)
    a3 = a3.reshape(g_count, max_m, k)
    rng = np.random.default_rng(k)
    sfa3 = np.ldexp(1.0, rng.integers(-2, 3, size=(g_count, k // 128, max_m))).astype(np.float32)
    d = synth.sentinel_output((g_count, max_m, n), dev)
    dg.m_grouped_fp8_gemm_nt_masked(_dev_fp8(a3, dev), torch.from_numpy(sfa3).to(dev), _dev_fp8(b3, dev),
                                    torch.from_numpy(sfb3).to(dev), d, torch.from_numpy(masked).to(dev))
    torch.cuda.synchronize()
    ref = O.m_grouped_fp8_gemm_nt_masked(a3, sfa3, b3, sfb3, masked, np.full((g_count, max_m, n), 0xFFFF, np.uint16))
    assert np.array_equal(NP(d), ref), f"masked: {np.sum(NP(d) != ref)} mismatching elements"


# ---------------------------------------------------------------------------
# Masked layout
# ---------------------------------------------------------------------------

def _check_masked(w, d, counts, what, sfa=None, sfb=None):
    got = NP(d)
    sfa = NP(w.sfa) if sfa is None else sfa
    sfb = NP(w.sfb) if sfb is None else sfb
    for g, c in enumerate(counts):
        v = min(max(int(c), 0), w.max_m)
        if v:
            ref, mag = O.dense_f64_at(NP(w.a)[g], sfa[g], NP(w.b)[g], sfb[g], np.arange(v), np.arange(w.n),
                                      abs_sum=True)
            check_close(got[g, :v], ref, f"{what} group {g}", mag, w.k)
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

def _check_nopad(w, d, what, sfa=None, sfb=None):
    got = NP(d)
    sfa = NP(w.sfa) if sfa is None else sfa
    sfb = NP(w.sfb) if sfb is None else sfb
    owned = np.zeros(w.m, bool)
    for g, (first, end) in enumerate(O.nopad_row_ranges(NP(w.group_rows), w.m)):
        if end > first:
            ref, mag = O.dense_f64_at(NP(w.a), sfa, NP(w.b)[g], sfb[g], np.arange(first, end), np.arange(w.n),
                                      abs_sum=True)
            check_close(got[first:end], ref, f"{what} group {g}", mag, w.k)
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
    ref, mag = _dense_ref(NP(w.a), O.e8m0_value(NP(w.sfa)), NP(w.b), O.e8m0_value(NP(w.sfb)))
    check_close(NP(d), ref, f"ue8m0 dense {m}x{n}x{k}", mag, k)


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
    _check_contiguous(w, d, "ue8m0 contiguous", O.e8m0_value(NP(w.sfa)), O.e8m0_value(NP(w.sfb)))
    counts = [0, 1, 200, 77]
    w = synth.make_masked(counts, 200, 256, k, seed=22, device=dev, poison_invalid=True, ue8m0=True)
    _assert_pow2(w.sfa, w.sfb)
    d = w.new_output()
    dg.m_grouped_fp8_gemm_nt_masked(w.a, w.sfa, w.b, w.sfb, d, w.masked_m, ue8m0=True)
    torch.cuda.synchronize()
    _check_masked(w, d, counts, "ue8m0 masked", O.e8m0_value(NP(w.sfa)), O.e8m0_value(NP(w.sfb)))
    w = synth.make_nopad(rows, 256, k, seed=23, device=dev, tail=7, poison_tail=True, ue8m0=True)
    _assert_pow2(w.sfa, w.sfb)
    d = w.new_output()
    dg.m_grouped_fp8_gemm_nt_nopad(w.a, w.sfa, w.b, w.sfb, d, w.group_rows, ue8m0=True)
    torch.cuda.synchronize()
    _check_nopad(w, d, "ue8m0 nopad", O.e8m0_value(NP(w.sfa)), O.e8m0_value(NP(w.sfb)))


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
    ref, mag = _dense_ref(NP(w.a), O.e8m0_value(NP(w.sfa)), NP(w.b), O.e8m0_value(NP(w.sfb)))
    check_close(NP(d1), ref, "ue8m0 mantissa dropped", mag, w.k)


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
    """(value, magnitude) of group g's W4A8 result at rows x cols."""
    a = NP(w.a) if a is None else a
    sfa = NP(w.sfa) if sfa is None else sfa
    return O.fp8_fp4_f64_at(a, sfa, NP(w.b)[g], NP(w.sfb)[g], rows, cols, abs_sum=True)


def _check_fp4(got, refmag, what, k):
    check_close(got, refmag[0], what, refmag[1], k)


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
            _check_fp4(got[idx], _fp4_ref_rows(w, g, idx, np.arange(w.n)), f"w4a8 contiguous group {g}", k)
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
            _check_fp4(got[g, :v], _fp4_ref_rows(w, g, np.arange(v), np.arange(n), NP(w.a)[g], NP(w.sfa)[g]),
                       f"w4a8 masked group {g}", k)
        check_untouched(got[g, v:], f"w4a8 masked group {g} rows >= {v}")


def test_fp8_fp4_masked_partial_band_copies(dev):
    """Valid rows ending at and next to the 32-, 64- and 96-row boundaries of
    each wave's 128 rows: a wave whose rows lie in its first 2, 4 or 6 bands
    runs the K loop copy without the other bands' MFMAs, and each copy is run
    with its last band valid (32, 64, 96; 160, 192, 224 for the second wave)
    and with one row past it. Three workgroups take all tiles so that the
    copies alternate in one workgroup."""
    counts = [32, 33, 64, 65, 96, 97, 160, 161, 192, 193, 224, 225, 48, 80, 16, 17, 256, 0, 1, 129]
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
            _check_fp4(got[g, :v], _fp4_ref_rows(w, g, np.arange(v), np.arange(512), NP(w.a)[g], NP(w.sfa)[g]),
                       f"w4a8 masked partial bands group {g}", 640)
        check_untouched(got[g, v:], f"w4a8 masked partial bands group {g} rows >= {v}")


@pytest.mark.parametrize("k", [128, 1024])
def test_fp8_fp4_float32_scales(dev, k):
    """FP32 logical scales that are not powers of two: each is taken as its
    E8M0 value (the float32 exponent field), for the LHS 1x128 and the RHS
    1x32 scales alike. The output equals the call on the scales rounded down
    to powers of two bit for bit, and the oracle within the tolerance; the
    page's adapted case is K = 128."""
    _say(f"w4a8 float32 scales k={k}")
    w = synth.make_contiguous([130, 77, 256], 256, k, seed=k + 43, device=dev, fp4=True)
    rng = np.random.default_rng(k)
    sfa = NP(w.sfa) * rng.uniform(1.0, 2.0, size=NP(w.sfa).shape).astype(np.float32)
    sfb = NP(w.sfb) * rng.uniform(1.0, 2.0, size=NP(w.sfb).shape).astype(np.float32)
    assert not np.array_equal(O.e8m0_value(sfb[sfb != 0]), sfb[sfb != 0].astype(np.float64))
    d1, d2 = w.new_output(), w.new_output()
    dg.m_grouped_fp8_fp4_gemm_nt_contiguous(w.a, torch.from_numpy(sfa).to(dev), w.b, torch.from_numpy(sfb).to(dev),
                                            d1, w.layout)
    floor_a = torch.from_numpy(O.e8m0_value(sfa).astype(np.float32)).to(dev)
    floor_b = torch.from_numpy(O.e8m0_value(sfb).astype(np.float32)).to(dev)
    dg.m_grouped_fp8_fp4_gemm_nt_contiguous(w.a, floor_a, w.b, floor_b, d2, w.layout)
    torch.cuda.synchronize()
    assert torch.equal(d1.view(torch.int16), d2.view(torch.int16))
    got, layout = NP(d1), NP(w.layout)
    for g in range(w.num_groups):
        idx = np.nonzero(layout == g)[0]
        ref = O.fp8_fp4_f64_at(NP(w.a), sfa, NP(w.b)[g], sfb[g], idx, np.arange(w.n), abs_sum=True)
        _check_fp4(got[idx], ref, f"w4a8 float32 scales group {g}", k)
    check_untouched(got[layout < 0], "w4a8 float32 scales padding rows")


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
    got = d.detach().cpu().numpy()                       # float32 [G, M, N]
    c_np = None if c0 is None else c0.detach().cpu().numpy()
    rows = np.arange(w.m) if rows is None else rows
    cols = np.arange(w.n) if cols is None else cols
    a, sfa, b, sfb = NP(w.a), NP(w.sfa), NP(w.b), NP(w.sfb)
    if w.ue8m0:
        sfa, sfb = O.e8m0_value(sfa), O.e8m0_value(sfb)
    for g in (range(w.num_groups) if groups is None else groups):
        ref, mag = O.k_grouped_f64_at(a, sfa, b, sfb, w.ks, g, rows, cols, c_np, abs_sum=True)
        cmag = 0.0 if c_np is None else np.abs(c_np[g][np.ix_(rows, cols)].astype(np.float64))
        out = got[g][np.ix_(rows, cols)].astype(np.float64)
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
# Special values inside the valid rows: the E4M3 NaN codes (0x7F, 0xFF) and a
# scale whose E8M0 reading is NaN make the elements they reach NaN and no
# other (IEEE arithmetic in the oracle fixes which); a zero scale, a negated
# scale (the E8M0 reading ignores the sign) and everything else are compared
# as usual. The BF16 outputs are compared as bits where they are NaN-free.
# ---------------------------------------------------------------------------

def _check_with_nans(got_bits, ref, mag, what, k):
    d = O.bf16_bits_to_f64(got_bits)
    assert np.array_equal(np.isnan(d), np.isnan(ref)), (
        f"{what}: NaN pattern differs, first at {np.argwhere(np.isnan(d) != np.isnan(ref))[:3].tolist()}")
    finite = ~np.isnan(ref)
    assert finite.any()
    check_close(got_bits[finite], ref[finite], what, mag[finite], k)


@pytest.mark.parametrize("ue8m0", [False, True])
def test_dense_special_values(dev, ue8m0):
    m, n, k = 300, 384, 512
    _say(f"dense special values ue8m0={ue8m0}")
    w = synth.make_dense(m, n, k, seed=41, device=dev, ue8m0=ue8m0)
    a8, b8 = w.a.view(torch.uint8), w.b.view(torch.uint8)
    a8[5, 130] = 0x7F                     # NaN codes: rows 5 and 77, column 300
    a8[77, 0] = 0xFF
    b8[300, 511] = 0x7F
    w.sfa[2, 256:300] = 0.0               # a zero scale: K block 2 of rows 256..299
    w.sfa[0, 3] = -w.sfa[0, 3]            # a negated scale
    w.sfb[1, 3] = float("nan")            # RHS scale of columns 128..255, K block 3
    d = w.new_output()
    dg.fp8_gemm_nt(w.a, w.sfa, w.b, w.sfb, d, ue8m0=ue8m0)
    torch.cuda.synchronize()
    sfa, sfb = NP(w.sfa), NP(w.sfb)
    if ue8m0:
        sfa, sfb = O.e8m0_value(sfa), O.e8m0_value(sfb)
    ref, mag = O.dense_f64_at(NP(w.a), sfa, NP(w.b), sfb, np.arange(m), np.arange(n), abs_sum=True)
    assert np.isnan(ref[5]).all() and np.isnan(ref[:, 300]).all() and np.isnan(ref[:, 128:256]).all()
    _check_with_nans(NP(d), ref, mag, f"dense special values ue8m0={ue8m0}", k)


def test_masked_special_values(dev):
    counts, max_m, n, k = [40, 0, 200, 17], 200, 256, 512
    _say("masked special values")
    w = synth.make_masked(counts, max_m, n, k, seed=43, device=dev, poison_invalid=True)
    a8 = w.a.view(torch.uint8)
    a8[0, 39, 300] = 0x7F                 # the last valid row of group 0
    a8[2, 0, 0] = 0xFF                    # the first row of group 2
    w.sfa[3, 1, 0:17] = 0.0               # group 3, K block 1: zero scales
    d = w.new_output()
    dg.m_grouped_fp8_gemm_nt_masked(w.a, w.sfa, w.b, w.sfb, d, w.masked_m)
    torch.cuda.synchronize()
    got, a, sfa, b, sfb = NP(d), NP(w.a), NP(w.sfa), NP(w.b), NP(w.sfb)
    for g, v in enumerate(counts):
        if v:
            ref, mag = O.dense_f64_at(a[g], sfa[g], b[g], sfb[g], np.arange(v), np.arange(n), abs_sum=True)
            if g in (0, 2):
                _check_with_nans(got[g, :v], ref, mag, f"masked special values group {g}", k)
            else:
                check_close(got[g, :v], ref, f"masked special values group {g}", mag, k)
        check_untouched(got[g, v:], f"masked special values group {g} rows >= {v}")


def test_k_grouped_special_values(dev):
    """A NaN code in group 1's K range reaches group 1's output row only."""
    ks, m, n = [256, 384, 128], 130, 256
    _say("k_grouped special values")
    w = synth.make_k_grouped(ks, m, n, seed=47, device=dev)
    w.a.view(torch.uint8)[9, 256 + 200] = 0x7F    # row 9, inside group 1's K columns
    d = w.new_output()
    c0 = d.clone()
    dg.k_grouped_fp8_gemm_nt_contiguous(w.a, w.sfa, w.b, w.sfb, d, w.ks, c=d)
    torch.cuda.synchronize()
    got = d.detach().cpu().numpy().astype(np.float64)
    c_np = c0.detach().cpu().numpy()
    a, sfa, b, sfb = NP(w.a), NP(w.sfa), NP(w.b), NP(w.sfb)
    for g in range(len(ks)):
        ref, mag = O.k_grouped_f64_at(a, sfa, b, sfb, w.ks, g, np.arange(m), np.arange(n), c_np, abs_sum=True)
        assert np.array_equal(np.isnan(got[g]), np.isnan(ref)), f"group {g}: NaN pattern differs"
        assert np.isnan(ref[9]).all() == (g == 1) and np.isnan(ref).sum() == (n if g == 1 else 0)
    keep = np.r_[0:9, 10:m]
    _check_k_grouped(w, d, c0, "k_grouped special values", rows=keep)


def test_fp8_fp4_special_values(dev):
    """W4A8 (every scale read as E8M0): a NaN code in A, a NaN RHS scale of
    one column and 32-K block, and a zero LHS scale (read as 2^-127)."""
    rows, n, k = [130, 0, 77, 256], 256, 512
    _say("w4a8 special values")
    w = synth.make_contiguous(rows, n, k, seed=53, device=dev, poison_padding=True, fp4=True)
    layout = NP(w.layout)
    w.a.view(torch.uint8)[int(np.nonzero(layout == 2)[0][5]), 257] = 0xFF
    w.sfb[0, 3, 17] = float("nan")
    w.sfa[1, int(np.nonzero(layout == 3)[0][0])] = 0.0
    d = w.new_output()
    dg.m_grouped_fp8_fp4_gemm_nt_contiguous(w.a, w.sfa, w.b, w.sfb, d, w.layout)
    torch.cuda.synchronize()
    got = NP(d)
    nan_groups = set()
    for g in range(w.num_groups):
        idx = np.nonzero(layout == g)[0]
        if idx.size:
            ref, mag = _fp4_ref_rows(w, g, idx, np.arange(n))
            if np.isnan(ref).any():
                nan_groups.add(g)
            _check_with_nans(got[idx], ref, mag, f"w4a8 special values group {g}", k)
    assert nan_groups == {0, 2}
    check_untouched(got[layout < 0], "w4a8 special values padding rows")


# ---------------------------------------------------------------------------
# The largest group count each grouped call accepts: the on-device group
# table of the masked (G + 1 entries) and no-padding (2G + 2) layouts filled
# to its last entry, and the K-grouped kernel's group offsets in its
# arguments filled to the last one. The last group always has rows (or K),
# so that the table's last entries are used. The groups hold a few rows
# each, so the BF16 outputs are checked as one output: the Frobenius and
# max-abs pair is a statement about a whole output (on 128 elements a single
# legitimate midpoint flip of a large element can exceed 1e-3), while the
# per-element bound and the midpoint rule apply to every element anyway.
# ---------------------------------------------------------------------------

MAX_GROUPS = {"masked": 4096, "w4a8_masked": 4096, "nopad": 2048, "k_grouped": 512}


@pytest.mark.parametrize("kind", list(MAX_GROUPS))
def test_maximum_group_counts(dev, kind):
    g_max = MAX_GROUPS[kind]
    rng = np.random.default_rng([71, g_max, len(kind)])
    _say(f"{kind}: {g_max} groups")
    if kind == "k_grouped":
        ks = [int(x) * 128 for x in rng.integers(0, 2, size=g_max)]
        ks[-1] = 128
        w = synth.make_k_grouped(ks, 64, 128, seed=7, device=dev)
        d = w.new_output()
        c0 = d.clone()
        dg.k_grouped_fp8_gemm_nt_contiguous(w.a, w.sfa, w.b, w.sfb, d, w.ks, c=d)
        torch.cuda.synchronize()
        _check_k_grouped(w, d, c0, kind)
        return
    if kind == "nopad":
        rows = [int(x) for x in rng.integers(0, 4, size=g_max)]
        rows[-1] = 3
        w = synth.make_nopad(rows, 128, 128, seed=8, device=dev, tail=5, poison_tail=True)
        d = w.new_output()
        dg.m_grouped_fp8_gemm_nt_nopad(w.a, w.sfa, w.b, w.sfb, d, w.group_rows)
        torch.cuda.synchronize()
        got, a, sfa, b, sfb = NP(d), NP(w.a), NP(w.sfa), NP(w.b), NP(w.sfb)
        owned = np.zeros(w.m, bool)
        parts = []
        for g, (first, end) in enumerate(O.nopad_row_ranges(NP(w.group_rows), w.m)):
            if end > first:
                ref, mag = O.dense_f64_at(a, sfa, b[g], sfb[g], np.arange(first, end), np.arange(w.n), abs_sum=True)
                parts.append((got[first:end], ref, mag))
                owned[first:end] = True
        d_all, ref_all, mag_all = (np.concatenate(x) for x in zip(*parts))
        check_close(d_all, ref_all, kind, mag_all, w.k)
        check_untouched(got[~owned], kind + " rows no group owns")
        return
    fp4 = kind == "w4a8_masked"
    counts = [int(x) for x in rng.integers(0, 17, size=g_max)]
    counts[-1] = 16
    w = synth.make_masked(counts, 16, 128, 128, seed=9, device=dev, poison_invalid=True, fp4=fp4)
    d = w.new_output()
    call = dg.m_grouped_fp8_fp4_gemm_nt_masked if fp4 else dg.m_grouped_fp8_gemm_nt_masked
    call(w.a, w.sfa, w.b, w.sfb, d, w.masked_m)
    torch.cuda.synchronize()
    got, a, sfa, b, sfb = NP(d), NP(w.a), NP(w.sfa), NP(w.b), NP(w.sfb)
    ref_at = O.fp8_fp4_f64_at if fp4 else O.dense_f64_at
    parts = []
    for g, v in enumerate(counts):
        if v:
            ref, mag = ref_at(a[g], sfa[g], b[g], sfb[g], np.arange(v), np.arange(w.n), abs_sum=True)
            parts.append((got[g, :v], ref, mag))
        check_untouched(got[g, v:], f"{kind} group {g} rows >= {v}")
    d_all, ref_all, mag_all = (np.concatenate(x) for x in zip(*parts))
    check_close(d_all, ref_all, kind, mag_all, w.k)


# ---------------------------------------------------------------------------
# Small persistent grids: every kernel with 1, 3 and 8 workgroups, so that one
# workgroup walks many tiles (3 also leaves the XCD renumbering off). The
# grid changes which tiles share a workgroup, not the arithmetic, so the
# output must equal the default grid's bit for bit; it is also checked
# against the oracle. K = 128 gives one K block per tile (the refills then
# reach the tile after next); K-grouped groups of zero and one K block
# exercise its first-block hand-over.
# ---------------------------------------------------------------------------

SMALL_GRID_CASES = [
    ("dense", dict(m=700, n=640, k=128)),
    ("dense", dict(m=700, n=640, k=640)),
    ("dense", dict(m=300, n=896, k=4096)),
    ("contiguous", dict(rows=[300, 0, 129, 512], n=384, k=256)),
    ("contiguous", dict(rows=[300, 0, 129, 512], n=384, k=4096)),
    ("nopad", dict(rows=[300, 0, 129, 77], n=384, k=384)),
    ("k_grouped", dict(ks=[128, 0, 384, 128, 256], m=300, n=384)),
    ("w4a8_contiguous", dict(rows=[300, 0, 129], n=384, k=512)),
]


def _small_grid_run(kind, w):
    if kind == "k_grouped":
        d = w.new_output()
        dg.k_grouped_fp8_gemm_nt_contiguous(w.a, w.sfa, w.b, w.sfb, d, w.ks)
    else:
        d = w.new_output()
        if kind == "dense":
            dg.fp8_gemm_nt(w.a, w.sfa, w.b, w.sfb, d)
        elif kind == "contiguous":
            dg.m_grouped_fp8_gemm_nt_contiguous(w.a, w.sfa, w.b, w.sfb, d, w.layout)
        elif kind == "nopad":
            dg.m_grouped_fp8_gemm_nt_nopad(w.a, w.sfa, w.b, w.sfb, d, w.group_rows)
        else:
            dg.m_grouped_fp8_fp4_gemm_nt_contiguous(w.a, w.sfa, w.b, w.sfb, d, w.layout)
    torch.cuda.synchronize()
    return d


@pytest.mark.parametrize("cus", [1, 3, 8])
@pytest.mark.parametrize("kind,args", SMALL_GRID_CASES)
def test_small_grids(dev, kind, args, cus):
    _say(f"small grid {kind} {args} cus={cus}")
    if kind == "dense":
        w = synth.make_dense(args["m"], args["n"], args["k"], seed=args["k"], device=dev)
    elif kind == "contiguous":
        w = synth.make_contiguous(args["rows"], args["n"], args["k"], seed=args["k"], device=dev, poison_padding=True)
    elif kind == "nopad":
        w = synth.make_nopad(args["rows"], args["n"], args["k"], seed=args["k"], device=dev, tail=5, poison_tail=True)
    elif kind == "k_grouped":
        w = synth.make_k_grouped(args["ks"], args["m"], args["n"], seed=args["m"], device=dev)
    else:
        w = synth.make_contiguous(args["rows"], args["n"], args["k"], seed=args["k"], device=dev,
                                  poison_padding=True, fp4=True)
    ref = _small_grid_run(kind, w)
    dg.set_num_cus(cus)
    try:
        d = _small_grid_run(kind, w)
    finally:
        dg.set_num_cus(0)
    what = f"small grid {kind} cus={cus}"
    if kind == "k_grouped":
        assert torch.equal(d, ref), f"{what}: differs from the default grid"
        _check_k_grouped(w, d, None, what)
        return
    assert torch.equal(d.view(torch.int16), ref.view(torch.int16)), f"{what}: differs from the default grid"
    if kind == "dense":
        r, mag = _dense_ref(NP(w.a), NP(w.sfa), NP(w.b), NP(w.sfb))
        check_close(NP(d), r, what, mag, w.k)
    elif kind == "contiguous":
        _check_contiguous(w, d, what)
    elif kind == "nopad":
        _check_nopad(w, d, what)
    else:
        got, owner = NP(d), O.contiguous_row_groups(NP(w.layout), w.num_groups)
        for g in range(w.num_groups):
            idx = np.nonzero(owner == g)[0]
            if idx.size:
                _check_fp4(got[idx], _fp4_ref_rows(w, g, idx, np.arange(w.n)), f"{what} group {g}", w.k)
        check_untouched(got[owner < 0], what + " padding rows")


# ---------------------------------------------------------------------------
# Graph capture of every other entry point: one captured call, replayed three
# times with new operand values copied in between and eager work between the
# replays; every replay must equal an eager call bit for bit.
# ---------------------------------------------------------------------------

def _graph_case(kind, dev):
    """(workload, a function that launches the call writing into d)."""
    if kind == "dense":
        w = synth.make_dense(300, 384, 1024, seed=41, device=dev)
        return w, lambda d: dg.fp8_gemm_nt(w.a, w.sfa, w.b, w.sfb, d)
    if kind == "dense_ue8m0":
        w = synth.make_dense(300, 384, 4096, seed=42, device=dev, ue8m0=True)
        return w, lambda d: dg.fp8_gemm_nt(w.a, w.sfa, w.b, w.sfb, d, ue8m0=True)
    if kind == "contiguous":
        w = synth.make_contiguous([130, 0, 77, 256, 1], 256, 512, seed=43, device=dev)
        return w, lambda d: dg.m_grouped_fp8_gemm_nt_contiguous(w.a, w.sfa, w.b, w.sfb, d, w.layout)
    if kind == "k_grouped":
        w = synth.make_k_grouped([128, 0, 384, 256], 300, 384, seed=44, device=dev)
        c = torch.randn(w.num_groups, w.m, w.n, device=dev)
        return w, lambda d: dg.k_grouped_fp8_gemm_nt_contiguous(w.a, w.sfa, w.b, w.sfb, d, w.ks, c=c)
    if kind == "w4a8_contiguous":
        w = synth.make_contiguous([130, 0, 77, 256, 1], 256, 512, seed=45, device=dev, fp4=True)
        return w, lambda d: dg.m_grouped_fp8_fp4_gemm_nt_contiguous(w.a, w.sfa, w.b, w.sfb, d, w.layout)
    w = synth.make_masked([40, 100, 7, 64], 128, 256, 512, seed=46, device=dev, fp4=True)
    return w, lambda d: dg.m_grouped_fp8_fp4_gemm_nt_masked(w.a, w.sfa, w.b, w.sfb, d, w.masked_m)


@pytest.mark.parametrize("kind", ["dense", "dense_ue8m0", "contiguous", "k_grouped", "w4a8_contiguous",
                                  "w4a8_masked"])
def test_graph_replay_every_entry_point(dev, kind):
    _say(f"graph replay {kind}")
    w, call = _graph_case(kind, dev)
    d = w.new_output()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        call(d)  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(d)
    gen = torch.Generator(device=dev)
    for rep in range(3):
        # new A values (same scales, so the codes stay valid E4M3 values)
        gen.manual_seed(100 + rep)
        perm = torch.randperm(w.a.shape[-1], device=dev, generator=gen)
        a8 = w.a.view(torch.uint8)
        a8.copy_(a8[..., perm].clone())
        (d.view(torch.int16) if d.dtype == torch.bfloat16 else d).fill_(-1)
        graph.replay()
        torch.cuda.synchronize()
        d_eager = w.new_output()
        call(d_eager)
        torch.cuda.synchronize()
        if d.dtype == torch.bfloat16:
            assert torch.equal(d.view(torch.int16), d_eager.view(torch.int16)), f"{kind} replay {rep}"
        else:
            assert torch.equal(d, d_eager), f"{kind} replay {rep}"


def test_concurrent_streams(dev):
    """Two calls in flight at once on two streams (a dense GEMM and a masked
    one; their persistent grids compete for the CUs): each result equals the
    same call made alone, bit for bit. The library keeps no state between
    calls apart from the CU-count setting."""
    wd = synth.make_dense(1000, 1024, 2048, seed=51, device=dev)
    wm = synth.make_masked([200, 17, 256, 0, 99], 256, 1024, 2048, seed=52, device=dev)
    dd, dm = wd.new_output(), wm.new_output()
    dg.fp8_gemm_nt(wd.a, wd.sfa, wd.b, wd.sfb, dd)
    dg.m_grouped_fp8_gemm_nt_masked(wm.a, wm.sfa, wm.b, wm.sfb, dm, wm.masked_m)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        d1, d2 = wd.new_output(), wm.new_output()
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            dg.fp8_gemm_nt(wd.a, wd.sfa, wd.b, wd.sfb, d1)
        with torch.cuda.stream(s2):
            dg.m_grouped_fp8_gemm_nt_masked(wm.a, wm.sfa, wm.b, wm.sfb, d2, wm.masked_m)
        torch.cuda.synchronize()
        assert torch.equal(d1.view(torch.int16), dd.view(torch.int16)), f"dense, round {rep}"
        assert torch.equal(d2.view(torch.int16), dm.view(torch.int16)), f"masked, round {rep}"


@pytest.mark.parametrize("m,n,k", [(64, 128, 262144), (130, 256, 65536)])
def test_dense_long_k(dev, m, n, k):
    """2048 and 512 K blocks: long K loops of the deep-prefetch pipeline and
    large row strides, against the oracle with the per-element bound at that
    many promotions."""
    _say(f"dense long K {m}x{n}x{k}")
    w = synth.make_dense(m, n, k, seed=53, device=dev)
    d = w.new_output()
    dg.fp8_gemm_nt(w.a, w.sfa, w.b, w.sfb, d)
    torch.cuda.synchronize()
    ref, mag = _dense_ref(NP(w.a), NP(w.sfa), NP(w.b), NP(w.sfb))
    check_close(NP(d), ref, f"dense long K {m}x{n}x{k}", mag, k)


# ---------------------------------------------------------------------------
# Seeded random shapes: every layout and scale format on shapes drawn from a
# fixed generator -- M, row counts and masked counts from 0 or 1 to a few
# hundred, N a multiple of 128 up to 1152, K from one 128-K block to 40 (both
# pipelines: the deep one from 32 blocks) -- each compared in full with the
# oracle. The draw is fixed, so every run checks the same shapes.
# ---------------------------------------------------------------------------

RANDOM_K_BLOCKS = [1, 2, 3, 5, 8, 16, 31, 32, 40]


def _random_cases(kind, count):
    rng = np.random.default_rng([2027, len(kind)] + [ord(ch) for ch in kind])
    cases = []
    for i in range(count):
        n = 128 * int(rng.integers(1, 10))
        k = 128 * int(rng.choice(RANDOM_K_BLOCKS))
        groups = int(rng.integers(1, 7))
        ue8m0 = i % 3 == 2
        fp4 = kind.startswith("w4a8")  # W4A8 reads every scale as E8M0: no flag
        if kind == "dense":
            cases.append((int(rng.integers(1, 700)), n, k, ue8m0))
        elif kind in ("contiguous", "w4a8_contiguous"):
            rows = [int(x) for x in rng.integers(0, 301, groups)]
            cases.append((rows, n, k) if fp4 else (rows, n, k, ue8m0))
        elif kind == "nopad":
            rows = [int(x) for x in rng.integers(0, 301, groups)]
            cases.append((rows, n, k, int(rng.integers(0, 11)), ue8m0))
        elif kind in ("masked", "w4a8_masked"):
            max_m = int(rng.integers(1, 301))
            counts = [int(x) for x in rng.integers(0, max_m + 1, groups)]
            cases.append((counts, max_m, n, k) if fp4 else (counts, max_m, n, k, ue8m0))
        elif kind == "k_grouped":
            ks = [128 * int(x) for x in rng.integers(0, 13, groups)]
            cases.append((ks, int(rng.integers(1, 401)), n, ("none", "separate", "in_place")[i % 3], ue8m0))
    return cases


def _e8(w, arr):
    return O.e8m0_value(arr) if w.ue8m0 else arr


@pytest.mark.parametrize("m,n,k,ue8m0", _random_cases("dense", 16))
def test_random_dense(dev, m, n, k, ue8m0):
    _say(f"random dense {m}x{n}x{k} ue8m0={ue8m0}")
    w = synth.make_dense(m, n, k, seed=m * 7 + k, device=dev, ue8m0=ue8m0)
    d = w.new_output()
    dg.fp8_gemm_nt(w.a, w.sfa, w.b, w.sfb, d, ue8m0=ue8m0)
    torch.cuda.synchronize()
    ref, mag = _dense_ref(NP(w.a), _e8(w, NP(w.sfa)), NP(w.b), _e8(w, NP(w.sfb)))
    check_close(NP(d), ref, f"random dense {m}x{n}x{k}", mag, k)


@pytest.mark.parametrize("rows,n,k,ue8m0", _random_cases("contiguous", 12))
def test_random_contiguous(dev, rows, n, k, ue8m0):
    _say(f"random contiguous rows={rows} n={n} k={k} ue8m0={ue8m0}")
    w = synth.make_contiguous(rows, n, k, seed=sum(rows) + k, device=dev, poison_padding=True, ue8m0=ue8m0)
    d = w.new_output()
    dg.m_grouped_fp8_gemm_nt_contiguous(w.a, w.sfa, w.b, w.sfb, d, w.layout, ue8m0=ue8m0)
    torch.cuda.synchronize()
    _check_contiguous(w, d, f"random contiguous {rows}", _e8(w, NP(w.sfa)), _e8(w, NP(w.sfb)))


@pytest.mark.parametrize("counts,max_m,n,k,ue8m0", _random_cases("masked", 12))
def test_random_masked(dev, counts, max_m, n, k, ue8m0):
    _say(f"random masked counts={counts} max_m={max_m} n={n} k={k} ue8m0={ue8m0}")
    w = synth.make_masked(counts, max_m, n, k, seed=max_m + k, device=dev, poison_invalid=True, ue8m0=ue8m0)
    d = w.new_output()
    dg.m_grouped_fp8_gemm_nt_masked(w.a, w.sfa, w.b, w.sfb, d, w.masked_m, ue8m0=ue8m0)
    torch.cuda.synchronize()
    _check_masked(w, d, counts, f"random masked {counts}", _e8(w, NP(w.sfa)), _e8(w, NP(w.sfb)))


@pytest.mark.parametrize("rows,n,k,tail,ue8m0", _random_cases("nopad", 12))
def test_random_nopad(dev, rows, n, k, tail, ue8m0):
    _say(f"random nopad rows={rows} tail={tail} n={n} k={k} ue8m0={ue8m0}")
    w = synth.make_nopad(rows, n, k, seed=sum(rows) + tail + k, device=dev, tail=tail, poison_tail=True,
                         ue8m0=ue8m0)
    d = w.new_output()
    dg.m_grouped_fp8_gemm_nt_nopad(w.a, w.sfa, w.b, w.sfb, d, w.group_rows, ue8m0=ue8m0)
    torch.cuda.synchronize()
    _check_nopad(w, d, f"random nopad {rows}", _e8(w, NP(w.sfa)), _e8(w, NP(w.sfb)))


@pytest.mark.parametrize("ks,m,n,c_mode,ue8m0", _random_cases("k_grouped", 12))
def test_random_k_grouped(dev, ks, m, n, c_mode, ue8m0):
    _say(f"random k_grouped ks={ks} m={m} n={n} c={c_mode} ue8m0={ue8m0}")
    if sum(ks) == 0:
        ks = ks[:-1] + [128]   # K = 0 is rejected; keep the case
    w = synth.make_k_grouped(ks, m, n, seed=m + sum(ks), device=dev, ue8m0=ue8m0)
    d = w.new_output()
    c0 = None if c_mode == "none" else d.clone()
    if c_mode == "none":
        d.fill_(float("nan"))
        dg.k_grouped_fp8_gemm_nt_contiguous(w.a, w.sfa, w.b, w.sfb, d, w.ks, ue8m0=ue8m0)
    elif c_mode == "separate":
        out = torch.full_like(d, float("nan"))
        dg.k_grouped_fp8_gemm_nt_contiguous(w.a, w.sfa, w.b, w.sfb, out, w.ks, c=d, ue8m0=ue8m0)
        torch.cuda.synchronize()
        assert torch.equal(d, c0), "C was modified"
        d = out
    else:
        dg.k_grouped_fp8_gemm_nt_contiguous(w.a, w.sfa, w.b, w.sfb, d, w.ks, c=d, ue8m0=ue8m0)
    torch.cuda.synchronize()
    _check_k_grouped(w, d, c0, f"random k_grouped {ks} {c_mode}")


@pytest.mark.parametrize("rows,n,k", _random_cases("w4a8_contiguous", 8))
def test_random_fp8_fp4_contiguous(dev, rows, n, k):
    _say(f"random w4a8 contiguous rows={rows} n={n} k={k}")
    w = synth.make_contiguous(rows, n, k, seed=sum(rows) + k + 1, device=dev, poison_padding=True, fp4=True)
    d = w.new_output()
    dg.m_grouped_fp8_fp4_gemm_nt_contiguous(w.a, w.sfa, w.b, w.sfb, d, w.layout)
    torch.cuda.synchronize()
    got, owner = NP(d), O.contiguous_row_groups(NP(w.layout), w.num_groups)
    for g in range(w.num_groups):
        idx = np.nonzero(owner == g)[0]
        if idx.size:
            _check_fp4(got[idx], _fp4_ref_rows(w, g, idx, np.arange(w.n)), f"random w4a8 contiguous group {g}", k)
    check_untouched(got[owner < 0], "random w4a8 contiguous padding rows")


@pytest.mark.parametrize("counts,max_m,n,k", _random_cases("w4a8_masked", 8))
def test_random_fp8_fp4_masked(dev, counts, max_m, n, k):
    _say(f"random w4a8 masked counts={counts} max_m={max_m} n={n} k={k}")
    w = synth.make_masked(counts, max_m, n, k, seed=max_m + k + 1, device=dev, poison_invalid=True, fp4=True)
    d = w.new_output()
    dg.m_grouped_fp8_fp4_gemm_nt_masked(w.a, w.sfa, w.b, w.sfb, d, w.masked_m)
    torch.cuda.synchronize()
    got = NP(d)
    for g, c in enumerate(counts):
        v = min(max(int(c), 0), max_m)
        if v:
            _check_fp4(got[g, :v], _fp4_ref_rows(w, g, np.arange(v), np.arange(n), NP(w.a)[g], NP(w.sfa)[g]),
                       f"random w4a8 masked group {g}", k)
        check_untouched(got[g, v:], f"random w4a8 masked group {g} rows >= {v}")


# ---------------------------------------------------------------------------
# The benchmark workloads at full size: every valid element
# ---------------------------------------------------------------------------
#
# The oracle runs group by group in chunks of rows: each group's RHS is
# dequantised once (dequant_rhs, or dequant_rhs_e2m1 for FP4), each chunk's
# LHS rows with dequant_lhs, and the float64 products give the reference and
# the magnitudes for the per-element bound. Every row no group owns is
# checked against the sentinel.

ROW_CHUNK = 2048


def _check_rows_full(got, a, sfa_v, bhat, rows, k, what):
    babs = np.abs(bhat)
    for i in range(0, rows.size, ROW_CHUNK):
        r = rows[i:i + ROW_CHUNK]
        ahat = O.dequant_lhs(a[r], sfa_v[:, r])
        check_close(got[r], ahat @ bhat.T, f"{what} rows {r[0]}..{r[-1]}", np.abs(ahat) @ babs.T, k)


def _rhs(w, g, sfb_v):
    b = NP(w.b)
    if getattr(w, "fp4", False):
        return O.dequant_rhs_e2m1(b[g], sfb_v[g])
    return O.dequant_rhs(b[g], sfb_v[g])


@pytest.mark.parametrize("index", list(range(synth.NUM_WORKLOADS)))
def test_workload_full_size(dev, index):
    spec = synth.workload_spec(index)
    _say(f"workload {index} {spec.name}")
    w = synth.make_workload(spec, seed=0, device=dev)
    d = w.new_output()
    c0 = d.clone() if spec.kind == "k_grouped" else None
    dg.run_workload(w, d)
    torch.cuda.synchronize()
    if spec.kind == "k_grouped":
        _check_k_grouped(w, d, c0, spec.name)
        return
    got = NP(d)
    a, sfa, sfb = NP(w.a), NP(w.sfa), NP(w.sfb)
    fp4 = getattr(w, "fp4", False)
    # The W4A8 calls read every scale as E8M0, as do the *_ue8m0 calls; the
    # FP4 RHS scales are decoded inside dequant_rhs_e2m1.
    sfa_v = O.e8m0_value(sfa) if (w.ue8m0 or fp4) else sfa
    sfb_v = O.e8m0_value(sfb) if (w.ue8m0 and not fp4) else sfb
    k = w.k
    if spec.kind == "dense":
        _check_rows_full(got, a, sfa_v, O.dequant_rhs(NP(w.b), sfb_v), np.arange(w.m), k, spec.name)
    elif spec.kind == "contiguous":
        owner = O.contiguous_row_groups(NP(w.layout), w.num_groups)
        for g in range(w.num_groups):
            rows = np.nonzero(owner == g)[0]
            if rows.size:
                _say(f"  group {g}: {rows.size} rows")
                _check_rows_full(got, a, sfa_v, _rhs(w, g, sfb_v), rows, k, f"{spec.name} group {g}")
        check_untouched(got[owner < 0], spec.name + " padding rows")
    elif spec.kind == "nopad":
        owned = np.zeros(w.m, bool)
        for g, (first, end) in enumerate(O.nopad_row_ranges(NP(w.group_rows), w.m)):
            if end > first:
                _say(f"  group {g}: rows {first}..{end - 1}")
                _check_rows_full(got, a, sfa_v, _rhs(w, g, sfb_v), np.arange(first, end), k, f"{spec.name} group {g}")
                owned[first:end] = True
        check_untouched(got[~owned], spec.name + " rows no group owns")
    else:
        for g in range(w.num_groups):
            v = min(max(int(w.counts[g]), 0), w.max_m)
            if v:
                _check_rows_full(got[g], a[g], sfa_v[g], _rhs(w, g, sfb_v), np.arange(v), k,
                                 f"{spec.name} group {g}")
            check_untouched(got[g, v:], f"{spec.name} group {g} rows >= {v}")
