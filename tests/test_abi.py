"""C-ABI checks that need no GPU: libdg.so loads, exports every function
include/dg.h declares, and rejects invalid arguments before enqueueing
anything (the pointers below are never dereferenced)."""

import ctypes
import os
import re

import pytest

from moe_grouped_gemm_amd import dg

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADERS = sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h"))

A = 0x10000        # fake 16-byte aligned "device" addresses
B = 0x20000
SFA = 0x30000
SFB = 0x40000
D = 0x50000
AUX = 0x60000


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b(dg_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    lib = dg.lib()
    names = declared_functions()
    assert len(names) == 18, names
    for name in names:
        assert hasattr(lib, name), name
    assert sorted(n for n, _, _ in dg.SIGNATURES) == names


def test_helpers():
    assert dg.get_mk_alignment_for_contiguous_layout() == 128
    assert dg.get_tma_aligned_size(0, 4) == 0
    assert dg.get_tma_aligned_size(1, 4) == 4
    assert dg.get_tma_aligned_size(4097, 4) == 4100
    assert dg.get_tma_aligned_size(5, 2) == 8
    assert dg.get_tma_aligned_size(17, 1) == 32
    assert dg.lib().dg_get_tma_aligned_size(-1, 4) == -1
    assert dg.lib().dg_get_tma_aligned_size(3, 3) == -1
    for s in range(7):
        assert dg.lib().dg_status_string(s)


def _dense(a=A, sfa=SFA, b=B, sfb=SFB, d=D, m=256, n=256, k=512):
    return dg.lib().dg_fp8_gemm_nt(a, sfa, b, sfb, d, m, n, k, None)


def _contig(a=A, sfa=SFA, b=B, sfb=SFB, d=D, lay=AUX, m=256, n=256, k=512, g=2):
    return dg.lib().dg_m_grouped_fp8_gemm_nt_contiguous(a, sfa, b, sfb, d, lay, m, n, k, g, None)


def _masked(a=A, sfa=SFA, b=B, sfb=SFB, d=D, mm=AUX, g=2, max_m=64, n=256, k=512):
    return dg.lib().dg_m_grouped_fp8_gemm_nt_masked(a, sfa, b, sfb, d, mm, g, max_m, n, k, None)


def _nopad(a=A, sfa=SFA, b=B, sfb=SFB, d=D, rows=AUX, m=256, n=256, k=512, g=2):
    return dg.lib().dg_m_grouped_fp8_gemm_nt_nopad(a, sfa, b, sfb, d, rows, m, n, k, g, None)


CALLS = [_dense, _contig, _masked, _nopad]


@pytest.mark.parametrize("call", CALLS)
def test_null_pointers(call):
    for arg in ("a", "sfa", "b", "sfb", "d"):
        assert call(**{arg: None}) == 1
    if call is _contig:
        assert call(lay=None) == 1
    if call is _masked:
        assert call(mm=None) == 1
    if call is _nopad:
        assert call(rows=None) == 1


@pytest.mark.parametrize("call", CALLS)
def test_shapes(call):
    assert call(n=0) == 2
    assert call(n=-128) == 2
    assert call(n=192) == 2          # n % 128
    assert call(k=0) == 2
    assert call(k=200) == 2          # k % 128
    assert call(n=1 << 21) == 4      # beyond the limits
    assert call(k=1 << 21) == 4


def test_dense_shapes():
    assert _dense(m=-1) == 2
    assert _dense(m=0) == 0          # empty: a successful no-op


def test_contiguous_shapes():
    assert _contig(m=-128) == 2
    assert _contig(m=130) == 2       # segments are 128-row aligned
    assert _contig(g=-1) == 2
    assert _contig(m=0) == 0
    assert _contig(g=0) == 0


def test_masked_shapes():
    assert _masked(max_m=0) == 2
    assert _masked(g=-1) == 2
    assert _masked(g=4097) == 4
    assert _masked(g=0) == 0


def test_nopad_shapes():
    assert _nopad(m=-1) == 2
    assert _nopad(g=-1) == 2
    assert _nopad(g=2049) == 4
    assert _nopad(m=0) == 0          # empty: successful no-ops
    assert _nopad(g=0) == 0


@pytest.mark.parametrize("call", CALLS)
def test_alignment(call):
    for arg, val in (("a", A + 8), ("b", B + 4), ("d", D + 2), ("sfa", SFA + 4), ("sfb", SFB + 8)):
        assert call(**{arg: val}) == 3


def test_ue8m0_variants_share_the_checks():
    lib = dg.lib()
    calls = {
        "dense": lambda **kw: lib.dg_fp8_gemm_nt_ue8m0(kw.get("a", A), SFA, B, SFB, D, 256, kw.get("n", 256), 512,
                                                        None),
        "contiguous": lambda **kw: lib.dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(
            kw.get("a", A), SFA, B, SFB, D, AUX, 256, kw.get("n", 256), 512, 2, None),
        "masked": lambda **kw: lib.dg_m_grouped_fp8_gemm_nt_masked_ue8m0(
            kw.get("a", A), SFA, B, SFB, D, AUX, 2, 64, kw.get("n", 256), 512, None),
        "nopad": lambda **kw: lib.dg_m_grouped_fp8_gemm_nt_nopad_ue8m0(
            kw.get("a", A), SFA, B, SFB, D, AUX, 256, kw.get("n", 256), 512, 2, None),
    }
    for name, call in calls.items():
        assert call(a=None) == 1, name
        assert call(a=A + 8) == 3, name
        assert call(n=192) == 2, name


def test_fp8_fp4_checks():
    lib = dg.lib()
    contig = lambda **kw: lib.dg_m_grouped_fp8_fp4_gemm_nt_contiguous(
        kw.get("a", A), SFA, B, SFB, D, kw.get("lay", AUX), kw.get("m", 256), kw.get("n", 256), kw.get("k", 512),
        2, None)
    masked = lambda **kw: lib.dg_m_grouped_fp8_fp4_gemm_nt_masked(
        kw.get("a", A), SFA, B, SFB, D, kw.get("lay", AUX), kw.get("g", 2), 64, kw.get("n", 256), kw.get("k", 512),
        None)
    for call in (contig, masked):
        assert call(a=None) == 1
        assert call(lay=None) == 1
        assert call(a=A + 8) == 3
        assert call(n=192) == 2
        assert call(k=200) == 2
    assert contig(m=130) == 2
    assert contig(m=0) == 0
    assert masked(g=4097) == 4
    assert masked(g=0) == 0


def test_k_grouped_checks():
    import ctypes
    lib = dg.lib()

    def call(a=A, c=None, d=D, ks=(128, 256), g=None, m=256, n=256):
        arr = (ctypes.c_int * max(len(ks), 1))(*ks)
        return lib.dg_k_grouped_fp8_gemm_nt_contiguous(a, SFA, B, SFB, c, d, arr, len(ks) if g is None else g,
                                                       m, n, None)
    assert call(a=None) == 1
    assert call(d=None) == 1
    assert lib.dg_k_grouped_fp8_gemm_nt_contiguous(A, SFA, B, SFB, None, D, None, 2, 256, 256, None) == 1
    assert call(ks=(), g=0) == 2         # an empty K-size list is rejected
    assert call(ks=(100, 128)) == 2      # K sizes are multiples of 128
    assert call(ks=(-128, 256)) == 2
    assert call(n=192) == 2
    assert call(m=-1) == 2
    assert call(ks=(1 << 20, 128)) == 4  # total K beyond the limit
    assert call(ks=(128,) * 513) == 4    # more than 512 groups
    assert call(c=D + 4) == 3
    assert call(a=A + 8) == 3
    assert call(m=0) == 0                # empty: a successful no-op


def test_no_device_reported_without_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert dg.get_num_cus() == 0
    assert _dense() == 6             # valid arguments, no device: nothing enqueued


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(dg, "_lib", None)
    monkeypatch.setattr(dg, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        dg.lib()
