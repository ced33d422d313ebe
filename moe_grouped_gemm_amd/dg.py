"""Python binding of libdg.so: the FP8 NT GEMM and its M-grouped variants.

Argument marshalling only: each function checks tensor dtypes, shapes,
devices and contiguity, then passes raw device pointers and the current HIP
stream to the C ABI declared in include/dg.h. All arithmetic runs in the
library's gfx950 kernels. There is no fallback: a missing library raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdg.so")

DG_OK = 0
_STATUS_NAMES = {0: "DG_OK", 1: "DG_ERR_NULL", 2: "DG_ERR_SHAPE", 3: "DG_ERR_ALIGN",
                 4: "DG_ERR_UNSUPPORTED", 5: "DG_ERR_LAUNCH", 6: "DG_ERR_DEVICE"}

# (name, argtypes, restype) of every symbol include/dg.h and include/dg_ceiling.h declare.
_vp, _i = ctypes.c_void_p, ctypes.c_int
SIGNATURES = [
    ("dg_fp8_gemm_nt", [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _vp], _i),
    ("dg_m_grouped_fp8_gemm_nt_contiguous", [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp], _i),
    ("dg_m_grouped_fp8_gemm_nt_masked", [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp], _i),
    ("dg_m_grouped_fp8_gemm_nt_nopad", [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp], _i),
    ("dg_fp8_gemm_nt_ue8m0", [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _vp], _i),
    ("dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0", [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp], _i),
    ("dg_m_grouped_fp8_gemm_nt_masked_ue8m0", [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp], _i),
    ("dg_m_grouped_fp8_gemm_nt_nopad_ue8m0", [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp], _i),
    ("dg_m_grouped_fp8_fp4_gemm_nt_contiguous", [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp], _i),
    ("dg_m_grouped_fp8_fp4_gemm_nt_masked", [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp], _i),
    ("dg_k_grouped_fp8_gemm_nt_contiguous", [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.POINTER(_i), _i, _i, _i, _vp], _i),
    ("dg_k_grouped_fp8_gemm_nt_contiguous_ue8m0", [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.POINTER(_i), _i, _i, _i, _vp],
     _i),
    ("dg_get_mk_alignment_for_contiguous_layout", [], _i),
    ("dg_get_tma_aligned_size", [_i, _i], _i),
    ("dg_get_num_cus", [], _i),
    ("dg_set_num_cus", [_i], _i),
    ("dg_status_string", [_i], ctypes.c_char_p),
    ("dg_mfma_fp8_ceiling", [_vp, _vp, _i, _i, ctypes.POINTER(ctypes.c_longlong), _vp], _i),
]

_lib: Optional[ctypes.CDLL] = None


class DGError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = lib().dg_status_string(status).decode()
        super().__init__(f"{what}: {_STATUS_NAMES.get(status, status)} ({msg})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library (loaded on first use; raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m moe_grouped_gemm_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, argtypes, restype in SIGNATURES:
            fn = getattr(handle, name)
            fn.argtypes = argtypes
            fn.restype = restype
        _lib = handle
    return _lib


def _entry(name: str, ue8m0: bool):
    """The C entry point `name`, or its power-of-two-scale variant."""
    return getattr(lib(), name + "_ue8m0" if ue8m0 else name)


def _check(status: int, what: str) -> None:
    if status != DG_OK:
        raise DGError(status, what)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype, ndim: int, device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ---------------------------------------------------------------------------
# Utilities (include/dg.h)
# ---------------------------------------------------------------------------

def get_mk_alignment_for_contiguous_layout() -> int:
    return lib().dg_get_mk_alignment_for_contiguous_layout()


def get_tma_aligned_size(x: int, element_size: int) -> int:
    r = lib().dg_get_tma_aligned_size(int(x), int(element_size))
    if r < 0:
        raise ValueError(f"bad arguments ({x}, {element_size})")
    return r


def get_num_cus() -> int:
    return lib().dg_get_num_cus()


def set_num_cus(n: int) -> None:
    _check(lib().dg_set_num_cus(int(n)), "dg_set_num_cus")


# The names the pages give these helpers ("DeepGEMM for PPU" README,
# "Utilities"): the persistent grid's width counts compute units here.
get_num_sms = get_num_cus
set_num_sms = set_num_cus


def get_mn_major_tma_aligned_tensor(sf: torch.Tensor) -> torch.Tensor:
    """Lays out LHS scales [..., M, K/128] (float32) transposed with an aligned
    leading dimension: [..., K/128, tma_aligned(M)], the layout the kernels
    read. Padding entries are zero. (A layout helper; no GEMM arithmetic.)"""
    *lead, m, kb = sf.shape
    ld = get_tma_aligned_size(m, 4)
    out = torch.zeros(*lead, kb, ld, dtype=torch.float32, device=sf.device)
    out[..., :m] = sf.transpose(-1, -2)
    return out


# The older name of the same helper, which the MATE wrapper page still lists
# among the re-exported utilities.
get_col_major_tma_aligned_tensor = get_mn_major_tma_aligned_tensor


# ---------------------------------------------------------------------------
# The GEMMs
# ---------------------------------------------------------------------------

def fp8_gemm_nt(a, sfa, b, sfb, d, ue8m0: bool = False) -> torch.Tensor:
    """d[m, n] = bf16(sum_k a[m,k] sfa[k/128][m] * b[n,k] sfb[n/128][k/128]).

    a [M, K] float8_e4m3fn, sfa [K/128, tma_aligned(M)] float32,
    b [N, K] float8_e4m3fn, sfb [N/128, K/128] float32, d [M, N] bfloat16.
    ue8m0=True calls the power-of-two-scale variant (each scale used as 2 to
    the power of its exponent field, applied by the matrix cores); the same
    flag exists on every GEMM below.
    """
    dev = a.device
    m, k = a.shape
    n = b.shape[0]
    _need(a, "a", torch.float8_e4m3fn, 2, dev)
    _need(b, "b", torch.float8_e4m3fn, 2, dev)
    _need(sfa, "sfa", torch.float32, 2, dev)
    _need(sfb, "sfb", torch.float32, 2, dev)
    _need(d, "d", torch.bfloat16, 2, dev)
    if b.shape[1] != k or tuple(d.shape) != (m, n):
        raise ValueError("shape mismatch between a, b and d")
    if k % 128 or n % 128:
        raise ValueError("k and n must be multiples of 128")
    if tuple(sfa.shape) != (k // 128, get_tma_aligned_size(m, 4)) or tuple(sfb.shape) != (n // 128, k // 128):
        raise ValueError("scale shapes do not match the (1, 128, 128) recipe layout")
    _check(_entry("dg_fp8_gemm_nt", ue8m0)(a.data_ptr(), sfa.data_ptr(), b.data_ptr(), sfb.data_ptr(), d.data_ptr(),
                                m, n, k, _stream(a)), "dg_fp8_gemm_nt")
    return d


def m_grouped_fp8_gemm_nt_contiguous(a, sfa, b, sfb, d, grouped_layout, ue8m0: bool = False) -> torch.Tensor:
    """Contiguous-layout grouped GEMM; grouped_layout [M] int32 holds each
    row's group (-1 for padding). b [G, N, K], sfb [G, N/128, K/128]."""
    dev = a.device
    m, k = a.shape
    g, n, _ = b.shape
    _need(a, "a", torch.float8_e4m3fn, 2, dev)
    _need(b, "b", torch.float8_e4m3fn, 3, dev)
    _need(sfa, "sfa", torch.float32, 2, dev)
    _need(sfb, "sfb", torch.float32, 3, dev)
    _need(d, "d", torch.bfloat16, 2, dev)
    _need(grouped_layout, "grouped_layout", torch.int32, 1, dev)
    if b.shape[2] != k or tuple(d.shape) != (m, n) or grouped_layout.shape[0] != m:
        raise ValueError("shape mismatch between a, b, d and grouped_layout")
    if tuple(sfa.shape) != (k // 128, get_tma_aligned_size(m, 4)) or tuple(sfb.shape) != (g, n // 128, k // 128):
        raise ValueError("scale shapes do not match the (1, 128, 128) recipe layout")
    _check(_entry("dg_m_grouped_fp8_gemm_nt_contiguous", ue8m0)(
        a.data_ptr(), sfa.data_ptr(), b.data_ptr(), sfb.data_ptr(), d.data_ptr(), grouped_layout.data_ptr(),
        m, n, k, g, _stream(a)), "dg_m_grouped_fp8_gemm_nt_contiguous")
    return d


def m_grouped_fp8_gemm_nt_masked(a, sfa, b, sfb, d, masked_m, ue8m0: bool = False) -> torch.Tensor:
    """Masked-layout grouped GEMM; masked_m [G] int32 (device) holds each
    group's valid rows. a [G, max_m, K], sfa [G, K/128, tma_aligned(max_m)],
    b [G, N, K], sfb [G, N/128, K/128], d [G, max_m, N]."""
    dev = a.device
    g, max_m, k = a.shape
    n = b.shape[1]
    _need(a, "a", torch.float8_e4m3fn, 3, dev)
    _need(b, "b", torch.float8_e4m3fn, 3, dev)
    _need(sfa, "sfa", torch.float32, 3, dev)
    _need(sfb, "sfb", torch.float32, 3, dev)
    _need(d, "d", torch.bfloat16, 3, dev)
    _need(masked_m, "masked_m", torch.int32, 1, dev)
    if b.shape[0] != g or b.shape[2] != k or tuple(d.shape) != (g, max_m, n) or masked_m.shape[0] != g:
        raise ValueError("shape mismatch between a, b, d and masked_m")
    if (tuple(sfa.shape) != (g, k // 128, get_tma_aligned_size(max_m, 4))
            or tuple(sfb.shape) != (g, n // 128, k // 128)):
        raise ValueError("scale shapes do not match the (1, 128, 128) recipe layout")
    _check(_entry("dg_m_grouped_fp8_gemm_nt_masked", ue8m0)(
        a.data_ptr(), sfa.data_ptr(), b.data_ptr(), sfb.data_ptr(), d.data_ptr(), masked_m.data_ptr(),
        g, max_m, n, k, _stream(a)), "dg_m_grouped_fp8_gemm_nt_masked")
    return d


def m_grouped_fp8_gemm_nt_nopad(a, sfa, b, sfb, d, group_rows, ue8m0: bool = False) -> torch.Tensor:
    """No-padding grouped GEMM; group_rows [G] int32 (device) holds each
    group's row count, the groups' rows following one another from row 0 of
    a with no alignment padding. a [M, K], sfa [K/128, tma_aligned(M)],
    b [G, N, K], sfb [G, N/128, K/128], d [M, N]."""
    dev = a.device
    m, k = a.shape
    g, n, _ = b.shape
    _need(a, "a", torch.float8_e4m3fn, 2, dev)
    _need(b, "b", torch.float8_e4m3fn, 3, dev)
    _need(sfa, "sfa", torch.float32, 2, dev)
    _need(sfb, "sfb", torch.float32, 3, dev)
    _need(d, "d", torch.bfloat16, 2, dev)
    _need(group_rows, "group_rows", torch.int32, 1, dev)
    if b.shape[2] != k or tuple(d.shape) != (m, n) or group_rows.shape[0] != g:
        raise ValueError("shape mismatch between a, b, d and group_rows")
    if tuple(sfa.shape) != (k // 128, get_tma_aligned_size(m, 4)) or tuple(sfb.shape) != (g, n // 128, k // 128):
        raise ValueError("scale shapes do not match the (1, 128, 128) recipe layout")
    _check(_entry("dg_m_grouped_fp8_gemm_nt_nopad", ue8m0)(
        a.data_ptr(), sfa.data_ptr(), b.data_ptr(), sfb.data_ptr(), d.data_ptr(), group_rows.data_ptr(),
        m, n, k, g, _stream(a)), "dg_m_grouped_fp8_gemm_nt_nopad")
    return d


def m_grouped_fp8_fp4_gemm_nt_contiguous(a, sfa, b, sfb, d, grouped_layout) -> torch.Tensor:
    """FP8 x FP4 (W4A8) contiguous-layout grouped GEMM: as the FP8 call, with
    b [G, N, K/2] uint8 (packed E2M1, element 2j in the low nibble of byte j)
    and sfb [G, K/32, tma_aligned(N)] float32; every scale is read as UE8M0."""
    dev = a.device
    m, k = a.shape
    g, n, kh = b.shape
    _need(a, "a", torch.float8_e4m3fn, 2, dev)
    _need(b, "b", torch.uint8, 3, dev)
    _need(sfa, "sfa", torch.float32, 2, dev)
    _need(sfb, "sfb", torch.float32, 3, dev)
    _need(d, "d", torch.bfloat16, 2, dev)
    _need(grouped_layout, "grouped_layout", torch.int32, 1, dev)
    if kh * 2 != k or tuple(d.shape) != (m, n) or grouped_layout.shape[0] != m:
        raise ValueError("shape mismatch between a, b, d and grouped_layout")
    if (tuple(sfa.shape) != (k // 128, get_tma_aligned_size(m, 4))
            or tuple(sfb.shape) != (g, k // 32, get_tma_aligned_size(n, 4))):
        raise ValueError("scale shapes do not match the (1, 128) x (1, 32) layout")
    _check(lib().dg_m_grouped_fp8_fp4_gemm_nt_contiguous(
        a.data_ptr(), sfa.data_ptr(), b.data_ptr(), sfb.data_ptr(), d.data_ptr(), grouped_layout.data_ptr(),
        m, n, k, g, _stream(a)), "dg_m_grouped_fp8_fp4_gemm_nt_contiguous")
    return d


def m_grouped_fp8_fp4_gemm_nt_masked(a, sfa, b, sfb, d, masked_m) -> torch.Tensor:
    """FP8 x FP4 (W4A8) masked-layout grouped GEMM: a [G, max_m, K],
    sfa [G, K/128, tma_aligned(max_m)], b [G, N, K/2] uint8 (packed E2M1),
    sfb [G, K/32, tma_aligned(N)], d [G, max_m, N]; every scale read as UE8M0."""
    dev = a.device
    g, max_m, k = a.shape
    n = b.shape[1]
    _need(a, "a", torch.float8_e4m3fn, 3, dev)
    _need(b, "b", torch.uint8, 3, dev)
    _need(sfa, "sfa", torch.float32, 3, dev)
    _need(sfb, "sfb", torch.float32, 3, dev)
    _need(d, "d", torch.bfloat16, 3, dev)
    _need(masked_m, "masked_m", torch.int32, 1, dev)
    if b.shape[0] != g or b.shape[2] * 2 != k or tuple(d.shape) != (g, max_m, n) or masked_m.shape[0] != g:
        raise ValueError("shape mismatch between a, b, d and masked_m")
    if (tuple(sfa.shape) != (g, k // 128, get_tma_aligned_size(max_m, 4))
            or tuple(sfb.shape) != (g, k // 32, get_tma_aligned_size(n, 4))):
        raise ValueError("scale shapes do not match the (1, 128) x (1, 32) layout")
    _check(lib().dg_m_grouped_fp8_fp4_gemm_nt_masked(
        a.data_ptr(), sfa.data_ptr(), b.data_ptr(), sfb.data_ptr(), d.data_ptr(), masked_m.data_ptr(),
        g, max_m, n, k, _stream(a)), "dg_m_grouped_fp8_fp4_gemm_nt_masked")
    return d


def k_grouped_fp8_gemm_nt_contiguous(a, sfa, b, sfb, d, ks, c=None, ue8m0: bool = False) -> torch.Tensor:
    """K-grouped GEMM (weight-gradient shape): for each group g,
    d[g] = (c[g] or 0) + A[:, K_g] . B[:, K_g]^T with per-row, per-128-K
    scales on both operands. a [M, K], sfa [K/128, tma_aligned(M)],
    b [N, K], sfb [K/128, tma_aligned(N)], d [G, M, N] float32; ks: the
    groups' K sizes as host integers (multiples of 128, summing to K);
    c: None, d itself (accumulate in place) or a separate [G, M, N] float32.
    ue8m0=True: power-of-two scales applied by the matrix cores."""
    dev = a.device
    m, k = a.shape
    n = b.shape[0]
    ks = [int(x) for x in ks]
    g = len(ks)
    _need(a, "a", torch.float8_e4m3fn, 2, dev)
    _need(b, "b", torch.float8_e4m3fn, 2, dev)
    _need(sfa, "sfa", torch.float32, 2, dev)
    _need(sfb, "sfb", torch.float32, 2, dev)
    _need(d, "d", torch.float32, 3, dev)
    if c is not None:
        _need(c, "c", torch.float32, 3, dev)
        if tuple(c.shape) != tuple(d.shape):
            raise ValueError("c and d shapes differ")
    if b.shape[1] != k or tuple(d.shape) != (g, m, n) or sum(ks) != k:
        raise ValueError("shape mismatch between a, b, d and ks")
    if (tuple(sfa.shape) != (k // 128, get_tma_aligned_size(m, 4))
            or tuple(sfb.shape) != (k // 128, get_tma_aligned_size(n, 4))):
        raise ValueError("scale shapes do not match the (1, 1, 128) recipe layout")
    ks_arr = (ctypes.c_int * max(g, 1))(*ks)
    _check(_entry("dg_k_grouped_fp8_gemm_nt_contiguous", ue8m0)(
        a.data_ptr(), sfa.data_ptr(), b.data_ptr(), sfb.data_ptr(), None if c is None else c.data_ptr(),
        d.data_ptr(), ks_arr, g, m, n, _stream(a)), "dg_k_grouped_fp8_gemm_nt_contiguous")
    return d


def run_workload(w, d: torch.Tensor) -> torch.Tensor:
    """Runs the GEMM that matches a synth workload (Dense / Contiguous /
    Masked / Nopad)."""
    kind = type(w).__name__
    e8 = getattr(w, "ue8m0", False)
    if getattr(w, "fp4", False):
        if kind == "Contiguous":
            return m_grouped_fp8_fp4_gemm_nt_contiguous(w.a, w.sfa, w.b, w.sfb, d, w.layout)
        return m_grouped_fp8_fp4_gemm_nt_masked(w.a, w.sfa, w.b, w.sfb, d, w.masked_m)
    if kind == "Dense":
        return fp8_gemm_nt(w.a, w.sfa, w.b, w.sfb, d, ue8m0=e8)
    if kind == "Contiguous":
        return m_grouped_fp8_gemm_nt_contiguous(w.a, w.sfa, w.b, w.sfb, d, w.layout, ue8m0=e8)
    if kind == "Masked":
        return m_grouped_fp8_gemm_nt_masked(w.a, w.sfa, w.b, w.sfb, d, w.masked_m, ue8m0=e8)
    if kind == "Nopad":
        return m_grouped_fp8_gemm_nt_nopad(w.a, w.sfa, w.b, w.sfb, d, w.group_rows, ue8m0=e8)
    if kind == "KGrouped":
        # the weight-gradient use: accumulate into d in place
        return k_grouped_fp8_gemm_nt_contiguous(w.a, w.sfa, w.b, w.sfb, d, w.ks, c=d, ue8m0=e8)
    raise TypeError(kind)
