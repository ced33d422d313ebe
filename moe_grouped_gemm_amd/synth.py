"""Seeded synthetic workloads for the FP8 NT GEMM and its M-grouped variants.

This module only makes inputs: N(0,1) float32 operands quantised to OCP E4M3
with one float32 scale per 1x128 LHS block and per 128x128 RHS block
(scale = max(amax, 1e-4) / 448), the M-major aligned LHS-scale layout, the
contiguous-layout row->group index, the masked-layout valid-row counts and
the no-padding layout's per-group row counts. It
holds none of the GEMM's arithmetic; the GPU path and the CPU oracle both take
its bytes as given.

Layouts (DeepGEMM for PPU README, "Interfaces > Notices" and "Utilities"):
  * a   [M, K] E4M3, K contiguous; b [N, K] E4M3 (the transposed RHS).
  * sfa [K/128, tma_aligned(M)] float32: the LHS scales transposed so that M
        is contiguous, with the leading dimension padded to 16 bytes.
  * sfb [N/128, K/128] float32.
Grouped variants add a leading group axis to b and sfb (and, for the masked
layout, to a, sfa and d).

Structural randomness (row counts, masked counts) comes from numpy's
default_rng([seed, 0]); operand values come from a torch generator seeded per
operand on the device where they are made.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

BLOCK = 128          # scale granularity along K (both operands) and N (RHS)
FP8_MAX = 448.0      # largest finite OCP E4M3 value
SCALE_FLOOR = 1e-4   # amax floor so that an all-zero block gets a finite scale
BF16_SENTINEL = 0xFFFF  # prefill pattern for outputs (a bfloat16 NaN)


def tma_aligned_size(x: int, element_size: int = 4) -> int:
    """Round x up so that x * element_size is a multiple of 16 bytes."""
    per16 = 16 // element_size
    return (x + per16 - 1) // per16 * per16


# ---------------------------------------------------------------------------
# Quantisation of float32 operands (input preparation, outside the GEMM)
# ---------------------------------------------------------------------------

def pow2_ceil(s: torch.Tensor) -> torch.Tensor:
    """The smallest power of two >= s (s > 0), exactly: the UE8M0 cast of a
    scale made at quantisation, so that x / scale stays within the E4M3 range."""
    mant, exp = torch.frexp(s)                 # s = mant * 2^exp, mant in [0.5, 1)
    return torch.ldexp(torch.ones_like(s), torch.where(mant == 0.5, exp - 1, exp))


def quantize_lhs(x: torch.Tensor, ue8m0: bool = False):
    """x float32 [M, K] -> (a float8_e4m3fn [M, K], sfa float32 [K/128, tma_aligned(M)]).
    ue8m0: scales rounded up to powers of two before quantising."""
    m, k = x.shape
    assert k % BLOCK == 0
    xb = x.view(m, k // BLOCK, BLOCK)
    scale = xb.abs().amax(dim=-1).clamp(min=SCALE_FLOOR) / FP8_MAX       # [M, K/128]
    if ue8m0:
        scale = pow2_ceil(scale)
    q = (xb / scale.unsqueeze(-1)).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    sfa = torch.zeros(k // BLOCK, tma_aligned_size(m), dtype=torch.float32, device=x.device)
    sfa[:, :m] = scale.t()
    return q.view(m, k), sfa


def quantize_rhs(x: torch.Tensor, ue8m0: bool = False):
    """x float32 [N, K] -> (b float8_e4m3fn [N, K], sfb float32 [N/128, K/128]).
    ue8m0: scales rounded up to powers of two before quantising."""
    n, k = x.shape
    assert n % BLOCK == 0 and k % BLOCK == 0
    xb = x.view(n // BLOCK, BLOCK, k // BLOCK, BLOCK)
    scale = xb.abs().amax(dim=(1, 3)).clamp(min=SCALE_FLOOR) / FP8_MAX   # [N/128, K/128]
    if ue8m0:
        scale = pow2_ceil(scale)
    q = (xb / scale[:, None, :, None]).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return q.view(n, k), scale.contiguous()


FP4_MAX = 6.0        # largest OCP E2M1 value
FP4_BLOCK = 32       # RHS scale granularity along K of the FP8 x FP4 GEMMs


def quantize_rhs_e2m1(x: torch.Tensor):
    """x float32 [N, K] -> (b uint8 [N, K/2]: OCP E2M1 codes packed two per
    byte, element 2j in the low nibble of byte j; sfb float32 [K/32,
    tma_aligned(N)]: one power-of-two scale per row and 32-wide K block,
    rounded up from amax / 6). Values round to the nearest E2M1 value, ties
    to the even code."""
    n, k = x.shape
    assert k % BLOCK == 0
    xb = x.view(n, k // FP4_BLOCK, FP4_BLOCK)
    scale = pow2_ceil(xb.abs().amax(dim=-1).clamp(min=SCALE_FLOOR) / FP4_MAX)   # [N, K/32]
    y = (xb / scale.unsqueeze(-1)).clamp(-FP4_MAX, FP4_MAX)
    a = y.abs()
    # E2M1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 (codes 0..7); at each midpoint
    # the even code wins: ">" where the lower code is even, ">=" where the upper is
    code = ((a > 0.25).int() + (a >= 0.75).int() + (a > 1.25).int() + (a >= 1.75).int()
            + (a > 2.5).int() + (a >= 3.5).int() + (a > 5.0).int())
    code = code | ((y < 0) & (code > 0)).int() * 8
    code = code.view(n, k).to(torch.uint8)
    packed = code[:, 0::2] | (code[:, 1::2] << 4)
    sfb = torch.zeros(k // FP4_BLOCK, tma_aligned_size(n), dtype=torch.float32, device=x.device)
    sfb[:, :n] = scale.t()
    return packed.contiguous(), sfb


def _gen(seed: int, stream: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000003 + int(stream))
    return g


def _randn(shape, seed, stream, device) -> torch.Tensor:
    return torch.randn(*shape, generator=_gen(seed, stream, device), dtype=torch.float32, device=device)


def _quantize_rhs_grouped_fp4(num_groups: int, n: int, k: int, seed: int, device):
    b = torch.empty(num_groups, n, k // 2, dtype=torch.uint8, device=device)
    sfb = torch.zeros(num_groups, k // FP4_BLOCK, tma_aligned_size(n), dtype=torch.float32, device=device)
    for g in range(num_groups):
        bq, s = quantize_rhs_e2m1(_randn((n, k), seed, 100 + g, device))
        b[g].copy_(bq)
        sfb[g].copy_(s)
    return b, sfb


def _quantize_rhs_grouped(num_groups: int, n: int, k: int, seed: int, device, ue8m0: bool = False,
                          fp4: bool = False):
    if fp4:
        return _quantize_rhs_grouped_fp4(num_groups, n, k, seed, device)
    b = torch.empty(num_groups, n, k, dtype=torch.float8_e4m3fn, device=device)
    sfb = torch.empty(num_groups, n // BLOCK, k // BLOCK, dtype=torch.float32, device=device)
    for g in range(num_groups):
        bq, s = quantize_rhs(_randn((n, k), seed, 100 + g, device), ue8m0)
        b[g].copy_(bq)
        sfb[g].copy_(s)
    return b, sfb


# ---------------------------------------------------------------------------
# Workload containers
# ---------------------------------------------------------------------------

def _b_bytes(n: int, k: int, fp4: bool) -> int:
    """Bytes of one group's B and its scales."""
    if fp4:
        return n * k // 2 + 4 * n * (k // FP4_BLOCK)
    return n * k + 4 * (n // BLOCK) * (k // BLOCK)


@dataclass
class Dense:
    a: torch.Tensor
    sfa: torch.Tensor
    b: torch.Tensor
    sfb: torch.Tensor
    m: int
    n: int
    k: int
    ue8m0: bool = False      # power-of-two scales, for the *_ue8m0 entry points

    def new_output(self) -> torch.Tensor:
        return sentinel_output((self.m, self.n), self.a.device)

    def flops(self) -> float:
        return 2.0 * self.m * self.n * self.k

    def algorithmic_bytes(self) -> float:
        m, n, k = self.m, self.n, self.k
        return n * k + 4 * (n // BLOCK) * (k // BLOCK) + m * (k + 4 * (k // BLOCK) + 2 * n)


@dataclass
class Contiguous:
    a: torch.Tensor          # [M_pad, K]
    sfa: torch.Tensor        # [K/128, tma_aligned(M_pad)]
    b: torch.Tensor          # [G, N, K]
    sfb: torch.Tensor        # [G, N/128, K/128]
    layout: torch.Tensor     # int32 [M_pad]
    rows: List[int]          # valid rows per group
    m: int                   # padded total rows
    n: int
    k: int
    num_groups: int
    ue8m0: bool = False
    fp4: bool = False        # B packed E2M1 [G, N, K/2] with sfb [G, K/32, tma_aligned(N)]

    def new_output(self) -> torch.Tensor:
        return sentinel_output((self.m, self.n), self.a.device)

    def valid_rows(self) -> int:
        return int(sum(self.rows))

    def flops(self) -> float:
        return 2.0 * self.n * self.k * self.valid_rows()

    def algorithmic_bytes(self) -> float:
        n, k = self.n, self.k
        used = sum(1 for r in self.rows if r > 0)
        return (used * _b_bytes(n, k, self.fp4)
                + self.valid_rows() * (k + 4 * (k // BLOCK) + 2 * n) + 4 * self.m)


@dataclass
class Masked:
    a: torch.Tensor          # [G, max_m, K]
    sfa: torch.Tensor        # [G, K/128, tma_aligned(max_m)]
    b: torch.Tensor          # [G, N, K]
    sfb: torch.Tensor        # [G, N/128, K/128]
    masked_m: torch.Tensor   # int32 [G]
    counts: List[int]
    max_m: int
    n: int
    k: int
    num_groups: int
    ue8m0: bool = False
    fp4: bool = False

    def new_output(self) -> torch.Tensor:
        return sentinel_output((self.num_groups, self.max_m, self.n), self.a.device)

    def valid_rows(self) -> int:
        return int(sum(min(max(c, 0), self.max_m) for c in self.counts))

    def flops(self) -> float:
        return 2.0 * self.n * self.k * self.valid_rows()

    def algorithmic_bytes(self) -> float:
        n, k = self.n, self.k
        used = sum(1 for c in self.counts if c > 0)
        return (used * _b_bytes(n, k, self.fp4)
                + self.valid_rows() * (k + 4 * (k // BLOCK) + 2 * n) + 4 * self.num_groups)


@dataclass
class Nopad:
    a: torch.Tensor          # [M, K]: the groups' rows back to back, then `tail` extra rows
    sfa: torch.Tensor        # [K/128, tma_aligned(M)]
    b: torch.Tensor          # [G, N, K]
    sfb: torch.Tensor        # [G, N/128, K/128]
    group_rows: torch.Tensor  # int32 [G]
    rows: List[int]          # the counts as given (before any clipping)
    m: int
    n: int
    k: int
    num_groups: int
    ue8m0: bool = False

    def new_output(self) -> torch.Tensor:
        return sentinel_output((self.m, self.n), self.a.device)

    def row_ranges(self) -> List[tuple]:
        """[first, end) of each group: counts below zero count as zero, rows
        at or past m do not exist."""
        out, s = [], 0
        for r in self.rows:
            c = max(int(r), 0)
            first = min(s, self.m)
            out.append((first, min(first + c, self.m)))
            s += c
        return out

    def valid_rows(self) -> int:
        return int(sum(e - f for f, e in self.row_ranges()))

    def flops(self) -> float:
        return 2.0 * self.n * self.k * self.valid_rows()

    def algorithmic_bytes(self) -> float:
        n, k = self.n, self.k
        used = sum(1 for f, e in self.row_ranges() if e > f)
        return (used * (n * k + 4 * (n // BLOCK) * (k // BLOCK))
                + self.valid_rows() * (k + 4 * (k // BLOCK) + 2 * n) + 4 * self.num_groups)


@dataclass
class KGrouped:
    a: torch.Tensor          # [M, K]: each group's K columns back to back
    sfa: torch.Tensor        # [K/128, tma_aligned(M)]
    b: torch.Tensor          # [N, K]
    sfb: torch.Tensor        # [K/128, tma_aligned(N)]
    ks: List[int]            # K of each group (multiples of 128)
    m: int
    n: int
    k: int
    num_groups: int
    seed: int = 0
    ue8m0: bool = False

    def new_output(self) -> torch.Tensor:
        """A float32 [G, M, N] accumulator with seeded N(0, 1) starting values."""
        return _randn((self.num_groups, self.m, self.n), self.seed, 7, self.a.device)

    def flops(self) -> float:
        return 2.0 * self.m * self.n * self.k

    def algorithmic_bytes(self) -> float:
        """Operands and scales once, D written and its prior value read
        (the in-place accumulation of the benchmark)."""
        m, n, k = self.m, self.n, self.k
        return (m + n) * (k + 4 * (k // BLOCK)) + 2 * 4 * self.num_groups * m * n


def sentinel_output(shape, device) -> torch.Tensor:
    """A BF16 output buffer prefilled with the 0xFFFF sentinel."""
    return torch.full(shape, -1, dtype=torch.int16, device=device).view(torch.bfloat16)


# ---------------------------------------------------------------------------
# Generators
# ---------------------------------------------------------------------------

def make_dense(m: int, n: int, k: int, seed: int = 0, device="cpu", ue8m0: bool = False) -> Dense:
    a, sfa = quantize_lhs(_randn((m, k), seed, 1, device), ue8m0)
    b, sfb = quantize_rhs(_randn((n, k), seed, 2, device), ue8m0)
    return Dense(a, sfa, b, sfb, m, n, k, ue8m0)


def contiguous_layout(rows: List[int], align: int = BLOCK) -> np.ndarray:
    """Per-row group index for concatenated segments, each padded to `align`
    rows; padding rows hold -1. Groups with zero rows get no segment."""
    parts = []
    for g, r in enumerate(rows):
        padded = (r + align - 1) // align * align
        seg = np.full(padded, -1, dtype=np.int32)
        seg[:r] = g
        parts.append(seg)
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int32)


def make_contiguous(rows: List[int], n: int, k: int, seed: int = 0, device="cpu",
                    poison_padding: bool = False, ue8m0: bool = False, fp4: bool = False) -> Contiguous:
    """fp4: B as packed E2M1 with per-32 power-of-two scales, and A's scales
    powers of two too (the FP8 x FP4 GEMMs read every scale as UE8M0)."""
    ue8m0 = ue8m0 or fp4
    layout_np = contiguous_layout(rows)
    m = int(layout_np.size)
    a, sfa = quantize_lhs(_randn((max(m, 1), k), seed, 1, device), ue8m0)
    a = a[:m].contiguous()
    sfa = sfa[:, :tma_aligned_size(m)].contiguous() if m else torch.zeros(k // BLOCK, 0, device=device)
    layout = torch.from_numpy(layout_np).to(device)
    if poison_padding and m:
        pad = layout < 0
        a.view(torch.uint8)[pad] = 0x7F  # E4M3 NaN
    b, sfb = _quantize_rhs_grouped(len(rows), n, k, seed, device, ue8m0, fp4)
    return Contiguous(a, sfa, b, sfb, layout, list(map(int, rows)), m, n, k, len(rows), ue8m0, fp4)


def make_masked(counts: List[int], max_m: int, n: int, k: int, seed: int = 0, device="cpu",
                poison_invalid: bool = False, ue8m0: bool = False, fp4: bool = False) -> Masked:
    ue8m0 = ue8m0 or fp4
    num_groups = len(counts)
    a = torch.empty(num_groups, max_m, k, dtype=torch.float8_e4m3fn, device=device)
    sfa = torch.zeros(num_groups, k // BLOCK, tma_aligned_size(max_m), dtype=torch.float32, device=device)
    for g in range(num_groups):
        aq, s = quantize_lhs(_randn((max_m, k), seed, 1000 + g, device), ue8m0)
        a[g].copy_(aq)
        sfa[g].copy_(s)
        if poison_invalid:
            valid = min(max(int(counts[g]), 0), max_m)
            a[g, valid:].view(torch.uint8).fill_(0x7F)
    b, sfb = _quantize_rhs_grouped(num_groups, n, k, seed, device, ue8m0, fp4)
    masked_m = torch.tensor(list(counts), dtype=torch.int32, device=device)
    return Masked(a, sfa, b, sfb, masked_m, list(map(int, counts)), max_m, n, k, num_groups, ue8m0, fp4)


def make_nopad(rows: List[int], n: int, k: int, seed: int = 0, device="cpu", tail: int = 0,
               m: Optional[int] = None, poison_tail: bool = False, ue8m0: bool = False) -> Nopad:
    """Groups' rows back to back with no padding, then `tail` rows that no
    group owns (or exactly m rows when m is given)."""
    if m is None:
        m = int(sum(max(int(r), 0) for r in rows)) + tail
    a, sfa = quantize_lhs(_randn((max(m, 1), k), seed, 1, device), ue8m0)
    a = a[:m].contiguous()
    sfa = sfa[:, :tma_aligned_size(m)].contiguous() if m else torch.zeros(k // BLOCK, 0, device=device)
    b, sfb = _quantize_rhs_grouped(len(rows), n, k, seed, device, ue8m0)
    group_rows = torch.tensor(list(rows), dtype=torch.int32, device=device)
    w = Nopad(a, sfa, b, sfb, group_rows, list(map(int, rows)), m, n, k, len(rows), ue8m0)
    if poison_tail and m:
        used = max([e for _, e in w.row_ranges()], default=0)
        a.view(torch.uint8)[used:] = 0x7F  # E4M3 NaN
    return w


def make_k_grouped(ks: List[int], m: int, n: int, seed: int = 0, device="cpu", ue8m0: bool = False) -> KGrouped:
    """K-grouped operands: A [M, K] and B [N, K] with one scale per row and
    128-wide K block for both (recipe (1, 1, 128)): each is quantised like
    the LHS of the other GEMMs."""
    k = int(sum(ks))
    assert all(x % BLOCK == 0 and x >= 0 for x in ks)
    a, sfa = quantize_lhs(_randn((m, max(k, BLOCK)), seed, 11, device), ue8m0)
    b, sfb = quantize_lhs(_randn((n, max(k, BLOCK)), seed, 12, device), ue8m0)
    a, b = a[:, :k].contiguous(), b[:, :k].contiguous()
    sfa, sfb = sfa[:k // BLOCK].contiguous(), sfb[:k // BLOCK].contiguous()
    return KGrouped(a, sfa, b, sfb, list(map(int, ks)), m, n, k, len(ks), seed, ue8m0)


# ---------------------------------------------------------------------------
# The benchmark workloads
# ---------------------------------------------------------------------------

@dataclass
class WorkloadSpec:
    index: int
    kind: str                      # "dense" | "contiguous" | "masked"
    name: str
    n: int
    k: int
    m: int = 0                     # dense
    rows: Optional[List[int]] = None      # contiguous: valid rows per group
    counts: Optional[List[int]] = None    # masked: masked_m per group
    max_m: int = 0
    extra: dict = field(default_factory=dict)


def _structure_rng(seed: int) -> np.random.Generator:
    return np.random.default_rng([seed, 0])


def zipf_rows(total: int, num_groups: int, s: float, seed: int) -> List[int]:
    """Token counts per expert when each of `total` tokens picks expert
    i in 1..G with probability proportional to i^-s (group 0 is the largest)."""
    i = np.arange(1, num_groups + 1, dtype=np.float64)
    p = i ** -s
    p /= p.sum()
    return [int(x) for x in _structure_rng(seed).multinomial(total, p)]


def workload_spec(index: int, seed: int = 0) -> WorkloadSpec:
    """The workloads, indexed 0..5:
    0 dense 128x256x512; 1 dense 4096x7168x2048;
    2 contiguous, 8 groups with rows uniform in [3000, 5000], N=4096, K=7168;
    3 masked decode, 16 groups, max_m=256, masked_m uniform in [1, 256], N=7168, K=2048;
    4 contiguous, 32 groups with Zipf(1.2) rows totalling 65536, N=4096, K=7168;
    5 no-padding layout of workload 2's groups (the same row counts, not padded);
    6, 7, 8: workloads 1, 2 and 3 with power-of-two (UE8M0-cast) scales, for
    the *_ue8m0 entry points;
    9 K-grouped weight gradient of workload 2's up projection: 8 groups with
      K = workload 2's row counts rounded up to 128, M = 4096 (output
      features), N = 7168 (input features), accumulated into D in place;
    10, 11: workloads 3 and 2 with B as packed E2M1 FP4 (per-32 scales), for
      the FP8 x FP4 (W4A8) entry points;
    12: workload 9 with power-of-two scales, for the K-grouped *_ue8m0 call.
    """
    if index == 0:
        return WorkloadSpec(0, "dense", "dense_128x256x512", n=256, k=512, m=128)
    if index == 1:
        return WorkloadSpec(1, "dense", "dense_4096x7168x2048", n=7168, k=2048, m=4096)
    if index == 2:
        rows = [int(x) for x in _structure_rng(seed).integers(3000, 5001, size=8)]
        return WorkloadSpec(2, "contiguous", "contiguous_8x[3000,5000]_n4096_k7168", n=4096, k=7168, rows=rows)
    if index == 3:
        counts = [int(x) for x in _structure_rng(seed).integers(1, 257, size=16)]
        return WorkloadSpec(3, "masked", "masked_16x256_n7168_k2048", n=7168, k=2048, counts=counts, max_m=256)
    if index == 4:
        rows = zipf_rows(65536, 32, 1.2, seed)
        return WorkloadSpec(4, "contiguous", "contiguous_zipf1.2_32x65536_n4096_k7168", n=4096, k=7168, rows=rows)
    if index == 5:
        rows = [int(x) for x in _structure_rng(seed).integers(3000, 5001, size=8)]
        return WorkloadSpec(5, "nopad", "nopad_8x[3000,5000]_n4096_k7168", n=4096, k=7168, rows=rows)
    if index in (6, 7, 8):
        base = workload_spec(index - 5, seed)
        return WorkloadSpec(index, base.kind, base.name + "_ue8m0", n=base.n, k=base.k, m=base.m, rows=base.rows,
                            counts=base.counts, max_m=base.max_m, extra={"ue8m0": True})
    if index == 9:
        rows = workload_spec(2, seed).rows
        ks = [(r + BLOCK - 1) // BLOCK * BLOCK for r in rows]
        return WorkloadSpec(9, "k_grouped", "k_grouped_8x[3000,5000]_m4096_n7168", n=7168, k=int(sum(ks)), m=4096,
                            rows=ks)
    if index in (10, 11):
        base = workload_spec(3 if index == 10 else 2, seed)
        return WorkloadSpec(index, base.kind, base.name.replace("_n", "_w4a8_n", 1), n=base.n, k=base.k, m=base.m,
                            rows=base.rows, counts=base.counts, max_m=base.max_m, extra={"fp4": True})
    if index == 12:
        base = workload_spec(9, seed)
        return WorkloadSpec(12, base.kind, base.name + "_ue8m0", n=base.n, k=base.k, m=base.m, rows=base.rows,
                            extra={"ue8m0": True})
    raise ValueError(f"no workload {index}")


NUM_WORKLOADS = 13


def make_workload(spec: WorkloadSpec, seed: int = 0, device="cpu"):
    e8 = bool(spec.extra.get("ue8m0", False))
    fp4 = bool(spec.extra.get("fp4", False))
    if spec.kind == "dense":
        return make_dense(spec.m, spec.n, spec.k, seed, device, ue8m0=e8)
    if spec.kind == "contiguous":
        return make_contiguous(spec.rows, spec.n, spec.k, seed, device, ue8m0=e8, fp4=fp4)
    if spec.kind == "masked":
        return make_masked(spec.counts, spec.max_m, spec.n, spec.k, seed, device, ue8m0=e8, fp4=fp4)
    if spec.kind == "nopad":
        return make_nopad(spec.rows, spec.n, spec.k, seed, device, ue8m0=e8)
    if spec.kind == "k_grouped":
        return make_k_grouped(spec.rows, spec.m, spec.n, seed, device, ue8m0=e8)
    raise ValueError(spec.kind)


def to_numpy_bytes(t: torch.Tensor) -> np.ndarray:
    """Raw host bytes of a tensor as the numpy dtype the oracle reads:
    E4M3 -> uint8, bfloat16 -> uint16, others unchanged."""
    t = t.detach().cpu()
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
