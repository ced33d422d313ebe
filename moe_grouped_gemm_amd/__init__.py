"""FP8 NT GEMM with fine-grained scaling and its M-grouped MoE variants for
AMD Instinct MI355X (gfx950): a C-ABI library (libdg.so, include/dg.h) of
hand-written HIP kernels and a thin ctypes binding (moe_grouped_gemm_amd.dg)."""

__all__ = ["dg", "synth"]
