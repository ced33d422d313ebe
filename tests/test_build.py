"""Build-level checks (CPU): facts about the generated gfx950 code that the
kernels rely on.

The f8f6f4 MFMAs are reached through the block-scaled builtin; the GEMMs
with float32 scales pass constant-zero scale operands (mfma_fp8 in
csrc/dg_device.h) and rely on the compiler selecting the plain
v_mfma_f32_16x16x128_f8f6f4, whose products are not scaled. This compiles
the ceiling kernel, which uses that wrapper and its scaled twin, to gfx950
assembly and checks the instruction chosen.
"""

import os
import re
import shutil
import subprocess

import pytest

from moe_grouped_gemm_amd import build as B


def _device_asm(src: str, tmp_path) -> str:
    hipcc = B.hipcc()
    if not (os.path.exists(hipcc) or shutil.which(hipcc)):
        pytest.skip("hipcc not available")
    out = tmp_path / "k.s"
    flags = [f for f in B.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [hipcc, *flags, "--cuda-device-only", "-S", "-I", os.path.join(B.ROOT, "include"),
           os.path.join(B.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _function_body(asm: str, needle: str) -> str:
    m = re.search(r"^(_Z\S*" + needle + r"\S*):", asm, flags=re.M)
    assert m, f"no function matching {needle}"
    start = m.end()
    end = asm.index("s_endpgm", start)
    return asm[start:end]


def test_zero_scale_codes_select_the_unscaled_mfma(tmp_path):
    asm = _device_asm("dg_ceiling.hip", tmp_path)
    bodies = [_function_body(asm, f"mfma_ceiling_kernelILi{v}E") for v in range(3)]
    for body in bodies:
        assert re.search(r"\bv_mfma_f32_16x16x128_f8f6f4\b", body)
        assert "v_mfma_scale_f32" not in body
