"""The HIP sources compile for gfx950 with the library's flags, and the
generated code contains no packed FP32 VALU instructions (they are
disabled in the build; see w8a8_int8_gemm_amd/build.py)."""
import subprocess
from pathlib import Path

import pytest

from w8a8_int8_gemm_amd import build as wb


@pytest.mark.parametrize("src", [s for s in wb.SOURCES if s.endswith(".hip")])
def test_no_packed_fp32_in_device_code(src, tmp_path):
    out = tmp_path / (Path(src).stem + ".s")
    cmd = [wb.HIPCC, *[f for f in wb.FLAGS if f not in ("-shared", "-fPIC")],
           "--cuda-device-only", "-S", "-o", str(out), str(wb.CSRC / src)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    for op in ("v_pk_add_f32", "v_pk_mul_f32", "v_pk_fma_f32"):
        assert op not in asm, f"{op} in {src}"
    assert "v_mfma" in asm or "gemm" not in src
