"""Compile-time checks of the HIP sources (CPU only: hipcc cross-compiles for gfx950).

Every kernel source must compile for gfx950 with inline-assembly diagnostics as errors: an
asm statement that clobbers a register the compiler reserves (such as M0) is undefined
behaviour the compiler warns about, and this keeps such a statement from coming back."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mla_tree_verify_paged_amd", "csrc")
SOURCES = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    pytest.skip("hipcc not available")


@pytest.mark.parametrize("src", SOURCES)
def test_kernel_source_has_no_inline_asm_diagnostics(src, tmp_path):
    cmd = [_hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-c",
           "-Werror=inline-asm", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-mllvm", "-amdgpu-mfma-vgpr-form", "-I" + os.path.join(ROOT, "include"),
           os.path.join(CSRC, src), "-o", str(tmp_path / (src + ".o"))]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "inline asm" not in r.stderr and "reserved register" not in r.stderr, r.stderr[-4000:]
