"""LDS tile layout of the bf16 d=128 kernels, checked on the host: the operand read
offsets of ra_device.h (row reads and transposing reads of the XOR-swizzled
256-byte rows) address exactly the rows and chunks each lane's MFMA operand needs,
and both read patterns spread over all 64 LDS banks.  The helpers themselves are
compiled (tests/lds_layout_check.cpp includes ra_device.h), not retyped."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_lds_operand_offsets_and_banks(tmp_path):
    exe = tmp_path / "lds_layout_check"
    src = os.path.join(ROOT, "tests", "lds_layout_check.cpp")
    subprocess.run([HIPCC, "-O1", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature",
                    "-Xclang", "-packed-fp32-ops", src, "-o", str(exe)], check=True, capture_output=True,
                   timeout=600)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.strip() == "ok"
