"""Host check that the LDS addresses of the bf16 causal kernel, formed from a
per-lane part and compile-time parts, equal the swizzled addresses of the
elements they stand for (every access site, lane, chunk and tile; every built
(D, M)).  Builds tests/lds_addressing_check.cpp with hipcc as host code."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")


@pytest.mark.skipif(HIPCC is None, reason="hipcc not available")
def test_lds_address_split_matches_swizzle():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "lds_check")
        res = subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17",
                              "-I", os.path.join(ROOT, "weight_recurrences_amd", "csrc"),
                              os.path.join(ROOT, "tests", "lds_addressing_check.cpp"), "-o", exe],
                             capture_output=True, text=True)
        assert res.returncode == 0, res.stderr
        run = subprocess.run([exe], capture_output=True, text=True)
        assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout
