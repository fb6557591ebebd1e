"""Host check of the gfx950 assembly of the MFMA kernels: no result of an MFMA is read by a
non-MFMA instruction within 4 issued instructions on any control path (the pattern of a known
compiler hazard when a data-dependent branch skips an MFMA block).  Compiles each source to
assembly with the library's flags."""
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "tests"))
from mfma_hazard_scan import min_read_distance  # noqa: E402

HIPCC = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")
MIN_DISTANCE = 5


@pytest.mark.skipif(HIPCC is None, reason="hipcc not available")
@pytest.mark.parametrize("src,pattern", [("causal_fused.hip", "causal_fused_kernel"),
                                         ("causal_fused32.hip", "causal_fused32_kernel"),
                                         ("noncausal.hip", "nc_"),
                                         ("causal_bwd_bf16.hip", "bf16_kernel"),
                                         ("featmap.hip", "fm_"),
                                         ("causal.hip", "kernel"),
                                         ("causal_bwd.hip", "kernel"),
                                         ("deltanet_chunk.hip", "kernel")])
def test_mfma_results_not_read_early(src, pattern):
    with tempfile.TemporaryDirectory() as d:
        asm = os.path.join(d, "k.s")
        cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-S",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "weight_recurrences_amd", "csrc", src), "-o", asm]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        found = min_read_distance(open(asm).read(), pattern)
        assert found, "no kernels matched"
        for name, (dist, mfma, reader) in found.items():
            assert dist >= MIN_DISTANCE, f"{name}: {mfma} read by {reader} at distance {dist}"
