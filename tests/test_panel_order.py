"""The XCD-aware order in which the pair-symmetric passes hand panel pairs to
blocks, checked on the host: every pair exactly once, each XCD a contiguous
stretch.  The header's __host__ __device__ functions are compiled by hipcc
into a host program (panel_order_check.cpp) that runs without a GPU."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None,
                    reason="needs hipcc")
def test_panel_order_covers_every_pair_once(tmp_path):
    exe = str(tmp_path / "panel_order_check")
    cmd = [HIPCC, "-O1", "-std=c++17", "-x", "hip", "--offload-arch=gfx950",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "direct_all_pairs_softened_amd", "csrc"),
           os.path.join(HERE, "panel_order_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert "ok" in r.stdout
