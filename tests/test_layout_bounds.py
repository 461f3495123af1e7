"""The kernels' LDS carve-ups and per-wave capacities, bounds-checked on the host.

``layout_bounds.cpp`` includes the kernels' own layout header and checks, for the list lengths,
buffer sizes, workgroups per request and hash sizes the library accepts (including four
speculative rows of k 2048 into B 10240), that every LDS region the RESOLVE, union, fused and
attention kernels index lies inside its allocation and below the 160 KiB a gfx950 workgroup
has, and that a wave's miss list can hold every miss it can own.  Host code only: no GPU.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="needs hipcc")
def test_lds_layouts_in_bounds(tmp_path):
    exe = str(tmp_path / "layout_bounds")
    hipcc = HIPCC if os.path.exists(HIPCC) else shutil.which("hipcc")
    build = subprocess.run([hipcc, "-std=c++17", "-O1", "-o", exe, os.path.join(HERE, "layout_bounds.cpp")],
                           capture_output=True, text=True)
    assert build.returncode == 0, build.stdout + build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and run.stdout.startswith("ok:"), run.stdout + run.stderr
