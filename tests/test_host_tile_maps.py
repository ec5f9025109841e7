"""The grouped GEMMs' workgroup-to-tile maps (the XCD-blocked plan order and
the weight-gradient launches' expert-per-XCD order), checked on the CPU:
tests/tile_maps_check.hip is compiled for the host from the library's own
header and must find every tile handed out exactly once over the launch
grid."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_tile_maps_hand_out_every_tile_once(tmp_path):
    exe = str(tmp_path / "tile_maps_check")
    cmd = [HIPCC, "-O1", "-std=c++17", "--offload-arch=gfx950", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "routed_relu_expert_amd", "csrc"), os.path.join(HERE, "tile_maps_check.hip"),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
