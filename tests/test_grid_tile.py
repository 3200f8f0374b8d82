"""The kernels' workgroup -> (head, tile) map (grid_tile in fa_device.h),
compiled for the host with hipcc (under AddressSanitizer and
UndefinedBehaviorSanitizer on the host side) and checked over heads 1..72,
1..256 tiles per head, dispatch groups of 1..16 heads and tail groups from
none to all heads, with and without XCD grouping: every tile exactly once,
every head on one XCD, ranks ascending within a head's sequence on its XCD
(tests/sanitize/grid_tile_check.hip).  CPU only."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_grid_tile_is_a_bijection(tmp_path):
    exe = str(tmp_path / "grid_tile_check")
    san = []
    for opt in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"):
        san += ["-Xarch_host", opt]
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "exact_attention_21_amd", "csrc"), *san,
           os.path.join(ROOT, "tests", "sanitize", "grid_tile_check.hip"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    assert "cases hold" in r.stdout
