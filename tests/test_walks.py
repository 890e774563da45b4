"""The kernels' grid walks (lsh_attention_hash_amd/csrc/walks.h: the chunk
kernels' head-grouped range walk, the sort's tile order, the hash's persistent
walk and its division-free (head, position) arithmetic) checked on the CPU:
tests/walks_check.hip runs the same functions over whole grids of many
shapes, requiring every index to stay in bounds and every unit of work to be
visited exactly once. Compiled with hipcc; the program makes no HIP call."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None,
                    reason="hipcc not available")
def test_grid_walks_cover_every_unit_once(tmp_path):
    exe = str(tmp_path / "walks_check")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", "-I",
                    os.path.join(ROOT, "lsh_attention_hash_amd", "csrc"),
                    os.path.join(ROOT, "tests", "walks_check.hip"), "-o", exe],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "walks ok" in r.stdout
