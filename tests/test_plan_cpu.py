"""Launch-plan invariants of the HIP library, checked on the host.

The plans (the flat split of the streamed rows over a launch's groups, the
draw chunks, the workspace layout) are plain C++ shared by the kernels, the
launchers and verify_workspace_size; tests/native/plan_check.cpp includes
that header, is compiled here with g++ and asserts, over a grid of sizes up to
the largest vocabularies, that the split covers the stream exactly once with
unique partial slots, that every row's partials are found again, and that
workspace sections are aligned and disjoint.
"""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "draft_block_verification_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_plan_invariants(tmp_path):
    exe = tmp_path / "plan_check"
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-I", CSRC,
                    os.path.join(HERE, "native", "plan_check.cpp"), "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
