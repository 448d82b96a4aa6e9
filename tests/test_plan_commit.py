"""The page manager's plan/commit split, on the host (CPU only).

kvc_append_frame plans an append without touching the cache, launches the
scatter, and commits only after a successful launch.  This builds the C++
page manager with a small driver (tests/cpp/plan_commit.cpp) and checks over
30 frames of a LingBot-shaped layer ("LingBot-Map Paged KV Cache", sections 2
and 3: three page streams, single-level rollback) that a plan changes
nothing, that the previous append's undo record survives an abandoned plan,
and that commit equals a plain append.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_sliding_window_kv_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_plan_changes_nothing_and_commit_equals_append(tmp_path):
    exe = str(tmp_path / "plan_commit")
    cmd = ["g++", "-std=c++17", "-O1", f"-I{CSRC}", f"-I{os.path.join(ROOT, 'include')}",
           os.path.join(ROOT, "tests", "cpp", "plan_commit.cpp"), os.path.join(CSRC, "page_cache.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "OK plan/commit 30 frames" in r.stdout
