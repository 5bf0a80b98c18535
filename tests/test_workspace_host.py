"""The split workspace registry on the host (g++, fake allocator): growth
keeps the smaller buffer alive for work and graphs that still use it,
release frees each buffer once, and two threads on one stream hold its
workspace one after the other (tests/host/workspace_registry_test.cpp)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_prefill_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "host", "workspace_registry_test.cpp")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_workspace_registry_host(tmp_path):
    exe = str(tmp_path / "workspace_registry_test")
    subprocess.run(["g++", "-std=c++17", "-O1", "-pthread", "-Wall", "-Werror", f"-I{CSRC}", SRC, "-o", exe],
                   check=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0 and res.stdout.strip() == "ok", res.stdout + res.stderr
