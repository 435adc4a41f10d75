"""Process exit while the run-time compiler works in the background, on the
host (CPU only): tests/jit_exit_check.cpp queues compiles through the
library's own jit_poll and leaves main while the worker thread compiles; the
process must exit with status 0, neither crashing nor hanging, at moments
when the first compile has returned and later ones are running or queued.
Before the worker was stopped ahead of the compiler's teardown, such exits
crashed or hung."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "elementwise_tensor_commands_amd")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    if not os.path.exists(os.path.join(PKG, "libecmd.so")) or not os.path.exists(HIPCC):
        pytest.skip("needs the built library and hipcc")
    out = str(tmp_path_factory.mktemp("jit_exit") / "jit_exit_check")
    subprocess.run([HIPCC, "-O1", "-std=c++20", "-I", os.path.join(PKG, "csrc"), "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "jit_exit_check.cpp"), "-o", out, "-L", PKG, "-lecmd",
                    "-Wl,-rpath," + PKG], check=True, capture_output=True)
    return out


@pytest.mark.parametrize("wait_ms", [1000, 2000])
def test_exit_while_compiling(exe, tmp_path, wait_ms):
    env = dict(os.environ, ECMD_CACHE_DIR=str(tmp_path / "cache"))
    r = subprocess.run([exe, "12", str(wait_ms)], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert "leaving main" in r.stdout and "queued 12" in r.stdout, r.stdout
    shutil.rmtree(str(tmp_path / "cache"), ignore_errors=True)
