"""The C ABI from a C caller: tests/abi_check.c, built with gcc against
include/ecmd.h and linked to libecmd.so, builds the mixed-precision
configuration through the cmd_* calls, plans it, walks every error status
(each with a message in cmd_last_error) and round-trips it through YAML; on a
GPU it also launches it over the hand-worked cases and times cmd_launch from
C."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "elementwise_tensor_commands_amd")
SRC = os.path.join(ROOT, "tests", "abi_check.c")
ROCM = "/opt/rocm"


def _build(tmp_path, gpu):
    exe = str(tmp_path / ("abi_check_gpu" if gpu else "abi_check"))
    cmd = ["gcc", "-O1", "-std=c11", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"), SRC,
           "-o", exe, "-L" + PKG, "-lecmd", "-Wl,-rpath," + PKG, "-Wl,-rpath-link," + ROCM + "/lib"]
    if gpu:
        cmd[1:1] = ["-DECMD_ABI_GPU", "-D__HIP_PLATFORM_AMD__", "-I", ROCM + "/include"]
        cmd += ["-L" + ROCM + "/lib", "-lamdhip64", "-Wl,-rpath," + ROCM + "/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_c_caller_host(tmp_path):
    exe = _build(tmp_path, gpu=False)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and "ABI OK" in r.stdout, r.stdout + r.stderr


@pytest.mark.gpu
def test_c_caller_gpu(tmp_path):
    exe = _build(tmp_path, gpu=True)
    r = subprocess.run([exe, "--gpu", str((1 << 20) + 13)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "GPU OK" in r.stdout, r.stdout + r.stderr
    line = [l for l in r.stdout.splitlines() if l.startswith("launch_us")][0]
    host_us, b2b_us = map(float, line.split()[1:])
    print("  cmd_launch from C: %.2f us host per call, %.2f us per launch back to back" % (host_us, b2b_us))
    assert 0 < host_us < 1000 and 0 < b2b_us < 1000
