"""Build libecmd.so (the C ABI and its gfx950 kernels) in-tree with hipcc.

    python elementwise_tensor_commands_amd/build.py [-v]

(run it as a script: importing the package would load the library first).

Every source is compiled for gfx950 only, non-relocatable device code (each
kernel's device code lives in its own translation unit, as clang's HIP support
document describes for the default -fno-gpu-rdc mode), with:
  -ffp-contract=off     every binary32 operation rounds on its own;
  -Xclang -target-feature -Xclang -packed-fp32-ops
                        no packed binary32 instructions;
  -mllvm -simplifycfg-sink-common=false
                        keeps the interpreter's register-slot switches from
                        being merged into one runtime-indexed (scratch) access.
Denormals are left at the default (kept; no -fgpu-flush-denormals-to-zero).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libecmd.so")

SOURCES = ["ecmd_host.cpp", "ecmd_serial.cpp", "kernels_linear.hip", "kernels_tiled.hip", "kernels_rows.hip", "kernels_gather.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++20", "-fPIC", "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-simplifycfg-sink-common=false",
    "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include"),
]


def _run_all(cmds):
    procs = [(c, subprocess.Popen(c, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)) for c in cmds]
    errors = []
    for c, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 target feature; that warning is noise.
        lines = [l for l in out.splitlines()
                 if l.strip() and "packed-fp32-ops" not in l and "'--hip-link'" not in l]
        if p.returncode != 0:
            errors.append("$ %s\n%s" % (" ".join(c), "\n".join(lines)))
        elif lines:
            sys.stderr.write("\n".join(lines) + "\n")
    if errors:
        raise RuntimeError("hipcc failed:\n" + "\n\n".join(errors))


def build(asm: bool = True, verbose: bool = False) -> str:
    """Compile every source and link libecmd.so next to this file.  With asm,
    also write each kernel file's gfx950 assembly to _build/<name>.s (used by the
    tests that inspect the generated code)."""
    os.makedirs(BUILD, exist_ok=True)
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
        if asm and src.endswith(".hip"):
            cmds.append([HIPCC, *FLAGS, "-x", "hip", "--offload-device-only", "-S",
                         os.path.join(CSRC, src), "-o", os.path.join(BUILD, os.path.splitext(src)[0] + ".s")])
    if verbose:
        for c in cmds:
            print(" ".join(c))
    _run_all(cmds)
    tmp = LIB + ".tmp%d" % os.getpid()
    _run_all([[HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(asm=True, verbose="-v" in sys.argv))
