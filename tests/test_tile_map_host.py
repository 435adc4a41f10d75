"""The tiled kernel's work split and LDS layout, checked on the host (CPU only).

tests/tile_map_check.cpp includes the library's own ecmd_tape.h and checks,
for every tile shape kernels_tiled.hip instantiates, that tile_split covers
each tile exactly once, that tile_word is one to one, and that neither LDS
phase has a bank conflict under gfx950's model for wave64 four-byte accesses
(32 banks, half-wavefronts served separately).  The same program first checks
the model against the conflict rates rocprofv3 measured on the previous,
padded-pitch layout.
"""
import os
import re
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "elementwise_tensor_commands_amd", "csrc")


def instantiated_shapes():
    src = open(os.path.join(CSRC, "kernels_tiled.hip")).read()
    shapes = set()
    for m in re.finditer(r"launch_nt<\s*\w+\s*,\s*(?:0x[0-9a-fA-F]+|\w+)\s*,\s*(\d+)\s*,\s*(\d+)\s*,\s*(\d+)\s*>", src):
        shapes.add(tuple(int(x) for x in m.groups()))
    return sorted(shapes)


def test_every_instantiated_tile_is_conflict_free(tmp_path):
    shapes = instantiated_shapes()
    assert (32, 256, 512) in shapes and (64, 64, 256) in shapes and len(shapes) >= 10, shapes
    exe = str(tmp_path / "tile_map_check")
    subprocess.run(["g++", "-std=c++20", "-O1", "-Wall", "-I", CSRC, os.path.join(ROOT, "tests", "tile_map_check.cpp"),
                    "-o", exe], check=True, capture_output=True)
    args = [str(x) for s in shapes for x in s]
    r = subprocess.run([exe, *args], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count("staging writes 1-way, chunk reads 1-way") == len(shapes), r.stdout
