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


# Shapes the kernels compiled at run time take: 32 x 256 x 512 (32 x 128 x 256
# with three staged inputs) and, for tiles of 16-bit operands, 64 x 256 x 512
# (64 x 128 x 256, 64 x 64 x 256 with more staged inputs) plus other
# ECMD_TILE shapes of 8-element vectors.
JIT_SHAPES = [(32, 256, 512), (32, 128, 256), (64, 64, 256)]
JIT_SHAPES8 = [(64, 256, 512), (64, 128, 256), (64, 64, 256), (64, 256, 256), (128, 128, 256), (128, 256, 512),
               (128, 128, 512)]


def test_compiled_tiles_are_conflict_free(tmp_path):
    exe = str(tmp_path / "tile_map_check")
    subprocess.run(["g++", "-std=c++20", "-O1", "-Wall", "-I", CSRC, os.path.join(ROOT, "tests", "tile_map_check.cpp"),
                    "-o", exe], check=True, capture_output=True)
    args = [str(x) for s in JIT_SHAPES for x in s] + ["-8"] + [str(x) for s in JIT_SHAPES8 for x in s]
    r = subprocess.run([exe, *args], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count("staging writes 1-way, chunk reads 1-way") == len(JIT_SHAPES) + len(JIT_SHAPES8), r.stdout
    assert r.stdout.count("8-element ") == len(JIT_SHAPES8), r.stdout


def test_pair_layout_catches_a_bad_swizzle(tmp_path):
    """The check is not vacuous: without the column-bit-5 term of
    tile_pair_word, the chunk reads of a 64 x 256 tile of 16-bit pairs have
    2-way conflicts (columns j and j + 4 of a half-wavefront share banks)."""
    src = open(os.path.join(ROOT, "tests", "tile_map_check.cpp")).read()
    hdr = open(os.path.join(CSRC, "ecmd_tape.h")).read()
    bad = hdr.replace("(p ^ (c & 31) ^ (((c >> 5) & 1) << 1))", "(p ^ (c & 31))")
    assert bad != hdr
    d = tmp_path / "inc"
    d.mkdir()
    (d / "ecmd_tape.h").write_text(bad)
    exe = str(tmp_path / "tile_map_check_bad")
    subprocess.run(["g++", "-std=c++20", "-O1", "-Wall", "-I", str(d), "-I", CSRC, "-x", "c++", "-", "-o", exe],
                   input=src, text=True, check=True, capture_output=True)
    r = subprocess.run([exe, "-8", "64", "256", "512"], capture_output=True, text=True)
    assert r.returncode != 0 and "bank conflict" in r.stdout, r.stdout
