"""The backward's tile packing on the host: tests/pack_check.cpp, built with g++
against the library's host-only source (lce_contract.cpp), replays the walk a
packed launch makes over its slots for about 37 000 tile-count and duration
cases and checks that every logical tile of every product runs exactly once,
that the reported makespan is the busiest slot's load within its bounds, and
that a slot never holds more than 255 tiles of one product.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lm_head_linear_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_pack_tiles_runs_every_tile_once(tmp_path):
    exe = str(tmp_path / "pack_check")
    cmd = ["g++", "-O2", "-std=c++17", "-Wall", "-Werror", f"-I{CSRC}",
           f"-I{os.path.join(ROOT, 'include')}", os.path.join(ROOT, "tests", "pack_check.cpp"),
           os.path.join(CSRC, "lce_contract.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    word, cases, packed, refused = r.stdout.split()
    assert word == "ok"
    # only the case with 256 tiles of one product on a slot is refused
    assert int(refused) == 1
    assert int(packed) == int(cases) - 1
