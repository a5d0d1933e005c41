"""The host planner of the CE calls, built with g++ against the library's
host-only source (lce_contract.cpp) and checked on the CPU.

* tests/pack_check.cpp replays the walk a packed backward launch makes over its
  slots for about 37 000 tile-count and duration cases: every logical tile of
  every product runs exactly once, the reported makespan is the busiest slot's
  load within its bounds, and a slot never holds more than 255 tiles of one
  product.
* tests/plan_check.cpp checks every plan over a grid of about 41 000 shapes,
  chunks and input types: refusals match the host checks, the logit-derived
  buffers stay within chunk * vocab cells, the slabs cover the vocabulary,
  and the workspace regions that live at once are aligned and disjoint.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lm_head_linear_amd", "csrc")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")


def _run(tmp_path, name):
    exe = str(tmp_path / name)
    cmd = ["g++", "-O2", "-std=c++17", "-Wall", "-Werror", f"-I{CSRC}",
           f"-I{os.path.join(ROOT, 'include')}", os.path.join(ROOT, "tests", name + ".cpp"),
           os.path.join(CSRC, "lce_contract.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    words = r.stdout.split()
    assert words[0] == "ok", r.stdout
    return [int(w) for w in words[1:]]


def test_pack_tiles_runs_every_tile_once(tmp_path):
    cases, packed, refused = _run(tmp_path, "pack_check")
    # only the case with 256 tiles of one product on a slot is refused
    assert refused == 1
    assert packed == cases - 1


def test_plans_keep_the_logit_budget(tmp_path):
    plans, refused, pipelined, packed, kept = _run(tmp_path, "plan_check")
    # every kind of plan is reached: refusals, the slab pipeline, packed
    # launches and the single call's kept logits
    assert min(plans, refused, pipelined, packed, kept) > 0
