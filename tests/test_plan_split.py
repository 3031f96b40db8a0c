"""Host checks of the key-axis split of the work plan (csrc/plan.h).

tests/plan_split_check.cpp includes plan.h with the host compiler and checks,
for each plan, that the items decode to every (entry, head, query tile) once
(in head-major order for a plan of one group over a shared K/V), that the
persistent claims take every unit exactly once, that
the units are every (item, part) of the split items and every other item
once, that an item's parts partition its key tiles, and that the split items
are the last items of the long group (entries with a predecessor) when there
is one, else the last of the launch.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "chunked_spatio_temporal_amd", "csrc")

# n first_pred heads lq lown lpred bm n_xcd n_split parts head_major
CASES = [
    (8, 1, 5, 6240, 6240, 6240, 384, 8, 256, 4, 0),   # 5-head queue shard, 680 items
    (8, 1, 5, 6240, 6240, 6240, 384, 8, 680, 2, 0),   # more than the long group asks
    (8, 1, 12, 6240, 6240, 6240, 384, 8, 384, 4, 0),  # 12-head queue
    (3, 1, 2, 1000, 1000, 1000, 384, 8, 18, 3, 0),    # every long item
    (3, 1, 2, 1000, 1000, 1000, 384, 8, 5, 2, 0),
    (3, 1, 2, 100, 100, 100, 384, 8, 6, 4, 0),        # two-tile items in 4 parts
    (1, 1, 3, 2000, 2000, 0, 384, 8, 7, 2, 0),        # no predecessor group
    (2, 2, 2, 1000, 1000, 0, 384, 3, 5, 4, 0),        # full attention: no long group
    (8, 1, 5, 6240, 6240, 6240, 384, 8, 0, 4, 0),     # no split
    (8, 1, 5, 6240, 6240, 6240, 384, 1, 100, 8, 0),   # one die
    # head-major order (shared K/V): 720p cross-attention with 6-block items,
    # a split full attention, one die, and a queue plan that must stay (b, h, t)
    (16, 16, 40, 14400, 512, 0, 2304, 8, 0, 1, 1),
    (3, 3, 5, 1000, 300, 0, 384, 8, 11, 4, 1),
    (2, 2, 3, 129, 1, 0, 384, 1, 0, 1, 1),
    (8, 1, 5, 6240, 6240, 6240, 384, 8, 256, 4, 1),
]


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("plan") / "plan_split_check")
    subprocess.run([cxx, "-std=c++17", "-O2", "-I", CSRC,
                    os.path.join(ROOT, "tests", "plan_split_check.cpp"), "-o", exe], check=True)
    return exe


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_split_plan_is_a_bijection(checker, case):
    r = subprocess.run([checker, *map(str, case)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
