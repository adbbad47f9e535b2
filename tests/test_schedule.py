"""Task order of the two persistent kernels, checked on the host (no GPU).

tests/native/schedule_check.cpp is built from the rule header the kernels themselves
include (two_sided_adaptive_amd/csrc/schedule.hpp).  For the factor stage it walks the
queue in order and requires every wait of every task to be met by the tasks before it
(then the queue drains with any number of resident workgroups: the earliest unfinished
task can always run); for the sweep it requires the band-update contributions each target
tile waits for to be published exactly once, with ranks in the order of their sources (so
every class queue, served first-in first-out, only waits for earlier tasks), and it executes
the sweep's rules with fixed numbers of band and update workers under random schedules,
which must all drain.  Shapes: the five layers (in 64-wide tiles), the odd sizes of the
parity tests and a few extremes.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "native", "schedule_check.cpp")
INC = os.path.join(ROOT, "two_sided_adaptive_amd", "csrc")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no C++ compiler")
    exe = str(tmp_path_factory.mktemp("sched") / "schedule_check")
    subprocess.run([cxx, "-std=c++17", "-O2", "-Wall", "-Werror", "-I", INC, "-o", exe, SRC],
                   check=True)
    return exe


def _run(exe, *args):
    r = subprocess.run([exe, *map(str, args)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr + r.stdout
    return r.stdout


# tiles of 64 per edge: 32 (C1), 512 (C2), 4096 (C3), 14336 / 4096 (C4), 8192 (C5), and the
# parity tests' odd orders (65, 130, 200, 257, 600, 1030, 1100)
@pytest.mark.parametrize("tiles", [(1, 1), (8, 8), (64, 64), (224, 64), (64, 224), (128, 128),
                                   (2, 3), (4, 2), (10, 17), (18,), (5,), (9, 1), (40, 33)])
def test_factor_queue_never_waits_for_a_later_task(checker, tiles):
    out = _run(checker, "factor", *tiles)
    assert "every wait met" in out


@pytest.mark.parametrize("blocks", [(64, 64), (224, 64), (64, 224), (128, 128), (1, 1), (1, 7),
                                    (7, 1), (2, 3), (5, 9), (16, 16), (21, 6), (3, 40)])
def test_sweep_contributions_complete_and_in_source_order(checker, blocks):
    out = _run(checker, "sweep", *blocks)
    assert "ranks complete" in out


# (blocks, XCDs, band workers per XCD, bands per group, near / next / far update workers):
# the five layers with the plans the sweep uses (eight XCDs; nine band workers in groups of
# eight bands for the 4096-wide layer, four in groups of four for the larger ones) and with
# the fewest workers the kernel allows (one per role), plus odd grids and XCD counts
SIM_CASES = [
    ((1, 1), 8, 1, 1, (1, 1, 1)), ((8, 8), 8, 3, 1, (4, 2, 17)),
    ((64, 64), 8, 9, 8, (32, 16, 136)), ((64, 64), 1, 1, 1, (1, 1, 1)),
    ((64, 64), 8, 1, 1, (1, 1, 1)), ((224, 64), 8, 4, 4, (40, 24, 160)),
    ((64, 224), 8, 4, 4, (40, 24, 160)), ((128, 128), 8, 4, 4, (40, 24, 160)),
    ((224, 64), 1, 1, 1, (1, 1, 1)), ((5, 9), 2, 1, 4, (1, 1, 1)), ((21, 6), 3, 2, 1, (1, 2, 1)),
    ((3, 40), 4, 2, 2, (2, 1, 3)), ((256, 16), 8, 4, 4, (40, 24, 160)),
]


@pytest.mark.parametrize("case", SIM_CASES, ids=lambda c: "x".join(map(str, c[0])) +
                         f"-{c[1]}xcd-{c[2]}bw-g{c[3]}-w" + "_".join(map(str, c[4])))
def test_sweep_drains_under_random_schedules(checker, case):
    # the rules executed with a fixed number of band and update workers, every enabled step
    # chosen at random: every schedule must finish (no worker set can wait on a task that
    # only a blocked worker could run)
    (mb, nb), nx, bw, gs, (wn, wx, wf) = case
    out = _run(checker, "run", mb, nb, nx, bw, gs, wn, wx, wf, 3)
    assert "random schedules drained" in out


@pytest.mark.parametrize("case", [((64, 64), 1), ((64, 64), 7), ((64, 64), 512), ((224, 64), 3),
                                  ((224, 64), 64), ((128,), 5), ((10, 17), 2), ((1, 1), 1)],
                         ids=lambda c: "x".join(map(str, c[0])) + f"-{c[1]}wg")
def test_factor_queue_drains_under_random_schedules(checker, case):
    # the factor's queue executed by a fixed number of workgroups (claims in queue order,
    # a task runs once its counters are met), enabled steps chosen at random
    tiles, wg = case
    out = _run(checker, "qrun", *tiles, wg, 2)
    assert "random schedules drained" in out
