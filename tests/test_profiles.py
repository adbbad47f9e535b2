"""The rocprofv3 summaries under profiles/ name the commands that produced them; those
commands must run committed files with options those files accept (CPU only: the options
are checked against bench.py's own --help, nothing is profiled)."""
import glob
import os
import re
import shlex
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md")))


def _commands(path):
    """The rocprofv3 command lines inside the summary's code blocks."""
    out, inside = [], False
    for line in open(path):
        line = line.strip()
        if line.startswith("```"):
            inside = not inside
        elif inside and line.startswith("rocprofv3 "):
            out.append(shlex.split(line))
    return out


@pytest.fixture(scope="module")
def bench_options():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                         capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert res.returncode == 0, res.stderr
    return set(re.findall(r"(--[a-z0-9-]+)", res.stdout))


def test_every_summary_names_its_commands():
    assert PROFILES
    for path in PROFILES:
        assert _commands(path), f"{os.path.basename(path)} names no rocprofv3 command"


@pytest.mark.parametrize("path", PROFILES, ids=os.path.basename)
def test_profile_commands_run_committed_files(path, bench_options):
    for cmd in _commands(path):
        assert "--" in cmd, cmd
        prog = cmd[cmd.index("--") + 1:]
        # the program itself follows "--" (no launcher in between): python3 <committed script>
        assert prog[0] in ("python3", "python"), cmd
        script = os.path.join(ROOT, prog[1])
        assert os.path.isfile(script), f"{prog[1]} is not in the repository"
        assert not prog[1].startswith("_work"), cmd
        if os.path.basename(script) == "bench.py":
            for arg in prog[2:]:
                if arg.startswith("--"):
                    opt = arg.split("=")[0]
                    assert opt in bench_options, f"{os.path.basename(path)}: bench.py has no {opt}"
        # results go under gpurun_out/, raw profiler output is not committed
        assert cmd[cmd.index("-d") + 1].startswith("gpurun_out/"), cmd
