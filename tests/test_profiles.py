"""The rocprofv3 summaries under profiles/ name the commands that produced them.

Each command must run committed files only: the program after ``--`` is
``bench.py`` at the repository root, and every option given to it is one that
bench.py's argument parser defines. Runs on the CPU (reads text only).
"""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")


def _bench_flags():
    src = open(os.path.join(ROOT, "bench.py")).read()
    return set(re.findall(r'add_argument\(\s*"(--[a-z0-9-]+)"', src))


def _commands():
    out = []
    for name in sorted(os.listdir(PROFILES)):
        if not name.endswith(".md"):
            continue
        text = open(os.path.join(PROFILES, name)).read()
        for block in re.findall(r"```\n(.*?)```", text, flags=re.S):
            for line in block.splitlines():
                if line.startswith("rocprofv3"):
                    out.append((name, line))
    return out


def test_every_summary_names_its_command():
    names = [n for n in os.listdir(PROFILES) if n.endswith(".md")]
    assert names, "no profile summaries"
    with_cmd = {n for n, _ in _commands()}
    assert with_cmd == set(names), f"summaries without a rocprofv3 command: {set(names) - with_cmd}"


@pytest.mark.parametrize("name,cmd", _commands())
def test_command_runs_committed_bench(name, cmd):
    assert " -- " in cmd, f"{name}: the program must follow `--`"
    prog = cmd.split(" -- ", 1)[1].split()
    assert prog[:2] == ["python", "-u"] and prog[2] == "bench.py", f"{name}: {prog[:3]}"
    flags = _bench_flags()
    for tok in prog[3:]:
        if tok.startswith("--"):
            assert tok in flags, f"{name}: bench.py has no option {tok}"
    # rocprofv3's own options: counters never combined with tracing domains
    opts = cmd.split(" -- ", 1)[0]
    if "--pmc" in opts:
        for bad in ("--sys-trace", "--runtime-trace", "-s ", "-r ", "--hip-trace", "--hsa-trace", "--marker-trace"):
            assert bad not in opts + " ", f"{name}: --pmc combined with {bad.strip()}"
