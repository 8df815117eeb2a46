"""Segment plans and grid limits of the long-row paths, checked on the CPU.

The segmented launches park two float64 values in the first elements of each
segment's own output range between their passes.  tests/plan_check.cpp compiles
the launcher's planning header (csrc/rlscan_plan.hpp) with the host C++ compiler
and walks every plan the launcher can make over 1..65 rows, every row length
from 16000 to 40000 steps, lengths k*len + r (r = -8..8) up to 2^30 - 1 steps and
several compute-unit counts: every segment must hold at least the 8 elements
the parked pair takes in a 16-bit format, and the segments must tile the row.
The same checks must reject the rule the launcher used before (segment count
rounded up), whose last segment could hold a single step.  The time-major item
form's shape rule is walked too: every shape it takes has whole 64-step chunks
(at least one) and whole blocks, so its loader and compute waves meet the same
number of barriers.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_recurrence_scan_reverse_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "plan_check.cpp")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("plan") / "plan_check")
    subprocess.run([cxx, "-O2", "-std=c++17", "-Wall", "-Werror", "-I" + CSRC, SRC, "-o", exe], check=True)
    return exe


def test_every_plan_keeps_parked_values_inside_their_segment(checker):
    res = subprocess.run([checker], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("OK"), res.stdout


def test_the_rounded_up_segment_count_is_rejected(checker):
    res = subprocess.run([checker, "--ceil-rule"], capture_output=True, text=True, timeout=120)
    assert res.returncode != 0, res.stdout
    assert "E=1 T=16385" in res.stdout and "parked" in res.stdout, res.stdout
