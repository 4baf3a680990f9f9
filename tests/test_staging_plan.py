"""The staged path's piece planner, checked on the host.

tests/host/staging_plan_check.cpp includes the library's lema_slot.cpp and
checks plan_pieces on random slot layouts (coverage of every array byte of
each direction once, spans within one ring chunk, no array of the other
direction inside a span).  It is compiled here with hipcc as host code and
linked against the built liblema.so for the symbols lema_slot.cpp uses."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "optimizer_step_lema_amd")


def test_stage_piece_planner(tmp_path):
    from optimizer_step_lema_amd import build as B
    lib = os.path.join(PKG, "liblema.so")
    if not os.path.exists(lib):
        pytest.fail("liblema.so is not built")
    exe = str(tmp_path / "staging_plan_check")
    cmd = [B.hipcc(), "-std=c++17", "-O1", "-w", "-I" + B.INCLUDE, "-I" + B.CSRC,
           os.path.join(ROOT, "tests", "host", "staging_plan_check.cpp"),
           "-L" + PKG, "-llema", "-Wl,-rpath," + PKG, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
