"""Compile the scheduler header for the host with g++ and run its checks."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_closed_form_full_tile_matches_tile_ranges(tmp_path):
    exe = tmp_path / "sched_check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-o", str(exe),
                    os.path.join(HERE, "native", "sched_check.cpp")], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "mismatches 0" in res.stdout
