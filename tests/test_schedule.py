"""CPU check of the (tile, stage) work decomposition used by the kernel."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_schedule_partition(tmp_path):
    exe = str(tmp_path / "sched_check")
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", os.path.join(HERE, "sched_check.cpp"), "-o", exe],
                   check=True)
    out = subprocess.run([exe], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.strip().endswith("OK")
