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


def test_split_tile_counter_protocol(tmp_path):
    """Threads play the contributors of a split tile with schedule.h's
    first_finishes / other_finishes (the decisions finish_segment takes),
    with random delays and wait limits down to 0 (the hand-over): exactly
    one finisher, and every partial published before it reads them."""
    exe = str(tmp_path / "fixup_protocol_check")
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-pthread",
                    os.path.join(HERE, "fixup_protocol_check.cpp"), "-o", exe], check=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.strip().endswith("OK")
