"""Layout functions of the search kernels, checked on the host: the gates'
table (group, pair and lane-bound regions in order, without overlap), and the
work-item order: the slot order (item_place) is a bijection onto the
column-group x segment-block grid rounded up to powers of two, with the column
group fastest inside a tile, and the parts (item_part) cover the slots once.
item_order_check.cpp calls the constexpr functions of plan.h that the kernels
call."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_item_order(tmp_path):
    exe = tmp_path / "item_order_check"
    subprocess.run(["g++", "-std=c++17", "-O2", "-Wall", "-Werror",
                    "-I" + os.path.join(ROOT, "include"),
                    "-I" + os.path.join(ROOT, "ising_ground_state_amd", "csrc"),
                    os.path.join(ROOT, "tests", "item_order_check.cpp"), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout + out.stderr
