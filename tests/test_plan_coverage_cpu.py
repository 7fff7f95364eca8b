"""The planner's launch plans, replayed on the CPU with the kernels' index
arithmetic: every element produced exactly once, every access inside its
buffer and 16-byte aligned where vectorised (see host/plan_coverage.cpp)."""

import subprocess
from pathlib import Path

ROOT = Path(__file__).resolve().parent.parent
CSRC = ROOT / "rank_reductions_amd" / "csrc"


def test_plan_coverage(tmp_path):
    exe = tmp_path / "plan_coverage"
    subprocess.run(["g++", "-std=c++17", "-O2", "-Wall", "-Werror", f"-I{ROOT / 'include'}", f"-I{CSRC}",
                    str(ROOT / "tests" / "host" / "plan_coverage.cpp"), str(CSRC / "plan.cpp"),
                    str(CSRC / "validate.cpp"), "-o", str(exe)], check=True)
    res = subprocess.run([str(exe), "300"], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "0 failures" in res.stdout
