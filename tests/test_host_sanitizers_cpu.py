"""The host-only layers (session, validation, planner) under AddressSanitizer +
UndefinedBehaviorSanitizer and ThreadSanitizer, built with g++ on the CPU:
a multi-threaded stress of the C ABI with random and malformed arguments, and
the planner coverage replay."""

import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
CSRC = ROOT / "rank_reductions_amd" / "csrc"
HOST = ROOT / "tests" / "host"


def build(tmp_path, name, sources, sanitize):
    exe = tmp_path / name
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", f"-fsanitize={sanitize}",
                    "-fno-sanitize-recover=all", f"-I{ROOT / 'include'}", f"-I{CSRC}", *map(str, sources),
                    "-o", str(exe), "-lpthread"], check=True)
    return exe


@pytest.mark.parametrize("sanitize", ["address,undefined", "thread"])
def test_abi_stress(tmp_path, sanitize):
    exe = build(tmp_path, "abi_stress", [HOST / "abi_stress.cpp", CSRC / "session.cpp", CSRC / "validate.cpp",
                                         CSRC / "plan.cpp"], sanitize)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "0 bad results" in res.stdout


def test_plan_coverage_sanitized(tmp_path):
    exe = build(tmp_path, "plan_coverage", [HOST / "plan_coverage.cpp", CSRC / "plan.cpp", CSRC / "validate.cpp"],
                "address,undefined")
    res = subprocess.run([str(exe), "60"], capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "0 failures" in res.stdout
