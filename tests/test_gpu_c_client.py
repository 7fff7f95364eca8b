"""The C ABI from a plain C program (tests/host/c_client.c, built with gcc
against include/rc.h, librankred.so and the HIP runtime; no Python or torch in
the process): all_reduce Sum and reduce_scatter Max on 4 and 7 ranks, bits
against the CPU oracle."""

import subprocess
from pathlib import Path

import numpy as np
import pytest

import oracle
import rank_reductions_amd as rr
import synth_inputs as si
from gpu_util import assert_bits

pytestmark = pytest.mark.gpu
ROOT = Path(__file__).resolve().parent.parent


@pytest.fixture(scope="module")
def client(tmp_path_factory):
    exe = tmp_path_factory.mktemp("c_client") / "c_client"
    lib_dir = rr.library_path().parent
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", f"-I{ROOT / 'include'}",
                    "-I/opt/rocm/include", str(ROOT / "tests" / "host" / "c_client.c"), f"-L{lib_dir}", "-lrankred",
                    "-L/opt/rocm/lib", "-lamdhip64", f"-Wl,-rpath,{lib_dir}", "-Wl,-rpath,/opt/rocm/lib",
                    "-o", str(exe)], check=True)
    return exe


@pytest.mark.parametrize("R,N", [(4, 1_000_004), (7, 7 * 30_011)])
def test_c_client(client, tmp_path, R, N):
    xs = si.numpy_rank_inputs(R, N, "f32", "normal", 500 + R)
    inp, outp = tmp_path / "in.bin", tmp_path / "out.bin"
    np.concatenate(xs).astype(np.float32).tofile(inp)
    res = subprocess.run([str(client), str(R), str(N), str(inp), str(outp)], capture_output=True, text=True,
                         timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    got = np.fromfile(outp, dtype=np.float32)
    assert got.size == N + N
    assert_bits(got[:N], oracle.all_reduce_closed_form(xs, "sum"), f"R={R} all_reduce from C")
    want = np.concatenate(oracle.reduce_scatter(xs, "max"))
    assert_bits(got[N:], want, f"R={R} reduce_scatter from C")
