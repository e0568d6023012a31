"""libattnres from plain C: tests/native/c_caller.c includes include/attnres.h as
C99, links against libattnres.so and uses only the C ABI and the HIP runtime's
C API.  Without a GPU it checks the calls that are rejected before any HIP call;
on a GPU it runs one fused call whose outputs are compared with the oracle."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import parity as P
from attention_residual_rmsnorm_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "attention_residual_rmsnorm_amd")
SRC = os.path.join(ROOT, "tests", "native", "c_caller.c")
ROCM = "/opt/rocm"

pytestmark = pytest.mark.skipif(
    shutil.which("gcc") is None or not os.path.isdir(os.path.join(ROCM, "include", "hip"))
    or not os.path.exists(os.path.join(PKG, "libattnres.so")),
    reason="needs gcc, the ROCm headers and the built library")


@pytest.fixture(scope="module")
def caller(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("c_caller") / "c_caller")
    cmd = ["gcc", "-std=c99", "-O1", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC,
           "-L", PKG, "-lattnres", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath," + PKG, "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert "c_caller.c" not in r.stderr, r.stderr  # no warning in the caller itself
    return exe


def test_c_caller_abi(caller):
    r = subprocess.run([caller, "abi"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi ok" in r.stdout


@pytest.mark.gpu
@pytest.mark.parametrize("M,N,add2", [(3, 5, True), (2, 0, False), (40, 12, True)])
def test_c_caller_run(caller, orc, tmp_path, M, N, add2):
    case = W.make_case(cfg=64, M=M, N=N, add2=add2)
    src = tmp_path / "in.bin"
    dst = tmp_path / "out.bin"
    with open(src, "wb") as fh:
        fh.write(np.array([M, case.H, N, int(add2)], np.int64).tobytes())
        fh.write(np.array([case.eps], np.float32).tobytes())
        for t in [case.prefix, case.add] + ([case.add2] if add2 else []) + list(case.snapshots):
            fh.write(np.ascontiguousarray(t, np.uint16).tobytes())
        fh.write(np.ascontiguousarray(case.query, np.uint16).tobytes())
        fh.write(np.ascontiguousarray(case.gamma, np.uint16).tobytes())
    print("c caller run", M, N, add2, flush=True)
    r = subprocess.run([caller, "run", str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    out = np.fromfile(dst, np.uint16).reshape(2, M, case.H)
    rp, rn = P.run_oracle(orc, case)
    P.assert_parity(out[0], out[1], rp, rn, "C caller M=%d N=%d" % (M, N))
