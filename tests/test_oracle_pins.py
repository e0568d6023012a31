"""CPU tests: pin the oracle to values the pages and the mathematics fix.

The oracle is what the GPU path is compared against, so it is itself checked
against independent routes first (see ``pins.py``).  Exhaustive rounding
checks run all 2^32 inputs through a test-side C checker.
"""
import os
import subprocess

import pytest

import pins

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("check", pins.QUICK, ids=lambda c: c.__name__)
def test_pin(orc, check):
    check(orc)


def test_round_vs_fractions(orc):
    pins.check_round_vs_fractions(orc)


def test_torch_keeps_subnormals():
    """The PyTorch library pin is meaningful only if its CPU bf16 add keeps
    subnormals on this host (some bf16 conversion instructions flush them)."""
    import numpy as np

    t = pins.bits_of(pins.tbf(np.array([0x0081], np.uint16)) + pins.tbf(np.array([0x8080], np.uint16)))
    assert t[0] == 0x0001


def build_checker(native_dir):
    exe = os.path.join(str(native_dir), "exhaustive_rounding")
    if not os.path.exists(exe):
        subprocess.run(["gcc", "-O2", "-pthread", "-o", exe,
                        os.path.join(HERE, "native", "exhaustive_rounding.c"), "-ldl"], check=True)
    return exe


def run_exhaustive(exe, lib, mode, threads=None):
    threads = threads or max(1, min(16, os.cpu_count() or 1))
    res = subprocess.run([exe, lib, mode, str(threads)], capture_output=True, text=True, timeout=900)
    return res.returncode, res.stdout + res.stderr


@pytest.mark.slow
@pytest.mark.parametrize("mode", ["round", "add"])
def test_exhaustive(orc, native_dir, mode):
    """mode round: every binary32 -> bf16; mode add: every pair of bf16
    patterns through the binary32 add, against the exact integer sum."""
    exe = build_checker(native_dir)
    rc, out = run_exhaustive(exe, orc.path, mode)
    assert rc == 0 and "mismatches 0" in out, out
