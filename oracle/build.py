"""Build the CPU oracle shared library with gcc.

Test infrastructure only: the tests, the smoke check and the CPU-baseline leg
of the benchmark load what this builds; the product path never does.

Flags: ``-O2 -fno-fast-math -ffp-contract=off`` keeps binary32 adds as
round-to-nearest-even with gradual underflow (no FTZ/DAZ start-up code) and
forbids contracting a*b+c into an FMA.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "attnres_oracle.c")
LIBRARY = os.path.join(HERE, "liboracle_attnres.so")

CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c11", "-Wall",
          "-Wextra", "-fPIC", "-shared"]


def build(source: str = SOURCE, output: str = LIBRARY, quiet: bool = True) -> str:
    """Compile ``source`` into the shared library ``output`` and return its path."""
    tmp = output + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, "-I", HERE, source, "-o", tmp, "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("oracle build failed:\n%s\n%s" % (" ".join(cmd), res.stderr))
    if not quiet and res.stderr:
        sys.stderr.write(res.stderr)
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build(quiet=False))
