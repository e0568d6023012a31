"""Build libattnres.so (HIP, gfx950) in-tree with hipcc.

Flags that matter for the numerics:
  -ffp-contract=off                   no implicit a*b+c -> fma; the kernels write
                                      every fma explicitly, so the add2 and
                                      no-add2 instantiations round identically
  -fno-gpu-flush-denormals-to-zero    IEEE binary32 denormals (the fold-add keeps
                                      subnormal sums)
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                      no packed binary32 instructions
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = [os.path.join(PKG, "csrc", n) for n in ("attnres.hip", "attnres_selftest.hip", "attnres_host.cpp")]
HEADERS = [os.path.join(PKG, "csrc", n) for n in ("attnres_device.hpp", "attnres_host.hpp")] + [
    os.path.join(ROOT, "include", "attnres.h")]
LIBRARY = os.path.join(PKG, "libattnres.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def build(output: str = LIBRARY, extra=(), quiet: bool = True) -> str:
    """Compile the library (always, even when a built one exists)."""
    tmp = output + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, *extra, "-I", os.path.join(ROOT, "include"), *SOURCES, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("libattnres build failed:\n%s\n%s" % (" ".join(cmd), res.stderr[-8000:]))
    if not quiet and res.stderr:
        sys.stderr.write(res.stderr[-4000:])
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    import time

    t = time.time()
    print(build(quiet=False), "%.1fs" % (time.time() - t))
