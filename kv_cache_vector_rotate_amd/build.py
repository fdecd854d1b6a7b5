"""Build the HIP library (libtq.so) in-tree with hipcc for gfx950."""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libtq.so")
SOURCES = [os.path.join(HERE, "csrc", "tq_host.cpp"), os.path.join(HERE, "csrc", "tq_kernels.hip"),
           os.path.join(HERE, "csrc", "tq_wide.hip"), os.path.join(HERE, "csrc", "tq_wider.hip")]


def hipcc_command(out=LIB):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    return [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-Wno-unused-function",
            # packed fp32 VALU forms are left to nothing but scalar code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), *SOURCES, "-o", out]


def build(verbose=True):
    tmp = LIB + ".tmp"
    cmd = hipcc_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if res.returncode != 0:
        sys.stderr.write(err + "\n")
        raise RuntimeError("hipcc failed building libtq.so")
    if err and verbose:
        sys.stderr.write(err + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
