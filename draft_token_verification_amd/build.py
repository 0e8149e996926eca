"""Build libspecverify.so (gfx950) in-tree with hipcc.

Every source under csrc/ is compiled into one shared library next to this
file. Packed-fp32 instructions are disabled for the device code.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libspecverify.so")
SOURCES = ["api.hip", "greedy.hip", "accept.hip", "warp.hip", "filter.hip", "gate.hip", "commit.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def command(out=OUT):
    return [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall", "-Wno-unused-result",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            "-o", out] + [os.path.join(CSRC, s) for s in SOURCES]


def build(verbose: bool = False) -> str:
    tmp = OUT + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
