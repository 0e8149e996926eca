"""Build libspecverify.so (gfx950) in-tree with hipcc.

Every source under csrc/ is compiled into one shared library next to this
file. Packed-fp32 instructions are disabled for the device code. The
compiler's per-kernel resource report (registers, scratch, occupancy, LDS) is
kept beside the library as libspecverify.resources.json.
"""
import json
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libspecverify.so")
RESOURCES = os.path.join(HERE, "libspecverify.resources.json")
SOURCES = ["api.hip", "greedy.hip", "accept.hip", "warp.hip", "filter.hip", "penalty.hip", "gate.hip", "commit.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def command(out=OUT):
    return [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall", "-Wno-unused-result",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Rpass-analysis=kernel-resource-usage",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            "-o", out] + [os.path.join(CSRC, s) for s in SOURCES]


def parse_resources(text: str) -> dict:
    """Kernel name -> {vgprs, agprs, sgprs, scratch, occupancy, lds} from the
    compiler's kernel-resource-usage remarks."""
    fields = {"VGPRs": "vgprs", "AGPRs": "agprs", "TotalSGPRs": "sgprs", "ScratchSize [bytes/lane]": "scratch",
              "Occupancy [waves/SIMD]": "occupancy", "LDS Size [bytes/block]": "lds"}
    out, cur = {}, None
    for line in text.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([^:]+(?:\[[^\]]*\])?): (\d+)", line)
        if m and cur is not None and m.group(1).strip() in fields:
            cur[fields[m.group(1).strip()]] = int(m.group(2))
    return out


def build(verbose: bool = False) -> str:
    tmp = OUT + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    log = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "remark:" not in l)
    if r.returncode != 0:
        sys.stderr.write(log + "\n")
        raise subprocess.CalledProcessError(r.returncode, cmd)
    if verbose and log.strip():
        sys.stderr.write(log + "\n")
    with open(RESOURCES, "w") as f:
        json.dump(parse_resources(r.stderr), f, indent=1, sort_keys=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
