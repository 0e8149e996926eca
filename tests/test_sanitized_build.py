"""Sanitized CPU builds (AddressSanitizer + UndefinedBehaviorSanitizer, any
report fatal):

  - the fp64 oracle, driven through every entry point on small inputs with
    edge cases (tests/sanitize/oracle_checks.c);
  - the host side of libspecverify's C ABI, built from the same sources as the
    library (device code for gfx950, sanitizers on the host pass only) and
    driven through every documented argument error and every workspace-size
    query over its whole range, with no GPU (tests/sanitize/abi_checks.cpp).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "draft_token_verification_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def run(cmd, cwd, timeout, env=None):
    r = subprocess.run(cmd, cwd=cwd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=timeout,
                       env=env)
    assert r.returncode == 0, f"{cmd[0]} exited {r.returncode}:\n{r.stdout[-4000:]}"
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_checks")
    run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", "-fopenmp", "-ffp-contract=off", "-I", os.path.join(ROOT, "oracle"),
         os.path.join(HERE, "oracle_checks.c"), os.path.join(ROOT, "oracle", "sv_oracle.c"), "-lm", "-o", exe],
        str(tmp_path), 300)
    out = run([exe], str(tmp_path), 300, SAN_ENV)
    assert "oracle checks clean" in out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="no hipcc")
def test_abi_host_checks_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_checks")
    sources = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    # the sanitizers apply to the host pass only (each flag behind -Xarch_host)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]  # noqa: E501
    run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops"] + san + ["-I", os.path.join(ROOT, "include"), "-I", CSRC] + sources +
        [os.path.join(HERE, "abi_checks.cpp"), "-o", exe], str(tmp_path), 600)
    out = run([exe], str(tmp_path), 300, SAN_ENV)
    assert "abi host checks: 0 failures" in out
