"""Sanitized CPU builds (AddressSanitizer + UndefinedBehaviorSanitizer, any
report fatal):

  - the fp64 oracle, driven through every entry point on small inputs with
    edge cases (tests/sanitize/oracle_checks.c);
  - the oracle's whole pin suite (tests/test_oracle_*.py but the mutants, which
    load builds of their own) run on a sanitized build of the oracle library,
    the sanitizer runtimes preloaded into the test process;
  - the host side of libspecverify's C ABI, built from the same sources as the
    library (device code for gfx950, sanitizers on the host pass only) and
    driven through every documented argument error and every workspace-size
    query over its whole range, with no GPU (tests/sanitize/abi_checks.cpp).
"""
import os
import shutil
import subprocess
import sys

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


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], stdout=subprocess.PIPE, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("gcc") is None or _runtime("libasan.so") is None or _runtime("libubsan.so") is None,
                    reason="no gcc sanitizer runtimes")
@pytest.mark.skipif(bool(os.environ.get("LD_PRELOAD")), reason="the environment already preloads a library")
def test_oracle_pins_on_a_sanitized_oracle(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
         os.path.join(ROOT, "oracle", "sv_oracle.c"), "-lm", "-o", lib], str(tmp_path), 300)
    pins = sorted(os.path.join("tests", f) for f in os.listdir(os.path.join(ROOT, "tests"))
                  if f.startswith("test_oracle_") and f.endswith(".py") and "mutants" not in f)
    env = dict(SAN_ENV, SV_ORACLE_LIBRARY=lib, ASAN_OPTIONS="detect_leaks=0",  # the interpreter's own leaks
               LD_PRELOAD=f"{_runtime('libasan.so')} {_runtime('libubsan.so')}")
    out = run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-p", "no:xdist", "-m", "not gpu"] + pins,
              ROOT, 900, env)
    assert " passed" in out and "failed" not in out
    print(out.strip().splitlines()[-1])


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
