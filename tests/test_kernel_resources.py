"""Compile-time resource checks of every kernel in libspecverify (no GPU).

The build keeps the compiler's kernel-resource-usage report beside the
library. Two properties the kernels' speed depends on, and that a harmless
looking source change can silently break:
  - no private (scratch) memory: a spill, a dynamically indexed local array,
    or a device function the inliner left out of line (a call passes its
    reference arguments through the stack) all show up as scratch;
  - 8 wavefronts per SIMD: the 1024-lane workgroups (warp rows, filtered warp,
    greedy, accept) fit two to a compute unit only at <= 64 VGPRs; at 65 half
    the workgroups wait (the filtered warp measured 25% slower that way).
"""
import json
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "draft_token_verification_amd")
RESOURCES = os.path.join(PKG, "libspecverify.resources.json")
CSRC = os.path.join(PKG, "csrc")

KERNELS = ["accept_kernel", "accept_logits_kernel", "accept_logits_sliced_kernel", "commit_kernel", "fill_empty",
           "fill_slots", "gate_choose_kernel", "gate_update_kernel", "greedy_kernel", "greedy_sliced_kernel",
           "warp_coop_kernel",
           "warp_filter_kernel", "warp_rows_kernel", "penalty_table_kernel", "penalty_rows_kernel"]


@pytest.fixture(scope="module")
def res():
    lib = os.path.join(PKG, "libspecverify.so")
    if not os.path.exists(RESOURCES) or (os.path.exists(lib) and os.path.getmtime(RESOURCES) + 60 <
                                         os.path.getmtime(lib)):
        pytest.fail("no resource report for the built library: run draft_token_verification_amd/build.py")
    return json.load(open(RESOURCES))


def short(mangled):
    m = re.match(r"_ZN2sv12_GLOBAL__N_1\d+(\w+?)(I|E)", mangled)
    return m.group(1) if m else mangled


def test_report_covers_every_kernel(res):
    names = {short(k) for k in res}
    src = " ".join(open(os.path.join(CSRC, f)).read() for f in os.listdir(CSRC) if f.endswith(".hip"))
    declared = set(re.findall(r"__global__[^;{]*?\bvoid\s+(\w+)\s*\(", src, flags=re.S))
    assert declared == set(KERNELS)
    assert names == declared


def test_no_scratch(res):
    bad = {short(k): v["scratch"] for k, v in res.items() if v.get("scratch", 0) != 0}
    assert not bad, f"kernels using private memory (spills, local arrays or out-of-line calls): {bad}"


def test_full_occupancy(res):
    low = {short(k): (v["vgprs"], v["occupancy"]) for k, v in res.items() if v.get("occupancy", 0) < 8}
    assert not low, f"kernels below 8 waves per SIMD (vgprs, waves): {low}"


def test_filter_fits_two_workgroups_per_cu(res):
    for k, v in res.items():
        if short(k) == "warp_filter_kernel":
            assert v["vgprs"] <= 64 and 2 * v["lds"] <= 160 * 1024, (k, v)
