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
    One kernel is exempt, with a floor of its own: the split fused sampled
    verify keeps each lane's share of the target row in registers through
    its exchanges and is bound by arithmetic, not by memory; forced to 64
    VGPRs it spills and ran 3.8x slower on MI355X, at its natural ~110 VGPRs
    (4 waves per SIMD) it is fastest. Its element-by-element variant (rows
    whose length or alignment rules out 16-byte loads) is exempt from the
    floor as well: it is correct but not tuned.
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


FLOOR = {"accept_logits_sliced_kernel": 4}  # waves per SIMD, for the 16-byte-load variants


def vector_variant(mangled):
    """True for the <BF16, VEC = true> instantiations (the second template argument)."""
    m = re.search(r"ILb[01]ELb([01])E", mangled)
    return m is None or m.group(1) == "1"


def test_full_occupancy(res):
    low = {}
    for k, v in res.items():
        name = short(k)
        if name in FLOOR:
            if vector_variant(k) and v.get("occupancy", 0) < FLOOR[name]:
                low[name] = (v["vgprs"], v["occupancy"])
        elif v.get("occupancy", 0) < 8:
            low[name] = (v["vgprs"], v["occupancy"])
    assert not low, f"kernels below their waves per SIMD (vgprs, waves): {low}"


def test_filter_fits_two_workgroups_per_cu(res):
    for k, v in res.items():
        if short(k) == "warp_filter_kernel":
            assert v["vgprs"] <= 64 and 2 * v["lds"] <= 160 * 1024, (k, v)
