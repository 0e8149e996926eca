"""Pins of the oracle's filtered warp (temperature, top-k, top-p, renormalise).

The sampler pipeline's order is the one the blog's section 38 gives; the
filters' exact semantics are readings: top-k keeps every id at least as large as
the k-th largest value, top-p keeps an id iff the mass strictly above it is
below top_p times the survivors' mass, one decision per group of equal values,
the most probable value always kept.

Pinned by: the `transformers` library's temperature / top-k / top-p warpers on
tie-free rows (an independent implementation of the same pipeline; its top-p
sorts ascending and cuts the cumulative mass at 1 - top_p), closed forms for
k = 1, ties and hand-built rows, and invariances.
"""
import functools

import numpy as np
import pytest
import torch

import oracle


@functools.lru_cache(maxsize=None)
def hf():
    try:
        from transformers.generation.logits_process import (TemperatureLogitsWarper, TopKLogitsWarper,
                                                            TopPLogitsWarper)
    except Exception:  # pragma: no cover - the library is part of this image
        pytest.skip("transformers is not importable")
    return TemperatureLogitsWarper, TopKLogitsWarper, TopPLogitsWarper


def hf_filtered(z, T, k, p):
    Temp, TopK, TopP = hf()
    s = torch.as_tensor(np.asarray(z, dtype=np.float64)).reshape(1, -1)
    s = Temp(T)(None, s)
    if 0 < k < s.shape[-1]:
        s = TopK(k)(None, s)
    if p < 1.0:
        s = TopP(p)(None, s)
    return torch.softmax(s, -1)[0].numpy()


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
@pytest.mark.parametrize("k,p,T", [(50, 1.0, 1.0), (0, 0.9, 1.0), (50, 0.9, 0.8), (7, 0.5, 1.3), (1000, 0.95, 0.7),
                                   (2, 0.999, 1.0), (300, 0.3, 2.0)])
def test_matches_transformers_warpers(dtype, k, p, T):
    rng = np.random.default_rng(k * 7 + int(p * 100))
    for _ in range(4):
        z = rng.permutation(np.unique((rng.standard_normal(6000) * rng.uniform(0.5, 5.0)).astype(dtype)))[:5000]
        assert len(np.unique(z)) == len(z) == 5000
        got, _ = oracle.warp_row_filtered(z, T, k, p)
        ref = hf_filtered(z, T, k, p)
        np.testing.assert_array_equal(got > 0, ref > 0)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-300)
        assert got.sum() == pytest.approx(1.0, abs=1e-12)


def test_bf16_rows_match_transformers():
    g = torch.Generator().manual_seed(3)
    z = (4 * torch.randn(20000, generator=g)).to(torch.bfloat16)
    zf = z.float().numpy()
    # bf16 has many exact ties: compare on the filter where ties cannot split (top-p only over a
    # distribution whose nucleus boundary group is checked by the tie tests below)
    got, _ = oracle.warp_row_filtered(z, 1.0, 40, 1.0)
    ref = hf_filtered(zf, 1.0, 40, 1.0)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-300)


def test_off_switches_equal_the_plain_warp():
    rng = np.random.default_rng(1)
    z = rng.standard_normal(999).astype(np.float32)
    plain = oracle.warp_row(z, 0.7)
    for k, p in [(0, 1.0), (-3, 1.0), (999, 1.0), (5000, 1.0), (0, float("nan")), (0, 1.5)]:
        got, fl = oracle.warp_row_filtered(z, 0.7, k, p)
        np.testing.assert_allclose(got, plain, rtol=1e-13, atol=0)  # sums in another order
        assert fl == 0


def test_top1_is_one_hot_and_ties_share():
    z = np.array([0.5, 3.0, -1.0, 2.0], dtype=np.float32)
    got, _ = oracle.warp_row_filtered(z, 1.0, 1, 1.0)
    np.testing.assert_array_equal(got, [0, 1, 0, 0])
    got, _ = oracle.warp_row_filtered(z, 1.0, 0, 1e-9)  # tiny top-p keeps the most probable value only
    np.testing.assert_array_equal(got, [0, 1, 0, 0])
    z = np.array([1.0, 3.0, 3.0, 0.0, 3.0], dtype=np.float32)
    for k, p in [(1, 1.0), (2, 1.0), (0, 0.01)]:
        got, _ = oracle.warp_row_filtered(z, 1.0, k, p)
        np.testing.assert_allclose(got, [0, 1 / 3, 1 / 3, 0, 1 / 3], rtol=1e-15)


def test_topk_keeps_every_tie_at_the_boundary():
    z = np.array([5.0, 4.0, 3.0, 4.0, 4.0, 1.0], dtype=np.float32)
    got, _ = oracle.warp_row_filtered(z, 1.0, 2, 1.0)
    w = np.exp(np.array([5.0, 4.0, 0, 4.0, 4.0, 0]) - 5.0) * np.array([1, 1, 0, 1, 1, 0])
    np.testing.assert_allclose(got, w / w.sum(), rtol=1e-15)
    got4, _ = oracle.warp_row_filtered(z, 1.0, 4, 1.0)
    np.testing.assert_array_equal(got4, got)
    got5, _ = oracle.warp_row_filtered(z, 1.0, 5, 1.0)
    assert (got5 > 0).sum() == 5 and got5[5] == 0


def test_topp_hand_built_rows_and_tie_groups():
    w = np.array([0.4, 0.2, 0.2, 0.1, 0.1])
    z = np.log(w)
    # mass above: 0.4-group 0, 0.2-group 0.4, 0.1-group 0.8
    got, _ = oracle.warp_row_filtered(z, 1.0, 0, 0.39)
    np.testing.assert_allclose(got, [1, 0, 0, 0, 0], atol=1e-15)
    got, _ = oracle.warp_row_filtered(z, 1.0, 0, 0.41)  # both 0.2s kept together
    np.testing.assert_allclose(got, [0.5, 0.25, 0.25, 0, 0], rtol=1e-12)
    got, _ = oracle.warp_row_filtered(z, 1.0, 0, 0.79)
    np.testing.assert_allclose(got, [0.5, 0.25, 0.25, 0, 0], rtol=1e-12)
    got, _ = oracle.warp_row_filtered(z, 1.0, 0, 0.81)
    np.testing.assert_allclose(got, w, rtol=1e-12)
    # top-p acts on the renormalised top-k survivors: k = 3 leaves (0.4, 0.2, 0.2) -> (0.5, 0.25, 0.25)
    got, _ = oracle.warp_row_filtered(z, 1.0, 3, 0.45)
    np.testing.assert_allclose(got, [1, 0, 0, 0, 0], atol=1e-15)
    got, _ = oracle.warp_row_filtered(z, 1.0, 3, 0.55)
    np.testing.assert_allclose(got, [0.5, 0.25, 0.25, 0, 0], rtol=1e-12)


def test_boundary_flag():
    w = np.array([0.4, 0.2, 0.2, 0.1, 0.1])
    z = np.log(w)
    _, fl = oracle.warp_row_filtered(z, 1.0, 0, 0.4 + 1e-7, window=1e-5)
    assert fl & oracle.FLAG_TOPP
    _, fl = oracle.warp_row_filtered(z, 1.0, 0, 0.45, window=1e-5)
    assert fl == 0
    # the most probable value is kept for any top_p: top_p = 0 or tiny is no close call
    for p in (0.0, 1e-7):
        _, fl = oracle.warp_row_filtered(z, 1.0, 0, p, window=1e-5)
        assert fl == 0


def test_invariances():
    rng = np.random.default_rng(5)
    z = rng.standard_normal(3000) * 3
    for k, p in [(40, 0.9), (0, 0.7), (500, 1.0)]:
        a, _ = oracle.warp_row_filtered(z, 0.9, k, p)
        b, _ = oracle.warp_row_filtered(z + 17.25, 0.9, k, p)
        np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-300)
        np.testing.assert_array_equal(a > 0, b > 0)
    # the top-k set does not depend on the temperature; the top-p set grows with top_p and with T
    s1 = oracle.warp_row_filtered(z, 0.5, 40, 1.0)[0] > 0
    s2 = oracle.warp_row_filtered(z, 2.0, 40, 1.0)[0] > 0
    np.testing.assert_array_equal(s1, s2)
    prev = None
    for p in [0.1, 0.3, 0.6, 0.9, 0.99]:
        cur = oracle.warp_row_filtered(z, 1.0, 0, p)[0] > 0
        if prev is not None:
            assert (cur | ~prev).all() and cur.sum() >= prev.sum()
        prev = cur
    lo = oracle.warp_row_filtered(z, 0.5, 0, 0.9)[0] > 0
    hi = oracle.warp_row_filtered(z, 2.0, 0, 0.9)[0] > 0
    assert (hi | ~lo).all()


def test_batched_per_sequence_parameters_and_ragged_rows():
    rng = np.random.default_rng(9)
    B, R, V = 5, 4, 777
    z = rng.standard_normal((B, R, V)).astype(np.float32)
    lens = np.array([0, 3, 1, 7, -2], dtype=np.int32)
    tk = np.array([0, 5, 100, 1, 20], dtype=np.int32)
    tp = np.array([0.9, 1.0, 0.5, 0.3, 2.0], dtype=np.float32)
    out, flags = oracle.softmax_warp_filtered(z, lens, 1, 0.8, tk, tp)
    for b in range(B):
        live = min(R - 1, max(0, lens[b])) + 1
        for r in range(R):
            if r < live:
                ref, _ = oracle.warp_row_filtered(z[b, r], 0.8, int(tk[b]), float(tp[b]))
                np.testing.assert_array_equal(out[b, r], ref)
            else:
                assert np.isnan(out[b, r]).all()
    assert flags.shape == (B, R)
    out2, _ = oracle.softmax_warp_filtered(z, lens, 1, 0.8, None, None)
    np.testing.assert_allclose(out2, oracle.softmax_warp(z, lens, 1, 0.8), rtol=1e-13, atol=0)
