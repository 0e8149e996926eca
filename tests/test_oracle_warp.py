"""Pins of the oracle's temperature warp p = softmax(z / T).

Library routine: torch.softmax in fp64 on the CPU on the same values.
Invariants: every row sums to one; adding a constant to a row changes
nothing; T scales the logits; ragged calls touch only live rows.
"""
import numpy as np
import pytest
import torch

import oracle


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float64])
@pytest.mark.parametrize("T", [0.8, 1.0, 2.5])
def test_warp_matches_torch_softmax_fp64(dtype, T):
    g = torch.Generator().manual_seed(17)
    z = (4.0 * torch.randn(6, 5003, generator=g)).to(dtype)
    ref = torch.softmax(z.double() / T, dim=-1).numpy()
    for r in range(z.shape[0]):
        p = oracle.warp_row(z[r], T)
        np.testing.assert_allclose(p, ref[r], atol=1e-15, rtol=1e-12)
        assert p.sum() == pytest.approx(1.0, abs=1e-12)


def test_warp_shift_invariance_and_extremes():
    rng = np.random.default_rng(1)
    z = rng.standard_normal(1000) * 10
    np.testing.assert_allclose(oracle.warp_row(z + 3.0), oracle.warp_row(z), atol=1e-15)
    np.testing.assert_allclose(oracle.warp_row(z * 2.0, 2.0), oracle.warp_row(z), atol=1e-15)
    big = np.array([1e4, 0.0, -1e4, 1e4 - 1.0])
    p = oracle.warp_row(big)
    assert np.isfinite(p).all() and p.sum() == pytest.approx(1.0)
    assert p[0] == pytest.approx(1.0 / (1.0 + np.exp(-1.0)))
    assert oracle.warp_row(np.array([3.0]))[0] == 1.0
    np.testing.assert_allclose(oracle.warp_row(np.zeros(7, dtype=np.float32)), np.full(7, 1 / 7), atol=1e-16)


def test_softmax_warp_ragged_rows():
    rng = np.random.default_rng(2)
    B, K, V = 9, 4, 300
    z = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    lens = np.array([0, 1, 2, 3, 4, 5, -1, 9, 2], dtype=np.int32)
    out = oracle.softmax_warp(z, lens, extra_rows=1, T=0.7)
    for b in range(B):
        live = min(K, max(0, lens[b])) + 1
        for r in range(K + 1):
            if r < live:
                np.testing.assert_allclose(out[b, r], oracle.warp_row(z[b, r], 0.7), atol=0)
            else:
                assert np.isnan(out[b, r]).all()
    out_d = oracle.softmax_warp(z[:, :K], lens, extra_rows=0, T=0.7)
    for b in range(B):
        live = min(K, max(0, lens[b]))
        assert np.isfinite(out_d[b, :live]).all() and np.isnan(out_d[b, live:]).all()
