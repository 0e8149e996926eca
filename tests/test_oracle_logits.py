"""Pins of the oracle's sampled verify from logits.

The fused verify is defined as the sampled verify of the warped rows
(llmstudio blog, sections 21-22 and 38: the verify compares the distributions
after the sampler's temperature step; spec-verify card, "Method"). The pin is
that composition, built from the two separately pinned oracle parts -- the
warp (pinned to torch.softmax) and the sampled verify on probabilities (pinned
by exact enumeration and the statistical tests) -- on every sequence, plus the
exact output law of the from-logits procedure itself on a tiny vocabulary.
"""
import numpy as np
import pytest

import oracle
from tests.exact_law import emitted_marginal, enumerate_law, prob_n_at_least


@pytest.mark.parametrize("T", [0.7, 1.0, 1.6])
@pytest.mark.parametrize("ragged", [False, True])
def test_logits_verify_equals_verify_of_warped_rows(T, ragged):
    rng = np.random.default_rng(int(T * 10) + ragged)
    B, K, V = 80, 5, 300
    zt = (3 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    zd = (zt[:, :K] + rng.standard_normal((B, K, V))).astype(np.float32)
    q = oracle.softmax_warp(zd, None, 0, T)
    # drafts drawn from q so that acceptance is realistic; a few out-of-range tokens
    t = np.array([[rng.choice(V, p=q[b, i]) for i in range(K)] for b in range(B)], dtype=np.int32)
    t[rng.random((B, K)) < 0.03] = V + 1
    u = rng.random((B, K + 1))
    lens = rng.integers(0, K + 1, size=B).astype(np.int32) if ragged else None
    p = oracle.softmax_warp(zt, None, 1, T)
    n1, x1, f1 = oracle.accept(p, q, t, u, lens)
    n2, x2, f2 = oracle.accept_logits(zt, zd, t, u, lens, T)
    np.testing.assert_array_equal(n1, n2)
    np.testing.assert_array_equal(x1, x2)
    np.testing.assert_array_equal(f1, f2)


def test_logits_verify_bf16_inputs():
    import torch
    g = torch.Generator().manual_seed(3)
    B, K, V = 16, 3, 1000
    zt = (4 * torch.randn(B, K + 1, V, generator=g)).to(torch.bfloat16)
    zd = (zt[:, :K].float() + torch.randn(B, K, V, generator=g)).to(torch.bfloat16)
    t = torch.randint(0, V, (B, K), generator=g, dtype=torch.int32)
    u = torch.rand(B, K + 1, generator=g)
    p = oracle.softmax_warp(zt, None, 1, 0.8)
    q = oracle.softmax_warp(zd, None, 0, 0.8)
    n1, x1, _ = oracle.accept(p, q, t, u)
    n2, x2, _ = oracle.accept_logits(zt, zd, t, u, None, 0.8)
    np.testing.assert_array_equal(n1, n2)
    np.testing.assert_array_equal(x1, x2)


def test_logits_verify_exact_law():
    """Exact law of the from-logits procedure on V = 6, K = 2: the emitted tokens follow softmax(z_t / T)."""
    rng = np.random.default_rng(9)
    K, V, T = 2, 6, 0.9
    zt = 2 * rng.standard_normal((K + 1, V))
    zd = zt[:K] + rng.standard_normal((K, V))
    p = np.exp(zt / T - (zt / T).max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    q = np.exp(zd / T - (zd / T).max(-1, keepdims=True))
    q /= q.sum(-1, keepdims=True)

    def run(P, Q, Tk, U):
        Bn = P.shape[0]
        n, nx, _ = oracle.accept_logits(np.broadcast_to(zt, (Bn, K + 1, V)).copy(),
                                        np.broadcast_to(zd, (Bn, K, V)).copy(), Tk, U, None, T)
        return n, nx

    law, bad = enumerate_law(p, q, run)
    assert bad == 0
    a = np.minimum(p[:K], q).sum(-1)
    for i in range(K + 1):
        assert prob_n_at_least(law, i) == pytest.approx(np.prod(a[:i]), abs=1e-12)
        np.testing.assert_allclose(emitted_marginal(law, i, V), np.prod(a[:i]) * p[i], atol=1e-12)


def test_abs_window_only_adds_flags():
    rng = np.random.default_rng(4)
    B, K, V = 60, 4, 200
    zt = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    zd = (zt[:, :K] + 0.3 * rng.standard_normal((B, K, V))).astype(np.float32)
    t = rng.integers(0, V, (B, K)).astype(np.int32)
    u = rng.random((B, K + 1))
    n1, x1, f1 = oracle.accept_logits(zt, zd, t, u)
    n2, x2, f2 = oracle.accept_logits(zt, zd, t, u, abs_window=1e-3)
    np.testing.assert_array_equal(n1, n2)
    np.testing.assert_array_equal(x1, x2)
    assert ((f1 & ~f2) == 0).all() and (f2 & oracle.FLAG_CDF).sum() >= (f1 & oracle.FLAG_CDF).sum()
