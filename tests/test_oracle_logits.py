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


def test_logits_verify_flags_use_relative_windows():
    """The boundary flags of the verify from logits are the relative windows of the
    verify on probabilities: a draw threshold at a cumulative weight C is flagged
    within 1e-5 * C of it and not beyond, however small C is (a residual of total
    mass 1e-3 is judged on its own scale), and a realistic batch flags almost
    nothing."""
    V = 4
    # target row 0 and draft row 0 differ only in ids 0 and 1: the residual sits on id 0 alone
    zt = np.log(np.array([[[0.25, 0.25, 0.25, 0.25], [0.4, 0.3, 0.2, 0.1]]]))
    zd = np.log(np.array([[[0.2495, 0.2505, 0.25, 0.25]]]))
    p = np.exp(zt[0, 0]) / np.exp(zt[0, 0]).sum()
    q = np.exp(zd[0, 0]) / np.exp(zd[0, 0]).sum()
    rho = p[0] / q[0]
    w = np.maximum(p - q, 0.0)
    assert w[0] > 0 and w[1:].sum() == 0  # all residual mass on id 0: a draw can only give 0
    t = np.array([[0]], dtype=np.int32)
    for u0, flagged in ((rho * 0.999, False), (rho * (1 - 3e-6), True), (rho * (1 + 3e-6), True),
                        (min(rho * 1.001, 0.9999), False)):
        _, _, fl = oracle.accept_logits(zt, zd, t, np.array([[u0, 0.5]]), None, 1.0)
        assert bool(fl[0] & oracle.FLAG_RATIO) == flagged, (u0, rho)
    # a residual of mass ~1e-3 split over ids 0 and 2: the boundary C(0) = w0 is
    # flagged within 1e-5 * w0 (a few 1e-9 absolute), not at 1e-5 absolute
    zd = np.log(np.array([[[0.2495, 0.2505, 0.2495, 0.2505]]]))
    q = np.exp(zd[0, 0]) / np.exp(zd[0, 0]).sum()
    w = np.maximum(p - q, 0.0)
    S = w.sum()
    assert w[0] > 0 and w[2] > 0 and 1e-4 < S < 1e-2
    t = np.array([[1]], dtype=np.int32)  # p/q < 1 at id 1; u = 0.9999 rejects
    for frac, flagged, want in ((1 - 3e-6, True, 0), (1 + 3e-6, True, 2), (0.999, False, 0), (1.001, False, 2)):
        uf = w[0] * frac / S
        n, nx, fl = oracle.accept_logits(zt, zd, t, np.array([[0.9999, uf]]), None, 1.0)
        assert n[0] == 0 and nx[0] == want, (frac, nx[0])
        assert bool(fl[0] & oracle.FLAG_CDF) == flagged, frac
    # the realistic batch: almost nothing flagged
    rng = np.random.default_rng(4)
    B, K, V = 300, 4, 400
    zt = (3 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    zd = (zt[:, :K] + rng.uniform(0.1, 3.0, (B, 1, 1)) * rng.standard_normal((B, K, V))).astype(np.float32)
    q = oracle.softmax_warp(zd, None, 0, 1.0)
    t = np.array([[rng.choice(V, p=q[b, i]) for i in range(K)] for b in range(B)], dtype=np.int32)
    u = rng.random((B, K + 1))
    _, _, fl = oracle.accept_logits(zt, zd, t, u, None, 1.0)
    assert ((fl & (oracle.FLAG_RATIO | oracle.FLAG_CDF)) != 0).sum() <= 3
