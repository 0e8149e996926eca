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


# ---- the draft distribution given by its log-normaliser (or_accept_logits_lse, R29) ----

def exact_lse(z, T):
    """log sum_x exp(z_x / T) of every row, with a compensated sum (math.fsum)."""
    import math
    y = np.asarray(z, dtype=np.float64) / T
    m = y.max(-1, keepdims=True)
    flat = (y - m).reshape(-1, y.shape[-1])
    s = np.array([math.fsum(np.exp(r)) for r in flat]).reshape(y.shape[:-1])
    return m[..., 0] + np.log(s)


@pytest.mark.parametrize("T", [0.8, 1.3])
def test_logits_verify_given_true_lse_matches_normalised(T):
    """With each draft row's true log-normaliser (rounded to fp32), the verify
    with a given normaliser decides and draws as the one that normalises the
    rows itself, on every sequence the latter does not flag."""
    rng = np.random.default_rng(int(T * 100))
    B, K, V = 60, 5, 300
    zt = (3 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    zd = (zt[:, :K] + rng.standard_normal((B, K, V))).astype(np.float32)
    q = oracle.softmax_warp(zd, None, 0, T)
    t = np.array([[rng.choice(V, p=q[b, i]) for i in range(K)] for b in range(B)], dtype=np.int32)
    t[rng.random((B, K)) < 0.03] = V + 1
    u = rng.random((B, K + 1))
    lens = rng.integers(0, K + 1, size=B).astype(np.int32)
    lse = exact_lse(zd, T).astype(np.float32)
    n1, x1, f1 = oracle.accept_logits(zt, zd, t, u, lens, T)
    n2, x2, _ = oracle.accept_logits(zt, zd, t, u, lens, T, draft_lse=lse)
    ok = f1 == 0
    assert ok.sum() >= B - 2
    np.testing.assert_array_equal(n1[ok], n2[ok])
    np.testing.assert_array_equal(x1[ok], x2[ok])


@pytest.mark.parametrize("c", [2.0, 0.5])
def test_logits_verify_given_lse_exact_law(c):
    """A normaliser larger than the row's by log(c) scales q by 1/c: exact
    law on V = 5, K = 2 with draft tokens drawn from the true q. Position i
    accepts with probability sum_x min(q_i(x), c * p_i(x)), and the emitted
    token mixes the accepted draft token with the residual max(0, p - q / c)
    (closed forms of the accept-or-resample step with q / c in place of q)."""
    rng = np.random.default_rng(int(10 * c))
    K, V, T = 2, 5, 0.9
    zt = 1.5 * rng.standard_normal((K + 1, V))
    zd = zt[:K] + rng.standard_normal((K, V))
    sm = lambda y: np.exp(y - y.max(-1, keepdims=True)) / np.exp(y - y.max(-1, keepdims=True)).sum(-1, keepdims=True)
    p, q = sm(zt / T), sm(zd / T)
    lse = (exact_lse(zd, T) + np.log(c)).astype(np.float32)
    qs = np.exp(zd / T - lse.astype(np.float64)[:, None])  # the q the procedure uses: about q / c

    def run(P, Q, Tk, U):
        Bn = P.shape[0]
        n, nx, _ = oracle.accept_logits(np.broadcast_to(zt, (Bn, K + 1, V)).copy(),
                                        np.broadcast_to(zd, (Bn, K, V)).copy(), Tk, U, None, T,
                                        draft_lse=np.broadcast_to(lse, (Bn, K)).copy())
        return n, nx

    law, bad = enumerate_law(p, qs, run)
    assert bad == 0
    scale = np.prod(qs.sum(-1))  # the enumeration weighs draft tuples by qs, which sums to about 1/c per row
    a = np.minimum(q, c * p[:K]).sum(-1)
    for i in range(K + 1):
        assert prob_n_at_least(law, i) / scale == pytest.approx(np.prod(a[:i]), abs=1e-6)
    for i in range(K):
        r = np.maximum(0.0, p[i] - q[i] / c)
        r = r / r.sum() if r.sum() > 0 else p[i]
        want = np.prod(a[:i]) * (np.minimum(q[i], c * p[i]) + (1.0 - a[i]) * r)
        np.testing.assert_allclose(emitted_marginal(law, i, V) / scale, want, atol=1e-6)
    np.testing.assert_allclose(emitted_marginal(law, K, V) / scale, np.prod(a) * p[K], atol=1e-6)


def test_logits_verify_given_infinite_lse_accepts_everything():
    """lse = +inf makes q = 0: every in-range draft token is accepted and the
    bonus is the inverse CDF of softmax(z_target,K_b / T) at u[K_b]; an
    out-of-range token still stops the walk there (R7)."""
    import torch
    rng = np.random.default_rng(12)
    B, K, V, T = 20, 4, 50, 1.1
    zt = (2 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    zd = (2 * rng.standard_normal((B, K, V))).astype(np.float32)
    t = rng.integers(0, V, (B, K)).astype(np.int32)
    t[3, 2] = -1
    u = rng.random((B, K + 1))
    lens = rng.integers(0, K + 1, size=B).astype(np.int32)
    lens[3] = K
    n, nx, _ = oracle.accept_logits(zt, zd, t, u, lens, T, draft_lse=np.full((B, K), np.inf, np.float32))
    kb = lens.copy()
    kb[3] = 2
    np.testing.assert_array_equal(n, kb)
    p = torch.softmax(torch.from_numpy(zt).double() / T, -1).numpy()
    for b in range(B):
        # sequence 3 stops at position 2, where the residual max(0, p - 0) is p_2 itself;
        # the final draw takes uniform column K_b (R1) either way
        cdf = np.cumsum(p[b, kb[b]])
        assert nx[b] == int(np.searchsorted(cdf, u[b, lens[b]] * cdf[-1], side="right"))


def given_lse_boundaries(zt, zd, T, c, lib=None):
    """Decision and draw boundaries of the verify with a given normaliser that is
    the row's true one plus log(c), against closed forms computed here in numpy
    (q_i / c in place of q_i): at every position i and draft token x with
    rho = c p_i(x) / q_i(x) < 1, a uniform 0.1% below rho accepts and 0.1% above
    rejects (earlier positions accept at u = 0); after that rejection, a draw
    threshold 0.1% past each cumulative weight of max(0, p_i - q_i / c) draws
    the next id of positive weight. zt [K+1, V], zd [K, V] (fp64)."""
    K, V = zd.shape
    sm = lambda y: np.exp(y - y.max(-1, keepdims=True)) / np.exp(y - y.max(-1, keepdims=True)).sum(-1, keepdims=True)
    p, q = sm(zt / T), sm(zd / T)
    lse = (exact_lse(zd, T) + np.log(c)).astype(np.float32)
    cases_t, cases_u, want_n, want_x = [], [], [], []
    for i in range(K):
        r = np.maximum(0.0, p[i] - q[i] / c)
        cdf = np.cumsum(r)
        for x in range(V):
            rho = c * p[i, x] / q[i, x]
            if not rho < 0.99:
                continue
            t = np.zeros(K, np.int32)
            t[i] = x
            t[:i] = 0
            for side, n_exp in ((1 - 1e-3, i + 1), (1 + 1e-3, i)):
                u = np.zeros(K + 1)
                u[i] = rho * side
                if n_exp == i:
                    # the correction: a threshold inside the first positive weight draws that id, and
                    # one just past each boundary C(y) draws the next id of positive weight
                    first = int(np.argmax(r > 0))
                    uu = u.copy()
                    uu[K] = 0.5 * r[first] / cdf[-1]
                    cases_t.append(t.copy()); cases_u.append(uu); want_n.append(i); want_x.append(first)
                    for y in range(V):
                        if r[y] <= 0 or cdf[y] >= cdf[-1] * (1 - 1e-9):
                            continue
                        nxt = y + 1 + int(np.argmax(r[y + 1:] > 0))
                        uu = u.copy()
                        uu[K] = cdf[y] * (1 + 1e-3) / cdf[-1]
                        cases_t.append(t.copy()); cases_u.append(uu); want_n.append(i); want_x.append(nxt)
                else:
                    cases_t.append(t.copy()); cases_u.append(u); want_n.append(-1); want_x.append(-1)
    B = len(cases_t)
    assert B > 0
    n, nx, _ = oracle.accept_logits(np.broadcast_to(zt, (B, K + 1, V)).copy(), np.broadcast_to(zd, (B, K, V)).copy(),
                                    np.array(cases_t), np.array(cases_u), None, T, lib=lib,
                                    draft_lse=np.broadcast_to(lse, (B, K)).copy())
    for b in range(B):
        if want_n[b] < 0:
            assert n[b] > int(np.flatnonzero(np.array(cases_u[b][:K]) > 0)[0]), b  # accepted past position i
        else:
            assert n[b] == want_n[b] and nx[b] == want_x[b], (b, n[b], nx[b], want_n[b], want_x[b])
    return B


@pytest.mark.parametrize("c", [0.8, 1.25])
def test_logits_verify_given_lse_boundaries(c):
    """Where a given normaliser puts the accept and draw boundaries (closed forms)."""
    rng = np.random.default_rng(int(100 * c))
    K, V, T = 3, 7, 0.7
    zt = 1.5 * rng.standard_normal((K + 1, V)) + 2.0
    zd = zt[:K] + rng.standard_normal((K, V)) + 3.0  # shifts leave the softmax as it is
    assert given_lse_boundaries(zt, zd, T, c) > 10
