"""Pins of the oracle's speculative-sampling verify by exact enumeration.

The spec-verify card ("Method") and the llmstudio blog (sections 15-17 and
47-48) fix what the procedure must achieve: a draft token is accepted with
probability min(1, p/q), the run stops at the first rejection, the correction
is drawn from norm(max(0, p - q)), the bonus from p, and the emitted tokens
follow the target rows exactly. Enumerating every draft tuple and every
u-region on a tiny vocabulary gives the procedure's exact law, which is
checked against those closed forms:
  P(n >= i) = prod_{j<i} sum_x min(p_j(x), q_j(x))
  P(token emitted at position i = y | n >= i) = p_i(y)
"""
import numpy as np
import pytest

import oracle
from tests.exact_law import emitted_marginal, enumerate_law, prob_n_at_least


def oracle_run(P, Q, T, U):
    n, nx, _ = oracle.accept(P, Q, T, U)
    return n, nx


def random_rows(rng, rows, V, zero_frac=0.0, conc=1.0):
    x = rng.gamma(conc, size=(rows, V))
    if zero_frac > 0:
        x[rng.random((rows, V)) < zero_frac] = 0.0
        x[:, 0] += 1e-3  # keep every row non-empty
    return x / x.sum(-1, keepdims=True)


@pytest.mark.parametrize("K,V,seed,zero_frac", [(1, 8, 0, 0.0), (2, 8, 1, 0.0), (3, 8, 2, 0.0),
                                                (3, 6, 3, 0.3), (2, 8, 4, 0.5)])
def test_exact_law_matches_closed_forms(K, V, seed, zero_frac):
    rng = np.random.default_rng(seed)
    p = random_rows(rng, K + 1, V, zero_frac)
    q = random_rows(rng, K, V, zero_frac, conc=0.5)
    law, bad = enumerate_law(p, q, oracle_run)
    assert bad == 0
    assert sum(law.values()) == pytest.approx(1.0, abs=1e-12)
    a = np.minimum(p[:K], q).sum(-1)
    for i in range(K + 1):
        assert prob_n_at_least(law, i) == pytest.approx(np.prod(a[:i]), abs=1e-12)
        marg = emitted_marginal(law, i, V)
        np.testing.assert_allclose(marg, np.prod(a[:i]) * p[i], atol=1e-12)
    # given an accepted first draft (weight min(p_0, q_0)), the second emitted token is an
    # independent draw from p_1
    if K >= 1:
        joint = np.zeros((V, V))
        for (n, em), pr in law.items():
            if n >= 1:
                joint[em[0], em[1]] += pr
        np.testing.assert_allclose(joint, np.outer(np.minimum(p[0], q[0]), p[1]), atol=1e-12)


def test_oracle_overlap_is_acceptance_probability():
    rng = np.random.default_rng(5)
    for _ in range(10):
        p, q = random_rows(rng, 1, 50)[0], random_rows(rng, 1, 50)[0]
        assert oracle.overlap(p, q) == pytest.approx(np.minimum(p, q).sum(), abs=1e-15)
        assert oracle.overlap(p, p) == pytest.approx(1.0, abs=1e-12)


def test_identical_rows_accept_everything():
    rng = np.random.default_rng(6)
    B, K, V = 64, 5, 40
    p = random_rows(rng, B * (K + 1), V).reshape(B, K + 1, V)
    q = p[:, :K].copy()
    t = rng.integers(0, V, size=(B, K)).astype(np.int32)
    t[p[np.arange(B)[:, None], np.arange(K)[None], t] == 0] = 0
    u = rng.random((B, K + 1))
    lens = rng.integers(0, K + 1, size=B).astype(np.int32)
    n, nx, fl = oracle.accept(p, q, t, u, lens)
    np.testing.assert_array_equal(n, lens)


def test_one_hot_target_sampled_equals_greedy():
    rng = np.random.default_rng(8)
    B, K, V = 200, 4, 12
    am = rng.integers(0, V, size=(B, K + 1))
    p = np.zeros((B, K + 1, V))
    p[np.arange(B)[:, None], np.arange(K + 1)[None], am] = 1.0
    q = random_rows(rng, B * K, V).reshape(B, K, V)
    t = rng.integers(0, V, size=(B, K)).astype(np.int32)
    hit = rng.random((B, K)) < 0.7
    t = np.where(hit, am[:, :K], t).astype(np.int32)
    u = rng.random((B, K + 1))
    n_s, nx_s, _ = oracle.accept(p, q, t, u)
    n_g, nx_g = oracle.verify_greedy(p, t)
    np.testing.assert_array_equal(n_s, n_g)
    np.testing.assert_array_equal(nx_s, nx_g)


def test_bonus_only_rows_draw_from_p0_with_u0():
    rng = np.random.default_rng(9)
    B, K, V = 50, 3, 16
    p = random_rows(rng, B * (K + 1), V).reshape(B, K + 1, V)
    q = random_rows(rng, B * K, V).reshape(B, K, V)
    t = rng.integers(0, V, size=(B, K)).astype(np.int32)
    u = rng.random((B, K + 1))
    n, nx, _ = oracle.accept(p, q, t, u, np.zeros(B, dtype=np.int32))
    assert (n == 0).all()
    for b in range(B):
        cdf = np.cumsum(p[b, 0])
        assert nx[b] == int(np.searchsorted(cdf, u[b, 0] * cdf[-1], side="right"))


def test_ragged_sequence_equals_dense_call_on_its_prefix():
    rng = np.random.default_rng(10)
    B, K, V = 40, 6, 20
    p = random_rows(rng, B * (K + 1), V).reshape(B, K + 1, V)
    q = random_rows(rng, B * K, V).reshape(B, K, V)
    t = rng.integers(0, V, size=(B, K)).astype(np.int32)
    u = rng.random((B, K + 1))
    lens = rng.integers(0, K + 1, size=B).astype(np.int32)
    n, nx, _ = oracle.accept(p, q, t, u, lens)
    for b in range(B):
        kb = lens[b]
        n1, nx1, _ = oracle.accept(p[b:b + 1, :kb + 1], q[b:b + 1, :kb], t[b:b + 1, :kb], u[b:b + 1, :kb + 1])
        assert n1[0] == n[b] and nx1[0] == nx[b]


def test_out_of_range_draft_token_is_rejected():
    p = np.full((1, 3, 4), 0.25)
    q = np.full((1, 2, 4), 0.25)
    for bad in [-1, 4, 99]:
        n, nx, _ = oracle.accept(p, q, np.array([[1, bad]]), np.array([[0.1, 0.0, 0.3]]))
        assert n[0] == 1
        # p == q leaves no residual mass: the correction falls back to p of the same row
        assert nx[0] == 1


def test_zero_draft_probability_and_zero_target_probability():
    # q(t) == 0 < p(t): always accepted; p(t) == 0: always rejected, even at u == 0
    p = np.array([[[0.5, 0.5, 0.0], [0.2, 0.3, 0.5]]])
    q = np.array([[[0.0, 0.5, 0.5]]])
    n, _, _ = oracle.accept(p, q, np.array([[0]]), np.array([[np.nextafter(1.0, 0.0), 0.5]]))
    assert n[0] == 1
    n, nx, _ = oracle.accept(p, q, np.array([[2]]), np.array([[0.0, 0.0]]))
    assert n[0] == 0 and nx[0] == 0  # residual (0.5, 0, 0): u = 0 picks the first positive-mass id


def test_unnormalised_rows_draw_by_their_own_mass():
    """The card ("Correctness"): probabilities need not be normalised for the draws."""
    rng = np.random.default_rng(12)
    p = random_rows(rng, 1, 30)[0]
    for scale in [1e-3, 1.0, 7.5, 1e6]:
        for u in np.linspace(0.0, 0.999, 17):
            x1, _ = oracle.icdf(p, u)
            x2, _ = oracle.icdf(p * scale, u)
            assert x1 == x2


def test_icdf_edges():
    w = np.array([0.0, 0.0, 2.0, 0.0, 1.0, 0.0])
    assert oracle.icdf(w, 0.0)[0] == 2
    assert oracle.icdf(w, 0.66)[0] == 2
    assert oracle.icdf(w, 0.67)[0] == 4
    assert oracle.icdf(w, np.nextafter(1.0, 0.0))[0] == 4
    x, flag = oracle.icdf(w, 1.0)  # outside the contract: the last id with positive mass
    assert x == 4 and flag & oracle.FLAG_CDF
    x, flag = oracle.icdf(np.zeros(5), 0.3)
    assert x == -1 and flag & oracle.FLAG_NO_MASS


def test_boundary_flags():
    p = np.array([[[0.9, 0.1], [0.5, 0.5]]])
    q = np.array([[[0.3, 0.7]]])
    rho = 0.1 / 0.7
    _, _, fl = oracle.accept(p, q, np.array([[1]]), np.array([[rho * (1 + 1e-7), 0.5]]))
    assert fl[0] & oracle.FLAG_RATIO
    _, _, fl = oracle.accept(p, q, np.array([[1]]), np.array([[rho * 0.9, 0.5]]))
    assert not fl[0] & oracle.FLAG_RATIO
