"""Pins of the oracle to values the pages print for worked examples.

Each case reads its numbers from a fixture under tests/golden/ that cites the
page and section it comes from.
"""
import numpy as np
import pytest

import oracle
from tests.exact_law import emitted_marginal, enumerate_law, prob_n_at_least


def oracle_run(P, Q, T, U):
    n, nx, _ = oracle.accept(P, Q, T, U)
    return n, nx


def accept_threshold(p_row, q_row, tok):
    """Bisect the uniform at which the oracle's decision for one draft token flips."""
    V = len(p_row)
    P = np.stack([p_row, p_row]).astype(np.float64)[None]   # [1, 2, V]; row 1 is the bonus row
    Q = np.asarray(q_row, dtype=np.float64)[None, None]       # [1, 1, V]
    T = np.array([[tok]], dtype=np.int32)

    def accepted(u):
        n, _, _ = oracle.accept(P, Q, T, np.array([[u, 0.5]]))
        return n[0] == 1

    if accepted(np.nextafter(1.0, 0.0)):
        return 1.0
    lo, hi = 0.0, 1.0
    assert accepted(lo) or not accepted(lo)
    for _ in range(80):
        mid = 0.5 * (lo + hi)
        if accepted(mid):
            lo = mid
        else:
            hi = mid
    assert V >= 2
    return 0.5 * (lo + hi)


def test_blog_s15_overconfident_draft(golden):
    g = golden("blog_s15_s16_accept_ratio.txt")
    # token C = id 1 of a two-token vocabulary; the other id takes the rest of the mass
    p = np.array([1.0 - g["s15_p"], g["s15_p"]])
    q = np.array([1.0 - g["s15_q"], g["s15_q"]])
    thr = accept_threshold(p, q, 1)
    assert abs(thr - g["s15_accept_prob"]) <= g["s15_printed_tol"]
    assert abs(g["s15_q"] * thr - g["s15_accepted_mass"]) <= g["s15_printed_tol"]
    assert thr == pytest.approx(g["s15_p"] / g["s15_q"], rel=1e-12)


def test_blog_s16_underconfident_draft_always_accepted(golden):
    g = golden("blog_s15_s16_accept_ratio.txt")
    p = np.array([1.0 - g["s16_p"], g["s16_p"]])
    q = np.array([1.0 - g["s16_q"], g["s16_q"]])
    assert g["s16_p"] / g["s16_q"] == pytest.approx(g["s16_ratio"])
    assert accept_threshold(p, q, 1) == g["s16_accept_prob"]
    P = np.stack([p, p])[None]
    Q = q[None, None]
    for u in [0.0, 0.25, 0.5, 0.99, np.nextafter(1.0, 0.0)]:
        n, _, _ = oracle.accept(P, Q, np.array([[1]]), np.array([[u, 0.5]]))
        assert n[0] == 1


def test_blog_s18_four_token_pair(golden):
    g = golden("blog_s18_four_token_example.txt")
    p0 = np.array(g["target"])
    q0 = np.array(g["draft"])
    assert oracle.overlap(p0, q0) == pytest.approx(g["acceptance"], abs=1e-15)
    # correction draws follow the normalised residual
    res = np.array(g["residual_normalised"])
    p = np.stack([p0, p0])        # K = 1: row 0 verifies, row 1 is the bonus row
    q = q0[None]
    law, bad = enumerate_law(p, q, oracle_run)
    assert bad == 0
    assert prob_n_at_least(law, 1) == pytest.approx(g["acceptance"], abs=1e-12)
    p_corr = np.zeros(4)
    for (n, em), pr in law.items():
        if n == 0:
            p_corr[em[0]] += pr
    np.testing.assert_allclose(p_corr / p_corr.sum(), res, atol=1e-12)
    # the emitted token's law is the target row
    np.testing.assert_allclose(emitted_marginal(law, 0, 4), p0, atol=1e-12)


def test_blog_s13_greedy_left_to_right(golden):
    g = golden("blog_s13_greedy_example.txt")
    draft = np.array(g["draft_tokens"], dtype=np.int32)
    am = [int(x) for x in g["target_argmax"]]
    K, V = len(draft), 4
    rng = np.random.default_rng(13)
    target = rng.uniform(0.0, 0.5, size=(1, K + 1, V))
    for i, a in enumerate(am):
        target[0, i, a] = 1.0
    for bonus_argmax in range(V):  # the row after the first miss must not matter
        target[0, K, :] = 0.0
        target[0, K, bonus_argmax] = 1.0
        n, nx = oracle.verify_greedy(target, draft[None])
        assert n[0] == g["n_accepted"] and nx[0] == g["next_token"]


def test_blog_s30_acceptance_law_example(golden):
    g = golden("blog_s30_acceptance_law.txt")
    alpha, gamma = g["alpha"], int(g["gamma"])
    # every position accepts with probability alpha: the target is sure of id 0, the draft
    # puts alpha on it
    p = np.tile(np.array([1.0, 0.0]), (gamma + 1, 1))
    q = np.tile(np.array([alpha, 1.0 - alpha]), (gamma, 1))
    law, bad = enumerate_law(p, q, oracle_run)
    assert bad == 0
    expected_tokens = sum(pr * (n + 1) for (n, _), pr in law.items())
    assert expected_tokens == pytest.approx(g["expected_tokens"], abs=1e-12)
    closed = (1 - alpha ** (gamma + 1)) / (1 - alpha)
    assert expected_tokens == pytest.approx(closed, abs=1e-12)
