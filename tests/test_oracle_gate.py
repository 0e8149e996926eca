"""Pins of the oracle's top-2 margin and acceptance-driven draft-length gate
(PocketLLM DSpark notes, "gating": expected tokens over cost, censored
observations, per-round decay, the 1.15 truncation margin, the pre-draft
top1 - top2 logit margin).

Pinned by: the cost model's printed values (tests/golden/dspark_gate_cost_model.txt),
the geometric closed form of E(n) at constant acceptance, brute-force argmax of
E/cost, the decay's geometric limit, a statistical check that censored counting
recovers the true per-position acceptance (and that counting unobserved positions
as misses would not), numpy for the margin.
"""
import numpy as np
import pytest

import oracle
from tests.conftest import read_golden

D = oracle.GATE_DEFAULTS


def cost(n):
    return D["plain_ms"] if n == 0 else D["draft_ms"] + D["verify_base_ms"] + D["verify_slope_ms"] * n


def test_cost_model_matches_printed_values():
    g = read_golden("dspark_gate_cost_model.txt")
    assert cost(5) == g["round_cost_n5_ms"]
    assert abs((cost(5) - cost(0)) - g["zero_accept_loss_n5_ms"]) <= 5
    assert round(1000.0 / cost(0), 2) == g["plain_tok_per_s"]
    assert round(1000.0 * 6 / cost(5), 2) == g["repeat_tok_per_s_accept_5_of_5"]
    assert round(1000.0 * 3 / cost(5), 2) == g["prose_tok_per_s_accept_2_of_5"]


def counts_for(p, K, trials=1000.0):
    """Counts whose ratio is p_j per position."""
    p = np.asarray(p, dtype=np.float64)
    return (p * trials).reshape(1, -1).copy(), np.full((1, K), trials)


def brute_choice(p, K, margin=1.15, min_draft=0):
    E = [1.0]
    for n in range(1, K + 1):
        E.append(E[-1] + np.prod(p[:n]))
    r = [E[n] / cost(n) for n in range(K + 1)]
    best = max(range(K + 1), key=lambda n: (r[n], n))
    if best < K and not r[best] >= margin * r[K]:
        best = K
    return max(best, min(min_draft, K))


@pytest.mark.parametrize("a", [0.0, 0.1, 0.3, 0.5, 0.7, 0.9, 1.0])
@pytest.mark.parametrize("K", [1, 3, 5, 8, 16])
def test_constant_acceptance_matches_brute_force(a, K):
    h, t = counts_for([a] * K, K)
    got = oracle.gate_choose(h, t, K)[0]
    assert got == brute_choice(np.full(K, a), K)
    # E(n) = 1 + a + ... + a^n = (1 - a^(n+1)) / (1 - a): the chosen n is where the ratio peaks
    if 0 < a < 1:
        r = [(1 - a ** (n + 1)) / (1 - a) / cost(n) for n in range(K + 1)]
        nstar = max(range(K + 1), key=lambda n: (r[n], n))
        expect = nstar if (nstar == K or r[nstar] >= 1.15 * r[K]) else K
        assert got == expect


def test_easy_and_hard_workloads():
    K = 5
    # the notes' accept rates: repeat 100%, code 82.5%, prose 40%, math 17.5%
    assert oracle.gate_choose(*counts_for([1.0] * K, K), K)[0] == K
    assert oracle.gate_choose(*counts_for([0.825] * K, K), K)[0] == K
    assert oracle.gate_choose(*counts_for([0.4] * K, K), K)[0] == 0
    assert oracle.gate_choose(*counts_for([0.175] * K, K), K)[0] == 0


def test_truncation_margin():
    # high acceptance early, none late: truncation at 2 wins by far more than 1.15
    K = 6
    p = [0.95, 0.95, 0.0, 0.0, 0.0, 0.0]
    assert oracle.gate_choose(*counts_for(p, K), K)[0] == 2
    # a margin factor the truncation cannot reach keeps the full draft
    r2 = (1 + 0.95 + 0.95 ** 2) / cost(2)
    rK = (1 + 0.95 + 0.95 ** 2) / cost(K)
    assert oracle.gate_choose(*counts_for(p, K), K, margin=r2 / rK * 1.001)[0] == K
    assert oracle.gate_choose(*counts_for(p, K), K, margin=r2 / rK * 0.999)[0] == 2


def test_min_draft_and_cold_gate_and_pre_draft_margin():
    K = 5
    h, t = counts_for([0.1] * K, K)
    assert oracle.gate_choose(h, t, K)[0] == 0
    assert oracle.gate_choose(h, t, K, min_draft=2)[0] == 2
    assert oracle.gate_choose(h, t, K, min_draft=9)[0] == K
    # a cold gate (no trials) drafts the full block so that it can learn
    assert oracle.gate_choose(np.zeros((1, K)), np.zeros((1, K)), K)[0] == K
    # pre-draft: a small committed-token margin skips the draft (when enabled)
    hh, tt = counts_for([1.0] * K, K)
    assert oracle.gate_choose(hh, tt, K, top2_margin=[1.0], margin_threshold=4.0)[0] == 0
    assert oracle.gate_choose(hh, tt, K, top2_margin=[5.0], margin_threshold=4.0)[0] == K
    assert oracle.gate_choose(hh, tt, K, top2_margin=[1.0], margin_threshold=0.0)[0] == K


def test_update_records_only_observed_positions():
    K, NB = 5, 5
    h = np.zeros((3, NB))
    t = np.zeros((3, NB))
    oracle.gate_update(h, t, K, lens=[5, 3, 0], n_accepted=[2, 3, 0], decay=1.0)
    # seq 0: positions 0, 1 accepted, 2 rejected, 3-4 unobserved
    np.testing.assert_array_equal(t[0], [1, 1, 1, 0, 0])
    np.testing.assert_array_equal(h[0], [1, 1, 0, 0, 0])
    # seq 1: all 3 drafted accepted (the bonus is no observation)
    np.testing.assert_array_equal(t[1], [1, 1, 1, 0, 0])
    np.testing.assert_array_equal(h[1], [1, 1, 1, 0, 0])
    # seq 2: no draft, nothing recorded
    assert t[2].sum() == 0


def test_decay_converges_to_geometric_limit():
    K, NB = 3, 3
    h = np.zeros((1, NB))
    t = np.zeros((1, NB))
    for _ in range(300):
        oracle.gate_update(h, t, K, lens=[3], n_accepted=[3], decay=0.9)
    np.testing.assert_allclose(t[0], 1 / (1 - 0.9), rtol=1e-9)
    np.testing.assert_allclose(h[0], 1 / (1 - 0.9), rtol=1e-9)
    # one round of a shifted workload moves the estimate by the decay's weight
    oracle.gate_update(h, t, K, lens=[3], n_accepted=[0], decay=0.9)
    assert h[0, 0] / t[0, 0] == pytest.approx(0.9 * 10 / (0.9 * 10 + 1), rel=1e-9)


def test_censored_counting_recovers_true_acceptance():
    rng = np.random.default_rng(0)
    a = np.array([0.8, 0.6, 0.9, 0.5])
    K = len(a)
    h = np.zeros((1, K))
    t = np.zeros((1, K))
    naive_h = np.zeros(K)
    naive_t = np.zeros(K)
    for _ in range(20000):
        acc = rng.random(K) < a
        n = K if acc.all() else int(np.argmin(acc))
        oracle.gate_update(h, t, K, lens=[K], n_accepted=[n], decay=1.0)
        naive_t += 1
        naive_h += np.arange(K) < n
    est = h[0] / t[0]
    sd = np.sqrt(a * (1 - a) / t[0])
    assert (np.abs(est - a) < 4 * sd).all()
    # counting unobserved positions as misses is biased low at every later position
    assert (naive_h[1:] / naive_t[1:] < a[1:] - 0.05).all()


def test_buckets_pool_positions():
    K, NB = 4, 2
    h = np.zeros((1, NB))
    t = np.zeros((1, NB))
    buckets = np.array([[1, 0, 1, 0]], dtype=np.int32)
    oracle.gate_update(h, t, K, lens=[4], n_accepted=[2], buckets=buckets, decay=1.0)
    np.testing.assert_array_equal(t[0], [1, 2])   # positions 1 -> bucket 0; 0 and 2 -> bucket 1
    np.testing.assert_array_equal(h[0], [1, 1])   # position 1 accepted (b0), 0 accepted (b1), 2 rejected (b1)
    # out-of-range bucket ids are clamped
    oracle.gate_update(h, t, K, lens=[1], n_accepted=[0], buckets=np.array([[7, 0, 0, 0]], np.int32), decay=1.0)
    assert t[0, 1] == 3


def test_top2_margin():
    rng = np.random.default_rng(3)
    for _ in range(20):
        r = rng.standard_normal(500).astype(np.float32)
        s = np.sort(r.astype(np.float64))
        assert oracle.top2_margin(r) == s[-1] - s[-2]
    assert oracle.top2_margin(np.array([1.0, 3.0, 3.0], np.float32)) == 0.0
    assert oracle.top2_margin(np.array([2.0], np.float32)) == np.inf
    assert oracle.top2_margin(np.array([-np.inf, 1.0, -np.inf], np.float32)) == np.inf
