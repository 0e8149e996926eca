"""Statistical pins of the oracle's sampled verify (fixed seeds, deterministic).

- Acceptance-length law over 600 rounds of the single-sequence K = 4,
  V = 32000 workload: the mean accepted length must lie within 3 sigma of
  E[n] = sum_{i=1..K} prod_{j<i} a_j, a_j = sum_x min(p_j, q_j) (PocketLLM
  DSpark notes, the gate's expected-tokens law; spec-verify card, "Measured"
  and "Correctness"). Var[n] = sum_i (2i - 1) P(n >= i) - E[n]^2.
- Per-position Monte-Carlo acceptance against sum_x min(p, q).
- Chi-square on V = 8 (1e5 rounds, K = 4): the emitted tokens follow the target
  rows (the llmstudio blog, sections 17 and 37: the result has the target's
  distribution). Negative controls -- the biased "accept if in the target's
  top-k" rule (same blog, section 18), drawing the correction from p instead of
  the residual, and a swapped ratio -- must fail the same test.
"""
import numpy as np
import pytest
from scipy import stats

import oracle
import synth

ROUNDS = 600


def law_moments(a):
    K = len(a)
    ge = np.array([np.prod(a[:i]) for i in range(1, K + 1)])  # P(n >= i), i = 1..K
    mean = ge.sum()
    second = sum((2 * i - 1) * ge[i - 1] for i in range(1, K + 1))
    return mean, second - mean ** 2


def test_acceptance_law_600_rounds():
    name = "probs-b1-k4-v32000"
    ns = []
    for r in range(ROUNDS):
        b = synth.generate(name, "cpu", round_index=r)
        n, nx, fl = oracle.accept(b.target, b.draft, b.tokens, b.uniforms, b.lens)
        assert 0 <= nx[0] < b.V
        ns.append(int(n[0]))
    K = b.K
    p = b.target[0].double().numpy()
    q = b.draft[0].double().numpy()
    a = np.minimum(p[:K], q).sum(-1)
    mean, var = law_moments(a)
    ns = np.array(ns)
    sigma = np.sqrt(var / ROUNDS)
    assert abs(ns.mean() - mean) <= 3 * sigma, (ns.mean(), mean, sigma, a)
    # per-position acceptance: position j is tested when n >= j and passes when n >= j + 1
    for j in range(K):
        tested = (ns >= j).sum()
        if tested < 30:
            continue
        rate = (ns >= j + 1).sum() / tested
        assert abs(rate - a[j]) <= 3 * np.sqrt(a[j] * (1 - a[j]) / tested), (j, rate, a[j])


def draw_rows(rng, rows, V):
    x = rng.gamma(2.0, size=(rows, V)) + 0.15
    return x / x.sum(-1, keepdims=True)


def sample_categorical(rng, probs, size):
    cdf = np.cumsum(probs)
    return np.minimum(np.searchsorted(cdf, rng.random(size) * cdf[-1], side="right"), len(probs) - 1)


@pytest.fixture(scope="module")
def chi2_setup():
    rng = np.random.default_rng(2024)
    K, V, R = 4, 8, 100_000
    p = draw_rows(rng, K + 1, V)
    q = draw_rows(rng, K, V)
    t = np.stack([sample_categorical(rng, q[i], R) for i in range(K)], axis=1).astype(np.int32)
    u = rng.random((R, K + 1))
    return K, V, R, p, q, t, u


def chi2_pvalue(tokens, probs):
    V = len(probs)
    counts = np.bincount(tokens, minlength=V)
    live = probs > 0
    assert counts[~live].sum() == 0, "a zero-probability id was emitted"
    exp = probs[live] / probs[live].sum() * counts.sum()
    return stats.chisquare(counts[live], exp).pvalue


def emitted_first(n, nx, t):
    return np.where(n >= 1, t[:, 0], nx)


def test_chi_square_emitted_tokens_follow_target(chi2_setup):
    K, V, R, p, q, t, u = chi2_setup
    P = np.broadcast_to(p, (R, K + 1, V)).copy()
    Q = np.broadcast_to(q, (R, K, V)).copy()
    n, nx, _ = oracle.accept(P, Q, t, u)
    assert chi2_pvalue(emitted_first(n, nx, t), p[0]) > 1e-3
    sel = n >= 1
    second = np.where(n[sel] >= 2, t[sel, 1], nx[sel])
    assert chi2_pvalue(second, p[1]) > 1e-3
    assert chi2_pvalue(nx[n == K], p[K]) > 1e-3
    for i in range(2):
        resid = np.maximum(0.0, p[i] - q[i])
        assert chi2_pvalue(nx[n == i], resid) > 1e-3


def biased_variant(p, q, t, u, rule):
    """Vectorised wrong procedures, used only as negative controls."""
    R, K = t.shape
    V = p.shape[1]
    n = np.full(R, K)
    alive = np.ones(R, dtype=bool)
    for i in range(K):
        pt, qt = p[i, t[:, i]], q[i, t[:, i]]
        if rule == "topk":
            top = np.argsort(-p[i])[:3]
            ok = np.isin(t[:, i], top)
        elif rule == "swapped_ratio":
            ok = u[:, i] < qt / pt
        else:
            ok = u[:, i] < pt / qt
        rej = alive & ~ok
        n[rej] = i
        alive &= ok
    nx = np.empty(R, dtype=np.int64)
    for b in range(R):
        i = n[b]
        if i < K:
            w = p[i] if rule in ("topk", "correct_from_p") else np.maximum(0.0, p[i] - q[i])
        else:
            w = p[K]
        c = np.cumsum(w)
        nx[b] = np.searchsorted(c, u[b, K] * c[-1], side="right")
    return n, nx


@pytest.mark.parametrize("rule", ["topk", "correct_from_p", "swapped_ratio"])
def test_chi_square_rejects_biased_procedures(chi2_setup, rule):
    K, V, R, p, q, t, u = chi2_setup
    R2 = 20_000
    n, nx = biased_variant(p, q, t[:R2], u[:R2], rule)
    assert chi2_pvalue(emitted_first(n, nx, t[:R2]), p[0]) < 1e-6
