"""Exact output law of a sampled-verify procedure on a tiny vocabulary.

The procedure's output is a piecewise-constant function of the draft tokens
t and the uniforms u. For fixed rows p [K+1, V], q [K, V] this module
enumerates every draft tuple t (weight prod_i q_i(t_i)) and, for each possible
first-rejection index n, one representative uniform vector from the interior
of the u-region that leads there:
  - an accepted position j:   u_j = min(1, rho_j) / 2            (u_j < rho_j)
  - the rejected position n:  u_n = (1 + min(1, rho_n)) / 2      (u_n >= rho_n)
  - the final draw column K:  the midpoint of each CDF interval of the final
    draw's weight row, weighted by the interval's length.
The procedure under test is called on all representatives at once (one batch)
and must land in the region the representative was taken from; the weights
then give the exact probability of every (n, emitted tokens) outcome.

``expected_region`` only fixes where the interval representatives sit; the
law itself is checked by the tests against closed forms (the acceptance
product and the target rows p), not against this module.
"""
from __future__ import annotations

import itertools
from collections import defaultdict

import numpy as np


def _final_weights(p, q, n, K):
    if n < K:
        w = np.maximum(0.0, p[n] - q[n])
        if w.sum() > 0:
            return w
        return np.maximum(0.0, p[n])
    return np.maximum(0.0, p[K])


def enumerate_law(p, q, run):
    """Exact law of ``run`` over draft tuples and uniforms.

    ``run(P, Q, T, U) -> (n[B], next[B])`` evaluates the procedure on a batch
    (P [B,K+1,V], Q [B,K,V], T [B,K] int, U [B,K+1] fp64).
    Returns (law: dict[(n, emitted_tuple)] -> probability, mismatches: int).
    """
    p = np.asarray(p, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    K1, V = p.shape
    K = K1 - 1
    cases_t, cases_u, meta = [], [], []
    for t in itertools.product(range(V), repeat=K):
        wt = 1.0
        for i in range(K):
            wt *= q[i, t[i]]
        if wt == 0.0:
            continue
        acc = []
        for i in range(K):
            pt, qt = p[i, t[i]], q[i, t[i]]
            acc.append(min(1.0, pt / qt))
        for n in range(K + 1):
            pr = wt
            for j in range(n):
                pr *= acc[j]
            if n < K:
                pr *= 1.0 - acc[n]
            if pr == 0.0:
                continue
            w = _final_weights(p, q, n, K)
            S = w.sum()
            c = np.cumsum(w)
            for x in range(V):
                if w[x] <= 0.0:
                    continue
                u = np.full(K + 1, 0.5)
                for j in range(n):
                    u[j] = 0.5 * acc[j]
                if n < K:
                    u[n] = 0.5 * (1.0 + acc[n])
                u[K] = (c[x] - 0.5 * w[x]) / S
                cases_t.append(t)
                cases_u.append(u)
                meta.append((n, tuple(t[:n]) + (x,), pr * w[x] / S))
    B = len(meta)
    P = np.broadcast_to(p, (B, K + 1, V)).copy()
    Q = np.broadcast_to(q, (B, K, V)).copy()
    T = np.asarray(cases_t, dtype=np.int32).reshape(B, K)
    U = np.asarray(cases_u, dtype=np.float64)
    n_out, next_out = run(P, Q, T, U)
    law = defaultdict(float)
    mismatches = 0
    for b, (n, emitted, pr) in enumerate(meta):
        if int(n_out[b]) != n or int(next_out[b]) != emitted[-1]:
            mismatches += 1
            emitted = tuple(T[b, :int(n_out[b])]) + (int(next_out[b]),)
            n = int(n_out[b])
        law[(n, emitted)] += pr
    return dict(law), mismatches


def prob_n_at_least(law, i):
    return sum(pr for (n, _), pr in law.items() if n >= i)


def emitted_marginal(law, i, V):
    """P(emitted token at position i = y, n >= i) for y in 0..V-1."""
    m = np.zeros(V)
    for (n, em), pr in law.items():
        if n >= i:
            m[em[i]] += pr
    return m
