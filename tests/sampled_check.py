"""Comparison of sampled-verify results with the oracle's, under the parity bar.

Accept decisions and drawn ids must equal the oracle's exactly, except on
sequences the oracle flags as lying within 1e-5 (relative) of a boundary:
  - a ratio flag (a tested uniform within 1e-5 * rho of its ratio p/q) may flip
    that accept decision, which moves n_accepted and the row drawn from, so
    such a sequence is exempt from both comparisons;
  - a CDF flag (the draw threshold u * S within 1e-5 * C of a cumulative weight
    C) can only move the drawn id, so n_accepted is still compared exactly.
Flagged counts are printed with every comparison, and at most 1% of a batch
(one sequence in a batch of fewer than 100) may be flagged: the expected rate
is about 1e-5 per test or draw, so a larger count means the windows hide
something.
"""
import numpy as np

import oracle

RATIO = oracle.FLAG_RATIO
CDF = oracle.FLAG_CDF


def compare_sampled(n, nx, n_o, nx_o, flags, label, max_flag_frac=0.01):
    """Assert the bar over arrays of one batch; returns (ratio-flagged, cdf-flagged) counts."""
    n, nx, n_o, nx_o, flags = (np.asarray(a) for a in (n, nx, n_o, nx_o, flags))
    ratio = (flags & RATIO) != 0
    cdf = ((flags & CDF) != 0) & ~ratio
    bad_n = np.nonzero((n != n_o) & ~ratio)[0]
    bad_x = np.nonzero((nx != nx_o) & ~ratio & ~cdf)[0]
    within = int((((n != n_o) | (nx != nx_o)) & (ratio | cdf)).sum())
    print(f"[{label}] sampled: {len(n)} sequences, mean n={n_o.mean():.3f}, ratio-flagged={int(ratio.sum())}, "
          f"cdf-flagged={int(cdf.sum())}, differing-within-flags={within}", flush=True)
    if len(bad_n):
        b = int(bad_n[0])
        raise AssertionError(f"{label}: n_accepted differs at {len(bad_n)} sequences without a ratio flag; first "
                             f"b={b}: gpu ({n[b]}, {nx[b]}) oracle ({n_o[b]}, {nx_o[b]}) flags {flags[b]}")
    if len(bad_x):
        b = int(bad_x[0])
        raise AssertionError(f"{label}: next_token differs at {len(bad_x)} unflagged sequences; first b={b}: gpu "
                             f"({n[b]}, {nx[b]}) oracle ({n_o[b]}, {nx_o[b]})")
    nflag = int((ratio | cdf).sum())
    allowed = max(1, int(max_flag_frac * len(n)))  # a batch under 100 sequences may hold one
    assert nflag <= allowed, f"{label}: {nflag} of {len(n)} sequences flagged (at most {allowed})"
    return int(ratio.sum()), int(cdf.sum())
