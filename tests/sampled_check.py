"""Comparison of sampled-verify results with the oracle's, under the parity bar.

The bar: accept decisions and drawn ids equal the oracle's exactly, except on
sequences the oracle flags as lying within 1e-5 (relative) of a boundary --
a tested uniform within 1e-5 * rho of its ratio p/q, or the draw threshold
u * S within 1e-5 * C of a cumulative weight C on either side of the drawn id.

The check applied here is stricter than the bar. It exempts only what the
oracle flags at AUDIT_WINDOW = 1e-7:
  - a ratio flag may flip that accept decision, which moves n_accepted and the
    row drawn from, so such a sequence is exempt from both comparisons;
  - a CDF flag can only move the drawn id, so n_accepted is still compared.
Every other sequence must match exactly, and at most 1% of a batch (one
sequence in a batch of fewer than 100) may be flagged at the audit window.

The flag counts at both windows are printed. They are properties of the
inputs alone (the oracle computes them without the GPU): a draw that lands on
an id whose weight is below 1e-5 of the cumulative weight before it is
flagged at the bar's window whatever computed it. Rows with heavy tails (the
ragged fp32 workload at T = 1 puts about 12% of its draws there) are flagged
that often at 1e-5, about 1% at 1e-7.
"""
import numpy as np

import oracle

BAR_WINDOW = 1e-5
AUDIT_WINDOW = 1e-7
RATIO = oracle.FLAG_RATIO
CDF = oracle.FLAG_CDF


def compare_sampled(n, nx, oracle_at, label, max_flag_frac=0.01, extra_ratio=None):
    """Assert the check for one batch.

    oracle_at(window) -> (n_o, nx_o, flags) runs the oracle with that relative
    window. extra_ratio: optional boolean mask of sequences to treat as
    ratio-flagged at both windows (a boundary decided upstream of the verify).
    Returns the oracle's (n_o, nx_o).
    """
    n, nx = np.asarray(n), np.asarray(nx)
    n_o, nx_o, fl_bar = (np.asarray(a) for a in oracle_at(BAR_WINDOW))
    n_a, nx_a, fl = (np.asarray(a) for a in oracle_at(AUDIT_WINDOW))
    assert (n_a == n_o).all() and (nx_a == nx_o).all(), "the oracle's result depends on its flag window"
    if extra_ratio is not None:
        fl_bar = np.where(extra_ratio, fl_bar | RATIO, fl_bar)
        fl = np.where(extra_ratio, fl | RATIO, fl)
    ratio = (fl & RATIO) != 0
    cdf = ((fl & CDF) != 0) & ~ratio
    bar = (fl_bar & (RATIO | CDF)) != 0
    differ = (n != n_o) | (nx != nx_o)
    print(f"[{label}] sampled: {len(n)} sequences, mean n={n_o.mean():.3f}, flagged at 1e-5: {int(bar.sum())}, "
          f"at 1e-7: {int(ratio.sum())} ratio + {int(cdf.sum())} cdf, differing: {int(differ.sum())}", flush=True)
    bad_n = np.nonzero((n != n_o) & ~ratio)[0]
    if len(bad_n):
        b = int(bad_n[0])
        raise AssertionError(f"{label}: n_accepted differs at {len(bad_n)} sequences without a ratio flag; first "
                             f"b={b}: gpu ({n[b]}, {nx[b]}) oracle ({n_o[b]}, {nx_o[b]}) flags {fl[b]}/{fl_bar[b]}")
    bad_x = np.nonzero((nx != nx_o) & ~ratio & ~cdf)[0]
    if len(bad_x):
        b = int(bad_x[0])
        raise AssertionError(f"{label}: next_token differs at {len(bad_x)} unflagged sequences; first b={b}: gpu "
                             f"({n[b]}, {nx[b]}) oracle ({n_o[b]}, {nx_o[b]}) flags {fl[b]}/{fl_bar[b]}")
    nflag = int((ratio | cdf).sum())
    allowed = max(1, int(max_flag_frac * len(n)))  # a batch under 100 sequences may hold one
    assert nflag <= allowed, f"{label}: {nflag} of {len(n)} sequences flagged at 1e-7 (at most {allowed})"
    return n_o, nx_o


def chunked(fn, B, chunk=64):
    """Concatenate fn(slice) -> (n, nx, flags) over slices of ``chunk`` sequences."""
    outs = [np.empty(B, np.int32) for _ in range(3)]
    for b0 in range(0, B, chunk):
        sl = slice(b0, min(B, b0 + chunk))
        for o, v in zip(outs, fn(sl)):
            o[sl] = v
    return outs
