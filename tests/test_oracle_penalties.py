"""Pins of the oracle's penalty stage (the sampler pipeline's first stage:
llmstudio blog "Как работает speculative decoding и MTP при инференсе LLM",
section 38; its state follows the speculative branch: section 39).

  - the repetition penalty equals the transformers library's
    RepetitionPenaltyLogitsProcessor on fp32 rows with a token history, bit for
    bit (both compute in fp32);
  - presence and frequency penalties against hand-computed rows (exactly
    representable values);
  - the speculative branch: row r of a sequence is penalised with the committed
    tokens followed by the draft tokens before position r, and nothing later;
  - invariants: neutral parameters and out-of-range histories leave the row
    unchanged, the history's order does not matter, each id is penalised once
    by the repetition penalty however often it occurs;
  - the penalised rows through the filtered warp are the sampler pipeline's
    distribution (penalties, then temperature, top-k, top-p).
"""
import numpy as np
import pytest
import torch

import oracle


def test_repetition_matches_transformers():
    from transformers.generation.logits_process import RepetitionPenaltyLogitsProcessor
    g = torch.Generator().manual_seed(1)
    B, V = 12, 3000
    scores = 4 * torch.randn(B, V, generator=g)
    scores[0, :50] = 0.0
    scores[1, :50] = -0.0
    for theta in (1.3, 0.7, 2.0):
        ids = torch.randint(0, V, (B, 40), generator=g)
        ids[2, :] = 7  # one id, many times
        ref = RepetitionPenaltyLogitsProcessor(penalty=theta)(ids, scores.clone())
        for b in range(B):
            got = oracle.penalize_row(scores[b].numpy(), ids[b].numpy(), theta)
            np.testing.assert_array_equal(got.view(np.int32), ref[b].numpy().view(np.int32))


def test_presence_and_frequency_closed_form():
    z = np.array([2.0, -1.0, 0.0, 3.0, -0.5, 1.5], np.float32)
    hist = [0, 0, 1, 4, 4, 4, 7, -1, 6]  # ids 7 and -1 (and 6 = V) lie outside [0, V): ignored
    # counts (2, 1, 0, 0, 3, 0); theta 2: (1, -2, ., ., -1, .) ; minus 0.25 * c + 0.5
    np.testing.assert_array_equal(oracle.penalize_row(z, hist, 2.0, 0.5, 0.25),
                                  np.array([0.0, -2.75, 0.0, 3.0, -2.25, 1.5], np.float32))
    # presence alone, frequency alone
    np.testing.assert_array_equal(oracle.penalize_row(z, hist, 1.0, 1.0, 0.0),
                                  np.array([1.0, -2.0, 0.0, 3.0, -1.5, 1.5], np.float32))
    np.testing.assert_array_equal(oracle.penalize_row(z, hist, 1.0, 0.0, 0.5),
                                  np.array([1.0, -1.5, 0.0, 3.0, -2.0, 1.5], np.float32))
    # negative penalties raise repeated ids
    np.testing.assert_array_equal(oracle.penalize_row(z, hist, 1.0, -1.0, 0.0),
                                  np.array([3.0, 0.0, 0.0, 3.0, 0.5, 1.5], np.float32))


def test_invariants():
    rng = np.random.default_rng(2)
    z = (3 * rng.standard_normal(500)).astype(np.float32)
    hist = rng.integers(0, 500, 80)
    np.testing.assert_array_equal(oracle.penalize_row(z, hist, 1.0, 0.0, 0.0), z)
    np.testing.assert_array_equal(oracle.penalize_row(z, [-5, 500, 10 ** 6], 1.7, 0.3, 0.2), z)
    a = oracle.penalize_row(z, hist, 1.4, 0.3, 0.1)
    np.testing.assert_array_equal(oracle.penalize_row(z, rng.permutation(hist), 1.4, 0.3, 0.1), a)
    # the repetition penalty acts once per id, however often it repeats
    np.testing.assert_array_equal(oracle.penalize_row(z, np.repeat(hist, 3), 1.4), oracle.penalize_row(z, hist, 1.4))
    # only history ids change
    changed = np.nonzero(a != z)[0]
    assert set(changed) <= set(hist.tolist())


def test_rows_follow_the_speculative_branch():
    """Row r of sequence b is penalised with seq[b, :seq_len[b]] followed by the
    draft tokens t[b, 0 .. r-1]; rows past the live count are not written."""
    rng = np.random.default_rng(3)
    B, K, V, cap = 5, 4, 200, 12
    z = (2 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    seq = rng.integers(0, V, (B, cap)).astype(np.int32)
    seq_len = np.array([0, 3, 12, 7, 20], np.int32)  # 20 > cap: clamped
    t = rng.integers(0, V, (B, K)).astype(np.int32)
    t[1] = [seq[1, 0], seq[1, 0], 17, 17]            # draft tokens repeating the history and each other
    lens = np.array([4, 2, 0, 4, 3], np.int32)
    theta = np.array([1.5, 2.0, 1.2, 1.0, 0.8], np.float32)
    pres = np.array([0.0, 0.5, 0.1, 0.3, 0.0], np.float32)
    freq = np.array([0.2, 0.25, 0.0, 0.1, 0.4], np.float32)
    out = oracle.apply_penalties(z, lens, 1, seq, seq_len, t, theta, pres, freq)
    for b in range(B):
        n0 = min(max(int(seq_len[b]), 0), cap)
        for r in range(K + 1):
            if r > lens[b]:
                assert np.isnan(out[b, r]).all()
                continue
            hist = np.concatenate([seq[b, :n0], t[b, :r]])
            ref = oracle.penalize_row(z[b, r], hist, theta[b], pres[b], freq[b])
            np.testing.assert_array_equal(out[b, r], ref)
    # sequence 1, row 2 (live: lens[1] = 2): its history is seq[1, :3] + (x, x), x = seq[1, 0], so x counts
    # its occurrences in seq[1, :3] plus 2; id 17 = t[1, 2] comes after position 2 and is not in it
    x = int(seq[1, 0])
    c = int((seq[1, :3] == x).sum()) + 2
    zx = z[1, 2, x]
    z1 = np.float32(zx * np.float32(2.0)) if zx < 0 else np.float32(zx / np.float32(2.0))
    d = np.float32(np.float64(np.float32(0.25)) * c + np.float64(np.float32(0.5)))  # one rounding, as fmaf
    assert out[1, 2, x] == np.float32(z1 - d)
    if 17 not in seq[1, :3].tolist() and x != 17:
        assert out[1, 2, 17] == z[1, 2, 17]
    # no prefix for row 0; no history at all without seq and tokens
    out0 = oracle.apply_penalties(z, None, 1, None, None, None, theta, pres, freq)
    np.testing.assert_array_equal(out0, z)
    out1 = oracle.apply_penalties(z, None, 1, seq, seq_len, None, theta, pres, freq)
    for b in range(B):  # without draft tokens every row sees the committed history alone
        n0 = min(max(int(seq_len[b]), 0), cap)
        for r in range(K + 1):
            np.testing.assert_array_equal(out1[b, r], oracle.penalize_row(z[b, r], seq[b, :n0], theta[b], pres[b],
                                                                          freq[b]))


def test_penalised_pipeline_is_the_filtered_warp_of_penalised_rows():
    """The sampler pipeline: penalties, then temperature, top-k, top-p, normalise.
    With neutral filters the result is softmax(z' / T) of the penalised row."""
    rng = np.random.default_rng(4)
    V, T = 300, 0.8
    z = (3 * rng.standard_normal(V)).astype(np.float32)
    hist = rng.integers(0, V, 30)
    zp = oracle.penalize_row(z, hist, 1.5, 0.4, 0.3)
    p, _ = oracle.warp_row_filtered(zp, T, 0, 1.0)
    ref = torch.softmax(torch.from_numpy(zp).double() / T, 0).numpy()
    np.testing.assert_allclose(p, ref, rtol=0, atol=1e-15)
    # a penalised id loses mass, an untouched one gains
    base = torch.softmax(torch.from_numpy(z).double() / T, 0).numpy()
    hit = int(hist[0])
    if z[hit] > 0:
        assert p[hit] < base[hit]
    untouched = [x for x in range(V) if x not in set(hist.tolist())]
    assert (p[untouched] >= base[untouched]).all()


def test_apply_penalties_parameters_broadcast():
    """A number stands for every sequence; an array must be [B]."""
    rng = np.random.default_rng(9)
    B, R, V = 3, 2, 40
    z = rng.standard_normal((B, R, V)).astype(np.float32)
    seq = rng.integers(0, V, (B, 10)).astype(np.int32)
    seq_len = np.array([10, 4, 0], np.int32)
    a = oracle.apply_penalties(z, None, 1, seq, seq_len, None, 1.3, 0.2, 0.1)
    b = oracle.apply_penalties(z, None, 1, seq, seq_len, None, np.full(B, 1.3), np.full(B, 0.2), np.full(B, 0.1))
    np.testing.assert_array_equal(a, b)
    with pytest.raises(ValueError):
        oracle.apply_penalties(z, None, 1, seq, seq_len, None, np.ones(B + 1))
