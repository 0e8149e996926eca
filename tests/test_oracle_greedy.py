"""Pins of the oracle's argmax and greedy verification.

- argmax: numpy.argmax (first occurrence) on the same values, with exact ties,
  signed zeros and bf16 rows;
- greedy: brute force over every draft on a tiny vocabulary, and identity with
  plain greedy decoding of a tiny deterministic model (the spec-verify card,
  "Method" and "Correctness": the emitted stream equals greedy target decoding).
"""
import itertools

import numpy as np
import pytest
import torch

import oracle


@pytest.mark.parametrize("V", [1, 2, 7, 64, 1000, 32003])
def test_argmax_matches_numpy_with_ties(V):
    rng = np.random.default_rng(V)
    for trial in range(20):
        row = rng.integers(-5, 5, size=V).astype(np.float32)  # many exact ties
        assert oracle.argmax_row(row) == int(np.argmax(row))
        row64 = rng.standard_normal(V)
        assert oracle.argmax_row(row64) == int(np.argmax(row64))


def test_argmax_signed_zero_and_negative_rows():
    assert oracle.argmax_row(np.array([-0.0, 0.0, -1.0], dtype=np.float32)) == 0
    assert oracle.argmax_row(np.array([-1.0, 0.0, -0.0], dtype=np.float32)) == 1
    assert oracle.argmax_row(np.array([-3.0, -2.0, -2.0, -5.0])) == 1
    assert oracle.argmax_row(np.array([-np.inf, -np.inf, -1e30])) == 2


def test_argmax_bf16_rows():
    g = torch.Generator().manual_seed(7)
    for _ in range(20):
        row = (5 * torch.randn(4096, generator=g)).to(torch.bfloat16)
        ref = int(np.argmax(row.float().numpy()))
        assert oracle.argmax_row(row) == ref


def lcp(a, b):
    n = 0
    while n < len(a) and n < len(b) and a[n] == b[n]:
        n += 1
    return n


def test_greedy_brute_force_tiny_vocab():
    """V = 3, K = 3: every one of the 27 drafts against fixed target rows."""
    rng = np.random.default_rng(3)
    V, K = 3, 3
    for trial in range(10):
        target = rng.permutation(np.arange((K + 1) * V)).reshape(1, K + 1, V).astype(np.float64)
        chain = [int(np.argmax(target[0, i])) for i in range(K + 1)]
        drafts = np.array(list(itertools.product(range(V), repeat=K)), dtype=np.int32)
        n, nx = oracle.verify_greedy(np.repeat(target, len(drafts), axis=0), drafts)
        for d, nn, xx in zip(drafts, n, nx):
            m = lcp(list(d), chain[:K])
            assert nn == m and xx == chain[m]


def test_greedy_perfect_draft_and_lens():
    rng = np.random.default_rng(11)
    B, K, V = 16, 6, 50
    target = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    chain = target.argmax(-1).astype(np.int32)
    lens = rng.integers(-2, K + 3, size=B).astype(np.int32)  # includes out-of-range lengths
    n, nx = oracle.verify_greedy(target, chain[:, :K], lens)
    kb = np.clip(lens, 0, K)
    np.testing.assert_array_equal(n, kb)
    np.testing.assert_array_equal(nx, chain[np.arange(B), kb])
    # NULL lens means K for every sequence
    n, nx = oracle.verify_greedy(target, chain[:, :K])
    np.testing.assert_array_equal(n, np.full(B, K))


def test_greedy_out_of_range_token_is_a_miss():
    target = np.zeros((1, 3, 4), dtype=np.float32)
    target[0, :, 2] = 1.0
    for bad in [-1, 4, 1 << 30]:
        n, nx = oracle.verify_greedy(target, np.array([[2, bad]], dtype=np.int32))
        assert n[0] == 1 and nx[0] == 2


class TinyModel:
    """A deterministic 'model': logits of the next token from the last two tokens."""

    def __init__(self, V, seed):
        rng = np.random.default_rng(seed)
        self.V = V
        self.table = rng.standard_normal((V, V, V))

    def logits(self, prefix):
        return self.table[prefix[-2], prefix[-1]]


def plain_greedy(model, prompt, n):
    seq = list(prompt)
    while len(seq) < len(prompt) + n:
        seq.append(int(np.argmax(model.logits(seq))))
    return seq


def speculative_greedy(model, prompt, n, K, drafter):
    seq = list(prompt)
    while len(seq) < len(prompt) + n:
        draft = drafter(seq, K)
        rows, ext = [], list(seq)
        for i in range(K + 1):
            rows.append(model.logits(ext))
            if i < K:
                ext.append(draft[i])
        na, nx = oracle.verify_greedy(np.array(rows)[None], np.array([draft], dtype=np.int32))
        seq += list(draft[:na[0]]) + [int(nx[0])]
    return seq[:len(prompt) + n]


@pytest.mark.parametrize("K", [1, 3, 5])
def test_greedy_reproduces_plain_greedy_decoding(K):
    V = 5
    model = TinyModel(V, seed=K)
    prompt = [0, 1]
    ref = plain_greedy(model, prompt, 200)
    rng = np.random.default_rng(K)

    def perfect(seq, k):
        return plain_greedy(model, seq, k)[len(seq):]

    def all_wrong(seq, k):
        good = perfect(seq, k)
        return [(t + 1) % V for t in good]

    def random_draft(seq, k):
        return [int(x) for x in rng.integers(0, V, size=k)]

    def half_right(seq, k):
        good = perfect(seq, k)
        cut = int(rng.integers(0, k + 1))
        return good[:cut] + [(t + 2) % V for t in good[cut:]]

    for drafter in [perfect, all_wrong, random_draft, half_right]:
        assert speculative_greedy(model, prompt, 200, K, drafter) == ref


def test_greedy_every_draft_emits_a_prefix_of_plain_decoding():
    V, K = 5, 3
    model = TinyModel(V, seed=99)
    ref = plain_greedy(model, [3, 4], 60)
    seq = [3, 4]
    while len(seq) < 40:
        rows_for = {}
        outs = set()
        for draft in itertools.product(range(V), repeat=K):
            rows, ext = [], list(seq)
            for i in range(K + 1):
                rows.append(model.logits(ext))
                if i < K:
                    ext.append(draft[i])
            na, nx = oracle.verify_greedy(np.array(rows)[None], np.array([draft], dtype=np.int32))
            emitted = list(draft[:na[0]]) + [int(nx[0])]
            assert seq + emitted == ref[:len(seq) + len(emitted)]
            outs.add(len(emitted))
            rows_for[draft] = emitted
        assert max(outs) == K + 1  # the perfect draft is among them
        seq = seq + rows_for[tuple(ref[len(seq):len(seq) + K])][:1]
