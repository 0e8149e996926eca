"""The oracle's pins have power: each plausible one-place mistake, planted in a
temporary copy of the oracle's C source and built on the CPU, must fail at
least one of the checks below, while the committed oracle passes them all.

The checks are condensed versions of the pins in test_oracle_*.py (numpy
argmax with ties, brute-force greedy, ragged vs dense, exact law of the
sampled verify against its closed forms, torch softmax in fp64, ICDF edges).
"""
import functools
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import oracle
from tests.exact_law import emitted_marginal, enumerate_law, prob_n_at_least

SRC_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


def check_argmax(lib):
    rng = np.random.default_rng(0)
    for _ in range(20):
        row = rng.integers(-3, 3, size=257).astype(np.float32)
        assert oracle.argmax_row(row, lib=lib) == int(np.argmax(row))


def check_greedy(lib):
    import itertools
    rng = np.random.default_rng(1)
    V, K = 3, 3
    target = rng.permutation(np.arange((K + 1) * V)).reshape(1, K + 1, V).astype(np.float64)
    chain = [int(np.argmax(target[0, i])) for i in range(K + 1)]
    drafts = np.array(list(itertools.product(range(V), repeat=K)), dtype=np.int32)
    n, nx = oracle.verify_greedy(np.repeat(target, len(drafts), axis=0), drafts, lib=lib)
    for d, nn, xx in zip(drafts, n, nx):
        m = 0
        while m < K and d[m] == chain[m]:
            m += 1
        assert nn == m and xx == chain[m]
    # lens and out-of-range tokens
    B, K, V = 12, 5, 30
    tgt = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    ch = tgt.argmax(-1).astype(np.int32)
    lens = rng.integers(-1, K + 2, size=B).astype(np.int32)
    n, nx = oracle.verify_greedy(tgt, ch[:, :K], lens, lib=lib)
    kb = np.clip(lens, 0, K)
    assert (n == kb).all() and (nx == ch[np.arange(B), kb]).all()
    bad = ch[:, :K].copy()
    bad[:, 1] = V
    n, _ = oracle.verify_greedy(tgt, bad, lib=lib)
    assert (n == 1).all()


def rows(rng, r, V, conc=1.0):
    x = rng.gamma(conc, size=(r, V))
    return x / x.sum(-1, keepdims=True)


def check_sampled_law(lib):
    rng = np.random.default_rng(2)
    K, V = 2, 6
    p = rows(rng, K + 1, V)
    q = rows(rng, K, V, 0.5)

    def run(P, Q, T, U):
        n, nx, _ = oracle.accept(P, Q, T, U, lib=lib)
        return n, nx

    law, bad = enumerate_law(p, q, run)
    a = np.minimum(p[:K], q).sum(-1)
    for i in range(K + 1):
        assert prob_n_at_least(law, i) == pytest.approx(np.prod(a[:i]), abs=1e-12)
        np.testing.assert_allclose(emitted_marginal(law, i, V), np.prod(a[:i]) * p[i], atol=1e-12)
    assert bad == 0


def check_ragged(lib):
    rng = np.random.default_rng(3)
    B, K, V = 30, 5, 12
    p = rows(rng, B * (K + 1), V).reshape(B, K + 1, V)
    q = rows(rng, B * K, V).reshape(B, K, V)
    t = rng.integers(0, V, size=(B, K)).astype(np.int32)
    u = rng.random((B, K + 1))
    lens = rng.integers(0, K + 1, size=B).astype(np.int32)
    n, nx, _ = oracle.accept(p, q, t, u, lens, lib=lib)
    for b in range(B):
        kb = lens[b]
        n1, nx1, _ = oracle.accept(p[b:b + 1, :kb + 1], q[b:b + 1, :kb], t[b:b + 1, :kb], u[b:b + 1, :kb + 1],
                                   lib=lib)
        assert n1[0] == n[b] and nx1[0] == nx[b]
    # p(t) == 0 is rejected even at u == 0
    pp = np.array([[[0.5, 0.5, 0.0], [0.2, 0.3, 0.5]]])
    qq = np.array([[[0.0, 0.5, 0.5]]])
    n, nx, _ = oracle.accept(pp, qq, np.array([[2]]), np.array([[0.0, 0.0]]), lib=lib)
    assert n[0] == 0 and nx[0] == 0


def check_warp(lib):
    g = torch.Generator().manual_seed(4)
    z = (3 * torch.randn(3, 777, generator=g)).float()
    ref = torch.softmax(z.double() / 0.8, -1).numpy()
    for r in range(3):
        np.testing.assert_allclose(oracle.warp_row(z[r], 0.8, lib=lib), ref[r], atol=1e-15, rtol=1e-12)
    lens = np.array([0, 2, 5], dtype=np.int32)
    zz = z.reshape(3, 1, 777).repeat(1, 4, 1).numpy()
    out = oracle.softmax_warp(zz, lens, extra_rows=1, T=0.8, lib=lib)
    for b in range(3):
        live = min(3, lens[b]) + 1
        assert np.isfinite(out[b, :live]).all() and np.isnan(out[b, live:]).all()


def check_icdf(lib):
    w = np.array([0.0, 0.0, 2.0, 0.0, 1.0, 0.0])
    assert oracle.icdf(w, 0.0, lib=lib)[0] == 2
    assert oracle.icdf(w, 0.66, lib=lib)[0] == 2
    assert oracle.icdf(w, 0.67, lib=lib)[0] == 4
    assert oracle.icdf(np.zeros(4), 0.5, lib=lib)[0] == -1


def check_logits(lib):
    rng = np.random.default_rng(5)
    B, K, V, T = 40, 4, 60, 0.8
    zt = (2 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    zd = (zt[:, :K] + rng.standard_normal((B, K, V))).astype(np.float32)
    # against the composition of the separately pinned warp (torch) and verify
    p_ref = torch.softmax(torch.from_numpy(zt).double() / T, -1).numpy()
    q_ref = torch.softmax(torch.from_numpy(zd).double() / T, -1).numpy()
    t = np.array([[rng.choice(V, p=q_ref[b, i]) for i in range(K)] for b in range(B)], dtype=np.int32)
    u = rng.random((B, K + 1))
    lens = rng.integers(0, K + 1, size=B).astype(np.int32)
    n1, x1, _ = oracle.accept(p_ref, q_ref, t, u, lens, lib=lib)
    n2, x2, _ = oracle.accept_logits(zt, zd, t, u, lens, T, lib=lib)
    assert (n1 == n2).all() and (x1 == x2).all()


def check_logits_lse(lib):
    # a draft normaliser larger by log(1.25) scales q by 0.8: exact law against
    # the closed forms, on rows where q < c * p at some ids and not at others (so
    # that acceptance and residual both depend on every row's scale)
    from tests.test_oracle_logits import exact_lse
    rng = np.random.default_rng(7)
    K, V, T, c = 2, 4, 0.6, 1.25
    zt = 1.5 * rng.standard_normal((K + 1, V)) + 2.0
    zd = zt[:K] + rng.standard_normal((K, V)) + 3.0  # softmax is unchanged; the normaliser is far from 0
    sm = lambda y: np.exp(y - y.max(-1, keepdims=True)) / np.exp(y - y.max(-1, keepdims=True)).sum(-1, keepdims=True)
    p, q = sm(zt / T), sm(zd / T)
    lse = (exact_lse(zd, T) + np.log(c)).astype(np.float32)
    qs = np.exp(zd / T - lse.astype(np.float64)[:, None])

    def run(P, Q, Tk, U):
        Bn = P.shape[0]
        n, nx, _ = oracle.accept_logits(np.broadcast_to(zt, (Bn, K + 1, V)).copy(),
                                        np.broadcast_to(zd, (Bn, K, V)).copy(), Tk, U, None, T, lib=lib,
                                        draft_lse=np.broadcast_to(lse, (Bn, K)).copy())
        return n, nx

    below = q < c * p[:K]
    assert below.any(-1).all() and (~below).any(-1).all()
    law, bad = enumerate_law(p, qs, run)
    scale = np.prod(qs.sum(-1))
    a = np.minimum(q, c * p[:K]).sum(-1)
    for i in range(K + 1):
        assert prob_n_at_least(law, i) / scale == pytest.approx(np.prod(a[:i]), abs=1e-6)
    for i in range(K):
        r = np.maximum(0.0, p[i] - q[i] / c)
        r = r / r.sum() if r.sum() > 0 else p[i]
        want = np.prod(a[:i]) * (np.minimum(q[i], c * p[i]) + (1.0 - a[i]) * r)
        np.testing.assert_allclose(emitted_marginal(law, i, V) / scale, want, atol=1e-6)
    assert bad == 0
    # the accept and draw boundaries themselves (closed forms), where a scale slip shows
    from tests.test_oracle_logits import given_lse_boundaries
    given_lse_boundaries(zt, zd, T, c, lib=lib)


def check_filtered(lib):
    # tie groups at the top-k boundary and in the nucleus (closed forms)
    z = np.array([5.0, 4.0, 3.0, 4.0, 4.0, 1.0], dtype=np.float32)
    got, _ = oracle.warp_row_filtered(z, 1.0, 2, 1.0, lib=lib)
    w = np.exp(np.array([5.0, 4.0, 0, 4.0, 4.0, 0]) - 5.0) * np.array([1, 1, 0, 1, 1, 0])
    np.testing.assert_allclose(got, w / w.sum(), rtol=1e-12)
    z = np.log(np.array([0.4, 0.2, 0.2, 0.1, 0.1]))
    np.testing.assert_allclose(oracle.warp_row_filtered(z, 1.0, 0, 0.41, lib=lib)[0], [0.5, 0.25, 0.25, 0, 0],
                               rtol=1e-12)
    np.testing.assert_allclose(oracle.warp_row_filtered(z, 1.0, 3, 0.55, lib=lib)[0], [0.5, 0.25, 0.25, 0, 0],
                               rtol=1e-12)
    # a k-then-p case against torch: sort, cut, renormalise (tie-free row)
    rng = np.random.default_rng(6)
    z = rng.permutation(np.linspace(-6.0, 6.0, 400)) + rng.uniform(0, 1e-3, 400)
    for k, p, T in [(60, 0.8, 0.9), (60, 1.0, 0.9)]:
        check_filtered_against_torch(z, k, p, T, lib)


def check_filtered_against_torch(z, k, p, T, lib):
    y = torch.as_tensor(z) / T
    kth = torch.topk(y, k).values[-1]
    y = torch.where(y >= kth, y, torch.tensor(-np.inf, dtype=y.dtype))
    pr = torch.softmax(y, -1)
    srt, idx = torch.sort(pr, descending=True)
    above = torch.cumsum(srt, 0) - srt
    keep = torch.zeros_like(pr, dtype=torch.bool)
    keep[idx[above < p]] = True
    ref = torch.where(keep, pr, torch.zeros_like(pr))
    ref = (ref / ref.sum()).numpy()
    np.testing.assert_allclose(oracle.warp_row_filtered(z, T, k, p, lib=lib)[0], ref, rtol=1e-10, atol=1e-300)


def check_gate(lib):
    from tests.test_oracle_gate import brute_choice
    K = 5
    h = np.zeros((2, K))
    t = np.zeros((2, K))
    oracle.gate_update(h, t, K, lens=[5, 0], n_accepted=[2, 0], decay=1.0, lib=lib)
    np.testing.assert_array_equal(t[0], [1, 1, 1, 0, 0])
    np.testing.assert_array_equal(h[0], [1, 1, 0, 0, 0])
    assert t[1].sum() == 0
    h = np.zeros((1, 2))
    t = np.zeros((1, 2))
    for _ in range(200):
        oracle.gate_update(h, t, 2, lens=[2], n_accepted=[1], decay=0.9, lib=lib)
    np.testing.assert_allclose(t[0], [10, 10], rtol=1e-9)
    np.testing.assert_allclose(h[0], [10, 0], rtol=1e-9, atol=1e-12)
    for p in ([0.9, 0.9, 0.0, 0.0, 0.0], [0.7, 0.5, 0.9, 0.3, 0.8], [0.3] * 5, [1.0] * 5):
        hh = np.asarray(p, dtype=np.float64).reshape(1, -1) * 1000
        tt = np.full((1, 5), 1000.0)
        assert oracle.gate_choose(hh, tt, 5, lib=lib)[0] == brute_choice(np.asarray(p), 5)
    # a truncation that wins by less than the margin factor keeps the full draft
    hh = np.array([[0.95, 0.95, 0, 0, 0, 0]]) * 1000
    tt = np.full((1, 6), 1000.0)
    assert oracle.gate_choose(hh, tt, 6, margin=4.0, lib=lib)[0] == 6
    assert oracle.gate_choose(hh, tt, 6, margin=1.15, lib=lib)[0] == 2
    assert oracle.top2_margin(np.array([1.0, 3.0, 3.0], np.float32), lib=lib) == 0.0
    assert oracle.top2_margin(np.array([1.0, 3.0, 2.5], np.float32), lib=lib) == 0.5


def check_penalties(lib):
    z = np.array([2.0, -1.0, 0.0, 3.0, -0.5, 1.5], np.float32)
    np.testing.assert_array_equal(oracle.penalize_row(z, [0, 0, 1, 4, 4, 4, 7, -1, 6], 2.0, 0.5, 0.25, lib=lib),
                                  np.array([0.0, -2.75, 0.0, 3.0, -2.25, 1.5], np.float32))
    # the speculative branch: the prefix of draft tokens before the row, from the committed length on
    zz = np.tile(np.array([1.0, -2.0, 4.0, 0.5], np.float32), (1, 3, 1))     # [1, K + 1 = 3, V = 4]
    seq = np.array([[3, 0, 0, 0]], np.int32)                                # seq_len 1: only id 3 counts
    t = np.array([[2, 2]], np.int32)
    out = oracle.apply_penalties(zz, None, 1, seq, np.array([1], np.int32), t, [2.0], [0.0], [1.0], lib=lib)
    np.testing.assert_array_equal(out[0, 0], [1.0, -2.0, 4.0, 0.25 - 1.0])    # history (3)
    np.testing.assert_array_equal(out[0, 1], [1.0, -2.0, 2.0 - 1.0, -0.75])   # history (3, 2)
    np.testing.assert_array_equal(out[0, 2], [1.0, -2.0, 2.0 - 2.0, -0.75])   # history (3, 2, 2)


ALL_CHECKS = [check_argmax, check_greedy, check_sampled_law, check_ragged, check_warp, check_icdf, check_logits,
              check_logits_lse, check_filtered, check_gate, check_penalties]

# (what goes wrong, exact source text, planted replacement)
MUTANTS = [
    ("argmax ties go to the highest index", "if (v > bv) {", "if (v >= bv) {"),
    ("greedy reads target rows with the draft's stride",
     "am = or_argmax_row(row_ptr(target, dtype, b * (K + 1) + n, V), dtype, V);",
     "am = or_argmax_row(row_ptr(target, dtype, b * K + n, V), dtype, V);"),
    ("greedy ignores the token comparison", "t != am) break;", "t == am + V) break;"),
    ("greedy ignores draft_lens", "int32_t kb = clamp_len(lens, b, K);\n        int32_t n = 0;",
     "int32_t kb = (int32_t)K;\n        int32_t n = 0;"),
    ("ratio inverted", "rho = pt / qt;", "rho = qt / pt;"),
    ("accept test not strict", "if (!(ui < rho)) { /* R2 */", "if (!(ui <= rho)) { /* R2 */"),
    ("draft rows indexed with the target's stride", "row_ptr(q, dtype, b * K + i, V)",
     "row_ptr(q, dtype, b * (K + 1) + i, V)"),
    ("residual sign flipped", "elem(p, dtype, x) - elem(q, dtype, x)", "elem(q, dtype, x) - elem(p, dtype, x)"),
    ("residual without the max(0, .)", "return w > 0.0 ? w : 0.0;", "return kind == 0 ? w : (w > 0.0 ? w : 0.0);"),
    ("final draw reuses the rejected position's uniform", "double uf = elem(uniforms, u_dtype, b * (K + 1) + kb);",
     "double uf = elem(uniforms, u_dtype, b * (K + 1) + n);"),
    ("bonus drawn from row K instead of K_b",
     "next = or_icdf(row_ptr(p, dtype, b * (K + 1) + kb, V), NULL",
     "next = or_icdf(row_ptr(p, dtype, b * (K + 1) + K, V), NULL"),
    ("correction drawn from p instead of the residual", "next = or_icdf(pn, qn, dtype, 0, V, uf, rel_window, &flag);",
     "next = or_icdf(pn, qn, dtype, 1, V, uf, rel_window, &flag);"),
    ("ICDF threshold not strict", "if (c > thr) {", "if (c >= thr) {"),
    ("warp ignores the temperature", "double e = exp(elem(z, dtype, x) / T - m);", "double e = exp(elem(z, dtype, x) - m);"),
    ("warp not normalised", "for (int64_t x = 0; x < V; ++x) p[x] /= s;", "(void)s;"),
    ("ragged warp writes one row too few", "if (live > R) live = R;", "if (live > R) live = R;\n        live -= 1;"),
    ("logits verify warps draft rows with the target's stride",
     "or_warp_row(row_ptr(zd, dtype, b * K + i, V), dtype, V, T, q);",
     "or_warp_row(row_ptr(zd, dtype, b * (K + 1) + i, V), dtype, V, T, q);"),
    ("logits verify draws the correction from the wrong row",
     "or_warp_row(row_ptr(zt, dtype, b * (K + 1) + n, V), dtype, V, T, p);",
     "or_warp_row(row_ptr(zt, dtype, b * (K + 1) + kb, V), dtype, V, T, p);"),
    ("given draft normaliser added instead of subtracted", "exp(elem(z, dtype, x) / T - lse)",
     "exp(elem(z, dtype, x) / T + lse)"),
    ("given draft normaliser without the temperature", "exp(elem(z, dtype, x) / T - lse)",
     "exp(elem(z, dtype, x) - lse)"),
    ("given draft normaliser of position 0 used at every position", "(double)draft_lse[b * K + i], q);",
     "(double)draft_lse[b * K], q);"),
    ("correction renormalises a given draft row",
     "draft_row_given_lse(row_ptr(zd, dtype, b * K + n, V), dtype, V, T, (double)draft_lse[b * K + n], q);",
     "or_warp_row(row_ptr(zd, dtype, b * K + n, V), dtype, V, T, q);"),
    ("top-k drops the ties of the k-th value", "while (n < V && s[n].y >= kth) ++n;", "while (n < V && s[n].y > kth) ++n;"),
    ("top-k keeps one value too many", "double kth = s[top_k - 1].y;", "double kth = s[top_k < V - 1 ? top_k : top_k - 1].y;"),
    ("top-p measured against the unfiltered mass", "for (int64_t i = 0; i < n; ++i) S += exp(s[i].y - m);",
     "for (int64_t i = 0; i < V; ++i) S += exp(s[i].y - m);"),
    ("top-p drops the group that crosses the threshold", "if (i > 0 && !(above < target)) break;",
     "if (i > 0 && !(above + g < target)) break;"),
    ("filtered rows not renormalised", "p[s[i].x] = exp(s[i].y - m) / Sk;", "p[s[i].x] = exp(s[i].y - m) / S;"),
    ("gate counts censored positions as misses", "int64_t last = n < kb ? n : kb - 1;", "int64_t last = kb - 1;"),
    ("gate forgets hits but not trials", "trials[b * NB + c] *= decay;", "trials[b * NB + c] *= 1.0;"),
    ("gate reads the next position's acceptance", "int32_t c = bucket_of(buckets, b, K, n - 1, NB);",
     "int32_t c = bucket_of(buckets, b, K, n < K ? n : K - 1, NB);"),
    ("gate truncation margin inverted", "if (nstar < K && !(best >= margin * full)) len = K;",
     "if (nstar < K && !(best * margin >= full)) len = K;"),
    ("gate verify cost without the per-token slope", "verify_slope_ms * (double)n);", "verify_slope_ms);"),
    ("top-2 margin drops every copy of a tied maximum", "if (x != am && elem(row, dtype, x) > v2)",
     "if (elem(row, dtype, x) < v1 && elem(row, dtype, x) > v2)"),
    ("penalties ignore the draft prefix", "int64_t np = tokens ? r : 0;", "int64_t np = 0;"),
    ("penalty prefix one token short", "int64_t np = tokens ? r : 0;", "int64_t np = tokens && r > 0 ? r - 1 : 0;"),
    ("repetition penalty sign rule inverted", "float z1 = v < 0.0f ? v * theta : v / theta;",
     "float z1 = v < 0.0f ? v / theta : v * theta;"),
    ("frequency penalty ignores the count", "float d = fmaf(frequency, (float)count[x], presence);",
     "float d = frequency + presence;"),
    ("penalty history ignores seq_len", "n0 = seq_len[b];", "n0 = cap;"),
]


@functools.lru_cache(maxsize=None)
def _source():
    with open(os.path.join(SRC_DIR, "sv_oracle.c")) as f:
        return f.read()


def build_variant(tmp_path, text):
    d = tmp_path
    shutil.copy(os.path.join(SRC_DIR, "sv_oracle.h"), d / "sv_oracle.h")
    (d / "sv_oracle.c").write_text(text)
    out = d / "libmutant.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o", str(out), str(d / "sv_oracle.c"),
                    "-lm"], check=True, capture_output=True)
    return oracle.load_library(str(out))


def run_checks(lib):
    failed = []
    for chk in ALL_CHECKS:
        try:
            chk(lib)
        except AssertionError:
            failed.append(chk.__name__)
    return failed


def test_committed_oracle_passes_every_check():
    assert run_checks(None) == []


@pytest.mark.parametrize("what,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, what, old, new):
    src = _source()
    assert src.count(old) == 1, f"mutation site not unique or missing: {old!r}"
    lib = build_variant(tmp_path, src.replace(old, new))
    assert run_checks(lib), f"no check caught: {what}"
